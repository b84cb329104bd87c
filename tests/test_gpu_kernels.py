"""Stage-level GPU checks of the HIP kernels against the oracle (gfx950 only).

Every case prints its name and shape before touching the GPU.
"""

import numpy as np
import pytest

from oracle import moe, mx
from tests import parity
from tests.frag_layout import to_fragment_order
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def LY():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_routing_mxfp4_amd import layer
    return layer


def _special_values(rng, rows, K):
    """fp32 test matrix: wide exponent range, zeros, -0, subnormals, exact
    midpoints of both grids, saturating blocks and powers of two."""
    v = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-140, 120, (rows, 1)))).astype(np.float32)
    v[0, :32] = 0.0
    v[1, :32] = -0.0
    v[2, :32] = np.float32(2.0 ** -149) * rng.integers(1, 100, 32)          # subnormals
    mids4 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0], np.float32)
    v[3, :32] = np.tile(mids4, 4) * np.sign(rng.standard_normal(32)).astype(np.float32)
    e4 = np.array([448.0, 470.0, 511.0, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 300.0], np.float32)
    v[4, :32] = np.tile(e4, 4)
    v[5, :32] = np.exp2(rng.integers(-20, 20, 32)).astype(np.float32)
    v[6, :32] = np.nextafter(np.exp2(rng.integers(-20, 20, 32)).astype(np.float32), np.float32(0))
    v[7, :32] = np.float32(3.0e38) * rng.uniform(-1, 1, 32).astype(np.float32)
    return v


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantize_bit_exact(LY, fmt):
    rng = np.random.default_rng(42)
    for rows, K in ((64, 256), (37, 96), (1, 32)):
        say(f"quantize {fmt} rows={rows} K={K}")
        v = _special_values(rng, max(rows, 8), K)[:rows] if rows >= 8 else rng.standard_normal((rows, K)).astype(np.float32)
        codes, scales = LY.mx_quantize(torch.from_numpy(v).cuda(), 0 if fmt == "e4m3" else 1)
        torch.cuda.synchronize()
        rc, rs = mx.quantize(v, fmt)
        if fmt == "e2m1":
            rc = mx.pack_e2m1(rc)
        assert np.array_equal(scales.cpu().numpy(), rs)
        assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_weights_fragment_order(LY):
    """Fragment-order E2M1 encoding = the oracle's codes, permuted as defined."""
    rng = np.random.default_rng(43)
    for G, N, K in ((3, 48, 384), (1, 16, 128), (2, 64, 1024)):
        say(f"quantize_weights G={G} N={N} K={K}")
        v = _special_values(rng, G * N, K).reshape(G, N, K)
        codes, scales = LY.mx_quantize_weights(torch.from_numpy(v).cuda())
        torch.cuda.synchronize()
        rc, rs = mx.quantize(v, "e2m1")
        fc, fs = to_fragment_order(mx.pack_e2m1(rc), rs)
        assert np.array_equal(scales.cpu().numpy(), fs)
        assert np.array_equal(codes.cpu().numpy(), fc)


def test_pack_weights_matches_fragment_quantiser(LY):
    rng = np.random.default_rng(44)
    G, N, K = 4, 32, 512
    say(f"pack_weights G={G} N={N} K={K}")
    v = torch.from_numpy(rng.standard_normal((G, N, K)).astype(np.float32)).cuda()
    rc, rs = LY.mx_quantize(v, 1)
    pc, ps = LY.mx_pack_weights(rc, rs)
    qc, qs = LY.mx_quantize_weights(v)
    torch.cuda.synchronize()
    assert torch.equal(pc, qc) and torch.equal(ps, qs)
    fc, fs = to_fragment_order(rc.cpu().numpy(), rs.cpu().numpy())
    assert np.array_equal(pc.cpu().numpy(), fc) and np.array_equal(ps.cpu().numpy(), fs)


def _rand_mx(rng, rows, K, fmt, spread=4.0):
    v = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-spread, spread, (rows, K // 32)).repeat(32, 1)))
    q = moe.quant(v.astype(np.float32), fmt)
    return q


def _gemm_case(LY, rng, M, N, K):
    say(f"mx_gemm M={M} N={N} K={K}")
    a = _rand_mx(rng, M, K, "e4m3")
    b = _rand_mx(rng, N, K, "e2m1")
    bc, bs = to_fragment_order(mx.pack_e2m1(b.codes), b.scales)
    c = LY.mx_gemm(torch.from_numpy(a.codes).cuda(), torch.from_numpy(a.scales).cuda(),
                   torch.from_numpy(bc).cuda(), torch.from_numpy(bs).cuda())
    torch.cuda.synchronize()
    got = c.cpu().numpy().astype(np.float64)
    ref = moe.mm(a, b)
    bound = parity.mx_mfma_bound(a, b, ref)
    return got, ref, bound, a, b


def test_single_mfma_tile_matches_exact_product(LY):
    """One 16x16x128 block-scaled MFMA: the operand/scale/result lane layout."""
    rng = np.random.default_rng(7)
    got, ref, bound, a, b = _gemm_case(LY, rng, 16, 16, 128)
    exact = mx.mx_matmul_exact(a.codes, a.scales, "e4m3", b.codes, b.scales, "e2m1")
    assert np.array_equal(ref, exact)
    bad = np.argwhere(np.abs(got - ref) > bound)
    assert len(bad) == 0, (f"{len(bad)} outputs outside the bound, first at {bad[:4].tolist()}; "
                           f"max err {np.abs(got - ref).max()}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (17, 80, 256), (64, 256, 512), (300, 384, 1024),
                                   (257, 128, 384), (1000, 96, 128)])
def test_mx_gemm_shapes(LY, M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    got, ref, bound, _, _ = _gemm_case(LY, rng, M, N, K)
    assert np.all(np.abs(got - ref) <= bound), f"max err/bound {np.max(np.abs(got - ref) / bound)}"


def test_mfma_rate_probe_checksum(LY):
    """The matrix-core rate probe really issues its MFMAs: every accumulator
    element gains 128 (128 products of 1.0 x 1.0 at scale 1) per MFMA, so each
    wave's checksum (8 accumulators x 4 values per lane, lane 0) is 4096 * iters."""
    from latent_routing_mxfp4_amd import _lib
    wg, iters = 8, 100
    out = torch.zeros(wg * 4, dtype=torch.float32, device="cuda")
    _lib.moe_mfma_rate_probe(iters, wg, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(out == 4096.0 * iters), out[:4]
