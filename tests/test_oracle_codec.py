"""Pins of the oracle's MX codecs and block quantiser (CPU only).

Each test checks the oracle against something other than itself: numbers the
pages print, PyTorch's own float8 / e8m0 decoders and its fp32->e4m3fn cast,
hand-worked blocks, or a closed form.
"""

import numpy as np
import pytest
import torch

from oracle import mx
from tests.conftest import golden


# ----------------------------------------------------------------- element tables


def test_e2m1_table_matches_printed_grid():
    # "Four bits from the start": E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    g = golden("e2m1_magnitudes.json")
    t = mx.e2m1_table()
    assert t[:8].tolist() == g["magnitudes"]          # codes 0..7 in increasing order
    assert t[8:].tolist() == [-m for m in g["magnitudes"]]  # sign is the top bit
    assert np.signbit(t[8])                           # 0x8 is negative zero


def test_e4m3_table_matches_torch_decoder():
    ours = mx.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e8m0_table_matches_torch_decoder():
    ours = mx.e8m0_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_block_cost_is_136_bits():
    # "Four bits from the start": a 32-element block carries 136 bits, 4.25 bits/weight.
    g = golden("e2m1_magnitudes.json")
    assert mx.mx_bits_per_element("e2m1") == g["effective_bits_per_weight"]
    assert mx.mx_bits_per_element("e2m1") * 32 == g["bits_per_block_of_32"]


# ----------------------------------------------------------------- quantiser vs library cast


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_e4m3_elements_match_torch_rne_cast(seed):
    """Within range, E4M3 rounding is IEEE-style RNE: torch's fp32->e4m3fn cast of
    v / 2^e must give the oracle's element codes (torch NaNs above 464, so those
    elements are skipped; the oracle saturates them)."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    v[0, :32] = 0.0
    v[1, 5] = -0.0
    codes, scales = mx.quantize(v, "e4m3")
    e = scales.astype(np.int64) - 127
    y = v.astype(np.float64).reshape(64, 8, 32) / np.ldexp(1.0, e)[..., None]
    y = y.reshape(64, 256).astype(np.float32)          # exact: power-of-two scaling
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inrange = np.abs(y) < 464
    assert inrange.mean() > 0.99
    assert np.array_equal(codes[inrange], ref[inrange])


def test_scale_is_floor_log2_amax_minus_emax():
    """The page's rule floor(log2(amax)) - emax (E2M1: emax = 2).

    Checked against its defining bracket 2^(e+emax) <= amax < 2^(e+emax+1) on
    fp64 values (including the fp64 neighbours just below powers of two, where
    an fp64 log2 itself rounds up to the integer), and against np.log2 on every
    fp32 value tested (all fp32 inputs are far enough from a power of two for
    fp64's log2 to keep the floor right).
    """
    rng = np.random.default_rng(5)
    amax = np.abs(rng.standard_normal(10000)) * np.exp(rng.uniform(-30, 30, 10000))
    p2 = 2.0 ** np.arange(-60, 60)
    amax = np.concatenate([amax, p2, np.nextafter(p2, 0)])
    e = mx.shared_exponent(amax, 2)
    assert np.all(np.ldexp(1.0, e + 2) <= amax) and np.all(amax < np.ldexp(1.0, e + 3))
    a32 = np.concatenate([amax.astype(np.float32), np.nextafter(p2.astype(np.float32), np.float32(0))])
    e32 = mx.shared_exponent(a32.astype(np.float64), 2)
    assert np.array_equal(e32, np.floor(np.log2(a32.astype(np.float64))).astype(np.int64) - 2)


# ----------------------------------------------------------------- hand-worked blocks


def _blk(vals):
    b = np.zeros(32, dtype=np.float32)
    b[: len(vals)] = vals
    return b[None, :]


def test_e2m1_midpoints_round_half_to_even():
    # amax 4 -> floor(log2 4) - 2 = 0 -> scale 1; midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.
    c, s = mx.quantize(_blk([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, 6.0]), "e2m1")
    assert s[0, 0] == 127
    # codes: 4->6, .25->0 (even), .75->2 (1.0), 1.25->2 (1.0), 1.75->4 (2.0), 2.5->4, 3.5->6, 5->6, -.75->0xA, 6->7
    assert c[0, :10].tolist() == [6, 0, 2, 2, 4, 4, 6, 6, 0xA, 7]


def test_e2m1_saturates_and_scales():
    # amax 7.9: floor(log2 7.9) = 2 -> e = 0; 7.9 clips to 6 (code 7); 6.9 -> 6
    c, s = mx.quantize(_blk([7.9, 6.9, -7.0, 0.1]), "e2m1")
    assert s[0, 0] == 127 and c[0, :4].tolist() == [7, 7, 0xF, 0]
    # amax 0.75 -> floor(log2 .75) = -1 -> e = -3, scale 1/8: 0.75*8 = 6 -> code 7
    c, s = mx.quantize(_blk([0.75, 0.1]), "e2m1")
    assert s[0, 0] == 124 and c[0, 0] == 7 and c[0, 1] == 2      # 0.1*8 = 0.8 -> 1.0 (code 2)


def test_e4m3_saturation_and_subnormals():
    # amax 511 -> floor(log2) = 8 -> e = 0; 511 and 470 clip to 448; 2^-10 is half the
    # smallest subnormal step (tie -> even code 0); 3*2^-10 -> code 2 (tie -> even)
    c, s = mx.quantize(_blk([511.0, 470.0, 2.0 ** -10, 3 * 2.0 ** -10, -(2.0 ** -9)]), "e4m3")
    assert s[0, 0] == 127
    assert c[0, :5].tolist() == [0x7E, 0x7E, 0x00, 0x02, 0x81]


def test_zero_block_and_negative_zero():
    c, s = mx.quantize(np.zeros((2, 32), np.float32), "e4m3")
    assert (s == 0).all() and (c == 0).all()
    v = np.zeros((1, 32), np.float32)
    v[0, 3] = -0.0
    v[0, 4] = 1.0
    v[0, 5] = -1e-30
    c, s = mx.quantize(v, "e4m3")
    assert c[0, 3] == 0x80 and c[0, 5] == 0x80 and c[0, 0] == 0x00


def test_tiny_amax_clamps_scale():
    # amax 2^-130 (fp32 subnormal) -> floor log2 = -130, minus 8 = -138, clamped to -127.
    v = _blk([2.0 ** -130, 2.0 ** -140])
    c, s = mx.quantize(v, "e4m3")
    assert s[0, 0] == 0
    # 2^-130 / 2^-127 = 2^-3 -> E4M3 normal, exponent field -3 + 7 = 4, mantissa 0
    assert c[0, 0] == (4 << 3)
    # 2^-140 / 2^-127 = 2^-13 < half the smallest subnormal (2^-10) -> 0
    assert c[0, 1] == 0


def test_dequantize_round_trip_on_grid_values():
    rng = np.random.default_rng(3)
    for fmt, f in (("e2m1", mx.E2M1), ("e4m3", mx.E4M3)):
        mags = f.levels
        codes = rng.integers(0, len(mags), (16, 64))
        sign = rng.integers(0, 2, (16, 64)) * f.sign_bit
        codes = (codes | sign).astype(np.uint8)
        codes[:, 0] = f.max_code                                  # pin the block max
        codes[:, 32] = f.max_code
        scales = rng.integers(100, 150, (16, 2)).astype(np.uint8)
        v = mx.dequantize(codes, scales, fmt)
        c2, s2 = mx.quantize(v, fmt)
        assert np.array_equal(s2, scales)
        same = mx.dequantize(c2, s2, fmt)
        assert np.array_equal(same, v)


def test_pack_unpack_e2m1():
    rng = np.random.default_rng(0)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    p = mx.pack_e2m1(c)
    assert p.shape == (5, 32)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))
    assert np.array_equal(mx.unpack_e2m1(p), c)


# ----------------------------------------------------------------- the page's grid experiment


def _grid_experiment_inputs(setup):
    rng = np.random.default_rng(setup["seed"])
    n = setup["n"]
    gauss = rng.normal(0, setup["sigma"], n)
    outl = gauss.copy()
    hit = rng.choice(n, n // setup["outlier_fraction_divisor"], replace=False)
    outl[hit] = rng.choice([-1, 1], hit.size) * setup["outlier_magnitude"]
    return {"gaussian": gauss, "gaussian+outliers": outl}


def _metrics(w, q):
    rel = np.linalg.norm(w - q) / np.linalg.norm(w)
    small = np.abs(w) < np.quantile(np.abs(w), 0.99)
    rel99 = np.linalg.norm(w[small] - q[small]) / np.linalg.norm(w[small])
    zeroed = (q[small] == 0).mean() * 100
    return rel, rel99, zeroed


def test_mxfp4_matches_printed_grid_experiment():
    """The MXFP4 rows printed on "Four bits from the start" (seed 7), to the
    printed number of decimals.  Inputs are fp64 there; the oracle quantises
    fp64 directly."""
    g = golden("mxfp4_grid_experiment.json")
    data = _grid_experiment_inputs(g["setup"])
    for name, want in g["mxfp4"].items():
        w = data[name]
        codes, scales = mx.quantize(w, "e2m1")
        q = mx.dequantize(codes, scales, "e2m1")
        rel, rel99, zeroed = _metrics(w, q)
        assert round(rel, 4) == want["relRMSE"], (name, rel)
        assert round(rel99, 4) == want["relRMSE_99"], (name, rel99)
        assert round(zeroed, 2) == want["zeroed_pct"], (name, zeroed)


def test_grid_experiment_detects_wrong_scale_rule():
    """Mutation check: an off-by-one shared exponent moves the printed numbers."""
    g = golden("mxfp4_grid_experiment.json")
    w = _grid_experiment_inputs(g["setup"])["gaussian"]
    blocks = w.reshape(-1, 32)
    amax = np.abs(blocks).max(1)
    e = mx.shared_exponent(amax, 1)                     # wrong emax
    y = np.minimum(np.abs(blocks) / np.ldexp(1.0, e)[:, None], 6.0)
    q = mx.E2M1.levels[mx.round_to_grid(y, "e2m1")] * np.ldexp(1.0, e)[:, None] * np.sign(blocks)
    rel, _, _ = _metrics(w, q.reshape(-1))
    assert round(rel, 4) != g["mxfp4"]["gaussian"]["relRMSE"]
