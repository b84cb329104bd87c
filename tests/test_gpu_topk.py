"""The router's top-k selection stage against the oracle's selection, through
the C-ABI (moe_router_topk, moe_router_reduce_topk).

The oracle's router runs on the identity matrix, so its logits are the given
fp32 logits exactly; with softmax gating the selection keys are logit +
selection bias in fp32 on both sides, so the ids must be equal element for
element (ties by ascending id).  Sigmoid keys differ from the oracle's by the
device's rounding of the sigmoid, so there ids must agree on every token
whose k-th and (k+1)-th oracle keys are more than a few ulps apart.  Cases
cover the threshold path (few candidates), the round-based path it falls
back to (many equal keys), exact ties, NaN and -inf logits, k = 1 and k = 64,
E not a multiple of 64, and E above 1024 (keys in LDS).  The fused variant
must reproduce the sequential fp32 sum of the K-slice partials plus the
logit bias bit for bit, and then the same ids and gates as the plain one.
"""

import numpy as np
import pytest

from oracle import moe as O
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    from latent_routing_mxfp4_amd import _lib
    return _lib


def _gpu_topk(logits, sel_bias, k, softmax):
    L = _lib()
    T, E = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    sb = torch.from_numpy(np.ascontiguousarray(sel_bias, dtype=np.float32)).cuda() if sel_bias is not None else None
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.moe_router_topk(lg.data_ptr(), sb.data_ptr() if sb is not None else 0, T, E, k, softmax, ids.data_ptr(),
                      gates.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), gates.cpu().numpy()


def _oracle(logits, sel_bias, k, softmax):
    E = logits.shape[1]
    return O.route(logits.astype(np.float32), np.eye(E), k, selection_bias=sel_bias, decide=np.float32,
                   gating="softmax" if softmax else "sigmoid")


CASES = [  # (T, E, k)
    (257, 896, 16), (64, 64, 8), (33, 37, 5), (100, 1024, 64), (100, 1000, 1), (50, 1280, 16), (20, 5, 5),
]


@pytest.mark.parametrize("T,E,k", CASES)
def test_softmax_keys_exact(T, E, k):
    rng = np.random.default_rng(1000 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    sel = (0.1 * rng.standard_normal(E)).astype(np.float32)
    ids, gates = _gpu_topk(logits, sel, k, softmax=True)
    r = _oracle(logits, sel, k, softmax=True)
    assert np.array_equal(ids, r.ids)
    np.testing.assert_allclose(gates, r.gates, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("T,E,k", [(257, 896, 16), (64, 1024, 64), (40, 1280, 8)])
def test_sigmoid_keys(T, E, k):
    rng = np.random.default_rng(2000 + E)
    logits = (2.0 * rng.standard_normal((T, E))).astype(np.float32)
    sel = (0.05 * rng.standard_normal(E)).astype(np.float32)
    ids, gates = _gpu_topk(logits, sel, k, softmax=False)
    r = _oracle(logits, sel, k, softmax=False)
    kth = np.take_along_axis(r.sel, r.ids[:, -1:], axis=1)[:, 0]
    clear = r.gap > 8 * np.spacing(np.abs(kth).astype(np.float32)).astype(np.float64)
    say(f"  {int(clear.sum())} of {T} tokens without a near-tie")
    assert np.array_equal(ids[clear], r.ids[clear])
    np.testing.assert_allclose(gates[clear], r.gates[clear], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("levels", [4, 200])
def test_exact_ties(levels):
    """Logits on a grid of `levels` values: many equal keys.  With 4 levels
    most lanes share the top key (the fallback path); with 200, a few equal
    keys among the candidates (the threshold path's tie order)."""
    rng = np.random.default_rng(3000 + levels)
    T, E, k = 128, 896, 16
    logits = (rng.integers(0, levels, size=(T, E)) / 8.0).astype(np.float32)
    ids, gates = _gpu_topk(logits, None, k, softmax=True)
    r = _oracle(logits, None, k, softmax=True)
    assert np.array_equal(ids, r.ids)
    np.testing.assert_allclose(gates, r.gates, rtol=1e-5, atol=1e-7)


def test_all_equal_and_zero():
    T, E, k = 8, 896, 16
    for softmax in (True, False):
        ids, gates = _gpu_topk(np.zeros((T, E), np.float32), None, k, softmax)
        assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (T, 1)))
        np.testing.assert_allclose(gates, np.full((T, k), 1.0 / k), rtol=1e-6)


def test_nan_and_minus_inf_rank_last():
    """NaN and -inf logits get the lowest finite key: after every finite key,
    among themselves by ascending id."""
    rng = np.random.default_rng(4000)
    T, E, k = 64, 896, 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bad = rng.random((T, E)) < 0.3
    logits[bad & (rng.random((T, E)) < 0.5)] = np.nan
    logits[bad & ~np.isnan(logits)] = -np.inf
    logits[5, :890] = np.nan   # a token with only 6 finite logits
    ids, _ = _gpu_topk(logits, None, k, softmax=True)
    clean = np.where(np.isfinite(logits), logits, -np.finfo(np.float32).max).astype(np.float32)
    r = _oracle(clean, None, k, softmax=True)
    assert np.array_equal(ids, r.ids)


@pytest.mark.parametrize("T,E,k,nz,bias", [(64, 896, 16, 28, True), (5, 100, 7, 2, False), (1, 1024, 64, 33, True),
                                           (3, 64, 64, 40, False), (70, 896, 16, 7, True)])
def test_reduce_topk_fused(T, E, k, nz, bias):
    L = _lib()
    rng = np.random.default_rng(5000 + nz)
    part = (0.3 * rng.standard_normal((nz, T, E))).astype(np.float32)
    part[0, 0, :3] = -0.0   # signed zeros through the sum
    lb = (0.2 * rng.standard_normal(E)).astype(np.float32) if bias else None
    sel = (0.05 * rng.standard_normal(E)).astype(np.float32)
    v = part[0].copy()
    for s in range(1, nz):   # slice order, fp32
        v = (v + part[s]).astype(np.float32)
    want = (v + (lb if bias else np.float32(0.0))).astype(np.float32)
    dp = torch.from_numpy(part).cuda()
    dlb = torch.from_numpy(lb).cuda() if bias else None
    dsel = torch.from_numpy(sel).cuda()
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    for softmax in (False, True):
        L.moe_router_reduce_topk(dp.data_ptr(), nz, dlb.data_ptr() if bias else 0, dsel.data_ptr(), T, E, k,
                                 softmax, lg.data_ptr(), ids.data_ptr(), gates.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got = lg.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        ids2, gates2 = _gpu_topk(want, sel, k, softmax)
        assert np.array_equal(ids.cpu().numpy(), ids2)
        assert np.array_equal(gates.cpu().numpy().view(np.uint32), gates2.view(np.uint32))
