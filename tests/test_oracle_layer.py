"""Pins of the oracle's routing, dispatch and layer (CPU only)."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import moe, mx, weights
from tests.conftest import golden


# ----------------------------------------------------------------- the page's MoE data-path toy


def _toy_inputs(g):
    s = g["setup"]
    rng = np.random.default_rng(s["seed"])
    T, D, E = s["T"], s["D"], s["E"]
    x = rng.normal(size=(T, D)).astype(np.float32)
    W = rng.normal(size=(E, D, D)).astype(np.float32) * 0.1
    router = rng.normal(size=(D, E)).astype(np.float32)
    return x, W, router


def test_toy_tokens_per_expert():
    """Selection + histogram against the printed tokens-per-expert list.

    The toy ranks raw logits; the oracle ranks sigmoid(logits), a monotone map,
    so the selected sets must agree.  The toy's router is [D][E] (x @ router);
    the oracle takes [E][D]."""
    g = golden("moe_datapath_toy.json")
    x, W, router = _toy_inputs(g)
    K = g["setup"]["K"]
    r = moe.route(x.astype(np.float64), router.T, K, decide=None)
    d = moe.dispatch(r.ids, g["setup"]["E"])
    assert d.counts.tolist() == g["tokens_per_expert"]
    assert d.pair_of_row.size == g["permuted_buffer_rows"]


def test_toy_grouped_path_matches_dense_loop():
    """The toy's own check: grouped (sorted-segment) evaluation == per-token loop."""
    g = golden("moe_datapath_toy.json")
    x, W, router = _toy_inputs(g)
    K, E, T = g["setup"]["K"], g["setup"]["E"], g["setup"]["T"]
    x64 = x.astype(np.float64)
    r = moe.route(x64, router.T, K, decide=None)
    d = moe.dispatch(r.ids, E)
    xp = x64[d.pair_of_row // K]
    yp = np.empty_like(xp)
    for e in range(E):
        lo, hi = d.offsets[e], d.offsets[e + 1]
        yp[lo:hi] = xp[lo:hi] @ W[e].astype(np.float64)
    y = np.zeros_like(x64)
    np.add.at(y, d.pair_of_row // K, yp * r.gates.reshape(-1)[d.pair_of_row][:, None])
    ref = np.zeros_like(x64)
    for t in range(T):
        for j in range(K):
            ref[t] += r.gates[t, j] * (x64[t] @ W[r.ids[t, j]].astype(np.float64))
    assert g["matches_dense_loop"] and np.allclose(y, ref, atol=1e-12)


# ----------------------------------------------------------------- invariants on the tiny preset


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny")
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    return cfg, W, x, moe.forward(x, W, cfg.top_k)


def test_routing_invariants(tiny):
    cfg, W, x, tr = tiny
    r, d = tr.routing, tr.disp
    T, k, E = cfg.T, cfg.top_k, cfg.n_routed
    assert r.ids.shape == (T, k)
    for t in range(T):
        assert len(set(r.ids[t].tolist())) == k
        keys = r.sel[t, r.ids[t]]
        assert np.all(np.diff(keys) <= 0)                      # slot order: descending key
        rest = np.setdiff1d(np.arange(E), r.ids[t])
        assert keys.min() >= r.sel[t, rest].max()             # the k winners really are on top
    assert np.allclose(r.gates.sum(1), 1.0, atol=1e-15, rtol=0)
    assert d.counts.sum() == T * k
    assert np.array_equal(np.sort(d.pair_of_row), np.arange(T * k))   # bijection
    assert np.array_equal(d.row_of_pair[d.pair_of_row], np.arange(T * k))
    for e in range(E):
        seg = d.pair_of_row[d.offsets[e]:d.offsets[e + 1]]
        assert np.all(r.ids.reshape(-1)[seg] == e)
        assert np.all(np.diff(seg // k) > 0)                  # ascending token order (stable)


def test_selection_bias_moves_selection_not_gates():
    """Moat page, Fig. 2: the bias decides who is picked but the gates are the
    raw sigmoid scores of the winners, normalised by their sum."""
    cfg = synth.config("tiny")
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    z = moe.mm(moe.quant(x), W.w_down)
    b = synth.gen_selection_bias(cfg, std=0.05)
    r0 = moe.route(z, W.w_router, cfg.top_k)
    r1 = moe.route(z, W.w_router, cfg.top_k, selection_bias=b)
    assert not np.array_equal(r0.ids, r1.ids)
    raw = np.take_along_axis(r1.scores, r1.ids, axis=1)
    assert np.allclose(r1.gates, raw / raw.sum(1, keepdims=True), rtol=0, atol=1e-15)
    assert np.array_equal(r1.scores, r0.scores)


def test_all_ties_pick_lowest_ids_and_zero_input_gives_zero_output():
    cfg = synth.config("tiny", T=8)
    W = weights.layer(cfg)
    x = np.zeros((8, cfg.d_model), np.float32)
    tr = moe.forward(x, W, cfg.top_k)
    assert np.all(tr.routing.ids == np.arange(cfg.top_k)[None, :])
    assert np.all(tr.routing.gap == 0)
    assert np.all(tr.routing.gates == 1.0 / cfg.top_k)
    assert np.all(tr.y == 0)


def test_grouped_layer_equals_dense_mask_bruteforce(tiny):
    """Every expert on every token, masked by a dense gate matrix, equals the
    permuted/segmented path (the toy's dense-loop check at layer level)."""
    cfg, W, x, tr = tiny
    y_dense = moe.forward_dense_mask(x, W, cfg.top_k)
    assert np.abs(y_dense - tr.y).max() <= 1e-12 * np.abs(tr.y).max()


def test_mx_matmul_is_exact_on_layer_operands(tiny):
    """fp64 accumulation of MX products equals exact rational arithmetic on the
    tiny layer's own operands (a sample of rows of each GEMM)."""
    cfg, W, x, tr = tiny
    cases = [(tr.xq[:3], W.w_down[:8]), (tr.zq[:3], W.w_gate_e[0][:8]),
             (tr.hq_rows[:3], W.w_down_e[1][:8]), (tr.yq[:3], W.w_up[:8])]
    for a, b in cases:
        got = moe.mm(a, b)
        ex = mx.mx_matmul_exact(a.codes, a.scales, a.fmt, b.codes, b.scales, b.fmt)
        assert np.array_equal(got, ex)


def test_mx_matmul_exact_vs_fp64_random_scales():
    rng = np.random.default_rng(11)
    a = moe.quant((rng.standard_normal((4, 128)) * np.exp(rng.uniform(-8, 8, (4, 128)))).astype(np.float32))
    b = moe.quant((rng.standard_normal((5, 128)) * np.exp(rng.uniform(-8, 8, (5, 128)))).astype(np.float32), "e2m1")
    assert np.array_equal(moe.mm(a, b), mx.mx_matmul_exact(a.codes, a.scales, "e4m3", b.codes, b.scales, "e2m1"))


# ----------------------------------------------------------------- single-expert reduction vs torch


def _torch_deq(codes, scales, fmt):
    """Independent decode via PyTorch's float8 / e8m0 dtypes (E2M1 via its E4M3 image:
    every E2M1 value is exactly representable in E4M3)."""
    c = torch.from_numpy(np.ascontiguousarray(codes))
    if fmt == "e4m3":
        v = c.view(torch.float8_e4m3fn).to(torch.float64)
    else:
        e2 = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float32).to(torch.float8_e4m3fn)
        mag = e2.view(torch.uint8)[(c & 7).long()]
        v = (mag | ((c & 8) << 4)).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).to(torch.float64)
    K = v.shape[-1]
    return (v.reshape(*v.shape[:-1], K // 32, 32) * s[..., None]).reshape(v.shape)


def _torch_mxfp8(v):
    """MXFP8 quantise with PyTorch primitives: exponent from frexp, elements via
    the library's fp32->e4m3fn RNE cast after clipping to 448."""
    v = torch.as_tensor(v, dtype=torch.float64).to(torch.float32).to(torch.float64)
    blocks = v.reshape(*v.shape[:-1], -1, 32)
    amax = blocks.abs().amax(-1)
    _, ex = torch.frexp(amax)
    e = torch.where(amax == 0, torch.full_like(ex, -127), ex - 1 - 8).clamp(-127, 127)
    y = (blocks / torch.ldexp(torch.ones_like(amax), e)[..., None]).clamp(-448, 448)
    q = y.to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * torch.ldexp(torch.ones_like(amax), e)[..., None]).reshape(v.shape)


def test_top1_layer_equals_textbook_swiglu_mlp():
    """k = 1: the gate is exactly 1 and the routed branch is a single SwiGLU MLP
    in the latent; built here from PyTorch primitives only (independent decode,
    independent MXFP8 quantiser), compared with the oracle's whole layer."""
    cfg = synth.config("tiny", T=16)
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    tr = moe.forward(x, W, top_k=1)
    assert np.all(tr.routing.gates == 1.0)

    xq = _torch_mxfp8(torch.from_numpy(x.astype(np.float64)))
    wdn = _torch_deq(W.w_down.codes, W.w_down.scales, "e2m1")
    z = xq @ wdn.T
    zq = _torch_mxfp8(z)
    y_lat = torch.zeros_like(z)
    for t in range(x.shape[0]):
        e = int(tr.routing.ids[t, 0])
        wg = _torch_deq(W.w_gate_e[e].codes, W.w_gate_e[e].scales, "e2m1")
        wu = _torch_deq(W.w_up_e[e].codes, W.w_up_e[e].scales, "e2m1")
        wd = _torch_deq(W.w_down_e[e].codes, W.w_down_e[e].scales, "e2m1")
        a = zq[t:t + 1]
        h = torch.nn.functional.silu(a @ wg.T) * (a @ wu.T)
        y_lat[t] = (_torch_mxfp8(h) @ wd.T)[0]
    y = _torch_mxfp8(y_lat) @ _torch_deq(W.w_up.codes, W.w_up.scales, "e2m1").T
    wgs = _torch_deq(W.w_gate_s[0].codes, W.w_gate_s[0].scales, "e2m1")
    wus = _torch_deq(W.w_up_s[0].codes, W.w_up_s[0].scales, "e2m1")
    wds = _torch_deq(W.w_down_s[0].codes, W.w_down_s[0].scales, "e2m1")
    hs = torch.nn.functional.silu(xq @ wgs.T) * (xq @ wus.T)
    y = y + _torch_mxfp8(hs) @ wds.T
    y = y.numpy()
    assert np.abs(y - tr.y).max() <= 1e-9 * np.abs(tr.y).max()


def test_oracle_quantiser_matches_torch_mxfp8_on_layer_tensors(tiny):
    cfg, W, x, tr = tiny
    for v, q in ((x, tr.xq), (tr.z, tr.zq), (tr.y_lat, tr.yq)):
        ref = _torch_mxfp8(torch.from_numpy(np.asarray(v, np.float64))).numpy()
        assert np.array_equal(q.deq(), ref)


# ----------------------------------------------------------------- presets and closed forms


def test_k3_preset_ratios():
    """Moat page, "Sparse computation": 16 of 896 routed, two shared experts,
    7,168-wide model, 3,584-wide latent."""
    for name in ("k3_decode", "k3_prefill", "k3_skew"):
        c = synth.config(name)
        assert (c.top_k, c.n_routed, c.n_shared) == (16, 896, 2)
        assert (c.d_model, c.d_latent) == (7168, 3584) and 2 * c.d_latent == c.d_model


def test_distinct_expert_closed_form_matches_page_simulation():
    """Expected distinct experts touched by B tokens under uniform top-k routing,
    E(1 - (1 - k/E)^B), times the page's 1.5 GB/expert over B, against the
    page's simulated uniform column (16 trials per point, so ~1% noise)."""
    g = golden("batch_amortization.json")
    E, k, gb = g["E"], g["k"], g["gb_per_expert"]
    for B, want in g["uniform_gb_per_token"].items():
        B = int(B)
        distinct = E * (1 - (1 - k / E) ** B)
        assert abs(distinct * gb / B - want) <= 0.01 * want + 0.005, (B, distinct * gb / B, want)


def test_zipf_bias_skews_load():
    cfg = synth.config("k3_skew")
    b = synth.gen_logit_bias(cfg)
    assert b.shape == (896,) and abs(b.max() - math.log(896 / sum(r ** -1.1 for r in range(1, 897)))) < 1e-5
    assert b.min() < -2 and b.max() > 5
