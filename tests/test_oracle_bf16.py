"""Pins of the oracle's higher-precision map (CPU only): bfloat16 latent
projections and shared experts, MXFP4 routed experts (Kimi K3 and the New
Open-Weights Moat, "Precision and deployment", Fig. 6)."""

import dataclasses

import numpy as np
import torch

import synth
from oracle import moe, mx, weights
from tests.test_oracle_layer import _torch_deq, _torch_mxfp8


def _special_f32():
    g = np.random.default_rng(11)
    v = [g.standard_normal(4000) * s for s in (1e-3, 1.0, 1e3, 1e30)]
    # exact midpoints between neighbouring bfloat16 values, both parities
    base = mx.bf16_value(g.integers(0x0080, 0x7F00, 2000).astype(np.uint16)).astype(np.float32)
    half = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    near = [np.nextafter(half, np.float32(np.inf)), np.nextafter(half, np.float32(0))]
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38, -3.4028235e38,
                        1e-45, -1e-45, 1.1754942e-38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 255.5, 256.5],
                       dtype=np.float32)
    return np.concatenate([np.concatenate(v).astype(np.float32), half, -half, *near, special])


def test_bf16_rounding_matches_torch():
    """Round to nearest even on the fp32 input, including exact ties of both
    parities, overflow to infinity, subnormals and signed zeros."""
    f = _special_f32()
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = mx.bf16_bits(f)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    nan = mx.bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(mx.bf16_value(nan)).all()


def test_bf16_values_match_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = mx.bf16_value(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_map_weights_are_the_same_fp32_weights_rounded():
    cfg = synth.config("tiny_bf16")
    W = weights.layer(cfg)
    assert W.precision == "bf16" and isinstance(W.w_down, moe.BF16Tensor)
    ref = torch.from_numpy(synth.gen_weight(cfg, "w_gate_s", 0)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(W.w_gate_s[0].deq(), ref)
    # the routed experts are the MX presets' own MXFP4 codes
    Wm = weights.layer(synth.config("tiny"))
    assert np.array_equal(W.w_gate_e[3].codes, Wm.w_gate_e[3].codes)


def test_bf16_map_top1_layer_equals_torch_pipeline():
    """k = 1 under the bfloat16 map, rebuilt from PyTorch primitives: its own
    bfloat16 casts of x, of the fp32 weights, of the shared hidden state and of
    the combined latent; its own MXFP8 quantiser and MXFP4 decode for the
    routed expert."""
    cfg = synth.config("tiny_bf16", T=16)
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    tr = moe.forward(x, W, top_k=1)
    assert np.all(tr.routing.gates == 1.0)

    bf = lambda v: torch.as_tensor(v).to(torch.float32).to(torch.bfloat16).to(torch.float64)
    wt = lambda n, i=0: bf(torch.from_numpy(synth.gen_weight(cfg, n, i)))
    xb = bf(torch.from_numpy(x))
    z = xb @ wt("w_down").T
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
    y = bf(y_lat) @ wt("w_up").T
    hs = torch.nn.functional.silu(xb @ wt("w_gate_s").T) * (xb @ wt("w_up_s").T)
    y = (y + bf(hs) @ wt("w_down_s").T).numpy()
    assert np.abs(y - tr.y).max() <= 1e-9 * np.abs(tr.y).max()


def test_bf16_map_grouped_layer_equals_dense_mask():
    cfg = synth.config("tiny_bf16", T=24)
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    tr = moe.forward(x, W, cfg.top_k)
    yd = moe.forward_dense_mask(x, W, cfg.top_k)
    assert np.abs(yd - tr.y).max() <= 1e-12 * np.abs(tr.y).max()


def test_bf16_map_changes_only_the_dense_parts():
    """Same fp32 weights and input: the two maps share the routed experts'
    codes, but the bfloat16 map reads x at bfloat16 (not MXFP8) in its dense
    GEMMs, so z and the output move by about the MXFP8-vs-bfloat16 input error."""
    x = synth.gen_hidden(synth.config("tiny", T=32))
    a = moe.forward(x, weights.layer(synth.config("tiny", T=32)), 4)
    b = moe.forward(x, weights.layer(synth.config("tiny_bf16", T=32)), 4)
    assert isinstance(b.xq, moe.BF16Tensor) and isinstance(b.hq_shared[0], moe.BF16Tensor)
    rel = np.linalg.norm(a.z - b.z) / np.linalg.norm(b.z)
    assert 1e-3 < rel < 0.2
