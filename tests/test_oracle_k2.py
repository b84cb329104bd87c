"""Pins of the oracle's second workload (CPU only): a non-latent MoE with the
softmax-over-winners gate of the MoE data-path toy (Four Bits at a Time,
"What it takes to serve it")."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe, weights
from tests.test_oracle_layer import _torch_deq, _torch_mxfp8


def _random_route(gating, k, T=40, E=24, L=16, seed=3, **kw):
    g = np.random.default_rng(seed)
    z = g.standard_normal((T, L))
    w = g.standard_normal((E, L)) / 4
    return moe.route(z, w, k, decide=None, gating=gating, **kw), z, w


def test_softmax_gates_sum_to_one_and_follow_the_logit_order():
    r, z, w = _random_route("softmax", 5)
    assert np.allclose(r.gates.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(r.gates > 0)
    # slots are in descending logit order, so the gates are non-increasing
    assert np.all(np.diff(r.gates, axis=1) <= 1e-15)


def test_softmax_gates_shift_invariant():
    """Adding one constant to every logit (a uniform logit bias) changes neither
    the selection nor the gates."""
    r0, z, w = _random_route("softmax", 4)
    r1 = moe.route(z, w, 4, logit_bias=np.full(w.shape[0], 3.25), decide=None, gating="softmax")
    assert np.array_equal(r0.ids, r1.ids)
    assert np.allclose(r0.gates, r1.gates, rtol=1e-13, atol=0)


def test_softmax_two_winners_closed_form():
    """k = 2: the first gate is the logistic function of the logit difference."""
    r, z, w = _random_route("softmax", 2)
    logits = z @ w.T
    l0 = np.take_along_axis(logits, r.ids[:, :1], axis=1)[:, 0]
    l1 = np.take_along_axis(logits, r.ids[:, 1:2], axis=1)[:, 0]
    assert np.allclose(r.gates[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-13, atol=0)


def test_softmax_single_winner_and_equal_winners():
    r, _, _ = _random_route("softmax", 1)
    assert np.all(r.gates == 1.0)
    z = np.ones((3, 4))
    w = np.ones((6, 4))                         # every logit equal: ties -> lowest ids
    r = moe.route(z, w, 3, decide=None, gating="softmax")
    assert np.array_equal(r.ids, np.tile(np.arange(3), (3, 1)))
    assert np.allclose(r.gates, 1.0 / 3.0, rtol=1e-15, atol=0)


def test_sigmoid_and_softmax_keys_select_the_same_experts():
    """sigmoid is increasing, so without a selection bias both gate variants
    select the same experts in the same slots."""
    a, z, w = _random_route("softmax", 6)
    b = moe.route(z, w, 6, decide=None, gating="sigmoid")
    assert np.array_equal(a.ids, b.ids)


def test_k2_preset_shape():
    for name in ("k2_tiny", "k2_prefill"):
        c = synth.config(name)
        assert not c.latent and c.gating == "softmax" and c.d_latent == c.d_model
    c = synth.config("k2_prefill")
    assert (c.d_model, c.n_routed, c.top_k, c.n_shared, c.d_ff_routed) == (7168, 384, 8, 1, 2048)


@pytest.fixture(scope="module")
def k2_tiny():
    cfg = synth.config("k2_tiny", T=24)
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    return cfg, W, x, moe.forward(x, W, cfg.top_k)


def test_nonlatent_layer_has_no_latent_steps(k2_tiny):
    cfg, W, x, tr = k2_tiny
    assert W.w_down is None and W.w_up is None and tr.yq is None
    assert np.array_equal(tr.zq.codes, tr.xq.codes)          # the experts read xq
    assert np.allclose(tr.y, tr.y_lat + sum(tr.y_shared), rtol=1e-14, atol=1e-14)


def test_nonlatent_grouped_path_equals_dense_mask(k2_tiny):
    """Brute force: every expert on every token, masked by the dense gate matrix."""
    cfg, W, x, tr = k2_tiny
    yb = moe.forward_dense_mask(x, W, cfg.top_k)
    assert np.abs(yb - tr.y).max() <= 1e-12 * np.abs(tr.y).max()


def test_nonlatent_top1_equals_textbook_swiglu_mlp():
    """k = 1: the softmax gate is exactly 1 and the layer is one SwiGLU MLP on
    the MXFP8 input plus the shared expert, built from PyTorch primitives only
    (independent decode and MXFP8 quantiser)."""
    cfg = synth.config("k2_tiny", T=12)
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    tr = moe.forward(x, W, top_k=1)
    assert np.all(tr.routing.gates == 1.0)
    xq = _torch_mxfp8(torch.from_numpy(x.astype(np.float64)))
    y = torch.zeros_like(xq)
    for t in range(x.shape[0]):
        e = int(tr.routing.ids[t, 0])
        wg = _torch_deq(W.w_gate_e[e].codes, W.w_gate_e[e].scales, "e2m1")
        wu = _torch_deq(W.w_up_e[e].codes, W.w_up_e[e].scales, "e2m1")
        wd = _torch_deq(W.w_down_e[e].codes, W.w_down_e[e].scales, "e2m1")
        a = xq[t:t + 1]
        h = torch.nn.functional.silu(a @ wg.T) * (a @ wu.T)
        y[t] = (_torch_mxfp8(h) @ wd.T)[0]
    wgs = _torch_deq(W.w_gate_s[0].codes, W.w_gate_s[0].scales, "e2m1")
    wus = _torch_deq(W.w_up_s[0].codes, W.w_up_s[0].scales, "e2m1")
    wds = _torch_deq(W.w_down_s[0].codes, W.w_down_s[0].scales, "e2m1")
    hs = torch.nn.functional.silu(xq @ wgs.T) * (xq @ wus.T)
    y = (y + _torch_mxfp8(hs) @ wds.T).numpy()
    assert np.abs(y - tr.y).max() <= 1e-9 * np.abs(tr.y).max()


def test_softmax_gates_ignore_the_selection_bias():
    """The selection bias moves the choice, never the gates: with the same
    winners, the gates are those of the raw logits."""
    r0, z, w = _random_route("softmax", 4)
    b = np.random.default_rng(9).standard_normal(w.shape[0]) * 0.5
    r1 = moe.route(z, w, 4, selection_bias=b, decide=None, gating="softmax")
    assert not np.array_equal(r0.ids, r1.ids)               # the bias changed some choices
    g = moe.winner_gates(z @ w.T, r1.ids, "softmax")
    assert np.allclose(r1.gates, g, rtol=1e-14, atol=0)
