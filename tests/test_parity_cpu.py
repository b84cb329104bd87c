"""CPU checks of the parity machinery itself: a perturbed oracle run standing
in for the GPU must pass; planted mistakes must fail."""

import numpy as np
import pytest

import synth
from oracle import moe, mx, weights
from tests import parity


def _fake_trace(cfg, W, x, eps, seed=0):
    """Run the oracle with noise of up to 3 eps * sum|ab| injected into every
    matrix product (inside the bound of every GEMM for eps = 2.5e-7), and
    package it like the GPU trace."""
    rng = np.random.default_rng(seed)
    orig = moe.mm

    def noisy(a, b):
        r = orig(a, b)
        return r + eps * (np.abs(a.deq()) @ np.abs(b.deq()).T) * np.clip(rng.standard_normal(r.shape), -3, 3)

    moe.mm = noisy
    try:
        n = moe.forward(x, W, cfg.top_k)
    finally:
        moe.mm = orig
    f32 = lambda v: np.asarray(v).astype(np.float32)
    tr = {
        "z": f32(n.z), "zq_codes": n.zq.codes,
        "zq_scales": n.zq.scales, "ids": n.routing.ids, "gates": f32(n.routing.gates),
        "counts": n.disp.counts.astype(np.int32), "offsets": n.disp.offsets.astype(np.int32),
        "pair_of_row": n.disp.pair_of_row.astype(np.int32), "row_of_pair": n.disp.row_of_pair.astype(np.int32),
        "h": f32(n.h_rows), "hq_codes": n.hq_rows.codes, "hq_scales": n.hq_rows.scales, "y_e": f32(n.ye_rows),
        "y_lat": f32(n.y_lat), "hs": np.stack([f32(h) for h in n.h_shared]),
    }
    i16 = lambda b: np.asarray(b, np.uint16).view(np.int16)   # as the GPU trace holds bf16 patterns
    if isinstance(n.xq, moe.BF16Tensor):
        tr.update(xb=i16(n.xq.bits), yb=i16(n.yq.bits), hs_bf16=np.stack([i16(q.bits) for q in n.hq_shared]))
    else:
        tr.update(xq_codes=n.xq.codes, xq_scales=n.xq.scales, hs_codes=np.stack([q.codes for q in n.hq_shared]),
                  hs_scales=np.stack([q.scales for q in n.hq_shared]))
        if n.yq is not None:
            tr.update(yq_codes=n.yq.codes, yq_scales=n.yq.scales)
    return f32(n.y), tr


@pytest.fixture(scope="module")
def tiny_case():
    cfg = synth.config("tiny")
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    o = moe.forward(x, W, cfg.top_k)
    y, tr = _fake_trace(cfg, W, x, eps=2.5e-7)
    return cfg, W, x, o, y, tr


def test_perturbed_run_passes_and_adopts_boundary_choices(tiny_case):
    cfg, W, x, o, y, tr = tiny_case
    rep = parity.check_layer(cfg, W, o, y, tr, x=x, say=lambda *a: None)
    adopted = sum(v["adopted_blocks"] for v in rep["replay"].values())
    assert adopted > 0            # the noise does move codes across boundaries ...
    assert rep["replay_rel_l2"] < 1e-4   # ... and the replay follows them exactly


def test_planted_code_error_fails(tiny_case):
    cfg, W, x, o, y, tr = tiny_case
    bad = dict(tr)
    codes = tr["hq_codes"].copy()
    # the largest-magnitude element of row 0 is far from any boundary: change its code
    j = int(np.argmax(np.abs(o.h_rows[0])))
    codes[0, j] ^= 0x01
    bad["hq_codes"] = codes
    with pytest.raises(AssertionError):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


def test_planted_permutation_error_fails(tiny_case):
    cfg, W, x, o, y, tr = tiny_case
    bad = dict(tr)
    por = tr["pair_of_row"].copy()
    por[[0, 1]] = por[[1, 0]]
    bad["pair_of_row"] = por
    with pytest.raises(AssertionError, match="pair_of_row"):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


def test_planted_output_error_fails(tiny_case):
    cfg, W, x, o, y, tr = tiny_case
    y2 = y.copy()
    y2[3, 7] += 0.1 * np.abs(y).max()
    with pytest.raises(AssertionError):
        parity.check_layer(cfg, W, o, y2, tr, x=x, say=lambda *a: None)


# --------------------------------------------------------------------------- no latent, softmax gates


@pytest.fixture(scope="module")
def k2_case():
    cfg = synth.config("k2_tiny")
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    o = moe.forward(x, W, cfg.top_k)
    y, tr = _fake_trace(cfg, W, x, eps=2.5e-7, seed=1)
    return cfg, W, x, o, y, tr


def test_k2_perturbed_run_passes(k2_case):
    cfg, W, x, o, y, tr = k2_case
    assert W.w_down is None and W.gating == "softmax"
    rep = parity.check_layer(cfg, W, o, y, tr, x=x, say=lambda *a: None)
    assert "zq" not in rep["replay"] and "yq" not in rep["replay"]
    assert rep["replay_rel_l2"] < 1e-4


def test_k2_planted_gate_error_fails(k2_case):
    cfg, W, x, o, y, tr = k2_case
    bad = dict(tr)
    g = tr["gates"].copy()
    g[5, 0] += 1e-4                 # a softmax gate off by far more than its logits allow
    g[5, 1] -= 1e-4
    bad["gates"] = g
    with pytest.raises(AssertionError, match="gate"):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


def test_k2_sigmoid_gates_of_a_softmax_layer_fail(k2_case):
    """Gates normalised as sigmoid scores (the latent layer's rule) are caught."""
    cfg, W, x, o, y, tr = k2_case
    bad = dict(tr)
    s = 1 / (1 + np.exp(-o.routing.scores))
    bad["gates"] = moe.winner_gates(s, tr["ids"], "sigmoid").astype(np.float32)
    with pytest.raises(AssertionError, match="gate"):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


def test_k2_router_input_must_be_x(k2_case):
    cfg, W, x, o, y, tr = k2_case
    bad = dict(tr)
    z = tr["z"].copy()
    z[0, 0] = np.nextafter(z[0, 0], np.float32(np.inf))
    bad["z"] = z
    with pytest.raises(AssertionError, match="router input"):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


# --------------------------------------------------------------------------- higher-precision map


@pytest.fixture(scope="module")
def bf16_case():
    cfg = synth.config("tiny_bf16")
    W = weights.layer(cfg)
    x = synth.gen_hidden(cfg)
    o = moe.forward(x, W, cfg.top_k)
    y, tr = _fake_trace(cfg, W, x, eps=2.5e-7, seed=2)
    return cfg, W, x, o, y, tr


def test_bf16_map_perturbed_run_passes_and_adopts(bf16_case):
    cfg, W, x, o, y, tr = bf16_case
    rep = parity.check_layer(cfg, W, o, y, tr, x=x, say=lambda *a: None)
    assert "yb" in rep["replay"] and "hs0" in rep["replay"]
    adopted = sum(v["adopted_blocks"] for v in rep["replay"].values())
    assert adopted > 0
    assert rep["replay_rel_l2"] < 1e-4


def test_bf16_map_planted_rounding_error_fails(bf16_case):
    """A shared hidden value one bfloat16 step off, far from any boundary."""
    cfg, W, x, o, y, tr = bf16_case
    bad = dict(tr)
    hb = tr["hs_bf16"].copy()
    j = int(np.argmax(np.abs(o.h_shared[0][2])))
    hb[0, 2, j] += 1
    bad["hs_bf16"] = hb
    with pytest.raises(AssertionError):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


def test_bf16_map_truncated_input_fails(bf16_case):
    """bf16(x) by truncation instead of round-to-nearest is caught."""
    cfg, W, x, o, y, tr = bf16_case
    bad = dict(tr)
    bad["xb"] = (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
    with pytest.raises(AssertionError, match="bf16"):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


def test_requantisation_mismatch_fails(tiny_case):
    """A yq code that is not the MXFP8 of the traced fp32 y_lat (rule ii)."""
    cfg, W, x, o, y, tr = tiny_case
    bad = dict(tr)
    codes = tr["yq_codes"].copy()
    j = int(np.argmax(np.abs(tr["y_lat"][1])))
    codes[1, j] ^= 0x01
    bad["yq_codes"] = codes
    with pytest.raises(AssertionError, match="MXFP8"):
        parity.check_layer(cfg, W, o, y, bad, x=x, say=lambda *a: None)


def test_max_abs_against_the_oracle_is_enforced(tiny_case):
    """One output element of a token with no quantiser near-tie off by 6% of
    rms: relative L2 stays small, the max-abs limit against the unconditioned
    oracle catches it."""
    cfg, W, x, o, y, tr = tiny_case
    same = np.all(np.sort(tr["ids"], 1) == np.sort(o.routing.ids, 1), 1)
    clean = np.where(parity.codes_equal_oracle(W, o, tr, cfg.top_k, same))[0]
    assert len(clean) > 10        # most tokens take no boundary choice at this noise level
    y2 = y.copy()
    rms = np.sqrt((o.y ** 2).mean())
    y2[clean[3], 3] += 0.06 * rms
    with pytest.raises(AssertionError, match="max abs"):
        parity.check_layer(cfg, W, o, y2, tr, x=None, say=lambda *a: None)
