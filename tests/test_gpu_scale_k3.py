"""Parity at the Kimi-K3 width on the benchmark workloads (gfx950 only).

The GPU runs the whole batch of each workload in the launch configuration the
benchmark times (64-token decode, 16384-token prefill, 8192 tokens with Zipf
expert popularity).  For EVERY token of every batch the routing is checked
against the oracle's own latent and router, computed for the whole batch: x
codes, the latent z within its bound, zq re-quantised bit for bit (and against
the oracle's own zq outside ambiguous blocks), the expert ids as sets (near-
ties flagged), gates and the dispatch.  The complete data path (expert FFNs,
combine, up-projection, shared experts, output) is checked against the fp64
oracle for every token of the 64-token decode batch, and for sampled tokens of
the large batches (a pair's GPU row does not depend on the other tokens, so a
token subset's rows are re-laid into the subset's own dispatch order).
"""

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from oracle import weights
from tests import parity
from tests.gpu_harness import gpu_weights, run_traced, run_traced_tokens, say, token_subset

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Sampled tokens of the large batches (full data path); "all" = every token.
SAMPLES = {"k3_decode": "all", "k3_prefill": [5, 9000, 16383], "k3_skew": [1, 4097],
           "k3_decode_bf16": [0, 63], "k3_prefill_bf16": [7, 16383]}
WORKERS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module")
def k3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_routing_mxfp4_amd import layer as LY
    base = synth.config("k3_prefill")
    say("K3: encoding all weights on the GPU")
    shape, gw = gpu_weights(base, workers=16)
    say("K3: oracle dense weights")
    W = weights.layer(base, experts="lazy")
    cache = weights.ExpertCache(base, maxsize=1024)
    yield LY, shape, gw, W, cache
    del gw


def _bf16_dense(LY, cfg):
    """The higher-precision map's bfloat16 latent projections and shared
    experts, rounded on the GPU by the library from the same fp32 weights."""
    shape = LY.LayerShape.of(cfg)
    return LY.encode_weights(shape, lambda n, i: synth.gen_weight(cfg, n, i), names=LY.DENSE + LY.SHARED)


def _run(k3, name):
    LY, shape, gw, W, cache = k3
    cfg = synth.config(name)
    tokens = SAMPLES[name]
    say(f"K3 parity {name}: T={cfg.T}, full data path on {tokens if tokens != 'all' else 'every'} token(s)")
    w = dict(gw)
    Wc = W
    if cfg.precision == "bf16":   # same routed experts, bfloat16 dense weights
        shape = LY.LayerShape.of(cfg)
        w.update(_bf16_dense(LY, cfg))
        Wc = weights.layer(cfg, experts="lazy")
    if cfg.logit_bias != "none":   # same weights, different router logit bias
        lb = synth.gen_logit_bias(cfg)
        w["router_logit_bias"] = torch.from_numpy(lb).cuda()
        Wc = dataclasses.replace(W, logit_bias=lb)
    lay = LY.LatentMoE(shape, w, cfg.T)
    x = synth.gen_hidden(cfg)
    if tokens == "all":
        y, full = run_traced(lay, x)
        tokens = list(range(cfg.T))
    else:
        y, sub, full = run_traced_tokens(lay, x, tokens)
    lay.close()
    say("  every token's routing against the oracle")
    rep = parity.check_batch_routing(cfg, Wc, x, full, workers=WORKERS, say=say)
    k = cfg.top_k
    if len(tokens) == cfg.T:   # every token: subsets of 4, checked in parallel
        chunks = [tokens[i:i + 4] for i in range(0, len(tokens), 4)]
        subs = [(c, token_subset(full, c, k), y[c]) for c in chunks]
    else:
        subs = [(tokens, sub, y)]
    need = sorted({int(e) for _, s, _ in subs for e in s["ids"].reshape(-1)})
    say(f"  oracle experts: {len(need)}")
    with ThreadPoolExecutor(max_workers=WORKERS) as ex:
        for i, _ in enumerate(ex.map(cache, need)):
            if (i + 1) % 64 == 0:
                say(f"    {i + 1} of {len(need)} experts encoded by the oracle")
    say(f"  full data path of {len(tokens)} token(s) in {len(subs)} subset(s)")

    def check(i):
        tok, sub, ys = subs[i]
        # each subset's stage lines, not its full report
        quiet = lambda *a: None if str(a[0]).startswith("parity report") else say(f"    subset {i}:", *a)
        return parity.check_tokens(cfg, Wc, x[tok], ys, sub, cache, say=quiet)

    with ThreadPoolExecutor(max_workers=WORKERS) as ex:
        reps = []
        for r in ex.map(check, range(len(subs))):
            reps.append(r)
            say(f"    subset {len(reps) - 1} of {len(subs)} checked")
    merged = parity.merge_reports(reps)
    # figures over all the checked tokens together (rms of the oracle's output
    # over them): relative L2, and max-abs per token, where a token above the
    # limit must have taken a quantiser near-tie (then it is held to the replay)
    yg = np.concatenate([r["_y"][0] for r in reps])
    yo = np.concatenate([r["_y"][1] for r in reps])
    clean = np.concatenate([r["_y"][2] for r in reps])
    rms = float(np.sqrt((yo ** 2).mean()))
    rel, maxabs, _ = parity.output_errors(yg, yo, rms)
    dev = np.abs(yg - yo).max(axis=1)
    over = dev > parity.MAXABS_FRAC * rms
    merged.update(batch_rel_l2=rel, batch_max_abs_over_rms=maxabs / rms,
                  batch_tokens_excused_over_max_abs=int((over & ~clean).sum()))
    say("  data path:", merged)
    assert rel <= parity.REL_L2 and not np.any(over & clean)
    return rep, merged


def test_k3_decode_64_tokens(k3):
    """All 64 tokens: routing and the full data path."""
    _, merged = _run(k3, "k3_decode")
    assert merged["tokens_vs_oracle"] + merged["ids_differ_flagged"] == 64


def test_k3_prefill_16384_tokens(k3):
    rep, _ = _run(k3, "k3_prefill")
    assert rep["tokens_routed"] == 16384


def test_k3_skewed_routing_8192_tokens(k3):
    rep, _ = _run(k3, "k3_skew")
    assert rep["max_expert_rows"] > 2 * 8192 * 16 / 896   # the Zipf bias does concentrate the load


def test_k3_bf16_map_decode_64_tokens(k3):
    """The higher-precision map at K3 width, 64 tokens (split-K bf16 GEMMs)."""
    _run(k3, "k3_decode_bf16")


def test_k3_bf16_map_prefill_16384_tokens(k3):
    """The higher-precision map at K3 width, 16384 tokens (LDS bf16 GEMMs)."""
    _run(k3, "k3_prefill_bf16")


def test_k3_row_major_weights_bitwise(k3):
    """The K3-width weights handed over row-major give bit for bit the
    fragment-order forward, at the decode and prefill batch sizes (the
    weight-streaming, K-split and LDS-staged kernels)."""
    LY, shape, gw, W, cache = k3
    from latent_routing_mxfp4_amd import _lib
    base = synth.config("k3_prefill")
    say("K3: encoding all weights row-major on the GPU")
    rshape, gr = gpu_weights(base, workers=16, weight_layout=_lib.MOE_WEIGHTS_ROW_MAJOR)
    for name in ("k3_decode", "k3_prefill"):
        cfg = synth.config(name)
        say(f"  {name}: T={cfg.T}, row-major against fragment order")
        x = torch.from_numpy(synth.gen_hidden(cfg)).cuda()
        outs = []
        for sh, w in ((shape, gw), (rshape, gr)):
            lay = LY.LatentMoE(sh, w, cfg.T)
            outs.append(lay.forward(x).cpu())
            torch.cuda.synchronize()
            lay.close()
        assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32)), name
    del gr
    torch.cuda.empty_cache()
