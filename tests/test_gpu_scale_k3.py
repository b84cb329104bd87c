"""Parity at the Kimi-K3 width on the benchmark workloads (gfx950 only).

The GPU runs the whole batch of each workload in the launch configuration the
benchmark times (64-token decode, 16384-token prefill, 8192 tokens with Zipf
expert popularity).  The batch-wide routing and dispatch are checked exactly
for every token; the full data path (codes, bounds, replay, output) is checked
against the fp64 oracle for a few sampled tokens, which the oracle can compute
one by one.
"""

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from oracle import weights
from tests import parity
from tests.gpu_harness import gpu_weights, run_traced_tokens, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SAMPLES = {"k3_decode": [0, 37], "k3_prefill": [5, 9000, 16383], "k3_skew": [1, 4097],
           "k3_decode_bf16": [0, 63], "k3_prefill_bf16": [7, 16383]}


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
    cache = weights.ExpertCache(base, maxsize=128)
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
    say(f"K3 parity {name}: T={cfg.T}, sampled tokens {tokens}")
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
    ysub, sub, full = run_traced_tokens(lay, x, tokens)
    lay.close()
    rep = parity.check_full_dispatch(full, cfg.n_routed, cfg.top_k)
    say("  batch:", rep)
    need = sorted(set(sub["ids"].reshape(-1).tolist()))
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(cache, need))
    rep2 = parity.check_tokens(cfg, Wc, x[tokens], ysub, sub, cache, say=say)
    return rep, rep2


def test_k3_decode_64_tokens(k3):
    _run(k3, "k3_decode")


def test_k3_prefill_16384_tokens(k3):
    _run(k3, "k3_prefill")


def test_k3_skewed_routing_8192_tokens(k3):
    rep, _ = _run(k3, "k3_skew")
    assert rep["max_expert_rows"] > 2 * rep["pairs"] / 896   # the Zipf bias does concentrate the load


def test_k3_bf16_map_decode_64_tokens(k3):
    """The higher-precision map at K3 width, 64 tokens (split-K bf16 GEMMs)."""
    _run(k3, "k3_decode_bf16")


def test_k3_bf16_map_prefill_16384_tokens(k3):
    """The higher-precision map at K3 width, 16384 tokens (LDS bf16 GEMMs)."""
    _run(k3, "k3_prefill_bf16")
