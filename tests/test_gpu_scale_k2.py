"""Parity at K2-like width without a latent (gfx950 only).

The 8192-token batch of the non-latent layer (7168 wide, 384 experts, top-8,
softmax-over-winners gates, one shared expert) runs whole on the GPU in the
configuration the benchmark times.  Every token's routing (router input,
ids as sets with near-ties flagged, gates, dispatch) is checked against the
oracle's router on the whole batch; the full data path of a few sampled tokens
against the fp64 oracle.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import pytest

import synth
from oracle import weights
from tests import parity
from tests.gpu_harness import gpu_weights, run_traced_tokens, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_k2_prefill_8192_tokens():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_routing_mxfp4_amd import layer as LY
    cfg = synth.config("k2_prefill")
    tokens = [3, 4100, 8191]
    say(f"K2 parity {cfg.name}: T={cfg.T}, sampled tokens {tokens}; encoding all weights on the GPU")
    shape, gw = gpu_weights(cfg, workers=16)
    assert gw["w_down"] is None and gw["w_up"] is None
    lay = LY.LatentMoE(shape, gw, cfg.T)
    x = synth.gen_hidden(cfg)
    ysub, sub, full = run_traced_tokens(lay, x, tokens)
    lay.close()
    del gw
    torch.cuda.empty_cache()
    W = weights.layer(cfg, experts="lazy")
    rep = parity.check_batch_routing(cfg, W, x, full, workers=min(16, len(os.sched_getaffinity(0))), say=say)
    assert rep["tokens_routed"] == cfg.T
    cache = weights.ExpertCache(cfg, maxsize=64)
    need = sorted(set(sub["ids"].reshape(-1).tolist()))
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(cache, need))
    parity.check_tokens(cfg, W, x[tokens], ysub, sub, cache, say=say)
