"""GPU-side helpers for the parity tests: build a seeded layer on the device
through the HIP library and run it with a full trace."""

from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from latent_routing_mxfp4_amd import layer as LY


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_weights(cfg, selection_bias=None, workers=8, weight_layout=None):
    shape = LY.LayerShape.of(cfg) if weight_layout is None else LY.LayerShape.of(cfg, weight_layout)
    extra = {"w_router": synth.gen_router(cfg), "router_logit_bias": synth.gen_logit_bias(cfg),
             "selection_bias": selection_bias}
    return shape, LY.encode_weights(shape, lambda n, i: synth.gen_weight(cfg, n, i), extra=extra, workers=workers,
                                    progress=lambda j, n: say(f"    {j} of {n} weight matrices encoded"))


def gpu_layer(cfg, max_tokens=None, selection_bias=None, weights=None, weight_layout=None):
    if weights is None:
        shape, weights = gpu_weights(cfg, selection_bias, weight_layout=weight_layout)
    else:
        shape = LY.LayerShape.of(cfg) if weight_layout is None else LY.LayerShape.of(cfg, weight_layout)
    return LY.LatentMoE(shape, weights, max_tokens or cfg.T), weights


def run_traced(layer, x_np: np.ndarray):
    T = x_np.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
    tr = layer.trace_buffers(T)
    y = layer.forward(x, trace=tr)
    torch.cuda.synchronize()
    return y.cpu().numpy(), {k: v.cpu().numpy() for k, v in tr.items()}


def to_np(t):
    return t.detach().cpu().numpy()


PER_TOKEN = ("xq_codes", "xq_scales", "z", "zq_codes", "zq_scales", "logits", "ids", "gates", "y_lat",
             "yq_codes", "yq_scales", "xb", "yb")
PER_ROW = ("h", "hq_codes", "hq_scales", "y_e")


def run_traced_tokens(layer, x_np: np.ndarray, tokens):
    """Run the whole batch with a full trace, but bring back only what the
    sampled ``tokens`` need: their per-token rows, the per-row (sorted) trace
    rows of their k pairs in (token, slot) order, and the batch-wide routing
    and dispatch arrays.  Returns (y[tokens], sub, full)."""
    T = x_np.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
    tr = layer.trace_buffers(T)
    y = layer.forward(x, trace=tr)
    torch.cuda.synchronize()
    tok = torch.as_tensor(np.asarray(tokens, np.int64), device="cuda")
    k = tr["ids"].shape[1]
    pairs = (tok[:, None] * k + torch.arange(k, device="cuda")[None, :]).reshape(-1)
    rows = tr["row_of_pair"].long()[pairs]
    sub = {n: to_np(tr[n][tok]) for n in PER_TOKEN if n in tr}
    sub.update({n: to_np(tr[n][rows]) for n in PER_ROW})
    for n in ("hs", "hs_codes", "hs_scales", "hs_bf16"):
        if n in tr:
            sub[n] = to_np(tr[n][:, tok])
    full = {n: to_np(tr[n]) for n in ("ids", "gates", "counts", "offsets", "pair_of_row", "row_of_pair", "z",
                                      "zq_codes", "zq_scales", "xq_codes", "xq_scales", "xb") if n in tr}
    ysub = to_np(y[tok])
    del tr, y, x
    torch.cuda.empty_cache()
    return ysub, sub, full


def token_subset(tr: dict, tokens, k: int) -> dict:
    """From a whole-batch numpy trace: the sampled tokens' per-token rows, the
    per-row (sorted) rows of their k pairs in (token, slot) order, and their
    shared hidden states -- the layout ``tests.parity.check_tokens`` takes."""
    tok = np.asarray(tokens, np.int64)
    pairs = (tok[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    rows = np.asarray(tr["row_of_pair"], np.int64)[pairs]
    sub = {n: tr[n][tok] for n in PER_TOKEN if n in tr}
    sub.update({n: tr[n][rows] for n in PER_ROW})
    for n in ("hs", "hs_codes", "hs_scales", "hs_bf16"):
        if n in tr:
            sub[n] = tr[n][:, tok]
    return sub
