"""Workload presets and seeded generators for the LatentMoE layer inputs.

Every tensor is drawn from numpy's PCG64 keyed by a ``SeedSequence`` of
``(seed, tensor_id, expert)``, so any single expert's matrix can be regenerated
on its own (random access), which lets the oracle check a sampled token at the
full Kimi-K3 width without materialising all 896 experts at once.

Shapes follow the layer as the pages describe it:

* Kimi K3 and the New Open-Weights Moat, "Sparse computation: latent experts
  and routing": model width 7,168, a 3,584-d routed latent, 896 routed experts
  of which a token uses 16, and two always-on shared experts at full width.
* Kimi K3: 2.8 Trillion Parameters, Four Bits at a Time, "What it takes to
  serve it" (the MoE data-path toy): per-expert matrices applied to token rows.

The expert intermediate width 3,072 is an estimate; the pages give none.

Weights are produced in the nn.Linear orientation ``[out][in]`` so that the
MX blocks of 32 run along the contraction (input) dimension.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int               # tokens in the batch
    d_model: int         # model width
    d_latent: int        # routed latent width
    n_routed: int        # routed experts
    top_k: int           # experts kept per token
    n_shared: int        # always-on shared experts (full width)
    d_ff_shared: int     # shared-expert intermediate width
    d_ff_routed: int     # routed-expert intermediate width
    router_init: str     # "normal" (std 1/sqrt(d_latent)) or "uniform" (+-1/sqrt(d_latent))
    logit_bias: str      # "none" or "zipf" (per-expert popularity bias on the router logits)
    seed_x: int          # seed of the hidden states
    seed_w: int          # seed of every weight tensor
    latent: bool = True          # False: no latent projections (routed width = model width)
    gating: str = "sigmoid"      # "sigmoid": winners' sigmoid scores / their sum;
                                 # "softmax": softmax over the winners' logits
    precision: str = "mx"        # "mx": every weight but the router MXFP4;
                                 # "bf16": latent projections and shared experts bfloat16

    def with_tokens(self, T: int) -> "LayerConfig":
        return dataclasses.replace(self, T=int(T))


# Tensor ids inside a seed; fixed forever so stored expectations stay valid.
_TID = {
    "x": 1,
    "w_down": 2,      # [d_latent][d_model]   latent down-projection
    "w_up": 3,        # [d_model][d_latent]   latent up-projection
    "w_router": 4,    # [n_routed][d_latent]  fp32 router
    "w_gate_e": 5,    # [E][F][L]
    "w_up_e": 6,      # [E][F][L]
    "w_down_e": 7,    # [E][L][F]
    "w_gate_s": 8,    # [S][Fs][d]
    "w_up_s": 9,      # [S][Fs][d]
    "w_down_s": 10,   # [S][d][Fs]
    "logit_bias": 11,
    "selection_bias": 12,
    "skew_rank": 13,
}

WEIGHT_NAMES = ("w_down", "w_up", "w_gate_e", "w_up_e", "w_down_e",
                "w_gate_s", "w_up_s", "w_down_s")


CONFIGS = {
    # Tiny LatentMoE forward: small enough for pure-Python checks.
    "tiny": LayerConfig("tiny", T=64, d_model=256, d_latent=128, n_routed=32, top_k=4,
                        n_shared=1, d_ff_shared=256, d_ff_routed=128,
                        router_init="normal", logit_bias="none", seed_x=1001, seed_w=1001),
    # Mid-size forward: several GEMM tiles in every dimension.
    "mid": LayerConfig("mid", T=4096, d_model=2048, d_latent=1024, n_routed=128, top_k=8,
                       n_shared=2, d_ff_shared=2048, d_ff_routed=768,
                       router_init="uniform", logit_bias="none", seed_x=1002, seed_w=1002),
    # Kimi-K3 width, 64-token decode batch (weight-read bound).
    "k3_decode": LayerConfig("k3_decode", T=64, d_model=7168, d_latent=3584, n_routed=896,
                             top_k=16, n_shared=2, d_ff_shared=3072, d_ff_routed=3072,
                             router_init="normal", logit_bias="none", seed_x=1003, seed_w=1003),
    # Kimi-K3 width, 16384-token prefill batch (matrix-core bound).
    "k3_prefill": LayerConfig("k3_prefill", T=16384, d_model=7168, d_latent=3584, n_routed=896,
                              top_k=16, n_shared=2, d_ff_shared=3072, d_ff_routed=3072,
                              router_init="normal", logit_bias="none", seed_x=1004, seed_w=1003),
    # Kimi-K3 width, 8192 tokens with Zipf(1.1) expert popularity on the logits.
    "k3_skew": LayerConfig("k3_skew", T=8192, d_model=7168, d_latent=3584, n_routed=896,
                           top_k=16, n_shared=2, d_ff_shared=3072, d_ff_routed=3072,
                           router_init="normal", logit_bias="zipf", seed_x=1005, seed_w=1003),
    # Non-latent MoE at K2-like width (384 experts, top-8, one shared expert):
    # the experts read the model-width activations, the router the fp32 input,
    # and the gates are the softmax over the winners' logits.
    "k2_tiny": LayerConfig("k2_tiny", T=64, d_model=256, d_latent=256, n_routed=48, top_k=4,
                           n_shared=1, d_ff_shared=256, d_ff_routed=128, router_init="normal",
                           logit_bias="none", seed_x=1006, seed_w=1006, latent=False, gating="softmax"),
    # The Moat page's precision map on the K3 layers: bfloat16 latent
    # projections and shared experts, MXFP4 routed experts (same seeds, so the
    # same fp32 weights as the MX presets).
    "tiny_bf16": LayerConfig("tiny_bf16", T=64, d_model=256, d_latent=128, n_routed=32, top_k=4,
                             n_shared=1, d_ff_shared=256, d_ff_routed=128,
                             router_init="normal", logit_bias="none", seed_x=1001, seed_w=1001, precision="bf16"),
    "k3_decode_bf16": LayerConfig("k3_decode_bf16", T=64, d_model=7168, d_latent=3584, n_routed=896,
                                  top_k=16, n_shared=2, d_ff_shared=3072, d_ff_routed=3072,
                                  router_init="normal", logit_bias="none", seed_x=1003, seed_w=1003,
                                  precision="bf16"),
    "k3_prefill_bf16": LayerConfig("k3_prefill_bf16", T=16384, d_model=7168, d_latent=3584, n_routed=896,
                                   top_k=16, n_shared=2, d_ff_shared=3072, d_ff_routed=3072,
                                   router_init="normal", logit_bias="none", seed_x=1004, seed_w=1003,
                                   precision="bf16"),
    # One GPU's share of an 8-way expert-parallel K3 decode step: 112 local
    # experts (the first 112 of the K3 set, same seeds) receiving 1024 token
    # copies, about 9 rows each; the latent projections, router and shared
    # experts run on the GPU's own 64 tokens.  The exchange is not modelled.
    "k3_ep8_share": LayerConfig("k3_ep8_share", T=64, d_model=7168, d_latent=3584, n_routed=112,
                                top_k=16, n_shared=2, d_ff_shared=3072, d_ff_routed=3072,
                                router_init="normal", logit_bias="none", seed_x=1003, seed_w=1003),
    "k2_prefill": LayerConfig("k2_prefill", T=8192, d_model=7168, d_latent=7168, n_routed=384, top_k=8,
                              n_shared=1, d_ff_shared=2048, d_ff_routed=2048, router_init="normal",
                              logit_bias="none", seed_x=1007, seed_w=1007, latent=False, gating="softmax"),
}


def config(name: str, T: Optional[int] = None) -> LayerConfig:
    cfg = CONFIGS[name]
    return cfg if T is None else cfg.with_tokens(T)


def _rng(seed: int, tensor: str, expert: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), _TID[tensor], int(expert)])
    return np.random.Generator(np.random.PCG64(ss))


def weight_shape(cfg: LayerConfig, name: str) -> tuple:
    """Shape of ONE matrix of a weight group ([out][in], in = contraction dim)."""
    d, L, F, Fs = cfg.d_model, cfg.d_latent, cfg.d_ff_routed, cfg.d_ff_shared
    return {
        "w_down": (L, d),
        "w_up": (d, L),
        "w_gate_e": (F, L),
        "w_up_e": (F, L),
        "w_down_e": (L, F),
        "w_gate_s": (Fs, d),
        "w_up_s": (Fs, d),
        "w_down_s": (d, Fs),
    }[name]


def n_matrices(cfg: LayerConfig, name: str) -> int:
    if name.endswith("_e"):
        return cfg.n_routed
    if name.endswith("_s"):
        return cfg.n_shared
    return 1 if cfg.latent else 0   # the latent projections exist only with a latent


def gen_weight(cfg: LayerConfig, name: str, expert: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 weight matrix ``[out][in]`` drawn from N(0, 1/sqrt(in))."""
    shape = weight_shape(cfg, name)
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    assert out.shape == shape and out.dtype == np.float32
    _rng(cfg.seed_w, name, expert).standard_normal(out=out, dtype=np.float32)
    out *= np.float32(1.0 / math.sqrt(shape[1]))
    return out


def gen_hidden(cfg: LayerConfig, T: Optional[int] = None, start: int = 0) -> np.ndarray:
    """Hidden states x ~ N(0, 1), fp32 ``[T][d_model]``.

    Rows are generated in fixed chunks of 256 tokens keyed by the chunk index, so
    a token's row is the same whatever ``T`` or ``start`` a caller asks for.
    """
    T = cfg.T if T is None else int(T)
    d = cfg.d_model
    out = np.empty((T, d), dtype=np.float32)
    chunk = 256
    t = 0
    while t < T:
        gt = start + t
        c = gt // chunk
        lo = gt - c * chunk
        n = min(chunk - lo, T - t)
        block = _rng(cfg.seed_x, "x", c).standard_normal((chunk, d), dtype=np.float32)
        out[t:t + n] = block[lo:lo + n]
        t += n
    return out


def gen_router(cfg: LayerConfig) -> np.ndarray:
    """fp32 router weights ``[n_routed][d_latent]`` (not quantised)."""
    E, L = cfg.n_routed, cfg.d_latent
    g = _rng(cfg.seed_w, "w_router")
    if cfg.router_init == "normal":
        w = g.standard_normal((E, L), dtype=np.float32)
        w *= np.float32(1.0 / math.sqrt(L))
    elif cfg.router_init == "uniform":
        a = 1.0 / math.sqrt(L)
        w = g.uniform(-a, a, size=(E, L)).astype(np.float32)
    else:
        raise ValueError(cfg.router_init)
    return w


def gen_logit_bias(cfg: LayerConfig) -> Optional[np.ndarray]:
    """Per-expert bias added to the router logits, or None.

    "zipf": experts get a seeded popularity rank r (1 = most popular); the rank's
    Zipf(s=1.1) probability p_r = r^-1.1 / sum_{q<=E} q^-1.1 becomes the logit
    bias ln(E * p_r), so a uniform expert would get 0.
    """
    if cfg.logit_bias == "none":
        return None
    if cfg.logit_bias != "zipf":
        raise ValueError(cfg.logit_bias)
    E = cfg.n_routed
    perm = _rng(cfg.seed_w, "skew_rank").permutation(E)      # perm[e] = rank-1 of expert e
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** -1.1
    p /= p.sum()
    return np.log(E * p[perm]).astype(np.float32)


def gen_selection_bias(cfg: LayerConfig, std: float = 0.05) -> np.ndarray:
    """A nonzero per-expert selection bias (used only by tests; the presets use none)."""
    return (_rng(cfg.seed_w, "selection_bias").standard_normal(cfg.n_routed) * std).astype(np.float32)
