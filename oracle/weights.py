"""Oracle-side MX weights for a seeded synthetic layer.

TEST INFRASTRUCTURE ONLY (part of the oracle).

The fp32 matrices come from ``synth`` (the shared seeded generator); the oracle
quantises them to MXFP4 itself with ``oracle.mx.quantize``.  Routed experts can
be produced lazily, one at a time, so a token sample at Kimi-K3 width never
needs all 896 experts in memory.
"""

from __future__ import annotations

import functools

import numpy as np

import synth
from . import moe


def _q(w: np.ndarray) -> moe.MXTensor:
    return moe.quant(w, "e2m1", decide=None)   # weights are fp32 already


def dense(cfg, name: str, idx: int = 0) -> moe.MXTensor:
    return _q(synth.gen_weight(cfg, name, idx))


def high(cfg, name: str, idx: int = 0):
    """A latent-projection or shared-expert weight: MXFP4, or bfloat16 under
    the higher-precision map (``cfg.precision == "bf16"``)."""
    if cfg.precision == "bf16":
        return moe.BF16Tensor(moe.mx.bf16_bits(synth.gen_weight(cfg, name, idx)))
    return dense(cfg, name, idx)


class ExpertCache:
    """Lazily quantised routed experts: ``cache(e) -> (w_gate, w_up, w_down)``."""

    def __init__(self, cfg, maxsize: int = 64):
        self.cfg = cfg
        self._get = functools.lru_cache(maxsize=maxsize)(self._build)

    def _build(self, e: int):
        return (dense(self.cfg, "w_gate_e", e), dense(self.cfg, "w_up_e", e),
                dense(self.cfg, "w_down_e", e))

    def __call__(self, e: int):
        return self._get(int(e))


def layer(cfg, experts: str = "all", selection_bias=None) -> moe.LayerWeights:
    """Oracle weights of the preset ``cfg``.

    ``experts="all"`` quantises every routed expert now (small presets);
    ``experts="lazy"`` leaves the routed lists empty (use ``ExpertCache``).
    """
    E, S = cfg.n_routed, cfg.n_shared
    if experts == "all":
        ge = [dense(cfg, "w_gate_e", e) for e in range(E)]
        ue = [dense(cfg, "w_up_e", e) for e in range(E)]
        de = [dense(cfg, "w_down_e", e) for e in range(E)]
    else:
        ge, ue, de = [], [], []
    return moe.LayerWeights(
        w_down=high(cfg, "w_down") if cfg.latent else None,
        w_up=high(cfg, "w_up") if cfg.latent else None,
        w_router=synth.gen_router(cfg),
        w_gate_e=ge, w_up_e=ue, w_down_e=de,
        w_gate_s=[high(cfg, "w_gate_s", s) for s in range(S)],
        w_up_s=[high(cfg, "w_up_s", s) for s in range(S)],
        w_down_s=[high(cfg, "w_down_s", s) for s in range(S)],
        logit_bias=synth.gen_logit_bias(cfg),
        selection_bias=selection_bias,
        gating=cfg.gating,
        precision=cfg.precision,
    )
