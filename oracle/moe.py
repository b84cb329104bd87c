"""The LatentMoE layer forward, step by step, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (part of the oracle; see ``oracle/__init__``).

The steps follow the pages in their order:

1. ``xq = MXFP8(x)`` per token row, blocks of 32 along the features
   (Kimi K3 and the New Open-Weights Moat, "Precision and deployment":
   the inputs of the MXFP4 GEMMs are MXFP8).
2. Latent down-projection ``z = deq(xq) @ deq(W_down)^T`` to the routed latent
   width (same page, "Sparse computation: latent experts and routing").
3. Router: a sigmoid score for every routed expert, computed on the latent
   (same page, "How the router picks 16 of 896", Fig. 2; Kimi K3: 2.8 Trillion
   Parameters, Four Bits at a Time, "The shape of the model": routing happens in
   a latent space).  The router weight is fp32 and not quantised.
4. Selection: top-k of score + per-expert selection bias; ties go to the
   lower expert id; slots are ordered by descending selection key.
5. Gates: the k winners' raw sigmoid scores divided by their sum (the
   selection bias is not part of the gates).
6. Dispatch: flatten the (token, slot) pairs token-major and stable-sort them
   by expert; counts per expert and their exclusive prefix sum give each
   expert's segment (Four Bits at a Time, "What it takes to serve it", the MoE
   data-path toy).
7. Per expert, on its segment rows: ``G = zq W_gate^T``, ``U = zq W_up^T``,
   ``h = SiLU(G) * U``, ``hq = MXFP8(h)``, ``y_e = deq(hq) @ deq(W_down_e)^T``.
8. Combine: ``y_lat[t] = sum_j gate[t, j] * y_e[row(t, j)]`` (the toy's
   gate-weighted scatter-add back to token order).
9. Up-projection of the combined latent back to model width
   (``yq = MXFP8(y_lat)``, ``y_up = deq(yq) @ deq(W_up)^T``).
10. Shared experts at full width on ``xq``, summed with the routed branch
    (Moat page, "How the router picks 16 of 896": both branches are summed).

A non-latent layer (``W.w_down is None``; the second workload, a K2-shaped
MoE) skips steps 2 and 9: the router reads the fp32 input, the experts read
``xq`` at model width, and the combined routed output is summed with the
shared experts as is.  With ``W.gating == "softmax"`` the selection key is the
logit (plus the selection bias) and the gates are the softmax over the k
winners' logits, the gate of the MoE data-path toy (Four Bits at a Time,
"What it takes to serve it").

Precision map.  ``W.precision == "mx"``: every weight but the fp32 router is
MXFP4 and each MX GEMM reads MXFP8 activations (the workload's own statement).
``"bf16"``: the Moat page's map ("Precision and deployment", Fig. 6) -- only
the routed experts are MXFP4 x MXFP8; the latent projections and the shared
experts keep higher-precision weights, taken as bfloat16, and their GEMMs read
bfloat16 activations: ``xb = bf16(x)`` feeds W_down and the shared gate/up
projections, the shared hidden state is ``bf16(h)``, and the up-projection
reads ``bf16(y_lat)``.  Products are exact in fp64 either way.

Decision precision.  Where a float decides an integer (an MX code, a
bfloat16 rounding, the top-k order), the oracle first rounds its fp64 value to
fp32, the precision the GPU path decides in (``decide=np.float32``);
``decide=None`` keeps pure fp64.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import mx


# --------------------------------------------------------------------------- containers


@dataclasses.dataclass
class MXTensor:
    codes: np.ndarray    # uint8, one code per element (unpacked), [..., K]
    scales: np.ndarray   # uint8, [..., K/32]
    fmt: str

    def deq(self) -> np.ndarray:
        return mx.dequantize(self.codes, self.scales, self.fmt)

    def __getitem__(self, idx) -> "MXTensor":
        return MXTensor(self.codes[idx], self.scales[idx], self.fmt)


@dataclasses.dataclass
class BF16Tensor:
    bits: np.ndarray     # uint16 bfloat16 patterns, [..., K]
    fmt: str = "bf16"

    def deq(self) -> np.ndarray:
        return mx.bf16_value(self.bits)

    def __getitem__(self, idx) -> "BF16Tensor":
        return BF16Tensor(self.bits[idx])


def quant(v, fmt="e4m3", decide=np.float32):
    """MX-encode ``v`` along its last axis, or round it to bfloat16 (``fmt="bf16"``);
    with ``decide`` the fp64 value is first rounded to that type."""
    if decide is not None:
        v = np.asarray(v).astype(decide)
    if fmt == "bf16":
        return BF16Tensor(mx.bf16_bits(v))
    c, s = mx.quantize(v, fmt)
    return MXTensor(c, s, fmt)


def mm(a, b) -> np.ndarray:
    """deq(a) @ deq(b)^T in fp64 (MX x MX through the MX matmul; a bfloat16
    operand makes every product exact in fp64)."""
    if isinstance(a, MXTensor) and isinstance(b, MXTensor):
        return mx.mx_matmul(a.codes, a.scales, a.fmt, b.codes, b.scales, b.fmt)
    return a.deq() @ b.deq().T


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-np.asarray(v, dtype=np.float64)))


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v * sigmoid(v)


@dataclasses.dataclass
class LayerWeights:
    """MX weights of one layer (oracle-side codes), fp32 router and biases."""
    w_down: Optional[MXTensor]        # [L][d]; None: no latent (L = d)
    w_up: Optional[MXTensor]          # [d][L]; None with w_down
    w_router: np.ndarray              # fp32 [E][L]
    w_gate_e: list                    # E x MXTensor [F][L]   (entries may be filled lazily)
    w_up_e: list                      # E x MXTensor [F][L]
    w_down_e: list                    # E x MXTensor [L][F]
    w_gate_s: list                    # S x MXTensor [Fs][d]
    w_up_s: list                      # S x MXTensor [Fs][d]
    w_down_s: list                    # S x MXTensor [d][Fs]
    logit_bias: Optional[np.ndarray] = None       # fp32 [E] or None
    selection_bias: Optional[np.ndarray] = None   # fp32 [E] or None
    gating: str = "sigmoid"                       # or "softmax" (over the winners' logits)
    precision: str = "mx"                         # or "bf16": latent projections + shared experts


# --------------------------------------------------------------------------- routing


@dataclasses.dataclass
class Routing:
    scores: np.ndarray     # [T][E] sigmoid scores (fp64); the logits with softmax gating
    sel: np.ndarray        # [T][E] selection keys
    ids: np.ndarray        # [T][k] int32, slot order = descending key, ties -> lower id
    gates: np.ndarray      # [T][k] fp64, sums to 1 per token
    gap: np.ndarray        # [T] key(k-th) - key(k+1-th); +inf when k == E


def winner_gates(scores: np.ndarray, ids: np.ndarray, gating: str = "sigmoid") -> np.ndarray:
    """Gates of the selected experts: sigmoid scores over their sum (Moat page,
    Fig. 2), or the softmax over the winners' logits (the MoE data-path toy)."""
    win = np.take_along_axis(scores, ids, axis=1)
    if gating == "softmax":
        e = np.exp(win - win.max(axis=1, keepdims=True))
        return e / e.sum(axis=1, keepdims=True)
    if gating != "sigmoid":
        raise ValueError(gating)
    return win / win.sum(axis=1, keepdims=True)


def route(z: np.ndarray, w_router: np.ndarray, k: int, logit_bias=None, selection_bias=None,
          decide=np.float32, gating: str = "sigmoid") -> Routing:
    """Sigmoid router on the latent and top-k selection (Moat page, Fig. 2).
    With ``gating="softmax"`` the keys are the logits themselves (a monotone
    change of the sigmoid's order) and the gates the softmax of the winners'."""
    z = np.asarray(z, dtype=np.float64)
    if decide is not None:
        z = z.astype(decide).astype(np.float64)   # the router reads the fp32 latent
    logits = z @ np.asarray(w_router, dtype=np.float64).T
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, dtype=np.float64)[None, :]
    if decide is not None:
        logits = logits.astype(decide).astype(np.float64)
    s = sigmoid(logits) if gating == "sigmoid" else logits
    if decide is not None:
        s = s.astype(decide).astype(np.float64)
    sel = s if selection_bias is None else s + np.asarray(selection_bias, dtype=np.float64)[None, :]
    if decide is not None:
        sel = sel.astype(decide).astype(np.float64)
    T, E = sel.shape
    ids = np.empty((T, k), dtype=np.int32)
    gap = np.full(T, np.inf)
    eidx = np.arange(E)
    for t in range(T):
        order = np.lexsort((eidx, -sel[t]))    # primary: descending key; secondary: ascending id
        ids[t] = order[:k]
        if k < E:
            gap[t] = sel[t, order[k - 1]] - sel[t, order[k]]
    gates = winner_gates(s, ids, gating)
    return Routing(scores=s, sel=sel, ids=ids, gates=gates, gap=gap)


@dataclasses.dataclass
class Dispatch:
    counts: np.ndarray       # [E] int64
    offsets: np.ndarray      # [E+1] int64, exclusive prefix sum
    pair_of_row: np.ndarray  # [T*k] flat pair index (t*k + j) held by each sorted row
    row_of_pair: np.ndarray  # [T*k] sorted row of each flat pair


def dispatch(ids: np.ndarray, n_experts: int) -> Dispatch:
    """Token-major flattening, then a stable sort by expert (the toy's permutation)."""
    flat = np.asarray(ids).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    row_of = np.empty_like(order)
    row_of[order] = np.arange(order.size)
    return Dispatch(counts, offsets, order.astype(np.int64), row_of.astype(np.int64))


# --------------------------------------------------------------------------- experts


def swiglu_expert(aq, wg, wu, wd, decide=np.float32, full=False, hfmt="e4m3"):
    """down(SiLU(gate a) * (up a)) with the hidden h re-encoded in ``hfmt``
    (MXFP8, or bfloat16 for a higher-precision expert).

    Returns (y, h, hq), plus (g, u) when ``full``.
    """
    g = mm(aq, wg)
    u = mm(aq, wu)
    h = silu(g) * u
    hq = quant(h, hfmt, decide)
    if full:
        return mm(hq, wd), h, hq, g, u
    return mm(hq, wd), h, hq


# --------------------------------------------------------------------------- layer


@dataclasses.dataclass
class Trace:
    xq: MXTensor
    z: np.ndarray
    zq: MXTensor
    routing: Routing
    disp: Dispatch
    h_rows: np.ndarray        # [T*k][F] fp64, in sorted-row order
    g_rows: np.ndarray        # [T*k][F] gate pre-activation, sorted rows
    u_rows: np.ndarray        # [T*k][F] up projection, sorted rows
    hq_rows: MXTensor         # [T*k][F]
    ye_rows: np.ndarray       # [T*k][L]
    y_lat: np.ndarray         # [T][L]
    yq: MXTensor
    y_up: np.ndarray
    h_shared: list
    g_shared: list
    u_shared: list
    hq_shared: list
    y_shared: list
    y: np.ndarray


def forward(x: np.ndarray, W: LayerWeights, top_k: int, decide=np.float32,
            expert_weights=None) -> Trace:
    """The whole layer.  ``expert_weights(e)`` may supply (wg, wu, wd) lazily."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    E = W.w_router.shape[0]
    L = W.w_router.shape[1]

    latent = W.w_down is not None
    hp = W.precision == "bf16"
    if hp and not latent:
        raise ValueError("the bfloat16 precision map is defined for the latent layer")
    xq = quant(x, "bf16" if hp else "e4m3", decide)                 # step 1 (xb under the bf16 map)
    z = mm(xq, W.w_down) if latent else x.astype(np.float64)        # step 2 (latent only)
    r = route(z, W.w_router, top_k, W.logit_bias, W.selection_bias, decide, W.gating)   # steps 3-5
    disp = dispatch(r.ids, E)                                       # step 6
    if latent:
        zq = quant(z, "e4m3", decide)
    else:
        zq = xq                                                     # the experts read xq
    sfmt = "bf16" if hp else "e4m3"                                 # shared hidden state, up-projection input

    P = T * top_k
    F = None
    ye_rows = np.zeros((P, L))
    h_rows = g_rows = u_rows = None
    hq_codes = hq_scales = None
    for e in range(E):                                              # step 7
        lo, hi = disp.offsets[e], disp.offsets[e + 1]
        if hi == lo:
            continue
        if expert_weights is not None:
            wg, wu, wd = expert_weights(e)
        else:
            wg, wu, wd = W.w_gate_e[e], W.w_up_e[e], W.w_down_e[e]
        toks = disp.pair_of_row[lo:hi] // top_k
        a = zq[toks]
        ye, h, hq, g, u = swiglu_expert(a, wg, wu, wd, decide, full=True)
        if h_rows is None:
            F = h.shape[1]
            h_rows = np.zeros((P, F))
            g_rows = np.zeros((P, F))
            u_rows = np.zeros((P, F))
            hq_codes = np.zeros((P, F), np.uint8)
            hq_scales = np.zeros((P, F // mx.BLOCK), np.uint8)
        ye_rows[lo:hi] = ye
        h_rows[lo:hi] = h
        g_rows[lo:hi] = g
        u_rows[lo:hi] = u
        hq_codes[lo:hi] = hq.codes
        hq_scales[lo:hi] = hq.scales

    y_lat = np.zeros((T, L))                                        # step 8
    for t in range(T):
        for j in range(top_k):
            y_lat[t] += r.gates[t, j] * ye_rows[disp.row_of_pair[t * top_k + j]]

    if latent:                                                      # step 9
        yq = quant(y_lat, sfmt, decide)
        y_up = mm(yq, W.w_up)
    else:
        yq, y_up = None, y_lat.copy()

    y = y_up.copy()                                                 # step 10
    hs_l, hsq_l, ys_l, gs_l, us_l = [], [], [], [], []
    for s in range(len(W.w_gate_s)):
        ys, hs, hsq, gs, us = swiglu_expert(xq, W.w_gate_s[s], W.w_up_s[s], W.w_down_s[s], decide, full=True,
                                            hfmt=sfmt)
        y += ys
        hs_l.append(hs)
        gs_l.append(gs)
        us_l.append(us)
        hsq_l.append(hsq)
        ys_l.append(ys)

    hq_rows = MXTensor(hq_codes, hq_scales, "e4m3") if hq_codes is not None else None
    return Trace(xq, z, zq, r, disp, h_rows, g_rows, u_rows, hq_rows, ye_rows, y_lat, yq, y_up, hs_l, gs_l, us_l,
                 hsq_l, ys_l, y)


def forward_dense_mask(x: np.ndarray, W: LayerWeights, top_k: int, decide=np.float32) -> np.ndarray:
    """Brute force: run EVERY routed expert on EVERY token, weight by a dense gate
    matrix that is zero off the selection, and sum; no permutation, no segments.
    This is the toy's 'dense loop' check in matrix form."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    E = W.w_router.shape[0]
    latent = W.w_down is not None
    sfmt = "bf16" if W.precision == "bf16" else "e4m3"
    xq = quant(x, sfmt, decide)
    z = mm(xq, W.w_down) if latent else x.astype(np.float64)
    r = route(z, W.w_router, top_k, W.logit_bias, W.selection_bias, decide, W.gating)
    dense_gate = np.zeros((T, E))
    np.put_along_axis(dense_gate, r.ids, r.gates, axis=1)
    zq = quant(z, "e4m3", decide) if latent else xq
    y_lat = np.zeros_like(z)
    for e in range(E):
        ye, _, _ = swiglu_expert(zq, W.w_gate_e[e], W.w_up_e[e], W.w_down_e[e], decide)
        y_lat += dense_gate[:, e:e + 1] * ye
    y = mm(quant(y_lat, sfmt, decide), W.w_up) if latent else y_lat.copy()
    for s in range(len(W.w_gate_s)):
        ys, _, _ = swiglu_expert(xq, W.w_gate_s[s], W.w_up_s[s], W.w_down_s[s], decide, hfmt=sfmt)
        y = y + ys
    return y


# --------------------------------------------------------------------------- comparison helpers


def ambiguous_codes(v: np.ndarray, bound: np.ndarray, fmt="e4m3") -> np.ndarray:
    """Elements whose MX code is not fixed by ``v`` to within +-``bound``.

    The code of an element is monotone in |v| once the block scale is fixed, and
    the scale is monotone in the block maximum.  Shrinking every magnitude by the
    bound and growing it by the bound gives the two extreme quantisations; where
    they agree (scale and code) every value inside the interval quantises the
    same.  Where |v| <= bound the sign itself is open.
    Returns a bool mask of v's shape.
    """
    v = np.asarray(v, dtype=np.float64)
    bound = np.broadcast_to(np.asarray(bound, dtype=np.float64), v.shape)
    mag = np.abs(v)
    lo = np.maximum(mag - bound, 0.0)
    hi = mag + bound
    c_lo, s_lo = mx.quantize(lo, fmt)
    c_hi, s_hi = mx.quantize(hi, fmt)
    K = v.shape[-1]
    scale_open = np.repeat(s_lo != s_hi, mx.BLOCK, axis=-1).reshape(v.shape)
    return (c_lo != c_hi) | scale_open | (mag <= bound)


def mm_abs(a: MXTensor, b: MXTensor) -> np.ndarray:
    """|deq(a)| @ |deq(b)|^T: the sum of absolute products, for fp32 error bounds."""
    return np.abs(a.deq()) @ np.abs(b.deq()).T
