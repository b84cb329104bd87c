"""The layer re-run along another implementation's admissible choices (test
infrastructure).

Every MX (or bfloat16) re-quantisation of a computed tensor -- zq, hq, yq, the
shared hidden states -- turns an accumulation difference that straddles a
rounding boundary into a whole code step, and such steps cascade through the
later stages.  Where several codes are correct, the unique part is compared
and the rest checked for validity: this module runs the layer step by step
with the oracle's own functions (``oracle.moe``: quantise, MX matmul, router,
dispatch, SiLU), on the ids the implementation chose, and at each
re-quantisation asks a ``chooser`` (``tests.parity.Replay``) which codes to
continue with.  The chooser keeps the oracle's codes except in blocks where
the oracle's own value lies within the proven error bound of a boundary and
the implementation's block is an admissible quantisation there.

The oracle package itself carries no such hook; nothing here changes its
arithmetic.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from oracle import moe, mx


@dataclasses.dataclass
class ReplayTrace:
    xq: object
    z: np.ndarray
    zq: object
    routing: moe.Routing
    disp: moe.Dispatch
    h_rows: np.ndarray
    hq_rows: Optional[moe.MXTensor]
    ye_rows: np.ndarray
    y_lat: np.ndarray
    yq: object
    h_shared: list
    hq_shared: list
    y: np.ndarray


def replay_forward(x, W: moe.LayerWeights, top_k: int, ids, chooser, expert_weights=None, decide=np.float32,
                   workers: int = 1) -> ReplayTrace:
    """The layer of ``oracle.moe.forward`` with the selection fixed to ``ids``
    and every re-quantisation of a computed tensor passed through ``chooser``
    (methods ``zq``, ``hq``, ``yq``, ``hs``).  ``workers`` > 1 runs the routed
    experts in a thread pool (each expert's rows are independent)."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    E = W.w_router.shape[0]
    L = W.w_router.shape[1]
    latent = W.w_down is not None
    hp = W.precision == "bf16"
    xq = moe.quant(x, "bf16" if hp else "e4m3", decide)
    z = moe.mm(xq, W.w_down) if latent else x.astype(np.float64)
    r = moe.route(z, W.w_router, top_k, W.logit_bias, W.selection_bias, decide, W.gating)
    ids = np.asarray(ids, dtype=np.int32)
    r = moe.Routing(r.scores, r.sel, ids, moe.winner_gates(r.scores, ids, W.gating), r.gap)
    disp = moe.dispatch(ids, E)
    zq = chooser.zq(z, moe.quant(z, "e4m3", decide)) if latent else xq
    sfmt = "bf16" if hp else "e4m3"

    P = T * top_k
    ye_rows = np.zeros((P, L))
    live = [e for e in range(E) if disp.offsets[e + 1] > disp.offsets[e]]

    def one(e):
        lo, hi = int(disp.offsets[e]), int(disp.offsets[e + 1])
        wg, wu, wd = expert_weights(e) if expert_weights is not None else (W.w_gate_e[e], W.w_up_e[e],
                                                                          W.w_down_e[e])
        a = zq[disp.pair_of_row[lo:hi] // top_k]
        g = moe.mm(a, wg)
        u = moe.mm(a, wu)
        h = moe.silu(g) * u
        hq = chooser.hq(e, (lo, hi), a, wg, wu, wd, g, u, h, moe.quant(h, "e4m3", decide))
        return lo, hi, h, hq, moe.mm(hq, wd)

    if workers > 1 and len(live) > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            done = list(ex.map(one, live))
    else:
        done = [one(e) for e in live]
    h_rows = hq_codes = hq_scales = None
    for lo, hi, h, hq, ye in done:
        if h_rows is None:
            F = h.shape[1]
            h_rows = np.zeros((P, F))
            hq_codes = np.zeros((P, F), np.uint8)
            hq_scales = np.zeros((P, F // mx.BLOCK), np.uint8)
        h_rows[lo:hi] = h
        hq_codes[lo:hi] = hq.codes
        hq_scales[lo:hi] = hq.scales
        ye_rows[lo:hi] = ye

    y_lat = np.zeros((T, L))
    for t in range(T):
        for j in range(top_k):
            y_lat[t] += r.gates[t, j] * ye_rows[disp.row_of_pair[t * top_k + j]]

    if latent:
        yq = chooser.yq(y_lat, moe.quant(y_lat, sfmt, decide), r, disp, ye_rows)
        y = moe.mm(yq, W.w_up)
    else:
        yq, y = None, y_lat.copy()
    hs_l, hsq_l = [], []
    for s in range(len(W.w_gate_s)):
        g = moe.mm(xq, W.w_gate_s[s])
        u = moe.mm(xq, W.w_up_s[s])
        h = moe.silu(g) * u
        hq = chooser.hs(s, W.w_gate_s[s], W.w_up_s[s], W.w_down_s[s], g, u, h, moe.quant(h, sfmt, decide))
        y = y + moe.mm(hq, W.w_down_s[s])
        hs_l.append(h)
        hsq_l.append(hq)
    hq_rows = moe.MXTensor(hq_codes, hq_scales, "e4m3") if hq_codes is not None else None
    return ReplayTrace(xq, z, zq, r, disp, h_rows, hq_rows, ye_rows, y_lat, yq, hs_l, hsq_l, y)
