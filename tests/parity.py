"""Comparison of a GPU layer trace with the oracle (test infrastructure).

What is compared
----------------
1. MX codes of the inputs (x) and weights: bit-exact.
2. The latent z (bf16 matrix cores on exactly decoded operands): within the
   fp32 accumulation bound K * 2^-24 * ||a_row|| * ||b_row||.
3. Expert ids: the same set per token unless the oracle's gap between the k-th
   and (k+1)-th selection key is below 1e-6 (a flagged near-tie, where the GPU's
   set must still be a valid top-k within 1e-6); gates within max(1e-6, the
   error the z bound propagates through the fp32 router).
4. Dispatch: counts, offsets and permutation equal the stable sort of the
   GPU's ids, bit-exactly.
5. Replay.  Every MXFP8 re-quantisation of a computed tensor (zq, hq, yq, hs;
   under the higher-precision map the bfloat16 roundings of y_lat and hs)
   turns any accumulation difference that straddles a rounding boundary into a
   whole-step code change, and such changes cascade through the later stages:
   even fp32-level noise in the oracle itself moves its own output by ~1e-3
   (relative L2).  Where several codes are correct, the unique part is
   compared and the rest is checked for validity: the oracle re-runs the layer
   (same fp64 arithmetic) and, only in blocks where ITS OWN value lies within
   the proven error bound of a boundary, continues with the GPU's block after
   checking that block is an admissible quantisation of some value inside that
   bound.  Against this replay every GPU code must then match bit-exactly and
   every fp32 tensor (h, y_e, y_lat, y) must lie within its bound, and the
   output must meet the tolerance (relative L2 <= 5e-3, max-abs <= 5e-2 rms).
6. The unconditioned oracle output: relative L2 <= 5e-3 (its max-abs error is
   reported).

Error bounds
------------
* bf16 matrix cores: fp32 accumulation, K * 2^-24 * sum |a_i b_i| (bounded by
  Cauchy-Schwarz).
* block-scaled MX matrix cores (measured on gfx950 with single-instruction
  probes): within one 32-element block the products are summed in a window
  ending 14 bits below the block's largest product (truncated); block sums
  accumulate in fp32.  Bound: 2^-9 * sum_b amax_a[b] * amax_b[b] (32 products,
  each off by less than 2^-14 of the block's largest product) plus
  (K/32 + 2) * 2^-24 * sum |a_i b_i|.
"""

from __future__ import annotations

import numpy as np

from oracle import moe, mx

EPS32 = 2.0 ** -24
NEAR_TIE = 1e-6
REL_L2 = 5e-3
MAXABS_FRAC = 5e-2


# --------------------------------------------------------------------------- bounds


def row_norms(t: moe.MXTensor) -> np.ndarray:
    return np.sqrt((t.deq() ** 2).sum(-1))


def gemm_bound(a: moe.MXTensor, b: moe.MXTensor, value: np.ndarray) -> np.ndarray:
    """fp32-accumulation bound (the bf16 matrix-core path)."""
    K = a.deq().shape[-1]
    return K * EPS32 * np.outer(row_norms(a), row_norms(b)) + EPS32 * np.abs(value)


def concat_gemm_bound(pairs, value: np.ndarray) -> np.ndarray:
    """fp32 bound of one bf16 GEMM whose K is the concatenation of the
    segments ``pairs`` = [(a, b), ...]: (total K) * 2^-24 * sum |a_i b_i| over
    every segment, plus the final rounding."""
    K = sum(a.deq().shape[-1] for a, _ in pairs)
    sab = sum(np.outer(row_norms(a), row_norms(b)) for a, b in pairs)
    return K * EPS32 * sab + EPS32 * np.abs(value)


def u16(a) -> np.ndarray:
    """bfloat16 patterns as uint16 (the trace holds them in int16 tensors)."""
    return np.ascontiguousarray(a).view(np.uint16)


def block_amax(t: moe.MXTensor) -> np.ndarray:
    v = np.abs(t.deq())
    return v.reshape(*v.shape[:-1], -1, 32).max(-1)


def mx_mfma_bound(a: moe.MXTensor, b: moe.MXTensor, value=None) -> np.ndarray:
    """Bound for the block-scaled MFMA path (module docstring)."""
    K = a.codes.shape[-1]
    sab = np.abs(a.deq()) @ np.abs(b.deq()).T
    win = 2.0 ** -9 * (block_amax(a) @ block_amax(b).T)
    out = win + (K // 32 + 2) * EPS32 * sab
    return out + EPS32 * (sab if value is None else np.abs(value))


def swiglu_bound(g, u, bg, bu, h):
    """Bound on |h_gpu - h| for h = silu(G) U given |dG| <= bg, |dU| <= bu."""
    sg = 1 / (1 + np.exp(-g))
    dsilu = sg * (1 + g * (1 - sg))          # |silu'| <= 1.1, |silu''| <= 0.5
    # The last term is the kernel's own fp32 evaluation G * U / (1 + 2^(-G log2 e)):
    # the rounded exponent puts 2|G| units of 2^-24 into t, exp2 two more, and
    # t / (1 + t) of that reaches the quotient; 1 + t, the reciprocal (two units)
    # and the two products add five -- at most 7 units for G >= 0 and 2|G| + 7
    # below; 9 + 2|G| leaves margin.
    # Both are taken at the kernel's own operands, |G| + bg and |h| + prop.
    prop = np.abs(dsilu) * np.abs(u) * bg + np.abs(g * sg) * bu + bg * bu + 0.5 * np.abs(u) * bg ** 2
    return prop + (9 + 2 * (np.abs(g) + bg)) * EPS32 * (np.abs(h) + prop) + 1e-30


def output_errors(y_gpu: np.ndarray, y_ref: np.ndarray):
    diff = y_gpu.astype(np.float64) - y_ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(y_ref), 1e-300)
    rms = np.sqrt((y_ref ** 2).mean())
    return float(rel), float(np.abs(diff).max()), float(rms)


# --------------------------------------------------------------------------- replay


class Replay:
    """``resolve`` hooks for ``oracle.moe.forward``: adopt the GPU's block where
    the oracle's own value is within its bound of a rounding boundary and the
    GPU's block is an admissible quantisation there."""

    def __init__(self, tr, W, k, dgate, xq):
        self.tr, self.W, self.k, self.dgate, self.xq = tr, W, k, dgate, xq
        self.hp = W.precision == "bf16"   # bfloat16 latent projections and shared experts
        self.stats = {}
        P = tr["hq_codes"].shape[0]
        L = tr["y_e"].shape[1]
        self.h_bound = np.zeros(tr["hq_codes"].shape)
        self.ye_bound = np.zeros((P, L))
        self.ylat_bound = None
        self.hs_bound = []

    def _adopt(self, name, v, bound, ref: moe.MXTensor, gcodes, gscales) -> moe.MXTensor:
        v32 = np.asarray(v, np.float64).astype(np.float32).astype(np.float64)   # the value the oracle quantised
        bound = np.asarray(bound, np.float64) + EPS32 * np.abs(v32) + 1e-300
        shp = v32.shape
        nb = shp[-1] // 32
        amb_blk = moe.ambiguous_codes(v32, bound).reshape(*shp[:-1], nb, 32).any(-1)
        mag = np.abs(v32)
        lo = np.maximum(mag - bound, 0.0)
        hi = mag + bound
        e_lo = mx.shared_exponent(lo.reshape(*shp[:-1], nb, 32).max(-1), 8)
        e_hi = mx.shared_exponent(hi.reshape(*shp[:-1], nb, 32).max(-1), 8)
        e_g = gscales.astype(np.int64) - 127
        ok_scale = (e_g >= e_lo) & (e_g <= e_hi)
        c_lo = mx.encode_with_exponent(lo, e_g, "e4m3") & 0x7F
        c_hi = mx.encode_with_exponent(hi, e_g, "e4m3") & 0x7F
        gm = gcodes & 0x7F
        ok_el = (gm >= c_lo) & (gm <= c_hi) & ((np.signbit(v32) == (gcodes >= 0x80)) | (mag <= bound))
        valid = ok_scale & ok_el.reshape(*shp[:-1], nb, 32).all(-1)
        use = amb_blk & valid
        st = self.stats.setdefault(name, {"ambiguous_blocks": 0, "adopted_blocks": 0, "inadmissible_blocks": 0})
        st["ambiguous_blocks"] += int(amb_blk.sum())
        differs = (gscales != ref.scales) | (gcodes != ref.codes).reshape(*shp[:-1], nb, 32).any(-1)
        st["adopted_blocks"] += int((use & differs).sum())
        st["inadmissible_blocks"] += int((amb_blk & ~valid & differs).sum())
        codes = np.where(np.repeat(use, 32, axis=-1).reshape(shp), gcodes, ref.codes).astype(np.uint8)
        scales = np.where(use, gscales, ref.scales).astype(np.uint8)
        return moe.MXTensor(codes, scales, "e4m3")

    def _adopt_bf16(self, name, v, bound, ref: moe.BF16Tensor, gbits) -> moe.BF16Tensor:
        """The bfloat16 rounding of each element is fixed unless the interval
        v +- bound reaches a rounding boundary (or zero, where the sign of a
        zero result is open); there the GPU's value must be the rounding of
        some value inside the interval."""
        gbits = u16(gbits)
        v32 = np.asarray(v, np.float64).astype(np.float32).astype(np.float64)
        b = np.asarray(bound, np.float64) + EPS32 * np.abs(v32) + 1e-300
        lo = mx.bf16_value(mx.bf16_bits(v32 - b))
        hi = mx.bf16_value(mx.bf16_bits(v32 + b))
        amb = (lo != hi) | (np.abs(v32) <= b)
        g = mx.bf16_value(gbits)
        valid = (g >= lo) & (g <= hi)
        use = amb & valid
        differs = gbits != ref.bits
        st = self.stats.setdefault(name, {"ambiguous_blocks": 0, "adopted_blocks": 0, "inadmissible_blocks": 0})
        st["ambiguous_blocks"] += int(amb.sum())
        st["adopted_blocks"] += int((use & differs).sum())
        st["inadmissible_blocks"] += int((amb & ~valid & differs).sum())
        return moe.BF16Tensor(np.where(use, gbits, ref.bits).astype(np.uint16))

    # hooks -----------------------------------------------------------------
    def zq(self, z, zq):
        bound = gemm_bound(self.xq, self.W.w_down, z)
        return self._adopt("zq", z, bound, zq, self.tr["zq_codes"], self.tr["zq_scales"])

    def hq(self, e, rows, a, wg, wu, wd, g, u, h, hq):
        lo, hi = rows
        bh = swiglu_bound(g, u, mx_mfma_bound(a, wg, g), mx_mfma_bound(a, wu, u), h)
        self.h_bound[lo:hi] = bh
        out = self._adopt("hq", h, bh, hq, self.tr["hq_codes"][lo:hi], self.tr["hq_scales"][lo:hi])
        self.ye_bound[lo:hi] = mx_mfma_bound(out, wd)
        return out

    def combine_bound(self, r, disp, ye_rows):
        """Bound of the fp32 gate-weighted sum of the k expert outputs: each
        term's own error (gate error, expert-output error) plus k + 1 roundings."""
        k = self.k
        rows = disp.row_of_pair.reshape(-1, k)
        g = np.abs(r.gates)
        b = np.zeros((rows.shape[0], ye_rows.shape[1]))
        acc = np.zeros_like(b)
        for j in range(k):
            ye = np.abs(ye_rows[rows[:, j]])
            b += g[:, j:j + 1] * self.ye_bound[rows[:, j]] + self.dgate[:, j:j + 1] * ye
            acc += g[:, j:j + 1] * ye
        b += (k + 1) * EPS32 * acc
        self.ylat_bound = b
        return b

    def yq(self, y_lat, yq, r, disp, ye_rows):
        b = self.combine_bound(r, disp, ye_rows)
        if self.hp:
            return self._adopt_bf16("yb", y_lat, b, yq, self.tr["yb"])
        return self._adopt("yq", y_lat, b, yq, self.tr["yq_codes"], self.tr["yq_scales"])

    def hs(self, s, wg, wu, wd, g, u, h, hq):
        if self.hp:   # bf16 matrix cores: fp32 accumulation of exact products
            bh = swiglu_bound(g, u, gemm_bound(self.xq, wg, g), gemm_bound(self.xq, wu, u), h)
            self.hs_bound.append(bh)
            return self._adopt_bf16(f"hs{s}", h, bh, hq, self.tr["hs_bf16"][s])
        bh = swiglu_bound(g, u, mx_mfma_bound(self.xq, wg, g), mx_mfma_bound(self.xq, wu, u), h)
        self.hs_bound.append(bh)
        return self._adopt(f"hs{s}", h, bh, hq, self.tr["hs_codes"][s], self.tr["hs_scales"][s])


# --------------------------------------------------------------------------- the check


def check_layer(cfg, W: moe.LayerWeights, o: moe.Trace, y: np.ndarray, tr: dict, x=None, say=print,
                expert_weights=None) -> dict:
    """Assert the GPU trace against the oracle (``o`` is its unconditioned run)."""
    T, k, E = y.shape[0], cfg.top_k, cfg.n_routed
    rep = {}

    # 1. input codes (MXFP8, or bfloat16 under the higher-precision map): bit-exact
    hp = W.precision == "bf16"
    if hp:
        assert np.array_equal(u16(tr["xb"]), o.xq.bits), "bf16(x)"
    else:
        assert np.array_equal(tr["xq_codes"], o.xq.codes), "xq codes"
        assert np.array_equal(tr["xq_scales"], o.xq.scales), "xq scales"

    # 2. latent down-projection (bf16 matrix cores); without a latent the
    #    router reads x and the experts xq, unchanged
    latent = W.w_down is not None
    if latent:
        bz = gemm_bound(o.xq, W.w_down, o.z)
        dz = np.abs(tr["z"].astype(np.float64) - o.z)
        assert np.all(dz <= bz), f"z outside the fp32 bound: worst ratio {np.max(dz / bz):.3g}"
        rep["z_err_over_bound"] = float(np.max(dz / bz))
    else:
        bz = np.zeros_like(o.z)
        assert np.array_equal(tr["z"].astype(np.float64), o.z), "router input is not x"
        assert np.array_equal(tr["zq_codes"], o.xq.codes) and np.array_equal(tr["zq_scales"], o.xq.scales)

    # 3. routing
    gi, ri = tr["ids"], o.routing.ids
    for t in range(T):
        assert len(set(gi[t].tolist())) == k and gi[t].min() >= 0 and gi[t].max() < E
    same = np.array([set(gi[t]) == set(ri[t]) for t in range(T)])
    near = o.routing.gap < NEAR_TIE
    assert np.all(same | near), f"ids differ on tokens {np.where(~(same | near))[0][:10]} without a near-tie"
    for t in np.where(~same)[0]:   # flagged near-ties: the GPU's choice must still be a valid top-k
        kth = np.sort(o.routing.sel[t])[::-1][k - 1]
        assert np.all(o.routing.sel[t, gi[t]] >= kth - NEAR_TIE), ("invalid near-tie choice", t)
    rep["near_tie_tokens"] = int(near.sum())
    rep["ids_differ_flagged"] = int((~same).sum())
    Wr = np.abs(W.w_router.astype(np.float64))
    zw = np.abs(o.z) @ Wr.T
    dlog = bz @ Wr.T + W.w_router.shape[1] * EPS32 * zw + 2 * EPS32 * (1 + zw)
    ds = 0.25 * dlog + 2 * EPS32
    dgate = np.zeros((T, k))
    worst_gate = 0.0
    if W.gating == "softmax":
        # softmax over the winners' logits: a logit error d_j moves gate j by a
        # factor within exp(+-(d_j + max_i d_i)); the fp32 evaluation adds the
        # subtraction of the maximum (EPS32 |l - m| inside exp), exp itself,
        # the k-term sum and the division.
        for t in range(T):
            gates_t = moe.winner_gates(o.routing.scores[t:t + 1], gi[t:t + 1], "softmax")[0]
            lw = o.routing.scores[t, gi[t]]
            dl = dlog[t, gi[t]]
            spread = float(lw.max() - lw.min())
            for j in range(k):
                tol = max(1e-6, gates_t[j] * (np.expm1(dl[j] + dl.max()) + (k + 6 + 2 * spread) * EPS32))
                dgate[t, j] = tol
                err = abs(float(tr["gates"][t, j]) - gates_t[j])
                worst_gate = max(worst_gate, err)
                assert err <= tol, ("gate", t, j, err, tol)
    for t in range(T if W.gating == "sigmoid" else 0):
        ssum = o.routing.scores[t, gi[t]].sum()
        gates_t = o.routing.scores[t, gi[t]] / ssum          # the oracle's gates of the GPU's set
        dsum = ds[t, gi[t]].sum()
        for j in range(k):
            e = int(gi[t, j])
            tol = max(1e-6, (ds[t, e] + gates_t[j] * dsum) / ssum + 4 * EPS32)
            dgate[t, j] = tol
            err = abs(float(tr["gates"][t, j]) - gates_t[j])
            worst_gate = max(worst_gate, err)
            assert err <= tol, ("gate", t, j, err, tol)
    rep["max_gate_err"] = worst_gate
    assert np.all(np.abs(tr["gates"].astype(np.float64).sum(1) - 1) <= 1e-6)

    # 4. dispatch = stable sort of the GPU's ids (bit-exact)
    d = moe.dispatch(gi, E)
    assert np.array_equal(tr["counts"], d.counts), "counts"
    assert np.array_equal(tr["offsets"], d.offsets), "offsets"
    assert np.array_equal(tr["pair_of_row"], d.pair_of_row), "pair_of_row"
    assert np.array_equal(tr["row_of_pair"], d.row_of_pair), "row_of_pair"

    # 5. replay along the GPU's admissible choices
    if x is not None:
        rp = Replay(tr, W, k, dgate, o.xq)
        c = moe.forward(x, W, k, ids_override=gi, resolve=rp, expert_weights=expert_weights)
        for name, st in rp.stats.items():
            assert st["inadmissible_blocks"] == 0, (name, st)
        rep["replay"] = rp.stats
        if not latent:
            rp.combine_bound(c.routing, c.disp, c.ye_rows)
        checks = [("hq", tr["hq_codes"], tr["hq_scales"], c.hq_rows)]
        if latent:
            checks += [("zq", tr["zq_codes"], tr["zq_scales"], c.zq)]
            if hp:
                nbad = int((u16(tr["yb"]) != c.yq.bits).sum())
                assert nbad == 0, f"bf16(y_lat): {nbad} mismatches against the replay"
            else:
                checks += [("yq", tr["yq_codes"], tr["yq_scales"], c.yq)]
        for name, gc, gs, ref in checks:
            nbad = int((gc != ref.codes).sum()) + int((gs != ref.scales).sum())
            if nbad:
                say(f"  {name} mismatches at {np.argwhere(gc != ref.codes)[:3].tolist()}")
            assert nbad == 0, f"{name}: {nbad} code/scale mismatches against the replay"
        for s in range(len(W.w_gate_s)):
            if hp:
                assert np.array_equal(u16(tr["hs_bf16"][s]), c.hq_shared[s].bits), f"hs{s} bf16"
            else:
                assert np.array_equal(tr["hs_codes"][s], c.hq_shared[s].codes), f"hs{s} codes"
                assert np.array_equal(tr["hs_scales"][s], c.hq_shared[s].scales), f"hs{s} scales"
            dh = np.abs(tr["hs"][s].astype(np.float64) - c.h_shared[s])
            assert np.all(dh <= rp.hs_bound[s]), f"hs{s} outside its bound"
        dh = np.abs(tr["h"].astype(np.float64) - c.h_rows)
        assert np.all(dh <= rp.h_bound), f"h outside its bound on {(dh > rp.h_bound).sum()} elements"
        dye = np.abs(tr["y_e"].astype(np.float64) - c.ye_rows)
        assert np.all(dye <= rp.ye_bound), f"y_e outside its bound on {(dye > rp.ye_bound).sum()} elements"
        dyl = np.abs(tr["y_lat"].astype(np.float64) - c.y_lat)
        assert np.all(dyl <= rp.ylat_bound), f"y_lat outside its bound on {(dyl > rp.ylat_bound).sum()} elements"
        if hp:   # one bf16 GEMM over K = [L | Fs ...]
            by = concat_gemm_bound([(c.yq, W.w_up)] + [(c.hq_shared[s], W.w_down_s[s])
                                                      for s in range(len(W.w_gate_s))], c.y)
        else:
            by = mx_mfma_bound(c.yq, W.w_up) if latent else rp.ylat_bound
            for s in range(len(W.w_gate_s)):
                by = by + mx_mfma_bound(c.hq_shared[s], W.w_down_s[s])
            by = by + (1 + len(W.w_gate_s)) * EPS32 * np.abs(c.y)
        dy = np.abs(y.astype(np.float64) - c.y)
        assert np.all(dy <= by), f"y outside its bound on {(dy > by).sum()} elements"
        rel, maxabs, rms = output_errors(y, c.y)
        rep.update(replay_rel_l2=rel, replay_max_abs_over_rms=maxabs / rms)
        assert rel <= REL_L2, f"relative L2 vs replay {rel:.3g}"
        assert maxabs <= MAXABS_FRAC * rms, f"max abs vs replay {maxabs:.3g} (rms {rms:.3g})"

    # 6. unconditioned oracle output
    rel, maxabs, rms = output_errors(y, o.y)
    rep.update(rel_l2=rel, max_abs_over_rms=maxabs / rms, rms=rms)
    say("parity report:", rep)
    assert rel <= REL_L2, f"relative L2 {rel:.3g}"
    return rep


# --------------------------------------------------------------------------- sampled tokens


def check_full_dispatch(full: dict, E: int, k: int):
    """Batch-wide properties that are unique and cheap: every token routes to k
    distinct valid experts, gates sum to one, and the GPU's dispatch is exactly
    the stable expert-sorted permutation of its own ids."""
    ids = full["ids"]
    T = ids.shape[0]
    assert ids.min() >= 0 and ids.max() < E, "expert id out of range"
    srt = np.sort(ids, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]), "repeated expert in a token's top-k"
    assert np.all(np.abs(full["gates"].astype(np.float64).sum(1) - 1) <= 1e-6), "gates do not sum to 1"
    d = moe.dispatch(ids, E)
    assert np.array_equal(full["counts"], d.counts), "counts"
    assert np.array_equal(full["offsets"], d.offsets), "offsets"
    assert np.array_equal(full["pair_of_row"], d.pair_of_row), "pair_of_row"
    assert np.array_equal(full["row_of_pair"], d.row_of_pair), "row_of_pair"
    return {"tokens": int(T), "pairs": int(T * k), "touched_experts": int((d.counts > 0).sum()),
            "max_expert_rows": int(d.counts.max())}


def subset_trace(sub: dict, E: int, k: int) -> dict:
    """A trace of the sampled tokens alone, laid out as the layer would lay out
    a batch of just those tokens: per-row arrays reordered into the subset's
    own stable expert-sorted dispatch (the GPU rows of a pair do not depend on
    the other tokens)."""
    tr = dict(sub)
    d = moe.dispatch(sub["ids"], E)
    for n in ("h", "hq_codes", "hq_scales", "y_e"):
        v = sub[n]                      # rows in (token, slot) order
        out = np.empty_like(v)
        out[d.row_of_pair] = v
        tr[n] = out
    tr.update(counts=d.counts, offsets=d.offsets, pair_of_row=d.pair_of_row, row_of_pair=d.row_of_pair)
    return tr


def check_tokens(cfg, W, x_sub, y_sub, sub, expert_weights, say=print) -> dict:
    """The sampled tokens' full path against the oracle, with the same checks
    as check_layer (replay included) on the subset's trace."""
    import dataclasses as _dc
    tr = subset_trace(sub, cfg.n_routed, cfg.top_k)
    csub = _dc.replace(cfg, T=x_sub.shape[0])
    o = moe.forward(x_sub, W, cfg.top_k, expert_weights=expert_weights)
    return check_layer(csub, W, o, y_sub, tr, x=x_sub, say=say, expert_weights=expert_weights)
