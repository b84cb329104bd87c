#!/usr/bin/env python3
"""LatentMoE layer forward at Kimi-K3 width on one MI355X.

One step = one full forward of the layer (MXFP8 quantise, latent
down-projection, sigmoid router + top-16 of 896, dispatch, grouped
MXFP4 x MXFP8 expert GEMMs with SwiGLU, combine, up-projection and the two
shared experts) over one batch of synthetic tokens already resident in HBM.

Default workload: the 16384-token prefill batch (matrix-core bound); the
64-token decode batch (HBM bound) is measured in the same run and reported
under "decode".  Inside the timed region the library records only the two
HIP events that bracket the dominant launch (expert_up) on the forward's
stream; the other per-stage times come from the same steps run again
untimed with an event at every stage boundary (each event record adds a few
microseconds to the stream, which would otherwise count in the step time).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_MX_TFLOPS = 5000.0        # dense MFMA at the FP8 rate (an FP8 activation operand), TFLOP/s


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


class StageEvents:
    """MOE_TRACE_EVENTS HIP events per step, for K steps (only those in `only`,
    if given: the other entries stay NULL and the library skips them)."""

    def __init__(self, hip, n_steps, n_ev, only=None):
        self.hip = hip
        self.arrays = []
        for _ in range(n_steps):
            arr = (ctypes.c_void_p * n_ev)()
            for i in range(n_ev):
                if only is not None and i not in only:
                    continue
                e = ctypes.c_void_p()
                assert hip.hipEventCreate(ctypes.byref(e)) == 0
                arr[i] = e.value
            self.arrays.append(arr)

    def elapsed(self, step, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arrays[step][a], self.arrays[step][b]) == 0
        return ms.value

    def close(self):
        for arr in self.arrays:
            for e in arr:
                if e:
                    self.hip.hipEventDestroy(e)


def algorithmic_work(cfg, counts):
    """Flops and bytes one forward must do (codes + scales; no padding, no re-reads)."""
    T, d, L, E, k, S, F, Fs = (cfg.T, cfg.d_model, cfg.d_latent, cfg.n_routed, cfg.top_k, cfg.n_shared,
                               cfg.d_ff_routed, cfg.d_ff_shared)
    P = T * k
    lat = int(getattr(cfg, "latent", True))   # 0: no latent projections (L = d)
    mxb = lambda n: n * 17 // 32          # E2M1 codes + E8M0 scales
    f8b = lambda n: n * 33 // 32          # E4M3 codes + E8M0 scales
    touched = int((counts > 0).sum())
    w_up_e = 2 * F * L                    # gate + up elements per expert
    w_dn_e = L * F
    work = {
        "touched_experts": touched,
        # dominant kernel: routed gate/up GEMM + SwiGLU + MXFP8(h)
        "expert_up_flops": 2.0 * P * L * 2 * F,
        "expert_up_bytes": touched * mxb(w_up_e) + P * f8b(L) + P * f8b(F),
        "expert_down_flops": 2.0 * P * F * L,
        "expert_down_bytes": touched * mxb(w_dn_e) + P * f8b(F) + P * L * 4,
    }
    # What one launch of the gate/up kernel does: at few tokens (weight-
    # streaming kernels, MX weights) the shared experts' gate/up GEMM runs in
    # the routed launch, so its work is part of that launch's.
    work["expert_up_launch_flops"] = work["expert_up_flops"]
    work["expert_up_launch_bytes"] = work["expert_up_bytes"]
    if T <= 256 and S > 0 and getattr(cfg, "precision", "mx") == "mx" and P <= 16 * E:
        work["expert_up_launch_flops"] += S * 2.0 * T * d * 2 * Fs
        work["expert_up_launch_bytes"] += S * mxb(2 * Fs * d) + T * f8b(d) + S * T * f8b(Fs)
    mx_flops = (lat * 4.0 * T * d * L + work["expert_up_flops"] + work["expert_down_flops"]
                + S * (2.0 * T * d * 2 * Fs + 2.0 * T * Fs * d))
    weight_bytes = (lat * mxb(2 * d * L) + touched * (mxb(w_up_e) + mxb(w_dn_e)) + S * mxb(3 * d * Fs) + E * L * 4)
    work.update(mx_flops=mx_flops, router_flops=2.0 * T * L * E, weight_bytes=weight_bytes,
                layer_bytes=weight_bytes + T * d * 8 + P * (f8b(L) + f8b(F) * 2 + 8 * L))
    return work


def run_workload(name, steps, warmup, weights, hip, say, logit_bias=None):
    import numpy as np
    import torch

    import synth
    from latent_routing_mxfp4_amd import _lib
    from latent_routing_mxfp4_amd import layer as LY

    cfg = synth.config(name)
    shape = LY.LayerShape.of(cfg)
    if logit_bias is not None:   # same weights, another router logit bias (the skewed batch)
        weights = dict(weights)
        weights["router_logit_bias"] = torch.from_numpy(logit_bias).cuda()
    lay = LY.LatentMoE(shape, weights, cfg.T)
    x = torch.from_numpy(synth.gen_hidden(cfg)).cuda()
    y = torch.empty_like(x)
    lay.workspace(cfg.T)
    stream = torch.cuda.current_stream().cuda_stream
    nev = _lib.MOE_TRACE_EVENTS
    dom = _lib.STAGES.index("expert_up")       # stage i lies between events i and i + 1
    tevs = StageEvents(hip, steps, nev, only=(dom, dom + 1))
    sevs = StageEvents(hip, steps, nev)
    mk = lambda evs: [_lib.MoeLayerTrace(*([None] * len(_lib.TRACE_FIELDS)), ctypes.cast(a, ctypes.c_void_p))
                      for a in evs.arrays]
    timed_traces, stage_traces = mk(tevs), mk(sevs)
    ws = lay.workspace(cfg.T)

    def step(tr=None):
        _lib.moe_layer_forward(lay.handle, x.data_ptr(), cfg.T, y.data_ptr(), ws.data_ptr(), ws.numel(), stream,
                               tr)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(timed_traces[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    # the same steps again, untimed, with an event at every stage boundary
    for i in range(steps):
        step(stage_traces[i])
    torch.cuda.synchronize()

    stage_ms = {}
    for si, sname in enumerate(_lib.STAGES):
        # median over the steps (a slow first step or a stray hiccup does not
        # move it; the profile summary takes the median the same way)
        stage_ms[sname] = statistics.median(sevs.elapsed(i, si, si + 1) for i in range(steps))
    # the dominant launch as timed inside the timed region
    stage_ms["expert_up"] = statistics.median(tevs.elapsed(i, dom, dom + 1) for i in range(steps))
    # per-step forward time between the first and the last stage event
    per_step = sorted(sevs.elapsed(i, 0, len(_lib.STAGES)) for i in range(steps))
    pick = lambda q: per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    step_stats = {"median": statistics.median(per_step), "p10": pick(0.1), "p90": pick(0.9)}
    tevs.close()
    sevs.close()

    # routing statistics of this batch (outside the timed region)
    tb = {"counts": torch.empty(cfg.n_routed, dtype=torch.int32, device="cuda")}
    lay.forward(x, y, trace=tb)
    torch.cuda.synchronize()
    counts = tb["counts"].cpu().numpy()
    work = algorithmic_work(cfg, counts)
    work["step_events_ms"] = step_stats
    lay.close()
    say(f"{name}: {ms_per_step:.3f} ms/step; stages (ms): " +
        ", ".join(f"{k}={v:.3f}" for k, v in stage_ms.items()))
    return cfg, ms_per_step, stage_ms, work, counts


def bf16_map_report(weights, steps, decode_steps, warmup, hip, say):
    """The higher-precision map at K3 width: the same MXFP4 routed experts,
    bfloat16 latent projections and shared experts (encoded here); prefill
    and decode throughput and the dense stages' times."""
    import synth
    from latent_routing_mxfp4_amd import layer as LY

    out = {}
    w = None
    for name, n in (("k3_prefill_bf16", steps), ("k3_decode_bf16", decode_steps)):
        cfg = synth.config(name)
        if w is None:
            t = time.perf_counter()
            w = dict(weights)
            w.update(LY.encode_weights(LY.LayerShape.of(cfg), lambda m, i: synth.gen_weight(cfg, m, i),
                                       names=LY.DENSE + LY.SHARED))
            say(f"bf16 dense weights encoded in {time.perf_counter() - t:.1f} s")
        c, ms, st, work, counts = run_workload(name, n, warmup, w, hip, say)
        out[name] = {"workload": f"{c.name}: T={c.T}, bf16 latent projections + shared experts",
                     "value": c.T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms, "stage_ms": st,
                     "step_events_ms": work["step_events_ms"]}
    return out


def k2_report(steps, warmup, hip, say):
    """The non-latent K2-like layer (its own weights, encoded after the K3
    weights are freed): throughput, MX matrix-core share and the expert GEMM's
    rate.  A report line beside the headline, not the headline."""
    import torch

    import synth
    from latent_routing_mxfp4_amd import layer as LY

    cfg = synth.config("k2_prefill")
    t = time.perf_counter()
    shape = LY.LayerShape.of(cfg)
    extra = {"w_router": synth.gen_router(cfg), "router_logit_bias": synth.gen_logit_bias(cfg)}
    weights = LY.encode_weights(shape, lambda n, i: synth.gen_weight(cfg, n, i), extra=extra,
                                workers=min(16, len(os.sched_getaffinity(0))))
    say(f"K2 weights encoded on the GPU in {time.perf_counter() - t:.1f} s")
    kcfg, kms, kst, kwork, kcounts = run_workload("k2_prefill", steps, warmup, weights, hip, say)
    del weights
    torch.cuda.empty_cache()
    return {"workload": f"{kcfg.name}: T={kcfg.T}, d={kcfg.d_model}, no latent, E={kcfg.n_routed} "
                        f"top-{kcfg.top_k} softmax gates, {kcfg.n_shared} shared, d_ff={kcfg.d_ff_routed}",
            "value": kcfg.T / (kms / 1e3), "unit": "tokens/s", "ms_per_step": kms,
            "mx_frac": kwork["mx_flops"] / (kms / 1e3) / 1e12 / PEAK_MX_TFLOPS,
            "expert_up_tflops": kwork["expert_up_launch_flops"] / (kst["expert_up"] / 1e3) / 1e12,
            "expert_up_frac": kwork["expert_up_launch_flops"] / (kst["expert_up"] / 1e3) / 1e12 / PEAK_MX_TFLOPS,
            "touched_experts": kwork["touched_experts"], "max_expert_load": int(kcounts.max()),
            "stage_ms": kst, "step_events_ms": kwork["step_events_ms"]}


def small_report(name, steps, warmup, hip, say):
    """The small parity workloads (tiny: 64 tokens; mid: 4096 tokens, 128
    experts): throughput and the MX matrix-core share, on their own weights.
    Report lines beside the headline; launch-bound (tiny) or short (mid)."""
    import torch

    import synth
    from latent_routing_mxfp4_amd import layer as LY

    cfg = synth.config(name)
    shape = LY.LayerShape.of(cfg)
    extra = {"w_router": synth.gen_router(cfg), "router_logit_bias": synth.gen_logit_bias(cfg)}
    weights = LY.encode_weights(shape, lambda n, i: synth.gen_weight(cfg, n, i), extra=extra,
                                workers=min(16, len(os.sched_getaffinity(0))))
    c, ms, st, work, counts = run_workload(name, steps, warmup, weights, hip, say)
    del weights
    torch.cuda.empty_cache()
    return {"workload": f"{c.name}: T={c.T}, d={c.d_model}, latent={c.d_latent}, E={c.n_routed} top-{c.top_k}, "
                        f"{c.n_shared} shared, d_ff={c.d_ff_routed}",
            "value": c.T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
            "mx_tflops": work["mx_flops"] / (ms / 1e3) / 1e12,
            "mx_frac": work["mx_flops"] / (ms / 1e3) / 1e12 / PEAK_MX_TFLOPS,
            "stage_ms": st, "step_events_ms": work["step_events_ms"]}


def ep8_share_report(steps, warmup, hip, say):
    """One GPU's share of an 8-way expert-parallel K3 decode step (112 local
    experts, 1024 token copies, ~9 rows per expert; latent, router and shared
    experts on the GPU's own 64 tokens), on the same kernels; the all-to-all
    exchange is not modelled.  Reported beside the headline, not counted."""
    import torch

    import synth
    from latent_routing_mxfp4_amd import layer as LY

    cfg = synth.config("k3_ep8_share")
    shape = LY.LayerShape.of(cfg)
    extra = {"w_router": synth.gen_router(cfg), "router_logit_bias": synth.gen_logit_bias(cfg)}
    weights = LY.encode_weights(shape, lambda n, i: synth.gen_weight(cfg, n, i), extra=extra,
                                workers=min(16, len(os.sched_getaffinity(0))))
    c, ms, st, work, counts = run_workload(cfg.name, steps, warmup, weights, hip, say)
    del weights
    torch.cuda.empty_cache()
    return {"workload": f"{c.name}: T={c.T} own tokens, E={c.n_routed} local experts top-{c.top_k} "
                        f"({c.T * c.top_k} copies), {c.n_shared} shared, d_ff={c.d_ff_routed}",
            "value": c.T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
            "layer_gbs": work["layer_bytes"] / (ms / 1e3) / 1e9,
            "expert_up_gbs": work["expert_up_launch_bytes"] / (st["expert_up"] / 1e3) / 1e9,
            "max_expert_rows": int(counts.max()), "stage_ms": st, "step_events_ms": work["step_events_ms"]}


def qb_report(steps, warmup, say):
    """Quantile Balancing of the selection bias at the K3 prefill shape (16384
    tokens x 896 experts, top-16) on seeded N(0, 1) logits: time per update and
    the rate at which it consumes the logits (read once by the threshold pass
    and once by the margin pass; the per-expert selection reads the transposed
    margins eight times, mostly from L2).  A report line beside the headline."""
    import numpy as np
    import torch

    from latent_routing_mxfp4_amd import layer as LY

    T, E, k = 16384, 896, 16
    rng = np.random.default_rng(1004)
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    bias = torch.zeros(E, dtype=torch.float32, device="cuda")
    out = torch.empty_like(bias)
    ws = torch.empty(LY._lib.moe_quantile_balance_workspace_bytes(T, E), dtype=torch.uint8, device="cuda")
    for _ in range(max(warmup, 1)):
        LY.quantile_balance(lg, bias, k, 0.5, out=out, workspace=ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record()
        LY.quantile_balance(lg, bias, k, 0.5, out=out, workspace=ws)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))[steps // 2]
    say(f"quantile balance at T={T}, E={E}, k={k}: {ms:.3f} ms per update")
    logit_bytes = T * E * 4
    return {"workload": f"quantile balance: T={T}, E={E}, top-{k}", "ms_per_update": ms,
            "logits_gbs": 2 * logit_bytes / (ms / 1e3) / 1e9, "logits_bytes": logit_bytes}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(name, n_tokens, say):
    """The oracle, as it stands, on the workload: the routing and dispatch of
    EVERY token of the batch (quantise x, latent, router, top-k, gates, expert
    sort), timed in full; the expert FFNs, combine, up-projection and shared
    experts on the first ``n_tokens`` tokens (tokens are independent: the layer
    is dropless), timed and extrapolated per token to the whole batch; and the
    same sample again with one BLAS thread.  Expert weights are encoded
    beforehand (load-time work, untimed)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import synth
    from oracle import moe, weights

    cfg = synth.config(name)
    T = cfg.T
    x = synth.gen_hidden(cfg)
    W = weights.layer(cfg, experts="lazy")
    cores = _blas_threads()
    # 1. routing and dispatch of every token
    t0 = time.perf_counter()
    xq = moe.quant(x)
    z = moe.mm(xq, W.w_down)
    r = moe.route(z, W.w_router, cfg.top_k, W.logit_bias, W.selection_bias)
    moe.dispatch(r.ids, cfg.n_routed)
    t_route = time.perf_counter() - t0
    say(f"cpu oracle: routing and dispatch of all {T} tokens in {t_route:.2f} s ({cores} BLAS threads)")
    # 2. the whole layer on the sample (its experts encoded first, untimed)
    xs = x[:n_tokens]
    cache = weights.ExpertCache(cfg, maxsize=n_tokens * cfg.top_k + 8)
    need = sorted(set(r.ids[:n_tokens].reshape(-1).tolist()))
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(cache, need))
    t0 = time.perf_counter()
    moe.forward(xs, W, cfg.top_k, expert_weights=cache)
    t_sample = time.perf_counter() - t0
    t_single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            moe.forward(xs, W, cfg.top_k, expert_weights=cache)
            t_single = time.perf_counter() - t0
    except ImportError:
        pass
    per_tok = t_sample / n_tokens
    total = t_route + per_tok * T     # routing of the batch + the sample's per-token cost for every token
    say(f"cpu oracle: whole layer on {n_tokens} tokens in {t_sample:.2f} s ({per_tok:.2f} s/token); "
        f"batch extrapolated {total:.0f} s")
    out = {"value": T / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": (f"{name}: routing and dispatch of all {T} tokens timed ({t_route:.1f} s); the whole layer "
                      f"on the first {n_tokens} tokens timed ({t_sample:.1f} s, {len(need)} routed experts, "
                      f"weights encoded beforehand) and extrapolated per token to {T} tokens: value is "
                      f"EXTRAPOLATED"),
           "routing_all_tokens_s": t_route, "sample_tokens": n_tokens, "layer_s_per_token": per_tok,
           "extrapolated": True}
    if t_single is not None:
        out["single_thread_layer_s_per_token"] = t_single / n_tokens
        out["single_thread_sample_tokens_per_s"] = n_tokens / t_single
    return out


# --------------------------------------------------------------------------- rocprofv3 summaries

PROFILE_MD = os.path.join(ROOT, "profiles", "k3_layer_kernels_and_hbm_traffic.md")
PROFILE_CMD = ("python3 /root/repo/bench.py --steps 3 --warmup 1 --decode-steps 5 --no-cpu-baseline "
               "--skew-steps 0 --k2-steps 0 --bf16-steps 0 --qb-steps 0 --small-steps 0 --ep8-steps 0")
SIMDS = 1024    # MI355X: 256 compute units x 4 SIMDs (the MfmaUtil denominator)
XCDS = 8        # the counter CSV holds GRBM_GUI_ACTIVE summed over the 8 XCDs' instances


def source_digest() -> str:
    """sha256 over the HIP sources: a traffic figure is only reported for the
    exact kernels its counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "latent_routing_mxfp4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _csv(path):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*.csv"), recursive=True)
    return files


def _grid(r):
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return int(r.get("Grid_Size_X", 1)) * int(r.get("Grid_Size_Y", 1)) * int(r.get("Grid_Size_Z", 1))


def summarize_profiles(stats_dir, fetch_dir, write_dir, mfma_dir=None) -> str:
    """Markdown summary of the rocprofv3 runs of PROFILE_CMD: per (kernel,
    grid) the dispatch count, the median duration over the dispatches after the
    first (the warm-up step), FETCH_SIZE and WRITE_SIZE per dispatch, HBM bytes
    per launch scaled by the same counters on the 1 GiB copy kernel the
    benchmark runs first, and the matrix cores' busy share
    (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs)); plus the
    machine-readable traffic lines the benchmark reads."""
    import csv
    import collections
    import re

    def one(d, suffix):
        f = [x for x in _csv(d) if x.endswith(suffix)]
        assert f, (d, suffix)
        return list(csv.DictReader(open(f[0])))

    trace = one(stats_dir, "kernel_trace.csv")
    dur = collections.defaultdict(list)
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        dur[(r["Kernel_Name"], _grid(r))].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)

    def counters(d, names):
        # per dispatch (rocprofv3 writes each counter's instances already summed)
        agg = collections.defaultdict(lambda: collections.defaultdict(float))
        rows = one(d, "counter_collection.csv")
        for r in rows:
            n = r["Counter_Name"]
            if n in names:
                agg[(r["Kernel_Name"], _grid(r), r.get("Dispatch_Id", ""))][n] += float(r["Counter_Value"])
        per = collections.defaultdict(lambda: collections.defaultdict(list))
        for (kn, gr, _), v in agg.items():
            for n, x in v.items():
                per[(kn, gr)][n].append(x)
        return {k: {n: sum(x) / len(x) for n, x in v.items()} for k, v in per.items()}

    cnt = {"FETCH_SIZE": {k: v["FETCH_SIZE"] for k, v in counters(fetch_dir, {"FETCH_SIZE"}).items()},
           "WRITE_SIZE": {k: v["WRITE_SIZE"] for k, v in counters(write_dir, {"WRITE_SIZE"}).items()}}
    mfma = counters(mfma_dir, {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"}) if mfma_dir else {}
    # calibration: torch.mul over 2^28 floats reads 1 GiB and writes 1 GiB
    probe = [k for k in cnt["FETCH_SIZE"] if "MulFunctor" in k[0]]   # the only torch.mul of the run
    assert probe, "no copy-probe dispatch in the counter runs"
    f_fac = (1 << 20) / cnt["FETCH_SIZE"][probe[0]]        # KiB actually read / KiB counted
    w_fac = (1 << 20) / cnt["WRITE_SIZE"][probe[0]]

    def short(n):
        n = re.sub(r"\(.*", "", n.replace("void ", "").replace("(anonymous namespace)::", ""))
        return n

    rows = []
    for key, ds in dur.items():
        fk, wk = cnt["FETCH_SIZE"].get(key), cnt["WRITE_SIZE"].get(key)
        hbm = None if fk is None or wk is None else (fk * f_fac + wk * w_fac) * 1024
        med = statistics.median(ds[1:] if len(ds) > 1 else ds)
        m = mfma.get(key)
        util = None
        if m and m.get("GRBM_GUI_ACTIVE"):   # busy cycles over (the GPU's active cycles x SIMDs)
            util = 100.0 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
        rows.append((sum(ds), short(key[0]), key[1], len(ds), med, fk, wk, hbm, util))
    rows.sort(reverse=True)
    out = ["# K3 LatentMoE layer on MI355X: kernel times, HBM traffic and matrix-core busy share", "",
           "Commands (run from /tmp with TMPDIR=/tmp; the benchmark runs the 16384-token prefill batch, "
           "then the 64-token decode batch, both at K3 width):", "",
           "    rocprofv3 --kernel-trace --stats --output-format csv -d /tmp/p_stats -o run -- " + PROFILE_CMD,
           "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d /tmp/p_fetch -o run -- " + PROFILE_CMD,
           "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d /tmp/p_write -o run -- " + PROFILE_CMD,
           "    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d /tmp/p_mfma -o run -- "
           + PROFILE_CMD,
           "    python3 /root/repo/bench.py --summarize /tmp/p_stats /tmp/p_fetch /tmp/p_write /tmp/p_mfma", "",
           f"Counter calibration (1 GiB read + 1 GiB write elementwise kernel): FETCH_SIZE x {f_fac:.3f}, "
           f"WRITE_SIZE x {w_fac:.3f} (KiB per dispatch -> KiB moved).  Median ms: over the dispatches after the "
           f"first of each (kernel, grid) (the first belongs to the warm-up step).  MFMA busy: "
           f"SQ_VALU_MFMA_BUSY_CYCLES / (GPU active cycles x {SIMDS} SIMDs) per dispatch, averaged; the CSV "
           f"holds GRBM_GUI_ACTIVE summed over the {XCDS} XCDs (a 0.154 ms fill kernel reads 8 x its 367 k "
           f"cycles), so the active cycles are GRBM_GUI_ACTIVE / {XCDS}.  The matrix-core rate probe "
           f"(moe::mfma_rate_kernel, back-to-back FP8 x FP4 MFMAs) reads about 79% busy at 3.9 PFLOP/s.", "",
           "| kernel | grid (threads) | dispatches | median ms | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB/launch | MFMA busy % |",
           "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for tot, name, grid, n, med, fk, wk, hbm, util in rows[:24]:
        out.append(f"| {name} | {grid} | {n} | {med:.4f} | {fk if fk is None else round(fk)} | "
                   f"{wk if wk is None else round(wk)} | {'-' if hbm is None else f'{hbm / 1e6:.1f}'} | "
                   f"{'-' if util is None else f'{util:.1f}'} |")
    # the dominant kernels: expert_up = largest-grid dispatch of the prefill / decode gate-up kernels
    out += ["", "Dominant kernels (expert_up: routed gate/up GEMM + SwiGLU + MXFP8), machine-readable:", ""]
    dig = source_digest()
    # (at decode the routed gate/up launch also carries the shared experts' gate/up)
    for wl, pats in (("k3_prefill", ("mx_gemm_wide_kernel<2>",)),
                     ("k3_decode", ("mx_gemm_stream_pair_kernel<1, 2, 2>", "mx_gemm_stream_kernel<1, 2, 2>"))):
        cand = [r for r in rows if any(r[1].endswith(pat) for pat in pats)]
        if not cand:
            continue
        r = max(cand, key=lambda r: r[2])
        out.append(f"    traffic {wl} expert_up median_ms={r[4]:.4f} hbm_bytes={0 if r[7] is None else int(r[7])} "
                   f"sources={dig}")
    return "\n".join(out) + "\n"


def profiled_traffic(workload: str):
    """HBM bytes per launch of expert_up from the committed counter summary,
    or None when the kernels changed since the counters were taken."""
    try:
        text = open(PROFILE_MD).read()
    except OSError:
        return None
    import re
    m = re.search(rf"traffic {workload} expert_up median_ms=([0-9.]+) hbm_bytes=([0-9]+) sources=([0-9a-f]+)", text)
    if not m or m.group(3) != source_digest():
        return None
    return {"bytes": int(m.group(2)), "profiled_ms": float(m.group(1))}


def main():
    if len(sys.argv) in (5, 6) and sys.argv[1] == "--summarize":
        sys.stdout.write(summarize_profiles(*sys.argv[2:]))
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="k3_prefill", choices=["k3_prefill", "k3_decode", "k3_skew"])
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--skew-steps", type=int, default=5,
                    help="steps of the 8192-token Zipf-skewed batch reported under 'skew' (0: skip)")
    ap.add_argument("--k2-steps", type=int, default=5,
                    help="steps of the non-latent K2-like 8192-token layer reported under 'k2' (0: skip)")
    ap.add_argument("--bf16-steps", type=int, default=5,
                    help="steps of the higher-precision map (bf16 dense weights) reported under 'bf16_map' (0: skip)")
    ap.add_argument("--qb-steps", type=int, default=10,
                    help="Quantile Balancing updates at the K3 prefill shape reported under 'quantile_balance' (0: skip)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2,
                    help="tokens of the batch the CPU oracle runs the whole layer on (extrapolated)")
    ap.add_argument("--small-steps", type=int, default=20,
                    help="steps of the tiny (64-token) and mid (4096-token) layers reported under 'tiny' and 'mid' "
                         "(0: skip)")
    ap.add_argument("--ep8-steps", type=int, default=20,
                    help="steps of one GPU's share of an 8-way expert-parallel K3 decode (112 local experts) "
                         "reported under 'ep8_share' (0: skip)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="kept for the profile command: the copy probe now always runs first")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: the layer is measured on one MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); multi-GPU expert parallelism is not "
              f"part of this build.", file=sys.stderr)
        sys.exit(2)

    say = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))

    import torch

    import synth
    from latent_routing_mxfp4_amd import layer as LY

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hip = _hip()
    # STREAM-style probe on this GPU: 1 GiB read + 1 GiB write (also the
    # calibration dispatch of the HBM counters in the committed profile).
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.mul(a, 1.0, out=b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.mul(a, 1.0, out=b)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    # Read-only stream of 4 GiB with 16-byte non-temporal loads (what the
    # decode expert GEMMs do with their weights): the reference for their GB/s.
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    rbuf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    rfold = torch.empty(16 * n_cu * 256, dtype=torch.int32, device="cuda")
    LY._lib.moe_hbm_read_probe(rbuf.data_ptr(), rbuf.numel(), 16 * n_cu, rfold.data_ptr(), LY._stream())
    e0.record()
    LY._lib.moe_hbm_read_probe(rbuf.data_ptr(), rbuf.numel(), 16 * n_cu, rfold.data_ptr(), LY._stream())
    e1.record()
    torch.cuda.synchronize()
    read_gbs = rbuf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    del rbuf, rfold
    # Matrix-core probe on the same GPU: back-to-back independent FP8 x FP4
    # block-scaled 16x16x128 MFMAs, two waves per SIMD on every CU.
    wg, iters = 2 * n_cu, 400
    mf = torch.empty(wg * 4, dtype=torch.float32, device="cuda")
    LY._lib.moe_mfma_rate_probe(20, wg, mf.data_ptr(), LY._stream())
    e0.record()
    LY._lib.moe_mfma_rate_probe(iters, wg, mf.data_ptr(), LY._stream())
    e1.record()
    torch.cuda.synchronize()
    mfma_tflops = wg * 4 * iters * 8 * (2 * 16 * 16 * 128) / (e0.elapsed_time(e1) / 1e3) / 1e12
    del mf
    cfg = synth.config(args.workload)
    t = time.perf_counter()
    shape = LY.LayerShape.of(cfg)
    workers = min(16, len(os.sched_getaffinity(0)))
    extra = {"w_router": synth.gen_router(cfg), "router_logit_bias": synth.gen_logit_bias(cfg)}
    weights = LY.encode_weights(shape, lambda n, i: synth.gen_weight(cfg, n, i), extra=extra, workers=workers,
                                progress=lambda j, n: say(f"  encoded {j}/{n} weight matrices "
                                                          f"({time.perf_counter() - t:.0f} s)"))
    say(f"K3 weights encoded on the GPU in {time.perf_counter() - t:.1f} s")

    cfg, ms, stages, work, counts = run_workload(args.workload, args.steps, args.warmup, weights, hip, say)
    value = cfg.T / (ms / 1e3)
    dom_ms = stages["expert_up"]
    tp = profiled_traffic(cfg.name)
    roof = {"bound": "mfma", "achieved": work["expert_up_launch_flops"] / (dom_ms / 1e3) / 1e12, "peak": PEAK_MX_TFLOPS,
            "unit": "TFLOP/s", "kernel": "expert_up (routed gate/up grouped GEMM + SwiGLU + MXFP8)",
            "traffic": None if tp is None else tp["bytes"],
            "algorithmic_bytes": work["expert_up_launch_bytes"]}
    roof["frac"] = roof["achieved"] / roof["peak"]
    out = {
        "metric": "LatentMoE layer tokens/s (K3 width); HBM GB/s decode, MFMA % prefill vs peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4xmxfp8",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,1/sqrt(fan_in)) weights encoded to MXFP4)",
        "config": {"workload": f"{cfg.name}: T={cfg.T}, d={cfg.d_model}, latent={cfg.d_latent}, "
                               f"E={cfg.n_routed} top-{cfg.top_k}, {cfg.n_shared} shared, "
                               f"d_ff={cfg.d_ff_routed}", "tokens": cfg.T, "parallelism": "single GPU"},
        "roofline": roof,
        "step_events_ms": work["step_events_ms"],
        "layer": {"mx_tflops": work["mx_flops"] / (ms / 1e3) / 1e12,
                  "mx_frac": work["mx_flops"] / (ms / 1e3) / 1e12 / PEAK_MX_TFLOPS,
                  "stage_ms": stages, "touched_experts": work["touched_experts"],
                  "max_expert_load": int(counts.max()), "empty_experts": int((counts == 0).sum())},
    }

    if not args.no_decode and args.workload != "k3_decode":
        dcfg, dms, dst, dwork, dcounts = run_workload("k3_decode", args.decode_steps, args.warmup, weights, hip, say)
        dom = dst["expert_up"]
        dtp = profiled_traffic(dcfg.name)
        droof = {"bound": "hbm", "achieved": dwork["expert_up_launch_bytes"] / (dom / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "kernel": "expert_up (routed gate/up weight-streaming GEMM + SwiGLU + MXFP8; the shared experts' gate/up rides in the same launch)",
                 "traffic": None if dtp is None else dtp["bytes"], "algorithmic_bytes": dwork["expert_up_launch_bytes"]}
        droof["frac"] = droof["achieved"] / droof["peak"]
        out["decode"] = {"workload": f"{dcfg.name}: T={dcfg.T}", "value": dcfg.T / (dms / 1e3), "unit": "tokens/s",
                         "ms_per_step": dms, "roofline": droof,
                         "layer_gbs": dwork["layer_bytes"] / (dms / 1e3) / 1e9,
                         "layer_hbm_frac": dwork["layer_bytes"] / (dms / 1e3) / 1e9 / PEAK_HBM_GBS,
                         "stage_ms": dst, "step_events_ms": dwork["step_events_ms"],
                         "touched_experts": dwork["touched_experts"]}
    if args.skew_steps > 0 and args.workload == "k3_prefill":
        scfg = synth.config("k3_skew")
        kcfg, kms, kst, kwork, kcounts = run_workload("k3_skew", args.skew_steps, args.warmup, weights, hip, say,
                                                      logit_bias=synth.gen_logit_bias(scfg))
        out["skew"] = {"workload": f"{kcfg.name}: T={kcfg.T}, Zipf(1.1) router logit bias", "value": kcfg.T / (kms / 1e3),
                       "unit": "tokens/s", "ms_per_step": kms,
                       "mx_frac": kwork["mx_flops"] / (kms / 1e3) / 1e12 / PEAK_MX_TFLOPS,
                       "expert_up_tflops": kwork["expert_up_launch_flops"] / (kst["expert_up"] / 1e3) / 1e12,
                       "max_expert_load": int(kcounts.max()), "mean_expert_load": float(kcounts.mean()),
                       "empty_experts": int((kcounts == 0).sum()), "stage_ms": kst,
                       "step_events_ms": kwork["step_events_ms"]}
    if args.bf16_steps > 0 and args.workload == "k3_prefill":
        out["bf16_map"] = bf16_map_report(weights, args.bf16_steps, args.decode_steps, args.warmup, hip, say)
    out["hbm_copy_probe_gbs"] = copy_gbs
    out["hbm_read_probe_gbs"] = read_gbs
    out["mfma_fp8xfp4_probe_tflops"] = mfma_tflops
    if args.workload == "k3_decode":
        dom = stages["expert_up"]
        tp = profiled_traffic(cfg.name)
        out["roofline"] = {"bound": "hbm", "achieved": work["expert_up_launch_bytes"] / (dom / 1e3) / 1e9,
                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "kernel": "expert_up (routed gate/up weight-streaming GEMM + SwiGLU + MXFP8; the shared experts' gate/up rides in the same launch)",
                           "traffic": None if tp is None else tp["bytes"],
                           "algorithmic_bytes": work["expert_up_launch_bytes"]}
        out["roofline"]["frac"] = out["roofline"]["achieved"] / PEAK_HBM_GBS

    del weights
    torch.cuda.empty_cache()
    if args.k2_steps > 0 and args.workload == "k3_prefill":
        out["k2"] = k2_report(args.k2_steps, args.warmup, hip, say)
    if args.small_steps > 0 and args.workload == "k3_prefill":
        for name in ("tiny", "mid"):
            out[name] = small_report(name, args.small_steps, args.warmup, hip, say)
    if args.ep8_steps > 0 and args.workload == "k3_prefill":
        out["ep8_share"] = ep8_share_report(args.ep8_steps, args.warmup, hip, say)
    if args.qb_steps > 0:
        out["quantile_balance"] = qb_report(args.qb_steps, args.warmup, say)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_tokens, say)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
