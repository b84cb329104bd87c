"""PyTorch-facing wrapper of the HIP LatentMoE layer.

PyTorch provides device memory and the current HIP stream; every step of the
layer runs in ``libmoe_layer.so``.  Nothing here computes layer values.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, Optional, Tuple

import numpy as np
import torch

from . import _lib

FMT_E4M3 = 0
FMT_E2M1 = 1

ROUTED = ("w_gate_e", "w_up_e", "w_down_e")
SHARED = ("w_gate_s", "w_up_s", "w_down_s")
DENSE = ("w_down", "w_up")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d_model: int
    d_latent: int
    n_routed: int
    top_k: int
    n_shared: int
    d_ff_routed: int
    d_ff_shared: int
    latent: bool = True          # False: no latent projections (d_latent == d_model)
    softmax_gates: bool = False  # gates = softmax over the winners' logits
    dense_bf16: bool = False     # latent projections and shared experts in bfloat16
    weight_layout: int = _lib.MOE_WEIGHTS_FRAGMENT   # or MOE_WEIGHTS_ROW_MAJOR ([out][in] as stored)

    @classmethod
    def of(cls, cfg, weight_layout: int = _lib.MOE_WEIGHTS_FRAGMENT) -> "LayerShape":
        return cls(cfg.d_model, cfg.d_latent, cfg.n_routed, cfg.top_k, cfg.n_shared, cfg.d_ff_routed,
                   cfg.d_ff_shared, bool(getattr(cfg, "latent", True)), getattr(cfg, "gating", "sigmoid") == "softmax",
                   getattr(cfg, "precision", "mx") == "bf16", int(weight_layout))

    def matrix_shape(self, name: str) -> Tuple[int, int]:
        d, L, F, Fs = self.d_model, self.d_latent, self.d_ff_routed, self.d_ff_shared
        return {"w_down": (L, d), "w_up": (d, L), "w_gate_e": (F, L), "w_up_e": (F, L), "w_down_e": (L, F),
                "w_gate_s": (Fs, d), "w_up_s": (Fs, d), "w_down_s": (d, Fs)}[name]

    def count(self, name: str) -> int:
        return self.n_routed if name in ROUTED else self.n_shared if name in SHARED else int(self.latent)

    def is_bf16(self, name: str) -> bool:
        """Stored as bfloat16 (the higher-precision map) rather than MXFP4."""
        return self.dense_bf16 and name not in ROUTED

    def c_config(self, max_tokens: int) -> _lib.MoeLayerConfig:
        return _lib.MoeLayerConfig(self.d_model, self.d_latent, self.n_routed, self.top_k, self.n_shared,
                                   self.d_ff_routed, self.d_ff_shared, int(max_tokens), int(not self.latent),
                                   int(self.softmax_gates), int(self.dense_bf16), int(self.weight_layout))


# --------------------------------------------------------------------------- MX helpers


def mx_quantize(x: torch.Tensor, fmt: int, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """MX-encode an fp32 CUDA tensor along its last axis; returns (codes, scales)."""
    assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()
    K = x.shape[-1]
    rows = x.numel() // K if K else 0
    if out is None:
        codes = torch.empty(*x.shape[:-1], K if fmt == FMT_E4M3 else K // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out
    _lib.moe_mx_quantize(x.data_ptr(), rows, K, fmt, codes.data_ptr(), scales.data_ptr(), _stream())
    return codes, scales


def mx_quantize_weights(x: torch.Tensor, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """MXFP4-encode fp32 weight matrices ``x`` ([N][K] or [G][N][K], CUDA) in
    fragment order; returns (codes, scales) shaped like the row-major result
    ([..., N, K/2] and [..., N, K/32]) but holding the permuted bytes."""
    assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.dim() in (2, 3)
    N, K = x.shape[-2], x.shape[-1]
    G = x.shape[0] if x.dim() == 3 else 1
    if out is None:
        codes = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out
    _lib.moe_mx_quantize_weights(x.data_ptr(), G, N, K, codes.data_ptr(), scales.data_ptr(), _stream())
    return codes, scales


def mx_pack_weights(codes: torch.Tensor, scales: torch.Tensor):
    """Row-major E2M1 ([..., N, K/2] codes, [..., N, K/32] scales) -> fragment order."""
    N, K = codes.shape[-2], codes.shape[-1] * 2
    G = codes.numel() // (N * K // 2)
    oc, os_ = torch.empty_like(codes), torch.empty_like(scales)
    _lib.moe_mx_pack_weights(codes.data_ptr(), scales.data_ptr(), G, N, K, oc.data_ptr(), os_.data_ptr(), _stream())
    return oc, os_


def mx_gemm(a_codes, a_scales, b_codes, b_scales) -> torch.Tensor:
    """fp32 deq(a) @ deq(b)^T with a E4M3 [M][K] (row-major) and b E2M1 [N][K]
    in fragment order (as from ``mx_quantize_weights``)."""
    M, K = a_codes.shape
    N = b_codes.shape[0]
    c = torch.empty(M, N, dtype=torch.float32, device=a_codes.device)
    _lib.moe_mx_gemm(a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(), b_scales.data_ptr(), M, N, K,
                     c.data_ptr(), _stream())
    return c


def quantile_balance(logits: torch.Tensor, bias: torch.Tensor, k: int, eta: float = 1.0,
                     out: Optional[torch.Tensor] = None, quantiles: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One Quantile Balancing step (``moe_quantile_balance``): the new fp32
    selection bias [E] from router logits [T][E] and the current bias.
    ``out`` may be ``bias`` itself; ``quantiles`` ([E] fp32) receives Q."""
    T, E = logits.shape
    assert logits.dtype == torch.float32 and logits.is_contiguous() and bias.dtype == torch.float32
    if out is None:
        out = torch.empty_like(bias)
    nbytes = _lib.moe_quantile_balance_workspace_bytes(T, E)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=logits.device)
    _lib.moe_quantile_balance(logits.data_ptr(), T, E, int(k), bias.data_ptr(), float(eta), out.data_ptr(),
                              0 if quantiles is None else quantiles.data_ptr(), workspace.data_ptr(), nbytes,
                              _stream())
    return out


def encode_weights(shape: LayerShape, host_fp32: Callable[[str, int], np.ndarray], device="cuda",
                   extra: Optional[Dict[str, Optional[np.ndarray]]] = None, workers: int = 8,
                   progress: Optional[Callable[[int, int], None]] = None,
                   names: Optional[Tuple[str, ...]] = None) -> Dict:
    """Encode every weight matrix on the GPU.

    ``host_fp32(name, index)`` returns the fp32 ``[out][in]`` matrix (numpy);
    matrices are produced by a thread pool, copied to the device one at a
    time and encoded there to MXFP4 in the shape's weight layout: row-major
    (``moe_mx_quantize``) or fragment order (``moe_mx_quantize_weights``).  Under the
    higher-precision map the latent projections and shared experts are
    rounded to bfloat16 instead (``moe_round_bf16``), stored row-major under
    ``<name>_bf16`` (their MX entries are None).
    ``extra`` carries the fp32 router (``w_router``) and the optional biases;
    ``names`` restricts the encoding to those weight names (e.g. the bfloat16
    ones, to pair with routed experts encoded before).
    """
    out: Dict = {}
    jobs = []
    for name in names if names is not None else DENSE + ROUTED + SHARED:
        n = shape.count(name)
        stacked = name in ROUTED + SHARED
        if shape.is_bf16(name):
            out[name] = None
            if n == 0:
                out[name + "_bf16"] = None
                continue
            r, c = shape.matrix_shape(name)
            wb = torch.empty(n, r, c, dtype=torch.int16, device=device)
            out[name + "_bf16"] = wb if stacked else wb[0]
            jobs += [(name, i, wb[i], None) for i in range(n)]
            continue
        if n == 0:
            out[name] = None
            continue
        r, c = shape.matrix_shape(name)
        codes = torch.empty(n, r, c // 2, dtype=torch.uint8, device=device)
        scales = torch.empty(n, r, c // 32, dtype=torch.uint8, device=device)
        out[name] = (codes if stacked else codes[0], scales if stacked else scales[0])
        jobs += [(name, i, codes[i], scales[i]) for i in range(n)]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(host_fp32, name, i) for (name, i, _, _) in jobs[:2 * workers]]
        nxt = len(futs)
        for j, (name, i, codes, scales) in enumerate(jobs):
            host = futs[j].result()
            futs[j] = None
            if nxt < len(jobs):
                futs.append(ex.submit(host_fp32, jobs[nxt][0], jobs[nxt][1]))
                nxt += 1
            dev = torch.from_numpy(np.ascontiguousarray(host, dtype=np.float32)).to(device, non_blocking=False)
            if scales is None:
                _lib.moe_round_bf16(dev.data_ptr(), dev.numel(), codes.data_ptr(), _stream())
            elif shape.weight_layout == _lib.MOE_WEIGHTS_ROW_MAJOR:
                mx_quantize(dev, FMT_E2M1, out=(codes, scales))
            else:
                mx_quantize_weights(dev, out=(codes, scales))
            if progress is not None and (j + 1) % max(1, len(jobs) // 10) == 0:
                progress(j + 1, len(jobs))
    extra = extra or {}
    for k in ("w_router", "router_logit_bias", "selection_bias"):
        if names is not None and k not in extra:
            continue
        v = extra.get(k)
        out[k] = None if v is None else torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device)
    torch.cuda.synchronize()
    return out


# --------------------------------------------------------------------------- the layer


class LatentMoE:
    """Handle around ``moe_layer_create`` / ``moe_layer_forward``.

    ``weights`` maps each weight name to ``(codes, scales)`` CUDA uint8 tensors
    (routed/shared groups with a leading expert axis), ``w_router`` to an fp32
    tensor, and the optional biases to fp32 tensors or None.
    """

    def __init__(self, shape: LayerShape, weights: Dict, max_tokens: int):
        self.shape = shape
        self.max_tokens = int(max_tokens)
        self.weights = weights  # keep the tensors alive: the handle does not own them
        self._cfg = shape.c_config(max_tokens)

        def mx(name):
            v = weights.get(name)
            if v is None:
                return _lib.MoeMxTensor(None, None)
            return _lib.MoeMxTensor(v[0].data_ptr(), v[1].data_ptr())

        self._w = _lib.MoeLayerWeights(
            mx("w_down"), mx("w_up"), _ptr(weights["w_router"]), _ptr(weights.get("router_logit_bias")),
            _ptr(weights.get("selection_bias")), mx("w_gate_e"), mx("w_up_e"), mx("w_down_e"), mx("w_gate_s"),
            mx("w_up_s"), mx("w_down_s"), *[_ptr(weights.get(n + "_bf16")) for n in DENSE + SHARED])
        self.handle = _lib.moe_layer_create(self._cfg, self._w)
        self._ws: Optional[torch.Tensor] = None

    def workspace_bytes(self, T: int) -> int:
        return _lib.moe_layer_workspace_size(self._cfg, T)

    def workspace(self, T: int) -> torch.Tensor:
        need = self.workspace_bytes(T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        return self._ws

    def trace_buffers(self, T: int) -> Dict[str, torch.Tensor]:
        s = self.shape
        d, L, E, k, F, S, Fs = s.d_model, s.d_latent, s.n_routed, s.top_k, s.d_ff_routed, s.n_shared, s.d_ff_shared
        P = T * k
        u8, i32, f32 = torch.uint8, torch.int32, torch.float32
        shapes = {
            "xq_codes": ((T, d), u8), "xq_scales": ((T, d // 32), u8), "z": ((T, L), f32),
            "zq_codes": ((T, L), u8), "zq_scales": ((T, L // 32), u8), "logits": ((T, E), f32),
            "ids": ((T, k), i32), "gates": ((T, k), f32), "counts": ((E,), i32), "offsets": ((E + 1,), i32),
            "pair_of_row": ((P,), i32), "row_of_pair": ((P,), i32), "h": ((P, F), f32), "hq_codes": ((P, F), u8),
            "hq_scales": ((P, F // 32), u8), "y_e": ((P, L), f32), "y_lat": ((T, L), f32),
            "yq_codes": ((T, L), u8), "yq_scales": ((T, L // 32), u8),
        }
        if not s.latent:  # no MXFP8 of the combined output: it is y's routed part
            del shapes["yq_codes"], shapes["yq_scales"]
        if s.dense_bf16:  # bf16 inputs of the higher-precision GEMMs instead of MXFP8 ones
            del shapes["xq_codes"], shapes["xq_scales"], shapes["yq_codes"], shapes["yq_scales"]
            shapes["xb"] = ((T, d), torch.int16)
            shapes["yb"] = ((T, L), torch.int16)
        if S > 0:
            shapes["hs"] = ((S, T, Fs), f32)
            if s.dense_bf16:
                shapes["hs_bf16"] = ((S, T, Fs), torch.int16)
            else:
                shapes["hs_codes"] = ((S, T, Fs), u8)
                shapes["hs_scales"] = ((S, T, Fs // 32), u8)
        return {n: torch.empty(sh, dtype=dt, device="cuda") for n, (sh, dt) in shapes.items()}

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, trace: Optional[Dict] = None,
                stream: Optional[int] = None) -> torch.Tensor:
        assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.dim() == 2
        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        ws = self.workspace(T)
        tr = None
        if trace is not None:
            tr = _lib.MoeLayerTrace(*[_ptr(trace.get(n)) for n in _lib.TRACE_FIELDS], None,
                                    *[_ptr(trace.get(n)) for n in _lib.BF16_TRACE_FIELDS])
        _lib.moe_layer_forward(self.handle, x.data_ptr(), T, y.data_ptr(), ws.data_ptr(), ws.numel(),
                               _stream() if stream is None else stream, tr)
        return y

    def close(self) -> None:
        if self.handle:
            _lib.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
