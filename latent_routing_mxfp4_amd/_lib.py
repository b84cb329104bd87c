"""ctypes binding of ``libmoe_layer.so`` (declared in ``include/moe_layer.h``).

Argument marshalling only: every computation happens in the HIP library.
Functions keep the C names; a non-zero status raises ``MoEError``.  Pointers
are plain integers (device addresses, e.g. ``tensor.data_ptr()``), streams are
``hipStream_t`` handles as integers (``torch.cuda.current_stream().cuda_stream``).
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_layer.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_WEIGHTS_ROW_MAJOR = 0
MOE_WEIGHTS_FRAGMENT = 1

EXPORTED = (
    "moe_status_string",
    "moe_layer_create",
    "moe_layer_workspace_size",
    "moe_layer_workspace_bytes",
    "moe_layer_forward",
    "moe_layer_forward_noalloc",
    "moe_layer_destroy",
    "moe_mx_quantize",
    "moe_round_bf16",
    "moe_mx_quantize_weights",
    "moe_mx_pack_weights",
    "moe_mx_gemm",
    "moe_quantile_balance_workspace_bytes",
    "moe_quantile_balance",
    "moe_mfma_rate_probe",
    "moe_router_topk",
    "moe_router_reduce_topk",
    "moe_hbm_read_probe",
)


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)} ({status})")


class MoeLayerConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_model", "d_latent", "n_routed", "top_k", "n_shared", "d_ff_routed", "d_ff_shared", "max_tokens",
        "identity_latent", "softmax_gates", "dense_bf16", "weight_layout")]


class MoeMxTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class MoeLayerWeights(ctypes.Structure):
    _fields_ = [
        ("w_down", MoeMxTensor),
        ("w_up", MoeMxTensor),
        ("w_router", ctypes.c_void_p),
        ("router_logit_bias", ctypes.c_void_p),
        ("selection_bias", ctypes.c_void_p),
        ("w_gate_e", MoeMxTensor),
        ("w_up_e", MoeMxTensor),
        ("w_down_e", MoeMxTensor),
        ("w_gate_s", MoeMxTensor),
        ("w_up_s", MoeMxTensor),
        ("w_down_s", MoeMxTensor),
        # bfloat16 weights of the higher-precision map (dense_bf16)
        ("w_down_bf16", ctypes.c_void_p),
        ("w_up_bf16", ctypes.c_void_p),
        ("w_gate_s_bf16", ctypes.c_void_p),
        ("w_up_s_bf16", ctypes.c_void_p),
        ("w_down_s_bf16", ctypes.c_void_p),
    ]


TRACE_FIELDS = (
    "xq_codes", "xq_scales", "z", "zq_codes", "zq_scales", "logits", "ids", "gates", "counts", "offsets",
    "pair_of_row", "row_of_pair", "h", "hq_codes", "hq_scales", "y_e", "y_lat", "yq_codes", "yq_scales",
    "hs", "hs_codes", "hs_scales",
)


MOE_TRACE_EVENTS = 11
STAGES = ("quant_x", "down", "logits", "topk", "dispatch", "expert_up", "expert_down", "combine", "shared_up",
          "out")


# written instead of xq / yq / hs codes under the higher-precision map
BF16_TRACE_FIELDS = ("xb", "yb", "hs_bf16")


class MoeLayerTrace(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in TRACE_FIELDS] + [("events", ctypes.c_void_p)]
                + [(n, ctypes.c_void_p) for n in BF16_TRACE_FIELDS])


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_layer_create.restype = ctypes.c_int
    lib.moe_layer_create.argtypes = [ctypes.POINTER(MoeLayerConfig), ctypes.POINTER(MoeLayerWeights),
                                     ctypes.POINTER(vp)]
    lib.moe_layer_workspace_size.restype = ctypes.c_int
    lib.moe_layer_workspace_size.argtypes = [ctypes.POINTER(MoeLayerConfig), i32, ctypes.POINTER(sz)]
    lib.moe_layer_workspace_bytes.restype = sz
    lib.moe_layer_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayerConfig), i32]
    lib.moe_layer_forward.restype = ctypes.c_int
    lib.moe_layer_forward.argtypes = [vp, vp, i32, vp, vp, sz, vp, ctypes.POINTER(MoeLayerTrace)]
    lib.moe_layer_forward_noalloc.restype = ctypes.c_int
    lib.moe_layer_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, ctypes.POINTER(MoeLayerTrace)]
    lib.moe_layer_destroy.restype = ctypes.c_int
    lib.moe_layer_destroy.argtypes = [vp]
    lib.moe_mx_quantize.restype = ctypes.c_int
    lib.moe_mx_quantize.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.moe_mx_quantize_weights.restype = ctypes.c_int
    lib.moe_mx_quantize_weights.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.moe_mx_pack_weights.restype = ctypes.c_int
    lib.moe_mx_pack_weights.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
    lib.moe_mx_gemm.restype = ctypes.c_int
    lib.moe_mx_gemm.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp]
    lib.moe_router_topk.restype = ctypes.c_int
    lib.moe_router_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.moe_router_reduce_topk.restype = ctypes.c_int
    lib.moe_router_reduce_topk.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.moe_round_bf16.restype = ctypes.c_int
    lib.moe_round_bf16.argtypes = [vp, i64, vp, vp]
    lib.moe_quantile_balance_workspace_bytes.restype = sz
    lib.moe_quantile_balance_workspace_bytes.argtypes = [i32, i32]
    lib.moe_mfma_rate_probe.restype = ctypes.c_int
    lib.moe_mfma_rate_probe.argtypes = [i32, i32, vp, vp]
    lib.moe_hbm_read_probe.restype = ctypes.c_int
    lib.moe_hbm_read_probe.argtypes = [vp, sz, i32, vp, vp]
    lib.moe_quantile_balance.restype = ctypes.c_int
    lib.moe_quantile_balance.argtypes = [vp, i32, i32, i32, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, where)


def moe_status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def moe_layer_create(cfg: MoeLayerConfig, weights: MoeLayerWeights) -> int:
    h = ctypes.c_void_p()
    _check(load().moe_layer_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h)), "moe_layer_create")
    return h.value


def moe_layer_workspace_size(cfg: MoeLayerConfig, T: int) -> int:
    n = ctypes.c_size_t()
    _check(load().moe_layer_workspace_size(ctypes.byref(cfg), int(T), ctypes.byref(n)), "moe_layer_workspace_size")
    return n.value


def moe_layer_workspace_bytes(cfg: MoeLayerConfig, T: int) -> int:
    return int(load().moe_layer_workspace_bytes(ctypes.byref(cfg), int(T)))


def moe_layer_forward(handle: int, x: int, T: int, y: int, ws: int, ws_bytes: int, stream: int = 0,
                      trace: MoeLayerTrace | None = None) -> None:
    tr = ctypes.byref(trace) if trace is not None else None
    _check(load().moe_layer_forward(handle, x, int(T), y, ws, int(ws_bytes), stream, tr), "moe_layer_forward")


MOE_NOALLOC_SCRATCH_BYTES = 96 << 20


def moe_layer_forward_noalloc(handle: int, x: int, T: int, y: int, stream: int = 0,
                              trace: MoeLayerTrace | None = None) -> None:
    tr = ctypes.byref(trace) if trace is not None else None
    _check(load().moe_layer_forward_noalloc(handle, x, int(T), y, stream, tr), "moe_layer_forward_noalloc")


def moe_layer_destroy(handle: int) -> None:
    _check(load().moe_layer_destroy(handle), "moe_layer_destroy")


def moe_mx_quantize(src: int, rows: int, K: int, fmt: int, codes: int, scales: int, stream: int = 0) -> None:
    _check(load().moe_mx_quantize(src, int(rows), int(K), int(fmt), codes, scales, stream), "moe_mx_quantize")


def moe_mx_quantize_weights(src: int, G: int, N: int, K: int, codes: int, scales: int, stream: int = 0) -> None:
    _check(load().moe_mx_quantize_weights(src, int(G), int(N), int(K), codes, scales, stream),
           "moe_mx_quantize_weights")


def moe_mx_pack_weights(codes: int, scales: int, G: int, N: int, K: int, out_codes: int, out_scales: int,
                        stream: int = 0) -> None:
    _check(load().moe_mx_pack_weights(codes, scales, int(G), int(N), int(K), out_codes, out_scales, stream),
           "moe_mx_pack_weights")


def moe_mx_gemm(a_codes: int, a_scales: int, b_codes: int, b_scales: int, M: int, N: int, K: int, c: int,
                stream: int = 0) -> None:
    _check(load().moe_mx_gemm(a_codes, a_scales, b_codes, b_scales, int(M), int(N), int(K), c, stream),
           "moe_mx_gemm")


def moe_router_topk(logits: int, selection_bias: int, T: int, E: int, k: int, softmax_gates: bool, ids: int,
                    gates: int, stream: int = 0) -> None:
    _check(load().moe_router_topk(logits, selection_bias, int(T), int(E), int(k), int(bool(softmax_gates)), ids,
                                  gates, stream), "moe_router_topk")


def moe_router_reduce_topk(partial: int, nz: int, logit_bias: int, selection_bias: int, T: int, E: int, k: int,
                           softmax_gates: bool, logits: int, ids: int, gates: int, stream: int = 0) -> None:
    _check(load().moe_router_reduce_topk(partial, int(nz), logit_bias, selection_bias, int(T), int(E), int(k),
                                         int(bool(softmax_gates)), logits, ids, gates, stream),
           "moe_router_reduce_topk")


def moe_round_bf16(src: int, n: int, out: int, stream: int = 0) -> None:
    _check(load().moe_round_bf16(src, int(n), out, stream), "moe_round_bf16")


def moe_quantile_balance_workspace_bytes(T: int, E: int) -> int:
    return int(load().moe_quantile_balance_workspace_bytes(int(T), int(E)))


def moe_quantile_balance(logits: int, T: int, E: int, k: int, bias_in: int, eta: float, bias_out: int,
                         quantile_out: int, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check(load().moe_quantile_balance(logits, int(T), int(E), int(k), bias_in, float(eta), bias_out,
                                       quantile_out, ws, int(ws_bytes), stream), "moe_quantile_balance")


def moe_hbm_read_probe(buf: int, nbytes: int, workgroups: int, out: int, stream: int = 0) -> None:
    _check(load().moe_hbm_read_probe(buf, int(nbytes), int(workgroups), out, stream), "moe_hbm_read_probe")


def moe_mfma_rate_probe(iters: int, workgroups: int, out: int, stream: int = 0) -> None:
    _check(load().moe_mfma_rate_probe(int(iters), int(workgroups), out, stream), "moe_mfma_rate_probe")
