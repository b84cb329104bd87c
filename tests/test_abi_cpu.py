"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments before any launch."""

import ctypes
import glob
import os
import re

import pytest

from latent_routing_mxfp4_amd import _lib
from tests.conftest import ROOT

FAKE = 0x10000000  # aligned, never dereferenced by host-side validation


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", src, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared()
    assert declared == set(_lib.EXPORTED)
    for n in declared:
        assert hasattr(lib, n), n


def _k3(max_tokens=16384):
    return _lib.MoeLayerConfig(7168, 3584, 896, 16, 2, 3072, 3072, max_tokens)


def _weights(shared=True):
    t = _lib.MoeMxTensor(FAKE, FAKE)
    z = _lib.MoeMxTensor(None, None)
    s = t if shared else z
    return _lib.MoeLayerWeights(t, t, FAKE, None, None, t, t, t, s, s, s)


def _create_status(cfg, w):
    h = ctypes.c_void_p()
    st = _lib.load().moe_layer_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h))
    if st == 0:
        _lib.moe_layer_destroy(h.value)
    return st


def test_create_accepts_k3_and_rejects_bad_shapes():
    assert _create_status(_k3(), _weights()) == _lib.MOE_OK
    bad = [
        (dict(top_k=897), _lib.MOE_ERR_INVALID_ARG),
        (dict(top_k=0), _lib.MOE_ERR_INVALID_ARG),
        (dict(d_model=7200), _lib.MOE_ERR_UNSUPPORTED),
        (dict(d_latent=-128), _lib.MOE_ERR_INVALID_ARG),
        (dict(max_tokens=0), _lib.MOE_ERR_INVALID_ARG),
        (dict(n_shared=9), _lib.MOE_ERR_INVALID_ARG),
        (dict(n_routed=5000, top_k=16), _lib.MOE_ERR_UNSUPPORTED),
        (dict(top_k=65, n_routed=128), _lib.MOE_ERR_UNSUPPORTED),
    ]
    for change, want in bad:
        cfg = _k3()
        for k, v in change.items():
            setattr(cfg, k, v)
        assert _create_status(cfg, _weights()) == want, change


def test_create_rejects_null_and_misaligned_weights():
    w = _weights()
    w.w_router = None
    assert _create_status(_k3(), w) == _lib.MOE_ERR_INVALID_ARG
    w = _weights()
    w.w_gate_e = _lib.MoeMxTensor(FAKE + 8, FAKE)
    assert _create_status(_k3(), w) == _lib.MOE_ERR_INVALID_ARG
    # shared tensors may be NULL only when there are no shared experts
    assert _create_status(_k3(), _weights(shared=False)) == _lib.MOE_ERR_INVALID_ARG
    cfg = _k3()
    cfg.n_shared = 0
    assert _create_status(cfg, _weights(shared=False)) == _lib.MOE_OK
    h = ctypes.c_void_p()
    assert _lib.load().moe_layer_create(None, ctypes.byref(_weights()), ctypes.byref(h)) == _lib.MOE_ERR_INVALID_ARG


def test_workspace_size_is_monotone_and_bounded():
    cfg = _k3()
    sizes = [_lib.moe_layer_workspace_size(cfg, T) for T in (0, 1, 64, 4096, 16384)]
    assert sizes == sorted(sizes)
    assert sizes[-1] < 8 << 30  # prefill workspace stays a few GB
    with pytest.raises(_lib.MoEError) as e:
        _lib.moe_layer_workspace_size(cfg, 16385)
    assert e.value.status == _lib.MOE_ERR_INVALID_ARG


def test_forward_argument_errors_need_no_gpu():
    cfg = _k3(max_tokens=64)
    h = _lib.moe_layer_create(cfg, _weights())
    try:
        lib = _lib.load()
        need = _lib.moe_layer_workspace_size(cfg, 64)
        # T == 0 is a no-op, even with null buffers
        assert lib.moe_layer_forward(h, None, 0, None, None, 0, None, None) == _lib.MOE_OK
        assert lib.moe_layer_forward(None, FAKE, 1, FAKE, FAKE, need, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert lib.moe_layer_forward(h, FAKE, 65, FAKE, FAKE, need, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert lib.moe_layer_forward(h, FAKE, -1, FAKE, FAKE, need, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert lib.moe_layer_forward(h, None, 8, FAKE, FAKE, need, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert lib.moe_layer_forward(h, FAKE, 64, FAKE, None, need, None, None) == _lib.MOE_ERR_WORKSPACE
        assert lib.moe_layer_forward(h, FAKE, 64, FAKE, FAKE, need - 1, None, None) == _lib.MOE_ERR_WORKSPACE
        assert lib.moe_layer_forward(h, FAKE, 64, FAKE, FAKE + 64, need, None, None) == _lib.MOE_ERR_WORKSPACE
    finally:
        _lib.moe_layer_destroy(h)
    assert _lib.load().moe_layer_destroy(None) == _lib.MOE_OK


def test_noalloc_forward_argument_errors_need_no_gpu():
    """The no-allocation forward checks its arguments, and refuses a batch whose
    workspace exceeds the static scratch, before any HIP call."""
    cfg = _k3(max_tokens=16384)
    h = _lib.moe_layer_create(cfg, _weights())
    try:
        lib = _lib.load()
        fwd = lib.moe_layer_forward_noalloc
        assert fwd(h, None, 0, None, None, None) == _lib.MOE_OK
        assert fwd(None, FAKE, 1, FAKE, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert fwd(h, FAKE, 16385, FAKE, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert fwd(h, FAKE, 8, None, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert fwd(h, FAKE + 4, 8, FAKE, None, None) == _lib.MOE_ERR_INVALID_ARG
        assert _lib.moe_layer_workspace_size(cfg, 1024) > _lib.MOE_NOALLOC_SCRATCH_BYTES
        assert fwd(h, FAKE, 1024, FAKE, None, None) == _lib.MOE_ERR_WORKSPACE
        # the K3-width forward of up to 192 tokens fits the scratch
        assert _lib.moe_layer_workspace_size(cfg, 192) <= _lib.MOE_NOALLOC_SCRATCH_BYTES
    finally:
        _lib.moe_layer_destroy(h)


def test_quantize_and_gemm_argument_errors():
    lib = _lib.load()
    assert lib.moe_mx_quantize(FAKE, 4, 48, 0, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize(FAKE, 4, 64, 2, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize(None, 4, 64, 0, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize(FAKE, 0, 64, 0, FAKE, FAKE, None) == _lib.MOE_OK
    assert lib.moe_mx_gemm(FAKE, FAKE, FAKE, FAKE, 4, 16, 96, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_gemm(FAKE, FAKE, FAKE, FAKE, 4, 8, 128, FAKE, None) == _lib.MOE_ERR_INVALID_ARG  # N % 16
    assert lib.moe_mx_gemm(FAKE, FAKE, FAKE, FAKE, 0, 16, 128, FAKE, None) == _lib.MOE_OK
    assert lib.moe_mx_gemm(FAKE + 4, FAKE, FAKE, FAKE, 4, 16, 128, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    # fragment-order weights: N % 16, K % 128, pointers
    assert lib.moe_mx_quantize_weights(FAKE, 1, 8, 128, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize_weights(FAKE, 1, 16, 96, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize_weights(None, 1, 16, 128, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize_weights(FAKE, 0, 16, 128, FAKE, FAKE, None) == _lib.MOE_OK
    assert lib.moe_mx_pack_weights(FAKE, FAKE, 1, 24, 128, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_pack_weights(FAKE, FAKE, 1, 16, 64, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_pack_weights(FAKE + 4, FAKE, 1, 16, 128, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_pack_weights(FAKE, FAKE, 0, 16, 128, FAKE, FAKE, None) == _lib.MOE_OK
    assert _lib.moe_status_string(-3).startswith("workspace")


# --------------------------------------------------------------------------- higher-precision map


def _bf16_weights(shared=True, mx_dense=False):
    t = _lib.MoeMxTensor(FAKE, FAKE)
    z = _lib.MoeMxTensor(None, None)
    d = t if mx_dense else z
    w = _lib.MoeLayerWeights(d, d, FAKE, None, None, t, t, t, d, d, d)
    w.w_down_bf16 = w.w_up_bf16 = FAKE
    if shared:
        w.w_gate_s_bf16 = w.w_up_s_bf16 = w.w_down_s_bf16 = FAKE
    return w


def test_bf16_map_create_needs_bf16_dense_weights_only():
    cfg = _k3()
    cfg.dense_bf16 = 1
    assert _create_status(cfg, _bf16_weights()) == _lib.MOE_OK   # MX dense tensors may be NULL
    assert _create_status(cfg, _bf16_weights(shared=False)) == _lib.MOE_ERR_INVALID_ARG
    w = _bf16_weights()
    w.w_up_bf16 = FAKE + 2                                         # misaligned
    assert _create_status(cfg, w) == _lib.MOE_ERR_INVALID_ARG
    w = _bf16_weights()
    w.w_down_bf16 = None
    assert _create_status(cfg, w) == _lib.MOE_ERR_INVALID_ARG
    # without the flag the bf16 pointers are ignored and the MX ones required
    cfg.dense_bf16 = 0
    assert _create_status(cfg, _bf16_weights()) == _lib.MOE_ERR_INVALID_ARG
    assert _create_status(cfg, _bf16_weights(mx_dense=True)) == _lib.MOE_OK
    # the map is defined for the latent layer
    cfg = _lib.MoeLayerConfig(7168, 7168, 384, 8, 1, 2048, 2048, 64, 1, 1, 1)
    assert _create_status(cfg, _bf16_weights()) == _lib.MOE_ERR_UNSUPPORTED


def test_bf16_map_workspace_is_monotone():
    cfg = _k3()
    cfg.dense_bf16 = 1
    sizes = [_lib.moe_layer_workspace_size(cfg, T) for T in (0, 1, 64, 256, 257, 4096, 16384)]
    assert sizes[0] <= sizes[1] <= sizes[2] <= sizes[3]
    assert sizes[4] <= sizes[5] <= sizes[6] < 8 << 30


def test_round_bf16_argument_errors():
    lib = _lib.load()
    assert lib.moe_round_bf16(FAKE, 6, FAKE, None) == _lib.MOE_ERR_INVALID_ARG     # n % 4
    assert lib.moe_round_bf16(FAKE + 4, 8, FAKE, None) == _lib.MOE_ERR_INVALID_ARG # in alignment
    assert lib.moe_round_bf16(FAKE, 8, FAKE + 2, None) == _lib.MOE_ERR_INVALID_ARG # out alignment
    assert lib.moe_round_bf16(None, 8, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_round_bf16(FAKE, 0, FAKE, None) == _lib.MOE_OK


# --------------------------------------------------------------------------- layer without a latent


def test_non_latent_create_needs_no_latent_projections():
    """identity_latent: d_latent must equal d_model and W_down / W_up may be
    NULL; softmax_gates is a plain flag."""
    cfg = _lib.MoeLayerConfig(7168, 7168, 384, 8, 1, 2048, 2048, 8192, 1, 1, 0)
    t = _lib.MoeMxTensor(FAKE, FAKE)
    z = _lib.MoeMxTensor(None, None)
    w = _lib.MoeLayerWeights(z, z, FAKE, None, None, t, t, t, t, t, t)
    assert _create_status(cfg, w) == _lib.MOE_OK
    cfg.d_latent = 3584                              # a latent width without latent projections
    assert _create_status(cfg, w) == _lib.MOE_ERR_INVALID_ARG
    cfg.d_latent, cfg.identity_latent = 7168, 0      # a latent layer needs W_down and W_up
    assert _create_status(cfg, w) == _lib.MOE_ERR_INVALID_ARG


def test_non_latent_workspace_has_no_latent_buffers():
    """Without a latent the workspace holds no z, zq, y_lat or yq, so it is
    smaller than that of the latent layer of the same model width."""
    lat = _lib.MoeLayerConfig(7168, 7168, 384, 8, 1, 2048, 2048, 8192, 0, 1, 0)
    non = _lib.MoeLayerConfig(7168, 7168, 384, 8, 1, 2048, 2048, 8192, 1, 1, 0)
    for T in (1, 64, 8192):
        assert _lib.moe_layer_workspace_size(non, T) < _lib.moe_layer_workspace_size(lat, T)


def test_quantile_balance_rejects_bad_arguments_before_any_launch():
    lib = _lib.load()
    T, E, k = 16384, 896, 16
    need = lib.moe_quantile_balance_workspace_bytes(T, E)
    assert need == 4 * (2 * T + E * T)
    assert lib.moe_quantile_balance_workspace_bytes(-1, E) == 0

    def call(T=T, E=E, k=k, eta=0.5, ws=FAKE, ws_bytes=need, logits=FAKE, bias=FAKE, out=FAKE):
        return lib.moe_quantile_balance(logits, T, E, k, bias, eta, out, None, ws, ws_bytes, None)

    bad = _lib.MOE_ERR_INVALID_ARG
    assert call(T=1) == bad
    assert call(k=0) == bad and call(k=E) == bad
    assert call(E=4097, k=16) == bad
    assert call(eta=0.0) == bad and call(eta=1.5) == bad and call(eta=float("nan")) == bad
    assert call(logits=None) == bad and call(bias=None) == bad and call(out=None) == bad
    assert call(logits=FAKE + 2) == bad
    assert call(ws=None) == _lib.MOE_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == _lib.MOE_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == _lib.MOE_ERR_WORKSPACE


def test_weight_layout_and_workspace_bytes():
    """The config names the MX weight layout (row-major = 0, the zero default,
    or fragment order); any other value is refused.  moe_layer_workspace_bytes
    returns moe_layer_workspace_size's figure, and 0 where that is an error."""
    lib = _lib.load()
    for layout in (_lib.MOE_WEIGHTS_ROW_MAJOR, _lib.MOE_WEIGHTS_FRAGMENT):
        cfg = _k3()
        cfg.weight_layout = layout
        assert _create_status(cfg, _weights()) == _lib.MOE_OK
        for T in (0, 1, 64, 16384):
            assert _lib.moe_layer_workspace_bytes(cfg, T) == _lib.moe_layer_workspace_size(cfg, T)
    cfg = _k3()
    cfg.weight_layout = 2
    assert _create_status(cfg, _weights()) == _lib.MOE_ERR_INVALID_ARG
    assert _lib.moe_layer_workspace_bytes(cfg, 64) == 0
    assert _lib.moe_layer_workspace_bytes(_k3(), 16385) == 0
    assert lib.moe_layer_workspace_bytes(None, 64) == 0


def test_topk_stage_argument_errors_need_no_gpu():
    """The top-k stage entries check sizes and pointers before any HIP call."""
    lib = _lib.load()
    topk, fused = lib.moe_router_topk, lib.moe_router_reduce_topk
    E_ = _lib.MOE_ERR_INVALID_ARG
    assert topk(None, None, 0, 896, 16, 0, None, None, None) == _lib.MOE_OK       # T = 0: no-op
    assert topk(FAKE, None, 4, 896, 0, 0, FAKE, FAKE, None) == E_                  # k < 1
    assert topk(FAKE, None, 4, 896, 65, 0, FAKE, FAKE, None) == E_                 # k > 64
    assert topk(FAKE, None, 4, 8, 9, 0, FAKE, FAKE, None) == E_                    # k > E
    assert topk(FAKE, None, 4, 4097, 16, 0, FAKE, FAKE, None) == E_                # E > 4096
    assert topk(None, None, 4, 896, 16, 0, FAKE, FAKE, None) == E_                 # null logits
    assert topk(FAKE + 2, None, 4, 896, 16, 0, FAKE, FAKE, None) == E_             # misaligned
    assert topk(FAKE, FAKE + 1, 4, 896, 16, 0, FAKE, FAKE, None) == E_
    assert fused(None, 2, None, None, 0, 896, 16, 0, None, None, None, None) == _lib.MOE_OK
    assert fused(FAKE, 0, None, None, 4, 896, 16, 0, FAKE, FAKE, FAKE, None) == E_  # nz < 1
    assert fused(FAKE, 2, None, None, 4, 1025, 16, 0, FAKE, FAKE, FAKE, None) == E_  # E > 1024
    assert fused(FAKE, 2, None, None, 4, 896, 16, 0, None, FAKE, FAKE, None) == E_  # null logits out
    assert fused(FAKE, 2, FAKE + 2, None, 4, 896, 16, 0, FAKE, FAKE, FAKE, None) == E_
