"""The forward that allocates nothing (``moe_layer_forward_noalloc``): its
workspace is the library's static per-GPU scratch instead of a caller's
buffer.  Through the C ABI, two calls in a row -- the second on a smaller
batch, so the scratch holds a different layout of the first call's
intermediates -- must give exactly what ``moe_layer_forward`` gives with a
fresh workspace of its own (same kernels: bit for bit), for the latent layer,
its higher-precision map and the layer without a latent.  A batch whose
workspace exceeds the scratch is refused before any launch."""

import ctypes

import numpy as np
import pytest

import synth
from latent_routing_mxfp4_amd import _lib
from tests.gpu_harness import gpu_weights, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _layer(name, max_tokens):
    from latent_routing_mxfp4_amd import layer as LY
    cfg = synth.config(name)
    shape, w = gpu_weights(cfg, workers=8)
    return LY.LatentMoE(shape, w, max_tokens), cfg


def _both(lay, x, tr_fields=("ids", "hq_codes", "y_lat")):
    """y from moe_layer_forward (fresh workspace) and from the no-alloc entry
    point, plus a few traced intermediates of each."""
    T = x.shape[0]
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for noalloc in (False, True):
        y = torch.full_like(x, float("nan"))
        full = lay.trace_buffers(T)
        tb = {n: full[n] for n in tr_fields if n in full}
        tr = _lib.MoeLayerTrace(*[tb[n].data_ptr() if n in tb else None for n in _lib.TRACE_FIELDS], None,
                                *[None for _ in _lib.BF16_TRACE_FIELDS])
        if noalloc:
            st = _lib.load().moe_layer_forward_noalloc(lay.handle, x.data_ptr(), T, y.data_ptr(), stream,
                                                       ctypes.byref(tr))
        else:
            ws = torch.empty(max(lay.workspace_bytes(T), 256), dtype=torch.uint8, device="cuda")
            st = _lib.load().moe_layer_forward(lay.handle, x.data_ptr(), T, y.data_ptr(), ws.data_ptr(),
                                               ws.numel(), stream, ctypes.byref(tr))
        assert st == _lib.MOE_OK, _lib.moe_status_string(st)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), {n: v.cpu().numpy() for n, v in tb.items()}))
    return out


@pytest.mark.parametrize("name,sizes", [("tiny", (64, 17)), ("mid", (200, 48)), ("tiny_bf16", (64, 5)),
                                        ("k2_tiny", (64, 33))])
def test_noalloc_forward_equals_the_workspace_forward(name, sizes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lay, cfg = _layer(name, max(sizes))
    for T in sizes:
        need = lay.workspace_bytes(T)
        say(f"no-alloc forward {name}: T={T}, workspace {need} bytes of {_lib.MOE_NOALLOC_SCRATCH_BYTES}")
        assert need <= _lib.MOE_NOALLOC_SCRATCH_BYTES
        x = torch.from_numpy(synth.gen_hidden(cfg, T=T)).cuda()
        (y0, t0), (y1, t1) = _both(lay, x)
        assert np.all(np.isfinite(y1))
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"{name} T={T}: outputs differ"
        for n in t0:
            assert np.array_equal(t0[n], t1[n]), f"{name} T={T}: traced {n} differs"
    lay.close()


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lay, cfg = _layer("mid", 4096)
    T = 4096
    need = lay.workspace_bytes(T)
    say(f"no-alloc forward mid: T={T} needs {need} bytes > {_lib.MOE_NOALLOC_SCRATCH_BYTES}: refused")
    assert need > _lib.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, cfg.d_model, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    st = _lib.load().moe_layer_forward_noalloc(lay.handle, x.data_ptr(), T, y.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    lay.close()
