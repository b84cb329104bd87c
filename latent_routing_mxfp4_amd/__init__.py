"""MI355X (gfx950) LatentMoE layer forward: MXFP4 weights x MXFP8 activations.

The compute lives in ``libmoe_layer.so`` (hand-written HIP kernels behind the C
ABI of ``include/moe_layer.h``); ``_lib`` is its ctypes binding and
``latent_routing_mxfp4_amd.layer`` a thin PyTorch-facing wrapper (device
memory and streams only; import it explicitly).
"""

from . import _lib  # noqa: F401
from ._lib import MoEError  # noqa: F401

__all__ = ["MoEError", "_lib"]
