"""Numpy statement of the fragment-order weight layout (include/moe_layer.h).

Used by the tests to build fragment-order inputs from row-major oracle codes
and to read GPU weight buffers back in row-major form.  Written from the
layout's definition, independently of the HIP quantiser and pack kernels.
"""

import numpy as np


def to_fragment_order(codes: np.ndarray, scales: np.ndarray):
    """Row-major E2M1 ``codes [..., N, K/2]`` and ``scales [..., N, K/32]`` ->
    the same shapes holding fragment-order bytes."""
    *lead, N, Kh = codes.shape
    K = 2 * Kh
    assert N % 16 == 0 and K % 128 == 0
    G = int(np.prod(lead)) if lead else 1
    c = codes.reshape(G, N // 16, 16, K // 128, 4, 16)        # g, nb, r, kb, q, byte
    c = c.transpose(0, 1, 3, 4, 2, 5)                         # g, nb, kb, q, r, byte  (lane = r + 16 q)
    s = scales.reshape(G, N, K // 128, 4).transpose(0, 2, 1, 3)  # g, kb, n, j
    return (np.ascontiguousarray(c).reshape(codes.shape), np.ascontiguousarray(s).reshape(scales.shape))


def from_fragment_order(codes: np.ndarray, scales: np.ndarray):
    """Inverse of ``to_fragment_order``."""
    *lead, N, Kh = codes.shape
    K = 2 * Kh
    G = int(np.prod(lead)) if lead else 1
    c = codes.reshape(G, N // 16, K // 128, 4, 16, 16).transpose(0, 1, 4, 2, 3, 5)
    s = scales.reshape(G, K // 128, N, 4).transpose(0, 2, 1, 3)
    return (np.ascontiguousarray(c).reshape(codes.shape), np.ascontiguousarray(s).reshape(scales.shape))
