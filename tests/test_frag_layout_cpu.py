"""Pins of the fragment-order layout helper against the layout's definition."""

import numpy as np

from oracle import mx
from tests.frag_layout import from_fragment_order, to_fragment_order


def test_element_positions_follow_the_definition():
    # Every E2M1 element of a 2 x 48 x 384 stack, located one by one: row n,
    # element k of matrix g lands in byte (nb*(K/128) + kb)*1024 + 16*(r + 16q)
    # + (k%32)//2 of matrix g, nibble k%2, with nb, r = divmod(n, 16),
    # kb = k//128, q = (k%128)//32.
    G, N, K = 2, 48, 384
    rng = np.random.default_rng(3)
    elems = rng.integers(0, 16, (G, N, K)).astype(np.uint8)
    codes = mx.pack_e2m1(elems)
    scales = rng.integers(0, 256, (G, N, K // 32)).astype(np.uint8)
    fc, fs = to_fragment_order(codes, scales)
    flat_c, flat_s = fc.reshape(G, -1), fs.reshape(G, -1)
    for g in range(G):
        for n in range(N):
            nb, r = divmod(n, 16)
            for k in range(0, K, 7):
                kb, q = k // 128, (k % 128) // 32
                byte = (nb * (K // 128) + kb) * 1024 + 16 * (r + 16 * q) + (k % 32) // 2
                nib = (flat_c[g, byte] >> (4 * (k % 2))) & 0xF
                assert nib == elems[g, n, k], (g, n, k)
            for j in range(K // 32):
                kb, jj = divmod(j, 4)
                assert flat_s[g, (kb * N + n) * 4 + jj] == scales[g, n, j]


def test_round_trip_and_sizes():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (3, 32, 256)).astype(np.uint8)     # N = 32, K = 512
    scales = rng.integers(0, 256, (3, 32, 16)).astype(np.uint8)
    fc, fs = to_fragment_order(codes, scales)
    assert fc.shape == codes.shape and fs.shape == scales.shape
    bc, bs = from_fragment_order(fc, fs)
    assert np.array_equal(bc, codes) and np.array_equal(bs, scales)
    # a single matrix is laid out exactly like one member of a stack
    f1, s1 = to_fragment_order(codes[1], scales[1])
    assert np.array_equal(f1, fc[1]) and np.array_equal(s1, fs[1])
