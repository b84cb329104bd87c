"""MX (microscaling) block formats: element codecs, the block quantiser, MX matmul.

TEST INFRASTRUCTURE ONLY.  This module is part of the CPU oracle: plain, slow,
fp64.  Only the test-suite, the package smoke check and the benchmark's
CPU-baseline leg may import it; the GPU library never does.

What the pages fix
------------------
* Kimi K3: 2.8 Trillion Parameters, Four Bits at a Time, section "Four bits
  from the start": an MX block is 32 elements that share one 8-bit
  power-of-two scale; an MXFP4 element is E2M1 (one sign, two exponent, one
  mantissa bit) whose magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6; a block costs
  136 bits.  The quantisation experiment in that section sets the shared
  exponent to floor(log2(amax)) minus the element format's largest exponent
  (2 for E2M1), divides by the power-of-two scale, clips to the largest element
  magnitude and rounds to the nearest grid level.
* Kimi K3 and the New Open-Weights Moat, section "Precision and deployment"
  (Fig. 6): MXFP8 uses E4M3 elements; the element encodings come from the OCP
  Microscaling Formats specification that page cites.

Readings where the pages are silent (each is listed in the design notes)
-----------------------------------------------------------------------
* Element rounding is round-to-nearest with ties to the even code (the code
  whose least significant bit is 0).  The page's nearest-level search would
  resolve exact ties toward the smaller magnitude instead; the two differ only
  at exact midpoints.
* E4M3 is the OCP "FN" variant: bias 7, no infinities, S.1111.111 is NaN, the
  largest finite magnitude is 448.  The E4M3 shared exponent subtracts 8 (its
  largest normal exponent), values clip to 448, and NaN is never produced.
* The shared exponent is clamped to the E8M0 range [-127, 127]; an all-zero
  block therefore gets scale code 0 (2^-127) and zero elements.
* The element sign bit is the sign bit of the input value, also when the
  magnitude rounds to zero.
* E2M1 codes are packed two per byte, the even-indexed element in the low
  nibble; scales are stored one byte per block, row-major ``[rows][K/32]``.
* Inputs must be finite.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32

# --------------------------------------------------------------------------- codecs


def _decode_minifloat(code: int, ebits: int, mbits: int, bias: int) -> float:
    """Value of a sign/exponent/mantissa code (no inf/NaN handling here)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:   # subnormal: 0.m * 2^(1-bias)
        mag = (m / (1 << mbits)) * 2.0 ** (1 - bias)
    else:        # normal: 1.m * 2^(e-bias)
        mag = (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return -mag if s else mag


def e2m1_table() -> np.ndarray:
    """fp64 value of each of the 16 E2M1 codes (1 sign, 2 exponent bits with bias 1, 1 mantissa bit)."""
    return np.array([_decode_minifloat(c, 2, 1, 1) for c in range(16)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """fp64 value of each of the 256 E4M3 (OCP FN) codes; S.1111.111 decodes to NaN."""
    t = np.array([_decode_minifloat(c, 4, 3, 7) for c in range(256)], dtype=np.float64)
    t[0x7F] = np.nan
    t[0xFF] = np.nan
    return t


def e8m0_table() -> np.ndarray:
    """fp64 value of each of the 256 E8M0 scale codes: 2^(c-127); 0xFF is NaN."""
    t = np.array([2.0 ** (c - 127) for c in range(256)], dtype=np.float64)
    t[0xFF] = np.nan
    return t


class ElemFormat:
    """One MX element format: its positive grid (indexed by magnitude code)."""

    def __init__(self, name: str, table: np.ndarray, sign_bit: int, max_code: int, emax: int):
        self.name = name
        self.table = table
        self.sign_bit = sign_bit          # value of the sign bit in a code
        self.max_code = max_code          # largest finite magnitude code
        self.emax = emax                  # exponent of the largest normal binade
        self.levels = table[: max_code + 1].copy()   # magnitudes for codes 0..max_code, increasing
        assert np.all(np.diff(self.levels) > 0)
        self.max_value = float(self.levels[-1])


E2M1 = ElemFormat("e2m1", e2m1_table(), sign_bit=0x8, max_code=0x7, emax=2)
E4M3 = ElemFormat("e4m3", e4m3_table(), sign_bit=0x80, max_code=0x7E, emax=8)
FORMATS = {"e2m1": E2M1, "e4m3": E4M3}
E8M0 = e8m0_table()


def _fmt(fmt) -> ElemFormat:
    return FORMATS[fmt] if isinstance(fmt, str) else fmt


# --------------------------------------------------------------------------- quantiser


def shared_exponent(amax: np.ndarray, emax: int) -> np.ndarray:
    """floor(log2(amax)) - emax, clamped to the E8M0 range; amax == 0 gives -127.

    floor(log2(a)) is taken exactly from the binary exponent: frexp(a) = (m, ex)
    with m in [0.5, 1) means a lies in [2^(ex-1), 2^ex).
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = ex.astype(np.int64) - 1 - emax
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127)


def round_to_grid(y: np.ndarray, fmt) -> np.ndarray:
    """Magnitude code of the grid level nearest to y >= 0 (y already clipped); ties -> even code."""
    f = _fmt(fmt)
    lv = f.levels
    y = np.asarray(y, dtype=np.float64)
    hi = np.searchsorted(lv, y, side="left")           # lv[hi-1] < y <= lv[hi]
    hi = np.clip(hi, 0, len(lv) - 1)
    lo = np.clip(hi - 1, 0, len(lv) - 1)
    d_lo = np.abs(y - lv[lo])
    d_hi = np.abs(lv[hi] - y)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.uint8)


def encode_with_exponent(v: np.ndarray, e: np.ndarray, fmt) -> np.ndarray:
    """Element codes of ``v`` (blocks of 32 along the last axis) under given
    block exponents ``e`` (shape ``v.shape[:-1] + (K/32,)``): divide by 2^e,
    clip to the largest magnitude, round to the nearest level (ties to even)."""
    f = _fmt(fmt)
    v64 = np.asarray(v).astype(np.float64)
    nb = v64.shape[-1] // BLOCK
    blocks = v64.reshape(v64.shape[:-1] + (nb, BLOCK))
    scale = np.ldexp(1.0, np.asarray(e))                      # exact power of two
    y = np.abs(blocks) / scale[..., None]                      # exact (power-of-two division)
    y = np.minimum(y, f.max_value)                             # clip to the largest magnitude
    mag = round_to_grid(y, f)
    codes = np.where(np.signbit(blocks), mag | f.sign_bit, mag).astype(np.uint8)
    return codes.reshape(v64.shape)


def quantize(v: np.ndarray, fmt) -> tuple:
    """Quantise ``v`` (any float array, last axis a multiple of 32) to MX blocks.

    Returns ``(codes, scales)``: codes uint8 of v's shape (one code per element,
    unpacked), scales uint8 of shape ``v.shape[:-1] + (K/32,)``.
    """
    f = _fmt(fmt)
    v = np.asarray(v)
    assert v.shape[-1] % BLOCK == 0, "the blocked axis must be a multiple of 32"
    v64 = v.astype(np.float64)
    assert np.all(np.isfinite(v64)), "MX quantisation of non-finite values is not defined here"
    nb = v.shape[-1] // BLOCK
    amax = np.abs(v64.reshape(v.shape[:-1] + (nb, BLOCK))).max(axis=-1)
    e = shared_exponent(amax, f.emax)                          # [..., nb]
    return encode_with_exponent(v64, e, f), (e + 127).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt) -> np.ndarray:
    """fp64 values of unpacked MX codes: element value times 2^(scale-127)."""
    f = _fmt(fmt)
    codes = np.asarray(codes)
    vals = f.table[codes]
    K = codes.shape[-1]
    s = E8M0[np.asarray(scales)]
    return (vals.reshape(codes.shape[:-1] + (K // BLOCK, BLOCK)) * s[..., None]).reshape(codes.shape)


# --------------------------------------------------------------------------- storage layout


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte along the last axis, even element in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------- MX matmul


def mx_matmul(a_codes, a_scales, a_fmt, b_codes, b_scales, b_fmt) -> np.ndarray:
    """C = deq(A) @ deq(B)^T in fp64, A ``[M][K]``, B ``[N][K]`` (both blocked along K).

    Every product of an E4M3 and an E2M1 value has at most 6 significant bits
    and the scales are powers of two, so for the operand ranges met here fp64
    accumulates these sums exactly (see ``mx_matmul_exact`` and its test).
    """
    A = dequantize(a_codes, a_scales, a_fmt)
    B = dequantize(b_codes, b_scales, b_fmt)
    return A @ B.T


def mx_matmul_exact(a_codes, a_scales, a_fmt, b_codes, b_scales, b_fmt) -> np.ndarray:
    """The same product evaluated in exact integer arithmetic, block by block.

    Each element is an integer multiple of its format's smallest step (2^-9 for
    E4M3, 2^-1 for E2M1), so a block's dot product is an exact integer sum
    times 2^(sa + sb - 254) times the two steps.  The per-block terms are
    summed with Python integers (arbitrary precision) after aligning exponents.
    Slow; meant for tiny shapes.
    """
    fa, fb = _fmt(a_fmt), _fmt(b_fmt)
    sta = {"e4m3": 9, "e2m1": 1}[fa.name]
    stb = {"e4m3": 9, "e2m1": 1}[fb.name]
    ia = np.rint(fa.table[a_codes] * (1 << sta)).astype(np.int64)
    ib = np.rint(fb.table[b_codes] * (1 << stb)).astype(np.int64)
    M, K = ia.shape
    N = ib.shape[0]
    nb = K // BLOCK
    out = np.empty((M, N), dtype=np.float64)
    from fractions import Fraction
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for b in range(nb):
                s = int(np.dot(ia[i, b * BLOCK:(b + 1) * BLOCK], ib[j, b * BLOCK:(b + 1) * BLOCK]))
                if s:
                    ex = int(a_scales[i, b]) + int(b_scales[j, b]) - 254 - sta - stb
                    acc += Fraction(s) * (Fraction(2) ** ex)
            out[i, j] = float(acc)
    return out


def mx_bits_per_element(fmt) -> float:
    """Storage cost per element including the shared scale: (32 * element bits + 8) / 32."""
    ebits = {"e2m1": 4, "e4m3": 8}[_fmt(fmt).name]
    return (BLOCK * ebits + 8) / BLOCK


# --------------------------------------------------------------------------- bfloat16
#
# The higher-precision weights of the Moat page's precision map ("Precision
# and deployment", Fig. 6) are taken as bfloat16: the upper half of an IEEE
# fp32 word (1 sign, 8 exponent, 7 mantissa bits).


def bf16_bits(v) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest, ties to even.

    The fp32 word splits into the 16 bits kept (``lo``, a sign-magnitude
    pattern whose magnitude bits count up with |v|) and the 16 dropped
    (``rem``).  The nearest bfloat16 is ``lo`` when ``rem`` is below half of
    the kept unit, ``lo`` plus one unit of magnitude above half, and the even
    one of the two at exactly half; one unit past the largest finite value is
    infinity, as IEEE rounding gives.  NaN inputs stay NaN (quiet bit set).
    """
    f = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    u = f.view(np.uint32).astype(np.int64)
    lo = u >> 16
    rem = u & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((lo & 1) == 1))
    out = np.where(up, lo + 1, lo)
    nan = np.isnan(f)
    out = np.where(nan, lo | 0x0040, out)
    return out.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bfloat16 bit patterns -> their values (fp64, exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)
