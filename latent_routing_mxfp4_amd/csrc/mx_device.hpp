// mx_device.hpp -- device helpers shared by the gfx950 kernels: MX encoding in
// integer arithmetic, wave reductions, and the block-scaled MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// MX encoding.  Four Bits at a Time, "Four bits from the start": the shared
// exponent of a block is floor(log2(amax)) minus the element format's largest
// exponent; elements are the value divided by 2^e, clipped to the largest grid
// magnitude and rounded to the nearest grid point.  Everything below is exact
// integer work on the fp32 bit pattern, so the result does not depend on the
// rounding mode of any float operation.

// E8M0 code of a block with maximum magnitude amax (fp32 bits, sign cleared):
// clamp(floor(log2 amax) - EMAX, -127, 127) + 127, with EMAX = 8 for E4M3
// and 2 for E2M1.  For a normal amax floor(log2 amax) is the exponent field
// minus 127, so the code is the field minus EMAX; the lower clamp (code 0)
// takes exactly the fields <= EMAX, which include every subnormal amax and
// amax == 0; the upper clamp is never reached (field <= 255).
template <int EMAX>
__device__ __forceinline__ int mx_scale_code(uint32_t amax_bits) {
  const int c = (int)(amax_bits >> 23) - EMAX;
  return c > 0 ? c : 0;
}

// fp32 -> bfloat16 bit pattern, round to nearest with ties to even: the upper
// 16 bits of the word, plus one unit of magnitude when the 16 dropped bits
// exceed half a unit, or equal it and the kept pattern is odd (adding 0x7FFF
// plus the kept low bit carries exactly then).  Past the largest finite value
// the carry reaches the infinity pattern, as IEEE rounding does.  Finite
// inputs (a NaN is not preserved).
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Element code of fp32 v under block exponent e = scale_code - 127.
// MB mantissa bits, EMIN smallest normal exponent, MAXC largest finite
// magnitude code, SBIT sign position.  Round to nearest, ties to even code.
template <int MB, int EMIN, int MAXC, int SBIT>
__device__ __forceinline__ uint32_t mx_encode(float v, int e) {
  uint32_t b = __float_as_uint(v);
  uint32_t sign = (b >> 31) << SBIT;
  uint32_t mag = b & 0x7fffffffu;
  if (mag == 0) return sign;
  uint32_t ex = mag >> 23;
  uint32_t M;   // integer significand: |v| = M * 2^E0
  int E0, fl;
  if (ex) {
    M = (mag & 0x7fffffu) | 0x800000u;
    E0 = (int)ex - 150;
    fl = (int)ex - 127;
  } else {
    M = mag;
    E0 = -149;
    fl = -149 + (31 - __clz(mag));
  }
  int fly = fl - e;                       // floor(log2(|v| / 2^e))
  int bin = fly > EMIN ? fly : EMIN;      // binade of the grid step
  int sh = bin - MB + e - E0;             // q = M / 2^sh, rounded
  uint32_t q;
  if (sh <= 0) {
    q = M << (-sh);                       // not reached for e >= -127; kept exact anyway
  } else if (sh >= 32) {
    q = 0;                                // below half a step
  } else {
    uint32_t qt = M >> sh;
    uint32_t rem = M & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    q = qt + ((rem > half) | ((rem == half) & (qt & 1u)));
  }
  uint32_t code = (uint32_t)(bin - EMIN) * (1u << MB) + q;
  code = code > (uint32_t)MAXC ? (uint32_t)MAXC : code;
  return sign | code;
}

__device__ __forceinline__ uint32_t enc_e4m3(float v, int e) { return mx_encode<3, -6, 0x7E, 7>(v, e); }
__device__ __forceinline__ uint32_t enc_e2m1(float v, int e) { return mx_encode<1, 0, 0x7, 3>(v, e); }

// Two E4M3 codes (bits 0-7 and 8-15) of v0, v1 under block exponent e: the
// hardware fp32 -> E4M3 conversion, which rounds to nearest with ties to even
// on the OCP grid, of v * 2^-e clamped to +-448.  Scaling by a power of two is
// exact and the clamp is the quantiser's clip to the largest magnitude, so the
// codes equal the integer encoder's (enc_e4m3) for every finite input.
__device__ __forceinline__ uint32_t e4m3x2(float v0, float v1, int e) {
  const float a = fminf(fmaxf(ldexpf(v0, -e), -448.0f), 448.0f);
  const float b = fminf(fmaxf(ldexpf(v1, -e), -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// Wave helpers.

// Maximum over each group of 8 neighbouring lanes (pairs, quads, half-rows).
__device__ __forceinline__ uint32_t lane8_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  return v;
}


// Max over aligned groups of W lanes (W a power of two <= 64), via xor shuffles.
template <int W>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o, kWave);
    v = v > w ? v : w;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Block-scaled MFMA, 16x16x128, A = E4M3, B = E2M1, fp32 accumulate.
//
// Operand layout (64 lanes, lane l, r = l % 16, g = l / 16), established by a
// one-tile probe against the exact product on gfx950:
//   A (E4M3, 8 dwords): row r; bytes 0-15 = K [16g, 16g+16),
//                       bytes 16-31 = K [64+16g, 64+16g+16)
//   B (E2M1, low 4 of 8 dwords): col r; 32 elements K [32g, 32g+32),
//                       element 2i in the low nibble of byte i
//   scale_a / scale_b: bits [7:0] = E8M0 of 32-element block g of row/col r
//                       (the scale lane need not hold that block's data)
//   D: col r, rows 4g .. 4g+3 -> 4 floats
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_f8f4(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, /*A fmt E4M3*/ 0, /*B fmt E2M1*/ 4,
                                                          0, sa, 0, sb);
}

}  // namespace moe
