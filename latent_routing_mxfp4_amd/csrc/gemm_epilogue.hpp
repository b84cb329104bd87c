// gemm_epilogue.hpp -- the output stage shared by the MX GEMM kernels:
// fp32 store, MXFP8 quantisation along N, and the SwiGLU expert hidden state.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "mx_device.hpp"

namespace moe {

// Output tile of one wave: group, first row, rows of the group, first sorted
// row of the group (routed), first output column.
struct Tile {
  int g, m0, rows, row_base, n0;
};

// exp(-a) for a >= 0: 2^(-a log2 e) with the exponent split into hi + lo
// (the product's rounding error recovered with an fma, plus log2 e's own
// low part), the hardware 2^x applied to hi and a first-order correction
// e * (1 + lo ln 2) for |lo| < 2^-17.  About 3 units of fp32 rounding.
__device__ __forceinline__ float exp_neg(float a) {
  constexpr float kLog2e = 1.44269502162933349609375f;        // log2(e) rounded to fp32
  constexpr float kLog2eLo = 1.925963033500011079e-8f;        // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147180559945309f;
  const float hi = -a * kLog2e;
  const float lo = fmaf(-a, kLog2eLo, fmaf(-a, kLog2e, -hi));
  const float e = __builtin_amdgcn_exp2f(hi);
  return fmaf(e, lo * kLn2, e);
}

// SiLU(x) = x * sigmoid(x), with sigmoid formed from t = exp(-|x|) in (0, 1]:
// 1 / (1 + t) for x >= 0 and t / (1 + t) for x < 0, so nothing overflows for
// any x.  The reciprocal is the hardware estimate refined by one Newton step;
// the result is within about 9 units of fp32 rounding of x * sigmoid(x).
__device__ __forceinline__ float silu(float x) {
  const float t = exp_neg(fabsf(x));
  const float d = 1.0f + t;
  float r = __builtin_amdgcn_rcpf(d);
  r = fmaf(fmaf(-d, r, 1.0f), r, r);
  return x * (x >= 0.0f ? r : t * r);
}

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

// Maximum over each row of 16 lanes with DPP lane swaps (no LDS round trip):
// swap within pairs, then pairs within quads, then quads within half-rows
// (half-row mirror), then half-rows (row mirror).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

// MXFP8 block (32 columns: this lane's v0 at column c, v1 at c + 16, over the
// 16 lanes of its row) -> two codes and the block's scale code.
__device__ __forceinline__ uint32_t quant_pair(float v0, float v1, int& sc) {
  uint32_t m = max(__float_as_uint(v0) & 0x7fffffffu, __float_as_uint(v1) & 0x7fffffffu);
  m = row16_max_u32(m);  // non-negative floats order like their bit patterns
  sc = mx_scale_code<8>(m);
  return e4m3x2(v0, v1, sc - 127);
}

// Write one wave's MW x NW accumulator tiles (16x16 each; NB accumulators per
// tile for SwiGLU) in the epilogue's form.  Lane (r16, g4) holds column
// n0 + 16*ni + r16 of rows m0 + 16*mi + 4*g4 + i.  The 16 lanes of a row
// share its row index, so the block reductions only combine lanes of one row.
template <int MW, int NW, int NB, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const Tile& t, const v4f (&acc)[MW][NW][NB], int r16,
                                         int g4) {
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT;
  constexpr bool QNT = EPI != EPI_F32;
  const bool dense = p.offsets == nullptr;
  // Kernel arguments read once (stores through these pointers cannot alias them).
  const int N = p.N;
  const int64_t ldc = p.ldc;
  float* const cbase = p.c ? p.c + (dense ? (int64_t)t.g * p.c_gstride : 0) + t.n0 + r16 : nullptr;
  uint8_t* const qbase = QNT ? p.q + (dense ? (int64_t)t.g * p.q_gstride : 0) + t.n0 + r16 : nullptr;
  uint8_t* const sbase = QNT ? p.qs + (dense ? (int64_t)t.g * p.qs_gstride : 0) + (t.n0 >> 5) : nullptr;
  const int64_t row0 = dense ? 0 : (int64_t)t.row_base;
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    // Values, block maxima and codes of the fragment's four rows first, with
    // no branches, so the independent DPP reductions interleave; then stores.
    constexpr int NQ = QNT ? NW / 2 : 1;
    float hv[4][NQ][2];
    uint32_t q2[4][NQ];
    int sc[4][NQ];
    if (QNT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < NQ; ++b) {
          if (SWI) {
            hv[i][b][0] = silu(acc[mi][2 * b][0][i]) * acc[mi][2 * b][NB - 1][i];
            hv[i][b][1] = silu(acc[mi][2 * b + 1][0][i]) * acc[mi][2 * b + 1][NB - 1][i];
          } else {
            hv[i][b][0] = acc[mi][2 * b][0][i];
            hv[i][b][1] = acc[mi][2 * b + 1][0][i];
          }
          q2[i][b] = quant_pair(hv[i][b][0], hv[i][b][1], sc[i][b]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t.m0 + 16 * mi + 4 * g4 + i;
      if (row >= t.rows) continue;  // uniform over the 16 lanes of the row
      const int64_t orow = row0 + row;
      if (!SWI && cbase != nullptr) {
        float* crow = cbase + orow * ldc;
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
          if (t.n0 + 16 * ni < N) crow[16 * ni] = acc[mi][ni][0][i];
      }
      if (QNT) {
        uint8_t* qrow = qbase + orow * N;
        uint8_t* srow = sbase + orow * (N >> 5);
#pragma unroll
        for (int b = 0; b < NQ; ++b) {
          if (t.n0 + 32 * b < N) {
            qrow[32 * b] = (uint8_t)(q2[i][b] & 0xFF);
            qrow[32 * b + 16] = (uint8_t)(q2[i][b] >> 8);
            if (r16 == 0) srow[b] = (uint8_t)sc[i][b];
            if (SWI && cbase != nullptr) {  // optional fp32 copy of h (tracing)
              float* crow = cbase + orow * ldc;
              crow[32 * b] = hv[i][b][0];
              crow[32 * b + 16] = hv[i][b][1];
            }
          }
        }
      }
    }
  }
}

}  // namespace moe
