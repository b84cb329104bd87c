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

// SiLU(x) = x * sigmoid(x), with sigmoid formed from t = exp(-|x|) in (0, 1]:
// 1 / (1 + t) for x >= 0 and t / (1 + t) for x < 0, so nothing overflows for
// any x.  The reciprocal is the hardware estimate refined by one Newton step;
// the result is within about 7 units of fp32 rounding of x * sigmoid(x).
__device__ __forceinline__ float silu(float x) {
  const float t = expf(-fabsf(x));
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
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// Write one wave's MW x NW accumulator tiles (16x16 each; NB accumulators per
// tile for SwiGLU) in the epilogue's form.  Lane (r16, g4) holds column
// n0 + 16*ni + r16 of rows m0 + 16*mi + 4*g4 + i.
template <int MW, int NW, int NB, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const Tile& t, const v4f (&acc)[MW][NW][NB], int r16,
                                         int g4) {
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT;
  const bool dense = p.offsets == nullptr;
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t.m0 + 16 * mi + 4 * g4 + i;
      const bool rok = row < t.rows;
      const int64_t orow = dense ? row : (int64_t)t.row_base + row;
      if (EPI == EPI_F32 || EPI == EPI_F32_QUANT) {
        float* crow = p.c + (dense ? (int64_t)t.g * p.c_gstride : 0) + orow * p.ldc;
#pragma unroll
        for (int ni = 0; ni < NW; ++ni) {
          const int col = t.n0 + 16 * ni + r16;
          if (rok && col < p.N) crow[col] = acc[mi][ni][0][i];
        }
      }
      if (EPI == EPI_F32_QUANT || EPI == EPI_SWIGLU_QUANT) {
        uint8_t* qrow = p.q + (dense ? (int64_t)t.g * p.q_gstride : 0) + orow * p.N;
        uint8_t* qsrow = p.qs + (dense ? (int64_t)t.g * p.qs_gstride : 0) + orow * (p.N >> 5);
#pragma unroll
        for (int b = 0; b < NW / 2; ++b) {
          float v0, v1;
          if (SWI) {
            v0 = silu(acc[mi][2 * b][0][i]) * acc[mi][2 * b][NB - 1][i];
            v1 = silu(acc[mi][2 * b + 1][0][i]) * acc[mi][2 * b + 1][NB - 1][i];
            if (p.c != nullptr && rok && t.n0 + 32 * b < p.N) {  // optional fp32 copy of h (tracing)
              float* crow = p.c + (dense ? (int64_t)t.g * p.c_gstride : 0) + orow * p.ldc;
              crow[t.n0 + 32 * b + r16] = v0;
              crow[t.n0 + 32 * b + 16 + r16] = v1;
            }
          } else {
            v0 = acc[mi][2 * b][0][i];
            v1 = acc[mi][2 * b + 1][0][i];
          }
          uint32_t m = max(__float_as_uint(v0) & 0x7fffffffu, __float_as_uint(v1) & 0x7fffffffu);
          m = row16_max_u32(m);
          const int sc = mx_scale_code<8>(m);
          const int e = sc - 127;
          const int cb = t.n0 + 32 * b;
          const uint32_t q2 = e4m3x2(v0, v1, e);
          if (rok && cb < p.N) {
            qrow[cb + r16] = (uint8_t)(q2 & 0xFF);
            qrow[cb + 16 + r16] = (uint8_t)(q2 >> 8);
            if (r16 == 0) qsrow[cb >> 5] = (uint8_t)sc;
          }
        }
      }
    }
  }
}

}  // namespace moe
