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

// SiLU(g) * u = g * u / (1 + e^-g), with e^-g = 2^(-g log2 e) from the
// hardware exp2 and 1 / (1 + t) from the hardware reciprocal.  For g < -88.7
// t is +inf and the result a signed zero (the exact value is below 1e-36).
// Relative error, in units of 2^-24: the rounded exponent -g log2 e carries
// 2|g| units into t, exp2 two more; t / (1 + t) of that reaches the quotient,
// plus 1 + t (one), the reciprocal (two) and the two products (one each) --
// at most 7 units for g >= 0 and 2|g| + 7 for g < 0.
__device__ __forceinline__ float swiglu(float g, float u) {
  constexpr float kLog2e = 1.44269502162933349609375f;  // log2(e) rounded to fp32
  const float t = __builtin_amdgcn_exp2f(-g * kLog2e);
  return g * __builtin_amdgcn_rcpf(1.0f + t) * u;
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
  uint32_t m = __float_as_uint(fmaxf(fabsf(v0), fabsf(v1)));
  m = row16_max_u32(m);  // non-negative floats order like their bit patterns
  sc = mx_scale_code<8>(m);
  return e4m3x2(v0, v1, sc - 127);
}

// Byte offset from a wave-uniform base: the address is the base (scalar
// registers) plus a zero-extended 32-bit lane offset, so no 64-bit vector
// arithmetic is spent per store.  A wave's rows of any output span less than
// 4 GB (the launchers bound N and ldc).
template <class T>
__device__ __forceinline__ T* at_byte(T* base, uint32_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(base) + off);
}

// Write one wave's MW x NW accumulator tiles (16x16 each; NB accumulators per
// tile for SwiGLU) in the epilogue's form (fp32, MXFP8 codes, or the bf16
// hidden state of a higher-precision SwiGLU expert).  Lane (r16, g4) holds column
// n0 + 16*ni + r16 of rows m0 + 16*mi + 4*g4 + i.  The 16 lanes of a row
// share its row index, so the block reductions only combine lanes of one row.
template <int MW, int NW, int NB, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const Tile& t, const v4f (&acc)[MW][NW][NB], int r16,
                                         int g4) {
  constexpr bool BFO = EPI == EPI_SWIGLU_BF16;   // bf16 hidden state, no MX codes
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT || BFO;
  constexpr bool QNT = EPI == EPI_F32_QUANT || EPI == EPI_SWIGLU_QUANT;
  constexpr bool PAIRS = QNT || BFO;              // values taken 32 columns (two fragments) at a time
  const bool dense = p.offsets == nullptr;
  // Kernel arguments read once (stores through these pointers cannot alias
  // them); bases at the wave's first output row and column.
  const int N = p.N;
  const uint32_t ldc = (uint32_t)p.ldc;
  const int64_t orow0 = (dense ? 0 : (int64_t)t.row_base) + t.m0;
  float* const cb = p.c ? p.c + (dense ? (int64_t)t.g * p.c_gstride : 0) + orow0 * (int64_t)ldc + t.n0 : nullptr;
  uint8_t* const qb = QNT ? p.q + (dense ? (int64_t)t.g * p.q_gstride : 0) + orow0 * N + t.n0 : nullptr;
  uint8_t* const sb = QNT ? p.qs + (dense ? (int64_t)t.g * p.qs_gstride : 0) + orow0 * (N >> 5) + (t.n0 >> 5)
                          : nullptr;
  uint16_t* const ob = BFO ? p.ob + (dense ? (int64_t)t.g * p.ob_gstride : 0) + orow0 * N + t.n0 : nullptr;
  const uint32_t c_lane = 4u * ((uint32_t)(4 * g4) * ldc + (uint32_t)r16);
  const uint32_t q_lane = (uint32_t)(4 * g4) * (uint32_t)N + (uint32_t)r16;
  const uint32_t s_lane = (uint32_t)(4 * g4) * (uint32_t)(N >> 5);
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    // Values, block maxima and codes of the fragment's four rows first, with
    // no branches, so the independent DPP reductions interleave; then stores.
    constexpr int NQ = PAIRS ? NW / 2 : 1;
    float hv[4][NQ][2];
    uint32_t q2[4][NQ];
    int sc[4][NQ];
    if (PAIRS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < NQ; ++b) {
          if (SWI) {
            hv[i][b][0] = swiglu(acc[mi][2 * b][0][i], acc[mi][2 * b][NB - 1][i]);
            hv[i][b][1] = swiglu(acc[mi][2 * b + 1][0][i], acc[mi][2 * b + 1][NB - 1][i]);
          } else {
            hv[i][b][0] = acc[mi][2 * b][0][i];
            hv[i][b][1] = acc[mi][2 * b + 1][0][i];
          }
          if (QNT) q2[i][b] = quant_pair(hv[i][b][0], hv[i][b][1], sc[i][b]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t.m0 + 16 * mi + 4 * g4 + i;
      if (row >= t.rows) continue;  // uniform over the 16 lanes of the row
      const uint32_t rr = (uint32_t)(16 * mi + i);  // row within the wave's rows, less 4*g4
      if (!SWI && cb != nullptr) {
        const uint32_t o = c_lane + 4u * rr * ldc;
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
          if (t.n0 + 16 * ni < N) {
            float* dst = at_byte(cb, o + 64u * ni);
            *dst = p.c_accumulate ? *dst + acc[mi][ni][0][i] : acc[mi][ni][0][i];
          }
      }
      if (QNT) {
        const uint32_t oq = q_lane + rr * (uint32_t)N;
        const uint32_t os = s_lane + rr * (uint32_t)(N >> 5);
#pragma unroll
        for (int b = 0; b < NQ; ++b) {
          if (t.n0 + 32 * b < N) {
            qb[oq + 32u * b] = (uint8_t)(q2[i][b] & 0xFF);
            qb[oq + 32u * b + 16u] = (uint8_t)(q2[i][b] >> 8);
            if (r16 == 0) sb[os + b] = (uint8_t)sc[i][b];
            if (SWI && cb != nullptr) {  // optional fp32 copy of h (tracing)
              const uint32_t o = c_lane + 4u * rr * ldc + 128u * b;
              *at_byte(cb, o) = hv[i][b][0];
              *at_byte(cb, o + 64u) = hv[i][b][1];
            }
          }
        }
      }
      if (BFO) {
        const uint32_t oq = q_lane + rr * (uint32_t)N;   // element offset, as for the codes
#pragma unroll
        for (int b = 0; b < NQ; ++b) {
          if (t.n0 + 32 * b < N) {
            ob[oq + 32u * b] = (uint16_t)bf16_rne(hv[i][b][0]);
            ob[oq + 32u * b + 16u] = (uint16_t)bf16_rne(hv[i][b][1]);
            if (cb != nullptr) {  // optional fp32 copy of h (tracing)
              const uint32_t o = c_lane + 4u * rr * ldc + 128u * b;
              *at_byte(cb, o) = hv[i][b][0];
              *at_byte(cb, o + 64u) = hv[i][b][1];
            }
          }
        }
      }
    }
  }
}

}  // namespace moe
