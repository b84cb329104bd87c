// combine_device.hpp -- the per-element work of the gate-weighted combine
// (combine.hip), shared by the combine kernel and the prefill launch that
// runs the combine beside the shared experts' gate/up GEMM (mx_gemm_wide.hip).
#pragma once

#include "gemm_epilogue.hpp"
#include "mx_device.hpp"

namespace moe {

// y_lat (if given), bf16 (yb, if given) and MXFP8 codes (yq, if given) of
// features 4f .. 4f+3 of token t from their fp32 sum `acc`.  With yq, the 8
// lanes holding f = 8b .. 8b+7 must be active together: they form MX block b.
__device__ __forceinline__ void combine_store(const float4& acc, int L, int64_t t, int f, float* __restrict__ y_lat,
                                              uint8_t* __restrict__ yq, uint8_t* __restrict__ yqs,
                                              uint16_t* __restrict__ yb) {
  if (y_lat) reinterpret_cast<float4*>(y_lat + t * L)[f] = acc;
  if (yb)  // bfloat16 input of a higher-precision up-projection
    reinterpret_cast<uint2*>(yb + t * L)[f] =
        make_uint2(bf16_rne(acc.x) | (bf16_rne(acc.y) << 16), bf16_rne(acc.z) | (bf16_rne(acc.w) << 16));
  if (yq) {
    uint32_t m = max(max(__float_as_uint(acc.x) & 0x7fffffffu, __float_as_uint(acc.y) & 0x7fffffffu),
                     max(__float_as_uint(acc.z) & 0x7fffffffu, __float_as_uint(acc.w) & 0x7fffffffu));
    m = lane8_max_u32(m);  // non-negative floats order like their bit patterns
    const int sc = mx_scale_code<8>(m);
    const int e = sc - 127;
    const uint32_t w = e4m3x2(acc.x, acc.y, e) | (e4m3x2(acc.z, acc.w, e) << 16);
    reinterpret_cast<uint32_t*>(yq + t * L)[f] = w;
    if ((f & 7) == 0) yqs[t * (L >> 5) + (f >> 3)] = (uint8_t)sc;
  }
}

// acc += gs[j] * y_e[rows[j]][4f .. 4f+3] over slots j = j0 .. j0+15 (< k), in
// slot order (fp32 fma), the row loads issued first so they are in flight
// together.  Slots past k re-read slot k-1's row and are not added (selects,
// not branches, so the loads of several calls can be in flight at once).
__device__ __forceinline__ void combine_rows16(const float* __restrict__ y_e, const int32_t* rows, const float* gs,
                                               int k, int L, int j0, int f, float4& acc) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  float4 v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {  // read once: non-temporal, so they do not evict other kernels' operands from L2
    const int j = min(j0 + u, k - 1);
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y_e + (int64_t)rows[j] * L) + f);
    v[u] = make_float4(w[0], w[1], w[2], w[3]);
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const bool in = j0 + u < k;
    const float g = gs[min(j0 + u, k - 1)];
    acc.x = in ? fmaf(g, v[u].x, acc.x) : acc.x;
    acc.y = in ? fmaf(g, v[u].y, acc.y) : acc.y;
    acc.z = in ? fmaf(g, v[u].z, acc.z) : acc.z;
    acc.w = in ? fmaf(g, v[u].w, acc.w) : acc.w;
  }
}

// Features 4f .. 4f+3 of token t: acc = sum over slots j = 0 .. k-1, in slot
// order, of gs[j] * y_e[rows[j]] (fp32 fma), then combine_store.
__device__ __forceinline__ void combine_slot(const float* __restrict__ y_e, const int32_t* rows, const float* gs,
                                             int k, int L, int64_t t, int f, float* __restrict__ y_lat,
                                             uint8_t* __restrict__ yq, uint8_t* __restrict__ yqs,
                                             uint16_t* __restrict__ yb) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 16) combine_rows16(y_e, rows, gs, k, L, j0, f, acc);
  combine_store(acc, L, t, f, y_lat, yq, yqs, yb);
}

}  // namespace moe
