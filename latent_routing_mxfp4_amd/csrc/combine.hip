// combine.hip -- gate-weighted combine of the expert outputs, fused with the
// MXFP8 quantisation of the combined latent (or its bfloat16 rounding, under
// the higher-precision map).
//
// Four Bits at a Time, "What it takes to serve it" (MoE data-path toy): the
// expert outputs are unpermuted and summed per token with the gates; Kimi K3
// and the New Open-Weights Moat, "Sparse computation": the combined latent is
// then projected back to model width, so it is quantised here to MXFP8, the
// input format of that projection.
//
// One workgroup per token with one thread per 4 consecutive latent features
// (L/4 threads, 896 at K3 width), so a thread issues its k 16-byte expert-row
// loads back to back; the k rows are summed in slot order in fp32
// (deterministic, no atomics).  The MXFP8 block maximum of 32 features is a
// reduction over 8 neighbouring lanes by DPP lane swaps, and the codes come
// from the hardware fp32 -> E4M3 conversion of the clamped, power-of-two
// scaled values (identical to the integer encoder).  HBM-bound: k*L*4 bytes
// read per token.
#include "gemm_epilogue.hpp"
#include "kernels.hpp"
#include "mx_device.hpp"

namespace moe {

// Maximum over each group of 8 neighbouring lanes (pairs, quads, half-rows).
__device__ __forceinline__ uint32_t lane8_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  return v;
}

__global__ void __launch_bounds__(1024) combine_kernel(const float* __restrict__ y_e,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ row_of_pair, int k, int L,
                                                      float* __restrict__ y_lat, uint8_t* __restrict__ yq,
                                                      uint8_t* __restrict__ yqs, uint16_t* __restrict__ yb) {
  __shared__ int32_t rows[64];
  __shared__ float gs[64];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of_pair[(int64_t)t * k + threadIdx.x];
    gs[threadIdx.x] = gates[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int n4 = L >> 2;  // a multiple of 8: the 8 lanes of a block are active together
  for (int f = threadIdx.x; f < n4; f += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += 8) {  // 8 row loads in flight, then the sums in slot order
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) v[u] = reinterpret_cast<const float4*>(y_e + (int64_t)rows[j0 + u] * L)[f];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) {
          const float g = gs[j0 + u];
          acc.x = fmaf(g, v[u].x, acc.x);
          acc.y = fmaf(g, v[u].y, acc.y);
          acc.z = fmaf(g, v[u].z, acc.z);
          acc.w = fmaf(g, v[u].w, acc.w);
        }
    }
    if (y_lat) reinterpret_cast<float4*>(y_lat + (int64_t)t * L)[f] = acc;
    if (yb)  // bfloat16 input of a higher-precision up-projection
      reinterpret_cast<uint2*>(yb + (int64_t)t * L)[f] =
          make_uint2(bf16_rne(acc.x) | (bf16_rne(acc.y) << 16), bf16_rne(acc.z) | (bf16_rne(acc.w) << 16));
    if (yq) {  // uniform over the launch
      uint32_t m = max(max(__float_as_uint(acc.x) & 0x7fffffffu, __float_as_uint(acc.y) & 0x7fffffffu),
                       max(__float_as_uint(acc.z) & 0x7fffffffu, __float_as_uint(acc.w) & 0x7fffffffu));
      m = lane8_max_u32(m);  // non-negative floats order like their bit patterns
      const int sc = mx_scale_code<8>(m);
      const int e = sc - 127;
      const uint32_t w = e4m3x2(acc.x, acc.y, e) | (e4m3x2(acc.z, acc.w, e) << 16);
      reinterpret_cast<uint32_t*>(yq + (int64_t)t * L)[f] = w;
      if ((f & 7) == 0) yqs[(int64_t)t * (L >> 5) + (f >> 3)] = (uint8_t)sc;
    }
  }
}

hipError_t launch_combine(const float* y_e, const float* gates, const int32_t* row_of_pair, int T, int k, int L,
                          float* y_lat, uint8_t* yq, uint8_t* yqs, hipStream_t s, uint16_t* yb) {
  if (T == 0) return hipSuccess;
  int threads = ((L / 4 + 63) / 64) * 64;
  threads = threads > 1024 ? 1024 : threads;
  combine_kernel<<<dim3(T), dim3(threads), 0, s>>>(y_e, gates, row_of_pair, k, L, y_lat, yq, yqs, yb);
  return hipGetLastError();
}

}  // namespace moe
