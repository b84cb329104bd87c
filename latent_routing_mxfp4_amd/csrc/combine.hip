// combine.hip -- gate-weighted combine of the expert outputs, fused with the
// MXFP8 quantisation of the combined latent.
//
// Four Bits at a Time, "What it takes to serve it" (MoE data-path toy): the
// expert outputs are unpermuted and summed per token with the gates; Kimi K3
// and the New Open-Weights Moat, "Sparse computation": the combined latent is
// then projected back to model width, so it is quantised here to MXFP8, the
// input format of that projection.
//
// One workgroup per token; each thread owns 4 consecutive latent features
// (one 16-byte load per expert row), sums the k rows in slot order in fp32
// (deterministic, no atomics), and 8 neighbouring lanes agree on the block
// maximum of their 32 features.  HBM-bound: k*L*4 bytes read per token.
#include "kernels.hpp"
#include "mx_device.hpp"

namespace moe {

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y_e,
                                                     const float* __restrict__ gates,
                                                     const int32_t* __restrict__ row_of_pair, int k, int L,
                                                     float* __restrict__ y_lat, uint8_t* __restrict__ yq,
                                                     uint8_t* __restrict__ yqs) {
  __shared__ int32_t rows[64];
  __shared__ float gs[64];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of_pair[(int64_t)t * k + threadIdx.x];
    gs[threadIdx.x] = gates[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int n4 = L >> 2;  // multiple of 8
  for (int f = threadIdx.x; f < n4; f += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 v = reinterpret_cast<const float4*>(y_e + (int64_t)rows[j] * L)[f];
      const float g = gs[j];
      acc.x = fmaf(g, v.x, acc.x);
      acc.y = fmaf(g, v.y, acc.y);
      acc.z = fmaf(g, v.z, acc.z);
      acc.w = fmaf(g, v.w, acc.w);
    }
    if (y_lat) reinterpret_cast<float4*>(y_lat + (int64_t)t * L)[f] = acc;
    uint32_t m = max(max(__float_as_uint(acc.x) & 0x7fffffffu, __float_as_uint(acc.y) & 0x7fffffffu),
                     max(__float_as_uint(acc.z) & 0x7fffffffu, __float_as_uint(acc.w) & 0x7fffffffu));
    m = group_max_u32<8>(m);
    const int sc = mx_scale_code<8>(m);
    const int e = sc - 127;
    const uint32_t w = enc_e4m3(acc.x, e) | (enc_e4m3(acc.y, e) << 8) | (enc_e4m3(acc.z, e) << 16) |
                       (enc_e4m3(acc.w, e) << 24);
    reinterpret_cast<uint32_t*>(yq + (int64_t)t * L)[f] = w;
    if ((f & 7) == 0) yqs[(int64_t)t * (L >> 5) + (f >> 3)] = (uint8_t)sc;
  }
}

hipError_t launch_combine(const float* y_e, const float* gates, const int32_t* row_of_pair, int T, int k, int L,
                          float* y_lat, uint8_t* yq, uint8_t* yqs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  combine_kernel<<<dim3(T), dim3(256), 0, s>>>(y_e, gates, row_of_pair, k, L, y_lat, yq, yqs);
  return hipGetLastError();
}

}  // namespace moe
