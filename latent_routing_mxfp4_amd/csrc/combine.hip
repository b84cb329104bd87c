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
// loads back to back (combine_device.hpp); the k rows are summed in slot order in fp32
// (deterministic, no atomics).  The MXFP8 block maximum of 32 features is a
// reduction over 8 neighbouring lanes by DPP lane swaps, and the codes come
// from the hardware fp32 -> E4M3 conversion of the clamped, power-of-two
// scaled values (identical to the integer encoder).  HBM-bound: k*L*4 bytes
// read per token.
#include "combine_device.hpp"
#include "kernels.hpp"

namespace moe {

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
  for (int f = threadIdx.x; f < n4; f += blockDim.x) combine_slot(y_e, rows, gs, k, L, t, f, y_lat, yq, yqs, yb);
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
