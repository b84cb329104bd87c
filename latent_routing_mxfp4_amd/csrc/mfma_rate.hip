// mfma_rate.hip -- the block-scaled FP8 x FP4 matrix-core rate of this GPU,
// measured: the peak against which the expert GEMMs' MFMA share is read.
//
// Every wave issues back-to-back v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 A,
// E2M1 B, E8M0 scales of 1.0) into eight independent accumulators, so the
// matrix core never waits on a result; 2 x 16 x 16 x 128 flops per MFMA.
// Operands are 1.0 (no NaN codes), the accumulators grow by 128 per MFMA and
// are summed into one float per wave at the end so the work is kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "mx_device.hpp"

namespace moe {

namespace {

__global__ void __launch_bounds__(256) mfma_rate_kernel(int iters, float* __restrict__ out) {
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838;                 // four E4M3 codes of 1.0
    b[i] = i < 4 ? 0x22222222 : 0;     // eight E2M1 codes of 1.0 (B uses four registers)
  }
  v4f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma_f8f4(a, b, acc[j], 127, 127);
    // keeps the accumulators in place across iterations (without it the
    // compiler rotates one of them through copies inside the loop)
    __builtin_amdgcn_sched_barrier(0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

hipError_t launch_mfma_rate(int iters, int workgroups, float* out, hipStream_t s) {
  mfma_rate_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, s>>>(iters, out);
  return hipGetLastError();
}

}  // namespace moe
