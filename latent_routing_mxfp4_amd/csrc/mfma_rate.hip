// mfma_rate.hip -- measurement probes, not part of the layer: the
// block-scaled FP8 x FP4 matrix-core rate of this GPU (the peak against which
// the expert GEMMs' MFMA share is read), and the rate at which a plain stream
// of 16-byte non-temporal loads reads HBM (the reference for the decode
// GEMMs, which only stream weights).
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

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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

// Each workgroup reads contiguous 32 KB chunks (a wave 8 x 1 KB, every load
// in flight), grid-stride over the buffer, and every thread folds its words
// into one so the loads are kept.
__global__ void __launch_bounds__(256) hbm_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                       uint32_t* __restrict__ out) {
  constexpr int U = 8;
  const int64_t chunk = (int64_t)blockDim.x * U;  // 16-byte words per workgroup and round
  uint32_t x = 0;
  int64_t c0 = (int64_t)blockIdx.x * chunk;
  for (; c0 + chunk <= n16; c0 += (int64_t)gridDim.x * chunk) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4_t w =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + c0 + u * blockDim.x + threadIdx.x));
      v[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = c0 + threadIdx.x; i < n16 && c0 < n16; i += blockDim.x) {  // the last, partial chunk
    const uint4 v = p[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace

hipError_t launch_hbm_read(const void* buf, int64_t bytes, int workgroups, uint32_t* out, hipStream_t s) {
  hbm_read_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, s>>>(static_cast<const uint4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(int iters, int workgroups, float* out, hipStream_t s) {
  mfma_rate_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, s>>>(iters, out);
  return hipGetLastError();
}

}  // namespace moe
