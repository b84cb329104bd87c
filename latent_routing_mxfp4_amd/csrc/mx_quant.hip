// mx_quant.hip -- fp32 -> MX (E4M3 or E2M1) block quantisation.
//
// Four Bits at a Time, "Four bits from the start": blocks of 32 along a row
// share one E8M0 scale 2^(floor(log2 amax) - emax); each element is divided
// by the scale, clipped and rounded to the nearest grid point (ties to even).
//
// Layout: one thread per 4 consecutive floats (one 16-byte load), so 8
// neighbouring lanes hold one 32-element block and agree on its maximum with
// three xor shuffles.  Reads and writes are fully coalesced; the kernel is
// HBM-bound (4 B read, 1.03 B (E4M3) or 0.53 B (E2M1) written per element).
#include "kernels.hpp"
#include "mx_device.hpp"

namespace moe {

template <int FMT>
__global__ void __launch_bounds__(256) quantize_kernel(const float4* __restrict__ in, int64_t n4,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    // n4 is a multiple of 8 and i starts 8-aligned per group of 8 lanes, so
    // the 8 lanes of a block are active together.
    float4 v = in[i];
    uint32_t m = max(max(__float_as_uint(v.x) & 0x7fffffffu, __float_as_uint(v.y) & 0x7fffffffu),
                     max(__float_as_uint(v.z) & 0x7fffffffu, __float_as_uint(v.w) & 0x7fffffffu));
    m = group_max_u32<8>(m);  // non-negative floats order like their bit patterns
    if (FMT == 0) {
      int sc = mx_scale_code<8>(m);
      int e = sc - 127;
      uint32_t w = enc_e4m3(v.x, e) | (enc_e4m3(v.y, e) << 8) | (enc_e4m3(v.z, e) << 16) |
                   (enc_e4m3(v.w, e) << 24);
      reinterpret_cast<uint32_t*>(codes)[i] = w;
      if ((i & 7) == 0) scales[i >> 3] = (uint8_t)sc;
    } else {
      int sc = mx_scale_code<2>(m);
      int e = sc - 127;
      uint32_t w = enc_e2m1(v.x, e) | (enc_e2m1(v.y, e) << 4) | (enc_e2m1(v.z, e) << 8) |
                   (enc_e2m1(v.w, e) << 12);
      reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)w;
      if ((i & 7) == 0) scales[i >> 3] = (uint8_t)sc;
    }
  }
}

hipError_t launch_quantize(const float* in, int64_t rows, int K, int fmt, uint8_t* codes, uint8_t* scales,
                           hipStream_t s) {
  int64_t n4 = rows * (int64_t)K / 4;
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (fmt == 0)
    quantize_kernel<0><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(reinterpret_cast<const float4*>(in), n4,
                                                                     codes, scales);
  else
    quantize_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(reinterpret_cast<const float4*>(in), n4,
                                                                     codes, scales);
  return hipGetLastError();
}

}  // namespace moe
