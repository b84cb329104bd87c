// mx_quant.hip -- fp32 -> MX (E4M3 or E2M1) block quantisation.
//
// Four Bits at a Time, "Four bits from the start": blocks of 32 along a row
// share one E8M0 scale 2^(floor(log2 amax) - emax); each element is divided
// by the scale, clipped and rounded to the nearest grid point (ties to even).
//
// Layout: one thread per 4 consecutive floats (one 16-byte load), so 8
// neighbouring lanes hold one 32-element block and agree on its maximum with
// three lane swaps.  Reads and writes are fully coalesced; the kernel is
// HBM-bound (4 B read, 1.03 B (E4M3) or 0.53 B (E2M1) written per element).
// For E4M3 it can also write the exact dequantised values as bf16 (the
// operand of the bf16 latent down-projection).
//
// Weight matrices consumed by the MX GEMMs are stored in fragment order (see
// kernels.hpp): the E2M1 quantiser can write that order directly, and a copy
// kernel converts row-major E2M1 into it.
#include "kernels.hpp"
#include "mx_device.hpp"

namespace moe {

// Exact value of an E4M3 / E2M1 code under block exponent e, as fp32
// (exact whenever the result is a normal fp32 number).
__device__ __forceinline__ float dec_e4m3(uint32_t c, int e) {
  const int E = (c >> 3) & 15, m = c & 7;
  const float v = ldexpf((float)(E ? 8 + m : m), (E ? E - 10 : -9) + e);
  return (c & 0x80) ? -v : v;
}
__device__ __forceinline__ float dec_e2m1(uint32_t c, int e) {
  const int E = (c >> 1) & 3, m = c & 1;
  const float v = ldexpf((float)(E ? 2 + m : m), (E ? E - 2 : -1) + e);
  return (c & 0x8) ? -v : v;
}
// bf16 bit pattern of a float with at most 8 significant bits (exact).
__device__ __forceinline__ uint32_t bf16_bits(float v) { return __float_as_uint(v) >> 16; }

// Byte offsets of element k (a multiple of 4) of row n of matrix g in the
// fragment-order layout of G matrices [N][K] (N % 16 == 0, K % 128 == 0).
__device__ __forceinline__ int64_t frag_code_offset(int64_t g, int n, int k, int N, int K) {
  const int lane = (n & 15) + 16 * ((k & 127) >> 5);
  return g * ((int64_t)N * K / 2) + ((int64_t)(n >> 4) * (K >> 7) + (k >> 7)) * 1024 + 16 * lane + ((k & 31) >> 1);
}
__device__ __forceinline__ int64_t frag_scale_offset(int64_t g, int n, int k, int N, int K) {
  return g * ((int64_t)N * K / 32) + ((int64_t)(k >> 7) * N + n) * 4 + ((k >> 5) & 3);
}

// FMT 0: E4M3 row-major; 1: E2M1 row-major; 2: E2M1 in fragment order with
// N rows per matrix (rows = G * N).
template <int FMT>
__global__ void __launch_bounds__(256) quantize_kernel(const float4* __restrict__ in, int64_t n4,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       uint2* __restrict__ deq, int N, int K) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    // n4 is a multiple of 8 and i starts 8-aligned per group of 8 lanes, so
    // the 8 lanes of a block are active together.
    float4 v = in[i];
    uint32_t m = max(max(__float_as_uint(v.x) & 0x7fffffffu, __float_as_uint(v.y) & 0x7fffffffu),
                     max(__float_as_uint(v.z) & 0x7fffffffu, __float_as_uint(v.w) & 0x7fffffffu));
    // non-negative floats order like their bit patterns; the 8 lanes of a
    // block are neighbours (DPP swaps for E4M3, shuffles for the weights)
    m = FMT == 0 ? lane8_max_u32(m) : group_max_u32<8>(m);
    if (FMT == 0) {
      int sc = mx_scale_code<8>(m);
      int e = sc - 127;
      // the hardware conversion of the clamped, scaled values: the same codes
      // as the integer encoder (enc_e4m3) for every finite input (e4m3x2)
      uint32_t w = e4m3x2(v.x, v.y, e) | (e4m3x2(v.z, v.w, e) << 16);
      reinterpret_cast<uint32_t*>(codes)[i] = w;
      if ((i & 7) == 0) scales[i >> 3] = (uint8_t)sc;
      if (deq) {  // bf16 copy of the dequantised values (exact), for the bf16 matrix cores
        uint2 o;
        o.x = bf16_bits(dec_e4m3(w & 0xff, e)) | (bf16_bits(dec_e4m3((w >> 8) & 0xff, e)) << 16);
        o.y = bf16_bits(dec_e4m3((w >> 16) & 0xff, e)) | (bf16_bits(dec_e4m3(w >> 24, e)) << 16);
        deq[i] = o;
      }
    } else {
      int sc = mx_scale_code<2>(m);
      int e = sc - 127;
      uint32_t w = enc_e2m1(v.x, e) | (enc_e2m1(v.y, e) << 4) | (enc_e2m1(v.z, e) << 8) |
                   (enc_e2m1(v.w, e) << 12);
      if (FMT == 1) {
        reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)w;
        if ((i & 7) == 0) scales[i >> 3] = (uint8_t)sc;
      } else {
        const int64_t row = (4 * i) / K;
        const int k = (int)(4 * i - row * K);
        const int64_t g = row / N;
        const int n = (int)(row - g * N);
        *reinterpret_cast<uint16_t*>(codes + frag_code_offset(g, n, k, N, K)) = (uint16_t)w;
        if ((i & 7) == 0) scales[frag_scale_offset(g, n, k, N, K)] = (uint8_t)sc;
      }
    }
  }
}

// E2M1 (packed) + E8M0 -> bf16, one thread per 32-element block.
// One thread per MX block (row, j) of the output order: block b = row * K/32 + j.
// Fragment-order input (frag != 0, N rows): its 16 code bytes are lane chunk
// (row % 16) + 16 (j % 4) of block (row / 16, j / 4), its scale byte j % 4 of
// dword (j / 4) * N + row.
__global__ void __launch_bounds__(256) decode_e2m1_bf16_kernel(const uint4* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales, int64_t nblk,
                                                              uint4* __restrict__ out, int frag, int N, int K) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int kblk = K >> 5;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
    int64_t cb = b, sb = b;
    if (frag) {
      const int64_t row = b / kblk;
      const int j = (int)(b - row * kblk);
      cb = ((row >> 4) * (K >> 7) + (j >> 2)) * 64 + (row & 15) + 16 * (j & 3);
      sb = ((int64_t)(j >> 2) * N + row) * 4 + (j & 3);
    }
    const uint4 c = codes[cb];
    const int e = (int)scales[sb] - 127;
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // 8 elements per dword
      uint4 o;
      uint32_t* op = &o.x;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t lo = (w[q] >> (8 * h)) & 0xf, hi = (w[q] >> (8 * h + 4)) & 0xf;
        op[h] = bf16_bits(dec_e2m1(lo, e)) | (bf16_bits(dec_e2m1(hi, e)) << 16);
      }
      out[4 * b + q] = o;
    }
  }
}

// fp32 -> bfloat16 (round to nearest even), 4 values per thread.
__global__ void __launch_bounds__(256) round_bf16_kernel(const float4* __restrict__ in, int64_t n4,
                                                         uint2* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = in[i];
    out[i] = make_uint2(bf16_rne(v.x) | (bf16_rne(v.y) << 16), bf16_rne(v.z) | (bf16_rne(v.w) << 16));
  }
}

hipError_t launch_round_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t s) {
  if (n % 4 != 0 || ((uintptr_t)in & 15) || ((uintptr_t)out & 7)) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  round_bf16_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(reinterpret_cast<const float4*>(in), n4,
                                                                  reinterpret_cast<uint2*>(out));
  return hipGetLastError();
}

hipError_t launch_decode_e2m1_bf16(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K, uint16_t* out,
                                   hipStream_t s, int frag) {
  const int64_t nblk = rows * (int64_t)K / 32;
  if (nblk == 0) return hipSuccess;
  if (frag && (rows % 16 || K % 128 || rows > 0x7fffffff)) return hipErrorInvalidValue;
  int64_t blocks = (nblk + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  decode_e2m1_bf16_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(reinterpret_cast<const uint4*>(codes), scales,
                                                                        nblk, reinterpret_cast<uint4*>(out), frag,
                                                                        (int)rows, K);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* in, int64_t rows, int K, int fmt, uint8_t* codes, uint8_t* scales,
                           hipStream_t s, uint16_t* deq_bf16, int frag_rows) {
  int64_t n4 = rows * (int64_t)K / 4;
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  const float4* in4 = reinterpret_cast<const float4*>(in);
  if (fmt == 0)
    quantize_kernel<0><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(in4, n4, codes, scales,
                                                                     reinterpret_cast<uint2*>(deq_bf16), 0, K);
  else if (frag_rows == 0)
    quantize_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(in4, n4, codes, scales, nullptr, 0, K);
  else
    quantize_kernel<2><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(in4, n4, codes, scales, nullptr, frag_rows, K);
  return hipGetLastError();
}

// Row-major E2M1 -> fragment order: one thread per 16-byte lane chunk of the
// codes, and one per scale dword.
__global__ void __launch_bounds__(256) pack_e2m1_kernel(const uint4* __restrict__ codes,
                                                        const uint32_t* __restrict__ scales, int64_t G, int N,
                                                        int K, uint4* __restrict__ out_codes,
                                                        uint32_t* __restrict__ out_scales) {
  const int nks = K >> 7;
  const int64_t nchunk = G * (int64_t)N * K / 32;  // 16-byte chunks (32 elements each)
  const int64_t nsc = G * (int64_t)N * nks;        // scale dwords
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nchunk + nsc; t += stride) {
    if (t < nchunk) {
      // output chunk t = ((g * N/16 + nb) * nks + kb) * 64 + lane
      const int lane = (int)(t & 63);
      const int64_t blk = t >> 6;
      const int kb = (int)(blk % nks);
      const int64_t gnb = blk / nks;  // g * N/16 + nb
      const int64_t row = gnb * 16 + (lane & 15);
      out_codes[t] = codes[row * (K >> 5) + 4 * kb + (lane >> 4)];
    } else {
      // output dword u = (g * nks + kb) * N + n
      const int64_t u = t - nchunk;
      const int n = (int)(u % N);
      const int64_t gk = u / N;
      const int kb = (int)(gk % nks);
      const int64_t g = gk / nks;
      out_scales[u] = scales[(g * N + n) * nks + kb];
    }
  }
}

hipError_t launch_pack_e2m1(const uint8_t* codes, const uint8_t* scales, int64_t G, int N, int K, uint8_t* out_codes,
                            uint8_t* out_scales, hipStream_t s) {
  const int64_t total = G * (int64_t)N * K / 32 + G * (int64_t)N * (K >> 7);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  pack_e2m1_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
      reinterpret_cast<const uint4*>(codes), reinterpret_cast<const uint32_t*>(scales), G, N, K,
      reinterpret_cast<uint4*>(out_codes), reinterpret_cast<uint32_t*>(out_scales));
  return hipGetLastError();
}

}  // namespace moe
