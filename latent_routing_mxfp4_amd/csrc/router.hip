// router.hip -- sigmoid router on the latent and top-k selection.
//
// Kimi K3 and the New Open-Weights Moat, "How the router picks 16 of 896"
// (Fig. 2): every routed expert gets a sigmoid score; selection takes the top
// k of score + a per-expert selection bias; the winners' raw scores,
// normalised by their sum, are the mixture weights.  Four Bits at a Time,
// "The shape of the model": routing runs in the latent space.
//
// Two kernels:
//   router_logits: logits[T][E] = z[T][L] W[E][L]^T (+ logit bias), fp32 in
//     and out, on the fp32 matrix cores (v_mfma_f32_16x16x4f32) with 64x64
//     tiles staged through LDS; for few tiles (decode) the K range is split
//     over extra workgroups and the slices summed in a fixed order.
//   topk: one wave per token (sigmoid scores, or the logits themselves with
//     softmax gates).  Up to 1024 experts the keys sit in registers, a
//     threshold (the k-th largest of the lanes' maxima) cuts them to a few
//     candidates, and each candidate's slot is the number of better ones;
//     otherwise (and when too many keys tie) k rounds of a 64-lane
//     (key desc, id asc) reduction (DPP within rows, readlane across) pick
//     the winners in slot order.  k <= 64 (slot j is held by lane j).  For
//     few tokens the K-slice sums of the logits are added by the top-k
//     kernel itself (one workgroup per token).
#include <float.h>

#include "kernels.hpp"
#include "launch_attr.hpp"
#include "mx_device.hpp"

namespace moe {

namespace {
typedef float v4f_t __attribute__((ext_vector_type(4)));
constexpr int RT = 64;   // tokens per tile
constexpr int RE = 64;   // experts per tile
constexpr int RK = 32;   // K chunk
constexpr int RPAD = 4;  // LDS row padding (floats)
}  // namespace

// One 64 x 64 tile of z W^T over the K range [kbeg, kend).  With split > 1
// (few tiles: small T) the K range is cut into `split` slices, one per
// blockIdx.z, and each slice writes its partial sums to out + z*T*E; a second
// kernel adds the slices in a fixed order (deterministic), plus the bias.
__global__ void __launch_bounds__(256) router_logits_kernel(const float* __restrict__ z,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ bias, int T, int E,
                                                           int L, int kslice, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float zs[RT][RK + RPAD];
  __shared__ __attribute__((aligned(16))) float ws[RE][RK + RPAD];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int t0 = blockIdx.y * RT, e0 = blockIdx.x * RE;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;  // wave's 32x32 sub-tile
  const int kbeg = blockIdx.z * kslice;
  const int kend = min(L, kbeg + kslice);
  float* const dst = out + (int64_t)blockIdx.z * T * E;
  const float* const bvec = gridDim.z == 1 ? bias : nullptr;  // the reduction adds it otherwise

  v4f_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = v4f_t{0.f, 0.f, 0.f, 0.f};

  // The K range in rounds of RC chunks: a round's global loads are all
  // issued first (in flight together, one memory latency per round rather
  // than per chunk), then each chunk goes through LDS into the MFMAs.
  constexpr int RC = 4;
  for (int kr = kbeg; kr < kend; kr += RC * RK) {
    // per chunk: 64 rows x 32 floats = 512 float4 per operand; 2 per thread
    float4 vz[RC][2], vw[RC][2];
#pragma unroll
    for (int c = 0; c < RC; ++c)
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int f = tid + 256 * it;
        const int r = f >> 3, c4 = (f & 7) * 4;
        const int k0 = kr + c * RK;
        vz[c][it] = make_float4(0.f, 0.f, 0.f, 0.f);
        vw[c][it] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (k0 < kend && t0 + r < T) vz[c][it] = *reinterpret_cast<const float4*>(z + (int64_t)(t0 + r) * L + k0 + c4);
        if (k0 < kend && e0 + r < E) vw[c][it] = *reinterpret_cast<const float4*>(w + (int64_t)(e0 + r) * L + k0 + c4);
      }
#pragma unroll
    for (int c = 0; c < RC; ++c) {
      if (kr + c * RK >= kend) break;  // uniform
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int f = tid + 256 * it;
        const int r = f >> 3, c4 = (f & 7) * 4;
        *reinterpret_cast<float4*>(&zs[r][c4]) = vz[c][it];
        *reinterpret_cast<float4*>(&ws[r][c4]) = vw[c][it];
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < RK; kk += 4) {
        float a0 = zs[wm + r16][kk + g4], a1 = zs[wm + 16 + r16][kk + g4];
        float b0 = ws[wn + r16][kk + g4], b1 = ws[wn + 16 + r16][kk + g4];
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int e = e0 + wn + 16 * b + r16;
      if (e >= E) continue;
      const float bb = bvec ? bvec[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + wm + 16 * a + 4 * g4 + i;
        if (t < T) dst[(int64_t)t * E + e] = acc[a][b][i] + bb;
      }
    }
}

// ---------------------------------------------------------------------------
// Many tokens: the same fp32 product on the bf16 matrix cores.  Every fp32
// value is split exactly into three bf16 pieces by truncation (x0 = the top 8
// significant bits, x1 = the next 8 of x - x0, x2 = x - x0 - x1, each exact),
// and z w ~ z0 w0 + z0 w1 + z1 w0 + z0 w2 + z1 w1 + z2 w0: every term is an
// exact product accumulated in fp32; the three dropped terms are below
// 2^-23 |z w| together, the size of one fp32 rounding of the product.  Six
// v_mfma_f32_32x32x16_bf16 run at about 2.2 PFLOP/s against 157 TFLOP/s for
// the fp32 instruction.  The router weight is split once per forward
// (split3_kernel); the latent is split while it is staged into LDS.
//
// Tile 128 tokens x 128 experts, 4 waves of 64 x 64 (2 x 2 MFMA tiles of
// 32 x 32), K chunks of 32 staged as three bf16 planes per operand with an
// 80-byte row stride (eight consecutive rows hit distinct banks); the next
// chunk's global loads are issued before the current chunk's MFMAs.
// v_mfma_f32_32x32x16_bf16 operands (probed on gfx950): lane l holds row
// (A) / column (B) l % 32, K [8 (l / 32), +8); D register i of lane l is
// column l % 32, row 8 (i / 4) + 4 (l / 32) + i % 4.
namespace {
constexpr int BT = 128, BE = 128, BK = 32;
constexpr int BROW = 80;                // bytes per LDS row (32 bf16 + 16 padding)
constexpr int BPLANE = 128 * BROW;      // one plane of one operand
constexpr int BOP = 3 * BPLANE;         // three planes
typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
typedef float f16v_r __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t hi16_pair(uint32_t lo_elem, uint32_t hi_elem) {
  return (lo_elem >> 16) | (hi_elem & 0xFFFF0000u);
}
// Three bf16 pieces of four fp32 values, packed two per dword per plane.
__device__ __forceinline__ void split3x4(const float4& v, uint2 (&pl)[3]) {
  const float x[4] = {v.x, v.y, v.z, v.w};
  uint32_t p0[4], p1[4], p2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b0 = __float_as_uint(x[i]) & 0xFFFF0000u;
    const float r = x[i] - __uint_as_float(b0);
    const uint32_t b1 = __float_as_uint(r) & 0xFFFF0000u;
    const float r2 = r - __uint_as_float(b1);
    p0[i] = b0;
    p1[i] = b1;
    p2[i] = __float_as_uint(r2);
  }
  pl[0] = make_uint2(hi16_pair(p0[0], p0[1]), hi16_pair(p0[2], p0[3]));
  pl[1] = make_uint2(hi16_pair(p1[0], p1[1]), hi16_pair(p1[2], p1[3]));
  pl[2] = make_uint2(hi16_pair(p2[0], p2[1]), hi16_pair(p2[2], p2[3]));
}
}  // namespace

// planes[p][i] = piece p of w[i] (bf16 bits), i < n (n % 4 == 0).
__global__ void __launch_bounds__(256) split3_kernel(const float4* __restrict__ w, int64_t n4,
                                                     uint2* __restrict__ planes) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    uint2 pl[3];
    split3x4(w[i], pl);
    planes[i] = pl[0];
    planes[n4 + i] = pl[1];
    planes[2 * n4 + i] = pl[2];
  }
}

__global__ void __launch_bounds__(256) router_logits_bf16x3_kernel(const float* __restrict__ z,
                                                                  const uint16_t* __restrict__ wpl,
                                                                  const float* __restrict__ bias, int T, int E,
                                                                  int L, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t rl_lds[];
  uint8_t* const As = rl_lds;        // 3 planes x 128 token rows
  uint8_t* const Bs = rl_lds + BOP;  // 3 planes x 128 expert rows
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int t0 = blockIdx.y * BT, e0 = blockIdx.x * BE;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int64_t plane = (int64_t)E * L;  // elements per weight plane

  // Staging: A, thread handles float4 f = tid + 256 it (it < 4): row f / 8,
  // K 4 (f % 8); B, uint4 g = tid + 256 it (it < 6): plane g / 512, row
  // (g % 512) / 4, K 8 (g % 4).  Rows past T or E repeat the last one.
  // Source pointers are fixed per thread; a chunk adds k0.
  const float* za[4];
  const uint16_t* wb[6];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int f = tid + 256 * it;
    int r = t0 + (f >> 3);
    r = r < T ? r : T - 1;
    za[it] = z + (int64_t)r * L + 4 * (f & 7);
  }
#pragma unroll
  for (int it = 0; it < 6; ++it) {
    const int g = tid + 256 * it;
    const int p = g >> 9, q = g & 511;
    int r = e0 + (q >> 2);
    r = r < E ? r : E - 1;
    wb[it] = wpl + p * plane + (int64_t)r * L + 8 * (q & 3);
  }
  float4 ra0, ra1, ra2, ra3;
  uint4 rb0, rb1, rb2, rb3, rb4, rb5;
#define RL_GLOAD(k0)                                                     \
  do {                                                                   \
    ra0 = *reinterpret_cast<const float4*>(za[0] + (k0));                \
    ra1 = *reinterpret_cast<const float4*>(za[1] + (k0));                \
    ra2 = *reinterpret_cast<const float4*>(za[2] + (k0));                \
    ra3 = *reinterpret_cast<const float4*>(za[3] + (k0));                \
    rb0 = *reinterpret_cast<const uint4*>(wb[0] + (k0));                 \
    rb1 = *reinterpret_cast<const uint4*>(wb[1] + (k0));                 \
    rb2 = *reinterpret_cast<const uint4*>(wb[2] + (k0));                 \
    rb3 = *reinterpret_cast<const uint4*>(wb[3] + (k0));                 \
    rb4 = *reinterpret_cast<const uint4*>(wb[4] + (k0));                 \
    rb5 = *reinterpret_cast<const uint4*>(wb[5] + (k0));                 \
  } while (0)
  auto store_a = [&](int it, const float4& v) {
    const int f = tid + 256 * it;
    uint2 pl[3];
    split3x4(v, pl);
#pragma unroll
    for (int p = 0; p < 3; ++p)
      *reinterpret_cast<uint2*>(As + p * BPLANE + (f >> 3) * BROW + 8 * (f & 7)) = pl[p];
  };
  auto store_b = [&](int it, const uint4& v) {
    const int g = tid + 256 * it;
    const int p = g >> 9, q = g & 511;
    *reinterpret_cast<uint4*>(Bs + p * BPLANE + (q >> 2) * BROW + 16 * (q & 3)) = v;
  };

  f16v_r acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  RL_GLOAD(0);
  for (int k0 = 0; k0 < L; k0 += BK) {
    __syncthreads();  // previous chunk's fragments are read
    store_a(0, ra0);
    store_a(1, ra1);
    store_a(2, ra2);
    store_a(3, ra3);
    store_b(0, rb0);
    store_b(1, rb1);
    store_b(2, rb2);
    store_b(3, rb3);
    store_b(4, rb4);
    store_b(5, rb5);
    __syncthreads();
    if (k0 + BK < L) RL_GLOAD(k0 + BK);  // lands during this chunk's MFMAs
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int koff = 2 * (16 * kk + 8 * lh);
      bf16x8_r af[2][3], bf[2][3];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          af[t][p] = *reinterpret_cast<const bf16x8_r*>(As + p * BPLANE + (wm + 32 * t + l32) * BROW + koff);
          bf[t][p] = *reinterpret_cast<const bf16x8_r*>(Bs + p * BPLANE + (wn + 32 * t + l32) * BROW + koff);
        }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          f16v_r c = acc[a][b];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][0], bf[b][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][0], bf[b][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][1], bf[b][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][0], bf[b][2], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][1], bf[b][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][2], bf[b][0], c, 0, 0, 0);
          acc[a][b] = c;
        }
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int e = e0 + wn + 32 * b + l32;
    if (e >= E) continue;
    const float bb = bias ? bias[e] : 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + wm + 32 * a + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (t < T) out[(int64_t)t * E + e] = acc[a][b][i] + bb;
      }
  }
#undef RL_GLOAD
}

// logits = sum over slices s = 0 .. split-1, in that order, + bias.
__global__ void __launch_bounds__(256) router_reduce_kernel(const float* __restrict__ part, const float* __restrict__ bias,
                                                           int64_t n, int E, int split, float* __restrict__ logits) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float v = part[i];
    for (int s = 1; s < split; ++s) v += part[(int64_t)s * n + i];
    logits[i] = v + (bias ? bias[i % E] : 0.f);
  }
}

int router_split(int T, int E, int L) {
  const int tiles = ((E + RE - 1) / RE) * ((T + RT - 1) / RT);
  if (tiles >= 256) return 1;
  int split = (512 + tiles - 1) / tiles;
  const int chunks = L / RK;
  return split > chunks ? chunks : split;
}

bool router_bf16x3(int T, int E, int L) {
  return L % BK == 0 && (int64_t)((T + BT - 1) / BT) * ((E + BE - 1) / BE) >= 128;
}

// Number of K slices the fp32 router kernel writes (1: it writes the logits).
int router_slices(int T, int E, int L) {
  if (T <= 0 || router_bf16x3(T, E, L)) return 1;
  const int split = router_split(T, E, L);
  const int kslice = ((L / RK + split - 1) / split) * RK;
  return (L + kslice - 1) / kslice;
}

bool router_reduce_in_topk(int T, int E, int L) { return E <= 1024 && router_slices(T, E, L) > 1; }

hipError_t launch_router_logits(const float* z, const float* w, const float* bias, int T, int E, int L,
                                float* logits, float* partial, uint16_t* wplanes, hipStream_t s,
                                bool leave_partial) {
  if (T == 0) return hipSuccess;
  if (router_bf16x3(T, E, L) && wplanes != nullptr) {
    const int64_t n4 = (int64_t)E * L / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    split3_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(reinterpret_cast<const float4*>(w), n4,
                                                               reinterpret_cast<uint2*>(wplanes));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr size_t smem = 2 * BOP;
    static DeviceOnce attr;
    e = lds_limit_once(attr, {reinterpret_cast<const void*>(&router_logits_bf16x3_kernel)}, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid((E + BE - 1) / BE, (T + BT - 1) / BT);
    router_logits_bf16x3_kernel<<<grid, dim3(256), smem, s>>>(z, wplanes, bias, T, E, L, logits);
    return hipGetLastError();
  }
  const int split = router_split(T, E, L);
  const int kslice = ((L / RK + split - 1) / split) * RK;
  const int nz = (L + kslice - 1) / kslice;
  dim3 grid((E + RE - 1) / RE, (T + RT - 1) / RT, nz);
  if (nz == 1) {
    router_logits_kernel<<<grid, dim3(256), 0, s>>>(z, w, bias, T, E, L, kslice, logits);
    return hipGetLastError();
  }
  router_logits_kernel<<<grid, dim3(256), 0, s>>>(z, w, bias, T, E, L, kslice, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || leave_partial) return e;
  const int64_t n = (int64_t)T * E;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  router_reduce_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(partial, bias, n, E, nz, logits);
  return hipGetLastError();
}

namespace {
__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// (key desc, id asc) "better than"
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}
}  // namespace

// Best (key, id) over the wave, in every lane: DPP swaps within rows of 16
// lanes (pairs, pairs of pairs, half-row mirror, row mirror), then the four
// row winners compared through readlane (uniform result, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ void best_step(float& wk, int& wi) {
  const float ok = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(wk), CTRL, 0xF, 0xF, true));
  const int oi = __builtin_amdgcn_mov_dpp(wi, CTRL, 0xF, 0xF, true);
  if (better(ok, oi, wk, wi)) { wk = ok; wi = oi; }
}
__device__ __forceinline__ void wave_best(float& wk, int& wi) {
  best_step<0xB1>(wk, wi);   // quad_perm 1,0,3,2
  best_step<0x4E>(wk, wi);   // quad_perm 2,3,0,1
  best_step<0x141>(wk, wi);  // row_half_mirror
  best_step<0x140>(wk, wi);  // row_mirror
  float bk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), 0));
  int bi = __builtin_amdgcn_readlane(wi, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float k2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), 16 * r));
    const int i2 = __builtin_amdgcn_readlane(wi, 16 * r);
    if (better(k2, i2, bk, bi)) { bk = k2; bi = i2; }
  }
  wk = bk;
  wi = bi;
}

// Gates of the k winners held by lanes 0..k-1 (raw score `mys` of slot
// `lane`): sigmoid scores over their slot-order sum `ssum`, or with softmax
// gates (raw score = the logit) the softmax over the winners, its sum taken in
// slot order so that every lane and every run divides by the same value.
__device__ __forceinline__ float winner_gate(bool softmax, int k, int lane, float mys, float ssum) {
  if (!softmax) return mys / ssum;
  float mx = lane < k ? mys : -INFINITY;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float ev = lane < k ? expf(mys - mx) : 0.f;
  float esum = 0.f;
  for (int j = 0; j < k; ++j) esum += __shfl(ev, j, 64);
  return ev / esum;
}

__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits,
                                                  const float* __restrict__ sel_bias, int T, int E, int k,
                                                  bool softmax, int32_t* __restrict__ ids,
                                                  float* __restrict__ gates) {
  extern __shared__ float keys_smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // no block-level barrier below
  float* keys = keys_smem + (int64_t)wave * 2 * E;  // selection keys, then raw scores
  float* scores = keys + E;
  const float* lrow = logits + (int64_t)t * E;

  float bk = -INFINITY;
  int bi = 0x7fffffff;
  for (int e0 = lane; e0 < E; e0 += 64 * 8) {
    float lv[8], bv[8];  // eight loads in flight, then their keys
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = min(e0 + 64 * j, E - 1);
      lv[j] = lrow[e];
      bv[j] = sel_bias ? sel_bias[e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + 64 * j;
      if (e >= E) break;
      const float sc = softmax ? lv[j] : sigmoidf(lv[j]);
      float key = sc;
      if (sel_bias) key += bv[j];
      key = fmaxf(key, -FLT_MAX);  // NaN / -inf inputs rank last but stay above "taken" (-inf)
      keys[e] = key;
      scores[e] = sc;
      if (better(key, e, bk, bi)) { bk = key; bi = e; }
    }
  }
  float ssum = 0.f;
  float mys = 0.f;  // raw score of the winner of slot `lane`
  int myid = 0;
  for (int r = 0; r < k; ++r) {
    float wk = bk;
    int wi = bi;
    wave_best(wk, wi);
    const float sw = scores[wi];
    ssum += sw;  // every lane adds the same values in the same (slot) order
    if (lane == r) { mys = sw; myid = wi; }
    if ((wi & 63) == lane) {  // owner marks it taken and rescans its slice
      keys[wi] = -INFINITY;
      bk = -INFINITY;
      bi = 0x7fffffff;
      for (int e = lane; e < E; e += 64) {
        const float key = keys[e];
        if (better(key, e, bk, bi)) { bk = key; bi = e; }
      }
    }
  }
  const float gt = winner_gate(softmax, k, lane, mys, ssum);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = myid;
    gates[(int64_t)t * k + lane] = gt;
  }
}

// Order-preserving map of a float to uint32 (for non-NaN values: a < b as
// floats implies map(a) < map(b); -0 maps below +0).
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Top-k of one token held by a wave: lane l holds expert e = l + 64 j in slot
// j (selection key key[j], -inf past E, and raw score scr[j]).  On return lane
// r < k holds the winner of slot r (id, raw score) and every lane the sum of
// the k winners' raw scores in slot order.  The winners are the k best by
// (key desc, id asc), in that order -- the same as k rounds of "take the best
// remaining", which is what the fallback below does.
//
// Threshold first: let theta be the k-th largest of the 64 lane maxima (a
// radix select over its bit pattern: 32 ballots).  At least k lanes hold a key
// >= theta, so no key below theta can be among the k best; the candidates are
// the keys >= theta, typically a little over k.  If there are at most 64, they
// are packed one per lane through LDS (`cand`: 3 x 64 words per wave), each
// counts the candidates better than itself -- its slot -- and the slots are
// filled through LDS again.  Otherwise (many equal keys) the round-based
// selection runs on the registers.
template <int KPL>
__device__ __forceinline__ void wave_topk(float (&key)[KPL], const float (&scr)[KPL], int lane, int k,
                                          float* cand, int& myid, float& mys, float& ssum) {
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < KPL; ++j) m = fmaxf(m, key[j]);
  const uint32_t um = orderable(m);
  uint32_t th = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = th | (1u << bit);
    if (__popcll(__ballot(um >= c)) >= k) th = c;
  }
  const float theta = from_orderable(th);
  uint32_t cm = 0;  // this lane's candidate slots
#pragma unroll
  for (int j = 0; j < KPL; ++j) cm |= (key[j] >= theta && key[j] > -INFINITY) ? (1u << j) : 0u;
  const int n = __popc(cm);
  int pos = 0, total = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) {  // prefix sum over lanes of n (<= 16 < 32) bit by bit
    const uint64_t bb = __ballot((n >> b) & 1);
    pos += lanes_below(bb) << b;
    total += __popcll(bb) << b;
  }
  ssum = 0.f;
  if (total <= 64) {
    float* ck = cand;
    int* ci = reinterpret_cast<int*>(cand + 64);
    float* cs = cand + 128;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (cm & (1u << j)) {
        ck[pos] = key[j];
        ci[pos] = lane + 64 * j;
        cs[pos] = scr[j];
        ++pos;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool have = lane < total;
    const float kk = have ? ck[lane] : -INFINITY;
    const int ii = have ? ci[lane] : 0x7fffffff;
    const float ss = have ? cs[lane] : 0.f;
    int rank = 0;
    for (int j = 0; j < total; ++j) {
      const float kj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kk), j));
      const int ij = __builtin_amdgcn_readlane(ii, j);
      rank += better(kj, ij, kk, ii) ? 1 : 0;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (have && rank < k) {  // slot `rank`
      ci[rank] = ii;
      cs[rank] = ss;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    myid = lane < k ? ci[lane] : 0;
    mys = lane < k ? cs[lane] : 0.f;
    for (int r = 0; r < k; ++r)  // every lane adds the same values in slot order
      ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mys), r));
    return;
  }
  // Round-based selection: the winner's lane marks it taken and rescans its
  // KPL keys without touching memory; the winner's score is broadcast by
  // readlane.
  float bk = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < KPL; ++j)
    if (better(key[j], lane + 64 * j, bk, bi)) { bk = key[j]; bi = lane + 64 * j; }
  mys = 0.f;
  myid = 0;
  for (int r = 0; r < k; ++r) {
    float wk = bk;
    int wi = bi;
    wave_best(wk, wi);
    const int wj = wi >> 6;  // uniform
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) mine = j == wj ? scr[j] : mine;
    const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), wi & 63));
    ssum += sw;
    if (lane == r) { mys = sw; myid = wi; }
    if ((wi & 63) == lane) {
      bk = -INFINITY;
      bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        key[j] = j == wj ? -INFINITY : key[j];
        if (better(key[j], lane + 64 * j, bk, bi)) { bk = key[j]; bi = lane + 64 * j; }
      }
    }
  }
}

// Same selection as topk_kernel with each lane's keys and raw scores in
// registers (expert e = lane + 64 j in slot j, E <= 64 * KPL): same keys, same
// order of comparisons and sums, so the same ids and gates.
template <int KPL>
__global__ void __launch_bounds__(256) topk_reg_kernel(const float* __restrict__ logits,
                                                      const float* __restrict__ sel_bias, int T, int E, int k,
                                                      bool softmax, int32_t* __restrict__ ids,
                                                      float* __restrict__ gates) {
  __shared__ float cand[4][3 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // no block-level barrier below
  const float* lrow = logits + (int64_t)t * E;
  float key[KPL], scr[KPL];
  // All of the lane's loads first (indices past E re-read the last logit and
  // are discarded below), so they are in flight together instead of one
  // memory latency per key.
  float lv[KPL], bv[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = min(lane + 64 * j, E - 1);
    lv[j] = lrow[e];
    bv[j] = sel_bias ? sel_bias[e] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < KPL; ++j) {  // (selects, not branches: the arrays stay in plain registers)
    const bool in = lane + 64 * j < E;
    const float sc = softmax ? lv[j] : sigmoidf(lv[j]);
    const float kk = fmaxf(sel_bias ? sc + bv[j] : sc, -FLT_MAX);  // NaN / -inf rank last, above "taken"
    key[j] = in ? kk : -INFINITY;  // past E: never selected (k <= E finite keys exist)
    scr[j] = in ? sc : 0.f;
  }
  int myid;
  float mys, ssum;
  wave_topk<KPL>(key, scr, lane, k, cand[wave], myid, mys, ssum);
  const float gt = winner_gate(softmax, k, lane, mys, ssum);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = myid;
    gates[(int64_t)t * k + lane] = gt;
  }
}

// Few tokens: the router's K-slice partial sums, reduced here instead of in a
// kernel of their own.  One workgroup per token: its 256 threads add the
// slices of the token's E logits in slice order and add the logit bias (the
// reduce kernel's arithmetic, so the same logits), write them out and to LDS;
// then the first wave selects the top k from LDS (E <= 1024).
__global__ void __launch_bounds__(256) router_reduce_topk_kernel(const float* __restrict__ part, int nz,
                                                                const float* __restrict__ logit_bias,
                                                                const float* __restrict__ sel_bias, int T, int E,
                                                                int k, bool softmax, float* __restrict__ logits,
                                                                int32_t* __restrict__ ids,
                                                                float* __restrict__ gates) {
  constexpr int EPT = 4;    // logits per thread (E <= 1024)
  constexpr int SB = 32;    // slices loaded per batch (all in flight)
  __shared__ float lg[256 * EPT];
  __shared__ float cand[3 * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int t = blockIdx.x;
  const int64_t n = (int64_t)T * E;
  int64_t o[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) o[i] = (int64_t)t * E + min(tid + 256 * i, E - 1);
  constexpr int KPL = 16;
  float bv[KPL];  // selection bias of wave 0's keys, loaded beside the slices
#pragma unroll
  for (int j = 0; j < KPL; ++j) bv[j] = sel_bias && tid < 64 ? sel_bias[min(lane + 64 * j, E - 1)] : 0.f;
  float v[EPT];
  for (int s0 = 0; s0 < nz; s0 += SB) {
    float p[EPT][SB];
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      const int64_t so = (int64_t)min(s0 + s, nz - 1) * n;
#pragma unroll
      for (int i = 0; i < EPT; ++i) p[i][s] = part[so + o[i]];
    }
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int sl = s0 + s;
        v[i] = sl == 0 ? p[i][s] : (sl < nz ? v[i] + p[i][s] : v[i]);
      }
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + 256 * i;
    if (e < E) {
      const float l = v[i] + (logit_bias ? logit_bias[e] : 0.f);
      logits[(int64_t)t * E + e] = l;
      lg[e] = l;
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  float key[KPL], scr[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = lane + 64 * j;
    const bool in = e < E;
    const float lv = lg[in ? e : E - 1];
    const float sc = softmax ? lv : sigmoidf(lv);
    const float kk = fmaxf(sel_bias ? sc + bv[j] : sc, -FLT_MAX);
    key[j] = in ? kk : -INFINITY;
    scr[j] = in ? sc : 0.f;
  }
  int myid;
  float mys, ssum;
  wave_topk<KPL>(key, scr, lane, k, cand, myid, mys, ssum);
  const float gt = winner_gate(softmax, k, lane, mys, ssum);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = myid;
    gates[(int64_t)t * k + lane] = gt;
  }
}

hipError_t launch_router_reduce_topk(const float* partial, int nz, const float* logit_bias, const float* sel_bias,
                                     int T, int E, int k, bool softmax_gates, float* logits, int32_t* ids,
                                     float* gates, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!partial || nz < 1 || E < 1 || E > 1024 || k < 1 || k > 64 || k > E) return hipErrorInvalidValue;
  router_reduce_topk_kernel<<<dim3((unsigned)T), dim3(256), 0, s>>>(partial, nz, logit_bias, sel_bias, T, E, k,
                                                                   softmax_gates, logits, ids, gates);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* sel_bias, int T, int E, int k, bool softmax_gates,
                       int32_t* ids, float* gates, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 64 * 16) {
    topk_reg_kernel<16><<<dim3((T + 3) / 4), dim3(256), 0, s>>>(logits, sel_bias, T, E, k, softmax_gates, ids,
                                                                gates);
    return hipGetLastError();
  }
  const size_t smem = (size_t)4 * 2 * E * sizeof(float);  // 4 waves x (keys + scores): 128 KB at E = 4096
  static DeviceOnce attr;  // the largest E (4096) once per device
  hipError_t e = lds_limit_once(attr, {reinterpret_cast<const void*>(&topk_kernel)}, 4 * 2 * 4096 * (int)sizeof(float));
  if (e != hipSuccess) return e;
  topk_kernel<<<dim3((T + 3) / 4), dim3(256), smem, s>>>(logits, sel_bias, T, E, k, softmax_gates, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
