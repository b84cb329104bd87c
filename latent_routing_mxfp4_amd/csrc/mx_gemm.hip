// mx_gemm.hip -- grouped / dense block-scaled GEMM on the gfx950 matrix cores.
//
// C = deq(A) deq(B)^T with A an MXFP8 (E4M3) activation matrix and B an MXFP4
// (E2M1) weight matrix [N][K], both blocked by 32 along K.  The MX scales are
// applied inside v_mfma_scale_f32_16x16x128_f8f6f4, so the weights are consumed
// as stored, never expanded to a wider copy (Kimi K3 open-weights serving,
// section "Native MXFP4": kernels should consume that representation).
//
// The MX kernels run
//   * the routed experts as one grouped GEMM over ragged, runtime-sized
//     segments (Four Bits at a Time, "What has to change in the serving
//     stacks": up to 896 runtime-sized groups per layer) -- the group of an
//     M-tile is found from the device-side prefix of M-tiles per expert, so
//     nothing is read back to the host;
//   * the dense projections (latent down/up) and the shared experts.
//
// Kernels here: the weight-streaming MX GEMM for few rows per group (decode),
// and the register-tiled bf16 GEMM of the dense latent down-projection for
// few rows (its prefill twin is in mx_gemm_wide.hip).  The prefill-shaped MX GEMM is in mx_gemm_wide.hip and the
// epilogues shared by all of them in gemm_epilogue.hpp.  MX weights are read
// in fragment order (kernels.hpp).
#include "kernels.hpp"
#include "mx_device.hpp"
#include "lds_pipe.hpp"
#include "gemm_epilogue.hpp"

namespace moe {

namespace {

struct Frag8 {  // E4M3 A fragment: 32 bytes per lane
  uint4 lo, hi;
};

__device__ __forceinline__ v8i as_v8i(const Frag8& f) {
  v8i r;
  r[0] = (int)f.lo.x; r[1] = (int)f.lo.y; r[2] = (int)f.lo.z; r[3] = (int)f.lo.w;
  r[4] = (int)f.hi.x; r[5] = (int)f.hi.y; r[6] = (int)f.hi.z; r[7] = (int)f.hi.w;
  return r;
}

__device__ __forceinline__ v8i as_v8i(const uint4& f) {
  v8i r;
  r[0] = (int)f.x; r[1] = (int)f.y; r[2] = (int)f.z; r[3] = (int)f.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 to_uint4(const u32x4& v) { return make_uint4(v[0], v[1], v[2], v[3]); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& f) {
  union {
    uint4 u;
    bf16x8 b;
  } c;
  c.u = f;
  return c.b;
}

}  // namespace

// Map a workgroup to (group, M-tile, N-tile).  Returns false for workgroups
// past the last M-tile (the grid is sized for the worst case).
template <int MT, int NT>
__device__ __forceinline__ bool decode_tile(const GemmArgs& p, int wave, int NWC, Tile& t) {
  const int n_ntiles = (p.N + NT - 1) / NT;
  const int gm = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - gm * n_ntiles;
  if (p.offsets) {
    const int total = p.mtile_start[p.G];
    if (gm >= total) return false;
    int lo = 0, hi = p.G;  // mtile_start[lo] <= gm < mtile_start[hi]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (p.mtile_start[mid] <= gm) lo = mid; else hi = mid;
    }
    t.g = lo;
    t.row_base = p.offsets[lo];
    t.rows = p.offsets[lo + 1] - t.row_base;
    t.m0 = (gm - p.mtile_start[lo]) * MT;
  } else {
    const int mpg = (p.M + MT - 1) / MT;
    t.g = gm / mpg;
    if (t.g >= p.G) return false;
    t.m0 = (gm - t.g * mpg) * MT;
    t.rows = p.M;
    t.row_base = 0;
  }
  t.n0 = nt * NT + wave * NWC;
  return true;
}

// Dense bf16 GEMM on exactly decoded MX operands (v_mfma_f32_16x16x32_bf16):
// A = bf16 [M][K], B = bf16 [N][K] (seg.a / seg.b, lda = K).  Every product of
// an E4M3 and an E2M1 value (with power-of-two scales) is exact in bf16 x bf16
// -> fp32, and this instruction accumulates at fp32 precision, unlike the
// block-scaled MFMA, which sums each 32-element block in a window of about 14
// bits below the block's largest product.  The latent down-projection feeds
// the router, whose top-k must be decided on an fp32-accurate latent, so it
// runs here.  A lane loads 64 contiguous bytes (32 K values) of its row per
// 128-wide K-step and issues four MFMAs, slice u taking K [32g + 8u, +8); A and
// B use the same slicing, so the pairing of K indices is consistent.
template <int MW, int NW, int EPI>
__global__ void __launch_bounds__(256) bf16_gemm_kernel(const GemmArgs p) {
  constexpr int MT = 16 * MW;
  constexpr int NT = 4 * 16 * NW;
  static_assert(EPI == EPI_F32 || NW % 2 == 0, "quantising epilogues need whole 32-column blocks per wave");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  Tile t;
  if (!decode_tile<MT, NT>(p, wave, 16 * NW, t)) return;
  const GemmSeg& sg = p.seg[0];
  const int K = sg.K;
  const int ksteps = K >> 7;
  const uint16_t* ap[MW];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    int r = t.m0 + 16 * mi + r16;
    r = r < t.rows ? r : t.rows - 1;
    ap[mi] = reinterpret_cast<const uint16_t*>(sg.a) + (int64_t)r * K + 32 * g4;
  }
  const uint16_t* bp[NW];
#pragma unroll
  for (int ni = 0; ni < NW; ++ni) {
    int c = t.n0 + 16 * ni + r16;
    c = c < p.N ? c : p.N - 1;
    bp[ni] = reinterpret_cast<const uint16_t*>(sg.b) + (int64_t)c * K + 32 * g4;
  }
  v4f acc[MW][NW][1];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi)
#pragma unroll
    for (int ni = 0; ni < NW; ++ni) acc[mi][ni][0] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 fa[MW][4], fb[NW][4];
  auto load = [&](int ks) {
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int u = 0; u < 4; ++u) fa[mi][u] = reinterpret_cast<const uint4*>(ap[mi] + 128 * ks)[u];
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int u = 0; u < 4; ++u) fb[ni][u] = reinterpret_cast<const uint4*>(bp[ni] + 128 * ks)[u];
  };
  load(0);
  for (int ks = 0; ks < ksteps; ++ks) {
    uint4 ca[MW][4], cb[NW][4];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int u = 0; u < 4; ++u) ca[mi][u] = fa[mi][u];
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int u = 0; u < 4; ++u) cb[ni][u] = fb[ni][u];
    if (ks + 1 < ksteps) load(ks + 1);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
          acc[mi][ni][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ca[mi][u]), as_bf16x8(cb[ni][u]),
                                                                   acc[mi][ni][0], 0, 0, 0);
  }
  epilogue<MW, NW, 1, EPI>(p, t, acc, r16, g4);
}

// Weight-streaming variant for few rows per group (decode).  The weights are
// read exactly once, so the kernel is HBM-bound.  A workgroup of 4 waves owns
// MT x NT outputs (each wave 16*NW weight rows); per 128-deep K-step a wave
// loads, for each of its weight fragments, the fragment-order block of codes
// (1 KB contiguous; lane l takes its 16-byte MFMA operand at 16 l, read
// non-temporally) and the 64 contiguous scale bytes of the block's 16 rows,
// one K-step ahead of the MFMAs.  The few activation rows (L2-resident) are
// read in the E4M3 operand layout straight from global memory.
template <int MW, int NW, int EPI>
__global__ void __launch_bounds__(256) mx_gemm_stream_kernel(const GemmArgs p) {
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT;
  constexpr int NB = SWI ? 2 : 1;
  constexpr int MT = 16 * MW;
  constexpr int NT = 4 * 16 * NW;
  static_assert(EPI == EPI_F32 || NW % 2 == 0, "quantising epilogues need whole 32-column blocks per wave");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  Tile t;
  if (!decode_tile<MT, NT>(p, wave, 16 * NW, t)) return;  // uniform across the workgroup

  int64_t arow[MW];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    int r = t.m0 + 16 * mi + r16;
    r = r < t.rows ? r : t.rows - 1;
    int sr = t.row_base + r;
    if (p.offsets) arow[mi] = p.gather ? (int64_t)(p.gather[sr] / p.gather_div) : (int64_t)sr;
    else arow[mi] = r;
  }
  // First weight row of fragment ni, clamped so that its 16-row block lies in
  // [0, N) (N % 16 == 0); rows past N are computed on repeated data, never stored.
  int fcol[NW];
#pragma unroll
  for (int ni = 0; ni < NW; ++ni) {
    const int c = t.n0 + 16 * ni;
    fcol[ni] = c < p.N - 16 ? c : p.N - 16;
  }

  v4f acc[MW][NW][NB];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi)
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int h = 0; h < NB; ++h) acc[mi][ni][h] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int s = 0; s < p.nseg; ++s) {
    const GemmSeg& sg = p.seg[s];
    const int K = sg.K;
    const int nks = K >> 7;
    const int kb = K >> 5;
    const uint8_t* ap[MW];
    const uint8_t* asp[MW];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
      ap[mi] = sg.a + arow[mi] * sg.lda + 16 * g4;
      asp[mi] = sg.as + arow[mi] * kb + g4;
    }
    const uint8_t* bp[NW][NB];
    const uint8_t* bsp[NW][NB];
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int h = 0; h < NB; ++h) {
        bp[ni][h] = (h == 0 ? sg.b : sg.b2) + (int64_t)t.g * sg.b_gstride + (int64_t)(fcol[ni] >> 4) * nks * 1024 +
                    16 * lane;
        bsp[ni][h] = (h == 0 ? sg.bs : sg.b2s) + (int64_t)t.g * sg.bs_gstride + 4 * (int64_t)(fcol[ni] + r16) + g4;
      }
    const int64_t bs_k = 4 * (int64_t)p.N;  // bytes between K-steps of the scales

    uint4 fb[NW][NB];
    int fs[NW][NB];
    auto load_b = [&](int ks) {
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) {
          fb[ni][h] = to_uint4(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp[ni][h] + 1024 * ks)));
          fs[ni][h] = bsp[ni][h][bs_k * ks];
        }
    };
    load_b(0);
    for (int ks = 0; ks < nks; ++ks) {
      uint4 cb[NW][NB];
      int cs[NW][NB];
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) {
          cb[ni][h] = fb[ni][h];
          cs[ni][h] = fs[ni][h];
        }
      if (ks + 1 < nks) load_b(ks + 1);
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const uint8_t* q = ap[mi] + 128 * ks;
        Frag8 fa;
        fa.lo = *reinterpret_cast<const uint4*>(q);
        fa.hi = *reinterpret_cast<const uint4*>(q + 64);
        const v8i av = as_v8i(fa);
        const int sa = asp[mi][4 * ks];
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
          for (int h = 0; h < NB; ++h) acc[mi][ni][h] = mfma_f8f4(av, as_v8i(cb[ni][h]), acc[mi][ni][h], sa, cs[ni][h]);
      }
    }
  }
  epilogue<MW, NW, NB, EPI>(p, t, acc, r16, g4);
}

template <int MW, int NW, int EPI>
static hipError_t launch_stream_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int NT = 4 * 16 * NW;
  if (a.N % 16 != 0) return hipErrorInvalidValue;  // fragment-order weights
  const int n_ntiles = (a.N + NT - 1) / NT;
  const int64_t grid = (int64_t)a.max_mtiles * n_ntiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  mx_gemm_stream_kernel<MW, NW, EPI><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

int gemm_mtile(int shape) {
  return shape == GEMM_STREAM16 ? 16 : shape == GEMM_STREAM64 ? 64 : gemm_wide_mtile();
}

template <int MW, int NW, int EPI>
static hipError_t launch_bf16_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int NT = 4 * 16 * NW;
  const int n_ntiles = (a.N + NT - 1) / NT;
  const int64_t grid = (int64_t)a.max_mtiles * n_ntiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  bf16_gemm_kernel<MW, NW, EPI><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

// The epilogue addresses a wave's output rows with 32-bit offsets from a
// wave-uniform base (gemm_epilogue.hpp): N and ldc below 2^22 keep 128 rows
// of fp32 output under 4 GB.
static bool epilogue_dims_ok(const GemmArgs& a) {
  return a.N > 0 && a.N < (1 << 22) && a.ldc >= 0 && a.ldc < (1 << 22);
}

hipError_t launch_bf16_gemm_quant(const GemmArgs& a, int shape, hipStream_t s) {
  if (!epilogue_dims_ok(a)) return hipErrorInvalidValue;
  if (shape == GEMM_WIDE) return launch_bf16_gemm_wide(a, s);
  return shape == GEMM_STREAM16 ? launch_bf16_cfg<1, 2, EPI_F32_QUANT>(a, s)
                                : launch_bf16_cfg<4, 2, EPI_F32_QUANT>(a, s);
}

hipError_t launch_mx_gemm(const GemmArgs& a, int epi, int shape, hipStream_t s) {
  if (!epilogue_dims_ok(a)) return hipErrorInvalidValue;
  if (shape == GEMM_WIDE) return launch_mx_gemm_wide(a, epi, s);
  if (shape == GEMM_STREAM16) {
    switch (epi) {
      case EPI_F32: return launch_stream_cfg<1, 4, EPI_F32>(a, s);  // 64 columns per wave: more bytes in flight
      case EPI_F32_QUANT: return launch_stream_cfg<1, 2, EPI_F32_QUANT>(a, s);
      default: return launch_stream_cfg<1, 2, EPI_SWIGLU_QUANT>(a, s);
    }
  }
  if (shape == GEMM_STREAM64) {
    switch (epi) {
      case EPI_F32: return launch_stream_cfg<4, 2, EPI_F32>(a, s);
      case EPI_F32_QUANT: return launch_stream_cfg<4, 2, EPI_F32_QUANT>(a, s);
      default: return launch_stream_cfg<4, 2, EPI_SWIGLU_QUANT>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
