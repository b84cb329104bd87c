// mx_gemm.hip -- grouped / dense block-scaled GEMM on the gfx950 matrix cores.
//
// C = deq(A) deq(B)^T with A an MXFP8 (E4M3) activation matrix and B an MXFP4
// (E2M1) weight matrix [N][K], both blocked by 32 along K.  The MX scales are
// applied inside v_mfma_scale_f32_16x16x128_f8f6f4, so the weights are consumed
// as stored, never expanded to a wider copy (Kimi K3 open-weights serving,
// section "Native MXFP4": kernels should consume that representation).
//
// The same kernel runs
//   * the routed experts as one grouped GEMM over ragged, runtime-sized
//     segments (Four Bits at a Time, "What has to change in the serving
//     stacks": up to 896 runtime-sized groups per layer) -- the group of an
//     M-tile is found from the device-side prefix of M-tiles per expert, so
//     nothing is read back to the host;
//   * the dense projections (latent down/up) and the shared experts.
//
// Work decomposition: a workgroup of 4 waves owns an (MT x NT) output tile;
// the waves split the N columns, each wave computes MT x (16*NW) with
// MW x NW 16x16 MFMA tiles (two accumulators per tile for SwiGLU: gate and
// up).  Operands go straight from global memory into the MFMA register
// layout, one 16-byte load per lane per E2M1 fragment, two per E4M3 fragment
// (the two K halves the E4M3 operand layout interleaves),
// one dword of 4 block scales per row per K-step.  The K loop is software
// pipelined one K-step deep.
//
// Epilogues: fp32 store; fp32 store plus MXFP8 quantisation along N; or
// h = SiLU(gate) * up quantised to MXFP8 (the expert hidden state; h itself is
// also stored in fp32 when an output pointer is given, for tracing), where the
// 32-column block of a row sits in one wave (two adjacent 16-column tiles x 16
// lanes), so its maximum is a 16-lane xor reduction.
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

template <int MW, int NW, int EPI>
__global__ void __launch_bounds__(256) mx_gemm_kernel(const GemmArgs p) {
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT;
  constexpr int NB = SWI ? 2 : 1;
  constexpr int MT = 16 * MW;
  constexpr int NT = 4 * 16 * NW;
  static_assert(EPI == EPI_F32 || NW % 2 == 0, "quantising epilogues need whole 32-column blocks per wave");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  Tile t;
  if (!decode_tile<MT, NT>(p, wave, 16 * NW, t)) return;

  // Rows of A this lane feeds (clamped into the group; results of clamped rows are dropped).
  int64_t arow[MW];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    int r = t.m0 + 16 * mi + r16;
    r = r < t.rows ? r : t.rows - 1;
    int sr = t.row_base + r;
    if (p.offsets) arow[mi] = p.gather ? (int64_t)(p.gather[sr] / p.gather_div) : (int64_t)sr;
    else arow[mi] = r;
  }
  int bcol[NW];
#pragma unroll
  for (int ni = 0; ni < NW; ++ni) {
    int c = t.n0 + 16 * ni + r16;
    bcol[ni] = c < p.N ? c : p.N - 1;
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
    const int ksteps = K >> 7;
    const int64_t lds = sg.lda >> 5;
    const uint8_t* ap[MW];
    const uint32_t* asp[MW];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
      ap[mi] = sg.a + arow[mi] * sg.lda + 16 * g4;
      asp[mi] = reinterpret_cast<const uint32_t*>(sg.as + arow[mi] * lds);
    }
    const uint8_t* bp[NW][NB];
    const uint32_t* bsp[NW][NB];
#pragma unroll
    for (int ni = 0; ni < NW; ++ni) {
#pragma unroll
      for (int h = 0; h < NB; ++h) {
        const uint8_t* bb = h == 0 ? sg.b : sg.b2;
        const uint8_t* bbs = h == 0 ? sg.bs : sg.b2s;
        bp[ni][h] = bb + (int64_t)t.g * sg.b_gstride + (int64_t)bcol[ni] * (K >> 1) + 16 * g4;
        bsp[ni][h] =
            reinterpret_cast<const uint32_t*>(bbs + (int64_t)t.g * sg.bs_gstride + (int64_t)bcol[ni] * (K >> 5));
      }
    }

    Frag8 fa[MW];
    uint32_t sa[MW];
    uint4 fb[NW][NB];
    uint32_t sb[NW][NB];
    auto load = [&](int ks) {
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const uint8_t* q = ap[mi] + 128 * ks;  // K [16g, +16) and [64+16g, +16) of this K-step
        fa[mi].lo = *reinterpret_cast<const uint4*>(q);
        fa[mi].hi = *reinterpret_cast<const uint4*>(q + 64);
        sa[mi] = asp[mi][ks] >> (8 * g4);
      }
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) {
          fb[ni][h] = *reinterpret_cast<const uint4*>(bp[ni][h] + 64 * ks);
          sb[ni][h] = bsp[ni][h][ks] >> (8 * g4);
        }
    };

    load(0);
    for (int ks = 0; ks < ksteps; ++ks) {
      Frag8 ca[MW];
      uint32_t csa[MW];
      uint4 cb[NW][NB];
      uint32_t csb[NW][NB];
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) { ca[mi] = fa[mi]; csa[mi] = sa[mi]; }
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) { cb[ni][h] = fb[ni][h]; csb[ni][h] = sb[ni][h]; }
      if (ks + 1 < ksteps) load(ks + 1);
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const v8i av = as_v8i(ca[mi]);
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
          for (int h = 0; h < NB; ++h)
            acc[mi][ni][h] = mfma_f8f4(av, as_v8i(cb[ni][h]), acc[mi][ni][h], (int)csa[mi], (int)csb[ni][h]);
      }
    }
  }
  epilogue<MW, NW, NB, EPI>(p, t, acc, r16, g4);
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
// read exactly once, so the kernel is HBM-bound and its loads are shaped for
// that:
//  * codes: per 256-wide K super-step each lane reads 32 contiguous bytes of its
//    weight row, and the four lane groups of a wave together read the row's
//    whole 128-byte line in one pass (a half-line read and its other half
//    issued one step later get evicted in between and fetched twice);
//  * scales: the workgroup copies its tile's E8M0 rows (contiguous in memory)
//    into LDS once per K segment, instead of touching each 128-byte scale line
//    once per K-step.
// The two 32-element blocks a lane loads per super-step feed two MFMAs (u = 0,
// 1); in MFMA u lane group g holds physical block 8s + 2g + u, and the E4M3
// operand gathers the matching K values in its split-half layout.  A K tail of
// 128 uses the plain one-step layout.
template <int MW, int NW, int EPI>
__global__ void __launch_bounds__(256) mx_gemm_stream_kernel(const GemmArgs p) {
  extern __shared__ uint8_t bscale_lds[];  // [NB][NT rows][K/32]
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
  const int tile_n0 = t.n0 - wave * 16 * NW;

  int64_t arow[MW];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    int r = t.m0 + 16 * mi + r16;
    r = r < t.rows ? r : t.rows - 1;
    int sr = t.row_base + r;
    if (p.offsets) arow[mi] = p.gather ? (int64_t)(p.gather[sr] / p.gather_div) : (int64_t)sr;
    else arow[mi] = r;
  }
  int bcol[NW];
#pragma unroll
  for (int ni = 0; ni < NW; ++ni) {
    int c = t.n0 + 16 * ni + r16;
    bcol[ni] = c < p.N ? c : p.N - 1;
  }
  const int nrows = min(NT, p.N - tile_n0);

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
    const int kb = K >> 5;  // scale bytes per row (multiple of 4)
    // ---- stage this tile's B scales in LDS
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>((h == 0 ? sg.bs : sg.b2s) +
                                                              (int64_t)t.g * sg.bs_gstride + (int64_t)tile_n0 * kb);
      uint32_t* dst = reinterpret_cast<uint32_t*>(bscale_lds + h * NT * kb);
      const int nw = nrows * kb / 4;
      for (int i = tid; i < nw; i += 256) dst[i] = src[i];
    }
    __syncthreads();

    const uint8_t* ap[MW];
    const uint8_t* asp[MW];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
      ap[mi] = sg.a + arow[mi] * sg.lda;
      asp[mi] = sg.as + arow[mi] * kb;
    }
    const uint8_t* bp[NW][NB];
    const uint8_t* bsl[NW][NB];
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int h = 0; h < NB; ++h) {
        bp[ni][h] = (h == 0 ? sg.b : sg.b2) + (int64_t)t.g * sg.b_gstride + (int64_t)bcol[ni] * (K >> 1);
        const int lr = min(wave * 16 * NW + 16 * ni + r16, nrows - 1);
        bsl[ni][h] = bscale_lds + h * NT * kb + lr * kb;
      }

    const int nsup = K >> 8;
    const int a_off = 32 * (2 * (g4 >> 1)) + 16 * (g4 & 1);   // + 32u, second half at +128
    uint4 fb[NW][NB][2];
    auto load_b = [&](int ss) {
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) {
          const u32x4* q = reinterpret_cast<const u32x4*>(bp[ni][h] + 128 * ss + 32 * g4);
          fb[ni][h][0] = to_uint4(__builtin_nontemporal_load(q));
          fb[ni][h][1] = to_uint4(__builtin_nontemporal_load(q + 1));
        }
    };
    if (nsup > 0) load_b(0);
    for (int ss = 0; ss < nsup; ++ss) {
      uint4 cb[NW][NB][2];
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) { cb[ni][h][0] = fb[ni][h][0]; cb[ni][h][1] = fb[ni][h][1]; }
      if (ss + 1 < nsup) load_b(ss + 1);
      uint32_t sbw[NW][NB];
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) sbw[ni][h] = *reinterpret_cast<const uint16_t*>(bsl[ni][h] + 8 * ss + 2 * g4);
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const uint32_t saw = *reinterpret_cast<const uint16_t*>(asp[mi] + 8 * ss + 2 * g4);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint8_t* q = ap[mi] + 256 * ss + a_off + 32 * u;
          Frag8 fa;
          fa.lo = *reinterpret_cast<const uint4*>(q);
          fa.hi = *reinterpret_cast<const uint4*>(q + 128);
          const v8i av = as_v8i(fa);
          const int sa = (int)(saw >> (8 * u));
#pragma unroll
          for (int ni = 0; ni < NW; ++ni)
#pragma unroll
            for (int h = 0; h < NB; ++h)
              acc[mi][ni][h] = mfma_f8f4(av, as_v8i(cb[ni][h][u]), acc[mi][ni][h], sa, (int)(sbw[ni][h] >> (8 * u)));
        }
      }
    }
    if (K & 255) {  // one 128-wide K-step left: plain layout
      const int kl = (K >> 7) - 1;
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const uint8_t* q = ap[mi] + 128 * kl + 16 * g4;
        Frag8 fa;
        fa.lo = *reinterpret_cast<const uint4*>(q);
        fa.hi = *reinterpret_cast<const uint4*>(q + 64);
        const v8i av = as_v8i(fa);
        const int sa = asp[mi][4 * kl + g4];
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
          for (int h = 0; h < NB; ++h) {
            const uint4 fbt = *reinterpret_cast<const uint4*>(bp[ni][h] + 64 * kl + 16 * g4);
            acc[mi][ni][h] = mfma_f8f4(av, as_v8i(fbt), acc[mi][ni][h], sa, (int)bsl[ni][h][4 * kl + g4]);
          }
      }
    }
  }
  epilogue<MW, NW, NB, EPI>(p, t, acc, r16, g4);
}

// LDS-staged tiled variant (many rows per group: prefill).  A workgroup owns
// a 128-row x 128-weight-row tile (for SwiGLU: 64 gate + the matching 64 up
// rows, i.e. 64 output columns); its 4 waves form a 2 x 2 grid, each computing
// 64 rows x 64 weight rows with 16 MFMAs per 128-wide K-step.
//
// Operands move global -> LDS with gfx950's direct loads (global_load_lds,
// 16 bytes per lane, no staging registers) through a 3-buffer ring: while the
// MFMAs consume K-step k, the loads of k+1 and k+2 are in flight.  A wave
// issues 7 loads per K-step (4 for A, 2 for B, 1 for the scales), so
// "vmcnt <= 7" means step k has landed.  A lane's LDS slot is fixed by the
// hardware (base + 16 * lane), so each lane fetches whichever global chunk
// belongs in that slot; the LDS rows are XOR-swizzled by 16-byte chunk so the
// 16 rows a fragment read touches fall on distinct banks.  The routed gate/up
// GEMM gathers its A rows through the permutation in these loads.
//
// Tile order: the flat tile list is cut into 8 contiguous chunks, one per XCD
// (workgroup i runs on XCD i % 8), so an expert's tiles share one L2; inside
// an expert the M-tiles of one weight column-tile are consecutive, so each
// weight tile is fetched from HBM once and reused from L2.
constexpr int LT_M = 128;   // rows per tile
constexpr int LT_B = 128;   // weight rows per tile
constexpr int LT_OFF_B = LT_M * 128;
constexpr int LT_OFF_AS = LT_OFF_B + LT_B * 64;
constexpr int LT_OFF_BS = LT_OFF_AS + 4 * LT_M;
constexpr int LT_STAGE = LT_OFF_BS + 4 * LT_B;   // bytes per LDS buffer (25600)
constexpr int LT_NBUF = 3;
constexpr int LT_LOADS = 7;                       // direct loads per wave per K-step

template <int EPI>
__global__ void __launch_bounds__(256) mx_gemm_lds_kernel(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT;
  constexpr int NB = SWI ? 2 : 1;
  constexpr int NCOL = SWI ? LT_B / 2 : LT_B;       // output columns per tile
  constexpr int NW = SWI ? 2 : 4;                     // 16-col fragments per wave (per matrix)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile decode (XCD-chunked, M-fastest inside an expert)
  const bool routed = p.offsets != nullptr;
  int g, mt, nt, rows, row_base;
  if (!decode_lds_tile<LT_M>(p, NCOL, g, mt, nt, rows, row_base)) return;
  const int m0 = mt * LT_M;
  const int col0 = nt * NCOL;

  // ---- what this lane loads.  A: load i (0..3) fills LDS bytes [1024*(4*wave+i), +1024):
  // tile row 32*wave + 8*i + lane/8, physical chunk lane%8.  B: load i (0..1) fills
  // [OFF_B + 1024*(2*wave+i), +1024): tile row 32*wave + 16*i + lane/4, physical
  // chunk lane%4.  Scales: wave w fills dwords [64w, 64w+64) of the A|B scale columns.
  auto a_src_row = [&](int trow) -> int64_t {
    int r = m0 + trow;
    r = r < rows ? r : rows - 1;
    const int sr = row_base + r;
    return routed ? (p.gather ? (int64_t)(p.gather[sr] / p.gather_div) : (int64_t)sr) : (int64_t)r;
  };
  auto b_col = [&](int trow, int& h) {
    int c;
    if (SWI) { h = trow >= NCOL; c = col0 + (trow - h * NCOL); }
    else { h = 0; c = col0 + trow; }
    return c < p.N ? c : p.N - 1;
  };
  int64_t a_row[4];
  int a_chunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    a_row[i] = a_src_row(r);
    a_chunk[i] = (lane & 7) ^ (r & 7);
  }
  int b_trow[2], b_chunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 32 * wave + 16 * i + (lane >> 2);
    b_trow[i] = r;
    b_chunk[i] = (lane & 3) ^ ((r >> 1) & 3);
  }
  const int s_trow = 64 * (wave & 1) + lane;        // tile row of this lane's scale dword
  const int64_t s_arow = wave < 2 ? a_src_row(s_trow) : 0;

  v4f acc[4][NW][NB];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int h = 0; h < NB; ++h) acc[mi][ni][h] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int sgi = 0; sgi < p.nseg; ++sgi) {
    const GemmSeg& sg = p.seg[sgi];
    const int K = sg.K;
    const int ksteps = K >> 7;
    const int kb = K >> 5;
    const uint8_t* ga[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ga[i] = sg.a + a_row[i] * sg.lda + 16 * a_chunk[i];
    const uint8_t* gb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int h;
      const int c = b_col(b_trow[i], h);
      gb[i] = (h ? sg.b2 : sg.b) + (int64_t)g * sg.b_gstride + (int64_t)c * (K >> 1) + 16 * b_chunk[i];
    }
    const uint8_t* gs;
    if (wave < 2) {
      gs = sg.as + s_arow * kb;
    } else {
      int h;
      const int c = b_col(s_trow, h);
      gs = (h ? sg.b2s : sg.bs) + (int64_t)g * sg.bs_gstride + (int64_t)c * kb;
    }
    auto issue = [&](int ks) {
      uint8_t* buf = lds + (ks % LT_NBUF) * LT_STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) gl_lds16(ga[i] + 128 * ks, buf + 1024 * (4 * wave + i));
#pragma unroll
      for (int i = 0; i < 2; ++i) gl_lds16(gb[i] + 64 * ks, buf + LT_OFF_B + 1024 * (2 * wave + i));
      gl_lds4(gs + 4 * ks, buf + LT_OFF_AS + 256 * wave);
    };

    __syncthreads();  // the previous segment's buffers are no longer read
    issue(0);
    if (ksteps > 1) issue(1);
    for (int ks = 0; ks < ksteps; ++ks) {
      if (ks + 1 < ksteps) wait_vmcnt<LT_LOADS>(); else wait_vmcnt<0>();
      barrier_lds();
      if (ks + 2 < ksteps) issue(ks + 2);
      const uint8_t* buf = lds + (ks % LT_NBUF) * LT_STAGE;
      v8i bf[NW][NB];
      int bsc[NW][NB];
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) {
          const int trow = SWI ? (h * NCOL + wn * 32 + 16 * ni + r16) : (wn * 64 + 16 * ni + r16);
          bf[ni][h] = as_v8i(*reinterpret_cast<const uint4*>(buf + LT_OFF_B + trow * 64 + ((g4 ^ ((trow >> 1) & 3)) << 4)));
          bsc[ni][h] = (int)(reinterpret_cast<const uint32_t*>(buf + LT_OFF_BS)[trow] >> (8 * g4));
        }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + 16 * mi + r16;
        Frag8 fa;
        fa.lo = *reinterpret_cast<const uint4*>(buf + r * 128 + ((g4 ^ (r & 7)) << 4));
        fa.hi = *reinterpret_cast<const uint4*>(buf + r * 128 + (((4 + g4) ^ (r & 7)) << 4));
        const v8i av = as_v8i(fa);
        const int sa = (int)(reinterpret_cast<const uint32_t*>(buf + LT_OFF_AS)[r] >> (8 * g4));
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
          for (int h = 0; h < NB; ++h) acc[mi][ni][h] = mfma_f8f4(av, bf[ni][h], acc[mi][ni][h], sa, bsc[ni][h]);
      }
    }
  }

  Tile t;
  t.g = g;
  t.m0 = m0 + wm * 64;
  t.rows = rows;
  t.row_base = row_base;
  t.n0 = col0 + wn * 16 * NW;
  epilogue<4, NW, NB, EPI>(p, t, acc, r16, g4);
}

// bf16 twin of the LDS-staged kernel for the dense latent down-projection
// (A = bf16 [M][K], B = bf16 [N][K], exact images of the MX operands).  Same
// 128 x 128 tile and 2 x 2 waves; a K-step is 64 elements (128 bytes per row
// for both operands), consumed as two 16x16x32 bf16 MFMAs per fragment pair
// (slice u takes chunk 4u + g of the row for lane group g, identically in A
// and B).  bf16 does half the MACs per staged byte of the MX path, so the ring
// has four 32 KB buffers (three K-steps in flight).
constexpr int LB_STAGE = LT_M * 128 + LT_B * 128;
constexpr int LB_NBUF = 4;
constexpr int LB_LOADS = 8;

template <int EPI>
__global__ void __launch_bounds__(256) bf16_gemm_lds_kernel(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NW = 4;
  static_assert(EPI != EPI_SWIGLU_QUANT, "dense projection only");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  int g, mt, nt, rows, row_base;
  if (!decode_lds_tile<LT_M>(p, LT_B, g, mt, nt, rows, row_base)) return;
  const int m0 = mt * LT_M;
  const int col0 = nt * LT_B;
  const GemmSeg& sg = p.seg[0];
  const int K = sg.K;
  const int ksteps = K >> 6;
  // load i (0..3) of this wave fills tile row 32*wave + 8*i + lane/8, physical chunk lane%8
  const uint8_t* ga[4];
  const uint8_t* gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    int ar = m0 + r;
    ar = ar < rows ? ar : rows - 1;
    int bc = col0 + r;
    bc = bc < p.N ? bc : p.N - 1;
    ga[i] = sg.a + ((int64_t)ar * K) * 2 + 16 * c;
    gb[i] = sg.b + (int64_t)g * sg.b_gstride + ((int64_t)bc * K) * 2 + 16 * c;
  }
  auto issue = [&](int ks) {
    uint8_t* buf = lds + (ks % LB_NBUF) * LB_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) gl_lds16(ga[i] + 128 * ks, buf + 1024 * (4 * wave + i));
#pragma unroll
    for (int i = 0; i < 4; ++i) gl_lds16(gb[i] + 128 * ks, buf + LT_M * 128 + 1024 * (4 * wave + i));
  };
  v4f acc[4][NW][1];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NW; ++ni) acc[mi][ni][0] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < LB_NBUF - 1 && j < ksteps; ++j) issue(j);
  for (int ks = 0; ks < ksteps; ++ks) {
    const int ahead = min(LB_NBUF - 2, ksteps - 1 - ks);  // K-steps still in flight after this one
    if (ahead >= 2) wait_vmcnt<2 * LB_LOADS>(); else if (ahead == 1) wait_vmcnt<LB_LOADS>(); else wait_vmcnt<0>();
    barrier_lds();
    if (ks + LB_NBUF - 1 < ksteps) issue(ks + LB_NBUF - 1);
    const uint8_t* buf = lds + (ks % LB_NBUF) * LB_STAGE;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 bfr[NW];
#pragma unroll
      for (int ni = 0; ni < NW; ++ni) {
        const int trow = wn * 64 + 16 * ni + r16;
        bfr[ni] = as_bf16x8(*reinterpret_cast<const uint4*>(buf + LT_M * 128 + trow * 128 +
                                                            (((4 * u + g4) ^ (trow & 7)) << 4)));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + 16 * mi + r16;
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(buf + r * 128 + (((4 * u + g4) ^ (r & 7)) << 4)));
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
          acc[mi][ni][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bfr[ni], acc[mi][ni][0], 0, 0, 0);
      }
    }
  }
  Tile t;
  t.g = g;
  t.m0 = m0 + wm * 64;
  t.rows = rows;
  t.row_base = row_base;
  t.n0 = col0 + wn * 64;
  epilogue<4, NW, 1, EPI>(p, t, acc, r16, g4);
}

template <int EPI>
static hipError_t launch_bf16_lds_cfg(const GemmArgs& a, hipStream_t s) {
  const int n_nt = (a.N + LT_B - 1) / LT_B;
  int64_t tiles = (int64_t)a.max_mtiles * n_nt;
  tiles = (tiles + 7) / 8 * 8;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  constexpr size_t smem = (size_t)LB_NBUF * LB_STAGE;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bf16_gemm_lds_kernel<EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  bf16_gemm_lds_kernel<EPI><<<dim3((unsigned)tiles), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_lds_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int NCOL = EPI == EPI_SWIGLU_QUANT ? LT_B / 2 : LT_B;
  const int n_nt = (a.N + NCOL - 1) / NCOL;
  int64_t tiles = (int64_t)a.max_mtiles * n_nt;
  tiles = (tiles + 7) / 8 * 8;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  constexpr size_t smem = (size_t)LT_NBUF * LT_STAGE;
  static bool attr_set = false;  // per-process, set before the first launch
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mx_gemm_lds_kernel<EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  mx_gemm_lds_kernel<EPI><<<dim3((unsigned)tiles), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

template <int MW, int NW, int EPI>
static hipError_t launch_stream_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int NT = 4 * 16 * NW;
  constexpr int NB = EPI == EPI_SWIGLU_QUANT ? 2 : 1;
  const int n_ntiles = (a.N + NT - 1) / NT;
  const int64_t grid = (int64_t)a.max_mtiles * n_ntiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  int kb = 0;
  for (int i = 0; i < a.nseg; ++i) kb = max(kb, a.seg[i].K >> 5);
  const size_t smem = (size_t)NB * NT * kb;
  if (smem > 65536) return hipErrorInvalidValue;
  mx_gemm_stream_kernel<MW, NW, EPI><<<dim3((unsigned)grid), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

template <int MW, int NW, int EPI>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int NT = 4 * 16 * NW;
  const int n_ntiles = (a.N + NT - 1) / NT;
  const int64_t grid = (int64_t)a.max_mtiles * n_ntiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  mx_gemm_kernel<MW, NW, EPI><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

int gemm_mtile(int shape) {
  return shape == GEMM_STREAM16 ? 16 : shape == GEMM_TILE128 ? LT_M : shape == GEMM_WIDE ? gemm_wide_mtile() : 64;
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

hipError_t launch_bf16_gemm_quant(const GemmArgs& a, int shape, hipStream_t s) {
  if (shape == GEMM_TILE128) return launch_bf16_lds_cfg<EPI_F32_QUANT>(a, s);
  return shape == GEMM_STREAM16 ? launch_bf16_cfg<1, 2, EPI_F32_QUANT>(a, s)
                                : launch_bf16_cfg<4, 2, EPI_F32_QUANT>(a, s);
}

hipError_t launch_mx_gemm(const GemmArgs& a, int epi, int shape, hipStream_t s) {
  if (shape == GEMM_WIDE) return launch_mx_gemm_wide(a, epi, s);
  if (shape == GEMM_STREAM16) {
    switch (epi) {
      case EPI_F32: return launch_stream_cfg<1, 2, EPI_F32>(a, s);
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
  if (shape == GEMM_TILE128) {
    switch (epi) {
      case EPI_F32: return launch_lds_cfg<EPI_F32>(a, s);
      case EPI_F32_QUANT: return launch_lds_cfg<EPI_F32_QUANT>(a, s);
      default: return launch_lds_cfg<EPI_SWIGLU_QUANT>(a, s);
    }
  }
  switch (epi) {
    case EPI_F32: return launch_cfg<4, 2, EPI_F32>(a, s);
    case EPI_F32_QUANT: return launch_cfg<4, 2, EPI_F32_QUANT>(a, s);
    default: return launch_cfg<4, 2, EPI_SWIGLU_QUANT>(a, s);
  }
}

}  // namespace moe
