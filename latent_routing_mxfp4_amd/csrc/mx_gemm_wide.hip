// mx_gemm_wide.hip -- grouped / dense MX GEMM for many rows per group
// (prefill): one 512-thread workgroup per CU owns a 128-row x 512-weight-row
// tile and streams both operands through a three-stage LDS ring.
//
// Why this shape on gfx950.  The expert weights are read from HBM once per
// (expert, N-tile) and the activations of an expert stay in L2 while its
// tiles run, so what bounds the loop is the number of bytes each CU keeps in
// flight (LDS capacity: 160 KB) against the latency of weight misses, and the
// L2 -> LDS traffic per MFMA.  A 128 x 512 tile moves 48 KB of codes per
// 128-deep K-step for 16.8 MFLOP -- half the bytes per flop of a 128 x 128
// tile -- and a 3 x 50.5 KB ring keeps two K-steps (64 KB of weights) in
// flight per CU.  Eight waves (two per SIMD) compute 64 x 128 each; every
// wave reads 16 KB of LDS per 32 MFMAs (about 63 B/clk/CU at the MFMA rate,
// plus 25 B/clk of staging writes, inside the ~117 B/clk LDS read rate).
//
// Ping-pong.  A K-step is a read half (LDS -> registers, then the next loads)
// and an MFMA half, each opened by a workgroup barrier, and the two waves of
// a SIMD (one from each M-half of the tile) run half a step apart: while one
// issues its 32 MFMAs the other reads its fragments, so the matrix core of
// the SIMD is fed across every barrier instead of idling while both waves
// wait for the barrier and then for LDS.
//
// Loads are direct global -> LDS (inline assembly, waits placed by hand; see
// lds_pipe.hpp): per K-step each wave issues 2 A-code, 4 B-code, one A-scale
// (16 lanes) and one B-scale load, and the stage for step ks+2 is issued at
// the end of the read half of step ks.
//
// The weights are stored in fragment order (kernels.hpp): one 16 x 128 block
// of codes is 1 KB contiguous in MFMA lane order, so each B load instruction
// moves one whole block (eight full cache lines) and a lane later reads its
// operand at 16 * lane, with no bank conflicts and no swizzle; a K-step's
// scale dwords of consecutive weight rows are contiguous too.  The A tile is
// gathered by row (activations), 128 bytes per row and K-step, with its
// 16-byte chunks XOR-swizzled by row in LDS.  The A scales are permuted so
// that a lane reads its four A fragments' scale dwords with one 16-byte read.
// The MFMA takes the scale from bits [7:0], so each dword is shifted right by
// 8 * (lane / 16).
//
// Column mapping.  SwiGLU: the tile's 512 weight rows are 256 gate rows and
// the 256 matching up rows (h columns col0 .. col0+255); wave (wm, wn) owns h
// columns col0 + 64 wn .. +63 (fragments 0..3 gate, 4..7 up).  Otherwise the
// tile is 512 output columns and wave wn owns col0 + 128 wn .. +127.
#include <type_traits>

#include "combine_device.hpp"
#include "gemm_epilogue.hpp"
#include "kernels.hpp"
#include "launch_attr.hpp"
#include "lds_pipe.hpp"
#include "mx_device.hpp"

namespace moe {

namespace {

constexpr int WD_M = 128;                        // rows per M-tile
constexpr int WD_B = 512;                        // weight rows per tile
constexpr int WD_OFF_B = WD_M * 128;             // A codes: 128 rows x 128 bytes
constexpr int WD_OFF_AS = WD_OFF_B + WD_B * 64;  // B codes: 512 rows x 64 bytes
constexpr int WD_OFF_BS = WD_OFF_AS + 4 * 512;   // A scales: 128 dwords in 512 slots
constexpr int WD_STAGE = WD_OFF_BS + 4 * WD_B;   // B scales: 512 dwords -> 53248 bytes
constexpr int WD_NBUF = 3;
constexpr int WD_LOADS = 8;  // direct loads per wave per K-step

template <int EPI>
__device__ __forceinline__ void wide_mx_tile(const GemmArgs& p, int bid) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT;
  constexpr int NB = SWI ? 2 : 1;              // accumulators per fragment (gate, up)
  constexpr int NW = SWI ? 4 : 8;              // output fragments per wave
  constexpr int NCOL = SWI ? WD_B / 2 : WD_B;  // output columns per tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;

  const bool routed = p.offsets != nullptr;
  int g, mt, nt, rows, row_base;
  if (!decode_lds_tile<WD_M>(p, bid, NCOL, g, mt, nt, rows, row_base)) return;
  const int m0 = mt * WD_M;
  const int col0 = nt * NCOL;
  // 16-row fragments of this wave that hold at least one row of the group
  // (the last M-tile of a group is usually partly past its rows).
  int mvalid = (rows - m0 - 64 * wm + 15) >> 4;
  mvalid = __builtin_amdgcn_readfirstlane(mvalid < 0 ? 0 : (mvalid > 4 ? 4 : mvalid));

  auto a_src_row = [&](int trow) -> int64_t {
    int r = m0 + trow;
    r = r < rows ? r : rows - 1;
    const int sr = row_base + r;
    return routed ? (p.gather ? (int64_t)(p.gather[sr] / p.gather_div) : (int64_t)sr) : (int64_t)r;
  };
  // Tile B row -> (matrix, output column), clamped into [0, N); for the first
  // row of a 16-row block the clamp keeps the whole block inside (N % 16 == 0).
  auto b_col = [&](int brow, int& up, int last) -> int {
    int c;
    if (SWI) {
      up = brow >= NCOL;
      c = col0 + (brow & (NCOL - 1));
    } else {
      up = 0;
      c = col0 + brow;
    }
    return c < last ? c : last;
  };
  // Tile B row of fragment ni (0..7) of wave column wc, lane row r.
  auto b_row = [&](int wc, int ni, int r) -> int {
    if (SWI) return (ni < 4 ? 0 : NCOL) + 64 * wc + 16 * (ni & 3) + r;
    return 128 * wc + 16 * ni + r;
  };

  // A codes: load i (0..1) of wave w fills LDS [1024*(2w+i), +1024): tile row
  // 8*(2w+i) + lane/8, physical chunk lane%8 (logical chunk XOR row%8).
  int64_t a_row[2];
  int a_chunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (2 * wave + i) + (lane >> 3);
    a_row[i] = a_src_row(r);
    a_chunk[i] = (lane & 7) ^ (r & 7);
  }
  // B codes: load i (0..3) of wave w copies the fragment-order block of tile
  // B rows 16*(4w+i) .. +15 into [OFF_B + 1024*(4w+i), +1024).
  // A scales: value d (0..127) = tile row 64*(d/64) + 16*(d%4) + (d/4)%16 is
  // loaded by lane d%16 of wave d/16 into slot 64*(d/16) + d%16 (lanes 16..63
  // load copies into the other slots, so the load needs no lane mask), and
  // lane (r16, g4) of M-half wm finds its rows 64wm + 16mi + r16 (mi = 0..3),
  // values 64wm + 4r16 .. +3, in four consecutive slots.
  const int as_d = 16 * wave + (lane & 15);
  const int64_t as_row = a_src_row(64 * (as_d >> 6) + 16 * (as_d & 3) + ((as_d >> 2) & 15));
  // B scales: dword tr of the stage holds tile B row tr; wave w loads rows
  // 64w .. 64w+63 (contiguous in memory for one K-step).

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
    const uint8_t* ga[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) ga[i] = sg.a + a_row[i] * sg.lda + 16 * a_chunk[i];
    // Weight source addresses.  Fragment order: the block of 16 rows x 128
    // elements is 1 KB contiguous and lane l takes bytes 16 l; row-major: lane
    // l = r + 16 q takes bytes 16 q of row r's 64 bytes for the K-step.  Either
    // way the LDS stage receives the block in fragment order.
    const bool brm = sg.b_rm != 0;
    const uint8_t* gb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int up;
      const int c = b_col(16 * (4 * wave + i), up, p.N - 16);  // first row of the block
      const uint8_t* base = (up ? sg.b2 : sg.b) + (int64_t)g * sg.b_gstride;
      gb[i] = brm ? base + (int64_t)(c + (lane & 15)) * (K >> 1) + 16 * (lane >> 4)
                  : base + (int64_t)(c >> 4) * ksteps * 1024 + 16 * lane;
    }
    const int64_t b_kstride = brm ? 64 : 1024;  // bytes between K-steps of a lane's weight codes
    const uint8_t* gas = sg.as + as_row * (sg.lda >> 5);
    const uint8_t* gbs;
    {
      int up;
      const int c = b_col(64 * wave + lane, up, p.N - 1);
      const uint8_t* base = (up ? sg.b2s : sg.bs) + (int64_t)g * sg.bs_gstride;
      gbs = brm ? base + (int64_t)c * kb : base + 4 * (int64_t)c;
    }
    const int64_t bs_kstride = brm ? 4 : 4 * (int64_t)p.N;  // bytes between K-steps of the B scales
    // A stage's loads of one wave, in four parts: 2 A-code; 2 B-code; 2
    // B-code; A-scale and B-scale.
    auto issue_part = [&](int ks, int part) {
      uint8_t* buf = lds + (ks % WD_NBUF) * WD_STAGE;
      if (part == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) gl_lds16(ga[i] + 128 * ks, buf + 1024 * (2 * wave + i));
      } else if (part < 3) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int i = 2 * (part - 1) + j;
          gl_lds16(gb[i] + b_kstride * ks, buf + WD_OFF_B + 1024 * (4 * wave + i));
        }
      } else {
        gl_lds4(gas + 4 * ks, buf + WD_OFF_AS + 256 * wave);
        gl_lds4(gbs + bs_kstride * ks, buf + WD_OFF_BS + 256 * wave);
      }
    };
    auto issue = [&](int ks) {
#pragma unroll
      for (int part = 0; part < 4; ++part) issue_part(ks, part);
    };
    auto rd_a = [&](const uint8_t* buf, int mi) -> v8i {
      const int r = 64 * wm + 16 * mi + r16;
      const uint4 lo = *reinterpret_cast<const uint4*>(buf + r * 128 + ((g4 ^ (r & 7)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(buf + r * 128 + (((4 + g4) ^ (r & 7)) << 4));
      v8i av;
      av[0] = (int)lo.x; av[1] = (int)lo.y; av[2] = (int)lo.z; av[3] = (int)lo.w;
      av[4] = (int)hi.x; av[5] = (int)hi.y; av[6] = (int)hi.z; av[7] = (int)hi.w;
      return av;
    };

    // One K-step in two halves, each opened by a barrier: a read half (the
    // step's scales and all A and B fragments from LDS into registers, then
    // the loads of the stage two steps ahead) and an MFMA half.  The tile's
    // two M-halves (waves 0-3 and 4-7: one wave of each per SIMD) run half a
    // step apart -- the second half passes one extra barrier before its first
    // step, the first half one after its last -- so on every SIMD one wave
    // issues MFMAs while the other reads LDS, and the barriers no longer stop
    // both waves of a SIMD at once.
    // Hazards.  Stage ks is complete in every wave before the barrier that
    // opens the first half's read of step ks: the first half waits for its
    // loads at the top of the step, the second half at the end of its read
    // half of step ks - 1 (or before its extra barrier, for stage 0).  The
    // loads of stage ks + 2 overwrite the buffer of step ks - 1; both halves
    // have finished reading it by then, because barrier_lds drains a wave's
    // LDS reads before it arrives.
    const bool late = wm == 1;
    auto step = [&](int ks) {
      if (!late) {
        if (ks + 1 < ksteps) wait_vmcnt<WD_LOADS>(); else wait_vmcnt<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* buf = lds + (ks % WD_NBUF) * WD_STAGE;
      const int sh = 8 * g4;
      uint32_t as_all[4] = {0u, 0u, 0u, 0u};
      uint32_t bs_all[8];
      v8i bf[8];
      v8i av[4];
      // A wave with no row of the group (the second M-half of a tail tile of
      // at most 64 rows) issues no MFMAs, so it reads no fragments either:
      // LDS data returning into one wave's registers stalls the matrix core
      // for the other wave of its SIMD too.
      if (mvalid > 0) {
        const uint4 asd =
            *reinterpret_cast<const uint4*>(buf + WD_OFF_AS + 1024 * wm + 256 * (r16 >> 2) + 16 * (r16 & 3));
        as_all[0] = asd.x; as_all[1] = asd.y; as_all[2] = asd.z; as_all[3] = asd.w;
#pragma unroll
        for (int ni = 0; ni < 8; ++ni)
          bs_all[ni] = *reinterpret_cast<const uint32_t*>(buf + WD_OFF_BS + 4 * b_row(wn, ni, r16));
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) {
          const int blk = b_row(wn, ni, 0) >> 4;
          const uint4 v = *reinterpret_cast<const uint4*>(buf + WD_OFF_B + 1024 * blk + 16 * lane);
          bf[ni][0] = (int)v.x; bf[ni][1] = (int)v.y; bf[ni][2] = (int)v.z; bf[ni][3] = (int)v.w;
          bf[ni][4] = 0; bf[ni][5] = 0; bf[ni][6] = 0; bf[ni][7] = 0;
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) av[mi] = rd_a(buf, mi);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 2 < ksteps) issue(ks + 2);
      if (late) {  // stage ks + 1, leaving stage ks + 2 in flight
        if (ks + 2 < ksteps) wait_vmcnt<WD_LOADS>(); else wait_vmcnt<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int sa = (int)(as_all[mi] >> sh);
        if (mi < mvalid) {  // fragments wholly past the group's last row are skipped
#pragma unroll
          for (int ni = 0; ni < 8; ++ni) {
            const int sb = (int)(bs_all[ni] >> sh);
            if (SWI) acc[mi][ni & 3][ni >> 2] = mfma_f8f4(av[mi], bf[ni], acc[mi][ni & 3][ni >> 2], sa, sb);
            else acc[mi][ni][0] = mfma_f8f4(av[mi], bf[ni], acc[mi][ni][0], sa, sb);
          }
        }
      }
    };

    // Every wave passes 2 * ksteps + 2 barriers per segment (the segment's
    // first, two per step, and its half's extra one), so the counts match.
    __syncthreads();  // the previous segment's stages are no longer read
    issue(0);
    if (ksteps > 1) issue(1);
    if (late) {
      if (ksteps > 1) wait_vmcnt<WD_LOADS>(); else wait_vmcnt<0>();
      barrier_lds();
    }
    for (int ks = 0; ks < ksteps; ++ks) step(ks);
    if (!late) barrier_lds();
  }

  Tile t;
  t.g = g;
  t.m0 = m0 + 64 * wm;
  t.rows = rows;
  t.row_base = row_base;
  t.n0 = SWI ? col0 + 64 * wn : col0 + 128 * wn;
  epilogue<4, NW, NB, EPI>(p, t, acc, r16, g4);
}

template <int EPI>
__global__ void __launch_bounds__(512) mx_gemm_wide_kernel(const GemmArgs p) {
  wide_mx_tile<EPI>(p, blockIdx.x);
}

// Prefill: the combine (HBM-bound) beside the shared experts' gate/up GEMM
// (matrix-core bound), which it does not depend on, in one launch.  Groups of
// 8 consecutive workgroups (one per XCD) are "slots"; every R-th slot is a
// combine slot whose 8 workgroups each combine `chunk` tokens, the others
// run the GEMM's tiles in their own order (GEMM slot = slot - slot / R), so
// a few CUs at a time stream the expert outputs while the rest keep the
// matrix cores busy.  The combine's arithmetic is the combine kernel's.
__device__ __forceinline__ void combine_chunk(const CombineArgs& c, int chunk, int ci) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int64_t t0 = (int64_t)ci * chunk;
  if (t0 >= c.T) return;  // uniform over the workgroup
  const int nt = (int)min((int64_t)chunk, (int64_t)c.T - t0);
  int32_t* rows = reinterpret_cast<int32_t*>(lds);
  float* gs = reinterpret_cast<float*>(lds) + chunk * c.k;
  for (int i = threadIdx.x; i < nt * c.k; i += blockDim.x) {
    rows[i] = c.row_of_pair[t0 * c.k + i];
    gs[i] = c.gates[t0 * c.k + i];
  }
  __syncthreads();
  // Two (token, feature-quad) items per thread at a time, so 2k row loads are
  // in flight per thread (the combine kernel's arithmetic for each item).
  const int n4 = c.L >> 2;  // a multiple of 8, and so is n4 * nt: MX blocks stay whole
  const int items = nt * n4;
  const int bs = blockDim.x;
  for (int it = threadIdx.x; it < items; it += 2 * bs) {
    const int ib = it + bs;
    const bool two = ib < items;  // the same for the 8 lanes of an MX block
    const int ta = it / n4, fa = it - ta * n4;
    const int tb = two ? ib / n4 : ta, fb = two ? ib - tb * n4 : fa;
    float4 acc_a = make_float4(0.f, 0.f, 0.f, 0.f), acc_b = acc_a;
    for (int j0 = 0; j0 < c.k; j0 += 16) {
      combine_rows16(c.y_e, rows + ta * c.k, gs + ta * c.k, c.k, c.L, j0, fa, acc_a);
      combine_rows16(c.y_e, rows + tb * c.k, gs + tb * c.k, c.k, c.L, j0, fb, acc_b);
    }
    combine_store(acc_a, c.L, t0 + ta, fa, c.y_lat, c.yq, c.yqs, nullptr);
    if (two) combine_store(acc_b, c.L, t0 + tb, fb, c.y_lat, c.yq, c.yqs, nullptr);
  }
}

template <int EPI>
__global__ void __launch_bounds__(512) mx_gemm_wide_combine_kernel(const GemmArgs p, const CombineArgs c,
                                                                   int chunk, int R) {
  const int slot = blockIdx.x >> 3, x = blockIdx.x & 7;
  if (slot % R == R - 1) combine_chunk(c, chunk, 8 * (slot / R) + x);
  else wide_mx_tile<EPI>(p, 8 * (slot - slot / R) + x);
}

// Dense bf16 GEMM: the latent down-projection on exact bf16 images of the MX
// operands (the reason it runs on bf16 matrix cores is in mx_gemm.hip), and
// the bfloat16 latent projections and shared experts of the higher-precision
// map.  Same 512-thread, one-workgroup-per-CU structure as the MX kernel: a
// 128 x 256 tile, waves 2 x 4 of 64 x 64, K-steps of 64 elements (128 bytes
// per row of either operand) staged by direct loads in a ring of three 48 KB
// buffers; each K-step is two 16x16x32 bf16 MFMAs per fragment pair, slice u
// taking 16-byte chunk 4u + g of a row for lane group g, identically in A and
// B.  Rows are XOR-swizzled by chunk.  K segments (e.g. the up-projection and
// the shared down-projections) run one after the other into the same
// accumulators.  SwiGLU: B tile row r holds column (r / 64) * 32 + r % 32 of
// the gate (r / 32 even) or up (odd) matrix, so a wave's fragments 0-1 and 2-3
// are the gate and up values of the same 32 columns.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int WB_M = 128, WB_N = 256;
constexpr int WB_OFF_B = WB_M * 128;
constexpr int WB_STAGE = WB_OFF_B + WB_N * 128;  // 49152 bytes
constexpr int WB_NBUF = 3;
constexpr int WB_LOADS = 6;  // 2 A + 4 B direct loads per wave per K-step

__device__ __forceinline__ bf16x8_t as_bf16x8_w(const uint4& f) {
  union {
    uint4 u;
    bf16x8_t b;
  } c;
  c.u = f;
  return c.b;
}

template <int EPI>
__global__ void __launch_bounds__(512) bf16_gemm_wide_kernel(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  static_assert(EPI != EPI_SWIGLU_QUANT, "bf16 kernels write the SwiGLU hidden state as bf16");
  constexpr bool SWI = EPI == EPI_SWIGLU_BF16;
  constexpr int NCOL = SWI ? WB_N / 2 : WB_N;  // output columns per tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;
  int g, mt, nt, rows, row_base;
  if (!decode_lds_tile<WB_M>(p, blockIdx.x, NCOL, g, mt, nt, rows, row_base)) return;
  const int m0 = mt * WB_M;
  const int col0 = nt * NCOL;
  v4f acc[4][4][1];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni][0] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int si = 0; si < p.nseg; ++si) {
    const GemmSeg& sg = p.seg[si];
    const int K = sg.K;
    const int ksteps = K >> 6;
    // A load i (0..1) of wave w: tile row 8*(2w+i) + lane/8; B load i (0..3):
    // tile B row 8*(4w+i) + lane/8; physical chunk lane%8 (logical XOR row%8).
    const uint8_t* ga[2];
    const uint8_t* gb[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * (2 * wave + i) + (lane >> 3);
      int ar = m0 + r;
      ar = ar < rows ? ar : rows - 1;
      ga[i] = sg.a + ((int64_t)ar * K) * 2 + 16 * ((lane & 7) ^ (r & 7));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * (4 * wave + i) + (lane >> 3);
      int bc = SWI ? col0 + (r >> 6) * 32 + (r & 31) : col0 + r;
      bc = bc < p.N ? bc : p.N - 1;
      const uint8_t* base = SWI && ((r >> 5) & 1) ? sg.b2 : sg.b;
      gb[i] = base + (int64_t)g * sg.b_gstride + ((int64_t)bc * K) * 2 + 16 * ((lane & 7) ^ (r & 7));
    }
    auto issue = [&](int ks) {
      uint8_t* buf = lds + (ks % WB_NBUF) * WB_STAGE;
#pragma unroll
      for (int i = 0; i < 2; ++i) gl_lds16(ga[i] + 128 * ks, buf + 1024 * (2 * wave + i));
#pragma unroll
      for (int i = 0; i < 4; ++i) gl_lds16(gb[i] + 128 * ks, buf + WB_OFF_B + 1024 * (4 * wave + i));
    };
    // Ping-pong as in the MX kernel: each K-step is a read half (all of the
    // step's fragments into registers, then the loads two steps ahead) and
    // an MFMA half, the tile's two M-halves half a step apart (the second
    // half passes an extra barrier before its first step, the first half one
    // after its last).  A new segment refills buffers the previous one's
    // last K-steps were read from, so every wave passes a barrier first.
    const bool late = wm == 1;
    if (si > 0) barrier_lds();
    issue(0);
    if (ksteps > 1) issue(1);
    if (late) {
      if (ksteps > 1) wait_vmcnt<WB_LOADS>(); else wait_vmcnt<0>();
      barrier_lds();
    }
    for (int ks = 0; ks < ksteps; ++ks) {
      if (!late) {
        if (ks + 1 < ksteps) wait_vmcnt<WB_LOADS>(); else wait_vmcnt<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* buf = lds + (ks % WB_NBUF) * WB_STAGE;
      bf16x8_t bfr[2][4], afr[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int trow = wn * 64 + 16 * ni + r16;
          bfr[u][ni] = as_bf16x8_w(*reinterpret_cast<const uint4*>(buf + WB_OFF_B + trow * 128 +
                                                                  (((4 * u + g4) ^ (trow & 7)) << 4)));
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int r = wm * 64 + 16 * mi + r16;
          afr[u][mi] = as_bf16x8_w(*reinterpret_cast<const uint4*>(buf + r * 128 + (((4 * u + g4) ^ (r & 7)) << 4)));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 2 < ksteps) issue(ks + 2);
      if (late) {  // stage ks + 1, leaving stage ks + 2 in flight
        if (ks + 2 < ksteps) wait_vmcnt<WB_LOADS>(); else wait_vmcnt<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[u][mi], bfr[u][ni], acc[mi][ni][0], 0, 0, 0);
    }
    if (!late) barrier_lds();
  }
  Tile t;
  t.g = g;
  t.m0 = m0 + wm * 64;
  t.rows = rows;
  t.row_base = row_base;
  if (SWI) {
    v4f pr[4][2][2];  // [mi][fragment][gate, up]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        pr[mi][ni][0] = acc[mi][ni][0];
        pr[mi][ni][1] = acc[mi][2 + ni][0];
      }
    t.n0 = col0 + wn * 32;
    epilogue<4, 2, 2, EPI>(p, t, pr, r16, g4);
  } else {
    t.n0 = col0 + wn * 64;
    epilogue<4, 4, 1, EPI>(p, t, acc, r16, g4);
  }
}

template <int EPI>
hipError_t launch_wide_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int NCOL = EPI == EPI_SWIGLU_QUANT ? WD_B / 2 : WD_B;
  if (a.N % 16 != 0) return hipErrorInvalidValue;  // fragment-order weights
  const int n_nt = (a.N + NCOL - 1) / NCOL;
  int64_t tiles = (int64_t)a.max_mtiles * n_nt;
  tiles = (tiles + 7) / 8 * 8;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  constexpr size_t smem = (size_t)WD_NBUF * WD_STAGE;
  static DeviceOnce attr;
  hipError_t e = lds_limit_once(attr, {reinterpret_cast<const void*>(&mx_gemm_wide_kernel<EPI>)}, (int)smem);
  if (e != hipSuccess) return e;
  mx_gemm_wide_kernel<EPI><<<dim3((unsigned)tiles), dim3(512), smem, s>>>(a);
  return hipGetLastError();
}

// Combine chunks of 32 tokens (7.3 MB of expert outputs at K3 width); one
// combine slot per R slots, R from the two counts so that both kinds of
// work are spread over the whole launch.
constexpr int kCombineChunk = 32;

hipError_t launch_wide_combine(const GemmArgs& a, const CombineArgs& c, hipStream_t s) {
  constexpr int EPI = EPI_SWIGLU_QUANT;
  constexpr int NCOL = WD_B / 2;
  if (a.N % 16 != 0 || a.offsets != nullptr) return hipErrorInvalidValue;  // a dense GEMM
  if (c.T <= 0 || c.k < 1 || c.k > 64 || c.L <= 0 || c.L % 32 != 0 || !c.y_e || !c.gates || !c.row_of_pair ||
      !c.yq || !c.yqs)
    return hipErrorInvalidValue;
  const int n_nt = (a.N + NCOL - 1) / NCOL;
  const int64_t tiles = (int64_t)a.max_mtiles * n_nt;
  const int64_t gemm_slots = (tiles + 7) / 8;
  const int64_t comb_slots = ((c.T + kCombineChunk - 1) / kCombineChunk + 7) / 8;
  if (gemm_slots <= 0) return hipErrorInvalidValue;
  int64_t R = (gemm_slots + comb_slots) / comb_slots;
  R = R < 2 ? 2 : R;  // (at least every other slot a GEMM slot, so the loop below ends)
  int64_t S = gemm_slots + comb_slots;
  while (S - S / R < gemm_slots || S / R < comb_slots) ++S;
  if (8 * S > 0x7fffffff) return hipErrorInvalidValue;
  constexpr size_t smem = (size_t)WD_NBUF * WD_STAGE;  // (the combine uses 2 * 32 * k * 4 bytes of it)
  static DeviceOnce attr;
  hipError_t e =
      lds_limit_once(attr, {reinterpret_cast<const void*>(&mx_gemm_wide_combine_kernel<EPI>)}, (int)smem);
  if (e != hipSuccess) return e;
  mx_gemm_wide_combine_kernel<EPI><<<dim3((unsigned)(8 * S)), dim3(512), smem, s>>>(a, c, kCombineChunk, (int)R);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_bf16_wide_cfg(const GemmArgs& a, hipStream_t s) {
  if (a.nseg < 1 || a.nseg > 9 || a.offsets != nullptr) return hipErrorInvalidValue;
  for (int i = 0; i < a.nseg; ++i) {
    if (a.seg[i].K <= 0 || a.seg[i].K % 64 != 0 || !a.seg[i].a || !a.seg[i].b) return hipErrorInvalidValue;
    if (EPI == EPI_SWIGLU_BF16 && !a.seg[i].b2) return hipErrorInvalidValue;
  }
  if (EPI == EPI_SWIGLU_BF16 && (a.N % 32 != 0 || !a.ob)) return hipErrorInvalidValue;
  constexpr int NCOL = EPI == EPI_SWIGLU_BF16 ? WB_N / 2 : WB_N;
  const int n_nt = (a.N + NCOL - 1) / NCOL;
  int64_t tiles = (int64_t)a.max_mtiles * n_nt;
  tiles = (tiles + 7) / 8 * 8;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  constexpr size_t smem = (size_t)WB_NBUF * WB_STAGE;
  static DeviceOnce attr;
  hipError_t e = lds_limit_once(attr, {reinterpret_cast<const void*>(&bf16_gemm_wide_kernel<EPI>)}, (int)smem);
  if (e != hipSuccess) return e;
  bf16_gemm_wide_kernel<EPI><<<dim3((unsigned)tiles), dim3(512), smem, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int gemm_wide_mtile() { return WD_M; }

hipError_t launch_bf16_gemm_wide(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return launch_bf16_wide_cfg<EPI_F32>(a, s);
    case EPI_F32_QUANT: return launch_bf16_wide_cfg<EPI_F32_QUANT>(a, s);
    case EPI_SWIGLU_BF16: return launch_bf16_wide_cfg<EPI_SWIGLU_BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mx_gemm_wide_combine(const GemmArgs& a, const CombineArgs& c, hipStream_t s) {
  if (a.N <= 0 || a.N >= (1 << 22) || a.ldc < 0 || a.ldc >= (1 << 22)) return hipErrorInvalidValue;
  return launch_wide_combine(a, c, s);
}

hipError_t launch_mx_gemm_wide(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return launch_wide_cfg<EPI_F32>(a, s);
    case EPI_F32_QUANT: return launch_wide_cfg<EPI_F32_QUANT>(a, s);
    default: return launch_wide_cfg<EPI_SWIGLU_QUANT>(a, s);
  }
}

}  // namespace moe
