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
// and the few-row latent down-projection, a bf16 GEMM that decodes the MXFP4
// weights in registers (its prefill twin is in mx_gemm_wide.hip).  The
// prefill-shaped MX GEMM is in mx_gemm_wide.hip and the epilogues shared by
// all of them in gemm_epilogue.hpp.  MX weights are read in fragment order
// (kernels.hpp), except W_down, which the bf16 paths read row-major.
#include "kernels.hpp"
#include "launch_attr.hpp"
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

// Map workgroup `bid` to (group, M-tile, N-tile).  Returns false for workgroups
// past the last M-tile (the grid is sized for the worst case).  The fields
// are computed in locals and stored once, so the tile stays in registers
// (filling them branch by branch through the reference left the tile in
// per-lane scratch memory).
template <int MT, int NT>
__device__ __forceinline__ bool decode_tile(const GemmArgs& p, int bid, int wave, int NWC, Tile& t) {
  const int n_ntiles = (p.N + NT - 1) / NT;
  int g, m0, rows, row_base, nt;
  if (p.offsets) {
    const int gm = bid / n_ntiles;
    nt = bid - gm * n_ntiles;
    const int total = p.mtile_start[p.G];
    if (gm >= total) return false;
    int lo = 0;
    if (p.mtile_group) {  // the dispatch's table: one load instead of a chain of ten
      lo = p.mtile_group[gm];
    } else {
      int hi = p.G;  // mtile_start[lo] <= gm < mtile_start[hi]
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (p.mtile_start[mid] <= gm) lo = mid; else hi = mid;
      }
    }
    g = lo;
    row_base = p.offsets[lo];
    rows = p.offsets[lo + 1] - row_base;
    m0 = (gm - p.mtile_start[lo]) * MT;
  } else {
    // Dense: workgroups are dealt to the 8 XCDs in turn (bid % 8); each XCD
    // takes a contiguous run of tiles, M-tiles of one N-tile adjacent, so the
    // M-tiles that share a weight tile run together on one XCD and its L2
    // serves the weights to all of them.  The grid is 8 * ceil(tiles / 8).
    const int mpg = (p.M + MT - 1) / MT;
    const int total = p.G * mpg * n_ntiles;
    const int per = (total + 7) >> 3;
    const int slot = bid >> 3;
    if (slot >= per) return false;
    const int lin = (bid & 7) * per + slot;
    if (lin >= total) return false;
    const int gn = lin / mpg;  // group * n_ntiles + N-tile
    g = gn / n_ntiles;
    nt = gn - g * n_ntiles;
    m0 = (lin - gn * mpg) * MT;
    rows = p.M;
    row_base = 0;
  }
  t = Tile{g, m0, rows, row_base, nt * NT + wave * NWC};
  return true;
}

// Exact bf16 image of one MX E2M1 block (32 elements, 16 bytes, scale code
// sc): dword h of output u holds elements 8u + 2h (low half) and 8u + 2h + 1
// (high half), element 2i being the low nibble of byte i.  For scale codes
// 2..252 the bf16 of magnitude code m in 1..7 is (sc << 7) + 64 (m - 2), less
// another 64 for m = 1 (0.5 has no mantissa bit); other scale codes (subnormal
// or overflowing results, never produced by the weight encoder for finite
// weights of useful size) take the general path through fp32.
__device__ __forceinline__ uint32_t e2m1_bf16_fast(uint32_t c, int sc) {
  const uint32_t m = c & 7u;
  uint32_t v = (uint32_t)(sc << 7) + 64u * m - 128u - (m == 1u ? 64u : 0u);
  v = m == 0u ? 0u : v;
  return v | ((c & 8u) << 12);
}
__device__ __forceinline__ uint32_t e2m1_bf16_slow(uint32_t c, int sc) {
  const int E = (c >> 1) & 3, m = c & 1;
  const float v = ldexpf((float)(E ? 2 + m : m), (E ? E - 2 : -1) + sc - 127);
  return __float_as_uint((c & 0x8) ? -v : v) >> 16;
}
struct Bf16Block {
  uint4 u[4];
};
// The general path for a whole block, out of line: inlined at every unrolled
// K-step it multiplied the kernel's code several times over (tens of KB of
// branches that never run), which then missed the instruction cache.
__device__ __noinline__ Bf16Block e2m1_block_bf16_general(uint4 codes, int sc) {
  Bf16Block r;
  const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t* o = &r.u[u].x;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo = (w[u] >> (8 * h)) & 0xf, hi = (w[u] >> (8 * h + 4)) & 0xf;
      o[h] = e2m1_bf16_slow(lo, sc) | (e2m1_bf16_slow(hi, sc) << 16);
    }
  }
  return r;
}
__device__ __forceinline__ void e2m1_block_bf16(const uint4& codes, int sc, uint4 (&out)[4]) {
  if (sc < 2 || sc > 252) {  // never for the weight encoder's blocks of useful size
    const Bf16Block r = e2m1_block_bf16_general(codes, sc);
#pragma unroll
    for (int u = 0; u < 4; ++u) out[u] = r.u[u];
    return;
  }
  // The block's eight magnitudes as two byte tables (low and high bytes of
  // the bf16 patterns, entry m = byte m, m = 0 giving 0), then per code byte
  // two byte permutes: each pair of elements costs a handful of instructions
  // instead of the formula per element.
  uint32_t B[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) B[m] = m == 0 ? 0u : e2m1_bf16_fast((uint32_t)m, sc);
  const uint32_t Llo = (B[0] & 0xffu) | ((B[1] & 0xffu) << 8) | ((B[2] & 0xffu) << 16) | ((B[3] & 0xffu) << 24);
  const uint32_t Lhi = (B[4] & 0xffu) | ((B[5] & 0xffu) << 8) | ((B[6] & 0xffu) << 16) | ((B[7] & 0xffu) << 24);
  const uint32_t Hlo = (B[0] >> 8) | ((B[1] >> 8) << 8) | ((B[2] >> 8) << 16) | ((B[3] >> 8) << 24);
  const uint32_t Hhi = (B[4] >> 8) | ((B[5] >> 8) << 8) | ((B[6] >> 8) << 16) | ((B[7] >> 8) << 24);
  const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t* o = &out[u].x;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t b = (w[u] >> (8 * h)) & 0xffu;  // elements 8u + 2h (low nibble) and 8u + 2h + 1
      // selector bytes: magnitude of the low element in byte 0, of the high
      // one in byte 2 (bytes 1 and 3 select entry 0, which is 0); the same
      // shifted up a byte places the high-byte table's entries
      const uint32_t sel = (b & 7u) | ((b & 0x70u) << 12);
      const uint32_t lo = __builtin_amdgcn_perm(Lhi, Llo, sel);
      const uint32_t hi = __builtin_amdgcn_perm(Hhi, Hlo, sel << 8);
      o[h] = lo | hi | ((b & 8u) << 12) | ((b & 0x80u) << 24);  // the two sign bits
    }
  }
}

// Few-row dense bf16 GEMMs with K split into slices (decode sizes): the latent
// down-projection straight from MXFP4 weights, and the bfloat16 projections
// and shared experts of the higher-precision map.  A = bf16 [M][K] (seg.a);
// B row-major [N][K], either MXFP4 (seg.b codes [N][K/2], seg.bs scales
// [N][K/32]) decoded to its exact bf16 image in registers, so the weights are
// read once at 17/32 bytes per element and no bf16 copy is written, or bf16
// read as is.  Why bf16 matrix cores for the MXFP8 x MXFP4 down-projection:
// every product of an E4M3 and an E2M1 value (power-of-two scales) is exact in
// bf16 x bf16 -> fp32 and v_mfma_f32_16x16x32_bf16 accumulates at fp32
// precision, unlike the block-scaled MFMA, which sums each 32-element block in
// a window of about 14 bits below its largest product; the router's top-k is
// decided on this latent.
//
// Slice blockIdx.y covers K-steps [ks0, ks0 + nks) (128 K values each) of one
// segment and writes its fp32 partial sums to part[slice][g][M][N]; the
// reduce kernels add the slices in slice order.  A workgroup (4 waves) owns
// MT = 16 MW rows and 4 x 16 NW columns.  The activation tile of a K-step
// (MT x 256 bytes, shared by the 4 waves) is staged in LDS by direct loads;
// each wave streams only its own weight rows into a D-deep register ring.
// (Loading the activations into every wave's registers put 4 MW L2 loads per
// K-step in the same in-order counter as the weight loads, and the waits
// before the first MFMAs of a step left almost no weight prefetch in flight.)
// The direct loads are inline assembly with hand-placed waits (as in the
// LDS-staged kernels); the weight loads are ordinary loads whose waits the
// compiler places.  They are issued unconditionally (past the slice's end
// they re-read its last K-step) and the main loop runs whole ring cycles with
// no per-step condition: a conditional load or step let the compiler's wait
// model assume, at the loop head, that a ring slot was loaded last, and it
// drained every load once per cycle.  Its model does not see the direct
// loads, so its waits are stricter than those need; the ring is a step deeper
// to make up for it.  K pairing (the same K range in both operands): with
// bf16 weights slice u of lane group g is K [32u + 8g, +8), so the four lane
// groups of a weight load read 64 contiguous bytes of a row; with MX weights
// it is K [32g + 8u, +8) (a lane's 32 values are one MX block).  The LDS copy
// of the activation tile keeps 16-byte chunk c of row r at chunk c ^ (r % 16)
// (conflict-free reads).
template <int MW, int D>
constexpr size_t splitk_lds_bytes() {
  return (size_t)(D + 1) * 16 * MW * 256;
}

template <int MW, int NW, int D, bool MXB>
__global__ void __launch_bounds__(256) bf16_splitk_kernel(const GemmArgs p, const SplitPlan sp,
                                                          float* __restrict__ part) {
  constexpr int MT = 16 * MW;
  constexpr int NT = 4 * 16 * NW;
  constexpr int NBUF = D + 1;             // the buffer refilled after step s was last read at step s - 1
  constexpr int ABYTES = MT * 256;        // activation tile of one K-step
  constexpr int BQ = MXB ? 1 : 4;         // 16-byte weight loads per fragment and K-step
  constexpr int BLOADS = MXB ? 2 * NW : 4 * NW;  // weight loads per lane and K-step (MX: codes + scale)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // NBUF * ABYTES
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  // Dense tiles only (the launcher checks): workgroup -> (group, M-tile,
  // N-tile), straight-line so the tile stays in registers.  Workgroup-uniform:
  // every wave of a workgroup returns here or none does.
  Tile t;
  {
    const int n_ntiles = (p.N + NT - 1) / NT;
    const int mpg = (p.M + MT - 1) / MT;
    const int gm = blockIdx.x / n_ntiles;
    const int nt = blockIdx.x - gm * n_ntiles;
    t.g = gm / mpg;
    if (t.g >= p.G) return;
    t.m0 = (gm - t.g * mpg) * MT;
    t.rows = p.M;
    t.row_base = 0;
    t.n0 = nt * NT + wave * 16 * NW;
  }
  const int slice = blockIdx.y;
  const GemmSeg& sg = p.seg[sp.seg[slice]];
  const int K = sg.K;
  const int ks0 = sp.ks0[slice];
  const int nks = sp.nks[slice];
  // Activation staging: instruction i of wave w fills chunks 256 i + 64 w + lane.
  const uint8_t* ga[MW];
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    const int c = 256 * i + tid;
    const int row = c >> 4, pch = c & 15;
    int ar = t.m0 + row;
    ar = ar < t.rows ? ar : t.rows - 1;
    ga[i] = sg.a + ((int64_t)ar * K + 128 * ks0) * 2 + 16 * (pch ^ (row & 15));
  }
  const int half = p.N >> 1;  // SwiGLU pair: columns [half, N) read b2
  const uint8_t* gb[NW];
  const uint8_t* gs[NW];
#pragma unroll
  for (int ni = 0; ni < NW; ++ni) {
    int c = t.n0 + 16 * ni + r16;
    c = c < p.N ? c : p.N - 1;
    const bool up = sg.b2 != nullptr && c >= half;
    const int cc = up ? c - half : c;
    const uint8_t* base = (up ? sg.b2 : sg.b) + (int64_t)t.g * sg.b_gstride;
    if (MXB && sg.b_rm) {  // row cc, MX block 4 ks + g4: 16 bytes of the row, its scale byte
      gb[ni] = base + (int64_t)cc * (K >> 1) + 64 * ks0 + 16 * g4;
      gs[ni] = (up ? sg.b2s : sg.bs) + (int64_t)t.g * sg.bs_gstride + (int64_t)cc * (K >> 5) + 4 * ks0 + g4;
    } else if (MXB) {      // the same block in fragment order (lane chunk cc % 16 + 16 g4 of block (cc / 16, ks))
      gb[ni] = base + ((int64_t)(cc >> 4) * (K >> 7) + ks0) * 1024 + 16 * ((cc & 15) + 16 * g4);
      gs[ni] = (up ? sg.b2s : sg.bs) + (int64_t)t.g * sg.bs_gstride + ((int64_t)ks0 * p.N + cc) * 4 + g4;
    } else {
      gb[ni] = base + ((int64_t)cc * K + 128 * ks0 + 8 * g4) * 2;
      gs[ni] = nullptr;
    }
  }
  const int64_t b_k = sg.b_rm ? 64 : 1024;              // MX weights: bytes between K-steps of a lane's codes
  const int64_t bs_k = sg.b_rm ? 4 : 4 * (int64_t)p.N;  // and of its scale
  struct BSlot {
    uint4 v[NW][BQ];
    int sc[NW];
  };
  BSlot bq[D];
  auto issue_a = [&](int ks) {
    uint8_t* buf = lds + (ks % NBUF) * ABYTES;
#pragma unroll
    for (int i = 0; i < MW; ++i) gl_lds16(ga[i] + 256 * ks, buf + 4096 * i + 1024 * wave);
  };
  auto issue_b = [&](int ks, BSlot& q) {
#pragma unroll
    for (int ni = 0; ni < NW; ++ni) {
      if (MXB) {
        q.v[ni][0] = to_uint4(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gb[ni] + b_k * ks)));
        q.sc[ni] = gs[ni][bs_k * ks];
      } else {
#pragma unroll
        for (int u = 0; u < BQ; ++u)
          q.v[ni][u] =
              to_uint4(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gb[ni] + 256 * ks + 64 * u)));
      }
    }
  };
  v4f acc[MW][NW][1];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi)
#pragma unroll
    for (int ni = 0; ni < NW; ++ni) acc[mi][ni][0] = v4f{0.f, 0.f, 0.f, 0.f};

  // Issue order per K-step k: its weight loads, then (real steps only) its
  // activation loads.
#pragma unroll
  for (int j = 0; j < D; ++j) {
    issue_b(j < nks ? j : nks - 1, bq[j]);
    if (j < nks) issue_a(j);
  }
  auto step = [&](int ks, BSlot& q) {
    // Issued after this step's activation loads: the D - 1 later steps'
    // weight loads and the real ones' activation loads.  At most that many
    // may still be in flight (the weight registers' own waits are the
    // compiler's).
    const int later = nks - 1 - ks < D - 1 ? nks - 1 - ks : D - 1;
    constexpr int WB = (D - 1) * BLOADS;
    switch (later) {
      case 0: wait_vmcnt<WB>(); break;
      case 1: wait_vmcnt<WB + MW>(); break;
      case 2: wait_vmcnt<WB + 2 * MW>(); break;
      default: wait_vmcnt<WB + 3 * MW>(); break;
    }
    barrier_lds();  // every wave's part of this step's activation tile is in LDS
    const uint8_t* buf = lds + (ks % NBUF) * ABYTES;
    uint4 bf[NW][4];
#pragma unroll
    for (int ni = 0; ni < NW; ++ni) {
      if (MXB) {
        e2m1_block_bf16(q.v[ni][0], q.sc[ni], bf[ni]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) bf[ni][u] = q.v[ni][BQ == 4 ? u : 0];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const int row = 16 * mi + r16;
        const int chunk = MXB ? 4 * g4 + u : 4 * u + g4;
        const uint4 av = *reinterpret_cast<const uint4*>(buf + row * 256 + ((chunk ^ (row & 15)) << 4));
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
          acc[mi][ni][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bf[ni][u]),
                                                                   acc[mi][ni][0], 0, 0, 0);
      }
    issue_b(ks + D < nks ? ks + D : nks - 1, q);
    if (ks + D < nks) issue_a(ks + D);  // its buffer was last read at step ks - 1
  };
  int ks = 0;
  for (; ks + D <= nks; ks += D) {  // whole ring cycles
#pragma unroll
    for (int j = 0; j < D; ++j) step(ks + j, bq[j]);
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j)   // the remaining steps
    if (ks + j < nks) step(ks + j, bq[j]);
  wait_vmcnt<0>();  // the re-reads past the slice's end

  GemmArgs q = p;  // the slice's partial sums, fp32 [G][M][N]
  q.c = part + (int64_t)slice * p.G * p.M * p.N;
  q.ldc = p.N;
  q.c_gstride = (int64_t)p.M * p.N;
  q.c_accumulate = 0;
  q.q = nullptr;
  epilogue<MW, NW, 1, EPI_F32>(q, t, acc, r16, g4);
}

// c = sum over slices of part[s][M][N] (slice order), and with QNT its MXFP8
// codes along N.  One thread per (row, 32-column block, r): columns 32b + r
// and 32b + 16 + r, so the 16 lanes of a block form one DPP row (quant_pair).
template <bool QNT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                            float* __restrict__ c, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ qs) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int nb = N >> 5;
  const int r = (int)(i & 15);
  const int64_t blk = i >> 4;  // row * nb + b; the 16 lanes of a DPP row share it
  if (blk >= (int64_t)M * nb) return;
  const int64_t row = blk / nb;
  const int b = (int)(blk - row * nb);
  const int64_t o = row * N + 32 * b + r;
  const int64_t MN = (int64_t)M * N;
  float v0 = 0.f, v1 = 0.f;
  for (int sl = 0; sl < S; ++sl) {
    v0 += part[sl * MN + o];
    v1 += part[sl * MN + o + 16];
  }
  c[o] = v0;
  c[o + 16] = v1;
  if (QNT) {
    int sc;
    const uint32_t w = quant_pair(v0, v1, sc);
    q[o] = (uint8_t)(w & 0xFF);
    q[o + 16] = (uint8_t)(w >> 8);
    if (r == 0) qs[row * nb + b] = (uint8_t)sc;
  }
}

// h = SiLU(gate) * up from the slice partials [S][G][M][2F] (slice order),
// as bf16 [G][M][F] and optionally fp32; one thread per output element.
__global__ void __launch_bounds__(256) splitk_swiglu_kernel(const float* __restrict__ part, int S, int G, int M,
                                                            int F, float* __restrict__ h32,
                                                            uint16_t* __restrict__ hb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)M * F;
  if (i >= (int64_t)G * per) return;
  const int64_t g = i / per;
  const int64_t rem = i - g * per;
  const int64_t row = rem / F;
  const int64_t col = rem - row * F;
  const int64_t o = (g * M + row) * (2 * (int64_t)F) + col;
  const int64_t stride = (int64_t)G * M * 2 * F;
  float gv = 0.f, uv = 0.f;
  for (int sl = 0; sl < S; ++sl) {
    gv += part[sl * stride + o];
    uv += part[sl * stride + o + F];
  }
  const float h = swiglu(gv, uv);
  hb[i] = (uint16_t)bf16_rne(h);
  if (h32) h32[i] = h;
}

// Weight-streaming variant for few rows per group (decode).  The weights are
// read exactly once, so the kernel is HBM-bound.  A workgroup of 4 waves owns
// MT x NT outputs (each wave 16*NW weight rows); per 128-deep K-step a wave
// loads, for each of its weight fragments, the fragment-order block of codes
// (1 KB contiguous; lane l takes its 16-byte MFMA operand at 16 l, read
// non-temporally) and the 64 contiguous scale bytes of the block's 16 rows,
// D K-steps ahead of the MFMAs, together with the few activation rows
// (L2-resident), read in the E4M3 operand layout straight from global memory.
//
// KS = 4 (dense GEMMs of few rows, where one accumulator per output leaves too
// few waves to keep enough weight bytes in flight): the workgroup's four
// waves own the same columns and each takes a contiguous quarter of the
// K-steps (counted over all K segments); waves 1-3 hand their accumulators to
// wave 0 through LDS, which adds them in wave order (deterministic) and runs
// the epilogue.
template <int MW, int NW, int EPI, int KS>
__device__ __forceinline__ void stream_gemm(const GemmArgs& p, int bid) {
  // K-steps in flight per wave: as many as keep two waves per SIMD.
  constexpr int D = MW == 1 ? (NW <= 2 ? 4 : 3) : 1;
  constexpr bool SWI = EPI == EPI_SWIGLU_QUANT;
  constexpr int NB = SWI ? 2 : 1;
  constexpr int MT = 16 * MW;
  constexpr int NT = (KS == 1 ? 4 : 1) * 16 * NW;
  static_assert(EPI == EPI_F32 || NW % 2 == 0, "quantising epilogues need whole 32-column blocks per wave");
  static_assert(KS == 1 || KS == 4, "one accumulator chain, or one per wave");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  Tile t;
  if (!decode_tile<MT, NT>(p, bid, wave, KS == 1 ? 16 * NW : 0, t)) return;  // uniform across the workgroup
  // This wave's K-steps [kc0, kc1) of the concatenated segments.
  int kc0 = 0, kc1 = 1 << 30;
  if (KS > 1) {
    int total = 0;
    for (int s = 0; s < p.nseg; ++s) total += p.seg[s].K >> 7;
    kc0 = (int)((int64_t)total * wave / KS);
    kc1 = (int)((int64_t)total * (wave + 1) / KS);
  }

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

  int kseg = 0;  // K-steps of the segments before this one
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSeg& sg = p.seg[s];
    const int K = sg.K;
    const int kb = K >> 5;
    // this wave's steps of the segment: [k0, k0 + nks)
    const int k0 = KS == 1 ? 0 : max(kc0 - kseg, 0);
    const int nks = KS == 1 ? K >> 7 : min(kc1 - kseg, K >> 7) - k0;
    kseg += K >> 7;
    if (KS > 1 && nks <= 0) continue;
    const uint8_t* ap[MW];
    const uint8_t* asp[MW];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
      ap[mi] = sg.a + arow[mi] * sg.lda + 16 * g4 + 128 * k0;
      asp[mi] = sg.as + arow[mi] * kb + g4 + 4 * k0;
    }
    // Weight operand of lane (r16, g4): row fcol + r16, elements 32 g4 .. +31
    // of the K-step -- 16 bytes at 16 lane of the fragment-order block, or
    // bytes 16 g4 of the row's 64 for the K-step when row-major.
    const bool brm = sg.b_rm != 0;
    const uint8_t* bp[NW][NB];
    const uint8_t* bsp[NW][NB];
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int h = 0; h < NB; ++h) {
        const uint8_t* cb = (h == 0 ? sg.b : sg.b2) + (int64_t)t.g * sg.b_gstride;
        const uint8_t* sb = (h == 0 ? sg.bs : sg.b2s) + (int64_t)t.g * sg.bs_gstride;
        bp[ni][h] = brm ? cb + (int64_t)(fcol[ni] + r16) * (K >> 1) + 16 * g4
                        : cb + (int64_t)(fcol[ni] >> 4) * (K >> 7) * 1024 + 16 * lane;
        bsp[ni][h] = brm ? sb + (int64_t)(fcol[ni] + r16) * kb + g4 : sb + 4 * (int64_t)(fcol[ni] + r16) + g4;
      }
    const int64_t b_k = brm ? 64 : 1024;                // bytes between K-steps of a lane's codes
    const int64_t bs_k = brm ? 4 : 4 * (int64_t)p.N;    // bytes between K-steps of the scales
#pragma unroll
    for (int ni = 0; ni < NW; ++ni)
#pragma unroll
      for (int h = 0; h < NB; ++h) {   // to this wave's first step
        bp[ni][h] += b_k * k0;
        bsp[ni][h] += bs_k * k0;
      }

    // Register ring of D K-steps: slot j holds the operands of step ks + j
    // (weight block and scale per fragment, activation fragment and scale per
    // M-fragment).  Each slot is refilled right after its MFMAs, so D steps
    // of loads stay in flight and a step's MFMAs wait only for its own slot.
    struct Slot {
      uint4 b[NW][NB];
      int bs[NW][NB];
      Frag8 a[MW];
      int as[MW];
    };
    Slot sl[D];
    auto load = [&](int ks, Slot& q) {
#pragma unroll
      for (int ni = 0; ni < NW; ++ni)
#pragma unroll
        for (int h = 0; h < NB; ++h) {
          q.b[ni][h] = to_uint4(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp[ni][h] + b_k * ks)));
          q.bs[ni][h] = bsp[ni][h][bs_k * ks];
        }
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const uint8_t* g = ap[mi] + 128 * ks;
        q.a[mi].lo = *reinterpret_cast<const uint4*>(g);
        q.a[mi].hi = *reinterpret_cast<const uint4*>(g + 64);
        q.as[mi] = asp[mi][4 * ks];
      }
    };
    auto compute = [&](const Slot& q) {
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        const v8i av = as_v8i(q.a[mi]);
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
          for (int h = 0; h < NB; ++h)
            acc[mi][ni][h] = mfma_f8f4(av, as_v8i(q.b[ni][h]), acc[mi][ni][h], q.as[mi], q.bs[ni][h]);
      }
    };
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < nks) load(j, sl[j]);
    int ks = 0;
    for (; ks + 2 * D <= nks; ks += D) {  // steady state: every refill is in range
#pragma unroll
      for (int j = 0; j < D; ++j) {
        compute(sl[j]);
        load(ks + j + D, sl[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < D; ++j)  // last refills
      if (ks + j < nks) {
        compute(sl[j]);
        if (ks + j + D < nks) load(ks + j + D, sl[j]);
      }
    ks += D;
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (ks + j < nks) compute(sl[j]);
  }
  if constexpr (KS > 1) {  // waves 1..3 hand their partial sums to wave 0, which adds them in order
    constexpr int NV = MW * NW * NB * 4;  // floats per lane
    __shared__ float red[KS > 1 ? KS - 1 : 1][NV][64];
    if (wave > 0) {
      int i = 0;
#pragma unroll
      for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
          for (int h = 0; h < NB; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave - 1][i++][lane] = acc[mi][ni][h][e];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w) {
      int i = 0;
#pragma unroll
      for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
          for (int h = 0; h < NB; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mi][ni][h][e] += red[w][i++][lane];
    }
  }
  epilogue<MW, NW, NB, EPI>(p, t, acc, r16, g4);
}

template <int MW, int NW, int EPI, int KS = 1>
__global__ void __launch_bounds__(256) mx_gemm_stream_kernel(const GemmArgs p) {
  stream_gemm<MW, NW, EPI, KS>(p, blockIdx.x);
}

// Two weight-streaming GEMMs with the same epilogue in one launch: workgroups
// [0, npre) compute `pre` (a dense GEMM, one accumulator chain per output),
// the rest `p`.  At decode the shared experts' gate/up GEMM, which needs only
// x, rides along with the routed experts' one: its few hundred workgroups
// stream their weights while the routed ones do, instead of a launch of its
// own bound by memory latency.
template <int MW, int NW, int EPI>
__global__ void __launch_bounds__(256) mx_gemm_stream_pair_kernel(const GemmArgs pre, int npre,
                                                                  const GemmArgs p) {
  const int b = blockIdx.x;
  if (b < npre) stream_gemm<MW, NW, EPI, 1>(pre, b);
  else stream_gemm<MW, NW, EPI, 1>(p, b - npre);
}

// Workgroups of a weight-streaming launch with NT-column tiles: one per
// (M-tile, N-tile) of a routed GEMM (max_mtiles bounds its M-tiles); a dense
// GEMM's tiles rounded up to whole rounds of the 8 XCDs (see decode_tile).
template <int MW>
static int64_t stream_tiles(const GemmArgs& a, int NT) {
  const int64_t n_ntiles = (a.N + NT - 1) / NT;
  if (a.offsets) return (int64_t)a.max_mtiles * n_ntiles;
  const int64_t mpg = (a.M + 16 * MW - 1) / (16 * MW);
  return ((int64_t)a.G * mpg * n_ntiles + 7) / 8 * 8;
}

template <int MW, int NW, int EPI>
static hipError_t launch_stream_cfg(const GemmArgs& a, hipStream_t s) {
  const bool chains = a.kchains == 4;
  if (a.kchains != 0 && a.kchains != 1 && !chains) return hipErrorInvalidValue;
  if (chains && a.offsets != nullptr) return hipErrorInvalidValue;  // dense GEMMs only
  const int NT = (chains ? 1 : 4) * 16 * NW;
  if (a.N % 16 != 0) return hipErrorInvalidValue;  // fragment-order weights
  if (a.M < 0 || a.G < 0) return hipErrorInvalidValue;
  const int64_t grid = stream_tiles<MW>(a, NT);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (chains) mx_gemm_stream_kernel<MW, NW, EPI, 4><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  else mx_gemm_stream_kernel<MW, NW, EPI, 1><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

int gemm_mtile(int shape) {
  return shape == GEMM_STREAM16 ? 16 : shape == GEMM_STREAM64 ? 64 : gemm_wide_mtile();
}

// The epilogue addresses a wave's output rows with 32-bit offsets from a
// wave-uniform base (gemm_epilogue.hpp): N and ldc below 2^22 keep 128 rows
// of fp32 output under 4 GB.
static bool epilogue_dims_ok(const GemmArgs& a) {
  return a.N > 0 && a.N < (1 << 22) && a.ldc >= 0 && a.ldc < (1 << 22);
}


template <int MW, int NW, int EPI>
static hipError_t launch_stream_pair_cfg(const GemmArgs& pre, const GemmArgs& a, hipStream_t s) {
  if (pre.offsets != nullptr || (pre.kchains != 0 && pre.kchains != 1) || (a.kchains != 0 && a.kchains != 1))
    return hipErrorInvalidValue;
  if (pre.N % 16 != 0 || a.N % 16 != 0) return hipErrorInvalidValue;
  if (pre.M < 0 || pre.G < 0) return hipErrorInvalidValue;
  const int64_t g0 = stream_tiles<MW>(pre, 4 * 16 * NW), g1 = stream_tiles<MW>(a, 4 * 16 * NW);
  if (g0 < 0 || g1 < 0 || g0 + g1 > 0x7fffffff) return hipErrorInvalidValue;
  if (g0 + g1 == 0) return hipSuccess;
  mx_gemm_stream_pair_kernel<MW, NW, EPI><<<dim3((unsigned)(g0 + g1)), dim3(256), 0, s>>>(pre, (int)g0, a);
  return hipGetLastError();
}

hipError_t launch_mx_gemm_pair(const GemmArgs& pre, const GemmArgs& a, int epi, hipStream_t s) {
  if (!epilogue_dims_ok(pre) || !epilogue_dims_ok(a)) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_F32: return launch_stream_pair_cfg<1, 4, EPI_F32>(pre, a, s);
    case EPI_SWIGLU_QUANT: return launch_stream_pair_cfg<1, 2, EPI_SWIGLU_QUANT>(pre, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bf16_gemm_quant(const GemmArgs& a, int shape, hipStream_t s) {
  if (!epilogue_dims_ok(a) || shape != GEMM_WIDE) return hipErrorInvalidValue;
  return launch_bf16_gemm_wide(a, EPI_F32_QUANT, s);
}

SplitPlan splitk_plan(const GemmArgs& a) {
  // About 2048 waves in all, at most 8 slices' worth of K cuts (the partial
  // sums stay small next to the weights; at 64 tokens the MX down-projection
  // with its reduce measured 27 us at 8 slices against 31 us at 14); segments
  // are cut separately.
  const int MT = a.M <= 16 ? 16 : 64;
  const int tiles = a.G * ((a.N + 127) / 128) * ((a.M + MT - 1) / MT);
  int target = (2048 + 4 * tiles - 1) / (4 * tiles);
  target = target < 1 ? 1 : (target > 8 ? 8 : target);
  int total = 0;
  for (int i = 0; i < a.nseg; ++i) total += a.seg[i].K / 128;
  const int kper = (total + target - 1) / target;
  SplitPlan sp = {};
  for (int i = 0; i < a.nseg; ++i) {
    const int ks = a.seg[i].K / 128;
    for (int k0 = 0; k0 < ks && sp.n < kMaxSlices; k0 += kper) {
      sp.seg[sp.n] = (int8_t)i;
      sp.ks0[sp.n] = (int16_t)k0;
      sp.nks[sp.n] = (int16_t)(ks - k0 < kper ? ks - k0 : kper);
      ++sp.n;
    }
  }
  return sp;
}

hipError_t launch_bf16_splitk(const GemmArgs& a, bool bf16_b, const SplitPlan& sp, float* part, hipStream_t s) {
  if (a.offsets != nullptr || a.nseg < 1 || a.nseg > 9 || a.G < 1 || a.M <= 0 || a.N % 32 != 0 || sp.n <= 0 ||
      sp.n > kMaxSlices || !part)
    return hipErrorInvalidValue;
  for (int i = 0; i < a.nseg; ++i) {
    const GemmSeg& g = a.seg[i];
    if (g.K <= 0 || g.K % 128 != 0 || g.K / 128 > 32767 || !g.a || !g.b || (!bf16_b && !g.bs))
      return hipErrorInvalidValue;
    if (g.b2 && (a.N % 2 != 0 || (!bf16_b && !g.b2s))) return hipErrorInvalidValue;
  }
  int covered = 0;
  for (int j = 0; j < sp.n; ++j) {  // every slice inside its segment, every K-step once
    if (sp.seg[j] < 0 || sp.seg[j] >= a.nseg || sp.ks0[j] < 0 || sp.nks[j] <= 0 ||
        sp.ks0[j] + sp.nks[j] > a.seg[sp.seg[j]].K / 128)
      return hipErrorInvalidValue;
    covered += sp.nks[j];
  }
  int total = 0;
  for (int i = 0; i < a.nseg; ++i) total += a.seg[i].K / 128;
  if (covered != total) return hipErrorInvalidValue;
  GemmArgs q = a;
  q.c = part;
  q.ldc = a.N;
  if (!epilogue_dims_ok(q)) return hipErrorInvalidValue;
  const bool small = a.M <= 16;
  const int MT = small ? 16 : 64;
  // MX weights at 64-row tiles: 16 columns per wave (NT = 64), twice the
  // workgroups, each decoding one weight fragment per K-step.
  const bool narrow = !bf16_b && !small;
  const int NT = narrow ? 64 : 128;
  const int64_t grid = (int64_t)a.G * ((a.M + MT - 1) / MT) * ((a.N + NT - 1) / NT);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 gd((unsigned)grid, (unsigned)sp.n);
  constexpr int D = 4;
  constexpr size_t lds1 = splitk_lds_bytes<1, D>(), lds4 = splitk_lds_bytes<4, D>();
  static DeviceOnce attr;
  hipError_t ea = lds_limit_once(attr, {reinterpret_cast<const void*>(&bf16_splitk_kernel<4, 2, D, false>),
                                        reinterpret_cast<const void*>(&bf16_splitk_kernel<4, 1, D, true>)},
                                 (int)lds4);
  if (ea != hipSuccess) return ea;
  if (bf16_b) {
    if (small) bf16_splitk_kernel<1, 2, D, false><<<gd, dim3(256), lds1, s>>>(a, sp, part);
    else bf16_splitk_kernel<4, 2, D, false><<<gd, dim3(256), lds4, s>>>(a, sp, part);
  } else {
    if (small) bf16_splitk_kernel<1, 2, D, true><<<gd, dim3(256), lds1, s>>>(a, sp, part);
    else bf16_splitk_kernel<4, 1, D, true><<<gd, dim3(256), lds4, s>>>(a, sp, part);
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int S, int M, int N, float* c, uint8_t* q, uint8_t* qs,
                                hipStream_t s) {
  if (S <= 0 || M <= 0 || N % 32 != 0 || !c) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)M * (N / 32) * 16;
  const int64_t blocks = (threads + 255) / 256;
  if (q) splitk_reduce_kernel<true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(part, S, M, N, c, q, qs);
  else splitk_reduce_kernel<false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(part, S, M, N, c, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_splitk_swiglu(const float* part, int S, int G, int M, int F, float* h32, uint16_t* hb,
                                hipStream_t s) {
  if (S <= 0 || G <= 0 || M <= 0 || F <= 0 || !hb) return hipErrorInvalidValue;
  const int64_t n = (int64_t)G * M * F;
  splitk_swiglu_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(part, S, G, M, F, h32, hb);
  return hipGetLastError();
}

int bf16_mx_splitk_slices(int M, int N, int K) {
  GemmArgs a = {};
  a.nseg = 1;
  a.seg[0].K = K;
  a.G = 1;
  a.M = M;
  a.N = N;
  return splitk_plan(a).n;
}

hipError_t launch_bf16_mx_splitk(const GemmArgs& a, float* part, int S, float* z, uint8_t* zq, uint8_t* zqs,
                                 hipStream_t s) {
  if (a.nseg != 1 || a.G != 1) return hipErrorInvalidValue;
  const SplitPlan sp = splitk_plan(a);
  if (sp.n != S) return hipErrorInvalidValue;  // the partial buffer was sized for S slices
  hipError_t e = launch_bf16_splitk(a, false, sp, part, s);
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(part, sp.n, a.M, a.N, z, zq, zqs, s);
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
