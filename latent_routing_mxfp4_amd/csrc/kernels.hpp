// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- MX quantisation (mx_quant.hip) -----------------------------------------
// fmt 0: E4M3 codes [rows][K]; fmt 1: E2M1 packed codes [rows][K/2] (row-major),
// or, with frag_rows = N > 0, in fragment order for rows/N matrices of N rows.
// deq_bf16 (E4M3 only, may be null): bf16 [rows][K] of the dequantised values.
//
// Fragment order (every weight matrix the MX GEMMs read), for G matrices
// [N][K] with N % 16 == 0 and K % 128 == 0:
//   codes:  per matrix, 1024-byte blocks (nb, kb) at (nb * K/128 + kb) * 1024,
//           nb = row / 16, kb = k / 128; inside, lane l = r + 16 q holds 16
//           bytes at 16 l: row 16 nb + r, elements 128 kb + 32 q .. +31, two per
//           byte, even element low -- the B operand of one 16x16x128 MFMA.
//   scales: per matrix, [K/128][N] dwords: the four E8M0 scales of row n for
//           K-step kb (byte j = block 4 kb + j).
// A matrix's codes and scales are N*K/2 and N*K/32 bytes, as in row-major.
hipError_t launch_quantize(const float* in, int64_t rows, int K, int fmt, uint8_t* codes,
                           uint8_t* scales, hipStream_t s, uint16_t* deq_bf16 = nullptr, int frag_rows = 0);
// Row-major E2M1 codes [G*N][K/2] + scales [G*N][K/32] -> fragment order.
hipError_t launch_pack_e2m1(const uint8_t* codes, const uint8_t* scales, int64_t G, int N, int K,
                            uint8_t* out_codes, uint8_t* out_scales, hipStream_t s);
// E2M1 codes + scales of one [rows][K] matrix -> exact bf16 [rows][K]; the
// input row-major (codes [rows][K/2], scales [rows][K/32]) or, with
// frag != 0, in fragment order (rows % 16 == 0, K % 128 == 0).
hipError_t launch_decode_e2m1_bf16(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                                   uint16_t* out, hipStream_t s, int frag = 0);
// fp32 [n] -> bfloat16 [n], round to nearest even (n % 4 == 0, in 16-byte and
// out 8-byte aligned).
hipError_t launch_round_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t s);

// ---- Router (router.hip) ----------------------------------------------------
// logits[T][E] = z[T][L] w[E][L]^T (+ bias[E]) at fp32 accuracy.  Many tokens
// (router_bf16x3 true): three exact bf16 pieces per operand on the bf16 matrix
// cores, with w's pieces written to `wplanes` (3 * E * L bf16) first.  Few
// tokens: the fp32 matrix cores; `partial` (router_split(T, E, L) * T * E
// floats, or null when that is 1) holds the K-slice sums when the tile grid is
// small.
int router_split(int T, int E, int L);
bool router_bf16x3(int T, int E, int L);
// leave_partial (with router_reduce_in_topk(T, E, L)): the K-slice sums stay
// in `partial` for launch_router_reduce_topk, which adds them.
hipError_t launch_router_logits(const float* z, const float* w, const float* logit_bias, int T, int E,
                                int L, float* logits, float* partial, uint16_t* wplanes, hipStream_t s,
                                bool leave_partial = false);
bool router_reduce_in_topk(int T, int E, int L);
int router_slices(int T, int E, int L);  // K-slice sums written to `partial` (<= router_split)
// Per token: s = sigmoid(logit), key = s + sel_bias, top-k by (key desc, id asc),
// gates = s / sum(s over the k winners).  softmax_gates: key = logit + sel_bias,
// gates = softmax over the k winners' logits.
hipError_t launch_topk(const float* logits, const float* sel_bias, int T, int E, int k, bool softmax_gates,
                       int32_t* ids, float* gates, hipStream_t s);
// The same selection on the router's nz = router_split(T, E, L) K-slice sums
// (E <= 1024): logits = sum of the slices in slice order + logit_bias, written
// to `logits`, then top-k as launch_topk.
hipError_t launch_router_reduce_topk(const float* partial, int nz, const float* logit_bias, const float* sel_bias,
                                     int T, int E, int k, bool softmax_gates, float* logits, int32_t* ids,
                                     float* gates, hipStream_t s);

// ---- Dispatch (permute.hip) -------------------------------------------------
size_t dispatch_scratch_ints(int T, int E);
// counts[E], offsets[E+1], row_of_pair[T*k], pair_of_row[T*k], and, for each of
// the two M-tile heights mt0/mt1, mtile_start_x[E+1] (prefix of ceil(count/mt)).
// mtile_group0/1 (nullable, mtile_start0/1[E] entries): the group of each
// M-tile of height mt0/mt1, so that a workgroup finds its group with one load.
hipError_t launch_dispatch(const int32_t* ids, int T, int E, int k, int32_t* scratch, int32_t* counts,
                           int32_t* offsets, int32_t* row_of_pair, int32_t* pair_of_row, int mt0,
                           int32_t* mtile_start0, int32_t* mtile_group0, int mt1, int32_t* mtile_start1,
                           int32_t* mtile_group1, hipStream_t s);

// ---- MX GEMM (mx_gemm.hip) --------------------------------------------------
enum Epilogue : int {
  EPI_F32 = 0,          // c = acc (fp32)
  EPI_F32_QUANT = 1,    // c = acc and q = MXFP8(acc) along N
  EPI_SWIGLU_QUANT = 2, // q = MXFP8(SiLU(acc_gate) * acc_up) along N
  EPI_SWIGLU_BF16 = 3   // ob = bf16(SiLU(acc_gate) * acc_up) (bf16 kernels only)
};

struct GemmSeg {
  const uint8_t* a;    // E4M3 codes, row stride lda bytes
  const uint8_t* as;   // scales, row stride lda/32
  int64_t lda;         // = K of this segment (codes bytes per row)
  const uint8_t* b;    // E2M1 packed codes of group 0: [N][K/2]
  const uint8_t* bs;   // scales of group 0: [N][K/32]
  const uint8_t* b2;   // second matrix (the "up" half of a SwiGLU), or null
  const uint8_t* b2s;
  int64_t b_gstride;   // bytes between groups' code matrices
  int64_t bs_gstride;  // bytes between groups' scale matrices
  int K;
  int b_rm;            // MX B (and b2) row-major: codes [N][K/2], scales [N][K/32]; 0 = fragment order
};

struct GemmArgs {
  int nseg;
  GemmSeg seg[9];           // K segments (up to 1 + 8 shared experts)
  // Groups.  Routed: rows of group g are [offsets[g], offsets[g+1]) and its
  // M-tiles are [mtile_start[g], mtile_start[g+1]).  Dense: G groups of M rows.
  const int32_t* offsets;      // null => dense
  const int32_t* mtile_start;  // routed only
  const int32_t* mtile_group;  // routed: group of each M-tile (null: binary search over mtile_start)
  int G;
  int M;                       // dense rows per group
  int N;                       // output columns (per matrix)
  const int32_t* gather;       // routed A-row gather: A row = gather[row] / gather_div (null = row)
  int gather_div;
  // Outputs: row index is the sorted row (routed) or m (dense, + g * c_gstride rows).
  float* c;
  int64_t ldc;
  int64_t c_gstride;           // elements between dense groups' outputs
  int c_accumulate;            // fp32 output (EPI_F32): c += acc instead of c = acc
  uint8_t* q;                  // E4M3 codes [rows][N]
  uint8_t* qs;                 // scales [rows][N/32]
  int64_t q_gstride;           // bytes between dense groups' code outputs
  int64_t qs_gstride;
  uint16_t* ob;                // EPI_SWIGLU_BF16: bfloat16 [rows][N]
  int64_t ob_gstride;          // elements between dense groups' bf16 outputs
  int max_mtiles;              // upper bound of M-tiles (grid size / n-tiles)
  int kchains;                 // weight-streaming dense GEMMs: 4 = the K-steps are split over the 4 waves
                               // of a workgroup (summed in wave order), 0 or 1 = one accumulator per output
};

// Kernel configurations: weight streaming with 16 or 64 rows per M-tile (few
// rows per group: decode) and the 512-thread kernels with 128-row tiles (many
// rows per group: prefill; 128 x 512 for MX, 128 x 256 for bf16).
enum GemmShape : int { GEMM_STREAM16 = 0, GEMM_STREAM64 = 1, GEMM_WIDE = 4 };
int gemm_mtile(int shape);
// Two weight-streaming GEMMs (GEMM_STREAM16 shape, EPI_F32 or
// EPI_SWIGLU_QUANT, one accumulator chain each) in one launch: the dense
// `pre` on the first workgroups, then `a` (dense or routed).
hipError_t launch_mx_gemm_pair(const GemmArgs& pre, const GemmArgs& a, int epi, hipStream_t s);

// Dense bf16 GEMM on the 512-thread 128 x 256 kernel (mx_gemm_wide.hip): G
// dense groups of M rows, A = bf16 [M][K] per K segment (seg[i].a, shared by
// the groups), B = bf16 [N][K] row-major (seg[i].b + g * b_gstride bytes), the
// segments' products summed in fp32; every K a multiple of 64.  Epilogues:
// EPI_F32, EPI_F32_QUANT, and EPI_SWIGLU_BF16 with seg[i].b2 the "up" matrix
// (128 output columns per tile instead of 256).
hipError_t launch_bf16_gemm_quant(const GemmArgs& args, int shape, hipStream_t s);
hipError_t launch_bf16_gemm_wide(const GemmArgs& args, int epilogue, hipStream_t s);

// Few-row dense bf16 GEMMs with K split into slices (decode sizes).  A =
// bf16 [M][K] per segment; B row-major, either MXFP4 (seg.b codes [N][K/2],
// seg.bs scales [N][K/32], decoded to exact bf16 in registers) or bf16
// [N][K].  G dense groups (B + g * b_gstride bytes); with seg.b2, columns
// [N/2, N) read b2 (the "up" half of a SwiGLU pair).  Each K segment is cut
// into slices of at most kper 128-wide K-steps; slice s writes its fp32
// partial sums to part[s][g][M][N].  Every K a multiple of 128, N of 32.
constexpr int kMaxSlices = 24;
struct SplitPlan {
  int n;                      // slices
  int8_t seg[kMaxSlices];     // segment of slice s
  int16_t ks0[kMaxSlices];    // its first K-step (128 wide) in the segment
  int16_t nks[kMaxSlices];    // its K-steps
};
SplitPlan splitk_plan(const GemmArgs& args);
hipError_t launch_bf16_splitk(const GemmArgs& args, bool bf16_b, const SplitPlan& sp, float* part, hipStream_t s);
// c[M][N] = sum of the S partials in slice order; with q, its MXFP8 codes along N.
hipError_t launch_splitk_reduce(const float* part, int S, int M, int N, float* c, uint8_t* q, uint8_t* qs,
                                hipStream_t s);
// h = SiLU(gate) * up from S partials of G pair-groups [S][G][M][2F] (gate
// columns [0, F), up columns [F, 2F)), written as bf16 [G][M][F] and, when
// h32 is given, fp32.
hipError_t launch_splitk_swiglu(const float* part, int S, int G, int M, int F, float* h32, uint16_t* hb,
                                hipStream_t s);

// The latent down-projection at decode sizes (MXFP4 weights): split-K as
// above, then z and, when zq is given, its MXFP8 codes.
int bf16_mx_splitk_slices(int M, int N, int K);
hipError_t launch_bf16_mx_splitk(const GemmArgs& args, float* part, int S, float* z, uint8_t* zq, uint8_t* zqs,
                                 hipStream_t s);

// Launch the grouped/dense MX GEMM with an automatically chosen tile shape.
hipError_t launch_mx_gemm(const GemmArgs& args, int epilogue, int shape, hipStream_t s);

// The 512-thread, 128 x 512 tile kernel for many rows per group (prefill);
// routed M-tiles are gemm_wide_mtile() rows.  Every K must be a multiple of 128.
int gemm_wide_mtile();
hipError_t launch_mx_gemm_wide(const GemmArgs& args, int epilogue, hipStream_t s);

// Operands of the gate-weighted combine (launch_combine's arguments, MXFP8
// output): y_lat[t] = sum_j gates[t][j] * y_e[row_of_pair[t][j]] in slot order.
struct CombineArgs {
  const float* y_e;
  const float* gates;
  const int32_t* row_of_pair;
  int T, k, L;
  float* y_lat;  // nullable
  uint8_t* yq;
  uint8_t* yqs;
};
// The 512-thread MX kernel's dense SwiGLU + MXFP8 GEMM (the shared experts'
// gate/up at prefill) and the combine in one launch: the combine runs on a
// fraction of the workgroups spread through the launch, the GEMM on the rest.
hipError_t launch_mx_gemm_wide_combine(const GemmArgs& args, const CombineArgs& c, hipStream_t s);

// ---- Quantile Balancing (balance.hip) ----------------------------------------
// New selection bias from one batch of router logits [T][E] (sigmoid keys):
// b_out = b_in - eta * Q, Q[e] the midpoint of expert e's n-th and (n+1)-th
// largest score margins, n = quantile_balance_target(T, E, k).  ws holds
// quantile_balance_workspace_floats(T, E) floats; q_out may be null; b_out may
// be b_in.  Requires 2 <= T, 1 <= k < E <= 4096.
size_t quantile_balance_workspace_floats(int T, int E);
int quantile_balance_target(int T, int E, int k);
hipError_t launch_quantile_balance(const float* logits, int T, int E, int k, const float* bias_in, float eta,
                                   float* bias_out, float* q_out, float* ws, hipStream_t s);

// ---- Matrix-core rate probe (mfma_rate.hip) ---------------------------------
// workgroups x 4 waves, each issuing 8 * iters independent FP8 x FP4 MFMAs of
// 16x16x128; out[workgroups * 4] receives one checksum per wave.
hipError_t launch_mfma_rate(int iters, int workgroups, float* out, hipStream_t s);
// Plain HBM read stream: `bytes` (a multiple of 16) from buf by `workgroups` x
// 256 threads; out[workgroups * 256] receives one fold per thread.
hipError_t launch_hbm_read(const void* buf, int64_t bytes, int workgroups, uint32_t* out, hipStream_t s);

// ---- Combine (combine.hip) --------------------------------------------------
// y_lat[t] = sum_j gates[t][j] * y_e[row_of_pair[t*k+j]] (slot order), then
// yq = MXFP8(y_lat) per row and/or yb = bf16(y_lat); any output may be null.
hipError_t launch_combine(const float* y_e, const float* gates, const int32_t* row_of_pair, int T, int k,
                          int L, float* y_lat_out, uint8_t* yq, uint8_t* yqs, hipStream_t s,
                          uint16_t* yb = nullptr);

}  // namespace moe
