/*
 * moe_layer.h -- C ABI of the MI355X (gfx950) LatentMoE layer forward.
 *
 * The layer (Kimi K3 and the New Open-Weights Moat, section "Sparse
 * computation: latent experts and routing" and section "How the router picks
 * 16 of 896", Fig. 2):
 *
 *   xq    = MXFP8(x)                                  per token, blocks of 32
 *   z     = deq(xq) deq(W_down)^T                     model width -> latent
 *   s     = sigmoid(z W_router^T + logit_bias)        one score per routed expert
 *   ids   = top_k(s + selection_bias)                 ties -> lower expert id
 *   gates = s[ids] / sum(s[ids])                      bias not in the gates
 *   per expert e, on the tokens routed to it (stable, token order):
 *       h   = SiLU(zq W_gate_e^T) * (zq W_up_e^T),  hq = MXFP8(h)
 *       y_e = deq(hq) deq(W_down_e)^T
 *   y_lat = sum_j gates[j] y_e[j]                     gate-weighted combine
 *   y     = deq(MXFP8(y_lat)) deq(W_up)^T
 *         + sum_s deq(MXFP8(SiLU(xq W_gate_s^T) * (xq W_up_s^T))) deq(W_down_s)^T
 *
 * Number formats (Kimi K3: 2.8 Trillion Parameters, Four Bits at a Time,
 * section "Four bits from the start"; Moat page, section "Precision and
 * deployment", Fig. 6): weights are MXFP4 (E2M1 elements), activations MXFP8
 * (E4M3, OCP "FN" variant), 32 elements per block sharing one E8M0 scale.
 * The router weight is fp32 and is not quantised.
 *
 * Row-major storage of an MX tensor [rows][K] (blocks run along K, the
 * contraction dim):
 *   E2M1 codes: [rows][K/2] bytes, element 2i in the low nibble of byte i;
 *   E4M3 codes: [rows][K] bytes;
 *   scales:     [rows][K/32] bytes, E8M0 (value 2^(c-127)).
 * Weight matrices are [out][in] (nn.Linear orientation; x @ W[e] of the MoE
 * data-path toy, Kimi K3: 2.8 Trillion Parameters, Four Bits at a Time,
 * section "What it takes to serve it").  The layer reads its MX weights in
 * either of two layouts, chosen by moe_layer_config.weight_layout:
 *   MOE_WEIGHTS_ROW_MAJOR: the row-major storage above, as a checkpoint holds
 *     the MXFP4 codes (consumed as stored);
 *   MOE_WEIGHTS_FRAGMENT: FRAGMENT ORDER, which keeps the same bytes per matrix
 *     but puts each operand of one 16x16x128 block-scaled MFMA in one
 *     contiguous 1 KB block (the prefill kernels then move whole cache lines
 *     per load; the faster layout).
 * For G matrices [N][K], N % 16 == 0, K % 128 == 0, fragment order is:
 *   codes:  matrix g starts at g*N*K/2; block (nb, kb) = rows 16nb..16nb+15,
 *           elements 128kb..128kb+127 sits at (nb*(K/128) + kb)*1024; inside
 *           it, bytes 16l..16l+15 (l = r + 16q, r < 16, q < 4) are the E2M1
 *           codes of row 16nb + r, elements 128kb + 32q .. +31 (two per byte,
 *           even element in the low nibble);
 *   scales: matrix g starts at g*N*K/32; then [K/128][N] groups of 4 bytes:
 *           group (kb, n) holds the E8M0 scales of blocks 4kb..4kb+3 of row n.
 * moe_mx_quantize_weights writes this order; moe_mx_pack_weights converts
 * row-major E2M1 into it.
 *
 * All tensor pointers are DEVICE pointers unless stated otherwise.  Every
 * call is asynchronous on the given HIP stream (a hipStream_t passed as
 * void*, NULL = the null stream); no call synchronises the host, allocates
 * device memory or copies between host and device.  Pointers stay owned by
 * the caller.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every entry point returns one of these (0 = success). */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, k > E, ...            */
  MOE_ERR_UNSUPPORTED = -2, /* valid layer this build does not run (see create) */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  MOE_ERR_HIP = -4          /* a HIP launch reported an error                 */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* Layouts of the MX weight tensors (see the top of this file). */
enum { MOE_WEIGHTS_ROW_MAJOR = 0, MOE_WEIGHTS_FRAGMENT = 1 };

/* Layer shape.  d_model, d_latent, d_ff_routed, d_ff_shared must be positive
 * multiples of 128: every one of them is the contraction of some MX GEMM,
 * which the block-scaled instruction consumes 128 elements (four MX blocks)
 * at a time (the pages' widths 7168, 3584 and the 3072 estimate all are);
 * 1 <= top_k <= n_routed <= 4096; 0 <= n_shared <= 8; 1 <= max_tokens <=
 * 2^20.  The Kimi-K3 width is {7168, 3584, 896, 16, 2, 3072, 3072, T}. */
typedef struct {
  int32_t d_model;     /* d:  model width                        */
  int32_t d_latent;    /* L:  routed latent width                */
  int32_t n_routed;    /* E:  routed experts                     */
  int32_t top_k;       /* k:  experts kept per token             */
  int32_t n_shared;    /* S:  always-on shared experts           */
  int32_t d_ff_routed; /* F:  routed-expert intermediate width   */
  int32_t d_ff_shared; /* Fs: shared-expert intermediate width   */
  int32_t max_tokens;  /* largest T a forward call may pass      */
  /* Second workload (zero = the LatentMoE above).  identity_latent != 0: no
   * latent projections (d_latent must equal d_model; w_down and w_up may be
   * NULL): the router reads x itself, the experts read xq, and
   *     y = y_lat + shared experts       (y_lat at model width, fp32).
   * softmax_gates != 0: selection keys are logit + selection_bias and the
   * gates are the softmax over the k winners' logits (the gate of the MoE
   * data-path toy, Kimi K3: 2.8 Trillion Parameters, Four Bits at a Time,
   * section "What it takes to serve it"). */
  int32_t identity_latent;
  int32_t softmax_gates;
  /* Higher-precision map (Moat page, section "Precision and deployment",
   * Fig. 6: only the routed experts are MXFP4 x MXFP8; the latent projections
   * and the shared experts stay at higher precision, here bfloat16).
   * dense_bf16 != 0 (latent layers only): W_down, W_up and the shared experts
   * are the bfloat16 tensors *_bf16 of moe_layer_weights (their MX tensors may
   * be NULL), and
   *     xb = bf16(x)   (round to nearest even)
   *     z  = xb W_down^T                  (fp32 accumulation)
   *     hs = bf16(SiLU(xb W_gate_s^T) * (xb W_up_s^T))
   *     y  = bf16(y_lat) W_up^T + sum_s hs W_down_s^T.
   * The router, top-k, dispatch and routed experts are unchanged. */
  int32_t dense_bf16;
  /* Layout of every MX weight tensor of moe_layer_weights: MOE_WEIGHTS_ROW_MAJOR
   * (0, the zero default) or MOE_WEIGHTS_FRAGMENT. */
  int32_t weight_layout;
} moe_layer_config;

/* One MXFP4 (E2M1) tensor: packed codes and E8M0 scales, device memory. */
typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
} moe_mx_tensor;

/* Layer weights.  Non-owning: every buffer must outlive the handle and must
 * not change while a forward that reads it is in flight.  Expert tensors are
 * the E (or S) matrices stored back to back (per-expert matrices W[E] of the
 * MoE data-path toy).  Every MX tensor is in the layout the config names;
 * codes 16-byte and scales 4-byte aligned. */
typedef struct {
  moe_mx_tensor w_down;            /* [L][d]      latent down-projection (row-major) */
  moe_mx_tensor w_up;              /* [d][L]      latent up-projection          */
  const float* w_router;           /* [E][L] fp32 router                        */
  const float* router_logit_bias;  /* [E] added to the logits, or NULL (zeros)  */
  const float* selection_bias;     /* [E] added for selection only, or NULL     */
  moe_mx_tensor w_gate_e;          /* [E][F][L]   routed gate projections       */
  moe_mx_tensor w_up_e;            /* [E][F][L]   routed up projections         */
  moe_mx_tensor w_down_e;          /* [E][L][F]   routed down projections       */
  moe_mx_tensor w_gate_s;          /* [S][Fs][d]  shared gate projections       */
  moe_mx_tensor w_up_s;            /* [S][Fs][d]  shared up projections         */
  moe_mx_tensor w_down_s;          /* [S][d][Fs]  shared down projections       */
  /* bfloat16 [out][in] row-major weights of the higher-precision map
   * (dense_bf16 != 0; otherwise ignored and may be NULL), 16-byte aligned. */
  const uint16_t* w_down_bf16;     /* [L][d]                                    */
  const uint16_t* w_up_bf16;       /* [d][L]                                    */
  const uint16_t* w_gate_s_bf16;   /* [S][Fs][d]                                */
  const uint16_t* w_up_s_bf16;     /* [S][Fs][d]                                */
  const uint16_t* w_down_s_bf16;   /* [S][d][Fs]                                */
} moe_layer_weights;

/* Stage boundaries at which moe_layer_forward records the optional timing
 * events of a trace (event i is recorded on the forward's stream right after
 * stage i finishes launching; event 0 before the first launch). */
enum {
  MOE_EV_START = 0,
  MOE_EV_QUANT_X = 1,    /* xq = MXFP8(x)                              */
  MOE_EV_DOWN = 2,       /* z, zq: latent down-projection              */
  MOE_EV_LOGITS = 3,     /* router logits                              */
  MOE_EV_TOPK = 4,       /* top-k ids and gates                        */
  MOE_EV_DISPATCH = 5,   /* counts, offsets, permutation               */
  MOE_EV_EXPERT_UP = 6,  /* routed gate/up GEMM + SwiGLU + MXFP8       */
  MOE_EV_EXPERT_DOWN = 7,/* routed down GEMM                           */
  MOE_EV_COMBINE = 8,    /* gate-weighted combine + MXFP8              */
  MOE_EV_SHARED_UP = 9,  /* shared gate/up GEMM + SwiGLU + MXFP8       */
  MOE_EV_OUT = 10,       /* up-projection + shared down-projections    */
  MOE_TRACE_EVENTS = 11
};

/* Optional device-side copies of the forward's intermediates, for testing.
 * Every member may be NULL; non-NULL members are filled by the forward (on
 * the same stream) with the sizes shown, for the T of that call.  Rows in
 * "sorted order" are the (token, slot) pairs stably sorted by expert.
 * `events`, if not NULL, is a HOST array of MOE_TRACE_EVENTS hipEvent_t
 * handles (created by the caller) recorded at the stage boundaries above; a
 * NULL entry leaves its boundary unrecorded (each record costs the stream a
 * few microseconds, so a timing run can bracket only the stage it needs). */
typedef struct {
  uint8_t* xq_codes;   uint8_t* xq_scales;   /* [T][d], [T][d/32]            */
  float* z;                                  /* [T][L] fp32 latent           */
  uint8_t* zq_codes;   uint8_t* zq_scales;   /* [T][L], [T][L/32]            */
  float* logits;                             /* [T][E] router logits (+bias) */
  int32_t* ids;        float* gates;         /* [T][k] slot order            */
  int32_t* counts;                           /* [E] pairs per expert         */
  int32_t* offsets;                          /* [E+1] exclusive prefix sum   */
  int32_t* pair_of_row;                      /* [T*k] pair t*k+j of sorted row */
  int32_t* row_of_pair;                      /* [T*k] sorted row of pair     */
  float* h;                                  /* [T*k][F] SiLU(gate)*up, sorted rows */
  uint8_t* hq_codes;   uint8_t* hq_scales;   /* [T*k][F], [T*k][F/32] sorted */
  float* y_e;                                /* [T*k][L] expert outputs, sorted */
  float* y_lat;                              /* [T][L] combined latent       */
  uint8_t* yq_codes;   uint8_t* yq_scales;   /* [T][L], [T][L/32]            */
  float* hs;                                 /* [S][T][Fs] shared hidden, fp32 */
  uint8_t* hs_codes;   uint8_t* hs_scales;   /* [S][T][Fs], [S][T][Fs/32]    */
  void* const* events;                       /* host array of hipEvent_t, or NULL */
  /* Higher-precision map only (the MX copies xq, yq, hs_codes are then not
   * written): */
  uint16_t* xb;                              /* [T][d] bf16(x)               */
  uint16_t* yb;                              /* [T][L] bf16(y_lat)           */
  uint16_t* hs_bf16;                         /* [S][T][Fs] shared hidden, bf16 */
} moe_layer_trace;

typedef struct moe_layer* moe_layer_t;

/* Validate the shape and record the (non-owning) weight pointers of one
 * LatentMoE layer (Kimi K3 and the New Open-Weights Moat, "Sparse
 * computation: latent experts and routing": the latent routed path and the
 * shared branch).  Host-side only: launches nothing.  *out is written only on
 * success.
 * Errors: MOE_ERR_INVALID_ARG for null pointers (the two biases may be NULL;
 * the shared tensors may be NULL when n_shared == 0) or out-of-range sizes;
 * MOE_ERR_UNSUPPORTED when a width is not a multiple of 128. */
int moe_layer_create(const moe_layer_config* cfg, const moe_layer_weights* w, moe_layer_t* out);

/* Device workspace, in bytes, that a forward over T tokens needs
 * (0 <= T <= cfg->max_tokens): every intermediate of the layer's steps (the
 * permuted buffer of T*k rows, Four Bits at a Time, "What it takes to serve
 * it").  Pure function of (cfg, T).
 * Errors: MOE_ERR_INVALID_ARG (cfg or bytes NULL, T out of range), or the
 * shape's error from moe_layer_create. */
int moe_layer_workspace_size(const moe_layer_config* cfg, int32_t T, size_t* bytes);

/* The same figure as a plain return value: the workspace bytes a forward over
 * T tokens needs, or 0 when cfg is NULL or invalid or T is out of range. */
size_t moe_layer_workspace_bytes(const moe_layer_config* cfg, int32_t T);

/* The forward pass (the formula at the top of this file: Moat page, "How the
 * router picks 16 of 896", Fig. 2, with the latent path of "Sparse
 * computation: latent experts and routing"): y[T][d] (fp32, fully overwritten)
 * from x[T][d] (fp32).
 * ws must be a device buffer of at least moe_layer_workspace_size(T) bytes,
 * 256-byte aligned; it is scratch owned by the caller and must not be shared
 * by two forwards in flight at once.  T == 0 returns MOE_OK and launches
 * nothing.  trace may be NULL.
 * Errors: MOE_ERR_INVALID_ARG (null handle/x/y, T < 0 or T > max_tokens),
 * MOE_ERR_WORKSPACE (ws NULL, misaligned or too small), MOE_ERR_HIP (a launch
 * failed; the stream's contents are then undefined). */
int moe_layer_forward(moe_layer_t layer, const float* x, int32_t T, float* y,
                      void* ws, size_t ws_bytes, void* stream, const moe_layer_trace* trace);

/* Largest workspace moe_layer_forward_noalloc takes from the library's static
 * scratch: 96 MiB, enough for the Kimi-K3-width forward of up to 192 tokens. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* moe_layer_forward for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc: the same forward (same kernels, same results), with its
 * workspace taken from a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.  It
 * calls no hipMalloc, hipFree or other allocating routine.  The first call on
 * a device looks that device's array up (make one call there before capturing
 * a graph).  All calls on one GPU share its array, which keeps the last
 * call's intermediates: calls that overlap on one GPU (other streams, other
 * threads, other handles) race and must be ordered by the caller.  Nothing in
 * the array needs clearing between calls.
 * Errors: as moe_layer_forward; MOE_ERR_WORKSPACE when the forward over T
 * tokens needs more than MOE_NOALLOC_SCRATCH_BYTES (moe_layer_workspace_size
 * gives the need); MOE_ERR_HIP when the array cannot be found on the current
 * device. */
int moe_layer_forward_noalloc(moe_layer_t layer, const float* x, int32_t T, float* y, void* stream,
                              const moe_layer_trace* trace);

/* Free the host-side handle (the weights are not touched).  NULL is a no-op. */
int moe_layer_destroy(moe_layer_t layer);

/* MX block quantisation of an fp32 matrix in[rows][K] (Four Bits at a Time,
 * "Four bits from the start": shared exponent floor(log2(amax)) - emax,
 * elements rounded to nearest, ties to even, saturating; scale clamped to the
 * E8M0 range).  fmt 0 = E4M3 (codes [rows][K]), 1 = E2M1 (packed codes
 * [rows][K/2]); scales [rows][K/32].  K must be a positive multiple of 32.
 * Used by the forward for activations and by callers to encode weights. */
int moe_mx_quantize(const float* in, int64_t rows, int32_t K, int32_t fmt,
                    uint8_t* codes, uint8_t* scales, void* stream);

/* MX E2M1 quantisation of G weight matrices in[G*N][K] (fp32, row-major),
 * written in fragment order (codes G*N*K/2 bytes, scales G*N*K/32 bytes): the
 * same codes and scales as moe_mx_quantize with fmt 1, permuted.  N must be a
 * positive multiple of 16 and K of 128; G >= 0.
 * Errors: MOE_ERR_INVALID_ARG (sizes, null or misaligned pointers: in 16-byte,
 * codes 2-byte aligned), MOE_ERR_HIP. */
int moe_mx_quantize_weights(const float* in, int64_t G, int32_t N, int32_t K,
                            uint8_t* codes, uint8_t* scales, void* stream);

/* Convert G row-major E2M1 matrices (codes [G*N][K/2], scales [G*N][K/32])
 * into fragment order (out_codes, out_scales; same sizes, must not overlap the
 * inputs).  N % 16 == 0, K % 128 == 0.  Codes buffers 16-byte aligned, scale
 * buffers 4-byte aligned.  Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP. */
int moe_mx_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t G, int32_t N, int32_t K,
                        uint8_t* out_codes, uint8_t* out_scales, void* stream);

/* fp32 -> bfloat16 (round to nearest, ties to even; finite inputs), n values;
 * n % 4 == 0, in 16-byte and out 8-byte aligned.  The forward's rounding of
 * x under the higher-precision map; callers use it to encode bfloat16 weights.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP. */
int moe_round_bf16(const float* in, int64_t n, uint16_t* out, void* stream);

/* Quantile Balancing of the selection bias from one batch of router logits.
 * The pages ("Kimi K3 and the New Open-Weights Moat: Inference Efficiency",
 * "How the router picks 16 of 896", Fig. 2 and the paragraph after it; "What
 * Kimi K3 asks of the hardware", "Width: 896 experts and the interconnect")
 * say only that each expert's bias is updated from the distribution of its
 * score margins so that its routed count approaches a target load.  Reading:
 * key = sigmoid(logit) + bias; an expert's margin on a token is its key minus
 * the k-th largest key among the token's other experts; n = round(T*k/E) (ties to even)
 * clamped to [1, T-1]; Q[e] = midpoint of expert e's n-th and (n+1)-th
 * largest margins over the batch; bias_out = bias_in - eta * Q.
 * logits: device fp32 [T][E] (the router's logits, before the sigmoid);
 * bias_in / bias_out: device fp32 [E] (may be the same buffer); quantile_out:
 * device fp32 [E] or NULL; 2 <= T, 1 <= k < E <= 4096, 0 < eta <= 1.
 * ws: device buffer of moe_quantile_balance_workspace_bytes(T, E) bytes,
 * 16-byte aligned, owned by the caller.  Asynchronous on `stream`.
 * Errors: MOE_ERR_INVALID_ARG (sizes, eta, null or misaligned pointers),
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
size_t moe_quantile_balance_workspace_bytes(int32_t T, int32_t E);
int moe_quantile_balance(const float* logits, int32_t T, int32_t E, int32_t k, const float* bias_in, float eta,
                         float* bias_out, float* quantile_out, void* ws, size_t ws_bytes, void* stream);

/* Measurement, not part of the layer: the block-scaled FP8 x FP4 matrix-core
 * rate of this GPU.  `workgroups` x 4 waves each issue 8 * iters independent
 * 16x16x128 E4M3 x E2M1 MFMAs (2 * 16 * 16 * 128 flops each) on operands of
 * 1.0; out (device fp32 [workgroups * 4]) receives one checksum per wave
 * (a sum of accumulators, not meant to be read).  Time it with
 * events on `stream`.  1 <= iters <= 2^24, 1 <= workgroups <= 2^20.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP. */
int moe_mfma_rate_probe(int32_t iters, int32_t workgroups, float* out, void* stream);

/* Measurement, not part of the layer: how fast this GPU streams HBM with plain
 * 16-byte non-temporal loads (the decode expert GEMMs' whole job is such a
 * stream of weights).  Reads `bytes` (a positive multiple of 16) from the
 * device buffer buf (16-byte aligned) with `workgroups` x 256 threads;
 * out (device uint32 [workgroups * 256]) receives one fold of the data per
 * thread, not meant to be read.  Time it with events on `stream`.
 * 1 <= workgroups <= 2^20.  Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP. */
int moe_hbm_read_probe(const void* buf, size_t bytes, int32_t workgroups, uint32_t* out, void* stream);

/* Dense MX GEMM c[M][N] = deq(a) deq(b)^T in fp32, a = E4M3 [M][K] (row-major),
 * b = E2M1 [N][K] in fragment order, N a positive multiple of 16, K of 128.
 * This is the block-scaled matrix-core kernel the layer's projections run on,
 * exposed for stage-level checks. */
int moe_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                const uint8_t* b_scales, int32_t M, int32_t N, int32_t K, float* c, void* stream);

/* The router's top-k selection (Kimi K3 and the New Open-Weights Moat, "How
 * the router picks 16 of 896", Fig. 2), exposed for stage-level checks: per
 * token t, score = sigmoid(logit) (softmax_gates = 0) or the logit itself
 * (softmax_gates != 0); key = score + selection_bias[e] (NULL: zeros), NaN
 * and -inf keys ranking last; ids[t][0..k) = the k best experts by (key
 * descending, id ascending), in that order; gates = the winners' scores over
 * their sum in slot order, or the softmax of the winners' logits.
 * logits: device fp32 [T][E]; ids: device int32 [T][k]; gates: device fp32
 * [T][k].  1 <= k <= min(E, 64), E <= 4096.  Asynchronous on `stream`.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP. */
int moe_router_topk(const float* logits, const float* selection_bias, int32_t T, int32_t E, int32_t k,
                    int32_t softmax_gates, int32_t* ids, float* gates, void* stream);

/* The same selection on the router's K-slice partial sums, as the layer runs
 * it for few tokens: logits[t][e] = (partial[0][t][e] + partial[1][t][e] +
 * ... + partial[nz-1][t][e], added in that order in fp32) + logit_bias[e]
 * (NULL: + 0), written to `logits`, then the top-k above.  partial: device
 * fp32 [nz][T][E], 1 <= nz; E <= 1024; other arguments as above. */
int moe_router_reduce_topk(const float* partial, int32_t nz, const float* logit_bias, const float* selection_bias,
                           int32_t T, int32_t E, int32_t k, int32_t softmax_gates, float* logits, int32_t* ids,
                           float* gates, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_H */
