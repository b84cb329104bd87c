// moe_layer.hip -- the C ABI: validation, workspace plan and the launch sequence
// of one LatentMoE forward on a single HIP stream.
//
// Launch sequence (all asynchronous, no host synchronisation, no allocation):
//   1. quantise x to MXFP8                                   mx_quant
//   2. z = xq W_down^T (fp32) and zq = MXFP8(z)               bf16 GEMM on exactly decoded MX
//                                                             operands (dense, F32_QUANT)
//   3. logits = z W_router^T + logit_bias                     router_logits (fp32 MFMA)
//   4. ids, gates = top-k(sigmoid + selection bias)           topk
//   5. counts, offsets, stable permutation, M-tile prefix     dispatch (count/scan/scatter)
//   6. hq = MXFP8(SiLU(zq_e W_gate_e^T) * (zq_e W_up_e^T))    mx_gemm (grouped, SWIGLU_QUANT,
//                                                             rows gathered through the permutation)
//   7. y_e = hq_e W_down_e^T                                  mx_gemm (grouped, F32)
//   8. y_lat = sum_j gate_j y_e[row(t,j)], yq = MXFP8(y_lat)   combine
//   9. hs_s = MXFP8(SiLU(xq W_gate_s^T) * (xq W_up_s^T))      mx_gemm (dense groups, SWIGLU_QUANT)
//  10. y = yq W_up^T + sum_s hs_s W_down_s^T                  mx_gemm (dense, 1+S K-segments)
// Step 10 runs the up-projection and every shared down-projection as one
// GEMM whose K dimension is the concatenation [L | Fs | Fs ...], so the sum of
// the routed and shared branches (Moat page, Fig. 2) happens in the fp32
// accumulators instead of an extra pass over y.  With MX weights and few
// rows (weight-streaming kernels) the shared experts ride in the routed
// experts' launches instead: step 9 in the workgroups of step 6 that come
// before the routed ones, the shared down-projections in step 7's (writing
// y), and step 10 adds only the up-projection to y.  With many rows, steps 8
// and 9 share one launch (the combine on some of the GEMM's workgroups).
//
// Higher-precision map (dense_bf16): step 1 rounds x to bf16 (xb), and steps
// 2, 9 and 10 are bf16 GEMMs on bfloat16 weights (LDS-staged 512-thread
// kernel for many tokens, K-split weight streaming plus a reduce for few);
// the combine writes bf16(y_lat) and the shared hidden state is bf16.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "../../include/moe_layer.h"
#include "kernels.hpp"

struct moe_layer {
  moe_layer_config cfg;
  moe_layer_weights w;
};

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kFewRows = 256;  // decode-shaped batches: weight-streaming kernels

inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Plan {
  size_t xq, xqs, xdq, wdn16, zpart, z, zq, zqs, logits, rpart, wrpl, ids, gates, dscr, counts, offsets, ms0, ms1,
      tg0, tg1, rop, por, hq, hqs, ye, ylat, yq, yqs, hs, hss, xb, yb, hb, dpart, total;
};

// The bf16 GEMMs of the higher-precision map (operand pointers left null:
// the shapes alone decide the K-slice plan and the partial-sum buffer).
moe::GemmArgs hp_down_args(const moe_layer_config& c, int T) {
  moe::GemmArgs a = {};
  a.nseg = 1;
  a.seg[0].K = a.seg[0].lda = c.d_model;
  a.G = 1;
  a.M = T;
  a.N = c.d_latent;
  return a;
}
// Shared gate/up; split-K form: N = 2 Fs partial columns (gate, then up).
moe::GemmArgs hp_shared_args(const moe_layer_config& c, int T, bool split) {
  moe::GemmArgs a = {};
  a.nseg = 1;
  a.seg[0].K = a.seg[0].lda = c.d_model;
  a.seg[0].b_gstride = (int64_t)c.d_ff_shared * c.d_model * 2;
  a.G = c.n_shared;
  a.M = T;
  a.N = split ? 2 * c.d_ff_shared : c.d_ff_shared;
  return a;
}
// Up-projection and shared down-projections, K = [L | Fs | Fs ...].
moe::GemmArgs hp_out_args(const moe_layer_config& c, int T) {
  moe::GemmArgs a = {};
  a.nseg = 1 + c.n_shared;
  a.seg[0].K = a.seg[0].lda = c.d_latent;
  for (int i = 0; i < c.n_shared; ++i) a.seg[1 + i].K = a.seg[1 + i].lda = c.d_ff_shared;
  a.G = 1;
  a.M = T;
  a.N = c.d_model;
  return a;
}
size_t splitk_floats(const moe::GemmArgs& a) { return (size_t)moe::splitk_plan(a).n * a.G * a.M * a.N; }

Plan make_plan(const moe_layer_config& c, int64_t T) {
  const int64_t d = c.d_model, L = c.d_latent, E = c.n_routed, k = c.top_k, F = c.d_ff_routed,
                S = c.n_shared, Fs = c.n_shared > 0 ? c.d_ff_shared : 0;
  const int64_t P = T * k;
  Plan p;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  // Without a latent (second workload) nothing of the latent path exists:
  // the router reads x, the experts read xq and the combine writes y.
  const int64_t lat = c.identity_latent ? 0 : 1;
  // Higher-precision map: no MXFP8 copy of x, of y_lat or of the shared
  // hidden state; bf16 ones instead.
  const int64_t hp = c.dense_bf16 ? 1 : 0, mxd = 1 - hp;
  p.xq = take(mxd * T * d);
  p.xqs = take(mxd * T * d / 32);
  p.xdq = take(mxd * lat * T * d * 2);
  // Latent down-projection: at most kFewRows tokens stream the MXFP4 weights
  // (K-slice partial sums), more tokens use a bf16 image of W_down.
  const bool few = T <= kFewRows;
  p.wdn16 = take(few ? 0 : mxd * lat * L * d * 2);
  p.zpart =
      take(few && T > 0 ? (size_t)mxd * lat * moe::bf16_mx_splitk_slices((int)T, (int)L, (int)d) * T * L * 4 : 0);
  p.xb = take(hp * T * d * 2);
  p.yb = take(hp * T * L * 2);
  p.hb = take(hp * S * T * Fs * 2);
  {
    size_t f = 0;
    if (hp && few && T > 0) {
      f = splitk_floats(hp_down_args(c, (int)T));
      if (S > 0) {
        const size_t f2 = splitk_floats(hp_shared_args(c, (int)T, true));
        f = f2 > f ? f2 : f;
      }
      const size_t f3 = splitk_floats(hp_out_args(c, (int)T));
      f = f3 > f ? f3 : f;
    }
    p.dpart = take(f * 4);  // K-slice partial sums of the few-row bf16 GEMMs (used one at a time)
  }
  p.z = take(lat * T * L * 4);
  p.zq = take(lat * T * L);
  p.zqs = take(lat * T * L / 32);
  p.logits = take(T * E * 4);
  {
    const int split = T > 0 ? moe::router_split((int)T, (int)E, (int)L) : 1;
    p.rpart = take(split > 1 ? (size_t)split * T * E * 4 : 0);  // router K-slice partial sums
    // bf16 pieces of the router weight (many-token router)
    p.wrpl = take(T > 0 && moe::router_bf16x3((int)T, (int)E, (int)L) ? (size_t)3 * E * L * 2 : 0);
  }
  p.ids = take(P * 4);
  p.gates = take(P * 4);
  p.dscr = take(moe::dispatch_scratch_ints((int)T, (int)E) * 4);
  p.counts = take(E * 4);
  p.offsets = take((E + 1) * 4);
  p.ms0 = take((E + 1) * 4);
  p.ms1 = take((E + 1) * 4);
  {  // group of each M-tile of the routed GEMMs: at most P / mt + min(P, E) tiles
    const size_t mt0 = (size_t)moe::gemm_mtile(moe::GEMM_STREAM16), mt1 = (size_t)moe::gemm_mtile(moe::GEMM_WIDE);
    const size_t pe = P < (size_t)E ? P : (size_t)E;
    p.tg0 = take(P <= (size_t)16 * E ? (P / mt0 + pe + 1) * 4 : 0);  // weight-streaming shape only
    p.tg1 = take((P / mt1 + pe + 1) * 4);
  }
  p.rop = take(P * 4);
  p.por = take(P * 4);
  p.hq = take(P * F);
  p.hqs = take(P * F / 32);
  p.ye = take(P * L * 4);
  p.ylat = take(lat * T * L * 4);
  p.yq = take(mxd * lat * T * L);
  p.yqs = take(mxd * lat * T * L / 32);
  p.hs = take(mxd * S * T * Fs);
  p.hss = take(mxd * S * T * Fs / 32);
  p.total = o;
  return p;
}

int check_config(const moe_layer_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->d_model <= 0 || c->d_latent <= 0 || c->d_ff_routed <= 0 || c->n_routed <= 0 || c->top_k <= 0 ||
      c->n_shared < 0 || c->max_tokens <= 0)
    return MOE_ERR_INVALID_ARG;
  if (c->top_k > c->n_routed || c->n_shared > 8 || c->max_tokens > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (c->n_shared > 0 && c->d_ff_shared <= 0) return MOE_ERR_INVALID_ARG;
  if (c->identity_latent && c->d_latent != c->d_model) return MOE_ERR_INVALID_ARG;
  if (c->dense_bf16 && c->identity_latent) return MOE_ERR_UNSUPPORTED;  // the map is the latent layer's
  if (c->weight_layout != MOE_WEIGHTS_ROW_MAJOR && c->weight_layout != MOE_WEIGHTS_FRAGMENT) return MOE_ERR_INVALID_ARG;
  if (c->n_routed > 4096 || c->top_k > 64) return MOE_ERR_UNSUPPORTED;
  if (c->d_model % 128 || c->d_latent % 128 || c->d_ff_routed % 128) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && c->d_ff_shared % 128) return MOE_ERR_UNSUPPORTED;
  if (c->d_model > (1 << 16) || c->d_latent > (1 << 16) || c->d_ff_routed > (1 << 16) ||
      (c->n_shared > 0 && c->d_ff_shared > (1 << 16)))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline bool mx_ok(const moe_mx_tensor& t) { return t.codes != nullptr && t.scales != nullptr; }

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline bool mx_aligned(const moe_mx_tensor& t) { return aligned(t.codes, 16) && aligned(t.scales, 4); }

template <class T>
inline T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported layer shape";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int moe_layer_create(const moe_layer_config* cfg, const moe_layer_weights* w, moe_layer_t* out) {
  if (!cfg || !w || !out) return MOE_ERR_INVALID_ARG;
  int st = check_config(cfg);
  if (st != MOE_OK) return st;
  const bool latent = !cfg->identity_latent;
  const bool hp = cfg->dense_bf16 != 0;
  const bool mx_dense = latent && !hp, shared = cfg->n_shared > 0;
  if ((mx_dense && (!mx_ok(w->w_down) || !mx_ok(w->w_up))) || !w->w_router || !mx_ok(w->w_gate_e) ||
      !mx_ok(w->w_up_e) || !mx_ok(w->w_down_e))
    return MOE_ERR_INVALID_ARG;
  if (shared && !hp && (!mx_ok(w->w_gate_s) || !mx_ok(w->w_up_s) || !mx_ok(w->w_down_s)))
    return MOE_ERR_INVALID_ARG;
  if ((mx_dense && (!mx_aligned(w->w_down) || !mx_aligned(w->w_up))) || !mx_aligned(w->w_gate_e) ||
      !mx_aligned(w->w_up_e) || !mx_aligned(w->w_down_e) || !aligned(w->w_router, 16))
    return MOE_ERR_INVALID_ARG;
  if (shared && !hp && (!mx_aligned(w->w_gate_s) || !mx_aligned(w->w_up_s) || !mx_aligned(w->w_down_s)))
    return MOE_ERR_INVALID_ARG;
  if (hp) {
    auto ok16 = [](const void* p) { return p != nullptr && aligned(p, 16); };
    if (!ok16(w->w_down_bf16) || !ok16(w->w_up_bf16)) return MOE_ERR_INVALID_ARG;
    if (shared && (!ok16(w->w_gate_s_bf16) || !ok16(w->w_up_s_bf16) || !ok16(w->w_down_s_bf16)))
      return MOE_ERR_INVALID_ARG;
  }
  moe_layer* h = new (std::nothrow) moe_layer;
  if (!h) return MOE_ERR_INVALID_ARG;
  h->cfg = *cfg;
  h->w = *w;
  *out = h;
  return MOE_OK;
}

int moe_layer_workspace_size(const moe_layer_config* cfg, int32_t T, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  int st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > cfg->max_tokens) return MOE_ERR_INVALID_ARG;
  *bytes = make_plan(*cfg, T).total;
  return MOE_OK;
}

size_t moe_layer_workspace_bytes(const moe_layer_config* cfg, int32_t T) {
  size_t bytes = 0;
  return moe_layer_workspace_size(cfg, T, &bytes) == MOE_OK ? bytes : 0;
}

int moe_layer_destroy(moe_layer_t layer) {
  delete layer;
  return MOE_OK;
}

#define MOE_HIP(expr)                                 \
  do {                                                \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;     \
  } while (0)

}  // extern "C"

namespace {

// The forward over a validated layer, T > 0, and a workspace of at least the
// plan's size (aligned to kAlign).  Every byte of the workspace that a kernel
// reads was written earlier in the same forward, so nothing needs clearing.
int forward_impl(moe_layer_t layer, const float* x, int32_t T, float* y, void* ws, void* stream,
                 const moe_layer_trace* tr) {
  const moe_layer_config& c = layer->cfg;
  const Plan pl = make_plan(c, T);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_layer_weights& w = layer->w;
  const int d = c.d_model, L = c.d_latent, E = c.n_routed, k = c.top_k, F = c.d_ff_routed, S = c.n_shared,
            Fs = c.d_ff_shared;
  const int64_t P = (int64_t)T * k;

  uint8_t* xq = at<uint8_t>(ws, pl.xq);
  uint8_t* xqs = at<uint8_t>(ws, pl.xqs);
  uint16_t* xdq = at<uint16_t>(ws, pl.xdq);
  uint16_t* wdn16 = at<uint16_t>(ws, pl.wdn16);
  float* zpart = at<float>(ws, pl.zpart);
  float* z = at<float>(ws, pl.z);
  uint8_t* zq = at<uint8_t>(ws, pl.zq);
  uint8_t* zqs = at<uint8_t>(ws, pl.zqs);
  float* logits = at<float>(ws, pl.logits);
  int32_t* ids = at<int32_t>(ws, pl.ids);
  float* gates = at<float>(ws, pl.gates);
  int32_t* dscr = at<int32_t>(ws, pl.dscr);
  int32_t* counts = at<int32_t>(ws, pl.counts);
  int32_t* offsets = at<int32_t>(ws, pl.offsets);
  int32_t* ms0 = at<int32_t>(ws, pl.ms0);
  int32_t* ms1 = at<int32_t>(ws, pl.ms1);
  int32_t* tg0 = at<int32_t>(ws, pl.tg0);
  int32_t* tg1 = at<int32_t>(ws, pl.tg1);
  int32_t* rop = at<int32_t>(ws, pl.rop);
  int32_t* por = at<int32_t>(ws, pl.por);
  uint8_t* hq = at<uint8_t>(ws, pl.hq);
  uint8_t* hqs = at<uint8_t>(ws, pl.hqs);
  float* ye = at<float>(ws, pl.ye);
  float* ylat = at<float>(ws, pl.ylat);
  uint8_t* yq = at<uint8_t>(ws, pl.yq);
  uint8_t* yqs = at<uint8_t>(ws, pl.yqs);
  uint8_t* hs = at<uint8_t>(ws, pl.hs);
  uint8_t* hss = at<uint8_t>(ws, pl.hss);
  uint16_t* xb = at<uint16_t>(ws, pl.xb);
  uint16_t* yb = at<uint16_t>(ws, pl.yb);
  uint16_t* hb = at<uint16_t>(ws, pl.hb);
  float* dpart = at<float>(ws, pl.dpart);
  const bool hp = c.dense_bf16 != 0;
  const bool few = T <= kFewRows;
  const int wrm = c.weight_layout == MOE_WEIGHTS_ROW_MAJOR ? 1 : 0;  // MX weights row-major [out][in]
  auto u8 = [](const void* p) { return reinterpret_cast<const uint8_t*>(p); };

  // Kernel shapes: weight streaming when a group has few rows (decode), the
  // LDS-staged 512-thread kernels otherwise.
  const int dense_shape = T <= kFewRows ? moe::GEMM_STREAM16 : moe::GEMM_WIDE;
  const int routed_shape = P <= (int64_t)16 * E ? moe::GEMM_STREAM16 : moe::GEMM_WIDE;
  const int mt_dense = moe::gemm_mtile(dense_shape);
  const int mt_small = moe::gemm_mtile(moe::GEMM_STREAM16), mt_big = moe::gemm_mtile(moe::GEMM_WIDE);

  hipEvent_t const* ev = tr && tr->events ? reinterpret_cast<hipEvent_t const*>(tr->events) : nullptr;
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], s) : hipSuccess; };
  MOE_HIP(mark(MOE_EV_START));

  // 1. xq (and its exact bf16 image for the latent down-projection)
  const bool latent = !c.identity_latent;
  if (hp) MOE_HIP(moe::launch_round_bf16(x, (int64_t)T * d, xb, s));
  else MOE_HIP(moe::launch_quantize(x, T, d, 0, xq, xqs, s, latent ? xdq : nullptr));
  MOE_HIP(mark(MOE_EV_QUANT_X));
  // What the router and the routed experts read: the latent, or x itself.
  const float* zr = latent ? z : x;
  const uint8_t* zqa = latent ? zq : xq;
  const uint8_t* zqsa = latent ? zqs : xqs;

  // 2. z, zq: bf16 matrix cores on the exactly decoded MX operands, so that the
  //    latent the router ranks is accurate to fp32 accumulation.  Few tokens:
  //    W_down is decoded in registers while it streams (K-slice partials, then
  //    their sum and MXFP8); many tokens: one bf16 image, then the LDS kernel.
  if (!latent) {
    // no latent projection
  } else if (hp) {  // bfloat16 W_down on bf16(x)
    moe::GemmArgs a = hp_down_args(c, T);
    a.seg[0].a = u8(xb);
    a.seg[0].b = u8(w.w_down_bf16);
    if (few) {
      const moe::SplitPlan sp = moe::splitk_plan(a);
      MOE_HIP(moe::launch_bf16_splitk(a, true, sp, dpart, s));
      MOE_HIP(moe::launch_splitk_reduce(dpart, sp.n, T, L, z, zq, zqs, s));
    } else {
      a.c = z;
      a.ldc = L;
      a.q = zq;
      a.qs = zqs;
      a.max_mtiles = (T + moe::gemm_mtile(moe::GEMM_WIDE) - 1) / moe::gemm_mtile(moe::GEMM_WIDE);
      MOE_HIP(moe::launch_bf16_gemm_wide(a, moe::EPI_F32_QUANT, s));
    }
  } else if (T <= kFewRows) {
    moe::GemmArgs a = {};
    a.nseg = 1;
    a.seg[0] = {reinterpret_cast<const uint8_t*>(xdq), nullptr, d, w.w_down.codes, w.w_down.scales,
                nullptr, nullptr, 0, 0, d, wrm};
    a.G = 1;
    a.M = T;
    a.N = L;
    a.ldc = L;
    MOE_HIP(moe::launch_bf16_mx_splitk(a, zpart, moe::bf16_mx_splitk_slices(T, L, d), z, zq, zqs, s));
  } else {
    MOE_HIP(moe::launch_decode_e2m1_bf16(w.w_down.codes, w.w_down.scales, L, d, wdn16, s, 1 - wrm));
    moe::GemmArgs a = {};
    a.nseg = 1;
    a.seg[0] = {reinterpret_cast<const uint8_t*>(xdq), nullptr, d, reinterpret_cast<const uint8_t*>(wdn16),
                nullptr, nullptr, nullptr, 0, 0, d};
    a.G = 1;
    a.M = T;
    a.N = L;
    a.c = z;
    a.ldc = L;
    a.q = zq;
    a.qs = zqs;
    a.max_mtiles = (T + moe::gemm_mtile(moe::GEMM_WIDE) - 1) / moe::gemm_mtile(moe::GEMM_WIDE);
    MOE_HIP(moe::launch_bf16_gemm_quant(a, moe::GEMM_WIDE, s));
  }
  MOE_HIP(mark(MOE_EV_DOWN));

  // 3-4. router
  // (few tokens: the K-slice sums of the logits are added by the top-k kernel)
  const bool reduce_in_topk = moe::router_reduce_in_topk(T, E, L);
  MOE_HIP(moe::launch_router_logits(zr, w.w_router, w.router_logit_bias, T, E, L, logits,
                                    at<float>(ws, pl.rpart), at<uint16_t>(ws, pl.wrpl), s, reduce_in_topk));
  MOE_HIP(mark(MOE_EV_LOGITS));
  if (reduce_in_topk)
    MOE_HIP(moe::launch_router_reduce_topk(at<float>(ws, pl.rpart), moe::router_slices(T, E, L),
                                           w.router_logit_bias, w.selection_bias, T, E, k, c.softmax_gates != 0,
                                           logits, ids, gates, s));
  else
    MOE_HIP(moe::launch_topk(logits, w.selection_bias, T, E, k, c.softmax_gates != 0, ids, gates, s));
  MOE_HIP(mark(MOE_EV_TOPK));

  // 5. dispatch
  MOE_HIP(moe::launch_dispatch(ids, T, E, k, dscr, counts, offsets, rop, por, mt_small, ms0,
                               routed_shape == moe::GEMM_STREAM16 ? tg0 : nullptr, mt_big, ms1, tg1, s));
  MOE_HIP(mark(MOE_EV_DISPATCH));

  const int mt_r = moe::gemm_mtile(routed_shape);
  const int32_t* ms_r = routed_shape == moe::GEMM_STREAM16 ? ms0 : ms1;
  const int64_t max_mt_r = P / mt_r + (P < E ? P : E) + 1;

  // The shared experts' gate/up GEMM (step 9) on MX weights, as arguments.
  auto shared_up_args = [&]() {
    moe::GemmArgs a = {};
    a.nseg = 1;
    a.seg[0] = {xq,
                xqs,
                d,
                w.w_gate_s.codes,
                w.w_gate_s.scales,
                w.w_up_s.codes,
                w.w_up_s.scales,
                (int64_t)Fs * d / 2,
                (int64_t)Fs * d / 32,
                d,
                wrm};
    a.G = S;
    a.M = T;
    a.N = Fs;
    a.c = tr ? tr->hs : nullptr;
    a.ldc = Fs;
    a.c_gstride = (int64_t)T * Fs;
    a.q = hs;
    a.qs = hss;
    a.q_gstride = (int64_t)T * Fs;
    a.qs_gstride = (int64_t)T * Fs / 32;
    a.max_mtiles = S * ((T + mt_dense - 1) / mt_dense);
    return a;
  };
  // The shared experts' down-projections (the K segments of step 10 after
  // the latent one): y = sum_s hs_s W_down_s^T.
  auto shared_down_args = [&]() {
    moe::GemmArgs a = {};
    a.nseg = S;
    for (int i = 0; i < S; ++i)
      a.seg[i] = {hs + (int64_t)i * T * Fs,
                  hss + (int64_t)i * T * Fs / 32,
                  Fs,
                  w.w_down_s.codes + (int64_t)i * d * Fs / 2,
                  w.w_down_s.scales + (int64_t)i * d * Fs / 32,
                  nullptr,
                  nullptr,
                  0,
                  0,
                  Fs,
                  wrm};
    a.G = 1;
    a.M = T;
    a.N = d;
    a.c = y;
    a.ldc = d;
    a.max_mtiles = (T + mt_dense - 1) / mt_dense;
    return a;
  };
  // Few rows: every GEMM after the router streams its weights, so the
  // shared experts' halves (which need only x, then hs) run in the routed
  // experts' launches -- gate/up with step 6, the down-projections with step
  // 7 (y = shared part, to which step 10 adds the up-projection) -- rather
  // than in launches of their own bound by memory latency.
  const bool shared_with_routed =
      !hp && S > 0 && dense_shape == moe::GEMM_STREAM16 && routed_shape == moe::GEMM_STREAM16;

  // 6. routed GEMM1 + SwiGLU + MXFP8 (+ the shared experts' gate/up)
  {
    moe::GemmArgs a = {};
    a.nseg = 1;
    a.seg[0] = {zqa,
                zqsa,
                L,
                w.w_gate_e.codes,
                w.w_gate_e.scales,
                w.w_up_e.codes,
                w.w_up_e.scales,
                (int64_t)F * L / 2,
                (int64_t)F * L / 32,
                L,
                wrm};
    a.offsets = offsets;
    a.mtile_start = ms_r;
    a.mtile_group = routed_shape == moe::GEMM_STREAM16 ? tg0 : tg1;
    a.G = E;
    a.N = F;
    a.gather = por;
    a.gather_div = k;
    a.c = tr ? tr->h : nullptr;
    a.ldc = F;
    a.q = hq;
    a.qs = hqs;
    a.max_mtiles = (int)max_mt_r;
    if (shared_with_routed) MOE_HIP(moe::launch_mx_gemm_pair(shared_up_args(), a, moe::EPI_SWIGLU_QUANT, s));
    else MOE_HIP(moe::launch_mx_gemm(a, moe::EPI_SWIGLU_QUANT, routed_shape, s));
  }
  MOE_HIP(mark(MOE_EV_EXPERT_UP));

  // 7. routed GEMM2
  {
    moe::GemmArgs a = {};
    a.nseg = 1;
    a.seg[0] = {hq, hqs, F, w.w_down_e.codes, w.w_down_e.scales, nullptr, nullptr, (int64_t)L * F / 2,
                (int64_t)L * F / 32, F, wrm};
    a.offsets = offsets;
    a.mtile_start = ms_r;
    a.mtile_group = routed_shape == moe::GEMM_STREAM16 ? tg0 : tg1;
    a.G = E;
    a.N = L;
    a.c = ye;
    a.ldc = L;
    a.max_mtiles = (int)max_mt_r;
    if (shared_with_routed && latent) MOE_HIP(moe::launch_mx_gemm_pair(shared_down_args(), a, moe::EPI_F32, s));
    else MOE_HIP(moe::launch_mx_gemm(a, moe::EPI_F32, routed_shape, s));
  }
  MOE_HIP(mark(MOE_EV_EXPERT_DOWN));

  // 8. combine
  // The fp32 combined latent is only kept for a trace; yq is what the
  // up-projection reads.  Many tokens with MX shared experts: the combine
  // (HBM-bound) runs in the same launch as the shared gate/up GEMM (matrix
  // cores), on a fraction of its workgroups.
  const bool combine_with_shared = !hp && latent && S > 0 && dense_shape == moe::GEMM_WIDE;
  if (combine_with_shared) {
    moe::GemmArgs a = shared_up_args();
    const moe::CombineArgs cb = {ye, gates, rop, (int)T, k, L, tr && tr->y_lat ? ylat : nullptr, yq, yqs};
    MOE_HIP(moe::launch_mx_gemm_wide_combine(a, cb, s));
  } else if (hp) {
    MOE_HIP(moe::launch_combine(ye, gates, rop, T, k, L, tr && tr->y_lat ? ylat : nullptr, nullptr, nullptr, s, yb));
  } else if (latent) {
    MOE_HIP(moe::launch_combine(ye, gates, rop, T, k, L, tr && tr->y_lat ? ylat : nullptr, yq, yqs, s));
  } else {  // the routed output at model width goes straight to y
    MOE_HIP(moe::launch_combine(ye, gates, rop, T, k, L, y, nullptr, nullptr, s));
    if (tr && tr->y_lat) MOE_HIP(hipMemcpyAsync(tr->y_lat, y, (size_t)T * L * 4, hipMemcpyDeviceToDevice, s));
  }
  MOE_HIP(mark(MOE_EV_COMBINE));

  // 9. shared experts, first half (with MX weights at few rows: in step 6's launch)
  if (S > 0 && hp) {  // bfloat16 gate/up on bf16(x), hidden state rounded to bf16
    moe::GemmArgs a = hp_shared_args(c, T, few);
    a.seg[0].a = u8(xb);
    a.seg[0].b = u8(w.w_gate_s_bf16);
    a.seg[0].b2 = u8(w.w_up_s_bf16);
    if (few) {
      const moe::SplitPlan sp = moe::splitk_plan(a);
      MOE_HIP(moe::launch_bf16_splitk(a, true, sp, dpart, s));
      MOE_HIP(moe::launch_splitk_swiglu(dpart, sp.n, S, T, Fs, tr ? tr->hs : nullptr, hb, s));
    } else {
      a.c = tr ? tr->hs : nullptr;
      a.ldc = Fs;
      a.c_gstride = (int64_t)T * Fs;
      a.ob = hb;
      a.ob_gstride = (int64_t)T * Fs;
      a.max_mtiles = S * ((T + moe::gemm_mtile(moe::GEMM_WIDE) - 1) / moe::gemm_mtile(moe::GEMM_WIDE));
      MOE_HIP(moe::launch_bf16_gemm_wide(a, moe::EPI_SWIGLU_BF16, s));
    }
  } else if (S > 0 && !shared_with_routed && !combine_with_shared) {
    moe::GemmArgs a = shared_up_args();
    a.kchains = dense_shape == moe::GEMM_STREAM16 ? 4 : 1;  // few rows: K split over each workgroup's waves
    MOE_HIP(moe::launch_mx_gemm(a, moe::EPI_SWIGLU_QUANT, dense_shape, s));
  }
  MOE_HIP(mark(MOE_EV_SHARED_UP));

  // 10. y = up-projection + shared down-projections (one K-concatenated
  //     GEMM); without a latent, y (the routed output) += the shared ones.
  if (hp) {
    moe::GemmArgs a = hp_out_args(c, T);
    a.seg[0].a = u8(yb);
    a.seg[0].b = u8(w.w_up_bf16);
    for (int i = 0; i < S; ++i) {
      a.seg[1 + i].a = u8(hb + (int64_t)i * T * Fs);
      a.seg[1 + i].b = u8(w.w_down_s_bf16 + (int64_t)i * d * Fs);
    }
    if (few) {
      const moe::SplitPlan sp = moe::splitk_plan(a);
      MOE_HIP(moe::launch_bf16_splitk(a, true, sp, dpart, s));
      MOE_HIP(moe::launch_splitk_reduce(dpart, sp.n, T, d, y, nullptr, nullptr, s));
    } else {
      a.c = y;
      a.ldc = d;
      a.max_mtiles = (T + moe::gemm_mtile(moe::GEMM_WIDE) - 1) / moe::gemm_mtile(moe::GEMM_WIDE);
      MOE_HIP(moe::launch_bf16_gemm_wide(a, moe::EPI_F32, s));
    }
  } else if (latent && shared_with_routed) {  // y (the shared part, step 7) += yq W_up^T
    moe::GemmArgs a = {};
    a.nseg = 1;
    a.seg[0] = {yq, yqs, L, w.w_up.codes, w.w_up.scales, nullptr, nullptr, 0, 0, L, wrm};
    a.c_accumulate = 1;
    a.G = 1;
    a.M = T;
    a.N = d;
    a.c = y;
    a.ldc = d;
    a.max_mtiles = (T + mt_dense - 1) / mt_dense;
    a.kchains = 4;
    MOE_HIP(moe::launch_mx_gemm(a, moe::EPI_F32, dense_shape, s));
  } else if (latent || S > 0) {
    moe::GemmArgs a = {};
    const int s0 = latent ? 1 : 0;
    a.nseg = s0 + S;
    if (latent) a.seg[0] = {yq, yqs, L, w.w_up.codes, w.w_up.scales, nullptr, nullptr, 0, 0, L, wrm};
    a.c_accumulate = latent ? 0 : 1;
    for (int i = 0; i < S; ++i)
      a.seg[s0 + i] = {hs + (int64_t)i * T * Fs,
                      hss + (int64_t)i * T * Fs / 32,
                      Fs,
                      w.w_down_s.codes + (int64_t)i * d * Fs / 2,
                      w.w_down_s.scales + (int64_t)i * d * Fs / 32,
                      nullptr,
                      nullptr,
                      0,
                      0,
                      Fs,
                      wrm};
    a.G = 1;
    a.M = T;
    a.N = d;
    a.c = y;
    a.ldc = d;
    a.max_mtiles = (T + mt_dense - 1) / mt_dense;
    a.kchains = dense_shape == moe::GEMM_STREAM16 ? 4 : 1;
    MOE_HIP(moe::launch_mx_gemm(a, moe::EPI_F32, dense_shape, s));
  }
  MOE_HIP(mark(MOE_EV_OUT));

  // Optional trace copies.
  if (tr) {
    auto cp = [&](void* dst, const void* src, size_t n) -> hipError_t {
      if (!dst || n == 0) return hipSuccess;
      return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, s);
    };
    const size_t Ts = (size_t)T, Ps = (size_t)P;
    if (hp) {
      MOE_HIP(cp(tr->xb, xb, Ts * d * 2));
    } else {
      MOE_HIP(cp(tr->xq_codes, xq, Ts * d));
      MOE_HIP(cp(tr->xq_scales, xqs, Ts * d / 32));
    }
    MOE_HIP(cp(tr->z, zr, Ts * L * 4));
    MOE_HIP(cp(tr->zq_codes, zqa, Ts * L));
    MOE_HIP(cp(tr->zq_scales, zqsa, Ts * L / 32));
    MOE_HIP(cp(tr->logits, logits, Ts * E * 4));
    MOE_HIP(cp(tr->ids, ids, Ps * 4));
    MOE_HIP(cp(tr->gates, gates, Ps * 4));
    MOE_HIP(cp(tr->counts, counts, (size_t)E * 4));
    MOE_HIP(cp(tr->offsets, offsets, (size_t)(E + 1) * 4));
    MOE_HIP(cp(tr->pair_of_row, por, Ps * 4));
    MOE_HIP(cp(tr->row_of_pair, rop, Ps * 4));
    MOE_HIP(cp(tr->hq_codes, hq, Ps * F));
    MOE_HIP(cp(tr->hq_scales, hqs, Ps * F / 32));
    MOE_HIP(cp(tr->y_e, ye, Ps * L * 4));
    if (latent) {  // (without a latent, y_lat was copied before the shared experts were added)
      MOE_HIP(cp(tr->y_lat, ylat, Ts * L * 4));
      if (hp) {
        MOE_HIP(cp(tr->yb, yb, Ts * L * 2));
      } else {
        MOE_HIP(cp(tr->yq_codes, yq, Ts * L));
        MOE_HIP(cp(tr->yq_scales, yqs, Ts * L / 32));
      }
    }
    if (S > 0 && hp) {
      MOE_HIP(cp(tr->hs_bf16, hb, (size_t)S * Ts * Fs * 2));
    } else if (S > 0) {
      MOE_HIP(cp(tr->hs_codes, hs, (size_t)S * Ts * Fs));
      MOE_HIP(cp(tr->hs_scales, hss, (size_t)S * Ts * Fs / 32));
    }
  }
  return MOE_OK;
}

// ---- static scratch of the no-allocation forward ---------------------------
//
// One array per GPU the library runs on (a __device__ variable has a copy on
// every device), held until the process ends.  In host code `scratch` names
// a host-side stand-in, not a device address: the device address is looked
// up per device with hipGetSymbolAddress and only that pointer is used.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// The current device's copy of `scratch` (looked up on the first call there).
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> g(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p || !aligned(p, kAlign)) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int moe_layer_forward(moe_layer_t layer, const float* x, int32_t T, float* y, void* ws, size_t ws_bytes,
                      void* stream, const moe_layer_trace* tr) {
  if (!layer) return MOE_ERR_INVALID_ARG;
  const moe_layer_config& c = layer->cfg;
  if (T < 0 || T > c.max_tokens) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < make_plan(c, T).total) return MOE_ERR_WORKSPACE;
  return forward_impl(layer, x, T, y, ws, stream, tr);
}

int moe_layer_forward_noalloc(moe_layer_t layer, const float* x, int32_t T, float* y, void* stream,
                              const moe_layer_trace* tr) {
  if (!layer) return MOE_ERR_INVALID_ARG;
  const moe_layer_config& c = layer->cfg;
  if (T < 0 || T > c.max_tokens) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  if (make_plan(c, T).total > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return MOE_ERR_HIP;
  return forward_impl(layer, x, T, y, ws, stream, tr);
}

int moe_mx_quantize(const float* in, int64_t rows, int32_t K, int32_t fmt, uint8_t* codes, uint8_t* scales,
                    void* stream) {
  if (rows < 0 || K <= 0 || K % 32 || (fmt != 0 && fmt != 1)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!in || !codes || !scales || !aligned(in, 16) || !aligned(codes, fmt == 0 ? 4 : 2))
    return MOE_ERR_INVALID_ARG;
  if (rows > ((int64_t)1 << 40) / K) return MOE_ERR_INVALID_ARG;
  if (moe::launch_quantize(in, rows, K, fmt, codes, scales, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_mx_quantize_weights(const float* in, int64_t G, int32_t N, int32_t K, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  if (G < 0 || N <= 0 || N % 16 || K <= 0 || K % 128) return MOE_ERR_INVALID_ARG;
  if (G == 0) return MOE_OK;
  if (!in || !codes || !scales || !aligned(in, 16) || !aligned(codes, 2)) return MOE_ERR_INVALID_ARG;
  if (G > ((int64_t)1 << 40) / ((int64_t)N * K)) return MOE_ERR_INVALID_ARG;
  if (moe::launch_quantize(in, G * N, K, 1, codes, scales, static_cast<hipStream_t>(stream), nullptr, N) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_mx_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t G, int32_t N, int32_t K,
                        uint8_t* out_codes, uint8_t* out_scales, void* stream) {
  if (G < 0 || N <= 0 || N % 16 || K <= 0 || K % 128) return MOE_ERR_INVALID_ARG;
  if (G == 0) return MOE_OK;
  if (!codes || !scales || !out_codes || !out_scales) return MOE_ERR_INVALID_ARG;
  if (!aligned(codes, 16) || !aligned(out_codes, 16) || !aligned(scales, 4) || !aligned(out_scales, 4))
    return MOE_ERR_INVALID_ARG;
  if (G > ((int64_t)1 << 40) / ((int64_t)N * K)) return MOE_ERR_INVALID_ARG;
  if (moe::launch_pack_e2m1(codes, scales, G, N, K, out_codes, out_scales, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_round_bf16(const float* in, int64_t n, uint16_t* out, void* stream) {
  if (n < 0 || n % 4) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!in || !out || !aligned(in, 16) || !aligned(out, 8)) return MOE_ERR_INVALID_ARG;
  if (moe::launch_round_bf16(in, n, out, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

size_t moe_quantile_balance_workspace_bytes(int32_t T, int32_t E) {
  if (T < 0 || E < 0) return 0;
  return moe::quantile_balance_workspace_floats(T, E) * sizeof(float);
}

int moe_quantile_balance(const float* logits, int32_t T, int32_t E, int32_t k, const float* bias_in, float eta,
                         float* bias_out, float* quantile_out, void* ws, size_t ws_bytes, void* stream) {
  if (T < 2 || E < 2 || E > 4096 || k < 1 || k >= E) return MOE_ERR_INVALID_ARG;
  if (!(eta > 0.0f && eta <= 1.0f)) return MOE_ERR_INVALID_ARG;
  if (!logits || !bias_in || !bias_out) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(bias_in, 4) || !aligned(bias_out, 4) ||
      (quantile_out && !aligned(quantile_out, 4)))
    return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 16) || ws_bytes < moe_quantile_balance_workspace_bytes(T, E)) return MOE_ERR_WORKSPACE;
  if (moe::launch_quantile_balance(logits, T, E, k, bias_in, eta, bias_out, quantile_out,
                                   static_cast<float*>(ws), static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_mfma_rate_probe(int32_t iters, int32_t workgroups, float* out, void* stream) {
  if (iters < 1 || iters > (1 << 24) || workgroups < 1 || workgroups > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (!out || !aligned(out, 4)) return MOE_ERR_INVALID_ARG;
  if (moe::launch_mfma_rate(iters, workgroups, out, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_hbm_read_probe(const void* buf, size_t bytes, int32_t workgroups, uint32_t* out, void* stream) {
  if (!buf || !out || bytes == 0 || bytes % 16 || workgroups < 1 || workgroups > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(out, 4)) return MOE_ERR_INVALID_ARG;
  if (moe::launch_hbm_read(buf, (int64_t)bytes, workgroups, out, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                int32_t M, int32_t N, int32_t K, float* c, void* stream) {
  if (M < 0 || N < 0 || N % 16 || K <= 0 || K % 128) return MOE_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return MOE_OK;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return MOE_ERR_INVALID_ARG;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4))
    return MOE_ERR_INVALID_ARG;
  const int shape = M <= 16 ? moe::GEMM_STREAM16 : M <= 256 ? moe::GEMM_STREAM64 : moe::GEMM_WIDE;
  moe::GemmArgs a = {};
  a.nseg = 1;
  a.seg[0] = {a_codes, a_scales, K, b_codes, b_scales, nullptr, nullptr, 0, 0, K};
  a.G = 1;
  a.M = M;
  a.N = N;
  a.c = c;
  a.ldc = N;
  a.max_mtiles = (M + moe::gemm_mtile(shape) - 1) / moe::gemm_mtile(shape);
  if (moe::launch_mx_gemm(a, moe::EPI_F32, shape, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_router_topk(const float* logits, const float* selection_bias, int32_t T, int32_t E, int32_t k,
                    int32_t softmax_gates, int32_t* ids, float* gates, void* stream) {
  if (T < 0 || E < 1 || E > 4096 || k < 1 || k > 64 || k > E) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !gates || !aligned(logits, 4) || !aligned(ids, 4) || !aligned(gates, 4) ||
      (selection_bias && !aligned(selection_bias, 4)))
    return MOE_ERR_INVALID_ARG;
  if (moe::launch_topk(logits, selection_bias, T, E, k, softmax_gates != 0, ids, gates,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_router_reduce_topk(const float* partial, int32_t nz, const float* logit_bias, const float* selection_bias,
                           int32_t T, int32_t E, int32_t k, int32_t softmax_gates, float* logits, int32_t* ids,
                           float* gates, void* stream) {
  if (T < 0 || nz < 1 || E < 1 || E > 1024 || k < 1 || k > 64 || k > E) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!partial || !logits || !ids || !gates || !aligned(partial, 4) || !aligned(logits, 4) || !aligned(ids, 4) ||
      !aligned(gates, 4) || (logit_bias && !aligned(logit_bias, 4)) ||
      (selection_bias && !aligned(selection_bias, 4)))
    return MOE_ERR_INVALID_ARG;
  if (moe::launch_router_reduce_topk(partial, nz, logit_bias, selection_bias, T, E, k, softmax_gates != 0, logits,
                                     ids, gates, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

}  // extern "C"
