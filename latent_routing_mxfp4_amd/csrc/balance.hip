// balance.hip -- Quantile Balancing of the expert selection bias.
//
// What it computes.  Each expert's selection bias moves so that the expert's
// routed token count approaches a target load, driven by the distribution of
// its score margins ("Kimi K3 and the New Open-Weights Moat: Inference
// Efficiency", section "How the router picks 16 of 896", Fig. 2 and the
// paragraph after it; "What Kimi K3 asks of the hardware", section "Width: 896
// experts and the interconnect": allocation from quantiles of the router
// scores).  The pages print no formula; the reading implemented here:
//   key(t, e)   = sigmoid(logit(t, e)) + b_e                       (fp32)
//   margin(t,e) = key(t, e) - (k-th largest key of token t among the other
//                 experts): key - K_{k+1}(t) if key >= K_k(t), else key - K_k(t)
//   n           = round(T k / E), clamped to [1, T-1]               (target load)
//   Q_e         = (n-th largest margin of e + (n+1)-th largest) / 2
//   b_e        <- b_e - eta Q_e
// Shifting b_e by -Q_e alone would route exactly n tokens to e.
//
// Three launches, all on the caller's stream:
//   1. per token (one wave): the k-th and (k+1)-th largest keys, by k+1
//      rounds of a wave arg-max over the token's keys (in registers up to
//      1024 experts, else in LDS);
//   2. margins, transposed to expert-major [E][T] through a 64 x 64 LDS tile
//      (coalesced reads of the token-major logits and coalesced writes);
//   3. per expert (one 256-thread workgroup): the n-th and (n+1)-th largest
//      margins, exactly, by a bit-by-bit search over the order-preserving
//      unsigned image of the fp32 margins (held in registers), then the bias
//      update.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.hpp"

namespace moe {

namespace {

__device__ __forceinline__ float qb_sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// Order-preserving map of fp32 onto uint32 (larger float -> larger key) and back.
__device__ __forceinline__ uint32_t f2ord(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// 1. thr[2t] = K_k(t), thr[2t+1] = K_{k+1}(t): the k-th and (k+1)-th largest
// keys of token t (values; which of equal keys is removed first does not
// change them).  Four tokens per 256-thread block, one wave each; up to 1024
// experts a lane keeps its keys (experts lane, lane + 64, ...) in registers,
// more experts sit in LDS.
constexpr int kThrPer = 16;

__global__ void __launch_bounds__(256) qb_threshold_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ bias, int T, int E,
                                                           int k, float* __restrict__ thr) {
  extern __shared__ float kv_all[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;  // no block-level barrier below
  const float* lg = logits + (size_t)t * E;
  float kk = 0.f, kk1 = 0.f;
  if (E <= 64 * kThrPer) {
    float kr[kThrPer];
#pragma unroll
    for (int j = 0; j < kThrPer; ++j) {
      const int e = lane + 64 * j;
      kr[j] = e < E ? qb_sigmoid(lg[e]) + bias[e] : -INFINITY;
    }
    for (int r = 0; r <= k; ++r) {
      float best = -INFINITY;
      int bj = 0;
#pragma unroll
      for (int j = 0; j < kThrPer; ++j)
        if (kr[j] > best) { best = kr[j]; bj = j; }  // j ascends: equal keys keep the lower id
      int bi = best > -INFINITY ? lane + 64 * bj : 0x7fffffff;
      for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (r == k - 1) kk = best;
      if (r == k) kk1 = best;
      // the winner leaves (E > k: a finite key remains in every round)
#pragma unroll
      for (int j = 0; j < kThrPer; ++j)
        if (lane + 64 * j == bi) kr[j] = -INFINITY;
    }
  } else {
    float* kv = kv_all + (size_t)w * E;
    for (int e = lane; e < E; e += 64) kv[e] = qb_sigmoid(lg[e]) + bias[e];
    for (int r = 0; r <= k; ++r) {
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int e = lane; e < E; e += 64) {
        const float v = kv[e];
        if (v > best) { best = v; bi = e; }  // e ascends, so equal keys keep the lower id
      }
      for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (r == k - 1) kk = best;
      if (r == k) kk1 = best;
      // The winner leaves.  E > k leaves a finite key in every round; the
      // bound only matters for NaN keys (unsupported input), which never win.
      if (bi < E && lane == (bi & 63)) kv[bi] = -INFINITY;
    }
  }
  if (lane == 0) {
    thr[2 * (size_t)t] = kk;
    thr[2 * (size_t)t + 1] = kk1;
  }
}

// 2. margins[e][t] for a 64-token x 64-expert tile: read along experts, write
// along tokens.
__global__ void __launch_bounds__(256) qb_margin_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ bias,
                                                        const float* __restrict__ thr, int T, int E,
                                                        float* __restrict__ margins) {
  __shared__ float tile[64][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int c = threadIdx.x & 63, r4 = threadIdx.x >> 6;
  for (int i = r4; i < 64; i += 4) {
    const int t = t0 + i, e = e0 + c;
    float m = 0.f;
    if (t < T && e < E) {
      const float key = qb_sigmoid(logits[(size_t)t * E + e]) + bias[e];
      const float kk = thr[2 * (size_t)t], kk1 = thr[2 * (size_t)t + 1];
      m = key - (key >= kk ? kk1 : kk);
    }
    tile[i][c] = m;
  }
  __syncthreads();
  for (int j = r4; j < 64; j += 4) {
    const int e = e0 + j, t = t0 + c;
    if (t < T && e < E) margins[(size_t)e * T + t] = tile[c][j];
  }
}

// 3. One workgroup per expert: the n-th and (n+1)-th largest margins, then
// the update.  Up to 256 * kSelPer tokens the expert's margins sit in
// registers (as order-preserving unsigned keys) and both ranks are found
// together, bit by bit from the top: the n-th largest key is the largest u
// with at least n keys >= u, so a bit is kept when the count of keys at or
// above the prefix with that bit set still reaches n (one block-wide count
// per bit and rank, no atomics).  More tokens: the same search re-reads the
// margins from global memory for every count.
constexpr int kSelPer = 64;

__global__ void __launch_bounds__(256) qb_select_kernel(const float* __restrict__ margins, int T, int n,
                                                        const float* __restrict__ bias_in, float eta,
                                                        float* __restrict__ bias_out,
                                                        float* __restrict__ q_out) {
  __shared__ uint32_t red[2][4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* m = margins + (size_t)e * T;
  const bool in_regs = T <= 256 * kSelPer;
  uint32_t v[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int t = tid + 256 * i;
    // 0 is below every finite key: padding never reaches a candidate (which has a bit set)
    v[i] = (in_regs && t < T) ? f2ord(m[t]) : 0u;
  }
  uint32_t p0 = 0, p1 = 0;  // prefixes of the n-th and (n+1)-th largest keys
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c0 = p0 | (1u << bit), c1 = p1 | (1u << bit);
    uint32_t n0 = 0, n1 = 0;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kSelPer; ++i) {
        n0 += v[i] >= c0;
        n1 += v[i] >= c1;
      }
    } else {
      for (int t = tid; t < T; t += 256) {
        const uint32_t o = f2ord(m[t]);
        n0 += o >= c0;
        n1 += o >= c1;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      n0 += __shfl_xor(n0, o, 64);
      n1 += __shfl_xor(n1, o, 64);
    }
    if (lane == 0) {
      red[0][w] = n0;
      red[1][w] = n1;
    }
    __syncthreads();
    const uint32_t s0 = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const uint32_t s1 = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    __syncthreads();  // red is rewritten by the next bit
    if (s0 >= (uint32_t)n) p0 = c0;
    if (s1 >= (uint32_t)n + 1u) p1 = c1;
  }
  if (tid == 0) {
    const float q = 0.5f * (ord2f(p0) + ord2f(p1));
    bias_out[e] = bias_in[e] - eta * q;
    if (q_out) q_out[e] = q;
  }
}

}  // namespace

size_t quantile_balance_workspace_floats(int T, int E) { return 2 * (size_t)T + (size_t)E * T; }

// round(T k / E) with ties to the even integer, in exact integer arithmetic.
int quantile_balance_target(int T, int E, int k) {
  const int64_t tk = (int64_t)T * k, q = tk / E, r = tk % E;
  int64_t n = q + ((2 * r > E) || (2 * r == E && (q & 1)) ? 1 : 0);
  if (n < 1) n = 1;
  if (n > T - 1) n = T - 1;
  return (int)n;
}

hipError_t launch_quantile_balance(const float* logits, int T, int E, int k, const float* bias_in, float eta,
                                   float* bias_out, float* q_out, float* ws, hipStream_t s) {
  float* thr = ws;
  float* margins = ws + 2 * (size_t)T;
  const size_t thr_lds = E <= 64 * kThrPer ? 0 : (size_t)4 * E * sizeof(float);
  qb_threshold_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), thr_lds, s>>>(
      logits, bias_in, T, E, k, thr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  qb_margin_kernel<<<dim3((unsigned)((T + 63) / 64), (unsigned)((E + 63) / 64)), dim3(256), 0, s>>>(
      logits, bias_in, thr, T, E, margins);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  qb_select_kernel<<<dim3((unsigned)E), dim3(256), 0, s>>>(margins, T, quantile_balance_target(T, E, k),
                                                           bias_in, eta, bias_out, q_out);
  return hipGetLastError();
}

}  // namespace moe
