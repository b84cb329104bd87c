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
//      rounds of a wave arg-max over the token's keys held in LDS;
//   2. margins, transposed to expert-major [E][T] through a 64 x 64 LDS tile
//      (coalesced reads of the token-major logits and coalesced writes);
//   3. per expert (one 256-thread workgroup): the n-th and (n+1)-th largest
//      margins by an exact 4-pass radix select over the order-preserving
//      unsigned image of the fp32 margins, then the bias update.
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
// change them).  Four tokens per 256-thread block, keys of each in LDS.
__global__ void __launch_bounds__(256) qb_threshold_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ bias, int T, int E,
                                                           int k, float* __restrict__ thr) {
  extern __shared__ float kv_all[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;  // no block-level barrier below
  float* kv = kv_all + (size_t)w * E;
  const float* lg = logits + (size_t)t * E;
  for (int e = lane; e < E; e += 64) kv[e] = qb_sigmoid(lg[e]) + bias[e];
  float kk = 0.f, kk1 = 0.f;
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
    // The winner leaves.  E > k leaves a finite key in every round; the bound
    // only matters for NaN keys (unsupported input), which never win.
    if (bi < E && lane == (bi & 63)) kv[bi] = -INFINITY;
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

// 3. One workgroup per expert: exact rank selection (1-based, largest first)
// by 8-bit digits from the top, then the update.
__global__ void __launch_bounds__(256) qb_select_kernel(const float* __restrict__ margins, int T, int n,
                                                        const float* __restrict__ bias_in, float eta,
                                                        float* __restrict__ bias_out,
                                                        float* __restrict__ q_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_rem;
  const int e = blockIdx.x, tid = threadIdx.x;
  const float* m = margins + (size_t)e * T;
  auto select = [&](uint32_t rank) -> uint32_t {
    uint32_t prefix = 0, mask = 0, rem = rank;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int t = tid; t < T; t += 256) {
        const uint32_t o = f2ord(m[t]);
        if ((o & mask) == prefix) atomicAdd(&hist[(o >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        // the candidates number at least rem, so some digit reaches it
        uint32_t cum = 0;
        int b = 255;
        for (; b > 0; --b) {
          if (cum + hist[b] >= rem) break;
          cum += hist[b];
        }
        s_prefix = prefix | ((uint32_t)b << shift);
        s_rem = rem - cum;
      }
      __syncthreads();
      prefix = s_prefix;
      rem = s_rem;
      mask |= 255u << shift;
    }
    return prefix;
  };
  const float vn = ord2f(select((uint32_t)n));
  const float vn1 = ord2f(select((uint32_t)n + 1u));
  if (tid == 0) {
    const float q = 0.5f * (vn + vn1);
    bias_out[e] = bias_in[e] - eta * q;
    if (q_out) q_out[e] = q;
  }
}

}  // namespace

size_t quantile_balance_workspace_floats(int T, int E) { return 2 * (size_t)T + (size_t)E * T; }

int quantile_balance_target(int T, int E, int k) {
  const double c = (double)T * k / E;
  long n = lround(c);
  if (n < 1) n = 1;
  if (n > T - 1) n = T - 1;
  return (int)n;
}

hipError_t launch_quantile_balance(const float* logits, int T, int E, int k, const float* bias_in, float eta,
                                   float* bias_out, float* q_out, float* ws, hipStream_t s) {
  float* thr = ws;
  float* margins = ws + 2 * (size_t)T;
  qb_threshold_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), (size_t)4 * E * sizeof(float), s>>>(
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
