// permute.hip -- expert histogram, prefix sums and the stable token permutation.
//
// Four Bits at a Time, "What it takes to serve it" (the MoE data-path toy):
// the (token, slot) pairs are flattened token-major and stably sorted by
// expert; per-expert counts and their exclusive prefix sum delimit each
// expert's segment.  Here the sort is a deterministic counting sort:
//
//   count   one wave per block of 64 tokens.  Each pair ORs its lane bit into
//           an LDS bitmask per expert; popcount of the mask is the block's
//           count for that expert.
//   scan    one workgroup.  Per expert, an exclusive scan over blocks gives
//           each block's base inside the expert segment; an exclusive scan over
//           experts gives the segment offsets; the same scan over
//           ceil(count / MT) gives the M-tile prefix the grouped GEMM walks.
//   scatter recomputes the block masks; the rank of a pair inside its block
//           is popcount(mask & lanes-below-me), i.e. the number of earlier
//           tokens of the block that chose the same expert (a token never
//           picks one expert twice).  row = offset[e] + base[b][e] + rank.
//
// A batch of at most 64 tokens (one block) runs all three in one workgroup.
//
// No atomics touch global memory and nothing depends on scheduling order, so
// the permutation is bitwise reproducible and stable (token order inside each
// segment).
#include "kernels.hpp"
#include "mx_device.hpp"

namespace moe {

constexpr int kTokBlock = 64;

size_t dispatch_scratch_ints(int T, int E) {
  const size_t nblk = (size_t)(T + kTokBlock - 1) / kTokBlock;
  return nblk * (size_t)E;  // per-block counts, rewritten in place as per-block bases
}

__global__ void __launch_bounds__(64) perm_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                       int32_t* __restrict__ blk) {
  extern __shared__ unsigned long long masks[];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += 64) masks[e] = 0ull;
  __syncthreads();
  const int t = b * kTokBlock + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicOr(&masks[ids[(int64_t)t * k + j]], 1ull << lane);
  __syncthreads();
  for (int e = lane; e < E; e += 64) blk[(int64_t)b * E + e] = __popcll(masks[e]);
}

// Single workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) perm_scan_kernel(int nblk, int E, int32_t* __restrict__ blk,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets, int mt0,
                                                        int32_t* __restrict__ ms0, int32_t* __restrict__ tg0,
                                                        int mt1, int32_t* __restrict__ ms1,
                                                        int32_t* __restrict__ tg1) {
  __shared__ int32_t part[3][16];
  const int tid = threadIdx.x;
  // 1) per expert: exclusive scan over blocks (in place), total = count; the
  //    blocks' counts are loaded 32 at a time, all in flight (one load at a
  //    time made this a chain of nblk memory latencies).
  constexpr int NB = 32;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += NB) {
      int c[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) c[i] = b0 + i < nblk ? blk[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (b0 + i < nblk) {
          blk[(int64_t)(b0 + i) * E + e] = run;
          run += c[i];
        }
    }
    counts[e] = run;
  }
  __syncthreads();
  // 2) exclusive scans over experts of count, ceil(count/mt0), ceil(count/mt1).
  //    Thread tid owns the contiguous experts [lo, hi).
  const int per = (E + 1023) / 1024;
  const int lo = tid * per < E ? tid * per : E;
  const int hi = lo + per < E ? lo + per : E;
  int s0 = 0, s1 = 0, s2 = 0;
  for (int e = lo; e < hi; ++e) {
    const int c = counts[e];
    s0 += c;
    s1 += (c + mt0 - 1) / mt0;
    s2 += (c + mt1 - 1) / mt1;
  }
  // Exclusive scan of the 1024 partials: inclusive within each wave by lane
  // shuffles, then the totals of the waves before this one (16 waves).
  const int lane = tid & 63, wave = tid >> 6;
  int i0 = s0, i1 = s1, i2 = s2;
  for (int o = 1; o < 64; o <<= 1) {
    const int a0 = __shfl_up(i0, o, 64), a1 = __shfl_up(i1, o, 64), a2 = __shfl_up(i2, o, 64);
    if (lane >= o) { i0 += a0; i1 += a1; i2 += a2; }
  }
  if (lane == 63) { part[0][wave] = i0; part[1][wave] = i1; part[2][wave] = i2; }
  __syncthreads();
  int r0 = i0 - s0, r1 = i1 - s1, r2 = i2 - s2;
  int t0 = 0, t1 = 0, t2 = 0;  // totals over all experts
  for (int w = 0; w < 16; ++w) {
    if (w < wave) { r0 += part[0][w]; r1 += part[1][w]; r2 += part[2][w]; }
    t0 += part[0][w]; t1 += part[1][w]; t2 += part[2][w];
  }
  for (int e = lo; e < hi; ++e) {
    const int c = counts[e];
    offsets[e] = r0; ms0[e] = r1; ms1[e] = r2;
    const int n0 = (c + mt0 - 1) / mt0, n1 = (c + mt1 - 1) / mt1;
    if (tg0)
      for (int q = 0; q < n0; ++q) tg0[r1 + q] = e;
    if (tg1)
      for (int q = 0; q < n1; ++q) tg1[r2 + q] = e;
    r0 += c;
    r1 += n0;
    r2 += n1;
  }
  if (tid == 1023) { offsets[E] = t0; ms0[E] = t1; ms1[E] = t2; }
}

__global__ void __launch_bounds__(64) perm_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                         const int32_t* __restrict__ base,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ row_of_pair,
                                                         int32_t* __restrict__ pair_of_row) {
  extern __shared__ unsigned long long masks[];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += 64) masks[e] = 0ull;
  __syncthreads();
  const int t = b * kTokBlock + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicOr(&masks[ids[(int64_t)t * k + j]], 1ull << lane);
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int64_t pair = (int64_t)t * k + j;
      const int e = ids[pair];
      const int row = offsets[e] + base[(int64_t)b * E + e] + __popcll(masks[e] & below);
      row_of_pair[pair] = row;
      pair_of_row[row] = (int32_t)pair;
    }
  }
}

// All of count, scan and scatter in one workgroup when the batch is one
// block of at most 64 tokens (decode): the same bitmask counting sort, with
// the per-expert masks and segment offsets kept in LDS.
__global__ void __launch_bounds__(1024) perm_small_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int mt0, int32_t* __restrict__ ms0,
                                                         int32_t* __restrict__ tg0, int mt1,
                                                         int32_t* __restrict__ ms1, int32_t* __restrict__ tg1,
                                                         int32_t* __restrict__ row_of_pair,
                                                         int32_t* __restrict__ pair_of_row) {
  extern __shared__ unsigned long long masks[];            // [E], then int32 offsets [E]
  int32_t* soff = reinterpret_cast<int32_t*>(masks + E);
  __shared__ int32_t part[3][16];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) masks[e] = 0ull;
  __syncthreads();
  if (tid < T)
    for (int j = 0; j < k; ++j) atomicOr(&masks[ids[(int64_t)tid * k + j]], 1ull << tid);
  __syncthreads();
  // exclusive scans over experts of count, ceil(count/mt0), ceil(count/mt1);
  // thread tid owns the contiguous experts [lo, hi).
  const int per = (E + 1023) / 1024;
  const int lo = tid * per < E ? tid * per : E;
  const int hi = lo + per < E ? lo + per : E;
  int s0 = 0, s1 = 0, s2 = 0;
  for (int e = lo; e < hi; ++e) {
    const int c = __popcll(masks[e]);
    s0 += c;
    s1 += (c + mt0 - 1) / mt0;
    s2 += (c + mt1 - 1) / mt1;
  }
  // Exclusive scan of the 1024 partials: inclusive within each wave by lane
  // shuffles, then the totals of the waves before this one (16 waves).
  const int lane = tid & 63, wave = tid >> 6;
  int i0 = s0, i1 = s1, i2 = s2;
  for (int o = 1; o < 64; o <<= 1) {
    const int a0 = __shfl_up(i0, o, 64), a1 = __shfl_up(i1, o, 64), a2 = __shfl_up(i2, o, 64);
    if (lane >= o) { i0 += a0; i1 += a1; i2 += a2; }
  }
  if (lane == 63) { part[0][wave] = i0; part[1][wave] = i1; part[2][wave] = i2; }
  __syncthreads();
  int r0 = i0 - s0, r1 = i1 - s1, r2 = i2 - s2;
  int t0 = 0, t1 = 0, t2 = 0;  // totals over all experts
  for (int w = 0; w < 16; ++w) {
    if (w < wave) { r0 += part[0][w]; r1 += part[1][w]; r2 += part[2][w]; }
    t0 += part[0][w]; t1 += part[1][w]; t2 += part[2][w];
  }
  for (int e = lo; e < hi; ++e) {
    const int c = __popcll(masks[e]);
    counts[e] = c;
    offsets[e] = r0; ms0[e] = r1; ms1[e] = r2;
    soff[e] = r0;
    const int n0 = (c + mt0 - 1) / mt0, n1 = (c + mt1 - 1) / mt1;
    if (tg0)
      for (int q = 0; q < n0; ++q) tg0[r1 + q] = e;
    if (tg1)
      for (int q = 0; q < n1; ++q) tg1[r2 + q] = e;
    r0 += c;
    r1 += n0;
    r2 += n1;
  }
  if (tid == 1023) { offsets[E] = t0; ms0[E] = t1; ms1[E] = t2; }
  __syncthreads();
  if (tid < T) {  // rank of a pair = earlier tokens of the block that chose the same expert
    const unsigned long long below = (1ull << tid) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int64_t pair = (int64_t)tid * k + j;
      const int e = ids[pair];
      const int row = soff[e] + __popcll(masks[e] & below);
      row_of_pair[pair] = row;
      pair_of_row[row] = (int32_t)pair;
    }
  }
}

hipError_t launch_dispatch(const int32_t* ids, int T, int E, int k, int32_t* scratch, int32_t* counts,
                           int32_t* offsets, int32_t* row_of_pair, int32_t* pair_of_row, int mt0,
                           int32_t* ms0, int32_t* tg0, int mt1, int32_t* ms1, int32_t* tg1, hipStream_t s) {
  const int nblk = (T + kTokBlock - 1) / kTokBlock;
  const size_t smem = (size_t)E * sizeof(unsigned long long);
  if (nblk == 1) {  // one block of tokens: one launch
    perm_small_kernel<<<dim3(1), dim3(1024), smem + (size_t)E * sizeof(int32_t), s>>>(
        ids, T, E, k, counts, offsets, mt0, ms0, tg0, mt1, ms1, tg1, row_of_pair, pair_of_row);
    return hipGetLastError();
  }
  if (nblk > 0) {
    perm_count_kernel<<<dim3(nblk), dim3(64), smem, s>>>(ids, T, E, k, scratch);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  perm_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(nblk, E, scratch, counts, offsets, mt0, ms0, tg0, mt1, ms1,
                                                   tg1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  perm_scatter_kernel<<<dim3(nblk), dim3(64), smem, s>>>(ids, T, E, k, scratch, offsets, row_of_pair,
                                                         pair_of_row);
  return hipGetLastError();
}

}  // namespace moe
