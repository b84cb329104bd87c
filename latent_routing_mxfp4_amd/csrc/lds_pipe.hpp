// lds_pipe.hpp -- pieces shared by the LDS-staged GEMM kernels: direct
// global -> LDS loads with hand-placed waits, and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace moe {

// Direct global -> LDS loads (16 or 4 bytes per lane; lane l lands at
// m0 + size * l) and their waits are issued as inline assembly: the compiler's
// wait-count pass would otherwise treat every in-flight LDS load as aliasing
// every LDS read and drain the whole pipeline (vmcnt(0)) before each fragment
// read.  Ordering is kept by hand: wait_vmcnt<N>() after issue, then a barrier.
// The sequences write m0, which the compiler cannot be told about (it is not
// an allocatable clobber); no compiler-generated instruction of these kernels
// uses m0, which a test checks on the built gfx950 assembly.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void gl_lds16(const void* g, const uint8_t* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr(lds)), "v"(g) : "memory");
}
__device__ __forceinline__ void gl_lds4(const void* g, const uint8_t* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr(lds)), "v"(g) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that waits only for this wave's LDS operations: the
// direct loads in flight are governed by wait_vmcnt, so the barrier must not
// drain them (__syncthreads would wait for vmcnt(0)).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Tile decode shared by the LDS-staged kernels: the flat tile list (group,
// weight column-tile, M-tile; M fastest) is cut into 8 contiguous chunks, one
// per XCD (workgroup bid runs on XCD bid % 8).  False for workgroups past the
// end.
template <int MT>
__device__ __forceinline__ bool decode_lds_tile(const GemmArgs& p, int bid, int ncol, int& g, int& mt, int& nt,
                                                int& rows, int& row_base) {
  const int n_nt = (p.N + ncol - 1) / ncol;
  const bool routed = p.offsets != nullptr;
  const int mpg = routed ? 0 : (p.M + MT - 1) / MT;
  const int total = routed ? p.mtile_start[p.G] * n_nt : p.G * mpg * n_nt;
  const int per = (total + 7) >> 3;
  const int slot = bid >> 3;
  if (slot >= per) return false;
  const int lin = (bid & 7) * per + slot;
  if (lin >= total) return false;
  if (routed) {
    if (p.mtile_group) {
      // lin = mtile_start[g]*n_nt + nt*mte + mt with nt*mte + mt < n_nt*mte, so
      // lin / n_nt is one of the group's M-tiles.
      g = p.mtile_group[lin / n_nt];
    } else {
      int lo = 0, hi = p.G;  // mtile_start[lo]*n_nt <= lin < mtile_start[hi]*n_nt
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.mtile_start[mid] * n_nt <= lin) lo = mid; else hi = mid;
      }
      g = lo;
    }
    const int mte = p.mtile_start[g + 1] - p.mtile_start[g];
    const int local = lin - p.mtile_start[g] * n_nt;
    nt = local / mte;
    mt = local - nt * mte;
    row_base = p.offsets[g];
    rows = p.offsets[g + 1] - row_base;
  } else {
    g = lin / (mpg * n_nt);
    const int local = lin - g * mpg * n_nt;
    nt = local / mpg;
    mt = local - nt * mpg;
    row_base = 0;
    rows = p.M;
  }
  return true;
}

}  // namespace moe
