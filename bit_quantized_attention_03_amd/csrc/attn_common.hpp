// Pieces shared by the fused attention kernels: tile sizes, the fence-free phase barrier,
// the cross-half reductions of the 32x32 accumulator layout and the LDS address space.
#pragma once
#include "device.hpp"

namespace sage {
namespace attn {

constexpr int QB = 128, KT = 64, NWAVES = 8, NTHREADS = 64 * NWAVES;
constexpr float LOG2E = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// Workgroup barrier without a memory fence.  Ordering is explicit in the kernels: tile loads
// are complete (wait_vmem) before the barrier that publishes them, and an LDS buffer is
// overwritten only after the barrier following the matrix instructions that consumed it.
__device__ __forceinline__ void phase_barrier() {
  __asm__ volatile("" ::: "memory");   // LDS may change across a phase boundary (direct loads land
  __builtin_amdgcn_s_barrier();       // unseen by the compiler): no LDS access moves across it
  __asm__ volatile("" ::: "memory");
}

// v_permlane32_swap on (x, x) returns, in an order that depends on the lane half, this
// lane's value and the value of lane l ^ 32; max and sum of the pair agree in both halves.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup -> (b*Hq + h, pair of Q blocks).  Consecutive work items go to one XCD
// (workgroups are dealt round-robin over the 8 XCDs), so neighbouring heads share its L2.
// Causal runs take two heads at a time and walk their pairs from the heaviest down, the two
// heads interleaved: the long pairs of a group start together and the short ones fill the
// tail, while each XCD still streams the K/V of only a few heads at once.
struct WgMap {
  int64_t bh, pair;
};
__device__ __forceinline__ WgMap map_workgroup(int64_t total_wg, int64_t n_pairs, bool causal) {
  int64_t wg = blockIdx.x;
  if ((total_wg & 7) == 0) wg = (wg & 7) * (total_wg >> 3) + (wg >> 3);
  if (!causal) return WgMap{wg / n_pairs, wg % n_pairs};
  const int64_t g = wg / (2 * n_pairs), j = wg % (2 * n_pairs);
  if ((g + 1) * 2 * n_pairs > total_wg)                  // odd head count: the last head alone
    return WgMap{2 * g, n_pairs - 1 - j};
  return WgMap{2 * g + (j & 1), n_pairs - 1 - (j >> 1)};
}

}  // namespace attn
}  // namespace sage
