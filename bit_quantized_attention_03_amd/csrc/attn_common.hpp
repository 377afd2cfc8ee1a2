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

// INT8 score tiles are computed transposed (S^T = K Q^T, 32x32 blocks, keys on the accumulator
// rows): accumulator row m of block b holds this key of the 64-key tile.  Lane half h of the
// wave holds keys 32 h .. 32 h + 31 across its two blocks.
__device__ __forceinline__ int tile_key(int b, int m) {
  return ((m >> 2) & 1) * 32 + 16 * b + (m >> 3) * 4 + (m & 3);
}

// Workgroup -> (b*Hq + h, pair of Q blocks).  Consecutive work items go to one XCD
// (workgroups are dealt round-robin over the 8 XCDs), so neighbouring heads share its L2.
// Causal runs take four heads at a time and walk their pairs from the heaviest down, the four
// heads interleaved.  Within an XCD the dispatcher deals workgroups round-robin over its four
// shader engines and waits when the next one has no free CU, so each run of four consecutive
// workgroups (one per engine) has the same length: they finish together and free one CU on
// every engine for the next four.  Heaviest first lets the short pairs fill the tail.
struct WgMap {
  int64_t bh, pair;
};
__device__ __forceinline__ WgMap map_workgroup(int64_t total_wg, int64_t n_pairs, bool causal) {
  int64_t wg = blockIdx.x;
  if ((total_wg & 7) == 0) wg = (wg & 7) * (total_wg >> 3) + (wg >> 3);
  if (!causal) return WgMap{wg / n_pairs, wg % n_pairs};
  constexpr int64_t G = 4;
  const int64_t heads = total_wg / n_pairs;
  const int64_t g = wg / (G * n_pairs), j = wg % (G * n_pairs);
  const int64_t r = heads - G * g < G ? heads - G * g : G;   // heads in this group
  return WgMap{G * g + j % r, n_pairs - 1 - j / r};
}

}  // namespace attn
}  // namespace sage
