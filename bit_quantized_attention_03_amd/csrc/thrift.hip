// Thrift block selection — "ThriftAttention: Selective Mixed Precision for Long-Context FP4
// Attention", ¶1 and ¶3: a small fraction (~5%) of the query-key blocks, the ones that
// dominate the output, runs in high precision.  The page does not print its heuristic; the
// score used here is the dot product of the bf16 block means of Q and of smoothed K.
//   1. pool_kernel:   block means (fp32 running sum in token order, / length, -> bf16)
//   2. score_kernel:  fp32 fma chain over channels for every (Q block, K block) pair; a
//                     workgroup holds 16 Q-block means in LDS and streams the K-block means
//   3. select_kernel: per (b, q-head) radix select of the n_sel-th largest score among the
//                     causal-valid pairs (4 passes of 8 bits on an order-preserving key),
//                     then ties at the threshold taken in ascending linear index via a
//                     workgroup ballot scan.  Deterministic: the selected set is unique.
#include "device.hpp"
#include "kernels.hpp"

namespace sage {
namespace {

constexpr int QBLK = 128, KBLK = 64;

__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ x, int64_t BH, int64_t N, int D, int T,
                                                   uint16_t* __restrict__ means) {
  const int64_t nblk = (N + T - 1) / T;
  const int cg = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= BH * nblk * cg) return;
  const int c8 = (int)(gid % cg);
  const int64_t blk = (gid / cg) % nblk, bh = gid / cg / nblk;
  const int64_t t0 = blk * T;
  const int rows = (int)((N - t0) < T ? (N - t0) : T);
  const uint16_t* p = x + (bh * N + t0) * D + c8 * 8;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add_row = [&](v4i raw) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + bf16_to_f32((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1))));
  };
  int t = 0;
  for (; t + 16 <= rows; t += 16) {   // 16 row loads in flight, then the adds in token order
    v4i raw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) raw[j] = *(const v4i*)(p + (int64_t)(t + j) * D);
#pragma unroll
    for (int j = 0; j < 16; ++j) add_row(raw[j]);
  }
  for (; t < rows; ++t) add_row(*(const v4i*)(p + (int64_t)t * D));
  v4i o;
#pragma unroll
  for (int w = 0; w < 4; ++w) o[w] = (int)pack_bf16x2(s[2 * w] / (float)rows, s[2 * w + 1] / (float)rows);
  *(v4i*)(means + (bh * nblk + blk) * D + c8 * 8) = o;
}

// block: (group of 16 Q blocks, b*Hq+h); thread: K blocks tid, tid+256, ...
__global__ __launch_bounds__(256) void score_kernel(const uint16_t* __restrict__ qbar, const uint16_t* __restrict__ kbar,
                                                    int64_t Hq, int64_t Hkv, int64_t nQB, int64_t nKB, int D,
                                                    float* __restrict__ scores) {
  __shared__ float qs[16][129];
  const int64_t bhq = blockIdx.y;
  const int64_t b = bhq / Hq, h = bhq % Hq, g = h / (Hq / Hkv);
  const int64_t qb0 = (int64_t)blockIdx.x * 16;
  const int nq = (int)((nQB - qb0) < 16 ? (nQB - qb0) : 16);
  for (int i = threadIdx.x; i < 16 * D; i += 256) {
    const int r = i / D, c = i % D;
    qs[r][c] = r < nq ? bf16_to_f32(qbar[(bhq * nQB + qb0 + r) * D + c]) : 0.0f;
  }
  __syncthreads();
  const uint16_t* kb_base = kbar + (b * Hkv + g) * nKB * D;
  for (int64_t kb = threadIdx.x; kb < nKB; kb += 256) {
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint16_t* kr = kb_base + kb * D;
    for (int c0 = 0; c0 < D; c0 += 8) {
      v4i raw = *(const v4i*)(kr + c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kv = bf16_to_f32((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1))));
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(qs[r][c0 + e], kv, acc[r]);
      }
    }
    for (int r = 0; r < nq; ++r) scores[(bhq * nQB + qb0 + r) * nKB + kb] = acc[r];
  }
}

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);   // -0 -> +0, so equal scores give equal keys
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool pair_valid(int64_t qb, int64_t kb, int causal) {
  return !causal || (int64_t)KBLK * kb <= (int64_t)QBLK * qb + QBLK - 1;
}

constexpr int SEL_THREADS = 1024;

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const float* __restrict__ scores, int64_t nQB, int64_t nKB,
                                                             int causal, int64_t n_sel, uint8_t* __restrict__ mask) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[SEL_THREADS / 64];
  __shared__ uint32_t sh_digit, sh_remaining, sh_eq;
  const int64_t bhq = blockIdx.x;
  const float* sc = scores + bhq * nQB * nKB;
  uint8_t* mk = mask + bhq * nQB * nKB;
  const int64_t npair = nQB * nKB;
  const int tid = threadIdx.x;
  if (n_sel <= 0) {
    for (int64_t i = tid; i < npair; i += SEL_THREADS) mk[i] = 0;
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)n_sel;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
    __syncthreads();
    // eight scores per thread in flight (the scores sit in L2; one load per step would leave
    // each step waiting for its load)
    for (int64_t base = 0; base < npair; base += 8 * SEL_THREADS) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t i = base + j * SEL_THREADS + tid;
        v[j] = i < npair ? sc[i] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t i = base + j * SEL_THREADS + tid;
        if (i >= npair) continue;
        const uint32_t qb = (uint32_t)i / (uint32_t)nKB, kb = (uint32_t)i - qb * (uint32_t)nKB;
        if (!pair_valid(qb, kb, causal)) continue;
        const uint32_t key = order_key(v[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + hist[d] >= remaining) break;
        above += hist[d];
      }
      sh_digit = (uint32_t)d;
      sh_remaining = remaining - above;
      sh_eq = hist[d];   // after the last pass: how many keys equal the threshold key
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    remaining = sh_remaining;
    __syncthreads();
  }
  // prefix = key of the n_sel-th largest; `remaining` keys equal to it are taken, lowest index first.
  const uint32_t T = prefix;
  if (remaining == sh_eq) {   // every key equal to T is taken: no ordering needed
    for (int64_t base = 0; base < npair; base += 8 * SEL_THREADS) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t i = base + j * SEL_THREADS + tid;
        v[j] = i < npair ? sc[i] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t i = base + j * SEL_THREADS + tid;
        if (i >= npair) continue;
        const uint32_t qb = (uint32_t)i / (uint32_t)nKB;
        const bool valid = pair_valid(qb, (uint32_t)i - qb * (uint32_t)nKB, causal);
        mk[i] = (uint8_t)(valid && order_key(v[j]) >= T);
      }
    }
    return;
  }
  uint32_t taken_eq = 0;
  const int lane = tid & 63, wv = tid >> 6;
  for (int64_t base = 0; base < npair; base += SEL_THREADS) {
    const int64_t i = base + tid;
    bool valid = false;
    uint32_t key = 0;
    if (i < npair) {
      const uint32_t qb = (uint32_t)i / (uint32_t)nKB;
      valid = pair_valid(qb, (uint32_t)i - qb * (uint32_t)nKB, causal);
      key = valid ? order_key(sc[i]) : 0u;
    }
    const bool eq = valid && key == T;
    const uint64_t bal = __ballot(eq);
    const uint32_t before_in_wave = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wv] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t before = taken_eq + before_in_wave;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    uint32_t chunk_eq = 0;
    for (int w = 0; w < SEL_THREADS / 64; ++w) chunk_eq += wave_tot[w];
    if (i < npair) mk[i] = (uint8_t)(valid && (key > T || (eq && before < remaining)));
    taken_eq += chunk_eq;
    __syncthreads();
  }
}

}  // namespace

size_t thrift_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int D) {
  const int64_t nQB = (N + QBLK - 1) / QBLK, nKB = (N + KBLK - 1) / KBLK;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up((size_t)(B * Hq * nQB * D) * 2) + up((size_t)(B * Hkv * nKB * D) * 2) + up((size_t)(B * Hq * nQB * nKB) * 4);
}

hipError_t launch_thrift_select(const uint16_t* q, const uint16_t* ks, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                int D, double frac, int causal, uint8_t* mask, void* ws, hipStream_t st) {
  const int64_t nQB = (N + QBLK - 1) / QBLK, nKB = (N + KBLK - 1) / KBLK;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  uint16_t* qbar = (uint16_t*)ws;
  uint16_t* kbar = (uint16_t*)((char*)ws + up((size_t)(B * Hq * nQB * D) * 2));
  float* scores = (float*)((char*)kbar + up((size_t)(B * Hkv * nKB * D) * 2));
  int64_t n_valid = 0;
  for (int64_t qb = 0; qb < nQB; ++qb) {
    if (!causal) { n_valid += nKB; continue; }
    int64_t lim = (QBLK * qb + QBLK - 1) / KBLK + 1;
    n_valid += lim < nKB ? lim : nKB;
  }
  double want = frac * (double)n_valid;
  int64_t n_sel = (int64_t)want;
  if ((double)n_sel < want) ++n_sel;
  if (n_sel > n_valid) n_sel = n_valid;
  const int cg = D / 8;
  int64_t t = B * Hq * nQB * cg;
  pool_kernel<<<(unsigned)((t + 255) / 256), 256, 0, st>>>(q, B * Hq, N, D, QBLK, qbar);
  t = B * Hkv * nKB * cg;
  pool_kernel<<<(unsigned)((t + 255) / 256), 256, 0, st>>>(ks, B * Hkv, N, D, KBLK, kbar);
  dim3 g((unsigned)((nQB + 15) / 16), (unsigned)(B * Hq));
  score_kernel<<<g, 256, 0, st>>>(qbar, kbar, Hq, Hkv, nQB, nKB, D, scores);
  select_kernel<<<(unsigned)(B * Hq), SEL_THREADS, 0, st>>>(scores, nQB, nKB, causal, n_sel, mask);
  return hipGetLastError();
}

}  // namespace sage
