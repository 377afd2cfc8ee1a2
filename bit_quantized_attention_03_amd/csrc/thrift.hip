// Thrift block selection — "ThriftAttention: Selective Mixed Precision for Long-Context FP4
// Attention", ¶1 and ¶3: a small fraction (~5%) of the query-key blocks, the ones that
// dominate the output, runs in high precision.  The page does not print its heuristic; the
// score used here is the dot product of the bf16 block means of Q and of smoothed K.
//   1. pool_kernel:   block means (fp32 running sum in token order, / length, -> bf16; the
//                     Q means stored widened to fp32)
//   2. score_kernel:  fp32 fma chain over channels for every (Q block, K block) pair; a
//                     workgroup holds 16 Q-block means in LDS and streams the K-block means,
//                     two K blocks per thread.
//                     Its pairs (16 Q blocks x all K blocks) form one selection chunk, and it
//                     also writes the chunk's histogram of the keys' top byte.
//   3. hist_kernel x3, mask_kernel: per (b, q-head) radix select of the n_sel-th largest
//                     score among the causal-valid pairs, 8 key bits per pass on an
//                     order-preserving key.  Each chunk writes its own 256-bin histogram per
//                     pass (no atomics across workgroups, nothing to clear); every workgroup
//                     of the next pass sums the chunks' histograms and derives the same digit.
//                     Ties at the threshold are taken in ascending linear index: a chunk
//                     starts its ballot scan after the tied keys of the chunks before it.
//                     Deterministic: the selected set is unique.
#include "device.hpp"
#include "kernels.hpp"

namespace sage {
namespace {

constexpr int QBLK = 128, KBLK = 64;

// Block means rounded to bf16; F32OUT stores them widened to fp32 (exact), for the score
// kernel's scalar operand.
template <bool F32OUT>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ x, Rows16 xr, int64_t BH, int64_t N,
                                                   int D, int T, void* __restrict__ means) {
  const int64_t nblk = (N + T - 1) / T;
  const int cg = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= BH * nblk * cg) return;
  const int c8 = (int)(gid % cg);
  const int64_t blk = (gid / cg) % nblk, bh = gid / cg / nblk;
  const int64_t t0 = blk * T;
  const int rows = (int)((N - t0) < T ? (N - t0) : T);
  const uint16_t* p = x + xr.at(bh, t0) + c8 * 8;
  const int64_t sn = xr.sn;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add_row = [&](v4i raw) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + bf16_to_f32((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1))));
  };
  int t = 0;
  for (; t + 16 <= rows; t += 16) {   // 16 row loads in flight, then the adds in token order
    v4i raw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) raw[j] = *(const v4i*)(p + (int64_t)(t + j) * sn);
#pragma unroll
    for (int j = 0; j < 16; ++j) add_row(raw[j]);
  }
  for (; t < rows; ++t) add_row(*(const v4i*)(p + (int64_t)t * sn));
  v4i o;
#pragma unroll
  for (int w = 0; w < 4; ++w) o[w] = (int)pack_bf16x2(s[2 * w] / (float)rows, s[2 * w + 1] / (float)rows);
  const int64_t at = (bh * nblk + blk) * D + c8 * 8;
  if (F32OUT) {
    v4i lo, hi;   // a bf16 is the top half of its fp32
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      lo[2 * w] = o[w] << 16;
      lo[2 * w + 1] = o[w] & (int)0xffff0000u;
      hi[2 * w] = o[2 + w] << 16;
      hi[2 * w + 1] = o[2 + w] & (int)0xffff0000u;
    }
    *(v4i*)((float*)means + at) = lo;
    *(v4i*)((float*)means + at + 4) = hi;
  } else {
    *(v4i*)((uint16_t*)means + at) = o;
  }
}

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);   // -0 -> +0, so equal scores give equal keys
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool pair_valid(int64_t qb, int64_t kb, int causal) {
  return !causal || (int64_t)KBLK * kb <= (int64_t)QBLK * qb + QBLK - 1;
}

constexpr int CHUNK_QB = 16;   // Q blocks per score workgroup = per selection chunk

// chunk histograms in the workspace: [pass][b*Hq+h][chunk][256]
__device__ __forceinline__ int64_t hist_at(int pass, int64_t bhq, int64_t chunk, int64_t BH, int64_t S) {
  return (((int64_t)pass * BH + bhq) * S + chunk) * 256;
}

// block: (group of 16 Q blocks, b*Hq+h); thread: K blocks tid + {0, 256} + 512 i (a wave's
// score stores stay contiguous).  The 16
// fp32 Q-block means sit in LDS (every lane reads the same address: a broadcast); one LDS
// read of 4 channels feeds the fmas of both K blocks.
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qbar, const uint16_t* __restrict__ kbar,
                                                    int64_t Hq, int64_t Hkv, int64_t nQB, int64_t nKB, int D,
                                                    int causal, float* __restrict__ scores,
                                                    uint32_t* __restrict__ chist) {
  __shared__ float qs[16 * 128];
  __shared__ uint32_t hist[256];
  const int64_t bhq = blockIdx.y;
  const int64_t b = bhq / Hq, h = bhq % Hq, g = h / (Hq / Hkv);
  const int64_t qb0 = (int64_t)blockIdx.x * 16;
  const int nq = (int)((nQB - qb0) < 16 ? (nQB - qb0) : 16);
  hist[threadIdx.x] = 0;
  const float* q_base = qbar + (bhq * nQB + qb0) * D;
  for (int i = threadIdx.x * 4; i < 16 * D; i += 256 * 4)   // row stride 128 in LDS (D <= 128)
    *(v4f*)&qs[(i / D) * 128 + i % D] = i < nq * D ? *(const v4f*)(q_base + i) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();
  const uint16_t* kb_base = kbar + (b * Hkv + g) * nKB * D;
  for (int64_t kb0 = threadIdx.x; kb0 < nKB; kb0 += 512) {
    const bool two = kb0 + 256 < nKB;
    float acc[2][16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][r] = acc[1][r] = 0.0f;
    const uint16_t* kr0 = kb_base + kb0 * D;
    const uint16_t* kr1 = two ? kr0 + 256 * (int64_t)D : kr0;   // without a partner: itself again
    for (int c0 = 0; c0 < D; c0 += 8) {   // one 16-byte load per K row and 8 channels
      const v4i r0 = *(const v4i*)(kr0 + c0), r1 = *(const v4i*)(kr1 + c0);
      float k0[8], k1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        k0[e] = bf16_to_f32((uint16_t)((uint32_t)r0[e >> 1] >> (16 * (e & 1))));
        k1[e] = bf16_to_f32((uint16_t)((uint32_t)r1[e >> 1] >> (16 * (e & 1))));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
          const v4f qv = *(const v4f*)&qs[r * 128 + c0 + 4 * h4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[0][r] = __builtin_fmaf(qv[e], k0[4 * h4 + e], acc[0][r]);
            acc[1][r] = __builtin_fmaf(qv[e], k1[4 * h4 + e], acc[1][r]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t kb = kb0 + 256 * u;
      if (u == 1 && !two) break;
      for (int r = 0; r < nq; ++r) {
        scores[(bhq * nQB + qb0 + r) * nKB + kb] = acc[u][r];
        if (pair_valid(qb0 + r, kb, causal)) atomicAdd(&hist[order_key(acc[u][r]) >> 24], 1u);
      }
    }
  }
  __syncthreads();
  chist[hist_at(0, bhq, blockIdx.x, gridDim.y, gridDim.x) + threadIdx.x] = hist[threadIdx.x];
}

constexpr int SEL_PASSES = 4;

struct SelState {
  uint32_t prefix, pmask;   // key bits fixed so far, and which bits those are
  uint32_t remaining;       // keys with that prefix still to take
  uint32_t eq;              // keys with that prefix
};

// Replays passes 0..np-1 from the chunk histograms: the digit of a pass is the highest bin
// whose suffix count (keys with this prefix and a digit >= the bin) reaches `remaining`.
// Stops after the pass that leaves every key with the prefix selected (remaining == eq);
// later passes are then neither built nor read.  Thread t of the 256 holds bin t; all
// threads return the same state.  sh: 10 words of LDS.
__device__ SelState resolve(const uint32_t* __restrict__ chist, int64_t bhq, int64_t BH, int64_t S, int np,
                            uint32_t n_sel, uint32_t* sh) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // bin t summed over the chunks, for every pass up front: the loads of all passes are
  // independent, so up to 64 go out at once (a pass decided early leaves the later
  // histograms unwritten; their sums are then never used)
  uint32_t cnt[SEL_PASSES] = {0u, 0u, 0u, 0u};
  for (int64_t s0 = 0; s0 < S; s0 += 16) {
    uint32_t x[SEL_PASSES][16];
#pragma unroll
    for (int p = 0; p < SEL_PASSES; ++p)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        x[p][j] = (p < np && s0 + j < S) ? chist[hist_at(p, bhq, s0 + j, BH, S) + t] : 0u;
#pragma unroll
    for (int p = 0; p < SEL_PASSES; ++p)
#pragma unroll
      for (int j = 0; j < 16; ++j) cnt[p] += x[p][j];
  }
  SelState st{0u, 0u, n_sel, 0u};
#pragma unroll
  for (int p = 0; p < SEL_PASSES; ++p) {
    if (p >= np) break;
    const uint32_t c = cnt[p];
    uint32_t suf = c;   // sum of the counts of bins >= t
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(suf, off);
      if (lane + off < 64) suf += o;
    }
    if (lane == 0) sh[wv] = suf;
    __syncthreads();
    for (int w = wv + 1; w < 4; ++w) suf += sh[w];
    const uint64_t ge = __ballot(suf >= st.remaining);
    if (lane == 0) sh[4 + wv] = (uint32_t)__popcll(ge);
    __syncthreads();
    const int n_ge = (int)(sh[4] + sh[5] + sh[6] + sh[7]);   // suffix counts fall with the bin
    const int d = n_ge > 0 ? n_ge - 1 : 0;
    if (t == d) {
      sh[8] = suf - c;   // keys above the digit: all taken
      sh[9] = c;
    }
    __syncthreads();
    st.remaining -= sh[8];
    st.eq = sh[9];
    st.prefix |= (uint32_t)d << (24 - 8 * p);
    st.pmask |= 255u << (24 - 8 * p);
    __syncthreads();   // sh is rewritten by the next pass
    if (st.remaining == st.eq) break;
  }
  return st;
}

constexpr int SPT = 32;   // scores per thread held in registers when a chunk has <= 256 * SPT pairs

// A chunk's scores, loaded before the histograms are resolved so that both waits overlap.
struct ChunkScores {
  float v[SPT];
  bool held;   // false: the chunk is larger; its scores are streamed in batches instead
};

__device__ __forceinline__ void load_chunk(const float* __restrict__ sc, int64_t i0, int64_t i1, ChunkScores& cs) {
  cs.held = i1 - i0 <= (int64_t)SPT * 256;
  if (!cs.held) return;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int64_t i = i0 + j * 256 + (int64_t)threadIdx.x;
    cs.v[j] = i < i1 ? sc[i] : 0.0f;
  }
}

// f(i, score) for every pair index i in [i0, i1) of this thread (i = i0 + t mod 256)
template <class F>
__device__ __forceinline__ void for_chunk(const float* __restrict__ sc, int64_t i0, int64_t i1, const ChunkScores& cs,
                                          F&& f) {
  const int t = threadIdx.x;
  if (cs.held) {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int64_t i = i0 + j * 256 + t;
      if (i < i1) f(i, cs.v[j]);
    }
    return;
  }
  for (int64_t base = i0; base < i1; base += 8 * 256) {
    float v[8];   // eight loads in flight per thread
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t i = base + j * 256 + t;
      v[j] = i < i1 ? sc[i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t i = base + j * 256 + t;
      if (i < i1) f(i, v[j]);
    }
  }
}

// Pass `pass` (1..3) of chunk blockIdx.x of head blockIdx.y: histogram of the next key byte
// over the valid keys that carry the prefix fixed by the earlier passes.
__global__ __launch_bounds__(256) void hist_kernel(const float* __restrict__ scores, int64_t nQB, int64_t nKB,
                                                   int causal, int64_t n_sel, int pass,
                                                   uint32_t* __restrict__ chist) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[10];
  const int64_t chunk = blockIdx.x, bhq = blockIdx.y, S = gridDim.x, BH = gridDim.y;
  const int t = threadIdx.x;
  if (n_sel <= 0) return;   // nothing is selected; mask_kernel reads no histogram then
  const int64_t qe = (chunk + 1) * CHUNK_QB < nQB ? (chunk + 1) * CHUNK_QB : nQB;
  const int64_t i0 = chunk * CHUNK_QB * nKB, i1 = qe * nKB;
  const float* sc = scores + bhq * nQB * nKB;
  ChunkScores cs;
  load_chunk(sc, i0, i1, cs);
  const SelState st = resolve(chist, bhq, BH, S, pass, (uint32_t)n_sel, sh);
  if (st.remaining == st.eq) return;   // decided by an earlier pass
  hist[t] = 0;
  __syncthreads();
  const int shift = 24 - 8 * pass;
  for_chunk(sc, i0, i1, cs, [&](int64_t i, float x) {
    const uint32_t qb = (uint32_t)i / (uint32_t)nKB, kb = (uint32_t)i - qb * (uint32_t)nKB;
    if (!pair_valid(qb, kb, causal)) return;
    const uint32_t key = order_key(x);
    if ((key & st.pmask) == st.prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
  });
  __syncthreads();
  chist[hist_at(pass, bhq, chunk, BH, S) + t] = hist[t];
}

// Mask of chunk blockIdx.x of head blockIdx.y.
__global__ __launch_bounds__(256) void mask_kernel(const float* __restrict__ scores, int64_t nQB, int64_t nKB,
                                                   int causal, int64_t n_sel, const uint32_t* __restrict__ chist,
                                                   uint8_t* __restrict__ mask) {
  __shared__ uint32_t sh[10];
  __shared__ uint32_t wave_tot[4];
  const int64_t chunk = blockIdx.x, bhq = blockIdx.y, S = gridDim.x, BH = gridDim.y;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t qe = (chunk + 1) * CHUNK_QB < nQB ? (chunk + 1) * CHUNK_QB : nQB;
  const int64_t i0 = chunk * CHUNK_QB * nKB, i1 = qe * nKB;
  const float* sc = scores + bhq * nQB * nKB;
  uint8_t* mk = mask + bhq * nQB * nKB;
  if (n_sel <= 0) {
    for (int64_t i = i0 + t; i < i1; i += 256) mk[i] = 0;
    return;
  }
  ChunkScores cs;
  load_chunk(sc, i0, i1, cs);
  const SelState st = resolve(chist, bhq, BH, S, SEL_PASSES, (uint32_t)n_sel, sh);
  if (st.remaining == st.eq) {
    // every key carrying the prefix is taken (the bits below it are zero): key >= prefix
    for_chunk(sc, i0, i1, cs, [&](int64_t i, float x) {
      const uint32_t qb = (uint32_t)i / (uint32_t)nKB;
      const bool valid = pair_valid(qb, (uint32_t)i - qb * (uint32_t)nKB, causal);
      mk[i] = (uint8_t)(valid && order_key(x) >= st.prefix);
    });
    return;
  }
  // All four bytes fixed: prefix is the threshold key, of which `remaining` are taken, lowest
  // index first.  Tied keys in the chunks before this one come first.
  const uint32_t T = st.prefix;
  uint32_t before_chunks = 0;
  for (int64_t c = t; c < chunk; c += 256) before_chunks += chist[hist_at(3, bhq, c, BH, S) + (T & 255u)];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) before_chunks += __shfl_xor(before_chunks, off);
  if (lane == 0) wave_tot[wv] = before_chunks;
  __syncthreads();
  uint32_t taken_eq = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
  __syncthreads();
  for (int64_t base = i0; base < i1; base += 256) {
    const int64_t i = base + t;
    bool valid = false;
    uint32_t key = 0;
    if (i < i1) {
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
    const uint32_t chunk_eq = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    if (i < i1) mk[i] = (uint8_t)(valid && (key > T || (eq && before < st.remaining)));
    taken_eq += chunk_eq;
    __syncthreads();
  }
}

// Sink-aware static selection ("Search Your Block Floating Point Scales!", Method >
// ScaleSearchAttention: the first and the last blocks of the KV cache stay at full
// precision).  For Q block qb, with kl its last causal-valid K block (nKB - 1 when not
// causal), K blocks kb <= kl with kb < n_first or kb > kl - n_last are marked.
__global__ __launch_bounds__(256) void sink_mask_kernel(int64_t total, int64_t nQB, int64_t nKB, int n_first,
                                                        int n_last, int causal, uint8_t* __restrict__ mask) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t kb = i % nKB, qb = (i / nKB) % nQB;
  int64_t kl = nKB - 1;
  if (causal) {
    const int64_t lim = (QBLK * qb + QBLK - 1) / KBLK;
    kl = lim < kl ? lim : kl;
  }
  mask[i] = (uint8_t)(kb <= kl && (kb < n_first || kb > kl - n_last));
}

}  // namespace

hipError_t launch_sink_mask(int64_t BH, int64_t N, int n_first, int n_last, int causal, uint8_t* mask, hipStream_t st) {
  const int64_t nQB = (N + QBLK - 1) / QBLK, nKB = (N + KBLK - 1) / KBLK, total = BH * nQB * nKB;
  if (total == 0) return hipSuccess;
  sink_mask_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(total, nQB, nKB, n_first, n_last, causal, mask);
  return hipGetLastError();
}

size_t thrift_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int D) {
  const int64_t nQB = (N + QBLK - 1) / QBLK, nKB = (N + KBLK - 1) / KBLK;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const int64_t S = (nQB + CHUNK_QB - 1) / CHUNK_QB;
  return up((size_t)(B * Hq * nQB * D) * 4) + up((size_t)(B * Hkv * nKB * D) * 2) + up((size_t)(B * Hq * nQB * nKB) * 4) +
         (size_t)SEL_PASSES * (size_t)(B * Hq * S) * 256 * 4;
}

hipError_t launch_thrift_select(const uint16_t* q, const Rows16& qr, const uint16_t* ks, const Rows16& kr, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t N, int D, double frac, int causal, uint8_t* mask,
                                void* ws, hipStream_t st) {
  const int64_t nQB = (N + QBLK - 1) / QBLK, nKB = (N + KBLK - 1) / KBLK;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  float* qbar = (float*)ws;   // Q block means as fp32 (exact widenings of the bf16 means)
  uint16_t* kbar = (uint16_t*)((char*)ws + up((size_t)(B * Hq * nQB * D) * 4));
  float* scores = (float*)((char*)kbar + up((size_t)(B * Hkv * nKB * D) * 2));
  uint32_t* chist = (uint32_t*)((char*)scores + up((size_t)(B * Hq * nQB * nKB) * 4));
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
  pool_kernel<true><<<(unsigned)((t + 255) / 256), 256, 0, st>>>(q, qr, B * Hq, N, D, QBLK, qbar);
  t = B * Hkv * nKB * cg;
  pool_kernel<false><<<(unsigned)((t + 255) / 256), 256, 0, st>>>(ks, kr, B * Hkv, N, D, KBLK, kbar);
  dim3 g((unsigned)((nQB + CHUNK_QB - 1) / CHUNK_QB), (unsigned)(B * Hq));
  score_kernel<<<g, 256, 0, st>>>(qbar, kbar, Hq, Hkv, nQB, nKB, D, causal, scores, chist);
  for (int pass = 1; pass < SEL_PASSES; ++pass)
    hist_kernel<<<g, 256, 0, st>>>(scores, nQB, nKB, causal, n_sel, pass, chist);
  mask_kernel<<<g, 256, 0, st>>>(scores, nQB, nKB, causal, n_sel, chist, mask);
  return hipGetLastError();
}

}  // namespace sage
