// Decode-shaped attention on a KV cache held in NVFP4 — "Search Your Block Floating Point
// Scales!", Method > ScaleSearchAttention (the KV cache kept in 4 bits).  A few new query rows
// attend to a long cache whose K and V rows are NVFP4 along D: per token and 16-channel group,
// 8 code bytes (two E2M1 codes each, even element in the low nibble) and one UE4M3 scale, the
// layout sage_quantize_blocks writes for blocks of (1, 16).  Q stays 16-bit and P fp32.
//
// The work is reading the cache (144 bytes per key per KV head at d = 128), so the kernel is
// shaped for HBM rather than for the matrix cores:
//   * split along the keys: a workgroup takes 512 keys of one (b, KV head) for RG query rows
//     (the rows are the q-heads of the KV head's group times the new tokens);
//   * lane = (key slot t, channel group g): 8 lanes cover a key's 128 channels, so a wave
//     reads 8 whole K and V rows per step (512 contiguous bytes each), and the codes of the
//     next 8 steps are in flight while a step's arithmetic runs;
//   * a key's dot products are summed over its 8 lanes with DPP; every lane of the key then
//     holds the same score, so each key slot keeps its own running max and sum and no value
//     crosses slots until the end, when slots, waves and splits are merged (log-sum-exp);
//   * the running max moves only when a score passes it by 16 (log2 units): P stays fp32 and
//     at most 2^16, and the rescale of O leaves the step loop almost always untaken.
// decode_combine_kernel merges the splits and writes O.
#include "device.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace sage {
namespace {

constexpr int DK = 128;             // head dimension
constexpr int DEC_CHUNK = 1024;     // keys per split workgroup
constexpr int DEC_THREADS = 256;    // 4 waves x 8 key slots
constexpr float kLazy = 16.0f;      // headroom of the running max, log2 units

struct DecodeArgs {
  const uint16_t* q;                           // [B, Hq, Nq, 128] 16-bit
  const uint8_t *kc, *ks, *vc, *vs;            // codes [B, Hkv, Nk, 64], scales [B, Hkv, Nk, 8]
  float* part_o;                               // [B * Hkv, nsplit, Rp, 128]
  float* part_ml;                              // [B * Hkv, nsplit, Rp, 2]
  int64_t Hq, Hkv, Nq, Nk, nsplit, R, nrg;     // R = (Hq / Hkv) * Nq rows per KV head; nrg groups of RG
  int q_f16, causal;
  float qscale;                                // sm_scale * log2(e)
};

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// the 16 E2M1 values of 8 code bytes (unscaled), element e = 2 * byte + nibble
__device__ __forceinline__ void e2m1x16(v2i w, float* x) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = (uint32_t)w[h];
    const auto d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 0);   // byte 0: elements 0, 1
    const auto d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 1);
    const auto d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 2);
    const auto d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 3);
    float* y = x + 8 * h;
    y[0] = d0[0]; y[1] = d0[1]; y[2] = d1[0]; y[3] = d1[1];
    y[4] = d2[0]; y[5] = d2[1]; y[6] = d3[0]; y[7] = d3[1];
  }
}

// Dot product of this lane's 16 channels: q as 8 packed 16-bit pairs (the input's own bits),
// the 16 E2M1 codes decoded to the same 16-bit type (exact), fp32 accumulation by dot2.
template <bool F16>
__device__ __forceinline__ float dot16(const uint32_t* qp, v2i w) {
  float acc = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = (uint32_t)w[h];
#pragma unroll
    for (int by = 0; by < 4; ++by) {
      const uint32_t qv = qp[4 * h + by];
      if constexpr (F16) {
        v2h k2;
        if (by == 0) k2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 0);
        else if (by == 1) k2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 1);
        else if (by == 2) k2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 2);
        else k2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 3);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, qv), k2, acc, false);
      } else {
        v2bf k2;
        if (by == 0) k2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 0);
        else if (by == 1) k2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 1);
        else if (by == 2) k2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 2);
        else k2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 3);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, qv), k2, acc, false);
      }
    }
  }
  return acc;
}

template <int RG, bool F16>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(DecodeArgs a) {
  __shared__ float sh_o[4][RG][DK];
  __shared__ float sh_m[4][RG], sh_l[4][RG];
  const int64_t id = blockIdx.x;
  const int64_t rg = id % a.nrg, split = (id / a.nrg) % a.nsplit, bkv = id / a.nrg / a.nsplit;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, t = lane >> 3, g = lane & 7;
  const int64_t G = a.Hq / a.Hkv, b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  constexpr float NEG = -__builtin_inff();

  // this lane's 16 channels of each row, as the input's 16-bit pairs
  uint32_t q[RG][8];
  int qpos[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t row = rg * RG + r;
    const bool act = row < a.R;
    const int64_t rr = act ? row : 0;   // rows past R compute on row 0 and are dropped
    const int64_t hq = kvh * G + rr / a.Nq, i = rr % a.Nq;
    qpos[r] = act ? (int)(a.Nk - a.Nq + i) : -1;   // -1: no key is visible
    const uint16_t* qp = a.q + ((b * a.Hq + hq) * a.Nq + i) * DK + g * 16;
    const v4i w0 = *(const v4i*)qp, w1 = *(const v4i*)(qp + 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[r][e] = (uint32_t)w0[e];
      q[r][4 + e] = (uint32_t)w1[e];
    }
  }
  float m[RG], l[RG], o[RG][16];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    m[r] = NEG;
    l[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) o[r][c] = 0.0f;
  }

  // 32-bit offsets from the (b, KV head)'s cache; keys past the cache read the last key (their
  // scores are masked), so no load needs a guard
  const int Nk = (int)a.Nk, j0 = (int)(split * DEC_CHUNK);
  const uint8_t* kc = a.kc + bkv * a.Nk * 64;
  const uint8_t* vc = a.vc + bkv * a.Nk * 64;
  const uint8_t* ks = a.ks + bkv * a.Nk * 8;
  const uint8_t* vs = a.vs + bkv * a.Nk * 8;
  const bool causal = a.causal != 0;
  const float qs = a.qscale;
  struct Step {
    v2i kc, vc;
    uint32_t ks, vs;
  };
  auto load = [&](int j, Step& s) __attribute__((always_inline)) {
    const uint32_t jc = (uint32_t)(j < Nk ? j : Nk - 1);
    s.kc = *(const v2i*)(kc + jc * 64u + (uint32_t)g * 8u);
    s.vc = *(const v2i*)(vc + jc * 64u + (uint32_t)g * 8u);
    s.ks = ks[jc * 8u + (uint32_t)g];
    s.vs = vs[jc * 8u + (uint32_t)g];
  };
  // steps of 32 keys; a ring of DEPTH steps of codes (18 bytes a lane each) is in flight, each
  // loaded DEPTH steps before its arithmetic
  constexpr int STEPS = DEC_CHUNK / 32, DEPTH = 8;
  static_assert(STEPS % DEPTH == 0, "whole rounds of the ring");
  const int jl = j0 + wv * 8 + t;   // this lane's key in step 0
  Step ring[DEPTH];
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) load(jl + 32 * u, ring[u]);
  for (int st0 = 0; st0 < STEPS; st0 += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int j = jl + 32 * (st0 + u);
      const Step cur = ring[u];
      if (st0 + DEPTH < STEPS) load(j + 32 * DEPTH, ring[u]);   // wave-uniform
      const float sk = e4m3_to_f32(cur.ks) * qs;
      float s[RG];
      bool up = false;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        float acc = dot16<F16>(q[r], cur.kc) * sk;
        acc += lane_xor<1>(acc);   // sum over the key's 8 lanes: every lane gets the same value
        acc += lane_xor<2>(acc);
        acc += lane_xor<4>(acc);
        const bool vis = j < Nk && (causal ? j <= qpos[r] : qpos[r] >= 0);
        s[r] = vis ? acc : NEG;
        up |= s[r] > m[r] + kLazy;   // also the first visible key (m = -inf)
      }
      if (__builtin_amdgcn_ballot_w64(up) != 0) {   // wave-uniform: move the running max
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const bool mv = s[r] > m[r] + kLazy;
          const float alpha = !mv ? 1.0f : (m[r] == NEG ? 0.0f : __builtin_amdgcn_exp2f(m[r] - s[r]));
          l[r] *= alpha;
#pragma unroll
          for (int c = 0; c < 16; ++c) o[r][c] *= alpha;
          m[r] = mv ? s[r] : m[r];
        }
      }
      float x[16];
      e2m1x16(cur.vc, x);
      const float vsc = e4m3_to_f32(cur.vs);
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const float pr = s[r] == NEG ? 0.0f : __builtin_amdgcn_exp2f(s[r] - m[r]);   // m may still be -inf
        l[r] += pr;
        const float ps = pr * vsc;
#pragma unroll
        for (int c = 0; c < 16; ++c) o[r][c] = __builtin_fmaf(ps, x[c], o[r][c]);
      }
    }
  }

  // merge the wave's 8 key slots (lanes that differ in bits 3..5 hold the same channels);
  // both lanes of a pair form the same two products and add them, so they stay equal
#pragma unroll
  for (int mask = 8; mask < 64; mask *= 2)
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const float mo = __shfl_xor(m[r], mask), lo = __shfl_xor(l[r], mask);
      const float M = __builtin_fmaxf(m[r], mo);
      const float wa = M == NEG ? 0.0f : __builtin_amdgcn_exp2f(m[r] - M);
      const float wb = M == NEG ? 0.0f : __builtin_amdgcn_exp2f(mo - M);
      l[r] = l[r] * wa + lo * wb;
#pragma unroll
      for (int c = 0; c < 16; ++c) o[r][c] = o[r][c] * wa + __shfl_xor(o[r][c], mask) * wb;
      m[r] = M;
    }
  if (t == 0) {
#pragma unroll
    for (int r = 0; r < RG; ++r) {
#pragma unroll
      for (int c = 0; c < 16; ++c) sh_o[wv][r][g * 16 + c] = o[r][c];
      if (g == 0) {
        sh_m[wv][r] = m[r];
        sh_l[wv][r] = l[r];
      }
    }
  }
  __syncthreads();
  // merge the 4 waves; write this split's unnormalized O with its max and sum
  const int64_t Rp = a.nrg * RG;
  for (int i = threadIdx.x; i < RG * DK; i += DEC_THREADS) {
    const int r = i / DK, c = i % DK;
    float M = sh_m[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = __builtin_fmaxf(M, sh_m[w][r]);
    float acc = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = M == NEG ? 0.0f : __builtin_amdgcn_exp2f(sh_m[w][r] - M);
      acc += sh_o[w][r][c] * wt;
      L += sh_l[w][r] * wt;
    }
    const int64_t prow = (bkv * a.nsplit + split) * Rp + rg * RG + r;
    a.part_o[prow * DK + c] = acc;
    if (c == 0) {
      a.part_ml[prow * 2] = M;
      a.part_ml[prow * 2 + 1] = L;
    }
  }
}

// out[b, h, i, c] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits.  One
// workgroup per output row (blockIdx.x = bkv * R + row), a thread per channel; the split
// weights are formed once in LDS (splits beyond 1024 are folded in by a loop).
__global__ __launch_bounds__(DK) void decode_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml, int64_t Hq,
                                                            int64_t Hkv, int64_t Nq, int64_t R, int64_t Rp,
                                                            int64_t nsplit, int out_bf16, void* out) {
  __shared__ float wt[1024];
  __shared__ float red[2];
  const int64_t row = blockIdx.x % R, bkv = blockIdx.x / R;
  const int c = threadIdx.x;
  constexpr float NEG = -__builtin_inff();
  auto ml = [&](int64_t s, int k) { return part_ml[((bkv * nsplit + s) * Rp + row) * 2 + k]; };
  float M = NEG;
  for (int64_t s = c; s < nsplit; s += DK) M = __builtin_fmaxf(M, ml(s, 0));
  M = wave_max(M);
  if ((c & 63) == 0) red[c >> 6] = M;
  __syncthreads();
  M = __builtin_fmaxf(red[0], red[1]);
  float num = 0.0f, den = 0.0f;
  for (int64_t s0 = 0; s0 < nsplit; s0 += 1024) {
    const int64_t n = (nsplit - s0) < 1024 ? nsplit - s0 : 1024;
    __syncthreads();
    for (int64_t s = c; s < n; s += DK) wt[s] = __builtin_amdgcn_exp2f(ml(s0 + s, 0) - M);   // no visible key: 0
    __syncthreads();
    for (int64_t s = 0; s < n; ++s) den += ml(s0 + s, 1) * wt[s];
    int64_t s = 0;
    for (; s + 8 <= n; s += 8) {   // eight independent loads in flight
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part_o[((bkv * nsplit + s0 + s + u) * Rp + row) * DK + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) num += v[u] * wt[s + u];
    }
    for (; s < n; ++s) num += part_o[((bkv * nsplit + s0 + s) * Rp + row) * DK + c] * wt[s];
  }
  const int64_t G = Hq / Hkv, b = bkv / Hkv, hq = (bkv % Hkv) * G + row / Nq, qi = row % Nq;
  const int64_t at = ((b * Hq + hq) * Nq + qi) * DK + c;
  const float v = num / den;
  if (out_bf16) ((uint16_t*)out)[at] = f32_to_bf16(v);
  else ((float*)out)[at] = v;
}

int64_t decode_rg(int64_t R) { return R >= 4 ? 4 : (R == 1 ? 1 : (R == 2 ? 2 : 4)); }

}  // namespace

size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk) {
  const int64_t R = (Hq / Hkv) * Nq, RG = decode_rg(R), Rp = (R + RG - 1) / RG * RG;
  const int64_t nsplit = (Nk + DEC_CHUNK - 1) / DEC_CHUNK;
  return (size_t)(B * Hkv * nsplit * Rp) * (DK + 2) * sizeof(float);
}

hipError_t launch_decode(const uint16_t* q, bool q_f16, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                         const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, int causal,
                         float sm_scale, void* out, bool out_bf16, void* ws, hipStream_t st) {
  const int64_t R = (Hq / Hkv) * Nq, RG = decode_rg(R), nrg = (R + RG - 1) / RG, Rp = nrg * RG;
  const int64_t nsplit = (Nk + DEC_CHUNK - 1) / DEC_CHUNK;
  DecodeArgs a;
  a.q = q;
  a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs;
  a.part_o = (float*)ws;
  a.part_ml = (float*)ws + B * Hkv * nsplit * Rp * DK;
  a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.nsplit = nsplit; a.R = R; a.nrg = nrg;
  a.q_f16 = q_f16 ? 1 : 0;
  a.causal = causal;
  a.qscale = (float)((double)sm_scale * 1.4426950408889634);
  const int64_t nwg = B * Hkv * nsplit * nrg;
  auto go = [&](auto rgc, auto f16c) {
    decode_split_kernel<decltype(rgc)::value, decltype(f16c)::value><<<(unsigned)nwg, DEC_THREADS, 0, st>>>(a);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (RG == 4) { if (q_f16) go(std::integral_constant<int, 4>{}, T_{}); else go(std::integral_constant<int, 4>{}, F_{}); }
  else if (RG == 2) { if (q_f16) go(std::integral_constant<int, 2>{}, T_{}); else go(std::integral_constant<int, 2>{}, F_{}); }
  else { if (q_f16) go(std::integral_constant<int, 1>{}, T_{}); else go(std::integral_constant<int, 1>{}, F_{}); }
  decode_combine_kernel<<<(unsigned)(B * Hkv * R), DK, 0, st>>>(a.part_o, a.part_ml, Hq, Hkv, Nq, R, Rp, nsplit,
                                                                 out_bf16 ? 1 : 0, out);
  return hipGetLastError();
}

}  // namespace sage
