// Fused INT8 attention forward for gfx950.
//
// SageAttention ("Accurate 8-Bit Attention for Plug-and-play Inference Acceleration",
// Technical approach): QK^T on 8-bit Q and smoothed K, P and V kept at 16 bits (here bf16,
// fp32 accumulation); the video-generation variant keeps P and V in FP8 (P scaled by 448,
// V per channel).  ThriftAttention (¶1, ¶3): tiles flagged in a block mask use bf16 Q and
// K_s instead, and every tile feeds one joint online softmax.
//
// Work decomposition: a workgroup (4 waves) owns one Q block of 128 rows of one (b, q-head);
// each wave owns 32 rows.  K/V tiles of 64 keys stream through double-buffered LDS
// (register-staged 16-byte loads).  Per tile and wave:
//   S^T (64 keys x 32 queries) = K . Q^T on v_mfma_i32_32x32x32_i8 (two 32-key halves, D/32
//       k-steps), so each lane holds 32 scores of ONE query row: softmax statistics are
//       per-lane scalars.  K rows are loaded permuted so that lane half h holds the keys
//       32h .. 32h+31 of the tile in register order (key = 32h + 16b + r for accumulator b,
//       register r): the P registers line up with 8 consecutive keys per k-group of the
//       next product.
//   dequantize: s = float(acc) * (s_q * s_k * sm_scale * log2 e); the row max is taken on the
//       raw accumulators and one swap across lane halves (v_permlane32_swap).
//   online softmax in fp32, base 2: the running max only moves (and O, l are rescaled) when
//       a row's tile max exceeds it by more than `tau` (0 for FP8 P, which must stay <= 448).
//   O^T (D x 32) += V^T . P^T on v_mfma_f32_32x32x16_bf16: V^T fragments come straight from
//       the row-major LDS tile through ds_read_b64_tr_b16 (each 16-lane group transposes a
//       4-key x 16-channel block); or on the scaled FP8 MFMA (32x32x64) with V stored
//       channel-major by its quantizer.
// The causal mask is top-left aligned; fully masked tiles are skipped per wave, and Q blocks
// are scheduled heaviest first.  Workgroup ids are remapped so consecutive Q blocks of a head
// run on the same XCD and share its L2.
#include "device.hpp"
#include "kernels.hpp"

namespace sage {
namespace {

constexpr int QB = 128, KT = 64, NTHREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;

struct Params {
  const int8_t* q; const float* qs;
  const int8_t* k; const float* ks;
  const void* v; const float* vs;
  const uint8_t* mask; const uint16_t* qhi; const uint16_t* khi;
  void* out;
  int64_t Hq, Hkv, N, nQB, nKB, total_wg;
  float sm_log2;   // sm_scale * log2(e)
  float tau;       // lazy-rescale threshold (log2 units)
};

template <int D, bool PV8, bool THRIFT>
struct Smem {
  static constexpr int PK = THRIFT ? (2 * D + 16) : (D + 16);   // K tile row pitch, bytes
  static constexpr int PV = PV8 ? 80 : (2 * D + 64);            // V tile row pitch, bytes
  static constexpr int K_BYTES = KT * PK;
  static constexpr int V_BYTES = PV8 ? D * PV : KT * PV;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int TOTAL = 2 * STAGE;
};

__device__ __forceinline__ int tile_key(int b, int m) {   // accumulator row m of half b -> key in tile
  return ((m >> 2) & 1) * 32 + 16 * b + (m >> 3) * 4 + (m & 3);
}

// v_permlane32_swap on (x, x) returns, in some order depending on the lane half, this lane's
// value and the value of lane l ^ 32; max and sum of the pair are the same in both halves.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, bool PV8, bool THRIFT, bool VF16>
struct Loader {
  // per-thread register staging for one tile
  static constexpr int K_CH = KT * D / 16 / NTHREADS;                 // 16-byte chunks of int8 K
  static constexpr int KH_CH = THRIFT ? KT * D * 2 / 16 / NTHREADS : 0;  // bf16 K_s
  static constexpr int V_CH = PV8 ? D * KT / 16 / NTHREADS : KT * D * 2 / 16 / NTHREADS;
  v4i kreg[K_CH > KH_CH ? K_CH : KH_CH];
  v4i vreg[V_CH];
  bool hi;

  __device__ __forceinline__ void load(const Params& p, int64_t bkv, int t, bool hi_tile, int tid) {
    hi = hi_tile;
    const int64_t key0 = (int64_t)t * KT;
    if (!hi_tile) {
#pragma unroll
      for (int i = 0; i < K_CH; ++i) {
        const int c = tid + NTHREADS * i, row = c / (D / 16), col = c % (D / 16);
        kreg[i] = (key0 + row < p.N) ? *(const v4i*)(p.k + ((bkv * p.N + key0 + row) * D + col * 16)) : v4i{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int i = 0; i < KH_CH; ++i) {
        const int c = tid + NTHREADS * i, row = c / (D / 8), col = c % (D / 8);
        kreg[i] = (key0 + row < p.N) ? *(const v4i*)(p.khi + ((bkv * p.N + key0 + row) * D + col * 8)) : v4i{0, 0, 0, 0};
      }
    }
    if (PV8) {   // V^T [D][N] bytes
      const uint8_t* vt = (const uint8_t*)p.v;
#pragma unroll
      for (int i = 0; i < V_CH; ++i) {
        const int c = tid + NTHREADS * i, ch = c / 4, col = c % 4;
        const int64_t tok = key0 + col * 16;
        const uint8_t* src = vt + (bkv * D + ch) * p.N + tok;
        if (tok + 16 <= p.N && (p.N & 15) == 0) {
          vreg[i] = *(const v4i*)src;
        } else {
          uint32_t w[4] = {0, 0, 0, 0};
          for (int j = 0; j < 16; ++j)
            if (tok + j < p.N) w[j >> 2] |= (uint32_t)src[j] << (8 * (j & 3));
          vreg[i] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
      }
    } else {     // V [N][D] 16-bit
      const uint16_t* v = (const uint16_t*)p.v;
#pragma unroll
      for (int i = 0; i < V_CH; ++i) {
        const int c = tid + NTHREADS * i, row = c / (D / 8), col = c % (D / 8);
        v4i x = (key0 + row < p.N) ? *(const v4i*)(v + ((bkv * p.N + key0 + row) * D + col * 8)) : v4i{0, 0, 0, 0};
        if (VF16) {   // fp16 V is read as bf16 (nearest-even) for the bf16 product
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t u = (uint32_t)x[w];
            x[w] = (int)pack_bf16x2(f16_to_f32((uint16_t)(u & 0xffffu)), f16_to_f32((uint16_t)(u >> 16)));
          }
        }
        vreg[i] = x;
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* stage, int tid) const {
    using S = Smem<D, PV8, THRIFT>;
    uint8_t* ks = stage;
    uint8_t* vs = stage + S::K_BYTES;
    if (!hi) {
#pragma unroll
      for (int i = 0; i < K_CH; ++i) {
        const int c = tid + NTHREADS * i, row = c / (D / 16), col = c % (D / 16);
        *(v4i*)(ks + row * S::PK + col * 16) = kreg[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < KH_CH; ++i) {
        const int c = tid + NTHREADS * i, row = c / (D / 8), col = c % (D / 8);
        *(v4i*)(ks + row * S::PK + col * 16) = kreg[i];
      }
    }
    if (PV8) {
#pragma unroll
      for (int i = 0; i < V_CH; ++i) {
        const int c = tid + NTHREADS * i, ch = c / 4, col = c % 4;
        *(v4i*)(vs + ch * S::PV + col * 16) = vreg[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < V_CH; ++i) {
        const int c = tid + NTHREADS * i, row = c / (D / 8), col = c % (D / 8);
        *(v4i*)(vs + row * S::PV + col * 16) = vreg[i];
      }
    }
  }
};

template <int D, bool CAUSAL, bool PV8, bool THRIFT, bool VF16, bool OUT_BF16>
__global__ __launch_bounds__(NTHREADS, 2) void attn_i8_kernel(Params p) {
  using S = Smem<D, PV8, THRIFT>;
  constexpr int NKC = D / 32;    // int8 k-steps of 32 channels
  constexpr int NCC = D / 32;    // 32-channel output chunks
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- workgroup -> (b, h, qb); XCD-aware: consecutive work items on one XCD
  int64_t wg = blockIdx.x;
  if ((p.total_wg & 7) == 0) wg = (wg & 7) * (p.total_wg >> 3) + (wg >> 3);
  const int64_t bh = wg / p.nQB;
  int64_t qb = wg % p.nQB;
  if (CAUSAL) qb = p.nQB - 1 - qb;            // heaviest Q blocks first
  const int64_t b = bh / p.Hq, h = bh % p.Hq;
  const int64_t bkv = b * p.Hkv + h / (p.Hq / p.Hkv);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t qrow0 = qb * QB + 32 * w;     // first row of this wave
  const int64_t qrow = qrow0 + li;            // this lane's query row
  const bool row_ok = qrow < p.N;

  int nT = (int)p.nKB;
  if (CAUSAL) {
    const int64_t last = (qb * QB + QB - 1) / KT + 1;
    nT = (int)(last < p.nKB ? last : p.nKB);
  }
  const uint8_t* mrow = THRIFT ? p.mask + (bh * p.nQB + qb) * p.nKB : nullptr;

  // ---- Q fragments (B operand of the S^T product): row qrow, channels 32kc + 16lh .. +16
  v4i qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    qf[kc] = row_ok ? *(const v4i*)(p.q + (bh * p.N + qrow) * D + 32 * kc + 16 * lh) : v4i{0, 0, 0, 0};
  const float qscale = p.qs[bh * p.nQB + qb];

  v16f o[NCC];
#pragma unroll
  for (int c = 0; c < NCC; ++c) o[c] = v16f{};
  float m_run = -__builtin_inff(), l_run = 0.0f;

  Loader<D, PV8, THRIFT, VF16> ld;
  ld.load(p, bkv, 0, THRIFT ? (mrow[0] != 0) : false, tid);
  ld.store(smem, tid);
  __syncthreads();

  for (int t = 0; t < nT; ++t) {
    const bool hi = THRIFT ? (mrow[t] != 0) : false;
    if (t + 1 < nT) ld.load(p, bkv, t + 1, THRIFT ? (mrow[t + 1] != 0) : false, tid);
    const uint8_t* ks = smem + (t & 1) * S::STAGE;
    const uint8_t* vs = ks + S::K_BYTES;
    const int64_t key0 = (int64_t)t * KT;
    const bool wave_active = !CAUSAL || key0 <= qrow0 + 31;
    if (wave_active) {
      // ---------------- scores S^T for keys 32h + 16b + r
      float s[2][16];
      float dq;
      if (!hi) {
        v16i acc[2] = {v16i{}, v16i{}};
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const v4i kf = *(const v4i*)(ks + tile_key(bb, li) * S::PK + 32 * kc + 16 * lh);
            acc[bb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[kc], acc[bb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[bb][r] = (float)acc[bb][r];
        dq = qscale * p.ks[bkv * p.nKB + t] * p.sm_log2;
      } else {
        v16f acc[2] = {v16f{}, v16f{}};
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const v8bf qh = row_ok ? *(const v8bf*)(p.qhi + (bh * p.N + qrow) * D + 16 * kc + 8 * lh) : v8bf{};
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const v8bf kh = *(const v8bf*)(ks + tile_key(bb, li) * S::PK + 2 * (16 * kc + 8 * lh));
            acc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh, acc[bb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[bb][r] = acc[bb][r];
        dq = p.sm_log2;
      }
      // ---------------- masks (causal diagonal tiles, ragged last tile)
      const bool need_mask = (key0 + KT > p.N) || (CAUSAL && key0 + KT - 1 > qrow0);
      if (need_mask) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t kg = key0 + 32 * lh + 16 * bb + r;
            if (kg >= p.N || (CAUSAL && kg > qrow)) s[bb][r] = -__builtin_inff();
          }
      }
      // ---------------- online softmax (base 2)
      float mx = s[0][0];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[bb][r]);
      mx = halves_max(mx);
      const float mt = mx * dq;                      // tile row max in scaled units (dq >= 0)
      const bool grow = mt > m_run + p.tau;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform: move the running max
        const float m_new = __builtin_fmaxf(m_run, mt);
        const float alpha = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < NCC; ++c) o[c] *= alpha;
      }
      const float moff = (m_run == -__builtin_inff() ? 0.0f : m_run) - (PV8 ? 8.807354922057604f : 0.0f);  // FP8: P * 448
      float pv[2][16];
      float lsum = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r], dq, -moff));
          if (need_mask && s[bb][r] == -__builtin_inff()) e = 0.0f;
          pv[bb][r] = e;
          lsum += e;
        }
      l_run += lsum;
      // ---------------- O^T += V^T P^T
      if (!PV8) {
        uint32_t pk[2][8];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) pk[bb][r >> 1] = pack_bf16x2(pv[bb][r], pv[bb][r + 1]);
        const int g16 = lane >> 4, j = lane & 15;
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
          const int bb = kg >> 1, r0 = 4 * (kg & 1);
          v4i pb = v4i{(int)pk[bb][r0], (int)pk[bb][r0 + 1], (int)pk[bb][r0 + 2], (int)pk[bb][r0 + 3]};
          const v8bf pf = __builtin_bit_cast(v8bf, pb);
#pragma unroll
          for (int cc = 0; cc < NCC; ++cc) {
            const int key = 32 * (g16 >> 1) + 8 * kg + (j >> 2);
            const int ch = 32 * cc + 16 * (g16 & 1) + 4 * (j & 3);
            const uint8_t* a0 = vs + key * S::PV + ch * 2;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(a0));
            const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(a0 + 4 * S::PV));
            const v8bf vf = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[cc], 0, 0, 0);
          }
        }
      } else {
        v8i pf;
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
          const int bb = q4 >> 2, r = 4 * (q4 & 3);
          uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[bb][r], pv[bb][r + 1], 0u, false);
          pf[q4] = (int)__builtin_amdgcn_cvt_pk_fp8_f32(pv[bb][r + 2], pv[bb][r + 3], wv, true);
        }
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
          const uint8_t* a0 = vs + (32 * cc + li) * S::PV + 32 * lh;
          const v4i v0 = *(const v4i*)a0, v1 = *(const v4i*)(a0 + 16);
          const v8i vf = v8i{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          o[cc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[cc], 0, 0, 0, 127, 0, 127);
        }
      }
    }
    if (t + 1 < nT) ld.store(smem + ((t + 1) & 1) * S::STAGE, tid);
    __syncthreads();
  }

  // ---- epilogue: O / l (and the FP8 V channel scales); lane (li, lh) holds row qrow,
  //      channels 32cc + 8(r/4) + 4lh + (r%4).
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_ok) {
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = 32 * cc + 8 * g + 4 * lh;
        float v0 = o[cc][4 * g] * inv, v1 = o[cc][4 * g + 1] * inv, v2 = o[cc][4 * g + 2] * inv, v3 = o[cc][4 * g + 3] * inv;
        if (PV8) {
          const float* vsc = p.vs + bkv * D + ch;
          v0 *= vsc[0]; v1 *= vsc[1]; v2 *= vsc[2]; v3 *= vsc[3];
        }
        const int64_t off = (bh * p.N + qrow) * D + ch;
        if (OUT_BF16) {
          *(v2i*)((uint16_t*)p.out + off) = v2i{(int)pack_bf16x2(v0, v1), (int)pack_bf16x2(v2, v3)};
        } else {
          *(v4f*)((float*)p.out + off) = v4f{v0, v1, v2, v3};
        }
      }
  }
}

template <int D, bool CAUSAL, bool PV8, bool THRIFT, bool VF16, bool OUT_BF16>
hipError_t launch_cfg(const Params& p, hipStream_t st) {
  using S = Smem<D, PV8, THRIFT>;
  auto kern = attn_i8_kernel<D, CAUSAL, PV8, THRIFT, VF16, OUT_BF16>;
  static bool attr_set = false;   // the attribute is per function; setting it twice is harmless
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, S::TOTAL);
    attr_set = true;
  }
  if (p.total_wg == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.total_wg), dim3(NTHREADS), S::TOTAL, st, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool PV8>
hipError_t dispatch_rest(const Params& p, bool thrift, bool vf16, bool out_bf16, hipStream_t st) {
  if (PV8) {
    return out_bf16 ? launch_cfg<D, CAUSAL, true, false, false, true>(p, st)
                    : launch_cfg<D, CAUSAL, true, false, false, false>(p, st);
  }
  if (thrift) {
    if (vf16) return out_bf16 ? launch_cfg<D, CAUSAL, false, true, true, true>(p, st) : launch_cfg<D, CAUSAL, false, true, true, false>(p, st);
    return out_bf16 ? launch_cfg<D, CAUSAL, false, true, false, true>(p, st) : launch_cfg<D, CAUSAL, false, true, false, false>(p, st);
  }
  if (vf16) return out_bf16 ? launch_cfg<D, CAUSAL, false, false, true, true>(p, st) : launch_cfg<D, CAUSAL, false, false, true, false>(p, st);
  return out_bf16 ? launch_cfg<D, CAUSAL, false, false, false, true>(p, st) : launch_cfg<D, CAUSAL, false, false, false, false>(p, st);
}

}  // namespace

hipError_t launch_attn_int8(const AttnArgs& a, int pv_fp8, hipStream_t st) {
  Params p;
  p.q = (const int8_t*)a.q_codes; p.qs = (const float*)a.q_scales;
  p.k = (const int8_t*)a.k_codes; p.ks = (const float*)a.k_scales;
  p.v = a.v_codes; p.vs = (const float*)a.v_scales;
  p.mask = a.mask; p.qhi = a.q_hi; p.khi = a.k_hi;
  p.out = a.out;
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N;
  p.nQB = (a.N + QB - 1) / QB; p.nKB = (a.N + KT - 1) / KT;
  p.total_wg = a.B * a.Hq * p.nQB;
  p.sm_log2 = a.sm_scale * LOG2E;
  p.tau = pv_fp8 ? 0.0f : 8.0f;
  const bool thrift = a.mask != nullptr;
  const bool causal = a.causal != 0;
  if (a.D == 64) {
    if (causal) return pv_fp8 ? dispatch_rest<64, true, true>(p, thrift, a.v_is_f16, a.out_bf16, st)
                              : dispatch_rest<64, true, false>(p, thrift, a.v_is_f16, a.out_bf16, st);
    return pv_fp8 ? dispatch_rest<64, false, true>(p, thrift, a.v_is_f16, a.out_bf16, st)
                  : dispatch_rest<64, false, false>(p, thrift, a.v_is_f16, a.out_bf16, st);
  }
  if (causal) return pv_fp8 ? dispatch_rest<128, true, true>(p, thrift, a.v_is_f16, a.out_bf16, st)
                            : dispatch_rest<128, true, false>(p, thrift, a.v_is_f16, a.out_bf16, st);
  return pv_fp8 ? dispatch_rest<128, false, true>(p, thrift, a.v_is_f16, a.out_bf16, st)
                : dispatch_rest<128, false, false>(p, thrift, a.v_is_f16, a.out_bf16, st);
}

}  // namespace sage
