// Fused microscaled attention forward for gfx950.
//
// SageAttention3 (microscaled FP4 attention): Q, K, P and V in E2M1 with one E8M0 scale per
// 32 elements along the contraction axis, both products on the scaled FP4 matrix
// instruction with fp32 accumulation.  "Search Your Block Floating Point Scales!"
// (ScaleSearchAttention): NVFP4 operands; the matrix cores here have no UE4M3-scaled FP4
// product, so Q, K and V arrive as FP8 with E8M0 scales (sage_nvfp4_to_mxfp8) and P is
// quantized in-kernel to NVFP4 by max-scaling per 16 keys and then to FP8 the same way.
//
// Work decomposition, schedule and tile movement are those of the INT8 kernel: a workgroup
// of 8 waves owns two adjacent Q blocks of 128 rows (group A = waves 0-3, group B = 4-7,
// 32 rows per wave); S^T = K . Q^T so each lane holds 32 scores of one query row; the two
// groups alternate MFMA and VALU phases one barrier apart; group A moves K/V tiles (and
// their scale bytes) global -> LDS with direct loads during its VALU phase.
//
// Operand layouts of v_mfma_scale_f32_32x32x64_f8f6f4 (measured on the device):
//   FP4: lane (row m, half h) supplies k = 32h .. 32h+31 (nibble i = k - 32h, low nibble
//        first); its own scale byte covers those 32 elements.
//   FP8: lane (m, h) supplies k = 16h .. 16h+15 (bytes 0-15) and 32+16h .. 32+16h+15
//        (bytes 16-31); the scale of k block kb (k = 32kb .. 32kb+31) comes from lane
//        (m, kb).
// Key order inside a tile follows from P being the B operand of O^T = V^T . P^T:
//   FP4: accumulator block b, register r of lane half h holds key 32h + 16b + r, so one
//        lane holds a whole 32-key scale block of P;
//   FP8: it holds key 32b + 16h + r, so a 16-key NVFP4 block of P is one lane's block b and
//        a 32-key FP8 block spans the lane pair (l, l ^ 32).
// The running max is exact (no lazy threshold): P is quantized relative to it, as the
// per-tile algorithm states, so both sides round the same values.
#include "attn_common.hpp"
#include "kernels.hpp"

#include <atomic>

namespace sage {
namespace {

using namespace attn;

struct MxParams {
  const uint8_t* q; const uint8_t* qe;   // codes [B*Hq][N][RB], E8M0 [B*Hq][N][D/32]
  const uint8_t* k; const uint8_t* ke;   // codes [B*Hkv][N][RB], E8M0 [B*Hkv][N][D/32]
  const uint8_t* v; const uint8_t* ve;   // V^T codes [B*Hkv][D][Np*VB/64], E8M0 [B*Hkv][Np/32][D]
  void* out;
  int64_t Hq, Hkv, N, Np, nQB, nKB, nPairs, total_wg;
  float sm_log2;   // sm_scale * log2(e)
  Rows16 outr;     // output rows
};

// LDS stages: K tile + its scales, V^T tile + its scales, two of each.
template <int D, bool FP4>
struct MxLayout {
  static_assert(D == 128, "microscaled attention is built for head dimension 128");
  static constexpr int RB = FP4 ? D / 2 : D;     // bytes of one Q/K row
  static constexpr int VB = FP4 ? KT / 2 : KT;   // bytes of one V^T row within a tile
  static constexpr int K_CH = RB / 16, V_CH = VB / 16;   // 16-byte chunks per row
  static constexpr int K_BYTES = KT * RB, KS_BYTES = KT * 4;   // 4 scale bytes per key row
  static constexpr int V_BYTES = D * VB, VS_BYTES = 2 * D;     // 2 key blocks x D channels
  static constexpr int K_STAGE = K_BYTES + KS_BYTES, V_STAGE = V_BYTES + VS_BYTES;
  static constexpr int V_BASE = 2 * K_STAGE;
  static constexpr int TOTAL = 2 * K_STAGE + 2 * V_STAGE;
  static constexpr int K_ROUNDS = K_BYTES / 4096, V_ROUNDS = V_BYTES / 4096;   // 256 lanes x 16 B
};

// XOR swizzles of the 16-byte chunk index within a row, chosen so that the 16 lanes of one
// ds_read_b128 pass (same lane half, 16 consecutive accumulator rows) hit 16 distinct
// 16-byte bank groups.
template <bool FP4>
__device__ __forceinline__ int k_swz(int row) {
  return FP4 ? (((row >> 2) & 1) | (((row >> 5) & 1) << 1))
             : (((row >> 1) & 1) | (((row >> 2) & 1) << 1) | (((row >> 4) & 1) << 2));
}
template <bool FP4>
__device__ __forceinline__ int v_swz(int row) { return FP4 ? ((row >> 3) & 1) : ((row >> 2) & 3); }

template <bool FP4>
__device__ __forceinline__ int tile_key(int b, int m) {   // accumulator row m of block b -> key in tile
  const int h = (m >> 2) & 1, r = (m >> 3) * 4 + (m & 3);
  return FP4 ? 32 * h + 16 * b + r : 32 * b + 16 * h + r;
}

template <int D, bool FP4>
struct MxDma {
  using L = MxLayout<D, FP4>;
  int koff[L::K_ROUNDS], krow[L::K_ROUNDS], voff[L::V_ROUNDS];
  __device__ __forceinline__ void init(int a, int lane, int64_t Np) {
    const int vrow_bytes = (int)(Np * L::VB / KT);   // V^T row pitch in global memory
#pragma unroll
    for (int i = 0; i < L::K_ROUNDS; ++i) {
      const int pos = (i * 4 + a) * 64 + lane, row = pos / L::K_CH, c = (pos % L::K_CH) ^ k_swz<FP4>(row);
      krow[i] = row; koff[i] = row * L::RB + 16 * c;
    }
#pragma unroll
    for (int i = 0; i < L::V_ROUNDS; ++i) {
      const int pos = (i * 4 + a) * 64 + lane, row = pos / L::V_CH, c = (pos % L::V_CH) ^ v_swz<FP4>(row);
      voff[i] = row * vrow_bytes + 16 * c;
    }
  }
  // K tile t (rows past N re-read row N-1: finite data for masked keys) and, by wave 0, its
  // 64 scale dwords.
  __device__ __forceinline__ void k_tile(const MxParams& p, int64_t bkv, int t, uint8_t* st, int a, int lane) const {
    const int64_t key0 = (int64_t)t * KT;
    const uint8_t* base = p.k + (bkv * p.N + key0) * L::RB;
    const bool full = key0 + KT <= p.N;
#pragma unroll
    for (int i = 0; i < L::K_ROUNDS; ++i) {
      int off = koff[i];
      if (!full && key0 + krow[i] >= p.N) off += (int)((p.N - 1 - key0 - krow[i]) * L::RB);
      __builtin_amdgcn_global_load_lds((const void*)(base + off), (lds_void*)(st + (i * 4 + a) * 1024), 16, 0, 0);
    }
    if (a == 0) {
      const int64_t row = key0 + lane < p.N ? key0 + lane : p.N - 1;
      __builtin_amdgcn_global_load_lds((const void*)(p.ke + (bkv * p.N + row) * 4), (lds_void*)(st + L::K_BYTES), 4, 0, 0);
    }
  }
  // V^T tile t (the token axis is padded to Np, so always in bounds) and, by wave 1, its
  // 2 x D scale bytes.
  __device__ __forceinline__ void v_tile(const MxParams& p, int64_t bkv, int t, uint8_t* st, int a, int lane) const {
    const uint8_t* base = p.v + bkv * D * (p.Np * L::VB / KT) + (int64_t)t * L::VB;
#pragma unroll
    for (int i = 0; i < L::V_ROUNDS; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(base + voff[i]), (lds_void*)(st + (i * 4 + a) * 1024), 16, 0, 0);
    if (a == 1 && lane < L::VS_BYTES / 4) {
      const uint8_t* src = p.ve + (bkv * (p.Np / 32) + 2 * (int64_t)t) * D + 4 * lane;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(st + L::V_BYTES), 4, 0, 0);
    }
  }
};

__device__ __forceinline__ v8i cat8(v4i lo, v4i hi) { return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; }
// An FP4 operand is 4 registers; the builtin's 8-register operand gets an undefined upper
// half (the instruction does not read it), so no zeros are materialized per fragment.
__device__ __forceinline__ v8i pad8(v4i lo) { return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1); }

// ScaleSearch for one 16-key block of P held in one lane ("Search Your Block Floating Point
// Scales!", Method > ScaleSearch, applied to P): besides the max-scale code c0, try the
// candidates of scale mode PS (1: fp32(smax * g_k) for the 8 grid multipliers g_k = 0.85 +
// k * 0.3 / 7; 2: the bit offsets -2, -1, 1 .. 6 on c0 that stay within 0x01..0x7E) and keep
// the first with the least squared error: e = x - E2M1(x * fp32(1 / s)) * s, e * e summed in
// fp32 as a pairwise tree in key order.
// A UE4M3 scale code's value and its fp32 reciprocal (correctly rounded, as the element rule
// states).  The FP8 kernels build the 128-entry table once per workgroup in LDS: the block
// scales of P and every ScaleSearch candidate read it instead of dividing.
struct ScaleRecip {
  float s, r;
};

template <class Row>
__device__ __forceinline__ float p_block_sse(const Row& x, ScaleRecip sr) {
  const float s = sr.s, r = sr.r;
  float se[16];
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[i] * r, x[i + 1] * r, 1.0f, 0);
    const auto xh = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
    // xhat * s is exact in fp32 (E2M1 x UE4M3: at most 6 significant bits), so one fma gives
    // the difference x - xhat * s with the same single rounding as a product and a subtraction
    const float e0 = __builtin_fmaf(-xh[0], s, x[i]), e1 = __builtin_fmaf(-xh[1], s, x[i + 1]);
    se[i] = e0 * e0;
    se[i + 1] = e1 * e1;
  }
#pragma unroll
  for (int w = 1; w < 16; w *= 2)
#pragma unroll
    for (int i = 0; i < 16; i += 2 * w) se[i] = se[i] + se[i + w];
  return se[0];
}

template <int PS, class Row>
__device__ __forceinline__ uint32_t p_scale_search(const Row& x, float smax, uint32_t c0, const ScaleRecip* tab) {
  uint32_t best_c = c0;
  float best = p_block_sse(x, tab[c0 & 127u]);
  if constexpr (PS == 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      constexpr float g[8] = {(float)(0.85 + 0 * 0.3 / 7.0), (float)(0.85 + 1 * 0.3 / 7.0), (float)(0.85 + 2 * 0.3 / 7.0),
                              (float)(0.85 + 3 * 0.3 / 7.0), (float)(0.85 + 4 * 0.3 / 7.0), (float)(0.85 + 5 * 0.3 / 7.0),
                              (float)(0.85 + 6 * 0.3 / 7.0), (float)(0.85 + 7 * 0.3 / 7.0)};
      uint32_t ck = f32_to_e4m3(smax * g[k]);
      ck = ck == 0 ? 1u : ck;
      const float e = p_block_sse(x, tab[ck & 127u]);
      if (e < best) { best = e; best_c = ck; }
    }
  } else if constexpr (PS == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = j < 2 ? j - 2 : j - 1;   // -2, -1, 1, 2, .., 6
      const int ck = (int)c0 + f;
      if (ck >= 0x01 && ck <= 0x7E) {
        const float e = p_block_sse(x, tab[ck]);
        if (e < best) { best = e; best_c = (uint32_t)ck; }
      }
    }
  }
  return best_c;
}

template <int D, bool CAUSAL, bool FP4, bool OUT_BF16, int PS>
__global__ __launch_bounds__(NTHREADS, 1) void attn_mx_kernel(MxParams p) {
  using L = MxLayout<D, FP4>;
  constexpr int NCC = D / 32;     // 32-channel output chunks
  constexpr int NKK = D / 64;     // 64-channel steps of S
  constexpr int FMT = FP4 ? 4 : 0;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ ScaleRecip ue4m3_tab[FP4 ? 1 : 128];   // FP8 kernels: UE4M3 code -> (value, 1 / value)

  const WgMap wm = map_workgroup(p.total_wg, p.nPairs, CAUSAL);
  const int64_t bh = wm.bh, pr = wm.pair;
  const int64_t b = bh / p.Hq, h = bh % p.Hq;
  const int64_t bkv = b * p.Hkv + h / (p.Hq / p.Hkv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, a = w & 3;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t qb = 2 * pr + grp;
  const int64_t qrow0 = qb * QB + 32 * a;
  const int64_t qrow = qrow0 + li;
  const bool row_ok = qrow < p.N;

  auto tiles_of = [&](int64_t q) __attribute__((always_inline)) -> int {
    if (q >= p.nQB) return 0;
    if (!CAUSAL) return (int)p.nKB;
    const int64_t last = (q * QB + QB - 1) / KT + 1;
    return (int)(last < p.nKB ? last : p.nKB);
  };
  const int nTg = tiles_of(qb);
  const int nT = tiles_of(2 * pr + 1) > tiles_of(2 * pr) ? tiles_of(2 * pr + 1) : tiles_of(2 * pr);
  auto active = [&](int t) __attribute__((always_inline)) { return t >= 0 && t < nTg && (!CAUSAL || (int64_t)t * KT <= qrow0 + 31); };
  auto kst = [&](int t) __attribute__((always_inline)) { return smem + (t & 1) * L::K_STAGE; };
  auto vst = [&](int t) __attribute__((always_inline)) { return smem + L::V_BASE + (t & 1) * L::V_STAGE; };

  // ---- per-lane LDS offsets (loop invariant)
  int kro[2][FP4 ? NKK : 2 * NKK];   // K fragment chunks of block b
  int ksro[2];                        // K scale dword of block b
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int row = tile_key<FP4>(bb, li);
    ksro[bb] = L::K_BYTES + 4 * row;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (FP4) {
        kro[bb][kk] = row * L::RB + 16 * ((2 * kk + lh) ^ k_swz<FP4>(row));
      } else {
        kro[bb][2 * kk] = row * L::RB + 16 * ((4 * kk + lh) ^ k_swz<FP4>(row));
        kro[bb][2 * kk + 1] = row * L::RB + 16 * ((4 * kk + 2 + lh) ^ k_swz<FP4>(row));
      }
    }
  }
  int vro[NCC][FP4 ? 1 : 2];
#pragma unroll
  for (int cc = 0; cc < NCC; ++cc) {
    const int row = 32 * cc + li;
    if (FP4) {
      vro[cc][0] = row * L::VB + 16 * (lh ^ v_swz<FP4>(row));
    } else {
      vro[cc][0] = row * L::VB + 16 * (lh ^ v_swz<FP4>(row));
      vro[cc][1] = row * L::VB + 16 * ((2 + lh) ^ v_swz<FP4>(row));
    }
  }

  // ---- Q fragments (B operand of S^T = K Q^T) and Q scales, shifted so byte 2kk is this
  //      lane half's block 2kk + lh
  v8i qf[NKK];
  uint32_t qsc = 0;
  {
    const uint8_t* qr = p.q + (bh * p.N + qrow) * L::RB;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (FP4) {
        qf[kk] = row_ok ? pad8(*(const v4i*)(qr + 32 * kk + 16 * lh)) : v8i{};
      } else {
        qf[kk] = row_ok ? cat8(*(const v4i*)(qr + 64 * kk + 16 * lh), *(const v4i*)(qr + 64 * kk + 32 + 16 * lh)) : v8i{};
      }
    }
    if (row_ok) qsc = *(const uint32_t*)(p.qe + (bh * p.N + qrow) * 4) >> (8 * lh);
  }

  v16f o[NCC];
#pragma unroll
  for (int c = 0; c < NCC; ++c) o[c] = v16f{};
  float m_run = -__builtin_inff(), l_run = 0.0f;
  v16f acc[2];              // S of the tile the next VALU phase works on
  uint32_t pk[FP4 ? 4 : 8]; // P of the tile the next MFMA phase works on
  uint32_t psc = 0;         // its scale byte (this lane's block)

  if (!FP4 && tid < 128) {   // published by the barrier below
    const float sv = e4m3_to_f32((uint32_t)tid);
    ue4m3_tab[tid] = ScaleRecip{sv, sv > 0.0f ? 1.0f / sv : 0.0f};
  }
  MxDma<D, FP4> dma;
  if (grp == 0) {
    dma.init(a, lane, p.Np);
    dma.k_tile(p, bkv, 0, kst(0), a, lane);
  }
  wait_vmem();
  __syncthreads();

  // ---- S of tile t: K fragments and scales from LDS (qk_load), then the matrix products
  v8i kf[2][NKK];
  uint32_t ksc[2];
  auto qk_load = [&](int t) __attribute__((always_inline)) {
    const uint8_t* ks = kst(t);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (FP4) kf[bb][kk] = pad8(*(const v4i*)(ks + kro[bb][kk]));
        else kf[bb][kk] = cat8(*(const v4i*)(ks + kro[bb][2 * kk]), *(const v4i*)(ks + kro[bb][2 * kk + 1]));
      }
      ksc[bb] = *(const uint32_t*)(ks + ksro[bb]);   // shifted at its use: no early wait
    }
  };
  auto qk_mfma = [&](int t) __attribute__((always_inline)) {
    (void)t;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const uint32_t kscb = ksc[bb] >> (8 * lh);
      v16f s = v16f{};
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[bb][0], qf[0], s, FMT, FMT, 0, kscb, 0, qsc);
      if (NKK > 1) s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[bb][1], qf[1], s, FMT, FMT, 2, kscb, 2, qsc);
      acc[bb] = s;
    }
  };

  // ---- VALU phase: softmax of tile t, P quantized into pk / psc
  auto valu_phase = [&](int t) __attribute__((always_inline)) {
    if (!active(t)) return;
    const int64_t key0 = (int64_t)t * KT;
    v16f (&s)[2] = acc;   // worked on in place: a copy would cost 32 moves a tile
    if ((key0 + KT > p.N) || (CAUSAL && key0 + KT - 1 > qrow0)) {   // causal diagonal or ragged tile
      // 32-bit key indices (N <= 2^24)
      const int k0 = (int)key0 + (FP4 ? 32 * lh : 16 * lh), n32 = (int)p.N, q32 = (int)qrow;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kg = k0 + (FP4 ? 16 * bb : 32 * bb) + r;
          if (kg >= n32 || (CAUSAL && kg > q32)) s[bb][r] = -__builtin_inff();
        }
    }
    float mb[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      mb[bb] = s[bb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mb[bb] = __builtin_fmaxf(mb[bb], s[bb][r]);
    }
    const float mlane = __builtin_fmaxf(mb[0], mb[1]);
    const float mt = halves_max(mlane) * p.sm_log2;   // tile row max in log2 units
    if (__builtin_amdgcn_ballot_w64(mt > m_run) != 0) {   // wave-uniform: move the running max
      const float m_new = __builtin_fmaxf(m_run, mt);
      const float alpha = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < NCC; ++c) o[c] *= alpha;
    }
    const float dq = p.sm_log2, moff = m_run;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[bb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r], dq, -moff));
    float ps[16];   // the row sum as a pairwise tree (short dependency chains)
#pragma unroll
    for (int r = 0; r < 16; ++r) ps[r] = s[0][r] + s[1][r];
#pragma unroll
    for (int w2 = 1; w2 < 16; w2 *= 2)
#pragma unroll
      for (int r = 0; r < 16; r += 2 * w2) ps[r] = ps[r] + ps[r + w2];
    l_run += ps[0];
    if (FP4) {
      // one E8M0 block = this lane's 32 keys; its largest P is exp2 of the lane max
      const float amax = __builtin_amdgcn_exp2f(__builtin_fmaf(mlane, dq, -moff));
      const int e = mx_exp_e2m1_frexp(amax);
      // the conversion divides by 2^(exponent of its scale operand): codes E2M1(P * 2^-e)
      // (an all-zero block, e = -127, converts with 2^-126: its codes are 0 either way)
      const float f = __uint_as_float((uint32_t)(127 + (e < -126 ? -126 : e)) << 23);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {   // nibble 8wd + j = key 32lh + 16(wd/2) + 8(wd%2) + j
        const int bb = wd >> 1, r0 = 8 * (wd & 1);
        uint32_t x = 0;
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[bb][r0], s[bb][r0 + 1], f, 0);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[bb][r0 + 2], s[bb][r0 + 3], f, 1);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[bb][r0 + 4], s[bb][r0 + 5], f, 2);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[bb][r0 + 6], s[bb][r0 + 7], f, 3);
        pk[wd] = x;
      }
      psc = (uint32_t)(e + 127);
    } else {
      // NVFP4 per 16 keys (block bb of this lane): c0 = UE4M3(amax / 6) (0 -> 0x01),
      // codes E2M1(P * fp32(1 / s)); then per 32 keys (block bb of both lane halves):
      // E = smallest with 448 * 2^E >= max |xhat|, FP8 = E4M3(xhat * 2^-E).
      float sc[2], rc[2], am[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const float amax = __builtin_amdgcn_exp2f(__builtin_fmaf(mb[bb], dq, -moff));
        uint32_t c0 = f32_to_e4m3(amax / 6.0f);
        c0 = c0 == 0 ? 1u : c0;
        if constexpr (PS != 0) c0 = p_scale_search<PS>(s[bb], amax / 6.0f, c0, ue4m3_tab);
        const ScaleRecip sr = ue4m3_tab[c0 & 127u];
        sc[bb] = sr.s;
        rc[bb] = sr.r;
        // largest |xhat| of the block: E2M1 rounding is monotonic, so it is the max element's
        const uint32_t cm = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, amax * rc[bb], 0.0f, 1.0f, 0);
        am[bb] = halves_max(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cm, 1.0f, 0)[0] * sc[bb]);
      }
      float tb[2];
      int E[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        E[bb] = mx_exp_e4m3(am[bb]);
        tb[bb] = sc[bb] * __uint_as_float((uint32_t)(127 - E[bb]) << 23);   // s * 2^-E, exact
      }
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {   // byte 4wd + j = key 32(wd/4) + 16lh + 4(wd%4) + j
        const int bb = wd >> 2, r0 = 4 * (wd & 3);
        const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s[bb][r0] * rc[bb], s[bb][r0 + 1] * rc[bb], 1.0f, 0);
        const uint32_t c2 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, s[bb][r0 + 2] * rc[bb], s[bb][r0 + 3] * rc[bb], 1.0f, 1);
        const auto x01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c2, 1.0f, 0);
        const auto x23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c2, 1.0f, 1);
        const uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(x01[0] * tb[bb], x01[1] * tb[bb], 0u, false);
        pk[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(x23[0] * tb[bb], x23[1] * tb[bb], wv, true);
      }
      psc = (uint32_t)((lh ? E[1] : E[0]) + 127);
    }
  };

  // ---- MFMA phase: O += P(t) V(t), then S of tile t+1
  auto mfma_phase = [&](int t) __attribute__((always_inline)) {
    const bool next = active(t + 1);
    if (next) qk_load(t + 1);
    if (active(t)) {
      const uint8_t* vs = vst(t);
      v4i vlo[NCC], vhi[NCC];
      uint32_t vsc[NCC];
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        vlo[cc] = *(const v4i*)(vs + vro[cc][0]);
        if (!FP4) vhi[cc] = *(const v4i*)(vs + vro[cc][1]);
        vsc[cc] = vs[L::V_BYTES + lh * D + 32 * cc + li];
      }
      // all fragment reads in flight before the first product (else each product waits out
      // its own read's latency)
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        __asm__ volatile("" : "+v"(vlo[cc]));
        if (!FP4) __asm__ volatile("" : "+v"(vhi[cc]));
        __asm__ volatile("" : "+v"(vsc[cc]));
      }
      v8i vf[NCC];
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) vf[cc] = FP4 ? pad8(vlo[cc]) : cat8(vlo[cc], vhi[cc]);
      const v8i pf = FP4 ? pad8(v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]})
                         : v8i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc)
        o[cc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[cc], pf, o[cc], FMT, FMT, 0, vsc[cc], 0, psc);
    }
    if (next) qk_mfma(t + 1);
  };

  // ---- the schedule (as in the INT8 kernel): group B one barrier behind group A
  if (grp == 1) phase_barrier();
  for (int t = -1; t < nT; ++t) {
    // group A issues the next tiles at the start of its MFMA phase (its vector slots are idle
    // there): the stages of K(t) and V(t-1) they fill were last read, by group B, in the phase
    // before, and the loads get two phases to land
    if (grp == 0) {
      if (t + 2 < nT) dma.k_tile(p, bkv, t + 2, kst(t + 2), a, lane);
      if (t + 1 < nT) dma.v_tile(p, bkv, t + 1, vst(t + 1), a, lane);
    }
    mfma_phase(t);
    phase_barrier();
    valu_phase(t + 1);
    if (grp == 0) wait_vmem();
    phase_barrier();
  }
  if (grp == 0) phase_barrier();

  // ---- epilogue: O / l; lane (li, lh) holds row qrow, channels 32cc + 8(r/4) + 4lh + (r%4)
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_ok) {
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = 32 * cc + 8 * g + 4 * lh;
        const float v0 = o[cc][4 * g] * inv, v1 = o[cc][4 * g + 1] * inv, v2 = o[cc][4 * g + 2] * inv,
                    v3 = o[cc][4 * g + 3] * inv;
        const int64_t off = p.outr.at(bh, qrow) + ch;
        if (OUT_BF16) *(v2i*)((uint16_t*)p.out + off) = v2i{(int)pack_bf16x2(v0, v1), (int)pack_bf16x2(v2, v3)};
        else *(v4f*)((float*)p.out + off) = v4f{v0, v1, v2, v3};
      }
  }
}

template <int D, bool CAUSAL, bool FP4, bool OUT_BF16, int PS>
hipError_t launch_mx_cfg(const MxParams& p, hipStream_t st) {
  using L = MxLayout<D, FP4>;
  auto kern = attn_mx_kernel<D, CAUSAL, FP4, OUT_BF16, PS>;
  // The dynamic-LDS limit is set once per device (bit d of the mask: done on device d), from
  // any thread; devices past 63 set it on every launch.
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit == 0 || (attr_set.load(std::memory_order_acquire) & bit) == 0) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL);
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  if (p.total_wg == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.total_wg), dim3(NTHREADS), L::TOTAL, st, p);
  return hipGetLastError();
}

template <bool CAUSAL, bool FP4, int PS>
hipError_t dispatch_mx(const MxParams& p, bool out_bf16, hipStream_t st) {
  return out_bf16 ? launch_mx_cfg<128, CAUSAL, FP4, true, PS>(p, st) : launch_mx_cfg<128, CAUSAL, FP4, false, PS>(p, st);
}

template <bool CAUSAL>
hipError_t dispatch_nv(const MxParams& p, bool out_bf16, int p_mode, hipStream_t st) {
  if (p_mode == 1) return dispatch_mx<CAUSAL, false, 1>(p, out_bf16, st);
  if (p_mode == 2) return dispatch_mx<CAUSAL, false, 2>(p, out_bf16, st);
  return dispatch_mx<CAUSAL, false, 0>(p, out_bf16, st);
}

}  // namespace

hipError_t launch_attn_mx(const AttnArgs& a, int nvfp4_variant, hipStream_t st) {
  if (a.D != 128) return hipErrorNotSupported;
  MxParams p;
  p.q = (const uint8_t*)a.q_codes; p.qe = (const uint8_t*)a.q_scales;
  p.k = (const uint8_t*)a.k_codes; p.ke = (const uint8_t*)a.k_scales;
  p.v = (const uint8_t*)a.v_codes; p.ve = (const uint8_t*)a.v_scales;
  p.out = a.out;
  p.outr = a.outr;
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N;
  p.Np = (a.N + KT - 1) / KT * KT;
  p.nQB = (a.N + QB - 1) / QB; p.nKB = (a.N + KT - 1) / KT;
  p.nPairs = (p.nQB + 1) / 2;
  p.total_wg = a.B * a.Hq * p.nPairs;
  p.sm_log2 = a.sm_scale * LOG2E;
  const bool causal = a.causal != 0, fp4 = nvfp4_variant == 0;
  if (fp4) return causal ? dispatch_mx<true, true, 0>(p, a.out_bf16, st) : dispatch_mx<false, true, 0>(p, a.out_bf16, st);
  return causal ? dispatch_nv<true>(p, a.out_bf16, a.p_scale_mode, st) : dispatch_nv<false>(p, a.out_bf16, a.p_scale_mode, st);
}

}  // namespace sage
