// Fused INT8 attention forward for gfx950.
//
// SageAttention ("Accurate 8-Bit Attention for Plug-and-play Inference Acceleration",
// Technical approach): QK^T on 8-bit Q and smoothed K, P and V kept at 16 bits (here bf16,
// fp32 accumulation); the video-generation variant keeps P and V in FP8 (P scaled by 448,
// V per channel).  ThriftAttention (¶1, ¶3): tiles flagged in a block mask use bf16 Q and
// K_s instead, and every tile feeds one joint online softmax.
//
// Work decomposition.  A workgroup of 8 waves owns two adjacent Q blocks of 128 rows of one
// (b, q-head); waves 0-3 (group A) take the first block, waves 4-7 (group B) the second, 32
// rows per wave.  Both groups stream the same K/V tiles of 64 keys through LDS.
//
// Per tile and wave:
//   S^T (64 keys x 32 queries) = K . Q^T on v_mfma_i32_32x32x32_i8, so each lane holds 32
//       scores of ONE query row and the softmax statistics are per-lane scalars.  K rows are
//       read permuted so that lane half h holds keys 32h .. 32h+31 of the tile in register
//       order (key = 32h + 16b + r for accumulator b, register r).
//   softmax: s = float(acc) * (s_q s_k sm_scale log2 e); row max over the lane and one
//       v_permlane32_swap; fp32 online softmax in base 2 with the exact running max (P is
//       rounded to bf16 / FP8 relative to it, as the per-tile algorithm states; O and l are
//       rescaled whenever some row of the wave raises its max).
//   O^T (D x 32) += V^T . P^T on v_mfma_f32_32x32x16_bf16 with V^T fragments read from the
//       row-major LDS tile by ds_read_b64_tr_b16 (each 16-lane group transposes a 4-key x
//       16-channel block), or on the scaled FP8 MFMA (32x32x64) with V stored channel-major.
//
// Ping-pong schedule.  Each wave alternates a VALU phase (softmax of tile t) and an MFMA
// phase (P.V of tile t and S of tile t+1; Thrift issues S first).  Group B runs one phase behind group A, so on
// every SIMD (one wave of each group) one wave keeps the matrix core busy while the other
// uses the vector ALU.  Phases are separated by workgroup barriers:
//     phase 2t+2: A = MFMA(t), B = VALU(t);   phase 2t+3: A = VALU(t+1), B = MFMA(t).
// (Both groups run the same straight-line program, offset by one barrier, so the phase code
// exists once and register pressure is that of one wave's program.)
// Group A also moves the tiles: at the start of its VALU phase 2t+3 it issues direct
// global->LDS loads (global_load_lds_dwordx4) of K(t+3) and V(t+2), and at the end of its
// next VALU phase (2t+5) waits for them, leaving that phase's own loads in flight; they are
// first read in phase 2t+6.  K(s) is read in phases 2s, 2s+1 and V(t) in 2t+2, 2t+3, so the
// loads land in the buffers of K(t) and V(t-1): three of each, used round-robin (the loop is
// unrolled by three so every buffer is a compile-time choice).  Tiles never pass through
// registers.
//
// The causal mask is top-left aligned; tiles entirely above a wave's rows are skipped and
// workgroups are scheduled heaviest first.  Workgroup ids are remapped so consecutive Q-block
// pairs of one head run on the same XCD and share its L2.
#include "attn_common.hpp"
#include "device.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace sage {
namespace {

using namespace attn;

// 1.5 * 2^23 and its bit pattern: an int32 x with |x| < 2^22 added to the pattern gives the
// float kMagic + x exactly.
constexpr float kMagic = 12582912.0f;
constexpr int kMagicBits = 0x4B400000;

struct Params {
  const int8_t* q; const float* qs;
  const int8_t* k; const float* ks;
  const void* v; const float* vs;
  const uint8_t* mask; const uint16_t* qhi; const uint16_t* khi;
  void* out;
  int64_t Hq, Hkv, N, Np, nQB, nKB, nPairs, total_wg;
  float sm_log2;     // sm_scale * log2(e), rounded to fp32
  float sm_log2_lo;  // sm_scale * log2(e) - sm_log2 (the FP8-P path carries the product exactly)
  Rows16 vr, qhr, khr, outr;   // rows of the 16-bit V, the Thrift tiles' Q and K_s, the output
};

// LDS: three K tiles (int8 [64][D]) and three V tiles (bf16 [64][D] row-major, or FP8 V^T
// [D][64]), all unpadded with XOR-swizzled 16-byte chunks.  Each tile buffer is a separate
// static array, so the compiler can tell the reads of one buffer from the direct loads still
// in flight into another.
template <int D, bool PV8>
struct Smem {
  static constexpr int K_BYTES = KT * D;
  static constexpr int V_BYTES = PV8 ? D * KT : KT * 2 * D;
};

// K: chunk c of row r at chunk position c ^ (r & (D/16 - 1)) of its row: the 32 rows one MFMA
// operand read touches spread over all bank groups.
template <int D>
__device__ __forceinline__ int k_off(int row, int c) { return row * D + 16 * (c ^ (row & (D / 16 - 1))); }
// bf16 V: chunk c of row r at c ^ f(r); f spreads the 4 consecutive rows that one transposed
// read group touches over distinct 64-byte bank groups.
template <int D>
__device__ __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
template <int D>
__device__ __forceinline__ int v_off(int row, int byte) {   // byte offset within the row (< 2D)
  return row * 2 * D + 16 * ((byte >> 4) ^ v_swz<D>(row)) + (byte & 15);
}
// FP8 V^T: chunk c (of 4) of channel row r at c ^ ((r >> 2) & 3).
__device__ __forceinline__ int v8_off(int row, int c) { return row * KT + 16 * (c ^ ((row >> 2) & 3)); }

// vmcnt(n), n < 16: wait until at most n vector memory operations of this wave are in flight
template <int n>
__device__ __forceinline__ void wait_vmem_n() { __builtin_amdgcn_s_waitcnt(0x0F70 | n); }

// Direct global -> LDS tile copies by the 4 waves of group A.  Lane l of wave a in round i
// fills LDS chunk (4i + a) * 64 + l; its source chunk (swizzle undone) is a per-lane
// constant computed once.  A ragged last K/V tile re-reads row N-1 for rows past N (finite
// data, masked keys).  FP8 V^T rows are padded to a multiple of 64 tokens by the quantizer.
template <int D, bool PV8>
struct DmaPlan {
  static constexpr int K_ROUNDS = KT * D / 16 / 256;
  static constexpr int V_ROUNDS = (PV8 ? D * KT : KT * 2 * D) / 16 / 256;
  int koff[K_ROUNDS], krow[K_ROUNDS];
  int voff[V_ROUNDS], vrow[V_ROUNDS];
  int vsn;   // row stride of the 16-bit V (elements)
  __device__ __forceinline__ void init(int a, int lane, int64_t Np, int64_t v_row_stride) {
    vsn = (int)v_row_stride;
#pragma unroll
    for (int i = 0; i < K_ROUNDS; ++i) {
      const int pos = (i * 4 + a) * 64 + lane, row = pos / (D / 16), c = (pos % (D / 16)) ^ (row & (D / 16 - 1));
      krow[i] = row; koff[i] = row * D + 16 * c;
    }
#pragma unroll
    for (int i = 0; i < V_ROUNDS; ++i) {
      const int pos = (i * 4 + a) * 64 + lane;
      if (PV8) {   // channel row of V^T, 4 chunks of 16 tokens
        const int row = pos / 4, c = (pos % 4) ^ ((row >> 2) & 3);
        vrow[i] = row; voff[i] = (int)(row * Np) + 16 * c;
      } else {
        const int row = pos / (2 * D / 16), c = (pos % (2 * D / 16)) ^ v_swz<D>(row);
        vrow[i] = row; voff[i] = row * 2 * vsn + 16 * c;   // < 2^31: checked at the boundary
      }
    }
  }
  __device__ __forceinline__ void k_tile(const Params& p, int64_t bkv, int t, uint8_t* kb, int a) const {
    const int64_t key0 = (int64_t)t * KT;
    const char* base = (const char*)(p.k + (bkv * p.N + key0) * D);
    const bool full = key0 + KT <= p.N;
#pragma unroll
    for (int i = 0; i < K_ROUNDS; ++i) {
      int off = koff[i];
      if (!full && key0 + krow[i] >= p.N) off += (int)((p.N - 1 - key0 - krow[i]) * D);
      __builtin_amdgcn_global_load_lds((const void*)(base + off), (lds_void*)(kb + (i * 4 + a) * 1024), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void v_tile(const Params& p, int64_t bkv, int t, uint8_t* vb, int a) const {
    const int64_t key0 = (int64_t)t * KT;
    if (PV8) {
      const char* base = (const char*)p.v + bkv * D * p.Np + key0;
#pragma unroll
      for (int i = 0; i < V_ROUNDS; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(base + voff[i]), (lds_void*)(vb + (i * 4 + a) * 1024), 16, 0, 0);
    } else {
      const char* base = (const char*)((const uint16_t*)p.v + p.vr.at(bkv, key0));
      const bool full = key0 + KT <= p.N;
#pragma unroll
      for (int i = 0; i < V_ROUNDS; ++i) {
        int off = voff[i];
        if (!full && key0 + vrow[i] >= p.N) off += (int)((p.N - 1 - key0 - vrow[i]) * 2 * vsn);
        __builtin_amdgcn_global_load_lds((const void*)(base + off), (lds_void*)(vb + (i * 4 + a) * 1024), 16, 0, 0);
      }
    }
  }
};

template <int D, bool CAUSAL, bool PV8, bool THRIFT, bool VF16, bool OUT_BF16>
__global__ __launch_bounds__(NTHREADS, 1) void attn_i8_kernel(Params p, const float* __restrict__ k_scales,
                                                              const float* __restrict__ q_scales,
                                                              const uint8_t* __restrict__ blk_mask) {
  using S = Smem<D, PV8>;
  constexpr int NCC = D / 32;    // 32-channel output chunks
  __shared__ __attribute__((aligned(16))) uint8_t kb0[S::K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[S::K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kb2[S::K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vb0[S::V_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vb1[S::V_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vb2[S::V_BYTES];

  const attn::WgMap wm = attn::map_workgroup(p.total_wg, p.nPairs, CAUSAL);
  const int64_t bh = wm.bh, pr = wm.pair;
  const int64_t b = bh / p.Hq, h = bh % p.Hq;
  const int64_t bkv = b * p.Hkv + h / (p.Hq / p.Hkv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int grp = w >> 2, a = w & 3;                         // group (0 = A, 1 = B), wave in group
  const int li = lane & 31, lh = lane >> 5;
  const int64_t qb = 2 * pr + grp;                           // this group's Q block
  const int64_t qrow0 = qb * QB + 32 * a;                    // first row of this wave
  const int64_t qrow = qrow0 + li;                           // this lane's query row
  const bool row_ok = qrow < p.N;
  const bool blk_ok = qb < p.nQB;

  // tiles of this group, and of the workgroup (the longer of the two groups)
  auto tiles_of = [&](int64_t q) __attribute__((always_inline)) -> int {
    if (q >= p.nQB) return 0;
    if (!CAUSAL) return (int)p.nKB;
    const int64_t last = (q * QB + QB - 1) / KT + 1;
    return (int)(last < p.nKB ? last : p.nKB);
  };
  const int nTg = tiles_of(qb);
  const int nT = tiles_of(2 * pr + 1) > tiles_of(2 * pr) ? tiles_of(2 * pr + 1) : tiles_of(2 * pr);
  const uint8_t* mrow = THRIFT && blk_ok ? blk_mask + (bh * p.nQB + qb) * p.nKB : nullptr;
  auto active = [&](int t) __attribute__((always_inline)) { return t >= 0 && t < nTg && (!CAUSAL || (int64_t)t * KT <= qrow0 + 31); };
  // buffer J % 3 of K and of V (J a compile-time constant)
  auto kbuf = [](auto jc) __attribute__((always_inline)) -> uint8_t* {
    constexpr int J = decltype(jc)::value % 3;
    if constexpr (J == 0) return kb0; else if constexpr (J == 1) return kb1; else return kb2;
  };
  auto vbuf = [](auto jc) __attribute__((always_inline)) -> uint8_t* {
    constexpr int J = decltype(jc)::value % 3;
    if constexpr (J == 0) return vb0; else if constexpr (J == 1) return vb1; else return vb2;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  // ---- per-lane LDS read offsets (loop invariant; tile and chunk terms become immediates)
  int kro[D / 32], vro[D / 32];
  {
    const int rk = tile_key(0, li);   // tile_key(b, li) = rk + 16 b; k_off's swizzle ignores the 16 b
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) kro[kc] = k_off<D>(rk, 2 * kc + lh);
    if (!PV8) {   // transposed V reads of k-group kg, half r2 touch row rv + 8 kg + 4 r2
      const int g16 = lane >> 4, j = lane & 15;
      const int rv = 32 * (g16 >> 1) + (j >> 2);
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) vro[cc] = v_off<D>(rv, 2 * (32 * cc + 16 * (g16 & 1) + 4 * (j & 3)));
    } else {      // V^T rows 32 cc + li, chunks 2 lh, 2 lh + 1
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) vro[cc] = 32 * cc + li;
    }
  }

  // ---- Q fragments (B operand of the S^T product): row qrow, channels 32kc + 16lh .. +16
  v4i qf[D / 32];
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc)
    qf[kc] = row_ok ? *(const v4i*)(p.q + (bh * p.N + qrow) * D + 32 * kc + 16 * lh) : v4i{0, 0, 0, 0};
  const float qscale = blk_ok ? q_scales[__builtin_amdgcn_readfirstlane((int)(bh * p.nQB + qb))] : 0.0f;

  v16f o[NCC];
#pragma unroll
  for (int c = 0; c < NCC; ++c) o[c] = v16f{};
  float m_run = -__builtin_inff(), l_run = 0.0f;
  float m_lo = 0.0f;            // FP8 P: the running max is the pair m_run + m_lo
  v16i acc[2];                  // S of the tile the next VALU phase works on (kMagic + S; Thrift: S)
  v16i magic;   // opaque to the compiler, so it stays in registers instead of being rebuilt per tile
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    int m;
    __asm__ volatile("v_mov_b32 %0, %1" : "=v"(m) : "s"(kMagicBits));
    magic[r] = m;
  }
  bool hi = false;              // that tile runs on bf16 (Thrift)
  float dq = 0.0f;              // its dequantization factor (log2 units)
  float dq_lo = 0.0f;           // FP8 P: dq + dq_lo = s_q s_k sm_scale log2(e) to ~2^-40
  uint32_t pk[PV8 ? 8 : 16];    // P of the tile the next MFMA phase works on (bf16 pairs / FP8 quads)

  DmaPlan<D, PV8> dma;
  if (grp == 0) {
    dma.init(a, lane, p.Np, p.vr.sn);
    dma.k_tile(p, bkv, 0, kbuf(I0{}), a);
    if (nT > 1) dma.k_tile(p, bkv, 1, kbuf(I1{}), a);
    if (nT > 0) dma.v_tile(p, bkv, 0, vbuf(I0{}), a);
  }
  wait_vmem();
  __syncthreads();

  // ---- S of tile t for this wave.  The int8 K fragments are read from LDS by qk_load and
  //      consumed by qk_mfma, so the reads can be issued ahead of other matrix work.
  v4i kf[D / 32][2];
  auto uni = [](int64_t x) __attribute__((always_inline)) { return (int64_t)__builtin_amdgcn_readfirstlane((int)x); };   // scalar loads below
  auto qk_load = [&](int t, const uint8_t* kb) __attribute__((always_inline)) {
    if (THRIFT && mrow[uni(t)] != 0) return;
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) kf[kc][bb] = *(const v4i*)(kb + kro[kc] + 16 * D * bb);
  };
  auto qk_mfma = [&](int t) __attribute__((always_inline)) {
    hi = THRIFT && mrow[uni(t)] != 0;
    if (PV8) {   // exact two-float product of the block scales and sm_scale * log2(e)
      const float ksc = k_scales[uni(bkv * p.nKB + t)];
      const float kh = qscale * ksc, kl = __builtin_fmaf(qscale, ksc, -kh);
      dq = kh * p.sm_log2;
      dq_lo = __builtin_fmaf(kh, p.sm_log2, -dq) + __builtin_fmaf(kh, p.sm_log2_lo, kl * p.sm_log2);
    } else if (!THRIFT) {
      dq = __builtin_fmaxf(qscale * k_scales[uni(bkv * p.nKB + t)] * p.sm_log2, 1.17549435e-38f);
    }
    const int64_t key0 = (int64_t)t * KT;
    if (!hi) {
      // The integer sums start at the bit pattern of 1.5 * 2^23 (held in registers), so each
      // result read as a float is 1.5 * 2^23 + S exactly (|S| <= 128 * 128 * D < 2^22): one
      // full-rate subtraction recovers S (FP8 P: S - S_max), where a conversion runs at half
      // rate.  Thrift keeps a zero start: its bf16 tiles return floats in the same registers.
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) acc[bb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[0][bb], qf[0], (PV8 || !THRIFT) ? magic : v16i{}, 0, 0, 0);
#pragma unroll
      for (int kc = 1; kc < D / 32; ++kc)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) acc[bb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kc][bb], qf[kc], acc[bb], 0, 0, 0);
    } else {   // Thrift tile: bf16 Q and K_s fragments straight from global memory (L2)
      v16f f[2] = {v16f{}, v16f{}};
      const int64_t k0 = key0 + tile_key(0, li), k1 = key0 + tile_key(1, li);
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const v8bf qh = row_ok ? *(const v8bf*)(p.qhi + p.qhr.at(bh, qrow) + 16 * kc + 8 * lh) : v8bf{};
        const v8bf kh0 = k0 < p.N ? *(const v8bf*)(p.khi + p.khr.at(bkv, k0) + 16 * kc + 8 * lh) : v8bf{};
        const v8bf kh1 = k1 < p.N ? *(const v8bf*)(p.khi + p.khr.at(bkv, k1) + 16 * kc + 8 * lh) : v8bf{};
        f[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh0, qh, f[0], 0, 0, 0);
        f[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh1, qh, f[1], 0, 0, 0);
      }
      acc[0] = __builtin_bit_cast(v16i, f[0]);
      acc[1] = __builtin_bit_cast(v16i, f[1]);
    }
  };

  // ---- VALU phase: softmax of tile t -> P in pk
  auto valu_phase = [&](int t) __attribute__((always_inline)) {
    if (!active(t)) return;
    // Thrift: the dequantization factor is formed here rather than next to the matrix
    // instructions, where a scalar load in flight would force every LDS wait to zero.
    if (THRIFT) dq = __builtin_fmaxf(hi ? p.sm_log2 : qscale * k_scales[uni(bkv * p.nKB + t)] * p.sm_log2, 1.17549435e-38f);
    const int64_t key0 = (int64_t)t * KT;
    const bool edge = (key0 + KT > p.N) || (CAUSAL && key0 + KT - 1 > qrow0);   // causal diagonal or ragged
    auto masked = [&](int bb, int r) __attribute__((always_inline)) {
      const int64_t kg = key0 + 32 * lh + 16 * bb + r;
      return kg >= p.N || (CAUSAL && kg > qrow);
    };
    if (PV8) {
      // FP8 P codes round P * 448, so P is computed to about one fp32 ulp of its exact value:
      // the exponent is (acc - acc_max) * dq + c with the integer tile max taken out first and
      // c = tile max - running max + log2(1.75), both maxima carried as exact two-float sums;
      // the remaining factor 2^8 of 448 is applied exactly by the conversion's scale.
      constexpr int SENT = 0;   // below every kMagic + S
      if (edge) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (masked(bb, r)) acc[bb][r] = SENT;
      }
      int im = acc[0][0];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) im = acc[bb][r] > im ? acc[bb][r] : im;
      {
        auto sw = __builtin_amdgcn_permlane32_swap((uint32_t)im, (uint32_t)im, false, false);
        const int i0 = (int)sw[0], i1 = (int)sw[1];
        im = i0 > i1 ? i0 : i1;
      }
      const float fi = __int_as_float(im) - kMagic;   // exact
      float th = -__builtin_inff(), tl = 0.0f;   // tile row max (log2 units) = th + tl
      if (im > SENT) {
        th = fi * dq;
        tl = __builtin_fmaf(fi, dq, -th) + fi * dq_lo;
      }
      const float gt = (th - m_run) + (tl - m_lo);
      if (__builtin_amdgcn_ballot_w64(gt > 0.0f) != 0) {   // wave-uniform: move the running max
        const bool up = gt > 0.0f;
        const float alpha = up ? __builtin_amdgcn_exp2f((m_run - th) + (m_lo - tl)) : 1.0f;   // 0 on the first tile
        if (up) { m_run = th; m_lo = tl; }
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < NCC; ++c) o[c] *= alpha;
      }
      const float c0 = ((th - m_run) + (tl - m_lo)) + 0.807354922057604f;   // + log2(1.75)
      float lsum = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {   // 1.75 P, kept in the accumulator registers
          // both terms lie in [2^23, 2^24): their difference S - S_max is exact
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(acc[bb][r]) - __int_as_float(im), dq, c0));
          lsum += e;
          acc[bb][r] = __float_as_int(e);
        }
      if (edge) {   // a zero scale leaves masked keys at exp2(c0): clear them
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (masked(bb, r)) { lsum -= __int_as_float(acc[bb][r]); acc[bb][r] = 0; }
      }
      l_run += lsum;
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) {   // E4M3(1.75 P * 2^8): the scale operand divides by 2^-8
        const int bb = q4 >> 2, r = 4 * (q4 & 3);
        const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, __int_as_float(acc[bb][r]),
                                                                __int_as_float(acc[bb][r + 1]), 0x1p-8f, false);
        const v2s w2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, __int_as_float(acc[bb][r + 2]),
                                                                __int_as_float(acc[bb][r + 3]), 0x1p-8f, true);
        pk[q4] = __builtin_bit_cast(uint32_t, w2);
      }
      return;
    }
    float s[2][16];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[bb][r] = THRIFT ? (hi ? __int_as_float(acc[bb][r]) : (float)acc[bb][r]) : __int_as_float(acc[bb][r]) - kMagic;
    if (edge) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (masked(bb, r)) s[bb][r] = -__builtin_inff();
    }
    float mx = s[0][0];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[bb][r]);
    mx = halves_max(mx);
    const float mt = mx * dq;                      // tile row max in scaled units
    if (__builtin_amdgcn_ballot_w64(mt > m_run) != 0) {   // wave-uniform: move the running max
      const float m_new = __builtin_fmaxf(m_run, mt);
      const float alpha = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < NCC; ++c) o[c] *= alpha;
    }
    float lsum = 0.0f;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[bb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r], dq, -m_run));
        lsum += s[bb][r];
      }
    l_run += lsum;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) pk[8 * bb + (r >> 1)] = pack_bf16x2(s[bb][r], s[bb][r + 1]);
  };

  // ---- MFMA phase: S of tile t+1 and O += P(t) V(t) (group A also issues the tile loads).
  //      Thrift: every LDS fragment read is issued well ahead of the matrix instruction that
  //      consumes it: the K fragments of tile t+1 and the first V k-group, then S(t+1) (whose
  //      bf16 tiles read Q and K_s from L2 and so start early), then per k-group the read of
  //      k-group kg + 1 and the P.V products of kg.  Scheduling barriers keep that order:
  //      left alone, the compiler sinks each read next to its use to save registers and then
  //      waits for every read in turn.  Plain bf16 P and FP8 P run P.V first with the V reads
  //      one k-group ahead, then S(t+1): measured faster for them (1.5 % and 3 %).
  auto v_read = [&](const uint8_t* vs, int kg, int cc) __attribute__((always_inline)) -> v8us {
    const uint8_t* a0 = vs + vro[cc] + 8 * kg * 2 * D;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(a0));
    const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(a0 + 4 * 2 * D));
    return __builtin_bit_cast(v8us, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto v_bf16 = [&](v8us raw) __attribute__((always_inline)) -> v8bf {
    if (VF16) {   // fp16 V is multiplied as bf16 (nearest-even)
      v4i pkd;
#pragma unroll
      for (int e = 0; e < 4; ++e) pkd[e] = (int)pack_bf16x2(f16_to_f32(raw[2 * e]), f16_to_f32(raw[2 * e + 1]));
      raw = __builtin_bit_cast(v8us, pkd);
    }
    return __builtin_bit_cast(v8bf, raw);
  };
  auto mfma_phase = [&](int t, const uint8_t* vs, const uint8_t* kbn) __attribute__((always_inline)) {
    const bool an = active(t + 1), at = active(t);
    if (an) qk_load(t + 1, kbn);
    if (THRIFT) {
      v8us vf[2][NCC];
      if (at) {
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) vf[0][cc] = v_read(vs, 0, cc);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (an) qk_mfma(t + 1);
      if (at) {
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
          if (kg + 1 < 4) {
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) vf[(kg + 1) & 1][cc] = v_read(vs, kg + 1, cc);
          }
          __builtin_amdgcn_sched_barrier(0);
          const v8bf pf = __builtin_bit_cast(v8bf, v4i{(int)pk[4 * kg], (int)pk[4 * kg + 1], (int)pk[4 * kg + 2],
                                                        (int)pk[4 * kg + 3]});
#pragma unroll
          for (int cc = 0; cc < NCC; ++cc)
            o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_bf16(vf[kg & 1][cc]), pf, o[cc], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (!PV8) {
      if (at) {
        v8us vf[2][NCC];
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) vf[0][cc] = v_read(vs, 0, cc);
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
          if (kg + 1 < 4) {
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) vf[(kg + 1) & 1][cc] = v_read(vs, kg + 1, cc);
          }
          __builtin_amdgcn_sched_barrier(0);
          const v8bf pf = __builtin_bit_cast(v8bf, v4i{(int)pk[4 * kg], (int)pk[4 * kg + 1], (int)pk[4 * kg + 2],
                                                        (int)pk[4 * kg + 3]});
#pragma unroll
          for (int cc = 0; cc < NCC; ++cc)
            o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_bf16(vf[kg & 1][cc]), pf, o[cc], 0, 0, 0);
        }
      }
      if (an) qk_mfma(t + 1);
    } else {
      if (at) {
        const v8i pf = v8i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
        v8i vf[NCC];
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
          // operand bytes 16e .. 16e+15 = V^T row 32 cc + li, tokens 32 lh + 16 e ..
          const int r = vro[cc];
          const v4i v0 = *(const v4i*)(vs + v8_off(r, 2 * lh));
          const v4i v1 = *(const v4i*)(vs + v8_off(r, 2 * lh + 1));
          vf[cc] = v8i{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        }
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc)
          o[cc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[cc], pf, o[cc], 0, 0, 0, 127, 0, 127);
      }
      if (an) qk_mfma(t + 1);
    }
  };

  // ---- the schedule.  Both groups run the same program (MFMA phase of tile t, barrier, VALU
  //      phase of tile t+1, barrier); group B starts it one barrier late and group A ends with
  //      one extra barrier, so B runs exactly one phase behind A and both pass the same number
  //      of barriers.  Group A waits for its tile loads at the end of its VALU phases.
  constexpr int KR = DmaPlan<D, PV8>::K_ROUNDS, VR = DmaPlan<D, PV8>::V_ROUNDS;
  static_assert(KR + VR < 16, "vmcnt immediate");
  // one step: MFMA phase of tile t, barrier, VALU phase of tile t+1, barrier; jc = t mod 3
  auto step = [&](int t, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    // Group A issues the tile loads at the start of its VALU phase; the FP8-P variant issues them
    // one phase earlier, at the start of its MFMA phase (measured faster there, slower for bf16
    // P): K(t) and V(t-1), whose buffers they fill, were last read (by group B) in the phase
    // before either.
    const bool ld_k = grp == 0 && t + 3 < nT, ld_v = grp == 0 && t + 2 < nT;   // ld_k implies ld_v
    auto issue_loads = [&]() __attribute__((always_inline)) {
      if (ld_k) dma.k_tile(p, bkv, t + 3, kbuf(std::integral_constant<int, J>{}), a);
      if (ld_v) dma.v_tile(p, bkv, t + 2, vbuf(std::integral_constant<int, J + 2>{}), a);
    };
    if (PV8) issue_loads();
    mfma_phase(t, vbuf(std::integral_constant<int, J>{}), kbuf(std::integral_constant<int, J + 1>{}));
    phase_barrier();
    if (!PV8) issue_loads();
    valu_phase(t + 1);
    if (grp == 0) {   // the previous step's loads are complete; this step's may still fly
      if (ld_k) wait_vmem_n<KR + VR>();
      else if (ld_v) wait_vmem_n<VR>();
      else wait_vmem();
    }
    phase_barrier();
  };
  if (grp == 1) phase_barrier();
  step(-1, I2{});
  for (int t = 0; t < nT; t += 3) {
    step(t, I0{});
    if (t + 1 < nT) step(t + 1, I1{});
    if (t + 2 < nT) step(t + 2, I2{});
  }
  if (grp == 0) phase_barrier();

  // ---- epilogue: O / l (and the FP8 V channel scales); lane (li, lh) holds row qrow,
  //      channels 32cc + 8(r/4) + 4lh + (r%4).
  // (FP8 P: l sums 1.75 P and O sums E4M3(448 P) V, so O / l carries an extra 256)
  const float l_tot = halves_sum(l_run) * (PV8 ? 256.0f : 1.0f);
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
        const int64_t off = p.outr.at(bh, qrow) + ch;
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
  auto kern = attn_i8_kernel<D, CAUSAL, PV8, THRIFT, VF16, OUT_BF16>;
  if (p.total_wg == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.total_wg), dim3(NTHREADS), 0, st, p, p.ks, p.qs, p.mask);
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
  p.vr = a.vr; p.qhr = a.qhr; p.khr = a.khr; p.outr = a.outr;
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N;
  p.Np = (a.N + KT - 1) / KT * KT;
  p.nQB = (a.N + QB - 1) / QB; p.nKB = (a.N + KT - 1) / KT;
  p.nPairs = (p.nQB + 1) / 2;
  p.total_wg = a.B * a.Hq * p.nPairs;
  {
    const double l2 = (double)a.sm_scale * 1.4426950408889634074;
    p.sm_log2 = (float)l2;
    p.sm_log2_lo = (float)(l2 - (double)p.sm_log2);
  }
  const bool thrift = a.mask != nullptr;
  const bool causal = a.causal != 0;
  // the software-pipelined kernel: INT8 Q.K with bf16 P.V (fp16 V at D = 128 stays here), and
  // with FP8 P.V on INT8 tiles (Thrift masks with FP8 P.V stay here)
  if (pv_fp8 ? !thrift : (!(a.v_is_f16 && a.D == 128) && (!thrift || (a.N + KT - 1) / KT <= PIPE_MAX_MASK_TILES)))
    return launch_attn_int8_pipe(a, pv_fp8, st);
  if (a.q16) return hipErrorNotSupported;   // 16-bit Q is quantized by the pipelined kernel only
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
