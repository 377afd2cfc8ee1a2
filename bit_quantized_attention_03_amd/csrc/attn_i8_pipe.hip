// Fused INT8 attention forward for gfx950, software-pipelined within each wave.
//
// SageAttention ("Accurate 8-Bit Attention for Plug-and-play Inference Acceleration",
// Technical approach): QK^T on 8-bit Q and smoothed K with per-block scales, an fp32 online
// softmax, and P and V kept at 16 bits for P.V (here bf16 with fp32 accumulation).  The
// video-generation form keeps P and V in FP8 instead (P scaled by 448 and V per channel, both
// E4M3) on the scaled FP8 product; its softmax is described at soft_a8 below.
//
// Work decomposition.  A workgroup of 8 waves owns two adjacent Q blocks of 128 rows of one
// (b, q-head): wave w takes rows 32w .. 32w+31 of the pair.  All waves stream the same K/V
// tiles of 64 keys through LDS, in ascending order, one tile per loop iteration.
//
// Operand layouts (per wave and tile):
//   S^T (64 keys x 32 queries) = K . Q^T on v_mfma_i32_32x32x32_i8, each lane holding 32 scores
//       of ONE query row (the row max and sum are lane scalars plus one v_permlane32_swap).
//       K rows are read permuted so that lane half h holds keys 32h .. 32h+31 in register
//       order, which is also the B-operand order P^T needs below.
//   O^T (D x 32) += V^T . P^T on v_mfma_f32_32x32x16_bf16, V^T fragments read from the
//       row-major LDS tile by ds_read_b64_tr_b16.
//
// Schedule.  Every wave overlaps its own matrix and vector work: iteration t issues the
// products P.V of tile t-1 and S of tile t+1 while its vector ALU computes the softmax of
// tile t.  The iteration is split in two halves at workgroup barriers, and the two wave
// groups of the workgroup (waves 0-3 and 4-7, one of each per SIMD) run half an iteration
// apart, so each SIMD always has one wave in each half and the matrix core is fed by both.
// The running max is exact: P of tile t is rounded to bf16 relative to max(m, rowmax S(t)),
// and O is rescaled by exp2(m_old - m_new) after the products of tile t-1 and before those
// of tile t, whenever some row of the wave raised its max.
//
// Tiles move by buffer loads that write LDS directly, shared by the 8 waves: the phase of
// iteration t issues K(t+3) and V(t+1), each wave waits for its own share two phases later,
// and the barrier that opens the next phase publishes them.  Three buffers of each kind
// rotate inside one LDS array.
//
// Thrift (ThriftAttention, ¶1, ¶3: one softmax over INT8 tiles and a few tiles in high
// precision, chosen by a block mask).  With a mask, the S of a flagged tile is computed again
// on bf16 Q and K_s rows read from global memory, after the interleaved INT8 products (whose
// result it replaces), and stored in the same accumulators as integers S * 2^k, so that the
// softmax treats both kinds alike; the tile's dequantization factor is sm_scale * log2(e) *
// 2^-k.  The workgroup's two mask rows are copied to LDS at the start.
#include "attn_common.hpp"
#include "device.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace sage {
namespace {

using namespace attn;

struct PipeParams {
  const int8_t* q; const float* qs;
  const int8_t* k; const float* ks;
  const uint16_t* v;
  void* out;
  int64_t Hq, Hkv, N, nQB, nKB, nPairs, total_wg;
  float sm_log2;   // sm_scale * log2(e), rounded to fp32
  float sm_log2_lo;   // sm_scale * log2(e) - sm_log2 (FP8 P carries the product to ~2^-40)
  // FP8 P.V: V^T codes [B, Hkv, D, Np] (E4M3, channel-major, tokens padded to Np) and the
  // per-channel V scales [B, Hkv, D] (then v is unused)
  const uint8_t* v8; const float* vs; int64_t Np;
  Rows16 vr, outr; // rows of V (per KV head) and of the output
  // Thrift: block mask [B, Hq, nQB, nKB] (1: the tile runs on bf16 Q and K_s) and those rows
  const uint8_t* mask;
  const uint16_t* qhi; const uint16_t* khi;
  // 16-bit Q [B, Hq, N, D] (rows q16r) quantized here per 128-token block, or null (q / qs hold
  // the codes and scales)
  const uint16_t* q16; Rows16 q16r; int q16_f16;
  Rows16 qhr, khr;
};


// K tile (int8 [64][D]): 16-byte chunk c of row r at chunk position c ^ k_swz(r).  An operand
// read (ds_read_b128) serves 16 lanes per pass, which must fall in 16 distinct 16-byte bank
// groups ((address >> 4) mod 16).  The 16 lanes of a pass read rows 32b + 4a + c' + 16bb
// (a, b in {0, 1}, c' in 0..3) at one chunk index: the row's low bit (D = 128) or low two bits
// (D = 64) pick part of the bank group, and the swizzle must spread the remaining rows, which
// differ in bits 2 and 5 (and bit 1 for D = 128), over distinct chunk positions.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? ((row & 6) | ((row >> 5) & 1)) : (((row >> 2) & 1) | (((row >> 5) & 1) << 1));
}
template <int D>
__device__ __forceinline__ int k_off(int row, int c) { return row * D + 16 * (c ^ k_swz<D>(row)); }
// bf16 V tile ([64][D] row-major): chunk c of row r at c ^ v_swz(r), which spreads the 4
// consecutive rows one transposed read group touches over distinct 64-byte bank groups.
template <int D>
__device__ __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
template <int D>
__device__ __forceinline__ int v_off(int row, int byte) {   // byte offset within the row (< 2D)
  return row * 2 * D + 16 * ((byte >> 4) ^ v_swz<D>(row)) + (byte & 15);
}
// FP8 V^T tile ([D][64] bytes): chunk c (of 4) of channel row r at c ^ v8_swz(r), so the 16
// rows one operand read pass touches (4 consecutive rows x 4 row groups) cover all chunk slots.
__device__ __forceinline__ int v8_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int v8_off(int row, int c) { return row * KT + 16 * (c ^ v8_swz(row)); }
// E4M3 P codes are formed from S - S_max read off integer sums that start at the bit pattern of
// 1.5 * 2^23: as floats they are 1.5 * 2^23 + S exactly (|S| < 2^22), and the difference of two
// is exact.
constexpr float kMagic = 12582912.0f;
constexpr int kMagicBits = 0x4B400000;
// Scheduling hints for the machine scheduler (instruction classes of sched_group_barrier):
// a region's instructions are placed in the order of the groups requested.
constexpr int SG_MFMA = 0x008, SG_VALU = 0x002, SG_DS_READ = 0x100;
#define SCHED_GROUP(mask, n, id) __builtin_amdgcn_sched_group_barrier((mask), (n), (id))
// A value pinned here is computed before this point (it cannot be sunk past it).
template <typename T>
__device__ __forceinline__ void pin(T& x) { __asm__ volatile("" : "+v"(x)); }

// vmcnt(n): wait until at most n vector memory operations of this wave are in flight.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F73); break;
  }
}

// Direct global -> LDS tile copies.  A buffer load with the lds modifier moves 64 chunks of 16
// bytes (one per lane, at the lane's byte offset from the buffer's base) into 1 KB of LDS at the
// M0 address (lane l writes bytes 16 l .. 16 l + 15 of the kilobyte).  The buffer descriptor
// (four scalars: base, record count in bytes, format word) starts at the tile's first row and
// covers the rows that remain below N: a lane whose offset falls past them reads zeros, so a
// ragged last tile needs no clamping (its masked keys see finite zeros).  The per-lane offsets
// are constants and the tile position lives in the scalar descriptor: no vector work per copy.
// Written as an asm statement so the compiler does not track it as an LDS write: it would
// otherwise wait for every such copy in flight before any LDS read of the same array, and the
// three tile buffers share one.  Ordering is explicit instead (waits for each wave's own copies
// two phases later, then a barrier before the first reads; a buffer is refilled only after its
// last reads).  The statement has no output register.
__device__ __forceinline__ void lds_dma16(int voff, v4i rsrc, uint32_t lds_off) {
  __asm__ volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_off) : "memory");
}
// Descriptor of a raw byte buffer (stride 0) of n bytes at base (both wave-uniform, in scalar
// registers); the last word is the gfx9 family's data format for untyped buffer access.
__device__ __forceinline__ v4i buffer_desc(uint64_t base, int n) {
  v4i r;
  r[0] = (int)(uint32_t)base;
  r[1] = (int)(uint32_t)(base >> 32);   // base < 2^48 (masked once), so the stride field is 0
  r[2] = n;
  r[3] = 0x00020000;
  return r;
}

// Tile copies shared by the 8 waves.  Instruction i of a tile (one kilobyte) is issued by wave
// i % 8.  Lane l of instruction i fills LDS chunk position 64 i + l, whose source chunk (the
// swizzle undone) sits at a per-lane constant offset from the tile's first row.  K and V tiles
// are copied in ascending order, each stream from a scalar address advanced by one tile per
// copy and a count of the keys left below N (and below the workgroup's last tile) from that
// tile on.  A copy takes the rows of its tile that lie below that bound: none past the
// workgroup's last tile (its buffer load then reads only zeros and touches no memory; such a
// buffer is never read).
template <int D, bool PV8>
struct PipeDma {
  static constexpr int K_INSTR = KT * D / 16 / 64;                  // D/16: 8 (D = 128) or 4
  static constexpr int V_INSTR = (PV8 ? D : 2 * D) * KT / 16 / 64;  // bf16: D/8; FP8 V^T: D/16
  static constexpr int K_PER = (K_INSTR + 7) / 8, V_PER = (V_INSTR + 7) / 8;
  // copy instructions of wave w per phase (the vmcnt of one phase's copies)
  __device__ __forceinline__ static int loads_of(int w) {
    return (K_INSTR % 8 == 0 ? K_PER : (w < K_INSTR ? 1 : 0)) + (V_INSTR % 8 == 0 ? V_PER : (w < V_INSTR ? 1 : 0));
  }
  uint64_t kaddr, vaddr;     // first byte of the next K tile and of the next V tile to copy
  int krem, vrem;            // keys from those tiles' first rows to N (<= 0: past the end)
  int vrow2;                 // bytes between V rows
  int koff[K_PER], voff[V_PER];
  // wave-uniform copy state, kept in scalar registers (the scalar unit does its arithmetic)
  template <typename T>
  __device__ __forceinline__ static void sgpr(T& x) { __asm__ volatile("" : "+s"(x)); }
  // min(max(rem, 0), KT) on the scalar unit (the pin keeps the pair from being fused into a
  // vector med3)
  __device__ __forceinline__ static int rows_of(int rem) {
    int r = rem < KT ? rem : KT;
    sgpr(r);
    return r > 0 ? r : 0;
  }
  // nT: the workgroup's tile count; rows from tile nT on are not copied
  __device__ __forceinline__ void init(const PipeParams& p, int64_t bkv, int nT, int w, int lane) {
    // 48-bit addresses; a copy's advance stays inside its buffer, so bit 48 is never reached
    kaddr = (uint64_t)(p.k + bkv * p.N * D) & 0xffffffffffffull;
    vaddr = (PV8 ? (uint64_t)(p.v8 + bkv * D * p.Np) : (uint64_t)(p.v + p.vr.head(bkv))) & 0xffffffffffffull;
    krem = vrem = (int)(p.N < (int64_t)nT * KT ? p.N : (int64_t)nT * KT);
    vrow2 = PV8 ? (int)p.Np : 2 * (int)p.vr.sn;
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
      const int i = w + 8 * j;
      const int pos = 64 * (i < K_INSTR ? i : 0) + lane, row = pos / (D / 16);
      const int c = (pos % (D / 16)) ^ k_swz<D>(row);
      koff[j] = row * D + 16 * c;
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      if (PV8) {   // V^T: channel row of 4 chunks of 16 tokens (N <= 2^24, so row * Np < 2^31)
        const int i = w + 8 * j;
        const int pos = 64 * (i < V_INSTR ? i : 0) + lane, row = pos / 4;
        voff[j] = row * vrow2 + 16 * ((pos % 4) ^ v8_swz(row));
      } else {
        const int pos = 64 * (w + 8 * j) + lane, row = pos / (2 * D / 16);
        const int c = (pos % (2 * D / 16)) ^ v_swz<D>(row);
        voff[j] = row * vrow2 + 16 * c;   // < 2^31: the row stride is checked at the boundary
      }
    }
  }
  // the next K tile into the LDS buffer at kb
  __device__ __forceinline__ void k_next(uint32_t kb, int w) {
    const v4i rsrc = buffer_desc(kaddr, rows_of(krem) * D);
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
      if (K_INSTR % 8 != 0 && w + 8 * j >= K_INSTR) break;   // every wave copies when D = 128
      lds_dma16(koff[j], rsrc, kb + (w + 8 * j) * 1024);
    }
    kaddr += KT * D;
    krem -= KT;
  }
  // the next V tile into the LDS buffer at vb.  The record count covers whole row strides of
  // the rows below N: a lane reads 16 bytes of the first 2D of its row, so the lanes of rows
  // below N read only their rows, and those of later rows read zeros.
  __device__ __forceinline__ void v_next(uint32_t vb, int w) {
    if constexpr (PV8) {
      // the tile's 64 token columns of every channel row (the rows are padded to Np tokens)
      const v4i rsrc = buffer_desc(vaddr, rows_of(vrem) > 0 ? (D - 1) * vrow2 + KT : 0);
#pragma unroll
      for (int j = 0; j < V_PER; ++j) {
        if (V_INSTR % 8 != 0 && w + 8 * j >= V_INSTR) break;
        lds_dma16(voff[j], rsrc, vb + (w + 8 * j) * 1024);
      }
      vaddr += KT;
    } else {
      // at most 64 rows of 2^25 bytes (the row stride is capped at the boundary): 32 bits unsigned
      const v4i rsrc = buffer_desc(vaddr, (int)((uint32_t)rows_of(vrem) * (uint32_t)vrow2));
#pragma unroll
      for (int j = 0; j < V_PER; ++j) lds_dma16(voff[j], rsrc, vb + (w + 8 * j) * 1024);
      vaddr += (uint64_t)KT * (uint32_t)vrow2;
    }
    vrem -= KT;
  }
};

template <int D, bool CAUSAL, bool VF16, bool OUT_BF16, bool THRIFT, bool PV8>
__global__ __launch_bounds__(NTHREADS, 1) void attn_i8_pipe_kernel(PipeParams p, const float* __restrict__ k_scales) {
  constexpr int NCC = D / 32;   // 32-channel chunks of O and 32-channel k-slices of S
  constexpr int K_BYTES = KT * D, V_BYTES = PV8 ? D * KT : KT * 2 * D;
  static_assert(!PV8 || (!THRIFT && !VF16), "FP8 P.V: INT8 tiles and FP8 V only");
  // three K tiles then three V tiles
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * K_BYTES + 3 * V_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);

  const WgMap wm = map_workgroup(p.total_wg, p.nPairs, CAUSAL);
  const int64_t bh = wm.bh, pr = wm.pair;
  const int64_t b = bh / p.Hq, h = bh % p.Hq;
  const int64_t bkv = b * p.Hkv + h / (p.Hq / p.Hkv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int li = lane & 31, lh = lane >> 5;
  const int64_t qrow0 = 2 * pr * QB + 32 * w;                 // first row of this wave
  const int64_t qrow = qrow0 + li;                            // this lane's query row
  const bool row_ok = qrow < p.N;
  const int64_t qb = qrow0 / QB;

  // last tile of this wave (-1: no rows) and the workgroup's tile count (its last wave's)
  auto last_tile = [&](int64_t r0) __attribute__((always_inline)) -> int {
    if (r0 >= p.N) return -1;
    if (!CAUSAL) return (int)p.nKB - 1;
    const int64_t l = (r0 + 31) / KT;
    return (int)(l < p.nKB - 1 ? l : p.nKB - 1);
  };
  const int tl = last_tile(qrow0);
  int nT = 0;
#pragma unroll
  for (int ww = 0; ww < NWAVES; ++ww) {
    const int l = last_tile(2 * pr * QB + 32 * ww) + 1;
    nT = l > nT ? l : nT;
  }
  // the wave's last tile needs key masks (causal diagonal, or keys past a ragged N)
  const bool tail_edge = CAUSAL || (p.N % KT) != 0;

  // LDS byte offsets of tile buffer j (0..2)
  auto kbuf = [&](int j) __attribute__((always_inline)) -> uint32_t { return (uint32_t)(j * K_BYTES); };
  auto vbuf = [&](int j) __attribute__((always_inline)) -> uint32_t { return (uint32_t)(3 * K_BYTES + j * V_BYTES); };

  // ---- per-lane LDS read offsets (loop invariant)
  int kro[NCC], vro[NCC];
  {
    const int rk = tile_key(0, li);   // tile_key(b, li) = rk + 16 b; k_off's swizzle ignores the 16 b
#pragma unroll
    for (int kc = 0; kc < NCC; ++kc) kro[kc] = k_off<D>(rk, 2 * kc + lh);
    // transposed V reads of k-group kg, half r2 touch row rv + 8 kg + 4 r2
    const int g16 = lane >> 4, j = lane & 15;
    const int rv = 32 * (g16 >> 1) + (j >> 2);
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) vro[cc] = PV8 ? 32 * cc + li : v_off<D>(rv, 2 * (32 * cc + 16 * (g16 & 1) + 4 * (j & 3)));
  }

  // ---- Q fragments (B operand of S^T = K Q^T): row qrow, channels 32kc + 16lh .. +16.
  //      From 16-bit Q, the kernel quantizes them itself, as the INT8 quantizer does for a block
  //      of 128 tokens (SageAttention, Technical approach): s = amax / 127 over the block, the
  //      rows of one wave group.  The loads fly with the first K copies; each wave's largest
  //      magnitude then goes through LDS at the barrier below, and the codes are formed after it.
  v4i qf[NCC];
  float qscale = 0.0f;
  const bool q_fused = p.q16 != nullptr;
  v4i q16raw[NCC][2];   // this lane's 16 NCC values of 16-bit Q
  __shared__ float qamax[NWAVES];
  auto q16_val = [&](int kc, int e) __attribute__((always_inline)) -> float {
    const uint16_t h = (uint16_t)((uint32_t)q16raw[kc][e >> 3][(e >> 1) & 3] >> (16 * (e & 1)));
    return p.q16_f16 ? in16_to_f32<true>(h) : in16_to_f32<false>(h);
  };
  // A row past N loads row N-1 instead (no branch, so no wait, around the loads): its scores,
  // softmax and products stay in its own lane column and it is never stored.
  const int64_t qrow_ld = row_ok ? qrow : p.N - 1;
  if (q_fused) {   // loads in flight with the first K copies (the wait below covers both)
    const uint16_t* src = p.q16 + p.q16r.at(bh, qrow_ld) + 16 * lh;
#pragma unroll
    for (int kc = 0; kc < NCC; ++kc) {
      q16raw[kc][0] = *(const v4i*)(src + 32 * kc);
      q16raw[kc][1] = *(const v4i*)(src + 32 * kc + 8);
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < NCC; ++kc) qf[kc] = *(const v4i*)(p.q + (bh * p.N + qrow_ld) * D + 32 * kc + 16 * lh);
    qscale = tl >= 0 ? p.qs[__builtin_amdgcn_readfirstlane((int)(bh * p.nQB + qb))] : 0.0f;
  }
  const float* kscales = k_scales + bkv * p.nKB;   // read-only: scalar loads

  v16f o[NCC];
#pragma unroll
  for (int c = 0; c < NCC; ++c) o[c] = v16f{};
  float m_run = -__builtin_inff(), l_run = 0.0f;
  v16i sacc[2];      // S of the tile the next softmax works on
  uint32_t pk[16];   // bf16 P of the tile the next P.V products work on (pairs of keys)
  // dequantization factor (s_q s_k sm_scale log2 e) of the tile being softmaxed, from the K
  // block scale loaded at the end of the previous iteration
  float dq = 0.0f;
  float dq_lo = 0.0f;   // FP8 P: dq + dq_lo = s_q s_k sm_scale log2(e) to ~2^-40
  float m_lo = 0.0f;    // FP8 P: the running max is the pair m_run + m_lo
  // FP8 P: the integer S sums start at kMagicBits (held in registers, opaque to the compiler)
  v16i magic;
  if constexpr (PV8) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int m;
      __asm__ volatile("v_mov_b32 %0, %1" : "=v"(m) : "s"(kMagicBits));
      magic[r] = m;
    }
  }
  float ksc_next = nT > 0 ? kscales[0] : 0.0f;
  // Thrift: whether the tile whose S is being computed runs on bf16, its scores then in units
  // of 2^-k (wave-uniform); the dequantization factor of the next softmax is qs_use * ksc_next *
  // sm_scale * log2(e), qs_use * ksc_next being s_q s_k for an INT8 tile and 2^-k for a bf16 one
  bool hi_nxt = false;
  int k_nxt = 0;
  float qs_use = qscale;

  // Thrift: the mask rows of the workgroup's two Q blocks (wave group g reads row g), zero past
  // the mask's last Q block; published by the barrier below
  __shared__ uint8_t mlds[THRIFT ? 2 * PIPE_MAX_MASK_TILES : 1];
  if constexpr (THRIFT) {
    for (int i = tid; i < 2 * (int)p.nKB; i += NTHREADS) {
      const int64_t qbi = 2 * pr + i / (int)p.nKB;
      mlds[i] = qbi < p.nQB ? p.mask[(bh * p.nQB + qbi) * p.nKB + i % (int)p.nKB] : (uint8_t)0;
    }
  }
  // tile tt of this wave runs on bf16 Q and K_s (wave-uniform)
  auto hi_tile = [&](int tt) __attribute__((always_inline)) -> bool {
    if constexpr (!THRIFT) return false;
    else return tt <= tl && __builtin_amdgcn_readfirstlane((int)mlds[(w >> 2) * (int)p.nKB + tt]) != 0;
  };

  PipeDma<D, PV8> dma;
  dma.init(p, bkv, nT, w, lane);
  dma.k_next(lds0 + kbuf(0), w);   // K(0), K(1)
  dma.k_next(lds0 + kbuf(1), w);
  wait_vm(0);
  if (q_fused) {
    __builtin_amdgcn_sched_barrier(0);
    float am = 0.0f;
#pragma unroll
    for (int kc = 0; kc < NCC; ++kc)
#pragma unroll
      for (int e = 0; e < 16; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(q16_val(kc, e)));
    am = wave_max(row_ok ? am : 0.0f);   // the block's rows only
    if (lane == 0) qamax[w] = am;
  }
  __syncthreads();
  if (q_fused) {
    const int g0 = 4 * (w >> 2);
    const float amax = __builtin_fmaxf(__builtin_fmaxf(qamax[g0], qamax[g0 + 1]), __builtin_fmaxf(qamax[g0 + 2], qamax[g0 + 3]));
    const float s = amax / 127.0f;
    const float r = int8_recip(s);
#pragma unroll
    for (int kc = 0; kc < NCC; ++kc) {
      uint32_t cb[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) cb[e] = int8_code_bits(q16_val(kc, e), r);
      qf[kc] = v4i{(int)pack_bytes(cb[0], cb[1], cb[2], cb[3]), (int)pack_bytes(cb[4], cb[5], cb[6], cb[7]),
                   (int)pack_bytes(cb[8], cb[9], cb[10], cb[11]), (int)pack_bytes(cb[12], cb[13], cb[14], cb[15])};
    }
    qscale = tl >= 0 ? s : 0.0f;
    qs_use = qscale;
  }

  // ---- matrix work of one wave.  S^T(t) = K(t) Q^T from the K tile at LDS offset kbs
  //      (fragments read first, so their LDS latency runs under other work); O^T += V^T P^T for
  //      one k-group kg of 16 keys from the V tile at vbs, with P's bf16 pairs pk[4kg .. 4kg+3].
  auto k_frags = [&](uint32_t kbs, v4i (&kf)[NCC][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < NCC; ++kc)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) kf[kc][bb] = *(const v4i*)(smem + kbs + kro[kc] + 16 * D * bb);
  };
  auto s_mfma = [&](const v4i (&kf)[NCC][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) sacc[bb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[0][bb], qf[0], PV8 ? magic : v16i{}, 0, 0, 0);
#pragma unroll
    for (int kc = 1; kc < NCC; ++kc)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) sacc[bb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kc][bb], qf[kc], sacc[bb], 0, 0, 0);
  };
  // Thrift tile tt: S^T on bf16 K_s and Q fragments straight from global memory (L2), in the
  // key order of the INT8 products.  The fp32 scores are stored in the INT8 accumulators as
  // integers S * 2^k, k the wave-uniform exponent that brings the tile's largest |S| into
  // [2^22, 2^23): the softmax then converts them like INT8 sums, and dequantizes them with
  // sm_scale * log2(e) * 2^-k.  The scaling by 2^k is exact; the rounding to an integer moves a
  // score by at most 2^-24 of the tile's largest.  Returns k.
  auto s_hi = [&](int tt) __attribute__((always_inline)) -> int {
    v16f f[2] = {v16f{}, v16f{}};
    // rows past N read row N-1 instead (no branches around the loads): their keys are masked
    // and their query rows are never stored, and every input value is finite
    const int64_t last = p.N - 1;
    const int64_t k0 = (int64_t)tt * KT + tile_key(0, li), k1 = (int64_t)tt * KT + tile_key(1, li);
    const uint16_t* qp = p.qhi + p.qhr.at(bh, qrow < last ? qrow : last) + 8 * lh;
    const uint16_t* kp0 = p.khi + p.khr.at(bkv, k0 < last ? k0 : last) + 8 * lh;
    const uint16_t* kp1 = p.khi + p.khr.at(bkv, k1 < last ? k1 : last) + 8 * lh;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const v8bf qh = *(const v8bf*)(qp + 16 * kc);
      const v8bf kh0 = *(const v8bf*)(kp0 + 16 * kc);
      const v8bf kh1 = *(const v8bf*)(kp1 + 16 * kc);
      f[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh0, qh, f[0], 0, 0, 0);
      f[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh1, qh, f[1], 0, 0, 0);
    }
    float mx = 0.0f;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, __builtin_fabsf(f[bb][r]));
    mx = wave_max(mx);
    // mx = m * 2^e with 1 <= m < 2 (mx = 0: e = -127): k = 22 - e, kept within fp32's exponents
    const uint32_t mb = (uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(mx));
    const int e = (int)((mb >> 23) & 255u) - 127;
    const int k = 22 - e > 126 ? 126 : 22 - e;
    const float sc = __builtin_ldexpf(1.0f, k);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[bb][r] = (int)__builtin_rintf(f[bb][r] * sc);
    return k;
  };
  auto v_read = [&](uint32_t vbs, int kg, int cc) __attribute__((always_inline)) -> v8bf {
    const uint8_t* a0 = smem + vbs + vro[cc] + 8 * kg * 2 * D;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(a0));
    const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(a0 + 4 * 2 * D));
    v8us raw = __builtin_bit_cast(v8us, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    if (VF16) {   // fp16 V is multiplied as bf16 (nearest-even)
      v4i pkd;
#pragma unroll
      for (int e = 0; e < 4; ++e) pkd[e] = (int)pack_bf16x2(f16_to_f32(raw[2 * e]), f16_to_f32(raw[2 * e + 1]));
      raw = __builtin_bit_cast(v8us, pkd);
    }
    return __builtin_bit_cast(v8bf, raw);
  };
  auto v_frags = [&](uint32_t vbs, int kg, v8bf (&vf)[NCC]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) vf[cc] = v_read(vbs, kg, cc);
  };
  auto pv_mfma = [&](const v8bf (&vf)[NCC], int kg) __attribute__((always_inline)) {
    const v8bf pf = __builtin_bit_cast(v8bf, v4i{(int)pk[4 * kg], (int)pk[4 * kg + 1], (int)pk[4 * kg + 2],
                                                  (int)pk[4 * kg + 3]});
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cc], pf, o[cc], 0, 0, 0);
  };

  // ---- softmax of tile t, in parts that run under the matrix products.  Part A (under
  //      S(t+1)): scores to fp32, key masks, row max, new running max, rescale factor.  Part B,
  //      per k-group kg (under the P.V(t-1) products of the same k-group, whose P registers it
  //      then overwrites): P = exp2(s dq - m) for the group's 8 keys of this lane, their sum,
  //      bf16 pairs.  k-group kg is keys s[kg/2][8(kg%2) .. 8(kg%2)+7] of the lane.
  struct Soft { float s[2][16]; float dq, alpha, lsum, c0; };
  auto soft_a = [&](Soft& sm, int64_t key0, bool edge) __attribute__((always_inline)) {
    sm.dq = dq;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.s[bb][r] = (float)sacc[bb][r];
    if (edge) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t kg = key0 + 32 * lh + 16 * bb + r;
          if (kg >= p.N || (CAUSAL && kg > qrow)) sm.s[bb][r] = -__builtin_inff();
        }
    }
    // row max as a tree of 3-input maxima (v_max3_f32): 4 per 8 keys, then 2
    auto max3 = [](float a, float b, float c) __attribute__((always_inline)) {
      return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
    };
    float mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* x = &sm.s[q >> 1][8 * (q & 1)];
      mq[q] = max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), __builtin_fmaxf(x[6], x[7]));
    }
    float mx = halves_max(__builtin_fmaxf(max3(mq[0], mq[1], mq[2]), mq[3]));
    const float mt = mx * sm.dq;                      // tile row max in scaled units
    const float m_new = __builtin_fmaxf(m_run, mt);
    sm.alpha = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    sm.lsum = 0.0f;
  };
  auto soft_b = [&](Soft& sm, int kg) __attribute__((always_inline)) {
    const int bb = kg >> 1, r0 = 8 * (kg & 1);
#pragma unroll
    for (int r = r0; r < r0 + 8; ++r) sm.s[bb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm.s[bb][r], sm.dq, -m_run));
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[4 * kg + e] = pack_bf16x2(sm.s[bb][r0 + 2 * e], sm.s[bb][r0 + 2 * e + 1]);
    // The row sum takes the bf16 P that the P.V products use: one 2-way dot product with
    // (1, 1) per pair of keys (half the adds of an fp32 sum), and numerator and denominator
    // then weigh the keys alike.  Pinned here, so the pairs are not kept alive past the MFMAs.
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sm.lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_ones(), __builtin_bit_cast(bf16x2_t, pk[4 * kg + e]), sm.lsum, false);
    pin(sm.lsum);
  };
  // ---- FP8 P (video-generation form: P rounded to E4M3 after scaling by 448, V in E4M3 with
  //      per-channel scales).  E4M3 codes round 448 P, so P is formed to about one fp32 ulp: the
  //      exponent is (S - S_max) dq + c0, with the integer tile max taken out exactly (both read
  //      off the magic-started sums), c0 = tile max - running max + log2(1.75), and both maxima
  //      carried as exact two-float sums; the remaining 2^8 of 448 = 1.75 * 2^8 is applied by
  //      the conversion's scale operand.  Part A (under P.V(t-1)): masks, integer row max, new
  //      running max, rescale factor, S - S_max, then part B of the first key block.  Part B
  //      of a block of 16 keys: exp2, the row sum of 1.75 P, E4M3 codes; the second block's
  //      runs under S(t+1).
  constexpr int SENT = 0;   // below every kMagic + S: a masked key
  auto soft_a8 = [&](Soft& sm, int64_t key0, bool edge) __attribute__((always_inline)) {
    sm.dq = dq;
    if (edge) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t kg = key0 + 32 * lh + 16 * bb + r;
          if (kg >= p.N || (CAUSAL && kg > qrow)) sacc[bb][r] = SENT;
        }
    }
    // integer row max as a tree of 3-input maxima (short dependency chains)
    auto imax = [](int x, int y) __attribute__((always_inline)) { return x > y ? x : y; };
    int mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v16i& x = sacc[q >> 1];
      const int o8 = 8 * (q & 1);
      mq[q] = imax(imax(imax(x[o8], x[o8 + 1]), x[o8 + 2]), imax(imax(x[o8 + 3], x[o8 + 4]), x[o8 + 5]));
      mq[q] = imax(mq[q], imax(x[o8 + 6], x[o8 + 7]));
    }
    int im = imax(imax(imax(mq[0], mq[1]), mq[2]), mq[3]);
    {
      auto sw = __builtin_amdgcn_permlane32_swap((uint32_t)im, (uint32_t)im, false, false);
      const int i0 = (int)sw[0], i1 = (int)sw[1];
      im = i0 > i1 ? i0 : i1;
    }
    const float fi = __int_as_float(im) - kMagic;   // exact
    float th = -__builtin_inff(), tlo = 0.0f;        // tile row max (log2 units) = th + tlo
    if (im > SENT) {
      th = fi * dq;
      tlo = __builtin_fmaf(fi, dq, -th) + fi * dq_lo;
    }
    const float gt = (th - m_run) + (tlo - m_lo);
    const bool up = gt > 0.0f;
    sm.alpha = up ? __builtin_amdgcn_exp2f((m_run - th) + (m_lo - tlo)) : 1.0f;   // 0 on the first tile
    if (up) { m_run = th; m_lo = tlo; }
    sm.c0 = ((th - m_run) + (tlo - m_lo)) + 0.807354922057604f;   // + log2(1.75)
    const float fm = __int_as_float(im);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.s[bb][r] = __int_as_float(sacc[bb][r]) - fm;   // S - S_max, exact
  };
  // part B for key block bb (keys 32 lh + 16 bb .. +15 of the lane): exp2, masked keys
  // cleared, their sum, and E4M3 codes into pk[4 bb .. 4 bb + 3]
  auto soft_b8 = [&](Soft& sm, int64_t key0, bool edge, int bb) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.s[bb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm.s[bb][r], sm.dq, sm.c0));   // 1.75 P
    if (edge) {   // a zero scale leaves masked keys at exp2(c0): clear them
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t kg = key0 + 32 * lh + 16 * bb + r;
        if (kg >= p.N || (CAUSAL && kg > qrow)) sm.s[bb][r] = 0.0f;
      }
    }
    float ps[8];   // the block's sum as a pairwise tree (short dependency chains)
#pragma unroll
    for (int r = 0; r < 8; ++r) ps[r] = sm.s[bb][r] + sm.s[bb][r + 8];
#pragma unroll
    for (int w2 = 1; w2 < 8; w2 *= 2)
#pragma unroll
      for (int r = 0; r < 8; r += 2 * w2) ps[r] = ps[r] + ps[r + w2];
    sm.lsum = bb == 0 ? ps[0] : sm.lsum + ps[0];
#pragma unroll
    for (int q4 = 4 * bb; q4 < 4 * bb + 4; ++q4) {   // E4M3(1.75 P * 2^8): the scale operand divides by 2^-8
      const int r = 4 * (q4 & 3);
      const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, sm.s[bb][r], sm.s[bb][r + 1], 0x1p-8f, false);
      const v2s w2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, sm.s[bb][r + 2], sm.s[bb][r + 3], 0x1p-8f, true);
      pk[q4] = __builtin_bit_cast(uint32_t, w2);
    }
  };
  // O^T += V^T P^T for the whole tile on the scaled FP8 product (unit scales): operand bytes
  // 16e .. 16e+15 of lane (li, lh) are V^T row 32 cc + li, tokens 32 lh + 16 e ..
  auto v8_frags = [&](uint32_t vbs, v8i (&vf)[NCC]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      const v4i v0 = *(const v4i*)(smem + vbs + v8_off(vro[cc], 2 * lh));
      const v4i v1 = *(const v4i*)(smem + vbs + v8_off(vro[cc], 2 * lh + 1));
      vf[cc] = v8i{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
  };
  auto pv8_mfma = [&](const v8i (&vf)[NCC]) __attribute__((always_inline)) {
    const v8i pf = v8i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) o[cc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[cc], pf, o[cc], 0, 0, 0, 127, 0, 127);
  };

  // alpha is exactly 1 for a row whose max did not move: O is rescaled only when some row of
  // the wave has a new max (a wave-uniform branch; the products then overwrite O in place).
  // Late in a long row most tiles leave every max where it was.
  auto rescale = [&](const Soft& sm) __attribute__((always_inline)) {
    l_run = l_run * sm.alpha + sm.lsum;
    if (__builtin_amdgcn_ballot_w64(sm.alpha != 1.0f) != 0) {
#pragma unroll
      for (int c = 0; c < NCC; ++c) o[c] *= sm.alpha;
    }
  };
  // the rescaled O and l, computed where they stand (not sunk into the loop latch)
  auto pin_o = [&]() __attribute__((always_inline)) {
    pin(l_run);
#pragma unroll
    for (int c = 0; c < NCC; ++c) pin(o[c]);
  };

  // ---- prologue: S(0); the copies of K(2) and V(0) land during iteration 0
  if (tl >= 0) {
    if (hi_tile(0)) {
      ksc_next = __builtin_ldexpf(1.0f, -s_hi(0));
      qs_use = 1.0f;
    } else {
      v4i kf0[NCC][2];
      k_frags(kbuf(0), kf0);
      s_mfma(kf0);
    }
  }
  // the copies of "phase -2" (K(2), V(0); a tile past the last reads nothing)
  dma.k_next(lds0 + kbuf(2), w);
  dma.v_next(lds0 + vbuf(0), w);

  // ---- The schedule.  Each wave's iteration t is two halves:
  //        H1: P.V(t-1), 16 products (k-groups 0-3)  under part A of the softmax of tile t and
  //            part B for k-groups 0, 1 (P(t) overwrites the registers of P(t-1) those
  //            products consumed); the K fragments of S(t+1) are read here
  //        H2: S(t+1), 8 products                    under part B for k-groups 2, 3 and the
  //            rescale of O (after all of P.V(t-1))
  //      Each half starts at a workgroup barrier.  Group 1 (waves 4-7, rows 128-255 of the pair)
  //      runs one half behind group 0 (waves 0-3), so each SIMD, which holds one wave of each
  //      group, always runs one wave's H1 beside the other's H2: 24 matrix products and about
  //      the same vector work in every phase.  Inside a half, group barriers interleave one
  //      matrix instruction with a few vector ones, and pins keep results from being sunk into
  //      a later half.
  //      Phase 2t holds group 0's H1(t) and group 1's H2(t-1).  Both issue their shares of the
  //      copies K(t+3) -> buffer t mod 3 (held K(t), last read in phase 2t-1) and V(t+1) ->
  //      buffer (t+1) mod 3 (held V(t-2), last read in phase 2t-1), and each waits for them at
  //      the end of phase 2t+3, before their first reads in phase 2t+4.
  //      Kinds: 0 (FAST) all parts present and tile t unmasked (0 < t < tl); 1 each part where it
  //      applies (first, last and drain iterations); 2 no work of this wave.
  const int grp = w >> 2;   // group 0: waves 0-3, group 1: waves 4-7 (one of each per SIMD)
  Soft sm;             // softmax state of tile t between the halves
  v4i kf[NCC][2];      // K fragments of S(t+1) between the halves
  v8bf vf[2][NCC];
  // Phase 2t's copies (this wave's share), always issued: the target buffers are free in that
  // phase whatever t is, and a tile past the last copies no rows (zeros that are never read),
  // so the copy code and the wait counts are the same in every phase (no branches).
  auto copies = [&](int t, int j) __attribute__((always_inline)) {
    const int j1 = j == 2 ? 0 : j + 1;
    dma.k_next(lds0 + kbuf(j), w);    // K(t+3)
    dma.v_next(lds0 + vbuf(j1), w);   // V(t+1)
  };
  // wait until at most one phase's copies of this wave are in flight
  auto wait_copies = [&]() __attribute__((always_inline)) {
    wait_vm(PipeDma<D, PV8>::loads_of(w));
  };
  auto begin_half = [&]() __attribute__((always_inline)) {
    phase_barrier();
  };

  auto half1 = [&](int t, int j, auto kindc) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kindc)::value;
    constexpr bool FAST = KIND == 0;
    begin_half();
    // The scalar load of this tile's K scale was issued at the end of the previous half; it is
    // consumed here, before any LDS read of this half, because scalar and LDS returns share a
    // counter and scalar ones come back out of order (an LDS wait with a scalar load
    // outstanding waits for everything).
    if constexpr (PV8) {   // exact two-float product of the block scales and sm_scale * log2(e)
      const float kh = qscale * ksc_next, kl = __builtin_fmaf(qscale, ksc_next, -kh);
      dq = kh * p.sm_log2;
      dq_lo = __builtin_fmaf(kh, p.sm_log2, -dq) + __builtin_fmaf(kh, p.sm_log2_lo, kl * p.sm_log2);
      pin(dq_lo);
    } else {
      dq = __builtin_fmaxf(qs_use * ksc_next * p.sm_log2, 1.17549435e-38f);
    }
    pin(dq);
    __builtin_amdgcn_sched_barrier(0);
    const int j1 = j == 2 ? 0 : j + 1, j2 = j == 0 ? 2 : j - 1;
    const uint32_t kbs = kbuf(j1);   // K(t+1)
    const uint32_t vbs = vbuf(j2);   // V(t-1)
    if constexpr (PV8 && KIND != 2) {
      const bool do_sm = t <= tl, do_s = do_sm && t + 1 <= tl, do_pv = t >= 1 && t - 1 <= tl;
      if (FAST) {
        v8i v8f[NCC];
        k_frags(kbs, kf);
        v8_frags(vbs, v8f);
        soft_a8(sm, (int64_t)t * KT, false);
        pv8_mfma(v8f);
        soft_b8(sm, (int64_t)t * KT, false, 0);   // P(t) codes 0-3 after P.V(t-1) has read them
        pin(sm.alpha);
#pragma unroll
        for (int e = 0; e < 4; ++e) pin(pk[e]);
        SCHED_GROUP(SG_DS_READ, 2 * NCC + 2 * NCC, 0);
#pragma unroll
        for (int i = 0; i < NCC; ++i) { SCHED_GROUP(SG_MFMA, 1, 0); SCHED_GROUP(SG_VALU, 24, 0); }
        __builtin_amdgcn_sched_barrier(0);
        if (grp == 0) copies(t, j);
      } else {
        if (do_s) k_frags(kbs, kf);
        if (do_sm) soft_a8(sm, (int64_t)t * KT, tail_edge && t == tl);
        if (do_pv) {
          v8i v8f[NCC];
          v8_frags(vbs, v8f);
          pv8_mfma(v8f);
        }
        if (do_sm) soft_b8(sm, (int64_t)t * KT, tail_edge && t == tl, 0);
        if (grp == 0) copies(t, j);
      }
    } else if constexpr (KIND != 2) {
      if (FAST) {
        k_frags(kbs, kf);
        v_frags(vbs, 0, vf[0]);
        v_frags(vbs, 1, vf[1]);
        soft_a(sm, (int64_t)t * KT, false);
        pv_mfma(vf[0], 0);
        pv_mfma(vf[1], 1);
        pin(sm.alpha);
        SCHED_GROUP(SG_DS_READ, 2 * NCC + 4 * NCC, 0);
#pragma unroll
        for (int i = 0; i < 2 * NCC; ++i) { SCHED_GROUP(SG_MFMA, 1, 0); SCHED_GROUP(SG_VALU, 7, 0); }
        __builtin_amdgcn_sched_barrier(0);
        v_frags(vbs, 2, vf[0]);
        v_frags(vbs, 3, vf[1]);
        if (grp == 0) copies(t, j);
        pv_mfma(vf[0], 2);
        pv_mfma(vf[1], 3);
        soft_b(sm, 0);
        soft_b(sm, 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) pin(pk[e]);
        SCHED_GROUP(SG_DS_READ, 4 * NCC, 0);
#pragma unroll
        for (int i = 0; i < 2 * NCC; ++i) { SCHED_GROUP(SG_MFMA, 1, 0); SCHED_GROUP(SG_VALU, 7, 0); }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        const bool do_sm = t <= tl, do_s = do_sm && t + 1 <= tl, do_pv = t >= 1 && t - 1 <= tl;
        if (do_s) k_frags(kbs, kf);
        if (do_sm) soft_a(sm, (int64_t)t * KT, tail_edge && t == tl);
        if (do_pv) {
          v_frags(vbs, 0, vf[0]);
          v_frags(vbs, 1, vf[1]);
          pv_mfma(vf[0], 0);
          pv_mfma(vf[1], 1);
          v_frags(vbs, 2, vf[0]);
          v_frags(vbs, 3, vf[1]);
        }
        if (grp == 0) copies(t, j);
        if (do_pv) {
          pv_mfma(vf[0], 2);
          pv_mfma(vf[1], 3);
        }
        if (do_sm) {
          soft_b(sm, 0);
          soft_b(sm, 1);
        }
      }
    } else if (grp == 0) {
      copies(t, j);
    }
    // group 1: the copies of phase 2t-2 (its H2(t-2)) have landed; those of phase 2t may fly
    if (grp == 1) wait_copies();
  };

  auto half2 = [&](int t, int j, auto kindc) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kindc)::value;
    constexpr bool FAST = KIND == 0;
    begin_half();
    hi_nxt = false;
    if constexpr (PV8 && KIND != 2) {
      const bool do_sm = t <= tl, do_s = do_sm && t + 1 <= tl;
      if (grp == 1) copies(t + 1, j == 2 ? 0 : j + 1);
      if (FAST) {
        s_mfma(kf);
        soft_b8(sm, (int64_t)t * KT, false, 1);
        rescale(sm);
        pin_o();
#pragma unroll
        for (int e = 4; e < 8; ++e) pin(pk[e]);
#pragma unroll
        for (int i = 0; i < 2 * NCC; ++i) { SCHED_GROUP(SG_MFMA, 1, 0); SCHED_GROUP(SG_VALU, 8, 0); }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        if (do_s) s_mfma(kf);
        if (do_sm) {
          soft_b8(sm, (int64_t)t * KT, tail_edge && t == tl, 1);
          rescale(sm);
        }
      }
    } else if constexpr (KIND != 2) {
      if (FAST) {
        if (grp == 1) copies(t + 1, j == 2 ? 0 : j + 1);
        s_mfma(kf);
        soft_b(sm, 2);
        soft_b(sm, 3);
        rescale(sm);
        pin_o();
#pragma unroll
        for (int e = 8; e < 16; ++e) pin(pk[e]);
#pragma unroll
        for (int i = 0; i < 2 * NCC; ++i) { SCHED_GROUP(SG_MFMA, 1, 0); SCHED_GROUP(SG_VALU, 14, 0); }
        __builtin_amdgcn_sched_barrier(0);
        hi_nxt = hi_tile(t + 1);   // Thrift: S(t+1) redone on bf16 (rare; outside the interleave)
        if (THRIFT && hi_nxt) k_nxt = s_hi(t + 1);
      } else {
        const bool do_sm = t <= tl, do_s = do_sm && t + 1 <= tl;
        if (grp == 1) copies(t + 1, j == 2 ? 0 : j + 1);
        if (do_s) s_mfma(kf);
        hi_nxt = do_s && hi_tile(t + 1);
        if (THRIFT && hi_nxt) k_nxt = s_hi(t + 1);
        if (do_sm) {
          soft_b(sm, 2);
          soft_b(sm, 3);
          rescale(sm);
        }
      }
    } else if (grp == 1) {
      copies(t + 1, j == 2 ? 0 : j + 1);
    }
    if (t + 1 < nT) ksc_next = kscales[t + 1];   // consumed after the next barrier
    qs_use = qscale;
    if (THRIFT && hi_nxt) {
      ksc_next = __builtin_ldexpf(1.0f, -k_nxt);
      qs_use = 1.0f;
    }
    // group 0: the copies of phase 2t-2 (its H1(t-1)) have landed; those of phase 2t may fly
    if (grp == 0) wait_copies();
  };

  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  // Group 1 first passes one barrier and issues its share of phase 0's copies (its H2(-1));
  // group 0 ends with one extra barrier: every wave passes 2 nT + 3 barriers.
  if (grp == 1) {
    begin_half();
    copies(0, 0);
  }
  int t = 0, j = 0;
  auto iter = [&](auto kindc) __attribute__((always_inline)) {
    half1(t, j, kindc);
    half2(t, j, kindc);
    ++t;
    j = j == 2 ? 0 : j + 1;
  };
  if (tl >= 0) {
    iter(K1{});                        // softmax(0), S(1)
    while (t < tl) iter(K0{});
    if (tl >= 1) iter(K1{});           // P.V(tl-1), softmax(tl) (masked if edge)
    iter(K1{});                        // P.V(tl)
  }
  while (t <= nT) iter(K2{});
  if (grp == 0) begin_half();

  // ---- epilogue: O / l; lane (li, lh) holds row qrow, channels 32cc + 8(r/4) + 4lh + (r%4)
  // (FP8 P: l sums 1.75 P and O sums E4M3(448 P) V, so O / l carries an extra 256; the V
  // channel scales are applied here)
  const float l_tot = halves_sum(l_run) * (PV8 ? 256.0f : 1.0f);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_ok) {
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = 32 * cc + 8 * g + 4 * lh;
        float v0 = o[cc][4 * g] * inv, v1 = o[cc][4 * g + 1] * inv, v2 = o[cc][4 * g + 2] * inv,
              v3 = o[cc][4 * g + 3] * inv;
        if (PV8) {
          const float* vsc = p.vs + bkv * D + ch;
          v0 *= vsc[0]; v1 *= vsc[1]; v2 *= vsc[2]; v3 *= vsc[3];
        }
        const int64_t off = p.outr.at(bh, qrow) + ch;
        if (OUT_BF16) *(v2i*)((uint16_t*)p.out + off) = v2i{(int)pack_bf16x2(v0, v1), (int)pack_bf16x2(v2, v3)};
        else *(v4f*)((float*)p.out + off) = v4f{v0, v1, v2, v3};
      }
  }
}

template <int D, bool CAUSAL, bool VF16, bool OUT_BF16>
hipError_t launch_pipe(const PipeParams& p, hipStream_t st) {
  if (p.total_wg == 0) return hipSuccess;
  if (p.mask)
    hipLaunchKernelGGL((attn_i8_pipe_kernel<D, CAUSAL, VF16, OUT_BF16, true, false>), dim3((unsigned)p.total_wg),
                       dim3(NTHREADS), 0, st, p, p.ks);
  else if (p.v8)
    hipLaunchKernelGGL((attn_i8_pipe_kernel<D, CAUSAL, false, OUT_BF16, false, true>), dim3((unsigned)p.total_wg),
                       dim3(NTHREADS), 0, st, p, p.ks);
  else
    hipLaunchKernelGGL((attn_i8_pipe_kernel<D, CAUSAL, VF16, OUT_BF16, false, false>), dim3((unsigned)p.total_wg),
                       dim3(NTHREADS), 0, st, p, p.ks);
  return hipGetLastError();
}

// fp16 V at D = 128 is not built here (its conversions would not fit the register budget)
template <int D, bool CAUSAL>
hipError_t dispatch_pipe(const PipeParams& p, bool vf16, bool out_bf16, hipStream_t st) {
  if constexpr (D == 64) {
    if (vf16) return out_bf16 ? launch_pipe<D, CAUSAL, true, true>(p, st) : launch_pipe<D, CAUSAL, true, false>(p, st);
  } else {
    if (vf16) return hipErrorNotSupported;
  }
  return out_bf16 ? launch_pipe<D, CAUSAL, false, true>(p, st) : launch_pipe<D, CAUSAL, false, false>(p, st);
}

}  // namespace

hipError_t launch_attn_int8_pipe(const AttnArgs& a, int pv_fp8, hipStream_t st) {
  PipeParams p;
  // FP8 P.V: FP8 V^T codes and channel scales (INT8 tiles only: no Thrift mask, no fp16 V)
  p.v8 = pv_fp8 ? (const uint8_t*)a.v_codes : nullptr;
  p.vs = pv_fp8 ? (const float*)a.v_scales : nullptr;
  if (pv_fp8 && (a.mask || a.v_is_f16)) return hipErrorNotSupported;
  p.q = (const int8_t*)a.q_codes; p.qs = (const float*)a.q_scales;
  p.k = (const int8_t*)a.k_codes; p.ks = (const float*)a.k_scales;
  p.v = (const uint16_t*)a.v_codes;
  p.out = a.out;
  p.vr = a.vr; p.outr = a.outr;
  p.mask = a.mask; p.qhi = a.q_hi; p.khi = a.k_hi;
  p.q16 = a.q16; p.q16r = a.q16r; p.q16_f16 = a.q16_f16;
  p.qhr = a.qhr; p.khr = a.khr;
  if (p.mask && (a.N + KT - 1) / KT > PIPE_MAX_MASK_TILES) return hipErrorInvalidValue;   // mask rows past LDS
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N;
  p.nQB = (a.N + QB - 1) / QB; p.nKB = (a.N + KT - 1) / KT;
  p.nPairs = (p.nQB + 1) / 2;
  p.total_wg = a.B * a.Hq * p.nPairs;
  {
    const double l2 = (double)a.sm_scale * 1.4426950408889634074;
    p.sm_log2 = (float)l2;
    p.sm_log2_lo = (float)(l2 - (double)p.sm_log2);
  }
  p.Np = (a.N + KT - 1) / KT * KT;
  const bool causal = a.causal != 0;
  if (a.D == 64) return causal ? dispatch_pipe<64, true>(p, a.v_is_f16, a.out_bf16, st)
                               : dispatch_pipe<64, false>(p, a.v_is_f16, a.out_bf16, st);
  return causal ? dispatch_pipe<128, true>(p, a.v_is_f16, a.out_bf16, st)
                : dispatch_pipe<128, false>(p, a.v_is_f16, a.out_bf16, st);
}

}  // namespace sage
