// Decode-shaped attention on a KV cache held in NVFP4 — "Search Your Block Floating Point
// Scales!", Method > ScaleSearchAttention (the KV cache kept in 4 bits).  A few new query rows
// attend to a long cache.  K rows are NVFP4 along D (per token and 16-channel group, 8 code
// bytes and one UE4M3 scale: sage_quantize_blocks' (1, 16) layout); V is NVFP4 along the
// tokens (per channel and 16-token group: the (16, 1) layout), the operand order P.V wants.
// Q stays 16-bit; P is rounded to f16 for the matrix product (its sum stays fp32).
//
// The work is reading the cache (144 bytes per key per KV head at d = 128).  Both products
// run on the matrix cores, so the vector work per key does not grow with the query rows:
//   * a workgroup takes consecutive 512-key chunks of one (b, KV head) for 16 query rows (the
//     q-heads of the KV head's group times the new tokens); in each chunk, each of its 4 waves
//     walks its own 128 keys in 16-key tiles with its own running max and sum (kept across the
//     chunks), merged at the end (log-sum-exp): the Q set-up and the merge are paid once per
//     workgroup, and the combine reads one partial per workgroup;
//   * S^T (16 keys x 16 rows) = K Q^T on v_mfma_f32_16x16x32_f16: lane (r, h) of the A
//     operand holds key r's 32 channels 32h..32h+31, dequantized in registers from one 16-byte
//     load (E2M1 pairs to f16 times the scale pair: exact); Q^T is the B operand with the same
//     channel order, loaded once (a bf16 row scaled by a power of two into f16's range: exact);
//   * the accumulator leaves lane (r, h) with row r's scores of keys 4h..4h+3: exactly the
//     B operand P^T of O^T (channels x rows) += V^T P^T on v_mfma_f32_16x16x16_f16, whose A
//     operand V^T needs 4 consecutive tokens of one channel: 2 bytes of the along-token codes;
//     f16 keeps 11 bits of P (bf16's 8 would cost about 1e-3 of max|O|);
//   * the running max moves only when a score passes it by 15 (log2 units), checked once per
//     tile for the whole wave; P <= 2^15 stays finite in f16;
//   * the workgroup's V codes and scales (512 tokens x 128 channels) go to LDS by direct
//     global->LDS loads (each channel row's 16-byte segments XOR-swizzled, so the 16 channel
//     lanes of a read hit distinct banks), after each wave's K loads for its first 4 tiles;
//     V's 2-byte pieces are then read from LDS, lane row r taking channels 8r..8r+7, whose
//     8 scale bytes are one 8-byte read (UE4M3 scales convert to f16 in pairs, exactly);
//   * a split writes only the R real rows of its partial O (not the 16 of the row group).
// decode_combine_kernel merges the splits and writes O.
#include "device.hpp"
#include "kernels.hpp"

#include <atomic>
#include <mutex>

namespace sage {
namespace {

constexpr int DK = 128;             // head dimension
constexpr int DEC_CHUNK = 512;      // keys staged in LDS at a time
constexpr int DEC_MAX_CHUNKS = 8;  // chunks one split workgroup may take
constexpr int DEC_SLOTS = 1024;     // workgroups resident at once: 256 CUs x 4
constexpr int DEC_THREADS = 256;    // 4 waves x 8 key slots
constexpr float kLazy = 15.0f;      // headroom of the running max, log2 units (P <= 2^15 fits f16)

struct DecodeArgs {
  const uint16_t* q;                           // [B, Hq, Nq, 128] 16-bit, rows qr
  Rows16 qr;
  const uint8_t *kc, *ks;                      // K codes [B, Hkv, Nk, 64], scales [B, Hkv, Nk, 8]
  const uint8_t *vc, *vs;                      // V codes [B, Hkv, 128, Np/2], scales [B, Hkv, Np/16, 128]
  float* part_o;                               // [B * Hkv, nsplit, R, 128]
  float* part_ml;                              // [B * Hkv, nsplit, R, 2]
  int64_t Hq, Hkv, Nq, Nk, Np, nsplit, R, nrg; // R = (Hq / Hkv) * Nq rows per KV head, nrg groups of 16
  int chunks;                                  // 512-key chunks per split
  int causal;
  float qscale;                                // sm_scale * log2(e)
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

struct Tile {
  v4i kw;          // key (key0 + r)'s code bytes 16h..16h+15
  uint32_t ks2;    // its two scale bytes (groups 2h, 2h + 1)
};

// V in LDS: channel c's codes in a 256-byte row whose 16-byte segment s sits at s ^ vswz(c),
// then the scales [32 token groups][128 channels].  The matrix product reads channels 8r + cb
// in lanes r = 0..15, so the swizzle (r) puts the 16 lanes' 4-byte words in distinct banks.
constexpr int VROW = DEC_CHUNK / 2;                  // LDS bytes of a channel's codes
constexpr int VSC0 = DK * VROW;                      // LDS offset of the scales
constexpr int VLDS = VSC0 + (DEC_CHUNK / 16) * DK;   // 36864 bytes
constexpr int SH_ROW = DK + 4;                       // merge rows padded: 16 rows hit distinct banks
static_assert(4 * 16 * SH_ROW * 4 <= VLDS, "the merge fits the V area");
__device__ __forceinline__ uint32_t vswz(uint32_t c) { return (c >> 3) & 15u; }
typedef __attribute__((address_space(3))) void lds_void;

// Up to four workgroups a CU (36 KB of LDS each): a register budget of 128 per lane.
template <bool F16>
__global__ __launch_bounds__(DEC_THREADS, 4) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t vl[VLDS];   // V codes + scales; later the merge
  __shared__ float sh_m[4][16], sh_l[4][16];
  const int64_t id = blockIdx.x;
  const int64_t rg = id % a.nrg, split = (id / a.nrg) % a.nsplit, bkv = id / a.nrg / a.nsplit;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r = lane & 15, h = lane >> 4;
  const int64_t G = a.Hq / a.Hkv, b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  constexpr float NEG = -__builtin_inff();

  // Q^T operand in f16: row r of the group, channels 32h + 8kk .. +7 for kk = 0..3 (rows past
  // R: zero).  A bf16 row is first scaled by 2^-E, E >= 0 the least that brings its largest
  // magnitude to 2^14 or below: every bf16 value then lands exactly in f16 (8 significant bits
  // of 11; a component below 2^-14 of that scale would become an f16 subnormal, below 2^-28 of
  // the row's largest term), and 2^E goes into the row's score scale.
  const int64_t row = rg * 16 + r;
  const bool act = row < a.R;
  int qpos = -1;   // the last visible key of this row (-1: none)
  v8h qb[4];
  float qs = a.qscale;
  {
    const int64_t rr = act ? row : 0;
    const int64_t hq = kvh * G + rr / a.Nq, i = rr % a.Nq;
    if (act) qpos = (int)(a.Nk - a.Nq + i);
    const uint16_t* qp = a.q + a.qr.at(b * a.Hq + hq, i) + 32 * h;
    v4i w[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) w[kk] = act ? *(const v4i*)(qp + 8 * kk) : v4i{0, 0, 0, 0};
    if constexpr (F16) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[kk] = __builtin_bit_cast(v8h, w[kk]);
    } else {
      float x[4][8];
      float mx = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[kk][e] = bf16_to_f32((uint16_t)((uint32_t)w[kk][e >> 1] >> (16 * (e & 1))));
          mx = __builtin_fmaxf(mx, __builtin_fabsf(x[kk][e]));
        }
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));   // the row's 128 channels sit in lanes r + 16h
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      const int ex = (int)((__float_as_uint(mx) >> 23) & 255u) - 127;   // mx = 1.f * 2^ex (or 0)
      const int E = ex > 14 ? ex - 14 : 0;
      const float down = __builtin_ldexpf(1.0f, -E);
      qs = qs * __builtin_ldexpf(1.0f, E);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[kk][e] = (_Float16)(x[kk][e] * down);
    }
  }
  float m = NEG, lpart = 0.0f;
  v4f o[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) o[cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int Nk = (int)a.Nk;
  const uint32_t hNp = (uint32_t)(a.Np / 2);
  const uint8_t* kc = a.kc + bkv * a.Nk * 64;
  const uint8_t* ks = a.ks + bkv * a.Nk * 8;
  const uint8_t* vc = a.vc + bkv * DK * (a.Np / 2);
  const uint8_t* vs = a.vs + bkv * (a.Np / 16) * DK;
  const bool causal = a.causal != 0;
  const int vis_all = causal ? Nk - (int)a.Nq + 1 : Nk;   // keys below it are visible to every row
  constexpr int TILES = DEC_CHUNK / 64, DEPTH = 4;   // 8 tiles of 16 keys per wave, 4 in flight
  static_assert(TILES % DEPTH == 0, "whole rounds of the ring");
  for (int chunk = 0; chunk < a.chunks; ++chunk) {
    const int j0 = (int)((split * a.chunks + chunk) * DEC_CHUNK);
    if (j0 >= Nk) break;   // workgroup-uniform
    if (chunk > 0) __syncthreads();   // every wave is done with the previous chunk's V
    // this wave's tile it starts at key j0 + (DEC_CHUNK / 4) wv + 16 it; K rows past the cache
    // are clamped (their keys are masked)
    auto load = [&](int it, Tile& T) __attribute__((always_inline)) {
      const int key0 = j0 + (DEC_CHUNK / 4) * wv + 16 * it;
      const uint32_t jk = (uint32_t)(key0 + r < Nk ? key0 + r : Nk - 1);
      T.kw = *(const v4i*)(kc + jk * 64u + 16u * (uint32_t)h);
      T.ks2 = *(const uint16_t*)(ks + jk * 8u + 2u * (uint32_t)h);
    };
    Tile ring[DEPTH];   // the first tiles' K loads go out before V's
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) load(u, ring[u]);
    // V of the chunk into LDS by direct global->LDS loads (no registers): a wave instruction
    // fills 1 KB of LDS, lane i its 16-byte slot i, and each lane fetches the global segment that
    // belongs to its slot.  Code slots: row c (channel) x 16 physical segments, the logical
    // segment being the physical one XOR vswz(c); then the scale slots: 32 token groups x 8
    // segments.  Segments past the padded cache fetch the row's last valid one (finite codes and
    // scales; their keys are masked).
    {
      constexpr int CODE_SLOTS = DK * (VROW / 16), SLOTS = CODE_SLOTS + (DEC_CHUNK / 16) * (DK / 16);
      static_assert(SLOTS % 64 == 0 && VROW == 256, "whole wave instructions; 16 segments a row");
      const uint32_t cb0 = (uint32_t)j0 / 2u, nb = (uint32_t)hNp;      // code bytes of a channel row
      const uint32_t g0 = (uint32_t)j0 / 16u, ng = (uint32_t)(a.Np / 16);
      for (int k = wv; k < SLOTS / 64; k += 4) {
        const uint32_t slot = 64u * (uint32_t)k + (uint32_t)lane;
        const uint8_t* src;
        if (slot < (uint32_t)CODE_SLOTS) {
          const uint32_t row = slot >> 4, seg = (slot & 15u) ^ vswz(row);
          uint32_t at = cb0 + 16u * seg;
          at = at < nb ? at : nb - 16u;
          src = vc + row * nb + at;
        } else {
          const uint32_t t2 = slot - (uint32_t)CODE_SLOTS, gi = t2 / (DK / 16), cs = t2 % (DK / 16);
          const uint32_t gg = g0 + gi < ng ? g0 + gi : ng - 1u;
          src = vs + gg * DK + 16u * cs;
        }
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(vl + 1024 * k), 16, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the direct loads (and the K ring) have landed
    __syncthreads();   // V is in LDS
    for (int it0 = 0; it0 < TILES; it0 += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int it = it0 + u;
        const Tile T = ring[u];
        if (it + DEPTH < TILES) load(it + DEPTH, ring[u]);   // wave-uniform
        const int kl0 = (DEC_CHUNK / 4) * wv + 16 * it;      // the tile's first key within the chunk
        const int key0 = j0 + kl0;
        // S^T = K Q^T over the 4 channel slices
        v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        // K in f16: the E2M1 pairs times the group's scale pair (exact: E2M1 x UE4M3); the two
        // UE4M3 scale bytes go to f16 in one conversion (E4M3 values are exact in f16)
        const v2h hs = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(T.ks2, 1.0f, false);
        const _Float16 h0 = hs[0], h1 = hs[1];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t u = (uint32_t)T.kw[kk];
          const v2h sc = kk < 2 ? v2h{h0, h0} : v2h{h1, h1};
          const v2h k0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 0) * sc;
          const v2h k1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 1) * sc;
          const v2h k2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 2) * sc;
          const v2h k3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, 3) * sc;
          const v8h ka = v8h{k0[0], k0[1], k1[0], k1[1], k2[0], k2[1], k3[0], k3[1]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[kk], acc, 0, 0, 0);
        }
        // row r's scores of keys key0 + 4h + e, in log2 units.  A tile below vis_all is
        // visible to every row and takes no mask (rows past R hold a zero query: finite scores,
        // never written); otherwise masked keys are -inf.
        float p[4];
        bool up = false;
        const bool full = key0 + 16 <= vis_all;   // wave-uniform
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = key0 + 4 * h + e;
          const bool vis = full || (j < Nk && (causal ? j <= qpos : qpos >= 0));
          p[e] = vis ? acc[e] * qs : NEG;
          up |= p[e] > m + kLazy;   // also the first visible key (m = -inf)
        }
        if (__builtin_amdgcn_ballot_w64(up) != 0) {   // wave-uniform: move the running max
          float tmax = __builtin_fmaxf(__builtin_fmaxf(p[0], p[1]), __builtin_fmaxf(p[2], p[3]));
          tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16));   // the row's 16 keys sit in lanes r + 16h
          tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
          if (tmax > m + kLazy) {
            const float alpha = m == NEG ? 0.0f : __builtin_amdgcn_exp2f(m - tmax);
            lpart *= alpha;
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) o[cb] *= alpha;
            m = tmax;
          }
        }
        if (full) {   // every score finite, so m is too
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = __builtin_amdgcn_exp2f(p[e] - m);
            lpart += p[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = p[e] == NEG ? 0.0f : __builtin_amdgcn_exp2f(p[e] - m);   // m may still be -inf
            lpart += p[e];
          }
        }
        const v4h pb = v4h{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
        // O^T += V^T P^T over the 8 channel blocks: block cb gives lane row r channel 8r + cb
        // (codes of tokens 4h..4h+3: two bytes; the 8 scale bytes of channels 8r..8r+7 are
        // adjacent and convert to f16 in pairs)
        const uint32_t vo = (uint32_t)kl0 / 2u + 2u * (uint32_t)h;
        const uint32_t vrow = (uint32_t)r * (8u * VROW) + ((((vo >> 4) ^ (uint32_t)r) << 4) | (vo & 15u));
        const uint2 sw = *(const uint2*)(vl + VSC0 + ((uint32_t)kl0 / 16u) * DK + 8u * (uint32_t)r);
        const v2h vs01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw.x, 1.0f, false);
        const v2h vs23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw.x, 1.0f, true);
        const v2h vs45 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw.y, 1.0f, false);
        const v2h vs67 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw.y, 1.0f, true);
        const _Float16 vsc8[8] = {vs01[0], vs01[1], vs23[0], vs23[1], vs45[0], vs45[1], vs67[0], vs67[1]};
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const uint32_t vw = *(const uint16_t*)(vl + vrow + (uint32_t)cb * VROW);   // channel 8r + cb
          const v2h sc2 = v2h{vsc8[cb], vsc8[cb]};
          const v2h d0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vw, 1.0f, 0) * sc2;   // exact: E2M1 x UE4M3
          const v2h d1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vw, 1.0f, 1) * sc2;
          const v4h va = v4h{d0[0], d0[1], d1[0], d1[1]};
          o[cb] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb, o[cb], 0, 0, 0);
        }
      }
    }
  }
  // this wave's row sums: row r's keys sit in lanes r + 16h
  float lrow = lpart + __shfl_xor(lpart, 16);
  lrow += __shfl_xor(lrow, 32);
  // O^T: lane (r, h) holds row r, channels 8 (4h + e) + cb; the V area becomes [4][16][SH_ROW]
  __syncthreads();   // every wave is done with V
  float(*sh_o)[16][SH_ROW] = reinterpret_cast<float(*)[16][SH_ROW]>(vl);
  // the lane's indices again from the thread id (an opaque copy: keeping the set-up's values
  // alive across the key loop would cost registers there)
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int mr = (int)(tid & 15u), mh = (int)((tid >> 4) & 3u);
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) sh_o[wv][mr][8 * (4 * mh + e) + cb] = o[cb][e];
  if (mh == 0) {
    sh_m[wv][mr] = m;
    sh_l[wv][mr] = lrow;
  }
  __syncthreads();
  // merge the 4 waves; write this split's unnormalized O with its max and sum
  for (int i = threadIdx.x; i < 16 * DK; i += DEC_THREADS) {
    const int rr = i / DK, c = i % DK;
    float M = sh_m[0][rr];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = __builtin_fmaxf(M, sh_m[w][rr]);
    float accv = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = M == NEG ? 0.0f : __builtin_amdgcn_exp2f(sh_m[w][rr] - M);
      accv += sh_o[w][rr][c] * wt;
      L += sh_l[w][rr] * wt;
    }
    const int64_t grow = rg * 16 + rr;   // the row within the KV head's R rows
    if (grow >= a.R) continue;
    const int64_t prow = (bkv * a.nsplit + split) * a.R + grow;
    a.part_o[prow * DK + c] = accv;
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
                                                            int64_t Hkv, int64_t Nq, int64_t R,
                                                            int64_t nsplit, int out_bf16, void* out) {
  __shared__ float wt[1024];
  __shared__ float red[2];
  const int64_t row = blockIdx.x % R, bkv = blockIdx.x / R;
  const int c = threadIdx.x;
  constexpr float NEG = -__builtin_inff();
  auto ml = [&](int64_t s, int k) { return part_ml[((bkv * nsplit + s) * R + row) * 2 + k]; };
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
      for (int u = 0; u < 8; ++u) v[u] = part_o[((bkv * nsplit + s0 + s + u) * R + row) * DK + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) num += v[u] * wt[s + u];
    }
    for (; s < n; ++s) num += part_o[((bkv * nsplit + s0 + s) * R + row) * DK + c] * wt[s];
  }
  const int64_t G = Hq / Hkv, b = bkv / Hkv, hq = (bkv % Hkv) * G + row / Nq, qi = row % Nq;
  const int64_t at = ((b * Hq + hq) * Nq + qi) * DK + c;
  const float v = num / den;
  if (out_bf16) ((uint16_t*)out)[at] = f32_to_bf16(v);
  else ((float*)out)[at] = v;
}

}  // namespace

// Chunks per split: as many as keep one round of resident workgroups busy (more chunks per
// workgroup pay the Q set-up and the merge fewer times and leave fewer partials to combine).
static int64_t decode_chunks(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk) {
  const int64_t nrg = ((Hq / Hkv) * Nq + 15) / 16, nchunk = (Nk + DEC_CHUNK - 1) / DEC_CHUNK;
  const int64_t c = (B * Hkv * nrg * nchunk) / DEC_SLOTS;
  return c < 1 ? 1 : c > DEC_MAX_CHUNKS ? DEC_MAX_CHUNKS : c;
}

static int64_t decode_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk) {
  const int64_t per = DEC_CHUNK * decode_chunks(B, Hq, Hkv, Nq, Nk);
  return (Nk + per - 1) / per;
}

size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk) {
  const int64_t R = (Hq / Hkv) * Nq;
  const int64_t nsplit = decode_splits(B, Hq, Hkv, Nq, Nk);
  return (size_t)(B * Hkv * nsplit * R) * (DK + 2) * sizeof(float);
}

hipError_t launch_decode(const uint16_t* q, const Rows16& qr, bool q_f16, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t Nq, int64_t Nk, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                         const uint8_t* vs, int causal, float sm_scale, void* out, bool out_bf16, void* ws,
                         hipStream_t st) {
  const int64_t R = (Hq / Hkv) * Nq, nrg = (R + 15) / 16;
  const int64_t nsplit = decode_splits(B, Hq, Hkv, Nq, Nk);
  DecodeArgs a;
  a.q = q;
  a.qr = qr;
  a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs;
  a.part_o = (float*)ws;
  a.part_ml = (float*)ws + B * Hkv * nsplit * R * DK;
  a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.Np = (Nk + 63) / 64 * 64;
  a.nsplit = nsplit; a.R = R; a.nrg = nrg;
  a.chunks = (int)decode_chunks(B, Hq, Hkv, Nq, Nk);
  a.causal = causal;
  a.qscale = (float)((double)sm_scale * 1.4426950408889634);
  const int64_t nwg = B * Hkv * nsplit * nrg;
  if (q_f16) decode_split_kernel<true><<<(unsigned)nwg, DEC_THREADS, 0, st>>>(a);
  else decode_split_kernel<false><<<(unsigned)nwg, DEC_THREADS, 0, st>>>(a);
  decode_combine_kernel<<<(unsigned)(B * Hkv * R), DK, 0, st>>>(a.part_o, a.part_ml, Hq, Hkv, Nq, R, nsplit,
                                                                 out_bf16 ? 1 : 0, out);
  return hipGetLastError();
}

// ---- scratch of the allocation-free entry point (sage_decode_fwd_noalloc): the split
// partials live in this array instead of a caller workspace.  Every GPU the library runs on
// holds its own copy until the process ends; calls on one GPU share it.  In host code the
// name is only a stand-in: kernels get the device address that decode_scratch looks up.
static __device__ __align__(256) uint8_t scratch[DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(void** p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* a = g_scratch[dev].load(std::memory_order_acquire);
  if (a == nullptr) {   // first call on this device: look the address up with the device current
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    a = g_scratch[dev].load(std::memory_order_relaxed);
    if (a == nullptr) {
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (a == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(a, std::memory_order_release);
    }
  }
  *p = a;
  return hipSuccess;
}

}  // namespace sage
