// Block quantizers.
//  * INT8 per block (SageAttention, Technical approach: Q and K in 8 bits): s = amax / 127,
//    code = clamp(round_half_even(x * (1/s)), -127, 127).  The block is held in registers
//    between the reduction and the encoding: 3 bytes of HBM per 16-bit element.
//  * E4M3 per channel for V: amax over all tokens (atomic max on the bit pattern of a
//    non-negative float), then codes written channel-major through an LDS transpose.
//  * MX-FP4 (SageAttention3's microscaled FP4): E8M0 per 32 elements, e = smallest integer
//    with 6 * 2^e >= amax, codes E2M1(x * 2^-e).
//  * NVFP4 with max-scaling or ScaleSearch ("Search Your Block Floating Point Scales!",
//    Method > ScaleSearch): per 16 elements, the UE4M3 scale among the candidates whose
//    E2M1 reconstruction has the least squared error (fp32, balanced index-order tree, first
//    strictly smaller wins, the max-scaling candidate first).  This one is ALU-bound: about
//    nine candidates x ten operations per element.
//  * NVFP4 -> MXFP8 for the FP8 matrix-core path.
//  * Optional Hadamard incoherence processing of the rows along D ("Search Your Block
//    Floating Point Scales!", Method > ScaleSearchAttention) inside the along-D quantizers:
//    each row times the normalized Sylvester Hadamard matrix, so Q'K'^T = QK^T.
// Compiled with -ffp-contract=off: every expression rounds as written.
#include "device.hpp"
#include "kernels.hpp"

#include <cmath>
#include <type_traits>

namespace sage {
namespace {

// K smoothing applied on the fly (sage_quantize_smoothed): eight 16-bit values of channels
// ch0 .. ch0+7 become round_to_dtype(fp32(x - mean)), the same arithmetic as the smoothing
// kernel's output, so the quantized result equals quantizing the stored K_s.
template <bool F16>
__device__ __forceinline__ v4i smooth_vals(v4i raw, const v4f m0, const v4f m1) {
  const float m[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
  v4i o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t u = (uint32_t)raw[w];
    const float a = in16_to_f32<F16>((uint16_t)(u & 0xffffu)) - m[2 * w];
    const float b = in16_to_f32<F16>((uint16_t)(u >> 16)) - m[2 * w + 1];
    o[w] = (int)((uint32_t)f32_to_in16<F16>(a) | ((uint32_t)f32_to_in16<F16>(b) << 16));
  }
  return o;
}
template <bool F16>
__device__ __forceinline__ v4i smooth_chunk(v4i raw, const float* __restrict__ mu) {
  return smooth_vals<F16>(raw, *(const v4f*)mu, *(const v4f*)(mu + 4));
}

// ------------------------------------------------------------------ INT8 codes
// int8_recip, int8_code_bits and pack_bytes (device.hpp) form the codes; the attention kernel's
// in-kernel quantization of 16-bit Q uses the same three.

// ------------------------------------------------------------------ Hadamard along D
// The fast Walsh-Hadamard transform of a row of D values in fp32: stages h = 1, 2, ...,
// D/2, each replacing the pair (v[j], v[j+h]) (j mod 2h < h) by (v[j] + v[j+h],
// v[j] - v[j+h]); then one multiply by fp32(1/sqrt(D)).  A thread holds n consecutive values
// of the row and the row's threads sit in consecutive lanes, so the stages h < n run inside
// the thread and the stage h = n m pairs lane L with lane L ^ m.  Every add and subtract is
// the same fp32 operation on the same operands as in the plain stage-by-stage transform.
template <int n>
__device__ __forceinline__ void fwht_in_thread(float* v) {
#pragma unroll
  for (int h = 1; h < n; h *= 2)
#pragma unroll
    for (int i = 0; i < n; i += 2 * h)
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

// The stages h = n m, m = 1, 2, .., LPR/2, for `cnt` values per lane, where a row's values
// sit n per lane in LPR consecutive lanes.  The lower lane of a pair forms mine + other, the
// upper one other - mine, written other + (-mine): the same IEEE result.  VIA_LDS: the
// partner's value comes through the LDS crossbar (ds_bpermute) instead of DPP, which keeps
// the exchange off the vector ALU (for kernels bound by it).
template <int LPR, bool VIA_LDS = false>
__device__ __forceinline__ void fwht_across_lanes(float* v, int cnt) {
  const int lane = threadIdx.x & 63;
  auto stage = [&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
    const uint32_t sign = (lane & m) ? 0x80000000u : 0u;
#pragma unroll
    for (int j = 0; j < cnt; ++j) {
      const float other = VIA_LDS ? __shfl_xor(v[j], m) : lane_xor<m>(v[j]);
      v[j] = other + __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[j]) ^ sign);
    }
  };
  if constexpr (LPR > 1) stage(std::integral_constant<int, 1>{});
  if constexpr (LPR > 2) stage(std::integral_constant<int, 2>{});
  if constexpr (LPR > 4) stage(std::integral_constant<int, 4>{});
  if constexpr (LPR > 8) stage(std::integral_constant<int, 8>{});
  static_assert(LPR <= 16, "a row spans at most 16 lanes");
}

// ------------------------------------------------------------------ INT8 per block
// One workgroup per block of T tokens x D channels; the block (T * D / 8 16-byte chunks)
// stays in registers between the amax reduction and the encoding, so HBM is read once.
// HAD: the rows are Hadamard-transformed first (D in {64, 128}: a row is D/8 chunks, held by
// D/8 consecutive lanes); the block is then held as fp32.
template <bool F16, int CPT, bool SMOOTH, bool HAD = false>   // CPT = 16-byte chunks per thread (T * D / 8 / 256)
__global__ __launch_bounds__(256) void quant_int8_kernel(const uint16_t* __restrict__ x, Rows16 xr, int64_t N, int D,
                                                         int T, const float* __restrict__ mean,
                                                         int8_t* __restrict__ codes, float* __restrict__ scales,
                                                         float hscale = 0.0f) {
  const int64_t nblk = (N + T - 1) / T;
  const int64_t blk = blockIdx.x, bh = blockIdx.y;
  const int64_t t0 = blk * T;
  const int rows = (int)((N - t0) < T ? (N - t0) : T);
  const int nchunk = rows * D / 8, cpr = D / 8;
  const uint16_t* base = x + xr.at(bh, t0);   // chunk c: row c / cpr, channels 8 (c % cpr) ..
  v4i raw[CPT];
  if (256 % cpr == 0) {   // chunks tid + 256 i share their channels: row tid / cpr + i * (256 / cpr)
    const int r0 = (int)threadIdx.x / cpr, rstep = 256 / cpr;
    const uint16_t* p0 = base + r0 * xr.sn + ((int)threadIdx.x - r0 * cpr) * 8;
    const int64_t step = rstep * xr.sn;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      raw[i] = r0 + i * rstep < rows ? *(const v4i*)(p0 + i * step) : v4i{0, 0, 0, 0};
  } else {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + 256 * i, r = c / cpr;
      raw[i] = c < nchunk ? *(const v4i*)(base + r * xr.sn + (c - r * cpr) * 8) : v4i{0, 0, 0, 0};
    }
  }
  if (SMOOTH) {
    if ((2048 % D) == 0) {   // chunks tid + 256 i all start at channel 8 tid mod D: one mean slice
      const float* mu = mean + bh * D + (threadIdx.x * 8) % D;
      const v4f m0 = *(const v4f*)mu, m1 = *(const v4f*)(mu + 4);
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        if ((int)threadIdx.x + 256 * i < nchunk) raw[i] = smooth_vals<F16>(raw[i], m0, m1);
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < nchunk) raw[i] = smooth_chunk<F16>(raw[i], mean + bh * D + (c * 8) % D);
      }
    }
  }
  float hv[HAD ? CPT : 1][8];   // HAD: the transformed block
  float amax = 0.0f;
  if (HAD) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[i][e] = in16_to_f32<F16>((uint16_t)((uint32_t)raw[i][e >> 1] >> (16 * (e & 1))));
      fwht_in_thread<8>(hv[i]);
    }
    // chunk k of a row sits in lane (row's first lane) + k: D / 8 lanes per row
    if (D == 128) fwht_across_lanes<16>(&hv[0][0], CPT * 8);
    else fwht_across_lanes<8>(&hv[0][0], CPT * 8);
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hv[i][e] = hv[i][e] * hscale;
        amax = __builtin_fmaxf(amax, __builtin_fabsf(hv[i][e]));
      }
  } else {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t u = (uint32_t)raw[i][w];
        amax = __builtin_fmaxf(amax, __builtin_fabsf(in16_to_f32<F16>((uint16_t)(u & 0xffffu))));
        amax = __builtin_fmaxf(amax, __builtin_fabsf(in16_to_f32<F16>((uint16_t)(u >> 16))));
      }
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  const float r = int8_recip(s);
  if (threadIdx.x == 0) scales[bh * nblk + blk] = s;
  int8_t* out = codes + (bh * N + t0) * D;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c >= nchunk) continue;
    uint32_t cb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xv = HAD ? hv[i][e] : in16_to_f32<F16>((uint16_t)((uint32_t)raw[i][e >> 1] >> (16 * (e & 1))));
      cb[e] = int8_code_bits(xv, r);
    }
    *(v2i*)(out + (int64_t)c * 8) = v2i{(int)pack_bytes(cb[0], cb[1], cb[2], cb[3]), (int)pack_bytes(cb[4], cb[5], cb[6], cb[7])};
  }
}

// Blocks too large for registers (over 4096 chunks): amax pass, then an encoding pass whose
// reads hit L2.
template <bool F16, bool SMOOTH>
__global__ __launch_bounds__(256) void quant_int8_twopass(const uint16_t* __restrict__ x, Rows16 xr, int64_t N, int D,
                                                          int T, const float* __restrict__ mean,
                                                          int8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t nblk = (N + T - 1) / T;
  const int64_t blk = blockIdx.x, bh = blockIdx.y;
  const int64_t t0 = blk * T;
  const int rows = (int)((N - t0) < T ? (N - t0) : T);
  const int64_t nchunk = (int64_t)rows * D / 8, cpr = D / 8;
  const uint16_t* base = x + xr.at(bh, t0);   // chunk c: row c / cpr, channels 8 (c % cpr) ..
  auto src = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t r = c / cpr;
    return base + r * xr.sn + (c - r * cpr) * 8;
  };
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < nchunk; c += 256) {
    v4i raw = *(const v4i*)src(c);
    if (SMOOTH) raw = smooth_chunk<F16>(raw, mean + bh * D + (c * 8) % D);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t u = (uint32_t)raw[w];
      amax = __builtin_fmaxf(amax, __builtin_fabsf(in16_to_f32<F16>((uint16_t)(u & 0xffffu))));
      amax = __builtin_fmaxf(amax, __builtin_fabsf(in16_to_f32<F16>((uint16_t)(u >> 16))));
    }
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  const float r = int8_recip(s);
  if (threadIdx.x == 0) scales[bh * nblk + blk] = s;
  int8_t* out = codes + (bh * N + t0) * D;
  for (int64_t c = threadIdx.x; c < nchunk; c += 256) {
    v4i raw = *(const v4i*)src(c);
    if (SMOOTH) raw = smooth_chunk<F16>(raw, mean + bh * D + (c * 8) % D);
    uint32_t cb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cb[e] = int8_code_bits(in16_to_f32<F16>((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1)))), r);
    *(v2i*)(out + c * 8) = v2i{(int)pack_bytes(cb[0], cb[1], cb[2], cb[3]), (int)pack_bytes(cb[4], cb[5], cb[6], cb[7])};
  }
}

// ------------------------------------------------------------------ E4M3 per channel
__global__ void fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <bool F16>
__global__ __launch_bounds__(256) void channel_amax_kernel(const uint16_t* __restrict__ x, Rows16 xr, int64_t BH,
                                                           int64_t N, int D, uint32_t* __restrict__ amax_bits) {
  // thread: (bh, run of 64 tokens, 4 channels); lanes of one wave cover D/4 channel groups of
  // consecutive runs.  Four channels a thread (8-byte loads) give this one-round kernel twice
  // the threads, and so the loads in flight, of eight.
  const int64_t nrun = (N + 63) / 64;
  const int cg = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = gid < BH * nrun * cg;
  const int c4 = (int)(gid % cg);
  const int64_t run = (gid / cg) % nrun, bh = gid / cg / nrun;
  float m[4] = {0, 0, 0, 0};
  auto take = [&](v2i raw) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(in16_to_f32<F16>((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1))))));
  };
  if (valid) {
    const int64_t t0 = run * 64;
    const int rows = (int)((N - t0) < 64 ? (N - t0) : 64);
    const uint16_t* p = x + xr.at(bh, t0) + c4 * 4;
    if (rows == 64) {   // all 64 rows in flight at once
      v2i raw[64];
#pragma unroll
      for (int j = 0; j < 64; ++j) raw[j] = *(const v2i*)(p + (int64_t)j * xr.sn);
#pragma unroll
      for (int j = 0; j < 64; ++j) take(raw[j]);
    } else {
      for (int t = 0; t < rows; ++t) take(*(const v2i*)(p + (int64_t)t * xr.sn));
    }
  }
  // Lanes l, l + cg, l + 2cg, ... hold the same channels of consecutive runs; when the whole
  // wave is valid and in one head, fold them (max is order-free) and let the first cg lanes
  // issue the atomics.
  const int lane = threadIdx.x & 63;
  const int64_t bh0 = __shfl(bh, 0), bh63 = __shfl(bh, 63);
  const bool fold = (cg & (cg - 1)) == 0 && cg < 64 && __all(valid) && bh0 == bh63;
  if (fold) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      for (int sft = cg; sft < 64; sft <<= 1) m[e] = __builtin_fmaxf(m[e], __shfl_xor(m[e], sft));
    if (lane < cg) {
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicMax(amax_bits + bh * D + c4 * 4 + e, __float_as_uint(m[e]));
    }
  } else if (valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicMax(amax_bits + bh * D + c4 * 4 + e, __float_as_uint(m[e]));
  }
}

__global__ void channel_scale_kernel(uint32_t* sc, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) sc[i] = __float_as_uint(__uint_as_float(sc[i]) / 448.0f);
}

template <bool F16>
__global__ __launch_bounds__(256) void fp8_channel_codes_kernel(const uint16_t* __restrict__ x, Rows16 xr, int64_t N,
                                                                int D,
                                                                const float* __restrict__ scales,
                                                                uint8_t* __restrict__ codes_t) {
  // block: (64-token run, bh); LDS tile [D][64] bytes, written transposed, stored as rows.
  __shared__ uint8_t tile[128 * 80];
  constexpr int PITCH = 80;
  const int64_t run = blockIdx.x, bh = blockIdx.y;
  const int64_t t0 = run * 64;
  const int64_t Np = (N + 63) / 64 * 64;
  const int rows = (int)((N - t0) < 64 ? (N - t0) : 64);
  // the channels' reciprocal scales, once per workgroup (saturated at the largest finite fp32,
  // as for INT8)
  __shared__ __attribute__((aligned(16))) float rcp[128];
  for (int c = threadIdx.x; c < D; c += 256) {
    const float s = scales[bh * D + c];
    rcp[c] = s > 0.0f ? __builtin_fminf(1.0f / s, 3.40282347e38f) : 0.0f;
  }
  __syncthreads();
  const int nchunk = 64 * D / 8;
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    const int t = c / (D / 8), c8 = (c % (D / 8)) * 8;
    if (t >= rows) {   // padding tokens: zero codes
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[(c8 + e) * PITCH + t] = 0;
      continue;
    }
    v4i raw = *(const v4i*)(x + xr.at(bh, t0 + t) + c8);
    const v4f r0 = *(const v4f*)&rcp[c8], r1 = *(const v4f*)&rcp[c8 + 4];
    const float r[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = in16_to_f32<F16>((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1))));
      tile[(c8 + e) * PITCH + t] = f32_to_e4m3(v * r[e]);
    }
  }
  __syncthreads();
  // each thread stores 16 bytes of one channel row (rows are Np = 64-multiple bytes long)
  for (int c = threadIdx.x; c < D * 4; c += 256) {
    const int ch = c / 4, t16 = (c % 4) * 16;
    *(v4i*)(codes_t + (bh * D + ch) * Np + t0 + t16) = *(const v4i*)&tile[ch * PITCH + t16];
  }
}

// ------------------------------------------------------------------ FP4 (MX and NV)
// fp32(1 / E4M3(c)) for every positive finite code, from the compiler's correctly rounded
// constant division (the same value a run-time IEEE division gives).
struct RecipTable {
  float v[128];
};
constexpr float e4m3_value(int c) {   // exact: (8 + m) * 2^(e - 10), or m * 2^-9 when e = 0
  const int e = (c >> 3) & 15, m = c & 7;
  float x = e == 0 ? (float)m : (float)(8 + m);
  int sh = e == 0 ? -9 : e - 10;
  for (; sh > 0; --sh) x *= 2.0f;
  for (; sh < 0; ++sh) x *= 0.5f;
  return x;
}
constexpr RecipTable make_recip() {
  RecipTable t{};
  for (int c = 1; c < 128; ++c) t.v[c] = 1.0f / e4m3_value(c);
  return t;
}
__constant__ RecipTable kRecipE4M3 = make_recip();

// Squared error of an NVFP4 candidate scale code over 16 values; codes written to c[0..1].
// x_i = E2M1(v_i * fp32(1/s)), xhat_i = x_i * s (exact), e_i = v_i - xhat_i, summed as the
// balanced index-order tree of e_i * e_i.
__device__ __forceinline__ float nv_candidate(const float* v, uint32_t scode, uint32_t* c) {
  const float s = e4m3_to_f32(scode);
  const float r = kRecipE4M3.v[scode & 127u];
  float se[16];
  c[0] = c[1] = 0u;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t two = f32x2_to_e2m1(v[i] * r, v[i + 1] * r);
    c[i >> 3] |= two << (4 * (i & 7));
    const auto xd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(two, 1.0f, 0);   // both E2M1 values of the byte
    const float e0 = v[i] - xd[0] * s, e1 = v[i + 1] - xd[1] * s;
    se[i] = e0 * e0;
    se[i + 1] = e1 * e1;
  }
#pragma unroll
  for (int w = 1; w < 16; w *= 2)
#pragma unroll
    for (int i = 0; i < 16; i += 2 * w) se[i] = se[i] + se[i + w];
  return se[0];
}

// NVFP4 scale choice for one 16-value group (mode 0 max-scaling, 1 grid search, 2 offsets).
// The grid codes E4M3(amax/6 * g_k) never decrease with k, so only the distinct ones that
// differ from the baseline are evaluated, baseline first and then in ascending order: a
// repeated code repeats the same error and could never be strictly smaller.
__device__ __forceinline__ uint32_t nv_quant16(const float* v, int mode, uint32_t* codes) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  const float smax = amax / 6.0f;
  uint32_t c0 = f32_to_e4m3(smax);
  if (c0 == 0) c0 = 1;
  uint32_t best_c = c0;
  float best = nv_candidate(v, c0, codes);
  if (mode == 1) {
    uint32_t lo = 0, mask = 0;   // grid codes as a bit mask over [lo, lo + 31]
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float g = (float)(0.85 + k * 0.3 / 7.0);
      uint32_t ck = f32_to_e4m3(smax * g);
      if (ck == 0) ck = 1;
      if (k == 0) lo = ck;
      if (ck != c0 && ck - lo < 32) mask |= 1u << (ck - lo);
    }
    // (the grid spans a factor 1.35, at most ~5 E4M3 codes, so the 32-bit window suffices)
    for (uint32_t j = 0; j < 32 && (mask >> j) != 0; ++j) {
      if (((mask >> j) & 1u) == 0) continue;
      const uint32_t ck = lo + j;
      uint32_t cc[2];
      const float sse = nv_candidate(v, ck, cc);
      if (sse < best) { best = sse; best_c = ck; codes[0] = cc[0]; codes[1] = cc[1]; }
    }
  } else if (mode == 2) {
    const int offs[8] = {-2, -1, 1, 2, 3, 4, 5, 6};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int ck = (int)c0 + offs[k];
      if (ck < 1 || ck > 0x7e) continue;
      uint32_t cc[2];
      float sse = nv_candidate(v, (uint32_t)ck, cc);
      if (sse < best) { best = sse; best_c = (uint32_t)ck; codes[0] = cc[0]; codes[1] = cc[1]; }
    }
  }
  return best_c;
}

// MX-FP4 of one 32-value group: returns the E8M0 byte, codes in c[0..3].
__device__ __forceinline__ uint32_t mx_quant32(const float* v, uint32_t* c) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  const int e = mx_exp_e2m1(amax);
#pragma unroll
  for (int w = 0; w < 4; ++w) c[w] = 0u;
#pragma unroll
  for (int i = 0; i < 32; i += 2)
    c[i >> 3] |= f32x2_to_e2m1(__builtin_ldexpf(v[i], -e), __builtin_ldexpf(v[i + 1], -e)) << (4 * (i & 7));
  return (uint32_t)(e + 127);
}

// Along D: one thread per group (32 values for MX, 16 for NV) of one token row.  HAD: the
// row is Hadamard-transformed first; its D / G groups sit in consecutive lanes, and whole
// rows leave together at the bound check, so every lane a stage pairs with is active.
template <bool F16, bool NV, bool SMOOTH, bool HAD = false>
__global__ __launch_bounds__(256) void fp4_rows_kernel(const uint16_t* __restrict__ x, Rows16 xr, int64_t rows,
                                                       int64_t N, int D, int mode, const float* __restrict__ mean,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                       float hscale = 0.0f) {
  constexpr int G = NV ? 16 : 32;
  const int gpr = D / G;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * gpr) return;
  const int64_t row = gid / gpr, bh_ = row / N;   // group gid: row (bh, n), channels G (gid % gpr) ..
  const uint16_t* p = x + xr.at(bh_, row - bh_ * N) + (gid - row * gpr) * G;
  float v[G];
#pragma unroll
  for (int q = 0; q < G / 8; ++q) {
    v4i raw = *(const v4i*)(p + q * 8);
    if (SMOOTH) raw = smooth_chunk<F16>(raw, mean + (gid / gpr / N) * D + (gid % gpr) * G + q * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[q * 8 + e] = in16_to_f32<F16>((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1))));
  }
  if (HAD) {   // D in {64, 128}: gpr = D / G lanes per row; NVFP4's search is VALU-bound
    fwht_in_thread<G>(v);
    if (gpr == 8) fwht_across_lanes<8, NV>(v, G);
    else if (gpr == 4) fwht_across_lanes<4, NV>(v, G);
    else fwht_across_lanes<2, NV>(v, G);
#pragma unroll
    for (int j = 0; j < G; ++j) v[j] = v[j] * hscale;
  }
  if (NV) {
    uint32_t c[2];
    scales[gid] = (uint8_t)nv_quant16(v, mode, c);
    *(v2i*)(codes + gid * 8) = v2i{(int)c[0], (int)c[1]};
  } else {
    uint32_t c[4];
    scales[gid] = (uint8_t)mx_quant32(v, c);
    *(v4i*)(codes + gid * 16) = v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  }
}

// Along tokens (V): block = (64-token run, bh); LDS tile [64][D] of fp32; thread per
// (channel, group of G tokens).  Code rows are channels, Np = N rounded up to 64; scales
// are token-group major [Np/G][D], so consecutive threads write consecutive bytes.
template <bool F16, bool NV>
__global__ __launch_bounds__(256) void fp4_cols_kernel(const uint16_t* __restrict__ x, Rows16 xr, int64_t N, int D,
                                                       int mode, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  constexpr int G = NV ? 16 : 32;
  __shared__ float tile[64][129];
  const int64_t run = blockIdx.x, bh = blockIdx.y;
  const int64_t t0 = run * 64;
  const int64_t Np = (N + 63) / 64 * 64;
  const int rows = (int)((N - t0) < 64 ? (N - t0) : 64);
  for (int c = threadIdx.x; c < 64 * D / 8; c += 256) {
    const int t = c / (D / 8), c8 = (c % (D / 8)) * 8;
    if (t < rows) {
      v4i raw = *(const v4i*)(x + xr.at(bh, t0 + t) + c8);
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[t][c8 + e] = in16_to_f32<F16>((uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1))));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[t][c8 + e] = 0.0f;
    }
  }
  __syncthreads();
  const int groups = 64 / G;
  const int tmax = (int)((Np - t0) < 64 ? (Np - t0) : 64);   // tokens of this run inside Np
  for (int w = threadIdx.x; w < D * groups; w += 256) {
    const int ch = w % D, g = w / D;
    if (g * G >= tmax) continue;
    float v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = tile[g * G + i][ch];
    const int64_t tok = t0 + g * G;
    if (NV) {
      uint32_t c[2];
      scales[(bh * (Np / 16) + tok / 16) * D + ch] = (uint8_t)nv_quant16(v, mode, c);
      *(v2i*)(codes + (bh * D + ch) * (Np / 2) + tok / 2) = v2i{(int)c[0], (int)c[1]};
    } else {
      uint32_t c[4];
      scales[(bh * (Np / 32) + tok / 32) * D + ch] = (uint8_t)mx_quant32(v, c);
      *(v4i*)(codes + (bh * D + ch) * (Np / 2) + tok / 2) = v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    }
  }
}

// ------------------------------------------------------------------ NVFP4 -> MXFP8
// One thread per 32-element group; group gid = row * gpr + j of `rows` code rows with gpr
// groups each.  Along D the scale bytes follow the codes' row order; along tokens
// (rows = bh * D + channel) they are token-group major: [bh][group][D].
__global__ __launch_bounds__(256) void nv_to_mx8_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, int64_t groups, int64_t gpr,
                                                        int D_tok, uint8_t* __restrict__ f8, uint8_t* __restrict__ e8) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // one 32-element group
  if (gid >= groups) return;
  v4i raw = *(const v4i*)(codes + gid * 16);
  int64_t nv0, nv1, mx;   // scale byte indices: NVFP4 groups 2j, 2j+1 and the MXFP8 group j
  if (D_tok == 0) {
    nv0 = gid * 2; nv1 = nv0 + 1; mx = gid;
  } else {
    const int64_t row = gid / gpr, j = gid % gpr, bh = row / D_tok, ch = row % D_tok;
    nv0 = (bh * 2 * gpr + 2 * j) * D_tok + ch; nv1 = nv0 + D_tok; mx = (bh * gpr + j) * D_tok + ch;
  }
  const float s0 = e4m3_to_f32(scales[nv0]), s1 = e4m3_to_f32(scales[nv1]);
  float xh[32];
  float A = 0.0f;
  auto dec2 = [&](int i, decltype(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(0u, 1.0f, 0)) xd) {
    xh[i] = xd[0] * (i < 16 ? s0 : s1);
    xh[i + 1] = xd[1] * (i < 16 ? s0 : s1);
    A = __builtin_fmaxf(A, __builtin_fmaxf(__builtin_fabsf(xh[i]), __builtin_fabsf(xh[i + 1])));
  };
#pragma unroll
  for (int w = 0; w < 4; ++w) {   // one conversion decodes the two E2M1 codes of a byte
    const uint32_t u = (uint32_t)raw[w];
    dec2(8 * w, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 0));
    dec2(8 * w + 2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 1));
    dec2(8 * w + 4, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 2));
    dec2(8 * w + 6, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 3));
  }
  const int E = mx_exp_e4m3(A);
  e8[mx] = (uint8_t)(E + 127);
  v8i out;
#pragma unroll
  for (int w = 0; w < 8; ++w)
    out[w] = (int)f32x4_to_e4m3(__builtin_ldexpf(xh[4 * w], -E), __builtin_ldexpf(xh[4 * w + 1], -E),
                                __builtin_ldexpf(xh[4 * w + 2], -E), __builtin_ldexpf(xh[4 * w + 3], -E));
  *(v8i*)(f8 + gid * 32) = out;
}

// ------------------------------------------------------------------ conversions (verification)
__global__ void convert_kernel(const float* __restrict__ x, int64_t n, int fmt, void* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  switch (fmt) {
    case 0: ((uint16_t*)out)[i] = f32_to_bf16(v); break;
    case 1: ((uint16_t*)out)[i] = f32_to_f16(v); break;
    case 4: ((uint8_t*)out)[i] = f32_to_e4m3(v); break;
    default: ((uint8_t*)out)[i] = (uint8_t)(f32x2_to_e2m1(v, 0.0f) & 15u); break;
  }
}

}  // namespace

float hadamard_scale(int D) { return (float)(1.0 / std::sqrt((double)D)); }

hipError_t launch_quant_int8(const void* x, const Rows16& xr, bool is_f16, int64_t BH, int64_t N, int D, int T,
                             const float* mean, int8_t* codes, float* scales, hipStream_t st, bool hadamard) {
  const int64_t nblk = (N + T - 1) / T;
  if (nblk == 0 || BH == 0) return hipSuccess;
  dim3 g((unsigned)nblk, (unsigned)BH);
  const int64_t chunks = (int64_t)T * D / 8;   // 16-byte chunks of a full block
  const uint16_t* xs = (const uint16_t*)x;
  if (hadamard) {   // D in {64, 128}, chunks <= 4096 (checked at the boundary)
    const float hs = hadamard_scale(D);
    auto goh = [&](auto cpt) {
      constexpr int C = decltype(cpt)::value;
      if (mean) {
        if (is_f16) quant_int8_kernel<true, C, true, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales, hs);
        else quant_int8_kernel<false, C, true, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales, hs);
      } else {
        if (is_f16) quant_int8_kernel<true, C, false, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales, hs);
        else quant_int8_kernel<false, C, false, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales, hs);
      }
    };
    if (chunks <= 256) goh(std::integral_constant<int, 1>{});
    else if (chunks <= 512) goh(std::integral_constant<int, 2>{});
    else if (chunks <= 1024) goh(std::integral_constant<int, 4>{});
    else if (chunks <= 2048) goh(std::integral_constant<int, 8>{});
    else if (chunks <= 4096) goh(std::integral_constant<int, 16>{});
    else return hipErrorNotSupported;
    return hipGetLastError();
  }
  auto go = [&](auto cpt) {
    constexpr int C = decltype(cpt)::value;
    if (mean) {
      if (is_f16) quant_int8_kernel<true, C, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
      else quant_int8_kernel<false, C, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
    } else {
      if (is_f16) quant_int8_kernel<true, C, false><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
      else quant_int8_kernel<false, C, false><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
    }
  };
  if (chunks <= 256) go(std::integral_constant<int, 1>{});
  else if (chunks <= 512) go(std::integral_constant<int, 2>{});
  else if (chunks <= 1024) go(std::integral_constant<int, 4>{});
  else if (chunks <= 2048) go(std::integral_constant<int, 8>{});
  else if (chunks <= 4096) go(std::integral_constant<int, 16>{});
  else if (mean) {
    if (is_f16) quant_int8_twopass<true, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
    else quant_int8_twopass<false, true><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
  } else {
    if (is_f16) quant_int8_twopass<true, false><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
    else quant_int8_twopass<false, false><<<g, 256, 0, st>>>(xs, xr, N, D, T, mean, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_quant_fp8_channel(const void* x, const Rows16& xr, bool is_f16, int64_t BH, int64_t N, int D,
                                    uint8_t* codes_t, float* scales, hipStream_t st) {
  const int64_t ns = BH * D;
  fill_u32<<<(unsigned)((ns + 255) / 256), 256, 0, st>>>((uint32_t*)scales, ns, 0u);
  const int64_t nrun = (N + 63) / 64;
  const int64_t t1 = BH * nrun * (D / 4);
  if (t1 > 0) {
    if (is_f16) channel_amax_kernel<true><<<(unsigned)((t1 + 255) / 256), 256, 0, st>>>((const uint16_t*)x, xr, BH, N, D, (uint32_t*)scales);
    else channel_amax_kernel<false><<<(unsigned)((t1 + 255) / 256), 256, 0, st>>>((const uint16_t*)x, xr, BH, N, D, (uint32_t*)scales);
  }
  channel_scale_kernel<<<(unsigned)((ns + 255) / 256), 256, 0, st>>>((uint32_t*)scales, ns);
  if (nrun > 0) {
    dim3 g((unsigned)nrun, (unsigned)BH);
    if (is_f16) fp8_channel_codes_kernel<true><<<g, 256, 0, st>>>((const uint16_t*)x, xr, N, D, scales, codes_t);
    else fp8_channel_codes_kernel<false><<<g, 256, 0, st>>>((const uint16_t*)x, xr, N, D, scales, codes_t);
  }
  return hipGetLastError();
}

hipError_t launch_quant_fp4(const void* x, const Rows16& xr, bool is_f16, int64_t BH, int64_t N, int D, bool nv,
                            int along_tokens, int mode, const float* mean, uint8_t* codes, uint8_t* scales,
                            hipStream_t st, bool hadamard) {
  const uint16_t* xs = (const uint16_t*)x;
  if (hadamard && along_tokens) return hipErrorNotSupported;
  if (!along_tokens) {
    const int64_t groups = BH * N * (D / (nv ? 16 : 32));
    if (groups == 0) return hipSuccess;
    const unsigned g = (unsigned)((groups + 255) / 256);
    const float hs = hadamard ? hadamard_scale(D) : 0.0f;
    auto go = [&](auto f16c, auto nvc, auto smc) {
      constexpr bool F16 = decltype(f16c)::value, NV = decltype(nvc)::value, SM = decltype(smc)::value;
      if (hadamard) fp4_rows_kernel<F16, NV, SM, true><<<g, 256, 0, st>>>(xs, xr, BH * N, N, D, mode, mean, codes, scales, hs);
      else fp4_rows_kernel<F16, NV, SM, false><<<g, 256, 0, st>>>(xs, xr, BH * N, N, D, mode, mean, codes, scales);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (nv) {
      if (mean) { if (is_f16) go(T_{}, T_{}, T_{}); else go(F_{}, T_{}, T_{}); }
      else { if (is_f16) go(T_{}, T_{}, F_{}); else go(F_{}, T_{}, F_{}); }
    } else {
      if (mean) { if (is_f16) go(T_{}, F_{}, T_{}); else go(F_{}, F_{}, T_{}); }
      else { if (is_f16) go(T_{}, F_{}, F_{}); else go(F_{}, F_{}, F_{}); }
    }
  } else {
    const int64_t nrun = (N + 63) / 64;
    if (nrun == 0 || BH == 0) return hipSuccess;
    dim3 g((unsigned)nrun, (unsigned)BH);
    if (nv) {
      if (is_f16) fp4_cols_kernel<true, true><<<g, 256, 0, st>>>(xs, xr, N, D, mode, codes, scales);
      else fp4_cols_kernel<false, true><<<g, 256, 0, st>>>(xs, xr, N, D, mode, codes, scales);
    } else {
      if (is_f16) fp4_cols_kernel<true, false><<<g, 256, 0, st>>>(xs, xr, N, D, mode, codes, scales);
      else fp4_cols_kernel<false, false><<<g, 256, 0, st>>>(xs, xr, N, D, mode, codes, scales);
    }
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_to_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t len, int D_tok,
                                 uint8_t* f8, uint8_t* e8, hipStream_t st) {
  const int64_t groups = rows * (len / 32);
  if (groups == 0) return hipSuccess;
  nv_to_mx8_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, st>>>(codes, scales, groups, len / 32, D_tok, f8, e8);
  return hipGetLastError();
}

hipError_t launch_convert_f32(const float* x, int64_t n, int fmt, void* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  convert_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, n, fmt, out);
  return hipGetLastError();
}

}  // namespace sage
