// Device helpers for gfx950 (CDNA4): vector types, number-format conversions and
// wave-level reductions used by every kernel of the library.
//
// Formats (OCP Microscaling v1.0 definitions, not printed on the pages):
//   E4M3 "FN": bias 7, max 448, no inf;  E2M1: {0, .5, 1, 1.5, 2, 3, 4, 6};  E8M0: 2^(c-127).
// Conversions use gfx950's convert instructions where their rounding (nearest-even) and
// saturation behaviour is what the quantizers need:
//   v_cvt_pk_bf16_f32        fp32 -> bf16, nearest-even
//   v_cvt_pk_fp8_f32         fp32 -> E4M3, nearest-even; inputs beyond +-464 become NaN, so
//                            every caller clamps to +-448 first (that makes it saturating)
//   v_cvt_scalef32_pk_fp4_f32 fp32 -> E2M1, nearest-even, saturating at +-6 (scale 1.0)
// Bit-exactness of each against the definitions is checked element by element in the GPU
// tests (sage_convert_f32 over every bf16 value).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8us __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

// ---- 16-bit floats -------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 f; __builtin_memcpy(&f, &h, 2); return (float)f;
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x; uint16_t u; __builtin_memcpy(&u, &b, 2); return u;
}
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  _Float16 f = (_Float16)x; uint16_t u; __builtin_memcpy(&u, &f, 2); return u;
}
template <bool IS_F16>
__device__ __forceinline__ float in16_to_f32(uint16_t h) { return IS_F16 ? f16_to_f32(h) : bf16_to_f32(h); }
template <bool IS_F16>
__device__ __forceinline__ uint16_t f32_to_in16(float x) { return IS_F16 ? f32_to_f16(x) : f32_to_bf16(x); }
// two bf16 (RNE) packed in one dword, low half = a: one v_cvt_pk_bf16_f32
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// bf16 pair (1, 1): with v_dot2_f32_bf16 it sums a packed pair into an fp32 accumulator
__device__ __forceinline__ bf16x2_t bf16x2_ones() { return __builtin_bit_cast(bf16x2_t, 0x3F803F80u); }

// ---- E4M3 ----------------------------------------------------------------------------
__device__ __forceinline__ float clamp448(float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f); }
// Four fp32 -> four E4M3 bytes (nearest-even, saturating), byte i = x_i.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
}
__device__ __forceinline__ uint8_t f32_to_e4m3(float a) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), 0.0f, 0u, false) & 0xff);
}
// E4M3 byte -> fp32 value, from the bit fields (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

// ---- E2M1 ----------------------------------------------------------------------------
// Two fp32 -> two E2M1 codes in the low byte (a in bits 0..3, b in 4..7).
__device__ __forceinline__ uint32_t f32x2_to_e2m1(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xffu;
}
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  // magnitude codes 0..7 -> 0, .5, 1, 1.5, 2, 3, 4, 6
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float v = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -v : v;
}

// ---- E8M0 exponents --------------------------------------------------------------------
// Smallest integer e with qmax * 2^e >= a (a > 0 finite), qmax = 6 (E2M1) or 448 (E4M3),
// from the bits of a: with a = 1.f * 2^E, qmax * 2^e >= a  <=>  e >= E - log2(qmax) + log2(1.f).
__device__ __forceinline__ int mx_exp_e2m1(float a) {
  // 6 * 2^e >= a: a = m * 2^E with m in [1, 2).  6 * 2^(E-2) = 1.5 * 2^E >= a iff m <= 1.5.
  if (a == 0.0f) return -127;
  uint32_t u = __float_as_uint(a);
  int E = (int)(u >> 23) - 127;
  uint32_t mant = u & 0x7fffffu;
  if (E == -127) {  // subnormal input: a = 1.f * 2^(-126 - lz) after normalising
    int lz = __clz(mant) - 8;
    E = -126 - lz;
    mant = (mant << lz) & 0x7fffffu;
  }
  int e = (mant <= 0x400000u) ? E - 2 : E - 1;   // m <= 1.5 ?
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// mx_exp_e2m1 through the hardware frexp (subnormal inputs included): a = f * 2^x with f in
// [0.5, 1), so m = 2f and E = x - 1; m <= 1.5 iff f <= 0.75.  Same result, fewer instructions.
__device__ __forceinline__ int mx_exp_e2m1_frexp(float a) {
  int x;
  const float f = __builtin_frexpf(a, &x);
  const int e = f <= 0.75f ? x - 3 : x - 2;
  return a == 0.0f ? -127 : (e < -127 ? -127 : (e > 127 ? 127 : e));
}
__device__ __forceinline__ int mx_exp_e4m3(float a) {
  // 448 * 2^e >= a: 448 = 1.75 * 2^8.  a = m * 2^E: 1.75 * 2^(E-8) >= a iff m <= 1.75.
  if (a == 0.0f) return -127;
  uint32_t u = __float_as_uint(a);
  int E = (int)(u >> 23) - 127;
  uint32_t mant = u & 0x7fffffu;
  if (E == -127) {  // subnormal input: a = 1.f * 2^(-126 - lz) after normalising
    int lz = __clz(mant) - 8;
    E = -126 - lz;
    mant = (mant << lz) & 0x7fffffu;
  }
  int e = (mant <= 0x600000u) ? E - 8 : E - 7;   // m <= 1.75 ?
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ float exp2i(int e) { return __builtin_ldexpf(1.0f, e); }

// ---- INT8 block codes (SageAttention, Technical approach: s = amax / 127, code =
//      clamp(round_half_even(x * (1/s)), -127, 127)) ------------------------------------------
// The reciprocal of a block scale s > 0, saturated at the largest finite fp32 (1 / s overflows
// only for a block whose largest magnitude is below about 3.7e-37; an element 0 then keeps code 0).
__device__ __forceinline__ float int8_recip(float s) {
  return s > 0.0f ? __builtin_fminf(1.0f / s, 3.40282347e38f) : 0.0f;
}
// The INT8 code of fp32(x * r) in the low byte: the product clamped to [-127, 127], then rounded
// to the nearest integer, ties to even, by one fp32 add of 1.5 * 2^23, after which the low bits
// of the sum's mantissa hold that integer in two's complement (|value| < 2^22).  Clamping first
// and rounding after gives the same integer as rounding first.
__device__ __forceinline__ uint32_t int8_code_bits(float x, float r) {
  const float v = __builtin_fminf(__builtin_fmaxf(x * r, -127.0f), 127.0f);
  return __float_as_uint(v + 12582912.0f);
}
__device__ __forceinline__ uint32_t pack_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return (a & 0xffu) | ((b & 0xffu) << 8) | ((c & 0xffu) << 16) | (d << 24);
}

// ---- wave reductions (64 lanes; DPP / swizzle via shuffles) -----------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// ---- lane exchange ----------------------------------------------------------------
// The value of lane ^ m (m in {1, 2, 4, 8}; the lanes of a row of 16 exchange) through DPP:
// xor 1 and xor 2 are quad permutations, xor 8 rotates the row by 8, xor 4 is the half-row
// mirror (i -> 7 - i within 8) followed by the reversed quad (i -> 3 - i within 4).
template <int m>
__device__ __forceinline__ float lane_xor(float v) {
  int x = __builtin_bit_cast(int, v);
  if constexpr (m == 1) x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  else if constexpr (m == 2) x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  else if constexpr (m == 8) x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);  // row_ror:8
  else {
    static_assert(m == 4, "lanes of one row of 16");
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);   // row_half_mirror
    x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true);    // quad_perm [3,2,1,0]
  }
  return __builtin_bit_cast(float, x);
}

}  // namespace sage
