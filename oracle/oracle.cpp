// CPU oracle for the quantized attention forward pass — TEST INFRASTRUCTURE ONLY.
//
// Plain, slow, single-purpose C++17 that restates what the pages compute: K smoothing,
// block quantization (INT8, FP8-E4M3 per channel, MX-FP4, NVFP4 with max-scaling or
// ScaleSearch), Thrift block selection, and a tiled online-softmax attention that mirrors
// the order of the quantize-and-attend steps.  Only tests, the smoke check and the bench's
// CPU-baseline leg may load it.  It shares no code, header, table or helper with the HIP
// library and must never be used as a fallback for it.
//
// Built with g++ -O2 -ffp-contract=off (no fused multiply-add is formed behind our back,
// no fast-math, no SIMD intrinsics), so every fp32 expression below rounds exactly once
// per operation, as written.
//
// Sources (page titles and sections):
//  * "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference Acceleration"
//    (hotpaper.ai summary): Contributions / Key idea / Technical approach — smoothing of
//    K's channel-wise outliers, Q and K in 8 bits, P and V kept at 16 bits.
//  * "Search Your Block Floating Point Scales!" (gist.science explainer), Method ›
//    ScaleSearch — max-scale s = round(amax/6) as an E4M3 scale, search of nearby scales
//    for the minimum block MSE; Method › ScaleSearchAttention — QK^T and PV on FP4 with
//    fp32 accumulation.
//  * SageAttention3 pages (ehanbit.net, dasgeld.co) — microscaled FP4 attention.
//  * "ThriftAttention: Selective Mixed Precision for Long-Context FP4 Attention"
//    (molayo1419.me), ¶1 and ¶3 — ~5% of query-key blocks in high precision, one joint
//    softmax over all blocks.
// Where the pages are silent the reading taken is stated at the function.
//
// Parity pins: every function here is checked in tests/ against brute force, closed
// forms, invariants or a library routine (see tests/test_oracle_*.py).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cfenv>
#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>
#include <limits>

namespace {

// ---------------------------------------------------------------------------------------
// Number formats, written from their definitions (OCP Microscaling v1.0 for E4M3, E2M1,
// E8M0; IEEE-754 binary16; bfloat16 = the top half of binary32).  Encoding rounds the
// exact value to the nearest representable value, ties to the even code, by scaling the
// value onto the integer grid of its binade and calling nearbyint (round-half-even).
// ---------------------------------------------------------------------------------------

// Round a >= 0 (finite) to a binary grid with `mbits` explicit mantissa bits whose
// smallest normal exponent is emin (values below 2^emin use the subnormal quantum
// 2^(emin-mbits)).  Returns the rounded value; it may be 2^(E+1) when rounding carries.
double round_to_grid(double a, int mbits, int emin) {
  if (a == 0.0) return 0.0;
  int k;
  std::frexp(a, &k);          // a = f * 2^k, f in [0.5, 1)
  int E = k - 1;              // a in [2^E, 2^(E+1))
  if (E < emin) E = emin;
  double quantum = std::ldexp(1.0, E - mbits);
  return std::nearbyint(a / quantum) * quantum;   // a/quantum is exact (power-of-two divisor)
}

// Split an on-grid value v > 0 into (biased exponent field, mantissa field).
void grid_fields(double v, int mbits, int emin, int bias, int* efield, int* mfield) {
  int k;
  std::frexp(v, &k);
  int E = k - 1;
  if (E < emin) {  // subnormal
    *efield = 0;
    *mfield = (int)(v / std::ldexp(1.0, emin - mbits));
  } else {
    *efield = E + bias;
    *mfield = (int)(v / std::ldexp(1.0, E - mbits)) - (1 << mbits);
  }
}

double grid_value(int efield, int mfield, int mbits, int emin, int bias) {
  if (efield == 0) return std::ldexp((double)mfield, emin - mbits);
  return std::ldexp(1.0 + (double)mfield / (1 << mbits), efield - bias);
}

// E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; max finite 448 = 0x7E,
// S.1111.111 is NaN, no infinities.  Encoding saturates to +-448 ("satfinite").
uint8_t e4m3_encode(float x) {
  uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  double a = std::fabs((double)x);
  if (std::isnan(x)) return 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  double v = round_to_grid(a, 3, -6);
  if (v > 448.0) v = 448.0;
  if (v == 0.0) return sign;
  int e, m;
  grid_fields(v, 3, -6, 7, &e, &m);
  return (uint8_t)(sign | (e << 3) | m);
}
double e4m3_decode(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  double v = grid_value(e, m, 3, -6, 7);
  return (c & 0x80) ? -v : v;
}

// E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
// No NaN or infinity; encoding saturates to +-6.
uint8_t e2m1_encode(float x) {
  uint8_t sign = std::signbit(x) ? 0x8 : 0x0;
  double a = std::fabs((double)x);
  if (a >= 6.0) return sign | 0x7;
  double v = round_to_grid(a, 1, 0);
  if (v > 6.0) v = 6.0;
  if (v == 0.0) return sign;
  int e, m;
  grid_fields(v, 1, 0, 1, &e, &m);
  return (uint8_t)(sign | (e << 1) | m);
}
double e2m1_decode(uint8_t c) {
  int e = (c >> 1) & 3, m = c & 1;
  double v = grid_value(e, m, 1, 0, 1);
  return (c & 0x8) ? -v : v;
}

// bfloat16: binary32 with the mantissa cut to 7 bits.  Overflow rounds to infinity.
uint16_t bf16_encode(float x) {
  if (std::isnan(x)) return 0x7FC0;
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs((double)x);
  double v = round_to_grid(a, 7, -126);
  if (v >= std::ldexp(1.0, 128)) return sign | 0x7F80;
  if (v == 0.0) return sign;
  int e, m;
  grid_fields(v, 7, -126, 127, &e, &m);
  return (uint16_t)(sign | (e << 7) | m);
}
float bf16_decode(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// IEEE binary16: 5 exponent bits (bias 15), 10 mantissa bits, max 65504.
uint16_t f16_encode(float x) {
  if (std::isnan(x)) return 0x7E00;
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs((double)x);
  double v = round_to_grid(a, 10, -14);
  if (v >= 65536.0) return sign | 0x7C00;
  if (v == 0.0) return sign;
  int e, m;
  grid_fields(v, 10, -14, 15, &e, &m);
  return (uint16_t)(sign | (e << 10) | m);
}
float f16_decode(uint16_t h) {
  int e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
  else v = grid_value(e, m, 10, -14, 15);
  return (float)((h & 0x8000) ? -v : v);
}

// Input tensors arrive as 16-bit patterns: dtype 0 = bfloat16, 1 = float16.
inline float in_value(const uint16_t* p, int64_t i, int dt) { return dt == 0 ? bf16_decode(p[i]) : f16_decode(p[i]); }
inline uint16_t in_encode(float x, int dt) { return dt == 0 ? bf16_encode(x) : f16_encode(x); }

// E8M0 exponent for MX blocks: the smallest integer e with 6 * 2^e >= amax, so that the
// block maximum lands on FP4's largest magnitude or below (max-scaling: the largest item
// fits).  amax = 0 gives -127.  Clamped to the E8M0 range [-127, 127].
int mx_exponent(double amax, double qmax) {
  if (amax == 0.0) return -127;
  int k;
  std::frexp(amax, &k);               // amax < 2^k <= qmax * 2^k: e = k satisfies the bound
  int e = k;
  while (qmax * std::ldexp(1.0, e - 1) >= amax) --e;   // walk down to the smallest that does
  return std::max(-127, std::min(127, e));
}

// ---------------------------------------------------------------------------------------
// Shape helpers: tensors are row-major [B, H, N, D] with D contiguous.
// ---------------------------------------------------------------------------------------
inline int64_t idx4(int64_t b, int64_t h, int64_t n, int64_t d, int64_t H, int64_t N, int64_t D) {
  return ((b * H + h) * N + n) * D + d;
}

template <class F>
void parallel_for(int64_t n, int threads, F f) {
  if (threads <= 1 || n <= 1) { for (int64_t i = 0; i < n; ++i) f(i); return; }
  std::atomic<int64_t> next(0);
  std::vector<std::thread> pool;
  int T = (int)std::min<int64_t>(threads, n);
  for (int t = 0; t < T; ++t)
    pool.emplace_back([&]() { for (int64_t i; (i = next.fetch_add(1)) < n;) f(i); });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// ----- format entry points (elementwise, for the format pins) -----
void orc_bf16_encode(const float* x, uint16_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = bf16_encode(x[i]); }
void orc_f16_encode(const float* x, uint16_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = f16_encode(x[i]); }
void orc_bf16_decode(const uint16_t* x, float* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = bf16_decode(x[i]); }
void orc_f16_decode(const uint16_t* x, float* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = f16_decode(x[i]); }
void orc_e4m3_encode(const float* x, uint8_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = e4m3_encode(x[i]); }
void orc_e4m3_decode(const uint8_t* x, double* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = e4m3_decode(x[i]); }
void orc_e2m1_encode(const float* x, uint8_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = e2m1_encode(x[i]); }
void orc_e2m1_decode(const uint8_t* x, double* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = e2m1_decode(x[i]); }
int orc_mx_exponent(double amax) { return mx_exponent(amax, 6.0); }

// ----- K smoothing -----
// SageAttention removes K's channel-wise outliers before 8-bit quantization ("smoothing
// of K", hotpaper.ai summary, Contributions / Technical approach).  The pages print no
// formula; the reading taken: subtract, per (b, h, channel), the mean of K over all N
// tokens.  Softmax is invariant to adding one constant to a row of scores, and
// q . (k_j - mu) = q . k_j - q . mu shifts every score of row q by the same amount, so
// the attention output is unchanged in exact arithmetic.
// Summation order (fixed so the GPU can reproduce it bit for bit): within each run of 64
// consecutive tokens, an fp32 running sum in token order starting from 0; then an fp32
// running sum of those partials in block order.  mu = S / N in fp32; K_s = the input
// dtype's rounding of fp32(k - mu).
void orc_smooth_k(const uint16_t* k, int dt, int64_t B, int64_t H, int64_t N, int64_t D,
                  float* mean_out, uint16_t* ks_out) {
  const int64_t TB = 64;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t c = 0; c < D; ++c) {
        float total = 0.0f;
        for (int64_t t0 = 0; t0 < N; t0 += TB) {
          float part = 0.0f;
          for (int64_t t = t0; t < std::min(N, t0 + TB); ++t) part = part + in_value(k, idx4(b, h, t, c, H, N, D), dt);
          total = total + part;
        }
        float mu = N > 0 ? total / (float)N : 0.0f;
        mean_out[(b * H + h) * D + c] = mu;
        if (ks_out)
          for (int64_t t = 0; t < N; ++t) {
            int64_t i = idx4(b, h, t, c, H, N, D);
            ks_out[i] = in_encode(in_value(k, i, dt) - mu, dt);
          }
      }
}

// ----- Hadamard incoherence processing ("Search Your Block Floating Point Scales!", Method ›
// ScaleSearchAttention: a Hadamard transform of Q and K, after QuIP#, spreads outliers
// before FP4 quantization).  Reading taken: each row of D channels (D a power of two) is
// multiplied by the normalized Sylvester Hadamard matrix H_D / sqrt(D), which is orthogonal,
// so Q'K'^T = QK^T.  Arithmetic, in fp32: the fast transform's stages h = 1, 2, 4, ..., D/2,
// each replacing every pair (v[j], v[j+h]) with j mod 2h < h by (v[j] + v[j+h],
// v[j] - v[j+h]), then one multiply by fp32(1 / sqrt(D)).  The result equals H_D v exactly
// in real arithmetic; the fp32 roundings are those of this stage order.
void hadamard_row(float* v, int64_t D) {
  for (int64_t h = 1; h < D; h *= 2)
    for (int64_t i = 0; i < D; i += 2 * h)
      for (int64_t j = i; j < i + h; ++j) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
  const float c = (float)(1.0 / std::sqrt((double)D));
  for (int64_t j = 0; j < D; ++j) v[j] = v[j] * c;
}

// Decoded values of a [B, H, N, D] tensor of 16-bit patterns, or of their row transforms.
struct Values {
  const uint16_t* x16;
  int dt;
  std::vector<float> rot;   // non-empty: the Hadamard-transformed rows
  Values(const uint16_t* x, int dtype, int64_t rows, int64_t D, int hadamard) : x16(x), dt(dtype) {
    if (!hadamard) return;
    rot.resize((size_t)(rows * D));
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t c = 0; c < D; ++c) rot[r * D + c] = in_value(x, r * D + c, dt);
      hadamard_row(&rot[r * D], D);
    }
  }
  float operator[](int64_t i) const { return rot.empty() ? in_value(x16, i, dt) : rot[i]; }
};

void orc_hadamard_rows(const uint16_t* x, int dt, int64_t rows, int64_t D, float* out) {
  Values v(x, dt, rows, D, 1);
  std::memcpy(out, v.rot.data(), sizeof(float) * rows * D);
}

// ----- INT8 per-block quantization (SageAttention: Q and K in 8 bits) -----
// A block is `block_tokens` consecutive tokens x all D channels of one (b, h); the last
// block may be short.  Symmetric absmax rule: s = fp32(amax / 127), r = fp32(1 / s),
// code = clamp(round_half_even(fp32(x * r)), -127, 127); an all-zero block has s = 0 and
// codes 0.  r is saturated at the largest finite fp32: 1 / s overflows only when amax is
// below about 3.7e-37, and an infinite r would turn an element 0 into 0 * inf = NaN.  Scales are [B, H, ceil(N / block_tokens)] fp32.  hadamard: quantize the
// transformed rows (hadamard_row) instead of x.
void orc_quant_int8(const uint16_t* x16, int dt, int64_t B, int64_t H, int64_t N, int64_t D,
                    int64_t block_tokens, int hadamard, int8_t* codes, float* scales) {
  const Values x(x16, dt, B * H * N, D, hadamard);
  int64_t nblk = (N + block_tokens - 1) / block_tokens;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t blk = 0; blk < nblk; ++blk) {
        int64_t t0 = blk * block_tokens, t1 = std::min(N, t0 + block_tokens);
        float amax = 0.0f;
        for (int64_t t = t0; t < t1; ++t)
          for (int64_t c = 0; c < D; ++c) amax = std::max(amax, std::fabs(x[idx4(b, h, t, c, H, N, D)]));
        float s = amax / 127.0f;
        scales[(b * H + h) * nblk + blk] = s;
        float r = s > 0.0f ? std::min(1.0f / s, std::numeric_limits<float>::max()) : 0.0f;
        for (int64_t t = t0; t < t1; ++t)
          for (int64_t c = 0; c < D; ++c) {
            int64_t i = idx4(b, h, t, c, H, N, D);
            float q = std::nearbyint(x[i] * r);
            codes[i] = (int8_t)std::max(-127.0f, std::min(127.0f, q));
          }
      }
}

// ----- FP8 E4M3 per-channel quantization of V -----
// Per (b, h, channel): s_c = fp32(amax_c / 448) over all N tokens, r_c = fp32(1 / s_c)
// (saturated at the largest finite fp32, as for INT8), code = E4M3(fp32(v * r_c)).  Codes are written channel-major, [B, H, D, Np] with Np = N
// rounded up to 64 and zero codes in the padding (tokens contiguous: the contraction axis of
// P.V), scales [B, H, D] fp32.
void orc_quant_fp8_channel(const uint16_t* v, int dt, int64_t B, int64_t H, int64_t N, int64_t D,
                           uint8_t* codes_t, float* scales) {
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t c = 0; c < D; ++c) {
        float amax = 0.0f;
        for (int64_t t = 0; t < N; ++t) amax = std::max(amax, std::fabs(in_value(v, idx4(b, h, t, c, H, N, D), dt)));
        float s = amax / 448.0f;
        scales[(b * H + h) * D + c] = s;
        float r = s > 0.0f ? std::min(1.0f / s, std::numeric_limits<float>::max()) : 0.0f;   // saturated as for INT8
        const int64_t Np = (N + 63) / 64 * 64;
        for (int64_t t = 0; t < Np; ++t)
          codes_t[((b * H + h) * D + c) * Np + t] = t < N ? e4m3_encode(in_value(v, idx4(b, h, t, c, H, N, D), dt) * r) : 0;
      }
}

// Scale byte of (head bh, layout row r, group g) for `groups` groups per row: row major
// along D (axis 0); group major along tokens (axis 1, rows = channels).
inline int64_t scale_index(int64_t bh, int64_t r, int64_t g, int64_t rows, int64_t groups, int axis) {
  return axis == 0 ? (bh * rows + r) * groups + g : (bh * groups + g) * rows + r;
}

// ----- MX-FP4 (E2M1 elements, one E8M0 scale per 32 elements) -----
// Used by SageAttention3's microscaled FP4 attention.  The block runs along the
// contraction axis: axis 0 = along D (Q, K), axis 1 = along tokens (V).
// Scale: e = smallest integer with 6 * 2^e >= amax (max-scaling: the largest element
// fits); element code = E2M1(x * 2^-e), exact scaling so the only rounding is E2M1's.
// Packing: two codes per byte along the block axis, even element in the low nibble.
// axis 0: codes [B,H,N,D/2], scales [B,H,N,D/32].
// axis 1: codes [B,H,D,Np/2] with Np = N rounded up to 64 (the padding tokens are zeros),
//         scales [B,H,Np/32,D] (token block major: the scales of 64 consecutive tokens
//         are 2*D consecutive bytes).
void orc_quant_mxfp4(const uint16_t* x16, int dt, int64_t B, int64_t H, int64_t N, int64_t D, int axis,
                     int hadamard, uint8_t* codes, uint8_t* scales) {
  const Values x(x16, dt, B * H * N, D, hadamard && axis == 0);
  const int64_t G = 32;
  int64_t Np = (N + 63) / 64 * 64;
  int64_t rows = axis == 0 ? N : D;        // rows of the output layout
  int64_t len = axis == 0 ? D : Np;        // elements along the block axis
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t r = 0; r < rows; ++r)
        for (int64_t g0 = 0; g0 < len; g0 += G) {
          float vals[32];
          double amax = 0.0;
          for (int64_t j = 0; j < G; ++j) {
            int64_t t = axis == 0 ? r : g0 + j, c = axis == 0 ? g0 + j : r;
            vals[j] = t < N ? x[idx4(b, h, t, c, H, N, D)] : 0.0f;
            amax = std::max(amax, std::fabs((double)vals[j]));
          }
          int e = mx_exponent(amax, 6.0);
          scales[scale_index(b * H + h, r, g0 / G, rows, len / G, axis)] = (uint8_t)(e + 127);
          for (int64_t j = 0; j < G; j += 2) {
            uint8_t lo = e2m1_encode((float)std::ldexp((double)vals[j], -e));
            uint8_t hi = e2m1_encode((float)std::ldexp((double)vals[j + 1], -e));
            codes[((b * H + h) * rows + r) * (len / 2) + (g0 + j) / 2] = (uint8_t)(lo | (hi << 4));
          }
        }
}

// ----- NVFP4 block quantization: E2M1 elements, one UE4M3 scale per 16 elements -----
// Max-scaling ("Search Your Block Floating Point Scales!", Method › ScaleSearch): the
// default scale is amax / 6 rounded to the E4M3 scale format.  Reading taken: rounding is
// to nearest-even with saturation, and a scale that rounds to zero is raised to the
// smallest positive code 0x01 (2^-9).  Elements are x * fp32(1 / s) rounded to E2M1 with
// saturation at +-6 (the rounded scale may put the block max slightly above 6 * s).
//
// ScaleSearch (same section): instead of keeping that one scale, try nearby scales and
// keep the one with the smallest squared error over the block.
//   mode 0: max-scaling only.
//   mode 1: candidate grid of 8 multipliers g_k = 0.85 + k * 0.3 / 7 (k = 0..7, computed
//           in fp64, rounded to fp32) applied to fp32(amax / 6), each rounded to E4M3;
//           the max-scaling scale is evaluated first so it is always a candidate.
//   mode 2: the page's own parameterisation: integer offsets f in [-2, 6] added to the
//           E4M3 bit pattern of the max-scaling scale (f = 0 evaluated first, then
//           -2, -1, 1, ..., 6; offsets that leave the codes 0x01..0x7E are skipped).
// Squared error per candidate: e_i = fp32(x_i - xhat_i), se_i = fp32(e_i * e_i), summed
// in fp32 as a balanced pairwise tree in index order ((se0+se1)+(se2+se3))+...; the
// first candidate with a strictly smaller sum wins (ties keep the earlier candidate).
// axis 0: codes [B,H,N,D/2], scales [B,H,N,D/16];  axis 1: codes [B,H,D,Np/2], scales
// [B,H,Np/16,D] with Np = N rounded up to 64.
float nv_block_sse(const float* x, float s, uint8_t* codes_out) {
  float r = 1.0f / s;
  float se[16];
  for (int i = 0; i < 16; ++i) {
    uint8_t c = e2m1_encode(x[i] * r);
    if (codes_out) codes_out[i] = c;
    float xhat = (float)e2m1_decode(c) * s;     // exact: 2 significant bits times 4
    float e = x[i] - xhat;
    se[i] = e * e;
  }
  for (int w = 1; w < 16; w *= 2)               // pairwise tree, index order
    for (int i = 0; i < 16; i += 2 * w) se[i] = se[i] + se[i + w];
  return se[0];
}

// One 16-element block's UE4M3 scale under scale mode `mode` (0, 1, 2 as above); writes the
// block's E2M1 codes and the index of the winning candidate in the full list (0: max-scale).
uint8_t nv_choose_scale(const float* vals, int mode, uint8_t* codes, int* chosen) {
  static const double* grid = [] {
    static double g[8];
    for (int k = 0; k < 8; ++k) g[k] = (double)(float)(0.85 + k * 0.3 / 7.0);
    return g;
  }();
  float amax = 0.0f;
  for (int j = 0; j < 16; ++j) amax = std::max(amax, std::fabs(vals[j]));
  float smax = amax / 6.0f;
  // cand[i] < 0 marks a candidate that does not exist (offset outside 0x01..0x7E);
  // the reported index is the position in the full list either way.
  std::vector<int> cand;
  uint8_t c0 = e4m3_encode(smax);
  if (c0 == 0) c0 = 0x01;
  cand.push_back(c0);
  if (mode == 1) {
    for (int k = 0; k < 8; ++k) {
      uint8_t ck = e4m3_encode((float)(smax * (float)grid[k]));
      if (ck == 0) ck = 0x01;
      cand.push_back(ck);
    }
  } else if (mode == 2) {
    const int offs[8] = {-2, -1, 1, 2, 3, 4, 5, 6};
    for (int f : offs) {
      int ck = (int)c0 + f;
      cand.push_back(ck >= 0x01 && ck <= 0x7E ? ck : -1);
    }
  }
  uint8_t best_c = (uint8_t)cand[0];
  float best = nv_block_sse(vals, (float)e4m3_decode(best_c), codes);
  int best_i = 0;
  for (size_t i = 1; i < cand.size(); ++i) {
    if (cand[i] < 0) continue;
    uint8_t cc[16];
    float sse = nv_block_sse(vals, (float)e4m3_decode((uint8_t)cand[i]), cc);
    if (sse < best) { best = sse; best_c = (uint8_t)cand[i]; best_i = (int)i; std::memcpy(codes, cc, 16); }
  }
  if (chosen) *chosen = best_i;
  return best_c;
}

void orc_quant_nvfp4(const uint16_t* x16, int dt, int64_t B, int64_t H, int64_t N, int64_t D, int axis, int mode,
                     int hadamard, uint8_t* codes, uint8_t* scales,
                     uint8_t* chosen /* nullable: index of winning candidate */) {
  const Values x(x16, dt, B * H * N, D, hadamard && axis == 0);
  const int64_t G = 16;
  int64_t Np = (N + 63) / 64 * 64;
  int64_t rows = axis == 0 ? N : D;
  int64_t len = axis == 0 ? D : Np;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t r = 0; r < rows; ++r)
        for (int64_t g0 = 0; g0 < len; g0 += G) {
          float vals[16];
          for (int64_t j = 0; j < G; ++j) {
            int64_t t = axis == 0 ? r : g0 + j, c = axis == 0 ? g0 + j : r;
            vals[j] = t < N ? x[idx4(b, h, t, c, H, N, D)] : 0.0f;
          }
          uint8_t best_codes[16];
          int best_i = 0;
          const uint8_t best_c = nv_choose_scale(vals, mode, best_codes, &best_i);
          int64_t srow = ((b * H + h) * rows + r), si = scale_index(b * H + h, r, g0 / G, rows, len / G, axis);
          scales[si] = best_c;
          if (chosen) chosen[si] = (uint8_t)best_i;
          for (int j = 0; j < G; j += 2)
            codes[srow * (len / 2) + (g0 + j) / 2] = (uint8_t)(best_codes[j] | (best_codes[j + 1] << 4));
        }
}

// ----- NVFP4 -> FP8 (E4M3 elements, one E8M0 scale per 32 elements) -----
// The target MFMA has no NVFP4 operand form, so NVFP4 operands are dequantized to FP8
// before the matrix product.  For each 32-element run along the block axis:
// xhat_i = E2M1 value * UE4M3 scale (exact in fp32); A = max |xhat|; E = smallest integer
// with 448 * 2^E >= A (A = 0 gives -127); f_i = E4M3(xhat_i * 2^-E).  Input layouts are
// orc_quant_nvfp4's for the same axis; outputs: codes one byte per element ([B,H,N,D] or
// [B,H,D,Np]) and E8M0 scales laid out like MX-FP4's ([B,H,N,D/32] or [B,H,Np/32,D]).
void orc_nvfp4_to_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t B, int64_t H, int64_t N, int64_t D,
                        int axis, uint8_t* f8, uint8_t* e8m0) {
  const int64_t Np = (N + 63) / 64 * 64;
  const int64_t rows = axis == 0 ? N : D, len = axis == 0 ? D : Np;
  for (int64_t bh = 0; bh < B * H; ++bh)
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t g0 = 0; g0 < len; g0 += 32) {
        double xh[32], A = 0.0;
        for (int j = 0; j < 32; ++j) {
          int64_t i = g0 + j;
          uint8_t byte = codes[(bh * rows + r) * (len / 2) + i / 2];
          uint8_t c = (i & 1) ? (byte >> 4) : (byte & 15);
          xh[j] = e2m1_decode(c) * e4m3_decode(scales[scale_index(bh, r, i / 16, rows, len / 16, axis)]);
          A = std::max(A, std::fabs(xh[j]));
        }
        int E = mx_exponent(A, 448.0);
        e8m0[scale_index(bh, r, g0 / 32, rows, len / 32, axis)] = (uint8_t)(E + 127);
        for (int j = 0; j < 32; ++j) f8[(bh * rows + r) * len + g0 + j] = e4m3_encode((float)std::ldexp(xh[j], -E));
      }
}

// ----- Thrift block selection ("ThriftAttention", ¶1 and ¶3) -----
// The page runs the most influential ~5% of query-key blocks in high precision but does
// not print its selection heuristic.  Reading taken: score each (Q block, K block) pair
// by the dot product of the blocks' mean vectors.
//   qbar = bf16(fp32(S / q_block)), S = fp32 running sum over the block's rows in token
//   order (a short last block divides by its own length); kbar likewise from K_s.
//   score = fp32 fused-multiply-add chain over channels, starting from 0 (products of two
//   bf16 values are exact in fp32).
// Per (b, q-head), over the pairs a causal mask leaves valid (some key <= some query:
// k_block * kb <= q_block * qb + q_block - 1), select the n_sel = min(n_valid,
// ceil(frac * n_valid)) highest scores; ties go to the lower linear index qb * nKB + kb.
// mask [B, Hq, nQB, nKB] gets 1 for selected pairs, 0 elsewhere.  GQA: q-head h reads
// kv-head h / (Hq / Hkv).
void orc_thrift_select(const uint16_t* q, const uint16_t* ks, int dt, int64_t B, int64_t Hq, int64_t Hkv,
                       int64_t N, int64_t D, int64_t q_block, int64_t k_block, double frac, int causal,
                       uint8_t* mask, float* scores_out /* nullable [B,Hq,nQB,nKB] */) {
  int64_t nQB = (N + q_block - 1) / q_block, nKB = (N + k_block - 1) / k_block;
  auto block_mean = [&](const uint16_t* x, int64_t H, int64_t b, int64_t h, int64_t t0, int64_t t1, float* out) {
    for (int64_t c = 0; c < D; ++c) {
      float s = 0.0f;
      for (int64_t t = t0; t < t1; ++t) s = s + in_value(x, idx4(b, h, t, c, H, N, D), dt);
      out[c] = bf16_decode(bf16_encode(s / (float)(t1 - t0)));
    }
  };
  std::vector<float> qbar(nQB * D), kbar(nKB * D), score(nQB * nKB);
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < Hq; ++h) {
      int64_t g = h / (Hq / Hkv);
      for (int64_t qb = 0; qb < nQB; ++qb) block_mean(q, Hq, b, h, qb * q_block, std::min(N, (qb + 1) * q_block), &qbar[qb * D]);
      for (int64_t kb = 0; kb < nKB; ++kb) block_mean(ks, Hkv, b, g, kb * k_block, std::min(N, (kb + 1) * k_block), &kbar[kb * D]);
      std::vector<int64_t> valid;
      for (int64_t qb = 0; qb < nQB; ++qb)
        for (int64_t kb = 0; kb < nKB; ++kb) {
          float s = 0.0f;
          for (int64_t c = 0; c < D; ++c) s = std::fma(qbar[qb * D + c], kbar[kb * D + c], s);
          score[qb * nKB + kb] = s;
          bool ok = !causal || k_block * kb <= q_block * qb + q_block - 1;
          if (ok) valid.push_back(qb * nKB + kb);
        }
      int64_t n_valid = (int64_t)valid.size();
      int64_t n_sel = std::min(n_valid, (int64_t)std::ceil(frac * (double)n_valid));
      std::stable_sort(valid.begin(), valid.end(), [&](int64_t a, int64_t c) { return score[a] > score[c]; });
      uint8_t* m = mask + (b * Hq + h) * nQB * nKB;
      std::memset(m, 0, nQB * nKB);
      for (int64_t i = 0; i < n_sel; ++i) m[valid[i]] = 1;
      if (scores_out) std::memcpy(scores_out + (b * Hq + h) * nQB * nKB, score.data(), sizeof(float) * nQB * nKB);
    }
}

// ----- Tiled quantized attention -----
// softmax(S) V with S = Q K^T * sm_scale computed from low-bit operands, evaluated the
// FlashAttention-2 way: per Q block of q_block rows, K/V tiles of k_block keys in
// ascending order, a running row max m and running denominator l in high precision, the
// output rescaled by exp(m_old - m_new) whenever the max grows.  The pages fix the
// ingredients (8-bit or FP4 QK^T with block-scale dequantization, one joint softmax over
// all tiles, P.V on 16-bit/FP8/FP4 operands with fp32 accumulation); the tile order is
// fixed here because quantizing P depends on the running max.
//
// Per tile: S (fp64, from exact dot products times the block scales and sm_scale;
// masked causal entries -inf) -> m' = max(m, rowmax S) -> Ptilde = fp32(exp(S - m'))
// -> l = l * exp(m - m') + sum Ptilde (the denominator uses the unquantized Ptilde) ->
// Phat = quantize_P(Ptilde) -> O = O * exp(m - m') + Phat . Vhat (fp64).  End of row:
// O / l, times the V channel scale (FP8 V) and / 448 (FP8 P).
enum { QK_INT8 = 0, QK_MXFP4 = 1, QK_MXFP8 = 2, QK_HI = 3 };
enum { P_BF16 = 0, P_E4M3 = 1, P_MXFP4 = 2, P_NVFP4_MXFP8 = 3, P_EXACT = 4 };
enum { V_HI = 0, V_E4M3 = 1, V_MXFP4 = 2, V_MXFP8 = 3 };

struct orc_attn_args {
  int64_t B, Hq, Hkv, N, D;
  int64_t q_block, k_block;
  int32_t causal;
  int32_t qk_fmt, p_fmt, v_fmt;
  double sm_scale;
  // QK_INT8: codes [B,H,N,D] int8 + fp32 scales [B,H,ceil(N/q_block or k_block)]
  const int8_t* q_i8; const float* q_s; const int8_t* k_i8; const float* k_s;
  // QK_MXFP4: packed E2M1 [B,H,N,D/2] + E8M0 [B,H,N,D/32];  QK_MXFP8: E4M3 [B,H,N,D] + E8M0 [B,H,N,D/32]
  const uint8_t* q_lp; const uint8_t* q_e8; const uint8_t* k_lp; const uint8_t* k_e8;
  // high-precision Q / K_s (16-bit patterns, dtype hi_dt): QK_HI tiles and Thrift-selected tiles
  const uint16_t* q_hi; const uint16_t* k_hi; int32_t hi_dt;
  const uint8_t* thrift_mask;  // nullable [B,Hq,nQB,nKB]; 1 = this tile uses q_hi/k_hi
  // V: V_HI 16-bit [B,Hkv,N,D] (v_dt; rounded to bf16 before use); V_E4M3 codes [B,Hkv,D,Np] + fp32 [B,Hkv,D];
  //    V_MXFP4 packed [B,Hkv,D,Np/2] + E8M0 [B,Hkv,Np/32,D]; V_MXFP8 E4M3 [B,Hkv,D,Np] + E8M0 [B,Hkv,Np/32,D]
  const uint16_t* v_hi; int32_t v_dt;
  const uint8_t* v_lp; const float* v_s; const uint8_t* v_e8;
  // work subset: flat (b*Hq + h) in [bh_begin, bh_end), Q blocks [qb_begin, qb_end)
  int64_t bh_begin, bh_end, qb_begin, qb_end;
  int32_t threads;
  double* out;   // [B,Hq,N,D]; only rows of the subset are written
  double* lse;   // nullable [B,Hq,N]: m + log(l) in natural-log units
  int32_t p_mode;  // P_NVFP4_MXFP8: the 16-key blocks' scale rule (0 max-scaling, 1 or 2 ScaleSearch)
};

namespace {

double mx_p_value(double p, int e) {  // E2M1 at exponent e (exact scaling)
  return e2m1_decode(e2m1_encode((float)std::ldexp(p, -e))) * std::ldexp(1.0, e);
}

// Quantize one row of Ptilde over a tile (n valid keys; invalid keys are 0) in place.
void quantize_p_row(double* p, int64_t n, int fmt, int p_mode) {
  if (fmt == P_EXACT) return;
  if (fmt == P_BF16) { for (int64_t j = 0; j < n; ++j) p[j] = bf16_decode(bf16_encode((float)p[j])); return; }
  if (fmt == P_E4M3) { for (int64_t j = 0; j < n; ++j) p[j] = e4m3_decode(e4m3_encode((float)(p[j] * 448.0))); return; }
  if (fmt == P_MXFP4) {   // one E8M0 scale per 32 consecutive keys of the tile
    for (int64_t g0 = 0; g0 < n; g0 += 32) {
      double amax = 0.0;
      for (int64_t j = g0; j < std::min(n, g0 + 32); ++j) amax = std::max(amax, std::fabs(p[j]));
      int e = mx_exponent(amax, 6.0);
      for (int64_t j = g0; j < std::min(n, g0 + 32); ++j) p[j] = mx_p_value(p[j], e);
    }
    return;
  }
  if (fmt == P_NVFP4_MXFP8) {  // NVFP4 per 16 keys (scale by p_mode), then FP8 with E8M0 per 32 keys
    for (int64_t g0 = 0; g0 < n; g0 += 16) {
      float vals[16];
      for (int64_t j = 0; j < 16; ++j) vals[j] = g0 + j < n ? (float)p[g0 + j] : 0.0f;
      uint8_t codes[16];
      const float s = (float)e4m3_decode(nv_choose_scale(vals, p_mode, codes, nullptr));
      for (int64_t j = g0; j < std::min(n, g0 + 16); ++j) p[j] = e2m1_decode(codes[j - g0]) * s;
    }
    for (int64_t g0 = 0; g0 < n; g0 += 32) {
      double A = 0.0;
      for (int64_t j = g0; j < std::min(n, g0 + 32); ++j) A = std::max(A, std::fabs(p[j]));
      int E = mx_exponent(A, 448.0);
      for (int64_t j = g0; j < std::min(n, g0 + 32); ++j)
        p[j] = e4m3_decode(e4m3_encode((float)std::ldexp(p[j], -E))) * std::ldexp(1.0, E);
    }
    return;
  }
}

inline uint8_t nib(const uint8_t* base, int64_t i) { uint8_t b = base[i / 2]; return (i & 1) ? (b >> 4) : (b & 15); }

}  // namespace

void orc_attention(const orc_attn_args* a) {
  const int64_t B = a->B, Hq = a->Hq, Hkv = a->Hkv, N = a->N, D = a->D, QB = a->q_block, KB = a->k_block;
  const int64_t nQB = (N + QB - 1) / QB, nKB = (N + KB - 1) / KB;
  const int64_t Np = (N + 63) / 64 * 64;   // padded token count of channel-major V layouts
  const double NEG_INF = -std::numeric_limits<double>::infinity();
  const bool need_hi = a->qk_fmt == QK_HI || a->thrift_mask != nullptr;
  (void)B;

  for (int64_t bh = a->bh_begin; bh < a->bh_end; ++bh) {
    const int64_t b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
    // Exact values of this head's operands, decoded once.  MX formats keep the element
    // value and the per-32 block exponent apart, as the scaled product uses them.
    std::vector<double> qd, kd, qhi, khi, vhat(N * D);
    std::vector<int> qe, ke;
    if (a->qk_fmt == QK_MXFP4 || a->qk_fmt == QK_MXFP8) {
      qd.resize(N * D); kd.resize(N * D); qe.resize(N * (D / 32)); ke.resize(N * (D / 32));
      for (int64_t t = 0; t < N; ++t) {
        for (int64_t c = 0; c < D; ++c) {
          if (a->qk_fmt == QK_MXFP4) {
            qd[t * D + c] = e2m1_decode(nib(a->q_lp + ((b * Hq + h) * N + t) * (D / 2), c));
            kd[t * D + c] = e2m1_decode(nib(a->k_lp + ((b * Hkv + g) * N + t) * (D / 2), c));
          } else {
            qd[t * D + c] = e4m3_decode(a->q_lp[idx4(b, h, t, c, Hq, N, D)]);
            kd[t * D + c] = e4m3_decode(a->k_lp[idx4(b, g, t, c, Hkv, N, D)]);
          }
        }
        for (int64_t c0 = 0; c0 < D / 32; ++c0) {
          qe[t * (D / 32) + c0] = (int)a->q_e8[((b * Hq + h) * N + t) * (D / 32) + c0] - 127;
          ke[t * (D / 32) + c0] = (int)a->k_e8[((b * Hkv + g) * N + t) * (D / 32) + c0] - 127;
        }
      }
    }
    if (need_hi) {   // 16-bit Q and K_s, used as bf16 values by high-precision tiles
      qhi.resize(N * D); khi.resize(N * D);
      for (int64_t t = 0; t < N; ++t)
        for (int64_t c = 0; c < D; ++c) {
          qhi[t * D + c] = bf16_decode(bf16_encode(in_value(a->q_hi, idx4(b, h, t, c, Hq, N, D), a->hi_dt)));
          khi[t * D + c] = bf16_decode(bf16_encode(in_value(a->k_hi, idx4(b, g, t, c, Hkv, N, D), a->hi_dt)));
        }
    }
    for (int64_t t = 0; t < N; ++t)
      for (int64_t c = 0; c < D; ++c) {
        double v;
        switch (a->v_fmt) {
          case V_HI: v = bf16_decode(bf16_encode(in_value(a->v_hi, idx4(b, g, t, c, Hkv, N, D), a->v_dt))); break;
          case V_E4M3: v = e4m3_decode(a->v_lp[((b * Hkv + g) * D + c) * Np + t]); break;
          case V_MXFP4: {
            int e = (int)a->v_e8[((b * Hkv + g) * (Np / 32) + t / 32) * D + c] - 127;
            v = e2m1_decode(nib(a->v_lp + ((b * Hkv + g) * D + c) * (Np / 2), t)) * std::ldexp(1.0, e);
            break;
          }
          default: {
            int e = (int)a->v_e8[((b * Hkv + g) * (Np / 32) + t / 32) * D + c] - 127;
            v = e4m3_decode(a->v_lp[((b * Hkv + g) * D + c) * Np + t]) * std::ldexp(1.0, e);
          }
        }
        vhat[t * D + c] = v;   // V_E4M3: the code value; its channel scale is applied at the end
      }

    // S[i][j] * (1 / sm_scale), from exact products of the low-bit operands and the block scales.
    auto raw_score = [&](int64_t i, int64_t j, bool hi_tile) -> double {
      if (hi_tile || a->qk_fmt == QK_HI) {
        double s = 0.0;
        for (int64_t c = 0; c < D; ++c) s += qhi[i * D + c] * khi[j * D + c];
        return s;
      }
      if (a->qk_fmt == QK_INT8) {
        int64_t acc = 0;   // exact integer dot product
        const int8_t* qi = a->q_i8 + idx4(b, h, i, 0, Hq, N, D);
        const int8_t* kj = a->k_i8 + idx4(b, g, j, 0, Hkv, N, D);
        for (int64_t c = 0; c < D; ++c) acc += (int64_t)qi[c] * (int64_t)kj[c];
        return (double)acc * (double)a->q_s[(b * Hq + h) * nQB + i / QB] * (double)a->k_s[(b * Hkv + g) * nKB + j / KB];
      }
      double s = 0.0;   // MX: sum over 32-element blocks of 2^(eq + ek) * sum(dec q * dec k)
      for (int64_t c0 = 0; c0 < D; c0 += 32) {
        double part = 0.0;
        for (int64_t c = c0; c < c0 + 32; ++c) part += qd[i * D + c] * kd[j * D + c];
        s += part * std::ldexp(1.0, qe[i * (D / 32) + c0 / 32] + ke[j * (D / 32) + c0 / 32]);
      }
      return s;
    };

    parallel_for(a->qb_end - a->qb_begin, a->threads, [&](int64_t w) {
      const int64_t qb = a->qb_begin + w;
      const int64_t r0 = qb * QB, r1 = std::min(N, r0 + QB), R = r1 - r0;
      if (R <= 0) return;
      std::vector<double> m(R, NEG_INF), l(R, 0.0), O(R * D, 0.0), S(KB), P(KB), acc(D);
      for (int64_t kb = 0; kb < nKB; ++kb) {
        const int64_t c0 = kb * KB, c1 = std::min(N, c0 + KB), C = c1 - c0;
        if (a->causal && c0 > r1 - 1) break;    // this tile and all later ones are masked
        const bool hi_tile = a->thrift_mask && a->thrift_mask[((b * Hq + h) * nQB + qb) * nKB + kb];
        for (int64_t ii = 0; ii < R; ++ii) {
          const int64_t i = r0 + ii;
          double rowmax = NEG_INF;
          for (int64_t jj = 0; jj < C; ++jj) {
            const int64_t j = c0 + jj;
            S[jj] = (a->causal && j > i) ? NEG_INF : raw_score(i, j, hi_tile) * a->sm_scale;
            rowmax = std::max(rowmax, S[jj]);
          }
          const double mnew = std::max(m[ii], rowmax);
          if (mnew == NEG_INF) continue;           // no valid key for this row yet
          const double alpha = m[ii] == NEG_INF ? 0.0 : std::exp(m[ii] - mnew);
          double psum = 0.0;
          for (int64_t jj = 0; jj < C; ++jj) {
            P[jj] = S[jj] == NEG_INF ? 0.0 : std::exp(S[jj] - mnew);
            if (a->p_fmt != P_EXACT) P[jj] = (double)(float)P[jj];   // the kernel holds Ptilde in fp32
            psum += P[jj];
          }
          l[ii] = l[ii] * alpha + psum;
          quantize_p_row(P.data(), C, a->p_fmt, a->p_mode);
          std::fill(acc.begin(), acc.end(), 0.0);
          for (int64_t jj = 0; jj < C; ++jj) {
            if (P[jj] == 0.0) continue;
            const double* vr = &vhat[(c0 + jj) * D];
            for (int64_t c = 0; c < D; ++c) acc[c] += P[jj] * vr[c];
          }
          for (int64_t c = 0; c < D; ++c) O[ii * D + c] = O[ii * D + c] * alpha + acc[c];
          m[ii] = mnew;
        }
      }
      for (int64_t ii = 0; ii < R; ++ii) {
        for (int64_t c = 0; c < D; ++c) {
          double o = O[ii * D + c] / l[ii];
          if (a->v_fmt == V_E4M3) o *= (double)a->v_s[(b * Hkv + g) * D + c];
          if (a->p_fmt == P_E4M3) o /= 448.0;
          a->out[idx4(b, h, r0 + ii, c, Hq, N, D)] = o;
        }
        if (a->lse) a->lse[(b * Hq + h) * N + r0 + ii] = m[ii] + std::log(l[ii]);
      }
    });
  }
}

// ----- fp64 reference attention: the textbook definition, full N x N score matrix -----
// O = softmax(Q K^T * sm_scale) V over fp64 copies of the inputs (q, k, v given as
// double arrays [B,Hq,N,D], [B,Hkv,N,D]); causal masks key j > query i.
void orc_attention_ref(const double* q, const double* k, const double* v, int64_t B, int64_t Hq, int64_t Hkv,
                       int64_t N, int64_t D, int causal, double sm_scale, int64_t bh_begin, int64_t bh_end,
                       int threads, double* out) {
  (void)B;
  parallel_for((bh_end - bh_begin) * N, threads, [&](int64_t work) {
    int64_t bh = bh_begin + work / N, i = work % N;
    int64_t b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
    std::vector<double> s(N);
    double mx = -std::numeric_limits<double>::infinity();
    int64_t jmax = causal ? i + 1 : N;
    for (int64_t j = 0; j < jmax; ++j) {
      double acc = 0.0;
      for (int64_t c = 0; c < D; ++c) acc += q[idx4(b, h, i, c, Hq, N, D)] * k[idx4(b, g, j, c, Hkv, N, D)];
      s[j] = acc * sm_scale;
      mx = std::max(mx, s[j]);
    }
    double den = 0.0;
    for (int64_t j = 0; j < jmax; ++j) { s[j] = std::exp(s[j] - mx); den += s[j]; }
    for (int64_t c = 0; c < D; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < jmax; ++j) acc += s[j] * v[idx4(b, g, j, c, Hkv, N, D)];
      out[idx4(b, h, i, c, Hq, N, D)] = acc / den;
    }
  });
}

int orc_hardware_threads(void) { return (int)std::max(1u, std::thread::hardware_concurrency()); }

}  // extern "C"
