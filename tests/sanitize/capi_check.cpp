// Host checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// capi.hip (argument validation, layouts, size queries) is compiled for the host and linked
// with stub launchers that only record what they were asked to launch, so every entry point
// runs its checks and its launch path with no GPU.  Device pointers are fake aligned
// addresses: the host code must never dereference them (ASan would report it).  A failed
// expectation or a sanitizer report ends the program with a non-zero status.
#include "../../include/sage.h"
#include "../../bit_quantized_attention_03_amd/csrc/kernels.hpp"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

namespace sage {
// ---- stubs: count launches and keep the last call's row layouts
static int g_launches = 0;
static std::string g_last;
static Rows16 g_rows[4];
static hipError_t rec(const char* name) {
  ++g_launches;
  g_last = name;
  return hipSuccess;
}
hipError_t launch_smooth_k(const void*, const Rows16& kr, bool, int64_t, int64_t, int, float*, void*, float*,
                           hipStream_t) {
  g_rows[0] = kr;
  return rec("smooth_k");
}
hipError_t launch_quant_int8(const void*, const Rows16& xr, bool, int64_t, int64_t, int, int, const float*, int8_t*,
                             float*, hipStream_t, bool) {
  g_rows[0] = xr;
  return rec("quant_int8");
}
hipError_t launch_quant_fp8_channel(const void*, const Rows16& xr, bool, int64_t, int64_t, int, uint8_t*, float*,
                                    hipStream_t) {
  g_rows[0] = xr;
  return rec("quant_fp8_channel");
}
hipError_t launch_quant_fp4(const void*, const Rows16& xr, bool, int64_t, int64_t, int, bool, int, int, const float*,
                            uint8_t*, uint8_t*, hipStream_t, bool) {
  g_rows[0] = xr;
  return rec("quant_fp4");
}
hipError_t launch_nvfp4_to_mxfp8(const uint8_t*, const uint8_t*, int64_t, int64_t, int, uint8_t*, uint8_t*,
                                 hipStream_t) {
  return rec("nvfp4_to_mxfp8");
}
hipError_t launch_convert_f32(const float*, int64_t, int, void*, hipStream_t) { return rec("convert_f32"); }
hipError_t launch_thrift_select(const uint16_t*, const Rows16& qr, const uint16_t*, const Rows16& kr, int64_t, int64_t,
                                int64_t, int64_t, int, double, int, uint8_t*, void*, hipStream_t) {
  g_rows[0] = qr;
  g_rows[1] = kr;
  return rec("thrift_select");
}
size_t thrift_ws_bytes(int64_t B, int64_t Hq, int64_t, int64_t N, int) { return (size_t)(B * Hq * (N + 1)) * 4; }
size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t, int64_t Nq, int64_t) { return (size_t)(B * Hq * Nq) * 520; }
hipError_t launch_decode(const uint16_t*, const Rows16& qr, bool, int64_t, int64_t, int64_t, int64_t, int64_t,
                         const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int, float, void*, bool,
                         void*, hipStream_t) {
  g_rows[0] = qr;
  return rec("decode");
}
hipError_t decode_scratch(void** p) {
  *p = (void*)(uintptr_t)0x7000000;
  return hipSuccess;
}
hipError_t launch_sink_mask(int64_t, int64_t, int, int, int, uint8_t*, hipStream_t) { return rec("sink_mask"); }
hipError_t launch_attn_int8(const AttnArgs& a, int pv_fp8, hipStream_t) {
  g_rows[0] = a.vr; g_rows[1] = a.qhr; g_rows[2] = a.khr; g_rows[3] = a.outr;
  return rec(pv_fp8 ? "attn_int8_fp8pv" : "attn_int8");
}
hipError_t launch_attn_int8_pipe(const AttnArgs& a, hipStream_t) {
  g_rows[0] = a.vr; g_rows[3] = a.outr;
  return rec("attn_int8_pipe");
}
hipError_t launch_attn_mx(const AttnArgs& a, int v, hipStream_t) {
  g_rows[3] = a.outr;
  return rec(v ? "attn_mx8" : "attn_mx4");
}
}  // namespace sage

using namespace sage;

static int g_fail = 0;
#define EXPECT(call, want)                                                                    \
  do {                                                                                        \
    const int got_ = (call);                                                                  \
    if (got_ != (want)) {                                                                     \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
                   got_, (int)(want));                                                        \
      ++g_fail;                                                                               \
    }                                                                                         \
  } while (0)
#define CHECK(cond)                                                                 \
  do {                                                                              \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                                     \
    }                                                                               \
  } while (0)

static void* P(uintptr_t a) { return (void*)a; }   // fake device addresses, never dereferenced
static sage_shape S(int64_t B, int64_t H, int64_t N, int64_t D, int64_t sb = 0, int64_t sh = 0, int64_t sn = 0) {
  return sage_shape{B, H, N, D, sb, sh, sn};
}
static sage_shape bnhd(int64_t B, int64_t H, int64_t N, int64_t D) { return S(B, H, N, D, N * H * D, D, H * D); }
static sage_qtensor QT(sage_fmt f, sage_shape s, int32_t bt, int32_t bc, uintptr_t codes = 0x100000,
                       uintptr_t scales = 0x200000) {
  sage_qtensor t;
  std::memset(&t, 0, sizeof t);
  t.fmt = f; t.codes = P(codes); t.scales = P(scales); t.shape = s; t.block = sage_block{bt, bc};
  return t;
}
static sage_attn_params params(sage_fmt p_fmt, int causal = 0) {
  sage_attn_params p;
  std::memset(&p, 0, sizeof p);
  p.causal = causal; p.p_fmt = p_fmt; p.hi_dt = SAGE_BF16; p.p_scale_mode = SAGE_SCALE_ABSMAX;
  return p;
}

static void strings() {
  CHECK(std::strlen(sage_version()) > 0);
  for (int s = -6; s <= 0; ++s) CHECK(sage_strerror(s) != nullptr);
}

static void smoothing() {
  const sage_shape ks = S(2, 4, 333, 128);
  const size_t ws = sage_smooth_k_workspace_bytes(ks);
  CHECK(ws == (size_t)2 * 4 * 6 * 128 * 4);
  const int n0 = g_launches;
  EXPECT(sage_smooth_k(P(0x1000), SAGE_BF16, ks, (float*)P(0x2000), P(0x3000), P(0x4000), ws, nullptr), SAGE_OK);
  EXPECT(sage_smooth_k(P(0x1000), SAGE_FP16, bnhd(2, 4, 333, 128), (float*)P(0x2000), nullptr, P(0x4000), ws, nullptr),
         SAGE_OK);
  CHECK(g_launches == n0 + 2 && g_rows[0].sn == 4 * 128 && g_rows[0].sh == 128);
  EXPECT(sage_smooth_k(P(0x1000), SAGE_BF16, ks, (float*)P(0x2000), nullptr, P(0x4000), ws - 4, nullptr),
         SAGE_EWORKSPACE);
  EXPECT(sage_smooth_k(P(0x1008), SAGE_BF16, ks, (float*)P(0x2000), nullptr, P(0x4000), ws, nullptr), SAGE_EALIGN);
  EXPECT(sage_smooth_k(P(0x1000), SAGE_FP32, ks, (float*)P(0x2000), nullptr, P(0x4000), ws, nullptr), SAGE_ENOTSUP);
  EXPECT(sage_smooth_k(nullptr, SAGE_BF16, ks, (float*)P(0x2000), nullptr, P(0x4000), ws, nullptr), SAGE_EINVAL);
  EXPECT(sage_smooth_k(P(0x1000), SAGE_BF16, S(2, 4, 333, 128, 0, 128, 100), (float*)P(0x2000), nullptr, P(0x4000),
                       ws, nullptr), SAGE_EINVAL);
  EXPECT(sage_smooth_k(nullptr, SAGE_BF16, S(0, 4, 333, 128), nullptr, nullptr, nullptr, 0, nullptr), SAGE_OK);
}

static void sizes_at_the_limits() {
  // the largest shapes shape_ok accepts must not overflow any size computation
  size_t cb = 0, sb = 0;
  const sage_shape big = S(65535, 1, int64_t(1) << 31, 16384);
  EXPECT(sage_quantized_bytes(SAGE_INT8, sage_block{128, 16384}, big, &cb, &sb), SAGE_OK);
  CHECK(cb == (size_t)65535 * (size_t(1) << 31) * 16384);
  EXPECT(sage_quantized_bytes(SAGE_E4M3, sage_block{0, 1}, big, &cb, &sb), SAGE_OK);
  EXPECT(sage_quantized_bytes(SAGE_MXFP4, sage_block{1, 32}, big, &cb, &sb), SAGE_OK);
  EXPECT(sage_quantized_bytes(SAGE_NVFP4, sage_block{16, 1}, big, &cb, &sb), SAGE_OK);
  EXPECT(sage_quantized_bytes(SAGE_INT8, sage_block{128, 16385}, S(1, 1, 1, 16385), &cb, &sb), SAGE_EINVAL);
  EXPECT(sage_quantized_bytes(SAGE_INT8, sage_block{128, 64}, S(1, 65536, 1, 64), &cb, &sb), SAGE_EINVAL);
  CHECK(sage_smooth_k_workspace_bytes(big) > 0);
  CHECK(thrift_workspace_bytes(S(1, 65535, int64_t(1) << 31, 128), S(1, 65535, int64_t(1) << 31, 128), 128, 64) == 0);
  CHECK(sage_decode_workspace_bytes(S(65535, 1, int64_t(1) << 31, 128), S(65535, 1, 100, 128)) == 0);
  CHECK(sage_decode_workspace_bytes(S(8, 32, 1, 128), S(8, 8, 32768, 128)) > 0);
  // strides near the 2^62 offset bound
  EXPECT(sage_smooth_k(P(0x1000), SAGE_BF16, S(3, 2, 2, 8, int64_t(1) << 61, 8, 16), (float*)P(0x2000), nullptr,
                       P(0x4000), 1 << 20, nullptr), SAGE_EINVAL);   // (3 - 1) 2^61 reaches 2^62
  EXPECT(sage_smooth_k(P(0x1000), SAGE_BF16, S(2, 2, 2, 8, int64_t(1) << 60, 8, 16), (float*)P(0x2000), nullptr,
                       P(0x4000), 1 << 20, nullptr), SAGE_OK);
}

static void quantizers() {
  const sage_shape xs = S(2, 4, 300, 128);
  const int n0 = g_launches;
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, xs, SAGE_INT8, sage_block{128, 128}, SAGE_SCALE_ABSMAX, P(0x2000),
                              P(0x3000), nullptr), SAGE_OK);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, bnhd(2, 4, 300, 128), SAGE_INT8, sage_block{128, 128},
                              (sage_scale_mode)(SAGE_SCALE_ABSMAX | SAGE_ROTATE_HADAMARD), P(0x2000), P(0x3000), nullptr),
         SAGE_OK);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_FP16, xs, SAGE_E4M3, sage_block{0, 1}, SAGE_SCALE_ABSMAX, P(0x2000),
                              P(0x3000), nullptr), SAGE_OK);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, xs, SAGE_MXFP4, sage_block{32, 1}, SAGE_SCALE_ABSMAX, P(0x2000),
                              P(0x3000), nullptr), SAGE_OK);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, bnhd(2, 4, 300, 128), SAGE_NVFP4, sage_block{1, 16},
                              SAGE_SCALE_SEARCH_OFFSETS, P(0x2000), P(0x3000), nullptr), SAGE_OK);
  CHECK(g_launches == n0 + 5 && g_last == "quant_fp4" && g_rows[0].sn == 4 * 128);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, xs, SAGE_MXFP4, sage_block{1, 32}, SAGE_SCALE_SEARCH, P(0x2000),
                              P(0x3000), nullptr), SAGE_EINVAL);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, xs, SAGE_INT8, sage_block{128, 64}, SAGE_SCALE_ABSMAX, P(0x2000),
                              P(0x3000), nullptr), SAGE_EINVAL);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, xs, SAGE_E4M3, sage_block{0, 1},
                              (sage_scale_mode)(SAGE_SCALE_ABSMAX | SAGE_ROTATE_HADAMARD), P(0x2000), P(0x3000), nullptr),
         SAGE_ENOTSUP);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, S(2, 4, 300, 96), SAGE_INT8, sage_block{128, 96},
                              (sage_scale_mode)(SAGE_SCALE_ABSMAX | SAGE_ROTATE_HADAMARD), P(0x2000), P(0x3000), nullptr),
         SAGE_ENOTSUP);
  EXPECT(sage_quantize_blocks(P(0x1000), SAGE_BF16, S(2, 4, 300, 128, 0, 0, 132), SAGE_INT8, sage_block{128, 128},
                              SAGE_SCALE_ABSMAX, P(0x2000), P(0x3000), nullptr), SAGE_EINVAL);
  EXPECT(sage_quantize_smoothed(P(0x1000), SAGE_BF16, bnhd(2, 4, 300, 128), (const float*)P(0x5000), SAGE_INT8,
                                sage_block{64, 128}, SAGE_SCALE_ABSMAX, P(0x2000), P(0x3000), nullptr), SAGE_OK);
  EXPECT(sage_quantize_smoothed(P(0x1000), SAGE_BF16, xs, nullptr, SAGE_INT8, sage_block{64, 128}, SAGE_SCALE_ABSMAX,
                                P(0x2000), P(0x3000), nullptr), SAGE_EINVAL);
  EXPECT(sage_nvfp4_to_mxfp8(P(0x1000), P(0x2000), xs, 1, P(0x3000), P(0x4000), nullptr), SAGE_OK);
  EXPECT(sage_nvfp4_to_mxfp8(P(0x1000), P(0x2000), bnhd(2, 4, 300, 128), 0, P(0x3000), P(0x4000), nullptr),
         SAGE_EINVAL);
  EXPECT(sage_convert_f32((const float*)P(0x1000), 1000, SAGE_NVFP4, P(0x2000), nullptr), SAGE_OK);
  EXPECT(sage_convert_f32((const float*)P(0x1000), -1, SAGE_BF16, P(0x2000), nullptr), SAGE_EINVAL);
}

static void attention() {
  const int64_t B = 2, H = 8, Hkv = 2, N = 1000, D = 128;
  const sage_shape qs = S(B, H, N, D), ks = S(B, Hkv, N, D);
  sage_qtensor q = QT(SAGE_INT8, qs, 128, D), k = QT(SAGE_INT8, ks, 64, D);
  sage_qtensor vb = QT(SAGE_BF16, ks, 0, 0, 0x300000, 0), vbs = QT(SAGE_BF16, bnhd(B, Hkv, N, D), 0, 0, 0x300000, 0);
  sage_attn_params p = params(SAGE_BF16);
  const sage_shape none = S(0, 0, 0, 0);
  EXPECT(sage_attn_fwd(&q, &k, &vb, &p, P(0x400000), SAGE_FP32, none, nullptr), SAGE_OK);
  CHECK(g_last == "attn_int8" && g_rows[3].sn == D && g_rows[0].sn == D);   // the INT8 launcher picks the kernel
  EXPECT(sage_attn_fwd(&q, &k, &vbs, &p, P(0x400000), SAGE_BF16, bnhd(B, H, N, D), nullptr), SAGE_OK);
  CHECK(g_rows[0].sn == Hkv * D && g_rows[3].sn == H * D && g_rows[3].sh == D);
  // Thrift tiles with a strided Q
  sage_attn_params pt = params(SAGE_BF16, 1);
  pt.block_mask = (const uint8_t*)P(0x500000); pt.q_hi = P(0x600000); pt.k_hi = P(0x700000);
  pt.q_hi_shape = bnhd(B, H, N, D);
  EXPECT(sage_attn_fwd(&q, &k, &vb, &pt, P(0x400000), SAGE_FP32, none, nullptr), SAGE_OK);
  CHECK(g_last == "attn_int8" && g_rows[1].sn == H * D && g_rows[2].sn == D);
  pt.k_hi_shape = S(B, H, N, D);   // dims are k's
  EXPECT(sage_attn_fwd(&q, &k, &vb, &pt, P(0x400000), SAGE_FP32, none, nullptr), SAGE_EINVAL);
  // FP8 P.V, microscaled sets
  sage_qtensor v8 = QT(SAGE_E4M3, ks, 0, 1);
  sage_attn_params p8 = params(SAGE_E4M3);
  EXPECT(sage_attn_fwd(&q, &k, &v8, &p8, P(0x400000), SAGE_FP32, none, nullptr), SAGE_OK);
  CHECK(g_last == "attn_int8_fp8pv");
  sage_qtensor m4q = QT(SAGE_MXFP4, qs, 1, 32), m4k = QT(SAGE_MXFP4, ks, 1, 32), m4v = QT(SAGE_MXFP4, ks, 32, 1);
  sage_attn_params p4 = params(SAGE_MXFP4);
  EXPECT(sage_attn_fwd(&m4q, &m4k, &m4v, &p4, P(0x400000), SAGE_FP32, bnhd(B, H, N, D), nullptr), SAGE_OK);
  CHECK(g_last == "attn_mx4" && g_rows[3].sn == H * D);
  sage_qtensor m8q = QT(SAGE_MXFP8, qs, 1, 32), m8k = QT(SAGE_MXFP8, ks, 1, 32), m8v = QT(SAGE_MXFP8, ks, 32, 1);
  sage_attn_params pn = params(SAGE_NVFP4);
  pn.p_scale_mode = SAGE_SCALE_SEARCH;
  EXPECT(sage_attn_fwd(&m8q, &m8k, &m8v, &pn, P(0x400000), SAGE_FP32, none, nullptr), SAGE_OK);
  CHECK(g_last == "attn_mx8");
  // refusals
  sage_qtensor qstr = QT(SAGE_INT8, bnhd(B, H, N, D), 128, D);
  EXPECT(sage_attn_fwd(&qstr, &k, &vb, &p, P(0x400000), SAGE_FP32, none, nullptr), SAGE_EINVAL);
  EXPECT(sage_attn_fwd(&q, &k, &vb, &p, P(0x400000), SAGE_FP32, S(B, H, N, 64), nullptr), SAGE_EINVAL);
  EXPECT(sage_attn_fwd(&q, &k, &vb, &p, P(0x400000), SAGE_FP32, S(B, H, N, D, 0, 0, D), nullptr), SAGE_EINVAL);
  sage_qtensor vfar = QT(SAGE_BF16, S(B, Hkv, N, D, Hkv * N * (int64_t(1) << 25), N * (int64_t(1) << 25),
                                      int64_t(1) << 25), 0, 0, 0x300000, 0);
  EXPECT(sage_attn_fwd(&q, &k, &vfar, &p, P(0x400000), SAGE_FP32, none, nullptr), SAGE_EINVAL);
  sage_qtensor qbig = QT(SAGE_INT8, S(1, 1, (int64_t(1) << 24) + 1, D), 128, D);
  sage_qtensor kbig = QT(SAGE_INT8, S(1, 1, (int64_t(1) << 24) + 1, D), 64, D);
  sage_qtensor vbig = QT(SAGE_BF16, S(1, 1, (int64_t(1) << 24) + 1, D), 0, 0, 0x300000, 0);
  EXPECT(sage_attn_fwd(&qbig, &kbig, &vbig, &p, P(0x400000), SAGE_FP32, none, nullptr), SAGE_EINVAL);
  EXPECT(sage_attn_fwd(&q, &k, &vb, nullptr, P(0x400000), SAGE_FP32, none, nullptr), SAGE_EINVAL);
  EXPECT(sage_attn_fwd(&m4q, &m4k, &m4v, &p, P(0x400000), SAGE_FP32, none, nullptr), SAGE_ENOTSUP);
}

static void selection_and_decode() {
  const sage_shape qs = S(1, 8, 5000, 128), ks = S(1, 2, 5000, 128);
  const size_t ws = thrift_workspace_bytes(qs, ks, 128, 64);
  CHECK(ws > 0);
  EXPECT(thrift_select_blocks(P(0x1000), P(0x2000), SAGE_BF16, bnhd(1, 8, 5000, 128), ks, 128, 64, 0.05, 1,
                              (uint8_t*)P(0x3000), P(0x4000), ws, nullptr), SAGE_OK);
  CHECK(g_last == "thrift_select" && g_rows[0].sn == 8 * 128);
  EXPECT(thrift_select_blocks(P(0x1000), P(0x2000), SAGE_BF16, qs, ks, 128, 64, 1.5, 1, (uint8_t*)P(0x3000),
                              P(0x4000), ws, nullptr), SAGE_EINVAL);
  EXPECT(sage_sink_blocks(qs, 128, 64, 1, 1, 1, (uint8_t*)P(0x3000), nullptr), SAGE_OK);
  const sage_shape qd = S(8, 32, 1, 128), kd = S(8, 8, 32768, 128);
  sage_qtensor kc = QT(SAGE_NVFP4, kd, 1, 16), vc = QT(SAGE_NVFP4, kd, 16, 1);
  const size_t dws = sage_decode_workspace_bytes(qd, kd);
  EXPECT(sage_decode_fwd(P(0x1000), SAGE_BF16, bnhd(8, 32, 1, 128), &kc, &vc, 1, 0.0f, P(0x5000), SAGE_FP32, P(0x6000),
                         dws, nullptr), SAGE_OK);
  CHECK(g_last == "decode" && g_rows[0].sn == 32 * 128);
  EXPECT(sage_decode_fwd_noalloc(P(0x1000), SAGE_BF16, qd, &kc, &vc, 0, 0.0f, P(0x5000), SAGE_BF16, nullptr), SAGE_OK);
  EXPECT(sage_decode_fwd(P(0x1000), SAGE_BF16, qd, &kc, &vc, 0, 0.0f, P(0x5000), SAGE_FP32, P(0x6000), dws - 1,
                         nullptr), SAGE_EWORKSPACE);
  EXPECT(sage_decode_fwd(P(0x1000), SAGE_BF16, S(8, 32, 40000, 128), &kc, &vc, 0, 0.0f, P(0x5000), SAGE_FP32,
                         P(0x6000), 1u << 30, nullptr), SAGE_EINVAL);   // more new tokens than the cache holds
}

int main() {
  strings();
  smoothing();
  sizes_at_the_limits();
  quantizers();
  attention();
  selection_and_decode();
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("capi host checks: ok (%d stub launches)\n", g_launches);
  return 0;
}
