// The oracle's C++ under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Every exported function runs on small shapes with ragged token counts (blocks, tiles and
// 64-token padding all cut short), with exactly sized heap buffers, so a read or write past
// a buffer, a signed overflow or an invalid shift is reported.  Quantized operands come from
// the oracle's own quantizers and feed every attention operand set.  The program also checks
// that the outputs that must be finite are.
#include "../../oracle/oracle.cpp"

#include <cstdio>
#include <random>

namespace {

int g_fail = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "check failed: %s\n", what);
    ++g_fail;
  }
}
bool all_finite(const std::vector<double>& v) {
  for (double x : v)
    if (!std::isfinite(x)) return false;
  return true;
}

// bf16 patterns of N(0, 1) values (plus a few outliers), seeded
std::vector<uint16_t> bf16_normal(size_t n, uint32_t seed) {
  std::mt19937 g(seed);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  std::vector<float> f(n);
  for (size_t i = 0; i < n; ++i) f[i] = nd(g) * (i % 97 == 0 ? 8.0f : 1.0f);
  std::vector<uint16_t> y(n);
  orc_bf16_encode(f.data(), y.data(), (int64_t)n);
  return y;
}

void formats() {
  // every 16-bit pattern and every byte code through the decoders; specials through the encoders
  std::vector<uint16_t> all16(65536);
  for (int i = 0; i < 65536; ++i) all16[i] = (uint16_t)i;
  std::vector<float> f(65536);
  orc_bf16_decode(all16.data(), f.data(), 65536);
  orc_f16_decode(all16.data(), f.data(), 65536);
  std::vector<uint8_t> all8(256);
  for (int i = 0; i < 256; ++i) all8[i] = (uint8_t)i;
  std::vector<double> d(256);
  orc_e4m3_decode(all8.data(), d.data(), 256);
  orc_e2m1_decode(all8.data(), d.data(), 16);
  const float specials[] = {0.0f, -0.0f, 1e-45f, -1e-45f, 1e-40f, 5e-39f, 1.0f, -448.0f, 449.0f, 1e30f, -1e30f,
                            std::numeric_limits<float>::infinity(), -std::numeric_limits<float>::infinity(),
                            std::numeric_limits<float>::quiet_NaN(), 6.0f, 7.0f, 0.25f, 0.75f};
  const int ns = (int)(sizeof specials / sizeof specials[0]);
  std::vector<uint16_t> y16(ns);
  std::vector<uint8_t> y8(ns);
  orc_bf16_encode(specials, y16.data(), ns);
  orc_f16_encode(specials, y16.data(), ns);
  orc_e4m3_encode(specials, y8.data(), ns);
  orc_e2m1_encode(specials, y8.data(), ns);
  for (int i = 0; i < ns; ++i)
    if (std::isfinite(specials[i])) (void)orc_mx_exponent(std::fabs((double)specials[i]));
  (void)orc_mx_exponent(0.0);
}

void one_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, uint32_t seed) {
  const int64_t Np = (N + 63) / 64 * 64, nQB = (N + 127) / 128, nKB = (N + 63) / 64;
  const size_t nq = (size_t)(B * Hq * N * D), nk = (size_t)(B * Hkv * N * D);
  const std::vector<uint16_t> q16 = bf16_normal(nq, seed), k16 = bf16_normal(nk, seed + 1),
                              v16 = bf16_normal(nk, seed + 2);
  // smoothing (K_s written in bf16) and the Hadamard rows
  std::vector<float> mean((size_t)(B * Hkv * D));
  std::vector<uint16_t> ks16(nk);
  orc_smooth_k(k16.data(), 0, B, Hkv, N, D, mean.data(), ks16.data());
  std::vector<float> rot(nq);
  orc_hadamard_rows(q16.data(), 0, B * Hq * N, D, rot.data());
  // INT8 (with and without the Hadamard rows)
  std::vector<int8_t> q8(nq), k8(nk);
  std::vector<float> qs((size_t)(B * Hq * nQB)), ks((size_t)(B * Hkv * nKB));
  for (int had = 0; had < 2; ++had) {
    orc_quant_int8(q16.data(), 0, B, Hq, N, D, 128, had, q8.data(), qs.data());
    orc_quant_int8(ks16.data(), 0, B, Hkv, N, D, 64, had, k8.data(), ks.data());
  }
  // E4M3 V per channel
  std::vector<uint8_t> v8t((size_t)(B * Hkv * D * Np));
  std::vector<float> vs((size_t)(B * Hkv * D));
  orc_quant_fp8_channel(v16.data(), 0, B, Hkv, N, D, v8t.data(), vs.data());
  // MX-FP4: Q, K along D; V along the tokens
  std::vector<uint8_t> q4(nq / 2), q4e(nq / 32), k4(nk / 2), k4e(nk / 32);
  std::vector<uint8_t> v4((size_t)(B * Hkv * D * Np / 2)), v4e((size_t)(B * Hkv * (Np / 32) * D));
  orc_quant_mxfp4(q16.data(), 0, B, Hq, N, D, 0, 1, q4.data(), q4e.data());
  orc_quant_mxfp4(ks16.data(), 0, B, Hkv, N, D, 0, 0, k4.data(), k4e.data());
  orc_quant_mxfp4(v16.data(), 0, B, Hkv, N, D, 1, 0, v4.data(), v4e.data());
  // NVFP4 with every scale rule, then to MX-FP8
  std::vector<uint8_t> qn(nq / 2), qne(nq / 16), qch(nq / 16), kn(nk / 2), kne(nk / 16);
  std::vector<uint8_t> vn((size_t)(B * Hkv * D * Np / 2)), vne((size_t)(B * Hkv * (Np / 16) * D)),
      vch((size_t)(B * Hkv * (Np / 16) * D));
  for (int mode = 0; mode < 3; ++mode) {
    orc_quant_nvfp4(q16.data(), 0, B, Hq, N, D, 0, mode, mode == 1, qn.data(), qne.data(), qch.data());
    orc_quant_nvfp4(ks16.data(), 0, B, Hkv, N, D, 0, mode, 0, kn.data(), kne.data(), nullptr);
    orc_quant_nvfp4(v16.data(), 0, B, Hkv, N, D, 1, mode, 0, vn.data(), vne.data(), vch.data());
  }
  std::vector<uint8_t> q8f(nq), q8e(nq / 32), k8f(nk), k8e(nk / 32);
  std::vector<uint8_t> v8f((size_t)(B * Hkv * D * Np)), v8e((size_t)(B * Hkv * (Np / 32) * D));
  orc_nvfp4_to_mxfp8(qn.data(), qne.data(), B, Hq, N, D, 0, q8f.data(), q8e.data());
  orc_nvfp4_to_mxfp8(kn.data(), kne.data(), B, Hkv, N, D, 0, k8f.data(), k8e.data());
  orc_nvfp4_to_mxfp8(vn.data(), vne.data(), B, Hkv, N, D, 1, v8f.data(), v8e.data());
  // Thrift selection (scores kept) and the static sink mask
  std::vector<uint8_t> mask((size_t)(B * Hq * nQB * nKB));
  std::vector<float> scores(mask.size());
  for (int causal = 0; causal < 2; ++causal)
    orc_thrift_select(q16.data(), ks16.data(), 0, B, Hq, Hkv, N, D, 128, 64, 0.05, causal, mask.data(), scores.data());

  // attention over every operand set
  std::vector<double> out(nq), lse((size_t)(B * Hq * N));
  auto run = [&](int qk, int pf, int vf, bool thrift, int p_mode, int causal, const char* what) {
    orc_attn_args a;
    std::memset(&a, 0, sizeof a);
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.D = D; a.q_block = 128; a.k_block = 64;
    a.causal = causal; a.qk_fmt = qk; a.p_fmt = pf; a.v_fmt = vf; a.sm_scale = 1.0 / std::sqrt((double)D);
    a.q_i8 = q8.data(); a.q_s = qs.data(); a.k_i8 = k8.data(); a.k_s = ks.data();
    if (qk == QK_MXFP4) { a.q_lp = q4.data(); a.q_e8 = q4e.data(); a.k_lp = k4.data(); a.k_e8 = k4e.data(); }
    if (qk == QK_MXFP8) { a.q_lp = q8f.data(); a.q_e8 = q8e.data(); a.k_lp = k8f.data(); a.k_e8 = k8e.data(); }
    a.q_hi = q16.data(); a.k_hi = ks16.data(); a.hi_dt = 0;
    a.thrift_mask = thrift ? mask.data() : nullptr;
    a.v_hi = v16.data(); a.v_dt = 0;
    if (vf == V_E4M3) { a.v_lp = v8t.data(); a.v_s = vs.data(); }
    if (vf == V_MXFP4) { a.v_lp = v4.data(); a.v_e8 = v4e.data(); }
    if (vf == V_MXFP8) { a.v_lp = v8f.data(); a.v_e8 = v8e.data(); }
    a.bh_begin = 0; a.bh_end = B * Hq; a.qb_begin = 0; a.qb_end = nQB;
    a.threads = 2; a.out = out.data(); a.lse = lse.data(); a.p_mode = p_mode;
    std::fill(out.begin(), out.end(), std::numeric_limits<double>::quiet_NaN());
    orc_attention(&a);
    check(all_finite(out) && all_finite(lse), what);
  };
  for (int causal = 0; causal < 2; ++causal) {
    run(QK_INT8, P_BF16, V_HI, false, 0, causal, "int8 + bf16 P.V");
    run(QK_INT8, P_BF16, V_HI, true, 0, causal, "int8 + Thrift tiles");
    run(QK_INT8, P_E4M3, V_E4M3, false, 0, causal, "int8 + fp8 P.V");
    run(QK_MXFP4, P_MXFP4, V_MXFP4, false, 0, causal, "mxfp4");
    for (int pm = 0; pm < 3; ++pm) run(QK_MXFP8, P_NVFP4_MXFP8, V_MXFP8, false, pm, causal, "nvfp4 -> mxfp8");
    run(QK_HI, P_EXACT, V_HI, false, 0, causal, "16-bit reference");
  }
  // the textbook fp64 reference
  std::vector<double> qd(nq), kd(nk), vd(nk), ref(nq);
  for (size_t i = 0; i < nq; ++i) qd[i] = (double)bf16_decode(q16[i]);
  for (size_t i = 0; i < nk; ++i) { kd[i] = (double)bf16_decode(k16[i]); vd[i] = (double)bf16_decode(v16[i]); }
  orc_attention_ref(qd.data(), kd.data(), vd.data(), B, Hq, Hkv, N, D, 1, 1.0 / std::sqrt((double)D), 0, B * Hq, 2,
                    ref.data());
  check(all_finite(ref), "fp64 reference");
}

}  // namespace

int main() {
  formats();
  check(orc_hardware_threads() >= 1, "hardware threads");
  one_shape(1, 2, 1, 77, 64, 1);     // GQA, one partial block/tile everywhere
  one_shape(2, 2, 2, 130, 128, 7);   // two batches, ragged second Q block and K tile
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("oracle checks: ok\n");
  return 0;
}
