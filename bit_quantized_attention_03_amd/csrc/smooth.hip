// K smoothing — "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
// Acceleration" (Contributions / Technical approach): K's channel-wise outliers are removed
// before 8-bit quantization by subtracting each channel's mean over the tokens.
//
// HBM-bound, 6 bytes per element for 16-bit K (read K twice, write K_s once):
//   1. smooth_partial: fp32 running sum over each run of 64 tokens, in token order, for 4
//      channels per thread (one 8-byte load per token row, all 64 rows in flight before the
//      adds) -> partials [BH, runs, D].  The kernel is a single round of threads, so its time
//      is about one load round trip: four channels a thread rather than eight double the
//      threads, and so the bytes in flight.
//   2. smooth_mean:    per (bh, channel) running sum of the partials in run order, / N.
//   3. smooth_apply:   K_s = round_to_dtype(fp32(k - mean)), 8 elements per thread.
// The fixed summation order makes the mean reproducible bit for bit.
#include "device.hpp"
#include "kernels.hpp"

namespace sage {
namespace {

constexpr int RUN = 64;

template <bool F16>
__global__ __launch_bounds__(256) void smooth_partial(const uint16_t* __restrict__ k, Rows16 kr, int64_t BH,
                                                      int64_t N, int D, float* __restrict__ part) {
  const int64_t nrun = (N + RUN - 1) / RUN;
  const int cg = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= BH * nrun * cg) return;
  const int c4 = (int)(gid % cg);
  const int64_t run = (gid / cg) % nrun, bh = gid / cg / nrun;
  const int64_t t0 = run * RUN;
  const int rows = (int)((N - t0) < RUN ? (N - t0) : RUN);
  const uint16_t* p = k + kr.at(bh, t0) + c4 * 4;
  const int64_t sn = kr.sn;
  float s[4] = {0, 0, 0, 0};
  auto add_row = [&](v2i raw) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t h = (uint16_t)((uint32_t)raw[e >> 1] >> (16 * (e & 1)));
      s[e] = s[e] + in16_to_f32<F16>(h);
    }
  };
  if (rows == RUN) {   // a full run: all 64 rows in flight at once, then added in token order
    v2i raw[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) raw[j] = *(const v2i*)(p + (int64_t)j * sn);
#pragma unroll
    for (int j = 0; j < RUN; ++j) add_row(raw[j]);
  } else {
    for (int t = 0; t < rows; ++t) add_row(*(const v2i*)(p + (int64_t)t * sn));
  }
  *(v4f*)(part + (bh * nrun + run) * D + c4 * 4) = v4f{s[0], s[1], s[2], s[3]};
}

__global__ __launch_bounds__(256) void smooth_mean(const float* __restrict__ part, int64_t BH, int64_t N, int D,
                                                   float* __restrict__ mean) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= BH * D) return;
  const int64_t nrun = (N + RUN - 1) / RUN;
  const int64_t bh = gid / D, c = gid % D;
  const float* p = part + bh * nrun * D + c;
  float total = 0.0f;
  int64_t r = 0;
  for (; r + 16 <= nrun; r += 16) {   // loads in flight, sums in run order
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p[(r + j) * D];
#pragma unroll
    for (int j = 0; j < 16; ++j) total = total + v[j];
  }
  for (; r < nrun; ++r) total = total + p[r * D];
  mean[gid] = N > 0 ? total / (float)N : 0.0f;
}

template <bool F16>
__global__ __launch_bounds__(256) void smooth_apply(const uint16_t* __restrict__ k, Rows16 kr,
                                                    const float* __restrict__ mean, int64_t BH, int64_t N, int D,
                                                    uint16_t* __restrict__ ks) {
  const int64_t n8 = BH * N * D / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = i * 8;   // element of the contiguous K_s
    const int64_t row = e0 / D, bh = row / N;
    const int c0 = (int)(e0 - row * D);
    v4i raw = *(const v4i*)(k + kr.at(bh, row - bh * N) + c0);
    const float* mu = mean + bh * D + c0;
    v4i outv;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t u = (uint32_t)raw[w];
      float a = in16_to_f32<F16>((uint16_t)(u & 0xffffu)) - mu[2 * w];
      float b = in16_to_f32<F16>((uint16_t)(u >> 16)) - mu[2 * w + 1];
      outv[w] = (int)((uint32_t)f32_to_in16<F16>(a) | ((uint32_t)f32_to_in16<F16>(b) << 16));
    }
    *(v4i*)(ks + e0) = outv;
  }
}

}  // namespace

hipError_t launch_smooth_k(const void* k, const Rows16& kr, bool is_f16, int64_t BH, int64_t N, int D, float* mean,
                           void* ks, float* partials, hipStream_t st) {
  const int64_t nrun = (N + RUN - 1) / RUN;
  const int64_t t1 = BH * nrun * (D / 4);
  if (t1 > 0) {
    dim3 g((unsigned)((t1 + 255) / 256));
    if (is_f16) smooth_partial<true><<<g, 256, 0, st>>>((const uint16_t*)k, kr, BH, N, D, partials);
    else smooth_partial<false><<<g, 256, 0, st>>>((const uint16_t*)k, kr, BH, N, D, partials);
  }
  smooth_mean<<<(unsigned)((BH * D + 255) / 256), 256, 0, st>>>(partials, BH, N, D, mean);
  if (ks && BH * N > 0) {
    int64_t n8 = BH * N * D / 8;
    int64_t blocks = (n8 + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (is_f16) smooth_apply<true><<<(unsigned)blocks, 256, 0, st>>>((const uint16_t*)k, kr, mean, BH, N, D, (uint16_t*)ks);
    else smooth_apply<false><<<(unsigned)blocks, 256, 0, st>>>((const uint16_t*)k, kr, mean, BH, N, D, (uint16_t*)ks);
  }
  return hipGetLastError();
}

}  // namespace sage
