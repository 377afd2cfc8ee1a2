// Internal launchers shared between the kernel translation units and the C-ABI layer.
// Arguments are validated by the C-ABI layer before any launcher is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Rows of a [B, H, N, D] tensor held with element strides (sb, sh, sn) and contiguous
// channels: row n of head bh = b H + h starts at element b sb + h sh + n sn.  The
// contiguous layout is (H N D, N D, D).  B H <= 65535, so the head split runs in 32 bits.
struct Rows16 {
  int64_t H, sb, sh, sn;
  __host__ __device__ int64_t head(int64_t bh) const {
    const int b = (int)bh / (int)H, h = (int)bh - b * (int)H;
    return (int64_t)b * sb + (int64_t)h * sh;
  }
  __host__ __device__ int64_t at(int64_t bh, int64_t n) const { return head(bh) + n * sn; }
};
inline Rows16 rows_contiguous(int64_t H, int64_t N, int64_t D) { return Rows16{H, H * N * D, N * D, D}; }

// K smoothing (three kernels: per-run partial sums, per-channel mean, subtract+round).
hipError_t launch_smooth_k(const void* k, const Rows16& kr, bool is_f16, int64_t BH, int64_t N, int D, float* mean,
                           void* ks, float* partials, hipStream_t st);

// Block quantizers.
// mean (nullable, [BH, D] fp32): quantize round_to_dtype(x - mean) instead of x (K smoothing
// applied on the fly, bit-identical to quantizing the smoothing kernel's K_s).
// hadamard: rows along D times the normalized Hadamard matrix first (D in {64, 128}; INT8
// blocks of at most 4096 16-byte chunks; FP4 along D only), else hipErrorNotSupported.
hipError_t launch_quant_int8(const void* x, const Rows16& xr, bool is_f16, int64_t BH, int64_t N, int D, int T,
                             const float* mean, int8_t* codes, float* scales, hipStream_t st, bool hadamard = false);
hipError_t launch_quant_fp8_channel(const void* x, const Rows16& xr, bool is_f16, int64_t BH, int64_t N, int D,
                                    uint8_t* codes_t, float* scales, hipStream_t st);
hipError_t launch_quant_fp4(const void* x, const Rows16& xr, bool is_f16, int64_t BH, int64_t N, int D, bool nv,
                            int along_tokens, int mode, const float* mean /* nullable; along D only */,
                            uint8_t* codes, uint8_t* scales, hipStream_t st, bool hadamard = false);
// rows x len elements along the block axis; D_tok = 0 along D, else the channel count of a
// token-axis (V) layout whose scales are token-group major.
hipError_t launch_nvfp4_to_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t len, int D_tok,
                                 uint8_t* f8, uint8_t* e8, hipStream_t st);
hipError_t launch_convert_f32(const float* x, int64_t n, int fmt, void* out, hipStream_t st);

// Thrift block selection.
hipError_t launch_thrift_select(const uint16_t* q, const Rows16& qr, const uint16_t* ks, const Rows16& kr, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t N, int D, double frac, int causal, uint8_t* mask,
                                void* ws, hipStream_t st);
size_t thrift_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int D);
// Decode-shaped attention on an NVFP4 KV cache (rows along D, d = 128): split workgroups
// write partial (O, max, sum) to ws (decode_ws_bytes), a combine kernel writes out.
size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk);
hipError_t launch_decode(const uint16_t* q, const Rows16& qr, bool q_f16, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t Nq, int64_t Nk, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                         const uint8_t* vs, int causal, float sm_scale, void* out, bool out_bf16, void* ws,
                         hipStream_t st);
// Static sink-and-recent block mask [BH, nQB, nKB] (blocks of 128 Q rows and 64 keys).
// The allocation-free decode keeps its split partials in a static device array of this size
// (SAGE_DECODE_NOALLOC_SCRATCH_BYTES); decode_scratch gives the current device's address of it.
constexpr size_t DECODE_SCRATCH_BYTES = size_t(8) << 20;
hipError_t decode_scratch(void** p);
hipError_t launch_sink_mask(int64_t BH, int64_t N, int n_first, int n_last, int causal, uint8_t* mask, hipStream_t st);

// Attention kernels.
struct AttnArgs {
  int64_t B, Hq, Hkv, N;
  int D;
  int causal;
  float sm_scale;
  // INT8 / MX codes and scales
  const void* q_codes; const void* q_scales;
  const void* k_codes; const void* k_scales;
  const void* v_codes; const void* v_scales;   // v_codes = 16-bit V for the bf16/fp16 P.V path
  int v_is_f16;
  // 16-bit Q quantized to INT8 in the kernel (per 128-token block, as the quantizer does):
  // then q_codes / q_scales are unused.  Pipelined kernel only.
  const uint16_t* q16 = nullptr;
  int q16_f16 = 0;
  // Thrift
  const uint8_t* mask; const uint16_t* q_hi; const uint16_t* k_hi;
  void* out;
  int out_bf16;
  int p_scale_mode;   // NVFP4 P: 0 max-scaling, 1 / 2 ScaleSearch per 16-key block
  // rows of the 16-bit V (bf16 / fp16 P.V), of the Thrift tiles' Q and K_s, and of the output
  // (elements of the output dtype); quantized operands are contiguous
  Rows16 vr, qhr, khr, outr, q16r;
};
hipError_t launch_attn_int8(const AttnArgs& a, int pv_fp8, hipStream_t st);
// INT8 QK^T, bf16 or FP8 P.V: the software-pipelined kernel (attn_i8_pipe.hip).  With a Thrift block
// mask it keeps the workgroup's two mask rows in LDS, so it takes at most this many K tiles.
constexpr int64_t PIPE_MAX_MASK_TILES = 4096;
hipError_t launch_attn_int8_pipe(const AttnArgs& a, int pv_fp8, hipStream_t st);
hipError_t launch_attn_mx(const AttnArgs& a, int nvfp4_variant, hipStream_t st);

}  // namespace sage
