// C ABI of libsage: argument validation on the host, then kernel launches on the
// caller's stream.  No allocation, no synchronisation.
#include "../../include/sage.h"
#include "kernels.hpp"

#include <math.h>
#include <stdint.h>

using namespace sage;

namespace {

constexpr int QBLK = 128, KBLK = 64;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool shape_ok(const sage_shape& s) {
  return s.B >= 0 && s.H >= 1 && s.N >= 0 && s.D >= 1 && s.D <= 16384 && s.B <= (1 << 20) && s.H <= 65535 &&
         s.B * s.H <= 65535 && s.N <= (1ll << 31);
}
// A call whose tensors hold no elements: it validates, then returns without reading a pointer.
bool empty_call(const sage_shape& s) { return s.B * s.H == 0 || s.N == 0; }
bool is16(sage_fmt f) { return f == SAGE_BF16 || f == SAGE_FP16; }
int64_t roundup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int launched(hipError_t e) { return e == hipSuccess ? SAGE_OK : (e == hipErrorNotSupported ? SAGE_ENOTSUP : SAGE_EHIP); }
bool block_is(const sage_qtensor* t, int32_t tokens, int32_t channels) {
  return t->block.tokens == tokens && t->block.channels == channels;
}
static_assert(SAGE_DECODE_NOALLOC_SCRATCH_BYTES == DECODE_SCRATCH_BYTES, "one scratch size");

bool zero_strides(const sage_shape& s) { return s.sb == 0 && s.sh == 0 && s.sn == 0; }
// Strides absent or exactly the contiguous ones (quantized operands, library-written tensors).
bool contiguous(const sage_shape& s) {
  return zero_strides(s) || (s.sb == s.H * s.N * s.D && s.sh == s.N * s.D && s.sn == s.D);
}
// The rows of a strided tensor (see sage_shape), checked: strides all zero (contiguous), or
// non-negative multiples of align elements (the kernels move 16-byte pieces), with no two
// (b, h, n) rows overlapping and the largest element offset below 2^62.
bool layout_of(const sage_shape& s, int64_t align, Rows16* r) {
  if (zero_strides(s)) {
    *r = rows_contiguous(s.H, s.N, s.D);
    return true;
  }
  if (s.sb < 0 || s.sh < 0 || s.sn < 0 || s.sb % align || s.sh % align || s.sn % align) return false;
  int64_t st[3] = {s.sb, s.sh, s.sn}, ext[3] = {s.B, s.H, s.N};
  for (int i = 1; i < 3; ++i)   // order the dimensions by stride
    for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
      const int64_t a = st[j], b = ext[j];
      st[j] = st[j - 1]; ext[j] = ext[j - 1];
      st[j - 1] = a; ext[j - 1] = b;
    }
  int64_t span = s.D;   // elements spanned by the dimensions inside the current one
  for (int i = 0; i < 3; ++i) {
    if (ext[i] <= 1) continue;
    if (st[i] < span) return false;                                   // rows would overlap
    if (ext[i] - 1 > ((int64_t(1) << 62) - span) / st[i]) return false;
    span += (ext[i] - 1) * st[i];
  }
  *r = Rows16{s.H, s.sb, s.sh, s.sn};
  return true;
}
bool same_dims(const sage_shape& a, const sage_shape& b) { return a.B == b.B && a.H == b.H && a.N == b.N && a.D == b.D; }
bool no_dims(const sage_shape& s) { return s.B == 0 && s.H == 0 && s.N == 0 && s.D == 0 && zero_strides(s); }
// The attention kernels address a V row within a tile with 32-bit byte offsets.
constexpr int64_t V_MAX_ROW_STRIDE = int64_t(1) << 24;
// The attention kernels address tiles with 32-bit offsets (a channel-major V row spans Np bytes).
constexpr int64_t ATTN_MAX_N = 1ll << 24;

}  // namespace

extern "C" {

const char* sage_version(void) { return "sage-gfx950 0.1.0"; }

const char* sage_strerror(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_EINVAL: return "invalid argument (null pointer, shape, or block not suited to the format)";
    case SAGE_ENOTSUP: return "not supported (head dimension or format combination)";
    case SAGE_EALIGN: return "pointer not 16-byte aligned";
    case SAGE_EWORKSPACE: return "workspace missing or too small";
    case SAGE_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

size_t sage_smooth_k_workspace_bytes(sage_shape ks) {
  if (!shape_ok(ks)) return 0;
  return (size_t)(ks.B * ks.H * ((ks.N + 63) / 64) * ks.D) * sizeof(float);
}

int sage_smooth_k(const void* k, sage_fmt dt, sage_shape ks, float* mean_out, void* k_smoothed_out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  if (!shape_ok(ks) || ks.D % 8 != 0) return SAGE_EINVAL;
  const bool no_heads = ks.B * ks.H == 0;   // N == 0 still writes the (zero) means
  if ((!k && !no_heads && ks.N > 0) || (!mean_out && !no_heads)) return SAGE_EINVAL;
  if (!is16(dt)) return SAGE_ENOTSUP;
  Rows16 kr;
  if (!layout_of(ks, 8, &kr)) return SAGE_EINVAL;
  if (!aligned16(k) || !aligned16(mean_out) || (k_smoothed_out && !aligned16(k_smoothed_out))) return SAGE_EALIGN;
  const size_t need = sage_smooth_k_workspace_bytes(ks);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SAGE_EWORKSPACE;
  if (workspace && !aligned16(workspace)) return SAGE_EALIGN;
  if (no_heads) return SAGE_OK;
  return launched(launch_smooth_k(k, kr, dt == SAGE_FP16, ks.B * ks.H, ks.N, (int)ks.D, mean_out, k_smoothed_out,
                                  (float*)workspace, stream));
}

int sage_quantized_bytes(sage_fmt fmt, sage_block block, sage_shape xs, size_t* codes_bytes, size_t* scale_bytes) {
  if (!codes_bytes || !scale_bytes || !shape_ok(xs)) return SAGE_EINVAL;
  const int64_t BH = xs.B * xs.H, N = xs.N, D = xs.D;
  const int64_t Np = roundup(N, 64);   // channel-major (token-axis) layouts are padded to 64 tokens
  switch (fmt) {
    case SAGE_INT8:
      if (block.tokens < 1 || block.channels != D) return SAGE_EINVAL;
      *codes_bytes = (size_t)(BH * N * D);
      *scale_bytes = (size_t)(BH * ((N + block.tokens - 1) / block.tokens)) * 4;
      return SAGE_OK;
    case SAGE_E4M3:
      if (block.tokens != 0 || block.channels != 1) return SAGE_EINVAL;
      *codes_bytes = (size_t)(BH * D * Np);
      *scale_bytes = (size_t)(BH * D) * 4;
      return SAGE_OK;
    case SAGE_MXFP4:
    case SAGE_NVFP4: {
      const int g = fmt == SAGE_MXFP4 ? 32 : 16;
      if (block.tokens == 1 && block.channels == g) {
        if (D % 32) return SAGE_EINVAL;
        *codes_bytes = (size_t)(BH * N * D / 2);
        *scale_bytes = (size_t)(BH * N * D / g);
      } else if (block.tokens == g && block.channels == 1) {
        *codes_bytes = (size_t)(BH * D * Np / 2);
        *scale_bytes = (size_t)(BH * D * Np / g);
      } else {
        return SAGE_EINVAL;
      }
      return SAGE_OK;
    }
    default: return SAGE_ENOTSUP;
  }
}

namespace {
int quantize_impl(const void* x, sage_fmt in_dt, sage_shape xs, const float* mean, sage_fmt fmt, sage_block block,
                  sage_scale_mode mode, void* codes_out, void* scales_out, hipStream_t stream) {
  if (!shape_ok(xs)) return SAGE_EINVAL;
  if (!empty_call(xs) && (!x || !codes_out || !scales_out)) return SAGE_EINVAL;
  if (!is16(in_dt)) return SAGE_ENOTSUP;
  if (xs.D % 8 != 0) return SAGE_EINVAL;
  Rows16 xr;
  if (!layout_of(xs, 8, &xr)) return SAGE_EINVAL;
  size_t cb, sb;
  int st = sage_quantized_bytes(fmt, block, xs, &cb, &sb);
  if (st != SAGE_OK) return st;
  const bool had = (mode & SAGE_ROTATE_HADAMARD) != 0;
  mode = (sage_scale_mode)(mode & ~SAGE_ROTATE_HADAMARD);
  if (had) {   // along D only, D in {64, 128}; INT8 blocks that stay in registers
    if (xs.D != 64 && xs.D != 128) return SAGE_ENOTSUP;
    if (fmt == SAGE_E4M3) return SAGE_ENOTSUP;
    if ((fmt == SAGE_MXFP4 || fmt == SAGE_NVFP4) && block.channels == 1) return SAGE_ENOTSUP;
    if (fmt == SAGE_INT8 && (int64_t)block.tokens * xs.D > 32768) return SAGE_ENOTSUP;
  }
  if (mode != SAGE_SCALE_ABSMAX && fmt != SAGE_NVFP4) return SAGE_EINVAL;
  if (mode != SAGE_SCALE_ABSMAX && mode != SAGE_SCALE_SEARCH && mode != SAGE_SCALE_SEARCH_OFFSETS) return SAGE_EINVAL;
  if (!aligned16(x) || !aligned16(codes_out) || !aligned16(scales_out)) return SAGE_EALIGN;
  if (fmt == SAGE_E4M3 && xs.D > 128) return SAGE_ENOTSUP;
  if ((fmt == SAGE_MXFP4 || fmt == SAGE_NVFP4) && block.channels == 1 && xs.D > 128) return SAGE_ENOTSUP;
  const int64_t BH = xs.B * xs.H;
  if (BH == 0 || xs.N == 0) return SAGE_OK;
  const bool f16 = in_dt == SAGE_FP16;
  switch (fmt) {
    case SAGE_INT8:
      return launched(launch_quant_int8(x, xr, f16, BH, xs.N, (int)xs.D, block.tokens, mean, (int8_t*)codes_out,
                                        (float*)scales_out, stream, had));
    case SAGE_E4M3:
      return launched(launch_quant_fp8_channel(x, xr, f16, BH, xs.N, (int)xs.D, (uint8_t*)codes_out, (float*)scales_out,
                                               stream));
    default:
      return launched(launch_quant_fp4(x, xr, f16, BH, xs.N, (int)xs.D, fmt == SAGE_NVFP4, block.channels == 1 ? 1 : 0,
                                       (int)mode, mean, (uint8_t*)codes_out, (uint8_t*)scales_out, stream, had));
  }
}
}  // namespace

int sage_quantize_blocks(const void* x, sage_fmt in_dt, sage_shape xs, sage_fmt fmt, sage_block block,
                         sage_scale_mode mode, void* codes_out, void* scales_out, hipStream_t stream) {
  return quantize_impl(x, in_dt, xs, nullptr, fmt, block, mode, codes_out, scales_out, stream);
}

int sage_quantize_smoothed(const void* k, sage_fmt in_dt, sage_shape ks, const float* mean, sage_fmt fmt,
                           sage_block block, sage_scale_mode mode, void* codes_out, void* scales_out,
                           hipStream_t stream) {
  if (!mean && !(shape_ok(ks) && empty_call(ks))) return SAGE_EINVAL;
  if (fmt == SAGE_E4M3) return SAGE_ENOTSUP;                                          // a V format
  if ((fmt == SAGE_MXFP4 || fmt == SAGE_NVFP4) && block.tokens != 1) return SAGE_ENOTSUP;   // along D only
  if (!aligned16(mean)) return SAGE_EALIGN;
  return quantize_impl(k, in_dt, ks, mean, fmt, block, mode, codes_out, scales_out, stream);
}

int sage_nvfp4_to_mxfp8(const void* codes, const void* scales, sage_shape xs, int along_tokens, void* f8_out,
                        void* e8m0_out, hipStream_t stream) {
  if (!shape_ok(xs)) return SAGE_EINVAL;
  if (!empty_call(xs) && (!codes || !scales || !f8_out || !e8m0_out)) return SAGE_EINVAL;
  if (along_tokens != 0 && along_tokens != 1) return SAGE_EINVAL;
  if (!contiguous(xs)) return SAGE_EINVAL;   // library-written codes
  if (!along_tokens && xs.D % 32) return SAGE_EINVAL;
  if (!aligned16(codes) || !aligned16(f8_out)) return SAGE_EALIGN;
  const int64_t Np = roundup(xs.N, 64);
  const int64_t rows = along_tokens ? xs.B * xs.H * xs.D : xs.B * xs.H * xs.N, len = along_tokens ? Np : xs.D;
  return launched(launch_nvfp4_to_mxfp8((const uint8_t*)codes, (const uint8_t*)scales, rows, len,
                                        along_tokens ? (int)xs.D : 0, (uint8_t*)f8_out, (uint8_t*)e8m0_out, stream));
}

int sage_attn_fwd(const sage_qtensor* q, const sage_qtensor* k, const sage_qtensor* v, const sage_attn_params* p,
                  void* out, sage_fmt out_dt, sage_shape os, hipStream_t stream) {
  if (!q || !k || !v || !p) return SAGE_EINVAL;
  const sage_shape &qs = q->shape, &ks = k->shape, &vs = v->shape;
  if (!shape_ok(qs) || !shape_ok(ks) || !shape_ok(vs)) return SAGE_EINVAL;
  const bool empty = empty_call(qs);
  if (!empty && (!out || !q->codes || !k->codes || !v->codes)) return SAGE_EINVAL;
  if (ks.B != qs.B || vs.B != qs.B || ks.N != qs.N || vs.N != qs.N || ks.D != qs.D || vs.D != qs.D || vs.H != ks.H)
    return SAGE_EINVAL;
  if (qs.H % ks.H != 0) return SAGE_EINVAL;
  if (qs.N > ATTN_MAX_N) return SAGE_EINVAL;
  if (qs.D != 64 && qs.D != 128) return SAGE_ENOTSUP;
  if (out_dt != SAGE_FP32 && out_dt != SAGE_BF16) return SAGE_ENOTSUP;
  if (!aligned16(q->codes) || !aligned16(k->codes) || !aligned16(v->codes) || !aligned16(out)) return SAGE_EALIGN;
  if (p->causal != 0 && p->causal != 1) return SAGE_EINVAL;
  if (!(p->sm_scale >= 0.0f) || isinf(p->sm_scale)) return SAGE_EINVAL;
  // layouts: quantized operands contiguous; 16-bit V, the Thrift tiles' Q and K_s and the
  // output may be strided
  AttnArgs a;
  // 16-bit Q with INT8 K: the kernel quantizes Q itself (it may be strided)
  const bool q16 = is16(q->fmt) && k->fmt == SAGE_INT8;
  if (q16) {
    if (!layout_of(qs, 8, &a.q16r)) return SAGE_EINVAL;
  } else if (!contiguous(qs)) {
    return SAGE_EINVAL;
  }
  if (!contiguous(ks)) return SAGE_EINVAL;
  if (is16(v->fmt)) {
    if (!layout_of(vs, 8, &a.vr) || a.vr.sn > V_MAX_ROW_STRIDE) return SAGE_EINVAL;
  } else {
    if (!contiguous(vs)) return SAGE_EINVAL;
    a.vr = rows_contiguous(vs.H, vs.N, vs.D);
  }
  const sage_shape o_dims = {qs.B, qs.H, qs.N, qs.D, 0, 0, 0};
  if (no_dims(os)) {
    a.outr = rows_contiguous(qs.H, qs.N, qs.D);
  } else if (!same_dims(os, o_dims) || !layout_of(os, 4, &a.outr)) {
    return SAGE_EINVAL;
  }
  auto hi_rows = [](const sage_shape& given, const sage_shape& dims, Rows16* r) {
    if (no_dims(given)) {
      *r = rows_contiguous(dims.H, dims.N, dims.D);
      return true;
    }
    return same_dims(given, dims) && layout_of(given, 8, r);
  };
  if (!hi_rows(p->q_hi_shape, qs, &a.qhr) || !hi_rows(p->k_hi_shape, ks, &a.khr)) return SAGE_EINVAL;

  a.B = qs.B; a.Hq = qs.H; a.Hkv = ks.H; a.N = qs.N; a.D = (int)qs.D;
  a.causal = p->causal;
  a.sm_scale = p->sm_scale > 0.0f ? p->sm_scale : 1.0f / sqrtf((float)qs.D);
  a.q_codes = q->codes; a.q_scales = q->scales;
  a.k_codes = k->codes; a.k_scales = k->scales;
  a.v_codes = v->codes; a.v_scales = v->scales;
  a.v_is_f16 = v->fmt == SAGE_FP16;
  a.mask = p->block_mask; a.q_hi = (const uint16_t*)p->q_hi; a.k_hi = (const uint16_t*)p->k_hi;
  a.out = out; a.out_bf16 = out_dt == SAGE_BF16;
  a.p_scale_mode = (int)p->p_scale_mode;
  if (p->p_scale_mode != SAGE_SCALE_ABSMAX && p->p_scale_mode != SAGE_SCALE_SEARCH &&
      p->p_scale_mode != SAGE_SCALE_SEARCH_OFFSETS)
    return SAGE_EINVAL;
  if (p->p_scale_mode != SAGE_SCALE_ABSMAX && p->p_fmt != SAGE_NVFP4) return SAGE_EINVAL;

  if ((q->fmt == SAGE_INT8 || q16) && k->fmt == SAGE_INT8) {
    if (!empty && ((!q16 && !q->scales) || !k->scales)) return SAGE_EINVAL;
    if ((!q16 && !block_is(q, QBLK, (int32_t)qs.D)) || !block_is(k, KBLK, (int32_t)ks.D)) return SAGE_EINVAL;
    if (q16) {
      // the pipelined kernel's operand sets: bf16 P.V, fp16 V only at D = 64, a block mask of at
      // most PIPE_MAX_MASK_TILES K tiles
      if (!is16(v->fmt) || p->p_fmt != SAGE_BF16 || (v->fmt == SAGE_FP16 && qs.D == 128) ||
          (p->block_mask && (qs.N + KBLK - 1) / KBLK > PIPE_MAX_MASK_TILES))
        return SAGE_ENOTSUP;
      a.q16 = (const uint16_t*)q->codes;
      a.q16_f16 = q->fmt == SAGE_FP16;
    }
    if (is16(v->fmt) && p->p_fmt == SAGE_BF16) {
      if (p->block_mask) {
        if (!empty && (!p->q_hi || !p->k_hi)) return SAGE_EINVAL;
        if (p->hi_dt == SAGE_FP16) return SAGE_ENOTSUP;
        if (p->hi_dt != SAGE_BF16) return SAGE_EINVAL;
        if (!aligned16(p->q_hi) || !aligned16(p->k_hi)) return SAGE_EALIGN;
      }
      if (qs.B * qs.H == 0 || qs.N == 0) return SAGE_OK;
      return launched(launch_attn_int8(a, 0, stream));
    }
    if (v->fmt == SAGE_E4M3 && p->p_fmt == SAGE_E4M3) {
      if ((!empty && !v->scales) || p->block_mask) return SAGE_EINVAL;
      if (!block_is(v, 0, 1)) return SAGE_EINVAL;
      if (qs.B * qs.H == 0 || qs.N == 0) return SAGE_OK;
      return launched(launch_attn_int8(a, 1, stream));
    }
    return SAGE_ENOTSUP;
  }
  if (p->block_mask) return SAGE_ENOTSUP;
  const bool mx4 = q->fmt == SAGE_MXFP4 && k->fmt == SAGE_MXFP4 && v->fmt == SAGE_MXFP4 && p->p_fmt == SAGE_MXFP4;
  const bool mx8 = q->fmt == SAGE_MXFP8 && k->fmt == SAGE_MXFP8 && v->fmt == SAGE_MXFP8 && p->p_fmt == SAGE_NVFP4;
  if (!mx4 && !mx8) return SAGE_ENOTSUP;
  if (!empty && (!q->scales || !k->scales || !v->scales)) return SAGE_EINVAL;
  if (qs.D != 128) return SAGE_ENOTSUP;   // the microscaled kernels are built for D = 128
  // scale bytes are read as dwords (4 per Q/K row, 2*D per V tile)
  if ((uintptr_t)q->scales % 4 || (uintptr_t)k->scales % 4 || (uintptr_t)v->scales % 4) return SAGE_EALIGN;
  if (!block_is(q, 1, 32) || !block_is(k, 1, 32) || !block_is(v, 32, 1)) return SAGE_EINVAL;
  if (qs.B * qs.H == 0 || qs.N == 0) return SAGE_OK;
  return launched(launch_attn_mx(a, mx4 ? 0 : 1, stream));
}

size_t thrift_workspace_bytes(sage_shape qs, sage_shape ks, int q_block, int k_block) {
  if (!shape_ok(qs) || !shape_ok(ks) || q_block != QBLK || k_block != KBLK) return 0;
  if (((qs.N + QBLK - 1) / QBLK) * ((qs.N + KBLK - 1) / KBLK) > INT32_MAX || qs.D > 128) return 0;   // as the call
  return thrift_ws_bytes(qs.B, qs.H, ks.H, qs.N, (int)qs.D);
}

int thrift_select_blocks(const void* q, const void* k_smoothed, sage_fmt dt, sage_shape qs, sage_shape ks,
                         int q_block, int k_block, double frac, int causal, uint8_t* mask_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!shape_ok(qs) || !shape_ok(ks)) return SAGE_EINVAL;
  if (!empty_call(qs) && (!q || !k_smoothed || !mask_out)) return SAGE_EINVAL;
  if (ks.B != qs.B || ks.N != qs.N || ks.D != qs.D || qs.H % ks.H != 0 || qs.D % 8 != 0) return SAGE_EINVAL;
  if (dt != SAGE_BF16 || q_block != QBLK || k_block != KBLK || qs.D > 128) return SAGE_ENOTSUP;
  if (!(frac >= 0.0 && frac <= 1.0) || (causal != 0 && causal != 1)) return SAGE_EINVAL;
  {   // the selection indexes a head's (Q block, K block) pairs with 32-bit integers
    const int64_t nqb = (qs.N + QBLK - 1) / QBLK, nkb = (qs.N + KBLK - 1) / KBLK;
    if (nqb * nkb > INT32_MAX) return SAGE_EINVAL;
  }
  Rows16 qr, kr;
  if (!layout_of(qs, 8, &qr) || !layout_of(ks, 8, &kr)) return SAGE_EINVAL;
  if (!aligned16(q) || !aligned16(k_smoothed)) return SAGE_EALIGN;
  const size_t need = empty_call(qs) ? 0 : thrift_ws_bytes(qs.B, qs.H, ks.H, qs.N, (int)qs.D);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SAGE_EWORKSPACE;
  if (!aligned16(workspace)) return SAGE_EALIGN;
  if (empty_call(qs)) return SAGE_OK;
  return launched(launch_thrift_select((const uint16_t*)q, qr, (const uint16_t*)k_smoothed, kr, qs.B, qs.H, ks.H, qs.N,
                                       (int)qs.D, frac, causal, mask_out, workspace, stream));
}

size_t sage_decode_workspace_bytes(sage_shape qs, sage_shape ks) {
  if (!shape_ok(qs) || !shape_ok(ks) || qs.H % ks.H != 0) return 0;
  if (ks.N < 1 || ks.N > (1 << 26) || qs.N > ks.N) return 0;   // the shapes sage_decode_fwd accepts
  return decode_ws_bytes(qs.B, qs.H, ks.H, qs.N, ks.N);
}

namespace {
// Validation shared by the two decode entry points; on SAGE_OK, *empty says whether there is
// nothing to launch.
int decode_check(const void* q, sage_fmt q_dt, sage_shape qs, const sage_qtensor* k, const sage_qtensor* v,
                 int causal, void* out, sage_fmt out_dt, bool* empty_out) {
  if (!k || !v || !shape_ok(qs)) return SAGE_EINVAL;
  const bool empty = empty_call(qs);   // no new tokens (or no batch): nothing is read
  if (!empty && (!q || !out || !k->codes || !k->scales || !v->codes || !v->scales)) return SAGE_EINVAL;
  const sage_shape &ks = k->shape, &vs = v->shape;
  if (!shape_ok(ks) || !shape_ok(vs)) return SAGE_EINVAL;
  if (ks.B != qs.B || vs.B != qs.B || vs.H != ks.H || vs.N != ks.N || ks.D != qs.D || vs.D != qs.D) return SAGE_EINVAL;
  if (qs.H % ks.H != 0 || (causal != 0 && causal != 1)) return SAGE_EINVAL;
  if (qs.N > ks.N || ks.N == 0) return SAGE_EINVAL;   // the new tokens are the cache's last positions
  if (ks.N > (1 << 26)) return SAGE_EINVAL;           // cache offsets are 32-bit (64 bytes a key)
  if (!is16(q_dt) || k->fmt != SAGE_NVFP4 || v->fmt != SAGE_NVFP4 || qs.D != 128) return SAGE_ENOTSUP;
  if (!block_is(k, 1, 16) || !block_is(v, 16, 1)) return SAGE_EINVAL;
  Rows16 qr;
  if (!layout_of(qs, 8, &qr) || !contiguous(ks) || !contiguous(vs)) return SAGE_EINVAL;
  if (out_dt != SAGE_FP32 && out_dt != SAGE_BF16) return SAGE_ENOTSUP;
  if (!aligned16(q) || !aligned16(k->codes) || !aligned16(v->codes) || !aligned16(out)) return SAGE_EALIGN;
  if ((uintptr_t)k->scales % 2) return SAGE_EALIGN;   // read as byte pairs
  *empty_out = empty;
  return SAGE_OK;
}

int decode_launch(const void* q, sage_fmt q_dt, sage_shape qs, const sage_qtensor* k, const sage_qtensor* v,
                  int causal, float sm_scale, void* out, sage_fmt out_dt, void* workspace, hipStream_t stream) {
  const sage_shape& ks = k->shape;
  const float sc = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)qs.D);
  Rows16 qr;
  layout_of(qs, 8, &qr);   // checked by decode_check
  return launched(launch_decode((const uint16_t*)q, qr, q_dt == SAGE_FP16, qs.B, qs.H, ks.H, qs.N, ks.N,
                                (const uint8_t*)k->codes, (const uint8_t*)k->scales, (const uint8_t*)v->codes,
                                (const uint8_t*)v->scales, causal, sc, out, out_dt == SAGE_BF16, workspace, stream));
}
}  // namespace

int sage_decode_fwd(const void* q, sage_fmt q_dt, sage_shape qs, const sage_qtensor* k, const sage_qtensor* v,
                    int causal, float sm_scale, void* out, sage_fmt out_dt, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  bool empty = false;
  const int st = decode_check(q, q_dt, qs, k, v, causal, out, out_dt, &empty);
  if (st != SAGE_OK) return st;
  const sage_shape& ks = k->shape;
  const size_t need = decode_ws_bytes(qs.B, qs.H, ks.H, qs.N, ks.N);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SAGE_EWORKSPACE;
  if (!aligned16(workspace)) return SAGE_EALIGN;
  if (empty) return SAGE_OK;
  return decode_launch(q, q_dt, qs, k, v, causal, sm_scale, out, out_dt, workspace, stream);
}

int sage_decode_fwd_noalloc(const void* q, sage_fmt q_dt, sage_shape qs, const sage_qtensor* k, const sage_qtensor* v,
                            int causal, float sm_scale, void* out, sage_fmt out_dt, hipStream_t stream) {
  bool empty = false;
  const int st = decode_check(q, q_dt, qs, k, v, causal, out, out_dt, &empty);
  if (st != SAGE_OK) return st;
  const sage_shape& ks = k->shape;
  if (decode_ws_bytes(qs.B, qs.H, ks.H, qs.N, ks.N) > SAGE_DECODE_NOALLOC_SCRATCH_BYTES) return SAGE_EWORKSPACE;
  if (empty) return SAGE_OK;
  void* scratch_at = nullptr;
  if (decode_scratch(&scratch_at) != hipSuccess) return SAGE_EHIP;
  return decode_launch(q, q_dt, qs, k, v, causal, sm_scale, out, out_dt, scratch_at, stream);
}

int sage_sink_blocks(sage_shape qs, int q_block, int k_block, int n_first, int n_last, int causal, uint8_t* mask_out,
                     hipStream_t stream) {
  if (!shape_ok(qs)) return SAGE_EINVAL;
  if (!empty_call(qs) && !mask_out) return SAGE_EINVAL;
  if (q_block != QBLK || k_block != KBLK) return SAGE_ENOTSUP;
  if (n_first < 0 || n_last < 0 || (causal != 0 && causal != 1)) return SAGE_EINVAL;
  return launched(launch_sink_mask(qs.B * qs.H, qs.N, n_first, n_last, causal, mask_out, stream));
}

int sage_convert_f32(const float* x, int64_t n, sage_fmt fmt, void* out, hipStream_t stream) {
  if (n < 0 || (n > 0 && (!x || !out))) return SAGE_EINVAL;
  if (fmt != SAGE_BF16 && fmt != SAGE_FP16 && fmt != SAGE_E4M3 && fmt != SAGE_MXFP4 && fmt != SAGE_NVFP4)
    return SAGE_ENOTSUP;
  return launched(launch_convert_f32(x, n, (int)fmt, out, stream));
}

}  // extern "C"
