/*
 * sage.h — C ABI of the MI355X (gfx950) quantized attention forward library (libsage.so).
 *
 * The calls split the quantized attention forward pass of the SageAttention family into
 * its steps: K smoothing, block quantization (INT8, FP8-E4M3, MX-FP4, NVFP4 with
 * max-scaling or ScaleSearch), an NVFP4 -> FP8 dequantization pass, Thrift block
 * selection, and the fused attention (low-bit QK^T, block-scale dequantization, fp32
 * online softmax, P.V on bf16 / FP8 / FP4 matrix cores).
 *
 * Conventions (all calls):
 *  - Every pointer argument is a DEVICE pointer unless stated otherwise; the caller
 *    allocates and owns every buffer.  The library never allocates, frees or synchronises:
 *    it validates on the host, enqueues kernels on `stream` and returns.
 *  - Tensors are contiguous, row-major [B, H, N, D] (D contiguous) unless a layout below
 *    says otherwise.  Base pointers must be 16-byte aligned.
 *  - Return value 0 = success; negative = error (SAGE_E*).  Validation happens before any
 *    launch, so on a validation error no output has been touched.  SAGE_EHIP reports a
 *    failed launch (hipGetLastError after the enqueue).
 *  - Calls are stateless and thread-safe; calls on different streams may overlap.
 *  - A call enqueues kernels only (no memset, copy, allocation or synchronisation), so it can
 *    be captured into a HIP graph and replayed; replays equal eager calls bit for bit.
 *  - Empty calls: when a call's tensors hold no elements (B = 0 or N = 0; for decode, no
 *    new tokens), it validates its shapes and arguments, touches no buffer and returns
 *    SAGE_OK.  Its data pointers may then be null (PyTorch gives an empty tensor a null data
 *    pointer).  Two outputs are not empty with N = 0: sage_smooth_k still writes the means
 *    of its B * H heads (0: no tokens, nothing to subtract), and an E4M3 per-channel scale
 *    array of an empty V is left untouched (the attention never reads it).  Decode needs at
 *    least one cached key.
 *  - NaN / Inf inputs are outside the contract.
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_OK 0
#define SAGE_EINVAL (-1)     /* null pointer, bad shape, block that does not suit the format */
#define SAGE_ENOTSUP (-2)    /* D not in {64, 128}, or a format combination that is not built */
#define SAGE_EALIGN (-3)     /* a base pointer that is not 16-byte aligned */
#define SAGE_EWORKSPACE (-4) /* workspace missing or smaller than the size query returns */
#define SAGE_EHIP (-5)       /* kernel launch failed */

typedef enum {
  SAGE_BF16 = 0,   /* bfloat16 */
  SAGE_FP16 = 1,   /* IEEE binary16 */
  SAGE_FP32 = 2,   /* IEEE binary32 */
  SAGE_INT8 = 3,   /* int8 codes in [-127, 127] with an fp32 scale per block */
  SAGE_E4M3 = 4,   /* OCP FP8 E4M3 ("FN": max 448, no inf) with an fp32 scale per channel */
  SAGE_MXFP4 = 5,  /* E2M1 codes, two per byte, one E8M0 scale byte per 32 elements */
  SAGE_NVFP4 = 6,  /* E2M1 codes, two per byte, one UE4M3 scale byte per 16 elements */
  SAGE_MXFP8 = 7   /* E4M3 codes, one per byte, one E8M0 scale byte per 32 elements */
} sage_fmt;

typedef enum {
  SAGE_SCALE_ABSMAX = 0,         /* max-scaling: the block maximum fits the format's range */
  SAGE_SCALE_SEARCH = 1,         /* ScaleSearch over max-scale x {0.85 .. 1.15} (8 steps) */
  SAGE_SCALE_SEARCH_OFFSETS = 2, /* ScaleSearch over UE4M3 bit offsets f in [-2, 6] */
  SAGE_ROTATE_HADAMARD = 0x100   /* flag, OR'ed into a mode: Hadamard rows first (see below) */
} sage_scale_mode;

/* Logical [B, H, N, D] of a tensor, and its layout: element (b, h, n, d) sits at element
 * b sb + h sh + n sn + d of the buffer (channels are contiguous).  sb = sh = sn = 0 is the
 * contiguous layout (H N D, N D, D); a model's [B, N, H, D] tensor is (N H D, D, H D).
 * Every entry point that takes one returns SAGE_EINVAL unless B >= 0, H >= 1, N >= 0,
 * 1 <= D <= 16384, B <= 2^20, B * H <= 65535 (heads index a launch dimension) and N <= 2^31.
 * Strides are read where a declaration says so (the 16-bit inputs, and the attention
 * output); there they must be non-negative multiples of 16 bytes' worth of elements (8 for
 * 16-bit data, 4 for fp32 output), no two (b, h, n) rows may overlap, and the largest
 * offset must stay below 2^62, else SAGE_EINVAL.  Everywhere else (quantized codes, tensors
 * the library writes) the tensor is contiguous: strides zero or exactly the contiguous
 * ones, else SAGE_EINVAL.                                                                  */
typedef struct { int64_t B, H, N, D, sb, sh, sn; } sage_shape;

/* Block of a quantizer.  Supported (tokens, channels):
 *   SAGE_INT8 : (T, D) with T >= 1   — T consecutive tokens x all channels (Q: 128, K: 64)
 *   SAGE_E4M3 : (0, 1)               — one scale per channel over all N tokens (V)
 *   SAGE_MXFP4: (1, 32) along D (Q, K)  or (32, 1) along tokens (V)
 *   SAGE_NVFP4: (1, 16) along D (Q, K)  or (16, 1) along tokens (V)                       */
typedef struct { int32_t tokens, channels; } sage_block;

/* A quantized (or 16-bit) operand of sage_attn_fwd / sage_decode_fwd; codes/scales in the
 * layouts of sage_quantize_blocks.  `shape` is the logical [B, H, N, D] of the tensor and
 * `block` the quantizer block the codes were made with: the attention reads one scale per
 * block, so a block other than the one an operand set takes returns SAGE_EINVAL (it would
 * read the scales at the wrong stride).  Unused (any value) for 16-bit tensors.           */
typedef struct {
  sage_fmt fmt;
  const void* codes;   /* codes, or the 16-bit tensor itself for SAGE_BF16 / SAGE_FP16 */
  const void* scales;  /* NULL for 16-bit tensors */
  sage_shape shape;
  sage_block block;
} sage_qtensor;

typedef struct {
  int32_t causal;             /* 1: key j > query i is masked (top-left aligned, N_q = N_k) */
  float sm_scale;             /* softmax scale on Q.K; 0 selects 1 / sqrt(D) */
  sage_fmt p_fmt;             /* P operand of P.V: SAGE_BF16 | SAGE_E4M3 | SAGE_MXFP4 | SAGE_NVFP4 */
  const uint8_t* block_mask;  /* NULL, or [B, Hq, ceil(N/128), ceil(N/64)]: 1 = run this (Q block,
                                 K block) tile on bf16 Q and K_s (Thrift), 0 = INT8 */
  const void* q_hi;           /* 16-bit Q   [B, Hq,  N, D] read for masked tiles (else NULL) */
  const void* k_hi;           /* 16-bit K_s [B, Hkv, N, D] read for masked tiles (else NULL) */
  sage_fmt hi_dt;             /* dtype of q_hi / k_hi: SAGE_BF16 (the masked tiles run on bf16 matrix
                                 instructions); SAGE_FP16 returns SAGE_ENOTSUP, others SAGE_EINVAL */
  sage_scale_mode p_scale_mode; /* p_fmt SAGE_NVFP4 only: how each 16-key block of P picks its UE4M3
                                 scale before the FP8 conversion.  SAGE_SCALE_ABSMAX (max-scaling),
                                 or SAGE_SCALE_SEARCH / SAGE_SCALE_SEARCH_OFFSETS: the ScaleSearch
                                 rule of sage_quantize_blocks applied to the block of fp32 P
                                 ("Search Your Block Floating Point Scales!", Method > ScaleSearch).
                                 Must be SAGE_SCALE_ABSMAX for every other p_fmt (else SAGE_EINVAL). */
  sage_shape q_hi_shape;      /* layout of q_hi: all zero = q's dims, contiguous; else q's dims and */
  sage_shape k_hi_shape;      /* any valid strides (likewise k_hi with k's dims)                    */
} sage_attn_params;

/* Library version string (static storage). */
const char* sage_version(void);
/* Static description of an error code. */
const char* sage_strerror(int status);

/* K smoothing — "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
 * Acceleration", Contributions / Technical approach: K's channel-wise outliers are removed
 * before 8-bit quantization.  Computes mean[b,h,c] = (1/N) sum_t k[b,h,t,c] in fp32 with a
 * fixed order (fp32 running sums over each run of 64 tokens in token order, then a running
 * sum of those partials in run order, then one division by N) and, if k_smoothed_out is
 * not NULL, k_smoothed_out = round_to_dtype(fp32(k - mean)) (round-to-nearest-even).
 *   k              [B,H,N,D] dtype dt (SAGE_BF16 | SAGE_FP16), strided as ks says
 *   mean_out       [B,H,D] fp32
 *   k_smoothed_out [B,H,N,D] dtype dt (contiguous), or NULL
 *   workspace      >= sage_smooth_k_workspace_bytes(ks) bytes of device memory      */
int sage_smooth_k(const void* k, sage_fmt dt, sage_shape ks, float* mean_out, void* k_smoothed_out,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t sage_smooth_k_workspace_bytes(sage_shape ks);

/* Block quantization — SageAttention (Technical approach: Q and K in 8 bits), SageAttention3
 * (microscaled FP4 attention) and "Search Your Block Floating Point Scales!" (Method >
 * ScaleSearch: max-scale s = amax / 6 rounded to E4M3, or the scale with the least squared
 * error among nearby candidates).  x is [B,H,N,D] in in_dt (SAGE_BF16 | SAGE_FP16).
 * Element rule for every format: code = round_to_format(fp32(x * fp32(1 / s))), ties to
 * even, saturating; the scale rules:
 *   INT8 : s = fp32(amax / 127) per block; codes int8 [B,H,N,D]; scales fp32 [B,H,ceil(N/T)].
 *          An all-zero block has s = 0 and codes 0.
 *   E4M3 : s_c = fp32(amax_c / 448) per channel over all tokens; codes u8 [B,H,D,Np]
 *          (channel-major: tokens contiguous, Np = N rounded up to 64, zero padding);
 *          scales fp32 [B,H,D].
 *   MXFP4: e = smallest integer with 6 * 2^e >= amax (amax = 0: -127), x * 2^-e is exact.
 *          Along D: codes [B,H,N,D/2], scales E8M0 [B,H,N,D/32].  Along tokens: codes
 *          [B,H,D,Np/2], Np = N rounded up to 64 (padding = zeros), scales [B,H,Np/32,D]
 *          (token-group major: the scales of 64 consecutive tokens are 2*D bytes).
 *          Two codes per byte along the block axis, even element in the low nibble.
 *   NVFP4: baseline scale code c0 = UE4M3(fp32(amax / 6)) (0 becomes 0x01); mode
 *          SAGE_SCALE_SEARCH also evaluates UE4M3(fp32(amax/6) * g_k), g_k = fp32(0.85 +
 *          k * 0.3 / 7), k = 0..7; SAGE_SCALE_SEARCH_OFFSETS evaluates c0 + f for f in
 *          {-2,-1,1,..,6} within 0x01..0x7E.  Each candidate's squared error is summed in
 *          fp32 as the balanced index-order pairwise tree; the first strictly smaller sum
 *          wins (c0 first).  Layout as MXFP4 with one scale byte per 16 elements
 *          (along tokens: scales [B,H,Np/16,D]).
 * Scale mode must be SAGE_SCALE_ABSMAX except for SAGE_NVFP4.
 * SAGE_ROTATE_HADAMARD ("Search Your Block Floating Point Scales!", Method >
 * ScaleSearchAttention: incoherence processing of Q and K): each row of D channels is
 * first replaced by fp32(fwht(x) * fp32(1/sqrt(D))), where fwht runs the fast
 * Walsh-Hadamard stages h = 1, 2, .., D/2 in fp32, each turning (v[j], v[j+h]) with
 * j mod 2h < h into (v[j] + v[j+h], v[j] - v[j+h]) (the Sylvester-ordered Hadamard matrix);
 * the block rules above then apply to those values.  The matrix is orthogonal, so quantizing
 * both Q and K this way leaves QK^T unchanged up to quantization, and sage_attn_fwd needs no
 * change.  Along D only (INT8 blocks of T * D <= 32768 elements, SAGE_MXFP4 / SAGE_NVFP4
 * along D) with D in {64, 128}; otherwise SAGE_ENOTSUP.
 * x is read with the strides of xs; codes and scales are written contiguous.              */
int sage_quantize_blocks(const void* x, sage_fmt in_dt, sage_shape xs, sage_fmt fmt, sage_block block,
                         sage_scale_mode mode, void* codes_out, void* scales_out, hipStream_t stream);
/* Block quantization of smoothed K without storing it — SageAttention (Technical approach:
 * K smoothing before 8-bit quantization).  Produces exactly the codes and scales
 * sage_quantize_blocks would produce for K_s = round_to_dtype(fp32(k - mean)), the K_s of
 * sage_smooth_k, without writing K_s (2 bytes per element less HBM traffic each way).
 *   k     [B,H,N,D] in in_dt (SAGE_BF16 | SAGE_FP16); mean [B,H,D] fp32 (sage_smooth_k's
 *         mean_out), 16-byte aligned.
 *   fmt   SAGE_INT8 (blocks (T, D)), SAGE_MXFP4 (1, 32) or SAGE_NVFP4 (1, 16) along D; other
 *         formats and token-axis blocks return SAGE_ENOTSUP.  Layouts as sage_quantize_blocks. */
int sage_quantize_smoothed(const void* k, sage_fmt in_dt, sage_shape ks, const float* mean, sage_fmt fmt,
                           sage_block block, sage_scale_mode mode, void* codes_out, void* scales_out,
                           hipStream_t stream);

/* Host-side size query for the outputs of sage_quantize_blocks (host pointers out). */
int sage_quantized_bytes(sage_fmt fmt, sage_block block, sage_shape xs, size_t* codes_bytes, size_t* scale_bytes);

/* NVFP4 -> MXFP8, the operand form the gfx950 matrix cores take for NVFP4 data (they have
 * no UE4M3-scaled FP4 product).  For each 32 elements along the block axis: xhat = E2M1 x
 * UE4M3 (exact), A = max |xhat|, E = smallest integer with 448 * 2^E >= A (A = 0: -127),
 * f = E4M3(xhat * 2^-E).  xs is the shape of the tensor that was quantized; codes and
 * scales are sage_quantize_blocks' NVFP4 outputs along D (along_tokens = 0: D a multiple
 * of 32) or along tokens (1).  Out: f8 one E4M3 byte per element ([B,H,N,D] or [B,H,D,Np])
 * and E8M0 scales laid out like MXFP4's ([B,H,N,D/32] or [B,H,Np/32,D]).                 */
int sage_nvfp4_to_mxfp8(const void* codes, const void* scales, sage_shape xs, int along_tokens, void* f8_out,
                        void* e8m0_out, hipStream_t stream);

/* Fused quantized attention forward — SageAttention (8-bit QK^T, 16-bit P.V), SageAttention3
 * and ScaleSearchAttention (FP4 QK^T and PV with fp32 accumulation), ThriftAttention
 * (selected tiles in high precision, one joint softmax).
 * out[b,h,i,:] = sum_j softmax_j(S[i,j]) V[j,:] with S = dequant(Q) dequant(K)^T * sm_scale,
 * evaluated per Q block of 128 rows over K tiles of 64 keys in ascending order with an fp32
 * running max and sum; P is quantized to p_fmt per tile before P.V.
 * Supported operand sets (Hq a multiple of Hkv = k->shape.H; q-head h reads kv-head
 * h / (Hq / Hkv)), with the blocks each operand must carry:
 *   q, k SAGE_INT8 (blocks (128, D) / (64, D)) + v SAGE_BF16 | SAGE_FP16 + p SAGE_BF16
 *        (+ optional block_mask with bf16 q_hi / k_hi)
 *   the same with q SAGE_BF16 | SAGE_FP16 (codes = the 16-bit Q, scales NULL, block unused;
 *        Q may be strided like v): the kernel quantizes Q itself, per block of 128 tokens, to
 *        the codes and scales sage_quantize_blocks(SAGE_INT8, (128, D), SAGE_SCALE_ABSMAX)
 *        would give, and the output is bit-identical to that two-step call.  Not with fp16 v
 *        at D = 128, nor with a block_mask of more than 4096 K tiles (SAGE_ENOTSUP).
 *   q, k SAGE_INT8 (blocks (128, D) / (64, D)) + v SAGE_E4M3 (block (0, 1): per channel)
 *        + p SAGE_E4M3 (P scaled by 448)
 *   q, k SAGE_MXFP4 (block (1, 32): along D) + v SAGE_MXFP4 (block (32, 1): along tokens)
 *        + p SAGE_MXFP4 (per 32 keys)
 *   q, k SAGE_MXFP8 (block (1, 32)) + v SAGE_MXFP8 (block (32, 1)) + p SAGE_NVFP4 (max-scaled
 *        per 16 keys, then to MXFP8 like sage_nvfp4_to_mxfp8)
 * Tile offsets inside the kernels are 32-bit: N <= 2^24 (else SAGE_EINVAL).
 * Layouts: q and k (codes) contiguous; a 16-bit q, v, q_hi and k_hi may be strided (v's row
 * stride sn <= 2^24 elements); out is [B,Hq,N,D] in out_dt (SAGE_FP32 | SAGE_BF16) with the
 * layout os (all zero: contiguous; else os's dims must be q's).  D in {64, 128} for the INT8 sets;
 * the microscaled sets take D = 128 (else SAGE_ENOTSUP) and 4-byte aligned scale arrays
 * (else SAGE_EALIGN); their running max is exact (P is quantized relative to it).        */
int sage_attn_fwd(const sage_qtensor* q, const sage_qtensor* k, const sage_qtensor* v, const sage_attn_params* p,
                  void* out, sage_fmt out_dt, sage_shape os, hipStream_t stream);

/* Thrift block selection — "ThriftAttention: Selective Mixed Precision for Long-Context FP4
 * Attention", ¶1 and ¶3: a small fraction of query-key blocks runs in high precision.
 * Score of (Q block qb, K block kb) = fp32 dot product (fma chain over channels) of
 * bf16(mean of the block's Q rows) and bf16(mean of the block's K_s rows) (fp32 running
 * sums in token order, one division by the block's length).  Per (b, q-head), over the
 * causal-valid pairs (k_block*kb <= q_block*qb + q_block - 1 when causal), the
 * min(n_valid, ceil(frac * n_valid)) highest scores are selected (ties: lower qb*nKB+kb).
 *   q [B,Hq,N,D], k_smoothed [B,Hkv,N,D] in dt (SAGE_BF16), each strided as its shape
 *   says;  mask_out [B,Hq,nQB,nKB] u8.
 *   D a multiple of 8 (else SAGE_EINVAL) and at most 128 (else SAGE_ENOTSUP).
 *   q_block = 128 and k_block = 64 are supported.  0 <= frac <= 1.  A head's pair count
 *   nQB * nKB must not exceed 2^31 - 1 (N up to about 4.2 million tokens), else SAGE_EINVAL. */
int thrift_select_blocks(const void* q, const void* k_smoothed, sage_fmt dt, sage_shape qs, sage_shape ks,
                         int q_block, int k_block, double frac, int causal, uint8_t* mask_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
size_t thrift_workspace_bytes(sage_shape qs, sage_shape ks, int q_block, int k_block);

/* Decode-shaped attention on an NVFP4 KV cache — "Search Your Block Floating Point Scales!"
 * (Method > ScaleSearchAttention: the KV cache stored in 4 bits).  Nq new query rows attend to
 * a cache of Nk keys; query i stands at position Nk - Nq + i, and with causal = 1 it sees keys
 * j <= Nk - Nq + i (else all Nk).  out = softmax(q K^T sm_scale) V, with K and V the cache's
 * NVFP4 values (E2M1 x UE4M3): scores fp32, P rounded to f16 for P.V with fp32 accumulation,
 * the softmax sum of the unrounded P; sm_scale 0 selects 1 / sqrt(D).  q-head h reads KV
 * head h / (Hq / Hkv).
 *   q   [B,Hq,Nq,D] in q_dt (SAGE_BF16 | SAGE_FP16), 16-byte aligned, strided as qs says;
 *   k   SAGE_NVFP4 along D, block (1, 16), shape [B,Hkv,Nk,D]: codes [B,Hkv,Nk,D/2] (16-byte
 *       aligned), UE4M3 scales [B,Hkv,Nk,D/16] (2-byte aligned);
 *   v   SAGE_NVFP4 along the tokens, block (16, 1), shape [B,Hkv,Nk,D]: codes [B,Hkv,D,Np/2],
 *       Np = Nk rounded up to 64 (16-byte aligned), UE4M3 scales [B,Hkv,Np/16,D];
 *   out [B,Hq,Nq,D] in out_dt (SAGE_FP32 | SAGE_BF16), contiguous;
 *   workspace >= sage_decode_workspace_bytes(q shape, k shape) bytes of device memory
 *   (partial results of the key splits).
 * D = 128 (else SAGE_ENOTSUP); 1 <= Nk <= 2^26 and Nq <= Nk (else SAGE_EINVAL).            */
int sage_decode_fwd(const void* q, sage_fmt q_dt, sage_shape qs, const sage_qtensor* k, const sage_qtensor* v,
                    int causal, float sm_scale, void* out, sage_fmt out_dt, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);
size_t sage_decode_workspace_bytes(sage_shape qs, sage_shape ks);

/* sage_decode_fwd without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and errors as sage_decode_fwd (bit-identical outputs), except that the
 * split partials go to a scratch array that the library holds on each GPU it runs on, from
 * this call's first use on that GPU until the process ends:
 *   - scratch size SAGE_DECODE_NOALLOC_SCRATCH_BYTES; a call whose partials need more
 *     (sage_decode_workspace_bytes(q shape, k shape) > the limit) returns SAGE_EWORKSPACE
 *     before any launch;
 *   - the call allocates nothing; its first call on a device looks the array up (no
 *     allocation) with that device current, and the stream must belong to the current device;
 *   - every call on a GPU shares that GPU's array: calls that overlap on one GPU (on
 *     different streams, or from several threads) race on it and must be serialized by
 *     the caller.  Calls in order on one stream are safe.                                    */
#define SAGE_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int sage_decode_fwd_noalloc(const void* q, sage_fmt q_dt, sage_shape qs, const sage_qtensor* k,
                            const sage_qtensor* v, int causal, float sm_scale, void* out, sage_fmt out_dt,
                            hipStream_t stream);

/* Sink-aware static block selection — "Search Your Block Floating Point Scales!" (Method >
 * ScaleSearchAttention: the first and the last blocks of the KV cache are kept at full
 * precision, the middle ones low-bit).  For every (b, q-head) and Q block qb, with kl its
 * last causal-valid K block (k_block*kl <= q_block*qb + q_block - 1 when causal, else the
 * last K block), mask_out[b,h,qb,kb] = 1 for kb <= kl with kb < n_first or kb > kl - n_last.
 * With causal masking the last valid blocks are the diagonal ones: each query's most recent
 * keys.  The mask feeds sage_attn_fwd's block_mask (bf16 tiles), as Thrift's does.
 *   qs: the [B,Hq,N,D] shape of q;  mask_out [B,Hq,nQB,nKB] u8 (device).  q_block = 128 and
 *   k_block = 64 are supported (else SAGE_ENOTSUP); n_first, n_last >= 0 (else SAGE_EINVAL). */
int sage_sink_blocks(sage_shape qs, int q_block, int k_block, int n_first, int n_last, int causal, uint8_t* mask_out,
                     hipStream_t stream);

/* Format conversion as the quantizers perform it, for verification: n fp32 values (device)
 * to fmt codes (device): SAGE_BF16 / SAGE_FP16 (uint16 each), SAGE_E4M3 (byte each,
 * saturating), SAGE_MXFP4 / SAGE_NVFP4 (an E2M1 code per byte, saturating).               */
int sage_convert_f32(const float* x, int64_t n, sage_fmt fmt, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H_ */
