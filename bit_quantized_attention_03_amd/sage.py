"""ctypes binding of libsage.so (the gfx950 HIP library).  Marshalling only.

Every function takes torch tensors that already live on the GPU, allocates its outputs with
torch (device memory and the current stream are all torch is used for), and calls the C ABI
of the same name.  There is no CPU path: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsage.so")

BF16, FP16, FP32, INT8, E4M3, MXFP4, NVFP4, MXFP8 = range(8)
ABSMAX, SEARCH, SEARCH_OFFSETS = 0, 1, 2
ROTATE_HADAMARD = 0x100   # flag OR'ed into a scale mode: rows along D Hadamard-transformed first
_TORCH_FMT = {torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32}


class Shape(C.Structure):
    """[B, H, N, D] and element strides (sb, sh, sn); zero strides mean contiguous."""
    _fields_ = [("B", C.c_int64), ("H", C.c_int64), ("N", C.c_int64), ("D", C.c_int64),
                ("sb", C.c_int64), ("sh", C.c_int64), ("sn", C.c_int64)]


class Block(C.Structure):
    _fields_ = [("tokens", C.c_int32), ("channels", C.c_int32)]


class QTensorC(C.Structure):
    _fields_ = [("fmt", C.c_int), ("codes", C.c_void_p), ("scales", C.c_void_p), ("shape", Shape), ("block", Block)]


class AttnParamsC(C.Structure):
    _fields_ = [("causal", C.c_int32), ("sm_scale", C.c_float), ("p_fmt", C.c_int),
                ("block_mask", C.c_void_p), ("q_hi", C.c_void_p), ("k_hi", C.c_void_p), ("hi_dt", C.c_int),
                ("p_scale_mode", C.c_int), ("q_hi_shape", Shape), ("k_hi_shape", Shape)]


_lib = None


def lib():
    """Load libsage.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_attention_03_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.sage_version.restype = C.c_char_p
        L.sage_strerror.restype = C.c_char_p
        L.sage_strerror.argtypes = [C.c_int]
        L.sage_smooth_k_workspace_bytes.restype = C.c_size_t
        L.sage_smooth_k_workspace_bytes.argtypes = [Shape]
        L.sage_smooth_k.argtypes = [C.c_void_p, C.c_int, Shape, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        L.sage_quantize_smoothed.argtypes = [C.c_void_p, C.c_int, Shape, C.c_void_p, C.c_int, Block, C.c_int, C.c_void_p,
                                             C.c_void_p, C.c_void_p]
        L.sage_quantize_blocks.argtypes = [C.c_void_p, C.c_int, Shape, C.c_int, Block, C.c_int, C.c_void_p, C.c_void_p,
                                           C.c_void_p]
        L.sage_quantized_bytes.argtypes = [C.c_int, Block, Shape, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]
        L.sage_nvfp4_to_mxfp8.argtypes = [C.c_void_p, C.c_void_p, Shape, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
        L.sage_attn_fwd.argtypes = [C.POINTER(QTensorC), C.POINTER(QTensorC), C.POINTER(QTensorC),
                                    C.POINTER(AttnParamsC), C.c_void_p, C.c_int, Shape, C.c_void_p]
        L.thrift_select_blocks.argtypes = [C.c_void_p, C.c_void_p, C.c_int, Shape, Shape, C.c_int, C.c_int, C.c_double,
                                           C.c_int, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        L.thrift_workspace_bytes.restype = C.c_size_t
        L.thrift_workspace_bytes.argtypes = [Shape, Shape, C.c_int, C.c_int]
        L.sage_convert_f32.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
        L.sage_sink_blocks.argtypes = [Shape, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.sage_decode_workspace_bytes.restype = C.c_size_t
        L.sage_decode_workspace_bytes.argtypes = [Shape, Shape]
        L.sage_decode_fwd.argtypes = [C.c_void_p, C.c_int, Shape, C.POINTER(QTensorC), C.POINTER(QTensorC), C.c_int,
                                      C.c_float, C.c_void_p, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]
        L.sage_decode_fwd_noalloc.argtypes = [C.c_void_p, C.c_int, Shape, C.POINTER(QTensorC), C.POINTER(QTensorC),
                                              C.c_int, C.c_float, C.c_void_p, C.c_int, C.c_void_p]
        _lib = L
    return _lib


def version() -> str:
    return lib().sage_version().decode()


class SageError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {lib().sage_strerror(status).decode()} (status {status})")
        self.status = status


def _check(fn: str, status: int):
    if status != 0:
        raise SageError(fn, status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _shape(t: torch.Tensor) -> Shape:
    """The tensor's [B,H,N,D] and, unless it is contiguous, its element strides."""
    B, H, N, D = t.shape
    if t.is_contiguous():
        return Shape(B, H, N, D, 0, 0, 0)
    sb, sh, sn, _ = t.stride()
    return Shape(B, H, N, D, sb, sh, sn)


def _dev(*ts):
    """Tensors the library reads or writes densely: on the GPU and contiguous."""
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _dev_rows(*ts):
    """[B,H,N,D] tensors the library addresses by rows (sage_shape strides): on the GPU with
    contiguous channels; the library checks the rest of the layout."""
    for t in ts:
        if t is not None and (not t.is_cuda or t.dim() != 4 or (t.shape[3] > 1 and t.stride(3) != 1)):
            raise ValueError("tensors must be on the GPU, 4-d, with contiguous channels")


# ------------------------------------------------------------------------------------ steps
def smooth_k(k: torch.Tensor, want_smoothed: bool = True):
    """K smoothing: returns (mean [B,H,D] fp32, K_s like k or None)."""
    _dev_rows(k)
    B, H, N, D = k.shape
    mean = torch.empty((B, H, D), dtype=torch.float32, device=k.device)
    ks = torch.empty(k.shape, dtype=k.dtype, device=k.device) if want_smoothed else None   # contiguous
    shp = _shape(k)
    ws = torch.empty(max(1, lib().sage_smooth_k_workspace_bytes(shp)), dtype=torch.uint8, device=k.device)
    _check("sage_smooth_k", lib().sage_smooth_k(_ptr(k), _TORCH_FMT[k.dtype], shp, _ptr(mean), _ptr(ks), _ptr(ws),
                                                ws.numel(), _stream()))
    return mean, ks


def quantized_bytes(fmt: int, block: tuple, shape: tuple):
    cb, sb = C.c_size_t(), C.c_size_t()
    _check("sage_quantized_bytes", lib().sage_quantized_bytes(fmt, Block(*block), Shape(*shape), C.byref(cb), C.byref(sb)))
    return cb.value, sb.value


@dataclass
class QT:
    """A quantized operand: format, code and scale tensors, logical [B,H,N,D] shape and the
    quantizer block (tokens, channels) the codes were made with ((0, 0) for 16-bit tensors)."""
    fmt: int
    codes: torch.Tensor
    scales: Optional[torch.Tensor]
    shape: tuple
    block: tuple = (0, 0)

    def c(self) -> QTensorC:
        # a 16-bit operand is the tensor itself, with its own layout
        shape = _shape(self.codes) if self.fmt in (BF16, FP16) and self.codes.dim() == 4 else Shape(*self.shape)
        return QTensorC(self.fmt, _ptr(self.codes), _ptr(self.scales), shape, Block(*self.block))


def quantize(x: torch.Tensor, fmt: int, block: tuple, mode: int = ABSMAX, hadamard: bool = False) -> QT:
    """Block quantization (layouts as in sage.h); returns a QT with flat code/scale buffers.
    hadamard: quantize the rows along D times the normalized Hadamard matrix (Q and K only)."""
    _dev_rows(x)
    mode = mode | (ROTATE_HADAMARD if hadamard else 0)
    cb, sb = quantized_bytes(fmt, block, tuple(x.shape))
    codes = torch.empty(max(cb, 16), dtype=torch.uint8, device=x.device)
    scales = torch.empty(max(sb, 16), dtype=torch.uint8, device=x.device)
    _check("sage_quantize_blocks", lib().sage_quantize_blocks(_ptr(x), _TORCH_FMT[x.dtype], _shape(x), fmt,
                                                              Block(*block), mode, _ptr(codes), _ptr(scales), _stream()))
    return QT(fmt, codes[:cb], scales[:sb], tuple(x.shape), tuple(block))


def quantize_smoothed(k: torch.Tensor, mean: torch.Tensor, fmt: int, block: tuple, mode: int = ABSMAX,
                      hadamard: bool = False) -> QT:
    """Quantize K_s = round(k - mean) without storing it (same codes as quantize(K_s, ...))."""
    _dev_rows(k)
    mode = mode | (ROTATE_HADAMARD if hadamard else 0)
    cb, sb = quantized_bytes(fmt, block, tuple(k.shape))
    codes = torch.empty(max(cb, 16), dtype=torch.uint8, device=k.device)
    scales = torch.empty(max(sb, 16), dtype=torch.uint8, device=k.device)
    _check("sage_quantize_smoothed", lib().sage_quantize_smoothed(_ptr(k), _TORCH_FMT[k.dtype], _shape(k), _ptr(mean), fmt,
                                                                  Block(*block), mode, _ptr(codes), _ptr(scales),
                                                                  _stream()))
    return QT(fmt, codes[:cb], scales[:sb], tuple(k.shape), tuple(block))


def nvfp4_to_mxfp8(qt: QT, along_tokens: bool) -> QT:
    """NVFP4 codes and UE4M3 scales (as sage_quantize_blocks wrote them) -> E4M3 codes with
    E8M0 scales per 32 elements, the operand form of the scaled FP8 matrix product."""
    B, H, N, D = qt.shape
    Np = (N + 63) // 64 * 64
    n = B * H * (D * Np if along_tokens else N * D)
    f8 = torch.empty(max(n, 16), dtype=torch.uint8, device=qt.codes.device)
    e8 = torch.empty(max(n // 32, 16), dtype=torch.uint8, device=qt.codes.device)
    _check("sage_nvfp4_to_mxfp8", lib().sage_nvfp4_to_mxfp8(_ptr(qt.codes), _ptr(qt.scales), Shape(*qt.shape),
                                                            int(along_tokens), _ptr(f8), _ptr(e8), _stream()))
    return QT(MXFP8, f8[:n], e8[:n // 32], qt.shape, (32, 1) if along_tokens else (1, 32))


def attn_fwd(q: QT, k: QT, v: QT, causal: bool, p_fmt: int, sm_scale: float = 0.0,
             block_mask: Optional[torch.Tensor] = None, q_hi: Optional[torch.Tensor] = None,
             k_hi: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
             out: Optional[torch.Tensor] = None, p_search: int = ABSMAX) -> torch.Tensor:
    """Fused attention on quantized operands.  p_search (NVFP4 P only): ABSMAX, SEARCH or
    SEARCH_OFFSETS, the rule by which each 16-key block of P picks its scale."""
    B, Hq, N, D = q.shape
    dev = q.codes.device
    if out is None:
        out = torch.empty((B, Hq, N, D), dtype=out_dtype, device=dev)
    hi_dt = BF16
    if q_hi is not None or k_hi is not None:
        if q_hi is None or k_hi is None or q_hi.dtype != k_hi.dtype:
            raise ValueError("q_hi and k_hi go together and share one 16-bit dtype")
        hi_dt = _TORCH_FMT[q_hi.dtype]   # the library accepts bf16 only (fp16: not supported)
    _dev_rows(out, q_hi, k_hi)
    if v.fmt in (BF16, FP16):
        _dev_rows(v.codes)
    if tuple(out.shape) != (B, Hq, N, D):
        raise ValueError(f"out shape {tuple(out.shape)} != {(B, Hq, N, D)}")
    params = AttnParamsC(int(causal), float(sm_scale), p_fmt, _ptr(block_mask), _ptr(q_hi), _ptr(k_hi), hi_dt,
                         int(p_search), _shape(q_hi) if q_hi is not None else Shape(),
                         _shape(k_hi) if k_hi is not None else Shape())
    qc, kc, vc = q.c(), k.c(), v.c()
    _check("sage_attn_fwd", lib().sage_attn_fwd(C.byref(qc), C.byref(kc), C.byref(vc), C.byref(params), _ptr(out),
                                                _TORCH_FMT[out.dtype], _shape(out), _stream()))
    return out


def thrift_select(q: torch.Tensor, k_smoothed: torch.Tensor, frac: float, causal: bool,
                  q_block: int = 128, k_block: int = 64) -> torch.Tensor:
    _dev_rows(q, k_smoothed)
    B, Hq, N, D = q.shape
    nQB, nKB = (N + q_block - 1) // q_block, (N + k_block - 1) // k_block
    mask = torch.empty((B, Hq, nQB, nKB), dtype=torch.uint8, device=q.device)
    wsb = lib().thrift_workspace_bytes(_shape(q), _shape(k_smoothed), q_block, k_block)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    _check("thrift_select_blocks", lib().thrift_select_blocks(_ptr(q), _ptr(k_smoothed), _TORCH_FMT[q.dtype], _shape(q),
                                                              _shape(k_smoothed), q_block, k_block, float(frac),
                                                              int(causal), _ptr(mask), _ptr(ws), ws.numel(), _stream()))
    return mask


def sink_select(q: torch.Tensor, n_first: int, n_last: int, causal: bool,
                q_block: int = 128, k_block: int = 64) -> torch.Tensor:
    """Static mask [B,Hq,nQB,nKB] u8: each Q block's first n_first and last n_last valid K blocks."""
    _dev(q)
    B, Hq, N, D = q.shape
    nQB, nKB = (N + q_block - 1) // q_block, (N + k_block - 1) // k_block
    mask = torch.empty((B, Hq, nQB, nKB), dtype=torch.uint8, device=q.device)
    _check("sage_sink_blocks", lib().sage_sink_blocks(_shape(q), q_block, k_block, int(n_first), int(n_last),
                                                      int(causal), _ptr(mask), _stream()))
    return mask


def decode(q: torch.Tensor, k: QT, v: QT, causal: bool = False, sm_scale: float = 0.0,
           out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Nq new rows q [B,Hq,Nq,D] against an NVFP4 KV cache: k from quantize(K, NVFP4, (1, 16), ...)
    (rows along D), v from quantize(V, NVFP4, (16, 1), ...) (along the tokens)."""
    _dev_rows(q)
    B, Hq, Nq, D = q.shape
    out = torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=q.device)
    ks = Shape(*k.shape)
    wsb = lib().sage_decode_workspace_bytes(_shape(q), ks)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    kc, vc = k.c(), v.c()
    _check("sage_decode_fwd", lib().sage_decode_fwd(_ptr(q), _TORCH_FMT[q.dtype], _shape(q), C.byref(kc), C.byref(vc),
                                                    int(causal), float(sm_scale), _ptr(out), _TORCH_FMT[out_dtype],
                                                    _ptr(ws), ws.numel(), _stream()))
    return out


DECODE_NOALLOC_SCRATCH_BYTES = 8 << 20


def decode_noalloc(q: torch.Tensor, k: QT, v: QT, out: torch.Tensor, causal: bool = False,
                   sm_scale: float = 0.0) -> torch.Tensor:
    """decode() without a workspace: the split partials go to the library's per-GPU scratch
    array (sage_decode_fwd_noalloc).  The caller passes the output out [B,Hq,Nq,D] (fp32 or
    bf16); nothing is allocated.  Calls that overlap on one GPU share the scratch and race."""
    _dev_rows(q)
    _dev(out)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out shape {tuple(out.shape)} != q shape {tuple(q.shape)}")
    kc, vc = k.c(), v.c()
    _check("sage_decode_fwd_noalloc",
           lib().sage_decode_fwd_noalloc(_ptr(q), _TORCH_FMT[q.dtype], _shape(q), C.byref(kc), C.byref(vc),
                                         int(causal), float(sm_scale), _ptr(out), _TORCH_FMT[out.dtype], _stream()))
    return out


def convert_f32(x: torch.Tensor, fmt: int) -> torch.Tensor:
    _dev(x)
    out = torch.empty(x.numel(), dtype=torch.int16 if fmt in (BF16, FP16) else torch.uint8, device=x.device)
    _check("sage_convert_f32", lib().sage_convert_f32(_ptr(x), x.numel(), fmt, _ptr(out), _stream()))
    return out


# ------------------------------------------------------------------------------------ whole pass
VARIANTS = ("int8", "int8_fp8pv", "mxfp4", "nvfp4_search", "thrift", "sink")


@dataclass
class Pass:
    """Intermediate tensors of one forward pass (kept for parity checks)."""
    mean: torch.Tensor
    k_smoothed: Optional[torch.Tensor]   # None when K was quantized with smoothing on the fly
    q: QT                                # 16-bit Q itself when the attention kernel quantized it
    k: QT
    v: QT
    mask: Optional[torch.Tensor]
    out: torch.Tensor


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool, variant: str = "int8",
            sm_scale: float = 0.0, thrift_frac: float = 0.05, search_mode: int = SEARCH,
            out_dtype: torch.dtype = torch.float32, keep_smoothed: bool = False, hadamard: bool = False,
            sink_first: int = 1, sink_last: int = 1, p_search: int = ABSMAX, fuse_q: bool = False) -> Pass:
    """K smoothing -> block quantization -> (Thrift selection) -> fused attention.  K_s is only
    materialized when Thrift needs it (or keep_smoothed); otherwise K is quantized with the
    smoothing applied on the fly (identical codes).  hadamard: Q and K_s are quantized after
    the orthogonal Hadamard transform of their rows (QK^T unchanged; V and Thrift's bf16
    tiles take the original rows).  variant "sink": INT8 tiles except each Q block's first
    sink_first and last sink_last valid K blocks, which run in bf16 (a static Thrift mask).
    p_search (variant "nvfp4_search"): the rule by which each 16-key block of P picks its
    scale (ABSMAX, SEARCH or SEARCH_OFFSETS).  fuse_q (variants "int8", "thrift", "sink",
    without hadamard): Q goes to the attention kernel in 16 bits and is quantized there, per
    128-token block, to the same codes and scales as quantize() gives (one pass over Q fewer)."""
    B, Hq, N, D = q.shape
    need_ks = variant in ("thrift", "sink") or keep_smoothed
    mean, ks = smooth_k(k, want_smoothed=need_ks)

    def quant_k(fmt, block, mode=ABSMAX):
        return (quantize(ks, fmt, block, mode, hadamard) if ks is not None
                else quantize_smoothed(k, mean, fmt, block, mode, hadamard))

    mask = None
    if variant in ("int8", "int8_fp8pv", "thrift", "sink"):
        if fuse_q and variant != "int8_fp8pv" and not hadamard:
            qq = QT(_TORCH_FMT[q.dtype], q, None, tuple(q.shape))
        else:
            qq = quantize(q, INT8, (128, D), hadamard=hadamard)
        kq = quant_k(INT8, (64, D))
        if variant == "int8_fp8pv":
            vq = quantize(v, E4M3, (0, 1))
            out = attn_fwd(qq, kq, vq, causal, E4M3, sm_scale, out_dtype=out_dtype)
        else:
            vq = QT(_TORCH_FMT[v.dtype], v, None, tuple(v.shape))
            if variant in ("thrift", "sink"):
                mask = (thrift_select(q, ks, thrift_frac, causal) if variant == "thrift"
                        else sink_select(q, sink_first, sink_last, causal))
                out = attn_fwd(qq, kq, vq, causal, BF16, sm_scale, block_mask=mask, q_hi=q, k_hi=ks,
                               out_dtype=out_dtype)
            else:
                out = attn_fwd(qq, kq, vq, causal, BF16, sm_scale, out_dtype=out_dtype)
    elif variant == "mxfp4":
        qq = quantize(q, MXFP4, (1, 32), hadamard=hadamard)
        kq = quant_k(MXFP4, (1, 32))
        vq = quantize(v, MXFP4, (32, 1))
        out = attn_fwd(qq, kq, vq, causal, MXFP4, sm_scale, out_dtype=out_dtype)
    elif variant == "nvfp4_search":
        qq = nvfp4_to_mxfp8(quantize(q, NVFP4, (1, 16), search_mode, hadamard), False)
        kq = nvfp4_to_mxfp8(quant_k(NVFP4, (1, 16), search_mode), False)
        vq = nvfp4_to_mxfp8(quantize(v, NVFP4, (16, 1), search_mode), True)
        out = attn_fwd(qq, kq, vq, causal, NVFP4, sm_scale, out_dtype=out_dtype, p_search=p_search)
    else:
        raise ValueError(f"unknown variant {variant!r}; one of {VARIANTS}")
    return Pass(mean, ks, qq, kq, vq, mask, out)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, variant: str = "int8",
              **kw) -> torch.Tensor:
    """Drop-in quantized attention: [B,Hq,N,D] x [B,Hkv,N,D] x [B,Hkv,N,D] -> [B,Hq,N,D]."""
    return forward(q, k, v, causal, variant, **kw).out
