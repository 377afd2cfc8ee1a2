"""CPU oracle for the quantized attention forward pass — TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over ``oracle.cpp`` (plain C++17, built with g++ and
``-ffp-contract=off``).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and is never a fallback for it.

Tensors cross this boundary as numpy arrays: 16-bit inputs as ``uint16`` bit
patterns plus a dtype code (0 = bfloat16, 1 = float16), everything else in the
layouts documented in ``oracle.cpp``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, FP16 = 0, 1
QK_INT8, QK_MXFP4, QK_MXFP8, QK_HI = 0, 1, 2, 3
P_BF16, P_E4M3, P_MXFP4, P_NVFP4_MXFP8, P_EXACT = 0, 1, 2, 3, 4
V_HI, V_E4M3, V_MXFP4, V_MXFP8 = 0, 1, 2, 3


def build() -> str:
    """Compile liboracle.so with g++ (no fast-math, no FMA contraction)."""
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-shared", "-fPIC", "-pthread", "-o", _LIB_PATH + ".tmp", _SRC]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = C.CDLL(_LIB_PATH)
    _lib.orc_mx_exponent.restype = C.c_int
    _lib.orc_mx_exponent.argtypes = [C.c_double]
    _lib.orc_hardware_threads.restype = C.c_int
    return _lib


def _p(a: Optional[np.ndarray]):
    return C.c_void_p(0) if a is None else C.c_void_p(a.ctypes.data)


def _i(x) -> C.c_int64:
    return C.c_int64(int(x))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def hardware_threads() -> int:
    return int(_load().orc_hardware_threads())


# ----------------------------------------------------------------------------- formats
def bf16_encode(x) -> np.ndarray:
    x = _c(x, np.float32); y = np.empty(x.shape, np.uint16)
    _load().orc_bf16_encode(_p(x), _p(y), _i(x.size)); return y


def f16_encode(x) -> np.ndarray:
    x = _c(x, np.float32); y = np.empty(x.shape, np.uint16)
    _load().orc_f16_encode(_p(x), _p(y), _i(x.size)); return y


def bf16_decode(h) -> np.ndarray:
    h = _c(h, np.uint16); y = np.empty(h.shape, np.float32)
    _load().orc_bf16_decode(_p(h), _p(y), _i(h.size)); return y


def f16_decode(h) -> np.ndarray:
    h = _c(h, np.uint16); y = np.empty(h.shape, np.float32)
    _load().orc_f16_decode(_p(h), _p(y), _i(h.size)); return y


def e4m3_encode(x) -> np.ndarray:
    x = _c(x, np.float32); y = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode(_p(x), _p(y), _i(x.size)); return y


def e4m3_decode(c) -> np.ndarray:
    c = _c(c, np.uint8); y = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode(_p(c), _p(y), _i(c.size)); return y


def e2m1_encode(x) -> np.ndarray:
    x = _c(x, np.float32); y = np.empty(x.shape, np.uint8)
    _load().orc_e2m1_encode(_p(x), _p(y), _i(x.size)); return y


def e2m1_decode(c) -> np.ndarray:
    c = _c(c, np.uint8); y = np.empty(c.shape, np.float64)
    _load().orc_e2m1_decode(_p(c), _p(y), _i(c.size)); return y


def mx_exponent(amax: float) -> int:
    return int(_load().orc_mx_exponent(C.c_double(float(amax))))


def decode16(h: np.ndarray, dt: int) -> np.ndarray:
    return bf16_decode(h) if dt == BF16 else f16_decode(h)


# ----------------------------------------------------------------------------- pipeline steps
def smooth_k(k16: np.ndarray, dt: int):
    """K smoothing: returns (mean [B,H,D] fp32, K_s 16-bit patterns like k16)."""
    k16 = _c(k16, np.uint16); B, H, N, D = k16.shape
    mean = np.empty((B, H, D), np.float32); ks = np.empty_like(k16)
    _load().orc_smooth_k(_p(k16), C.c_int(dt), _i(B), _i(H), _i(N), _i(D), _p(mean), _p(ks))
    return mean, ks


def hadamard_rows(x16: np.ndarray, dt: int) -> np.ndarray:
    """fp32 rows of x times the normalized Sylvester Hadamard matrix (fast-transform stage
    order, then one multiply by fp32(1/sqrt(D)))."""
    x16 = _c(x16, np.uint16); D = x16.shape[-1]
    out = np.empty(x16.shape, np.float32)
    _load().orc_hadamard_rows(_p(x16), C.c_int(dt), _i(x16.size // D), _i(D), _p(out))
    return out


def quant_int8(x16: np.ndarray, dt: int, block_tokens: int, hadamard: bool = False):
    x16 = _c(x16, np.uint16); B, H, N, D = x16.shape
    nblk = (N + block_tokens - 1) // block_tokens
    codes = np.empty((B, H, N, D), np.int8); scales = np.empty((B, H, nblk), np.float32)
    _load().orc_quant_int8(_p(x16), C.c_int(dt), _i(B), _i(H), _i(N), _i(D), _i(block_tokens), C.c_int(int(hadamard)),
                           _p(codes), _p(scales))
    return codes, scales


def quant_fp8_channel(v16: np.ndarray, dt: int):
    """Per-channel E4M3 of V: codes [B,H,D,Np] (tokens contiguous, Np = N rounded up to 64,
    zero padding), scales [B,H,D]."""
    v16 = _c(v16, np.uint16); B, H, N, D = v16.shape
    Np = (N + 63) // 64 * 64
    codes = np.empty((B, H, D, Np), np.uint8); scales = np.empty((B, H, D), np.float32)
    _load().orc_quant_fp8_channel(_p(v16), C.c_int(dt), _i(B), _i(H), _i(N), _i(D), _p(codes), _p(scales))
    return codes, scales


def quant_mxfp4(x16: np.ndarray, dt: int, axis: int, hadamard: bool = False):
    x16 = _c(x16, np.uint16); B, H, N, D = x16.shape
    Np = (N + 63) // 64 * 64
    rows, length = (N, D) if axis == 0 else (D, Np)
    codes = np.empty((B, H, rows, length // 2), np.uint8)
    scales = np.empty((B, H, rows, length // 32) if axis == 0 else (B, H, Np // 32, D), np.uint8)
    if hadamard and axis != 0:
        raise ValueError("the Hadamard transform runs along D (axis 0)")
    _load().orc_quant_mxfp4(_p(x16), C.c_int(dt), _i(B), _i(H), _i(N), _i(D), C.c_int(axis), C.c_int(int(hadamard)),
                            _p(codes), _p(scales))
    return codes, scales


def quant_nvfp4(x16: np.ndarray, dt: int, axis: int, mode: int, hadamard: bool = False):
    """mode 0 = max-scaling, 1 = ScaleSearch on the 0.85..1.15 grid, 2 = the page's bit offsets [-2, 6].
    Returns (codes, ue4m3 scales, index of the winning candidate per block)."""
    x16 = _c(x16, np.uint16); B, H, N, D = x16.shape
    Np = (N + 63) // 64 * 64
    rows, length = (N, D) if axis == 0 else (D, Np)
    codes = np.empty((B, H, rows, length // 2), np.uint8)
    sshape = (B, H, rows, length // 16) if axis == 0 else (B, H, Np // 16, D)
    scales = np.empty(sshape, np.uint8)
    chosen = np.empty(sshape, np.uint8)
    if hadamard and axis != 0:
        raise ValueError("the Hadamard transform runs along D (axis 0)")
    _load().orc_quant_nvfp4(_p(x16), C.c_int(dt), _i(B), _i(H), _i(N), _i(D), C.c_int(axis), C.c_int(mode),
                            C.c_int(int(hadamard)), _p(codes), _p(scales), _p(chosen))
    return codes, scales, chosen


def nvfp4_to_mxfp8(codes: np.ndarray, scales: np.ndarray, N: int, D: int, axis: int):
    """NVFP4 in quant_nvfp4's layout for `axis` -> (E4M3 codes, E8M0 scales): along D
    [B,H,N,D] + [B,H,N,D/32]; along tokens [B,H,D,Np] + [B,H,Np/32,D]."""
    codes = _c(codes, np.uint8); scales = _c(scales, np.uint8)
    B, H = codes.shape[:2]
    Np = (N + 63) // 64 * 64
    if axis == 0:
        f8 = np.empty((B, H, N, D), np.uint8); e8 = np.empty((B, H, N, D // 32), np.uint8)
    else:
        f8 = np.empty((B, H, D, Np), np.uint8); e8 = np.empty((B, H, Np // 32, D), np.uint8)
    _load().orc_nvfp4_to_mxfp8(_p(codes), _p(scales), _i(B), _i(H), _i(N), _i(D), C.c_int(axis), _p(f8), _p(e8))
    return f8, e8


def thrift_select(q16: np.ndarray, ks16: np.ndarray, dt: int, q_block: int, k_block: int, frac: float, causal: bool):
    q16 = _c(q16, np.uint16); ks16 = _c(ks16, np.uint16)
    B, Hq, N, D = q16.shape; Hkv = ks16.shape[1]
    nQB = (N + q_block - 1) // q_block; nKB = (N + k_block - 1) // k_block
    mask = np.empty((B, Hq, nQB, nKB), np.uint8); scores = np.empty((B, Hq, nQB, nKB), np.float32)
    _load().orc_thrift_select(_p(q16), _p(ks16), C.c_int(dt), _i(B), _i(Hq), _i(Hkv), _i(N), _i(D), _i(q_block),
                              _i(k_block), C.c_double(frac), C.c_int(int(causal)), _p(mask), _p(scores))
    return mask, scores


def sink_mask(B: int, Hq: int, N: int, q_block: int, k_block: int, n_first: int, n_last: int, causal: bool):
    """Sink-aware static selection ("Search Your Block Floating Point Scales!", Method ›
    ScaleSearchAttention: the first and last KV-cache blocks stay at full precision).  Per Q
    block qb, the valid K blocks are 0..kl, kl = the last one a causal row of the block sees
    (the last K block when not causal); marked: the first n_first and the last n_last of them."""
    nQB = (N + q_block - 1) // q_block
    nKB = (N + k_block - 1) // k_block
    mask = np.zeros((B, Hq, nQB, nKB), np.uint8)
    for qb in range(nQB):
        # the causal-valid rule of the Thrift selection: a K block is valid for Q block qb if
        # its first key is at or before the Q block's last row
        valid = [kb for kb in range(nKB) if not causal or k_block * kb <= q_block * qb + q_block - 1]
        chosen = set(valid[:n_first]) | set(valid[len(valid) - n_last:] if n_last > 0 else [])
        for kb in chosen:
            mask[:, :, qb, kb] = 1
    return mask


def nvfp4_rows_value(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 values of NVFP4 rows along D: codes [..., D/2] (even element in the low nibble),
    UE4M3 scales [..., D/16]; value = E2M1(code) * UE4M3(scale of its 16-element group)."""
    codes = np.asarray(codes, np.uint8); scales = np.asarray(scales, np.uint8)
    lo = e2m1_decode(codes & 15); hi = e2m1_decode(codes >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    return vals * np.repeat(e4m3_decode(scales), 16, axis=-1)


def nvfp4_tokens_value(codes: np.ndarray, scales: np.ndarray, N: int) -> np.ndarray:
    """fp64 values [..., N, D] of NVFP4 along the tokens: codes [..., D, Np/2] (channel rows,
    token pairs, even token in the low nibble), UE4M3 scales [..., Np/16, D] (one per channel
    and 16-token group); Np = N rounded up to 64."""
    codes = np.asarray(codes, np.uint8); scales = np.asarray(scales, np.uint8)
    lo = e2m1_decode(codes & 15); hi = e2m1_decode(codes >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)   # [..., D, Np]
    s = np.repeat(e4m3_decode(scales), 16, axis=-2)                                        # [..., Np, D]
    return (np.swapaxes(vals, -1, -2) * s)[..., :N, :]


def decode_attention(q16: np.ndarray, dt: int, k_codes, k_scales, v_codes, v_scales, causal: bool,
                     sm_scale: float) -> np.ndarray:
    """Decode-shaped attention on a KV cache held in NVFP4 ("Search Your Block Floating Point
    Scales!", Method › ScaleSearchAttention: the KV cache stored in 4 bits).  q [B,Hq,Nq,D]
    16-bit; K as NVFP4 rows along D ([B,Hkv,Nk,D/2] codes, [B,Hkv,Nk,D/16] scales), V as NVFP4
    along the tokens ([B,Hkv,D,Np/2] codes, [B,Hkv,Np/16,D] scales, Np = Nk rounded up to 64).
    Query i stands at position Nk - Nq + i (the newest tokens); with causal masking it sees
    keys j <= Nk - Nq + i.  Textbook fp64 softmax(q K^T sm_scale) V on the cache's values;
    q-head h reads KV head h // (Hq / Hkv)."""
    q = decode16(np.asarray(q16, np.uint16), dt).astype(np.float64)
    K = nvfp4_rows_value(k_codes, k_scales)
    V = nvfp4_tokens_value(v_codes, v_scales, K.shape[2])
    B, Hq, Nq, D = q.shape
    Hkv, Nk = K.shape[1], K.shape[2]
    G = Hq // Hkv
    out = np.empty((B, Hq, Nq, D), np.float64)
    pos = Nk - Nq + np.arange(Nq)
    for b in range(B):
        for h in range(Hq):
            S = (q[b, h] @ K[b, h // G].T) * sm_scale
            if causal:
                S = np.where(np.arange(Nk)[None, :] <= pos[:, None], S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            out[b, h] = (P @ V[b, h // G]) / P.sum(axis=1, keepdims=True)
    return out


class _AttnArgs(C.Structure):
    _fields_ = [
        ("B", C.c_int64), ("Hq", C.c_int64), ("Hkv", C.c_int64), ("N", C.c_int64), ("D", C.c_int64),
        ("q_block", C.c_int64), ("k_block", C.c_int64),
        ("causal", C.c_int32), ("qk_fmt", C.c_int32), ("p_fmt", C.c_int32), ("v_fmt", C.c_int32),
        ("sm_scale", C.c_double),
        ("q_i8", C.c_void_p), ("q_s", C.c_void_p), ("k_i8", C.c_void_p), ("k_s", C.c_void_p),
        ("q_lp", C.c_void_p), ("q_e8", C.c_void_p), ("k_lp", C.c_void_p), ("k_e8", C.c_void_p),
        ("q_hi", C.c_void_p), ("k_hi", C.c_void_p), ("hi_dt", C.c_int32),
        ("thrift_mask", C.c_void_p),
        ("v_hi", C.c_void_p), ("v_dt", C.c_int32),
        ("v_lp", C.c_void_p), ("v_s", C.c_void_p), ("v_e8", C.c_void_p),
        ("bh_begin", C.c_int64), ("bh_end", C.c_int64), ("qb_begin", C.c_int64), ("qb_end", C.c_int64),
        ("threads", C.c_int32),
        ("out", C.c_void_p), ("lse", C.c_void_p), ("p_mode", C.c_int32),
    ]


@dataclass
class AttnOperands:
    """Operands of the tiled attention mirror; fields not used by the chosen formats stay None."""
    qk_fmt: int
    p_fmt: int
    v_fmt: int
    q_i8: Optional[np.ndarray] = None
    q_s: Optional[np.ndarray] = None
    k_i8: Optional[np.ndarray] = None
    k_s: Optional[np.ndarray] = None
    q_lp: Optional[np.ndarray] = None
    q_e8: Optional[np.ndarray] = None
    k_lp: Optional[np.ndarray] = None
    k_e8: Optional[np.ndarray] = None
    q_hi: Optional[np.ndarray] = None
    k_hi: Optional[np.ndarray] = None
    hi_dt: int = BF16
    thrift_mask: Optional[np.ndarray] = None
    v_hi: Optional[np.ndarray] = None
    v_dt: int = BF16
    v_lp: Optional[np.ndarray] = None
    v_s: Optional[np.ndarray] = None
    v_e8: Optional[np.ndarray] = None
    p_mode: int = 0   # NVFP4 P: 0 max-scaling, 1 / 2 ScaleSearch per 16-key block (as quant_nvfp4)


def attention(ops: AttnOperands, B: int, Hq: int, Hkv: int, N: int, D: int, causal: bool, sm_scale: float,
              q_block: int = 128, k_block: int = 64, bh: Optional[tuple] = None, qb: Optional[tuple] = None,
              threads: Optional[int] = None, want_lse: bool = False):
    """Tiled quantized attention.  Returns out [B,Hq,N,D] float64 (NaN outside the requested
    subset of flat (b*Hq+h) heads `bh` = (begin, end) and Q blocks `qb` = (begin, end))."""
    keep = []

    def arr(a, dtype):
        if a is None:
            return None
        a = _c(a, dtype); keep.append(a); return a

    nQB = (N + q_block - 1) // q_block
    bh = bh or (0, B * Hq)
    qb = qb or (0, nQB)
    out = np.full((B, Hq, N, D), np.nan, np.float64)
    lse = np.full((B, Hq, N), np.nan, np.float64) if want_lse else None
    a = _AttnArgs()
    a.B, a.Hq, a.Hkv, a.N, a.D = B, Hq, Hkv, N, D
    a.q_block, a.k_block = q_block, k_block
    a.causal, a.qk_fmt, a.p_fmt, a.v_fmt = int(causal), ops.qk_fmt, ops.p_fmt, ops.v_fmt
    a.sm_scale = float(sm_scale)
    a.q_i8 = _p(arr(ops.q_i8, np.int8)).value; a.q_s = _p(arr(ops.q_s, np.float32)).value
    a.k_i8 = _p(arr(ops.k_i8, np.int8)).value; a.k_s = _p(arr(ops.k_s, np.float32)).value
    a.q_lp = _p(arr(ops.q_lp, np.uint8)).value; a.q_e8 = _p(arr(ops.q_e8, np.uint8)).value
    a.k_lp = _p(arr(ops.k_lp, np.uint8)).value; a.k_e8 = _p(arr(ops.k_e8, np.uint8)).value
    a.q_hi = _p(arr(ops.q_hi, np.uint16)).value; a.k_hi = _p(arr(ops.k_hi, np.uint16)).value
    a.hi_dt = ops.hi_dt
    a.thrift_mask = _p(arr(ops.thrift_mask, np.uint8)).value
    a.v_hi = _p(arr(ops.v_hi, np.uint16)).value; a.v_dt = ops.v_dt
    a.v_lp = _p(arr(ops.v_lp, np.uint8)).value; a.v_s = _p(arr(ops.v_s, np.float32)).value
    a.v_e8 = _p(arr(ops.v_e8, np.uint8)).value
    a.bh_begin, a.bh_end = bh
    a.qb_begin, a.qb_end = qb
    a.threads = int(threads or hardware_threads())
    a.out = out.ctypes.data
    a.lse = lse.ctypes.data if lse is not None else None
    a.p_mode = int(ops.p_mode)
    _load().orc_attention(C.byref(a))
    return (out, lse) if want_lse else out


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, sm_scale: float,
                  bh: Optional[tuple] = None, threads: Optional[int] = None) -> np.ndarray:
    """Textbook fp64 softmax(Q K^T sm_scale) V on float64 inputs [B,Hq,N,D], [B,Hkv,N,D]."""
    q = _c(q, np.float64); k = _c(k, np.float64); v = _c(v, np.float64)
    B, Hq, N, D = q.shape; Hkv = k.shape[1]
    bh = bh or (0, B * Hq)
    out = np.full(q.shape, np.nan, np.float64)
    _load().orc_attention_ref(_p(q), _p(k), _p(v), _i(B), _i(Hq), _i(Hkv), _i(N), _i(D), C.c_int(int(causal)),
                              C.c_double(sm_scale), _i(bh[0]), _i(bh[1]), C.c_int(int(threads or hardware_threads())),
                              _p(out))
    return out
