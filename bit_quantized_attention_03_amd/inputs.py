"""Seeded synthetic Q/K/V for the five workloads (no method arithmetic here).

Shapes and value recipes stand in for the pages' workloads (LLM decoding/prefill, video
generation, FP4 attention, 32K long context); the models and datasets the pages measure on
are not used.  Draws are numpy PCG64 float64 in the order Q, K, V, then the extras; the
float64 values are cast to fp32 and then to the workload's 16-bit dtype with
round-to-nearest-even (torch casts).  Both the oracle and the HIP path consume these tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: torch.dtype
    causal: bool
    recipe: str
    Nq: int = 0      # query rows when they differ from N (decode: a few new tokens against N keys)


WORKLOADS = {
    "tiny_int8": Workload("tiny_int8", 1, 2, 2, 256, 64, torch.float16, False, "tiny"),
    "llm_int8": Workload("llm_int8", 4, 32, 32, 4096, 128, torch.bfloat16, False, "llm"),
    "video_fp8": Workload("video_fp8", 2, 24, 24, 16384, 64, torch.bfloat16, False, "video"),
    "fp4_search": Workload("fp4_search", 2, 16, 16, 8192, 128, torch.bfloat16, False, "fp4"),
    "thrift_long": Workload("thrift_long", 1, 32, 8, 32768, 128, torch.bfloat16, True, "thrift"),
    # one new token per sequence against a 32K-token KV cache (held in NVFP4 by the decode path)
    "decode_nvfp4": Workload("decode_nvfp4", 8, 32, 8, 32768, 128, torch.bfloat16, False, "decode", Nq=1),
}


def workload(name: str, **overrides) -> Workload:
    return replace(WORKLOADS[name], **overrides)


def _to16(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(x.astype(np.float32)).to(dtype)


def make_qkv(w: Workload, seed: int = 0):
    """Returns CPU tensors (q [B,Hq,Nq or N,D], k [B,Hkv,N,D], v [B,Hkv,N,D]) of dtype w.dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qs, ks = (w.B, w.Hq, w.Nq or w.N, w.D), (w.B, w.Hkv, w.N, w.D)
    q = rng.standard_normal(qs)
    k = rng.standard_normal(ks)
    v = rng.standard_normal(ks)
    if w.recipe == "tiny":        # per-channel offset ~ N(0, variance 4), shared across tokens
        k += rng.standard_normal((w.B, w.Hkv, 1, w.D)) * 2.0
    elif w.recipe == "llm":       # 5% of channels per (b, h) carry an offset 8 * N(0, variance 4)
        n_out = math.ceil(0.05 * w.D)
        for b in range(w.B):
            for h in range(w.Hkv):
                ch = rng.choice(w.D, size=n_out, replace=False)
                k[b, h, :, ch] += (8.0 * 2.0 * rng.standard_normal(n_out))[:, None]
    elif w.recipe == "video":     # every channel offset ~ N(0, variance 2)
        k += rng.standard_normal((w.B, w.Hkv, 1, w.D)) * math.sqrt(2.0)
    elif w.recipe == "fp4":       # 1% of entries replaced by 4 * Student-t(3)
        for x in (q, k, v):
            sel = rng.random(x.shape) < 0.01
            x[sel] = 4.0 * rng.standard_t(3, size=int(sel.sum()))
    elif w.recipe == "thrift":    # 64 attention-sink keys (the first K block) scaled x6
        k[:, :, :64, :] *= 6.0
    elif w.recipe == "decode":    # plain N(0, 1) queries, keys and values
        pass
    else:
        raise ValueError(w.recipe)
    return _to16(q, w.dtype), _to16(k, w.dtype), _to16(v, w.dtype)


def bits16(t: torch.Tensor) -> np.ndarray:
    """16-bit tensor -> numpy uint16 bit patterns (for the oracle)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def dtype_code(dtype: torch.dtype) -> int:
    """0 = bfloat16, 1 = float16 (the oracle's input dtype codes)."""
    return {torch.bfloat16: 0, torch.float16: 1}[dtype]
