"""Strided operands at the boundary: every entry point that reads 16-bit tensors by rows (and
the attention output) takes a model's [B, N, H, D] tensors as [B, H, N, D] views, with no
copy.  The kernels do the same arithmetic whatever the layout, so each result must equal,
bit for bit, the result on contiguous copies of the same values."""
import pytest
import torch

from bit_quantized_attention_03_amd import inputs as I

pytestmark = pytest.mark.gpu


def _sage():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from bit_quantized_attention_03_amd import sage
    sage.lib()
    return sage


def bnhd_view(x: torch.Tensor) -> torch.Tensor:
    """The same values held as [B, N, H, D] in memory, seen as a [B, H, N, D] view."""
    v = x.transpose(1, 2).contiguous().transpose(1, 2)
    assert not v.is_contiguous() and v.stride(3) == 1
    return v


def padded_view(x: torch.Tensor, pad: int = 8) -> torch.Tensor:
    """The same values in rows of D + pad elements (a row stride that is not D)."""
    B, H, N, D = x.shape
    buf = torch.zeros((B, H, N, D + pad), dtype=x.dtype, device=x.device)
    buf[..., :D] = x
    return buf[..., :D]


def _qkv(name, seed=0, **ov):
    w = I.workload(name, **ov)
    return w, [t.cuda() for t in I.make_qkv(w, seed=seed)]


def _same(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(a.contiguous().view(torch.uint8) if a.dtype != torch.uint8 else a.contiguous(),
                       b.contiguous().view(torch.uint8) if b.dtype != torch.uint8 else b.contiguous()), what


@pytest.mark.parametrize("make_view", [bnhd_view, padded_view])
def test_smoothing_and_quantizers_on_views(make_view):
    sage = _sage()
    print(f"[case] quantizers on {make_view.__name__}", flush=True)
    w, (q, k, v) = _qkv("llm_int8", B=2, Hq=4, Hkv=2, N=333)
    D = w.D
    qv, kv, vv = make_view(q), make_view(k), make_view(v)
    m0, ks0 = sage.smooth_k(k)
    m1, ks1 = sage.smooth_k(kv)
    _same(m0, m1, "smoothing mean")
    _same(ks0, ks1, "K_s")
    assert ks1.is_contiguous()
    for name, fn in (
        ("int8 Q", lambda x: sage.quantize(x, sage.INT8, (128, D))),
        ("int8 Q hadamard", lambda x: sage.quantize(x, sage.INT8, (128, D), hadamard=True)),
        ("mxfp4 rows", lambda x: sage.quantize(x, sage.MXFP4, (1, 32))),
        ("nvfp4 rows search", lambda x: sage.quantize(x, sage.NVFP4, (1, 16), sage.SEARCH)),
        ("mxfp4 cols", lambda x: sage.quantize(x, sage.MXFP4, (32, 1))),
        ("nvfp4 cols search", lambda x: sage.quantize(x, sage.NVFP4, (16, 1), sage.SEARCH)),
        ("e4m3 channel", lambda x: sage.quantize(x, sage.E4M3, (0, 1))),
    ):
        a, b = fn(q), fn(qv)
        _same(a.codes, b.codes, name + " codes")
        _same(a.scales, b.scales, name + " scales")
    a = sage.quantize_smoothed(k, m0, sage.INT8, (64, D))
    b = sage.quantize_smoothed(kv, m0, sage.INT8, (64, D))
    _same(a.codes, b.codes, "int8 K smoothed codes")
    _same(a.scales, b.scales, "int8 K smoothed scales")
    # a model's long INT8 block (T * D beyond the one-pass kernel) takes the two-pass kernel
    a, b = sage.quantize(v, sage.INT8, (512, D)), sage.quantize(vv, sage.INT8, (512, D))
    _same(a.codes, b.codes, "int8 two-pass codes")


@pytest.mark.parametrize("name,ov,causal,variant", [
    ("llm_int8", dict(B=2, Hq=4, Hkv=2, N=333), False, "int8"),
    ("llm_int8", dict(B=1, Hq=4, Hkv=4, N=700), True, "int8"),
    ("tiny_int8", {}, True, "int8"),                                        # D = 64, fp16
    ("thrift_long", dict(B=1, Hq=4, Hkv=2, N=1100), True, "thrift"),
    ("thrift_long", dict(B=1, Hq=2, Hkv=2, N=640), False, "sink"),
    ("fp4_search", dict(B=1, Hq=4, Hkv=2, N=333), False, "mxfp4"),
    ("fp4_search", dict(B=1, Hq=2, Hkv=2, N=512), True, "nvfp4_search"),
])
def test_attention_with_strided_v_and_output(name, ov, causal, variant):
    """V (when 16-bit), the Thrift tiles' Q and the output as [B, N, H, D] views."""
    sage = _sage()
    import bench
    print(f"[case] strided attention {name} {ov} causal={causal} {variant}", flush=True)
    w, (q, k, v) = _qkv(name, **ov)
    B, Hq, N, D = q.shape
    qq, kq, vq, pf, mask, ks = bench.prepare(sage, variant, q, k, v, causal)
    want = sage.attn_fwd(qq, kq, vq, causal, pf, block_mask=mask,
                         q_hi=q if mask is not None else None, k_hi=ks if mask is not None else None)
    if vq.fmt in (sage.BF16, sage.FP16):
        vq = sage.QT(vq.fmt, bnhd_view(v), None, tuple(v.shape))
    out_mem = torch.full((B, N, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    out = out_mem.transpose(1, 2)
    got = sage.attn_fwd(qq, kq, vq, causal, pf, block_mask=mask,
                        q_hi=bnhd_view(q) if mask is not None else None, k_hi=ks if mask is not None else None,
                        out=out)
    assert got.data_ptr() == out_mem.data_ptr()
    _same(want, out, f"{variant} output")
    # bf16 output into a padded-row view
    want16 = sage.attn_fwd(qq, kq, vq, causal, pf, block_mask=mask,
                           q_hi=q if mask is not None else None, k_hi=ks if mask is not None else None,
                           out_dtype=torch.bfloat16)
    out16 = padded_view(torch.zeros((B, Hq, N, D), dtype=torch.bfloat16, device="cuda"))
    sage.attn_fwd(qq, kq, vq, causal, pf, block_mask=mask,
                  q_hi=q if mask is not None else None, k_hi=ks if mask is not None else None, out=out16)
    _same(want16, out16, f"{variant} bf16 output")


def test_fp16_v_at_d128_strided():
    """fp16 V at D = 128 runs on the other INT8 kernel: its V rows are strided too."""
    sage = _sage()
    print("[case] fp16 V, D=128, strided", flush=True)
    w, (q, k, v) = _qkv("llm_int8", B=1, Hq=2, Hkv=2, N=300)
    q, k, v = q.half(), k.half(), v.half()
    D = w.D
    mean, _ = sage.smooth_k(k, want_smoothed=False)
    qq = sage.quantize(q, sage.INT8, (128, D))
    kq = sage.quantize_smoothed(k, mean, sage.INT8, (64, D))
    want = sage.attn_fwd(qq, kq, sage.QT(sage.FP16, v, None, tuple(v.shape)), True, sage.BF16)
    got = sage.attn_fwd(qq, kq, sage.QT(sage.FP16, padded_view(v), None, tuple(v.shape)), True, sage.BF16)
    _same(want, got, "fp16 V output")


def test_thrift_selection_and_decode_on_views():
    sage = _sage()
    print("[case] thrift_select and decode on views", flush=True)
    w, (q, k, v) = _qkv("thrift_long", B=1, Hq=4, Hkv=2, N=777)
    _, ks = sage.smooth_k(k)
    a = sage.thrift_select(q, ks, 0.05, True)
    b = sage.thrift_select(bnhd_view(q), bnhd_view(ks), 0.05, True)
    _same(a, b, "thrift mask")
    wd, (qd, kd, vd) = _qkv("decode_nvfp4", B=2, Hq=8, Hkv=2, N=1000, Nq=3)
    kq = sage.quantize(kd, sage.NVFP4, (1, 16), sage.SEARCH)
    vq = sage.quantize(vd, sage.NVFP4, (16, 1), sage.SEARCH)
    a = sage.decode(qd, kq, vq, True)
    b = sage.decode(bnhd_view(qd), kq, vq, True)
    _same(a, b, "decode output")
    out = torch.empty_like(a)
    sage.decode_noalloc(padded_view(qd), kq, vq, out, True)
    _same(a, out, "decode (no-alloc) output")
