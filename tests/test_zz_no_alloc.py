"""The allocation-free decode entry point (sage_decode_fwd_noalloc) against sage_decode_fwd.

Both run the same split and combine kernels; only where the split partials live differs (a
caller workspace, or the library's per-GPU scratch array), so outputs must be bit-identical.
Two no-alloc calls run back to back, the second on a smaller problem, so the second starts
with the first one's partials still in the scratch."""
import pytest
import torch

from bit_quantized_attention_03_amd import inputs as I

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Nq, Nk, causal): the second problem is the smaller one
CASES = [(2, 16, 4, 3, 3000, True), (1, 4, 1, 1, 700, False)]


def _sage():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from bit_quantized_attention_03_amd import sage
    sage.lib()
    return sage


def _problem(sage, B, Hq, Hkv, Nq, Nk, seed):
    w = I.workload("decode_nvfp4", B=B, Hq=Hq, Hkv=Hkv, N=Nk, Nq=Nq)
    q, k, v = (t.cuda() for t in I.make_qkv(w, seed=seed))
    kq = sage.quantize(k, sage.NVFP4, (1, 16), sage.SEARCH)
    vq = sage.quantize(v, sage.NVFP4, (16, 1), sage.SEARCH)
    return q, kq, vq


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_decode_matches_workspace_decode(out_dtype):
    sage = _sage()
    lib = sage.lib()
    probs, wants, outs = [], [], []
    for i, (B, Hq, Hkv, Nq, Nk, causal) in enumerate(CASES):
        q, kq, vq = _problem(sage, B, Hq, Hkv, Nq, Nk, seed=11 + i)
        need = lib.sage_decode_workspace_bytes(sage.Shape(B, Hq, Nq, 128), sage.Shape(B, Hkv, Nk, 128))
        assert 0 < need <= sage.DECODE_NOALLOC_SCRATCH_BYTES
        probs.append((q, kq, vq, causal, need))
        wants.append(sage.decode(q, kq, vq, causal, out_dtype=out_dtype))
        outs.append(torch.full((B, Hq, Nq, 128), float("nan"), dtype=out_dtype, device="cuda"))
    assert probs[1][4] < probs[0][4]
    torch.cuda.synchronize()
    for (q, kq, vq, causal, _), out, case in zip(probs, outs, CASES):   # back to back, nothing between
        print(f"[case] decode_noalloc B,Hq,Hkv,Nq,Nk,causal={case} out={out_dtype}", flush=True)
        sage.decode_noalloc(q, kq, vq, out, causal)
    torch.cuda.synchronize()
    for want, out, case in zip(wants, outs, CASES):
        assert torch.equal(out, want), case


def test_noalloc_decode_long_cache_many_splits():
    """A long cache with one KV head: 1025 key splits, whose partials fill about 1 MiB of the
    scratch; outputs stay bit-identical to the workspace call."""
    sage = _sage()
    B, Hq, Hkv, Nq, Nk = 1, 2, 1, 1, (1 << 19) + 77
    print(f"[case] decode_noalloc many splits B,Hq,Hkv,Nq,Nk={B, Hq, Hkv, Nq, Nk}", flush=True)
    q, kq, vq = _problem(sage, B, Hq, Hkv, Nq, Nk, seed=5)
    want = sage.decode(q, kq, vq, True)
    out = torch.full_like(want, float("nan"))
    sage.decode_noalloc(q, kq, vq, out, True)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
