"""HIP graph capture of the C-ABI calls (the launch-bound decode step and a whole INT8
pass): the library enqueues only kernels on the caller's stream (no memsets, no
allocations, no synchronisation), so a captured call replays.  Each replay gets new inputs
copied into the captured buffers, with eager work and synchronisation between replays, and
must equal the eager result bit for bit (every kernel sums in a fixed order)."""
import pytest
import torch

from bit_quantized_attention_03_amd import inputs as I

pytestmark = pytest.mark.gpu


def _sage():
    from bit_quantized_attention_03_amd import sage
    return sage


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph; returns (graph, output)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


def test_decode_graph_replays_match_eager():
    sage = _sage()
    w = I.workload("decode_nvfp4", B=2, Hq=8, Hkv=2, N=3000, Nq=2)
    q0, k, v = I.make_qkv(w, seed=21)
    kq = sage.quantize(k.cuda(), sage.NVFP4, (1, 16), sage.SEARCH)
    vq = sage.quantize(v.cuda(), sage.NVFP4, (16, 1), sage.SEARCH)
    static_q = q0.cuda()
    g, out = _capture(lambda: sage.decode(static_q, kq, vq, True))
    for seed in (22, 23, 24):
        print(f"[case] decode graph replay seed={seed}", flush=True)
        qn = I.make_qkv(w, seed=seed)[0].cuda()
        want = sage.decode(qn, kq, vq, True)          # eager, between replays
        torch.cuda.synchronize()
        static_q.copy_(qn)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want)


def test_int8_pass_graph_replays_match_eager():
    sage = _sage()
    w = I.workload("llm_int8", B=1, Hq=2, Hkv=2, N=700)
    q0, k0, v0 = (t.cuda() for t in I.make_qkv(w, seed=31))
    sq, sk, sv = q0.clone(), k0.clone(), v0.clone()
    g, res = _capture(lambda: sage.forward(sq, sk, sv, causal=True, variant="int8"))
    for seed in (32, 33, 34):
        print(f"[case] int8 pass graph replay seed={seed}", flush=True)
        qn, kn, vn = (t.cuda() for t in I.make_qkv(w, seed=seed))
        want = sage.forward(qn, kn, vn, causal=True, variant="int8")
        torch.cuda.synchronize()
        sq.copy_(qn); sk.copy_(kn); sv.copy_(vn)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(res.out, want.out)
        assert torch.equal(res.mean, want.mean)
