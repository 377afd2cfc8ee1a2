"""Pins for the oracle's tiled attention mirror.

- the fp64 textbook reference equals torch's scaled_dot_product_attention in fp64;
- the tiled online-softmax mirror with every format set to exact passthrough equals it;
- the dequantize-then-attend identity for INT8, MX-FP4 and FP8-V operands;
- closed forms: Q = 0 gives the (prefix) mean of V for every P format; causal row 0 gives V[0];
  V = 1 gives rows that sum to one; GQA equals MHA with repeated K/V.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_attention_03_amd import inputs as I


def _val(h, dt=oracle.BF16):
    return oracle.decode16(h, dt).astype(np.float64)


def _bf16(x):
    return I.bits16(torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16))


def _hi_ops(q16, k16, v16, p_fmt=oracle.P_EXACT):
    return oracle.AttnOperands(qk_fmt=oracle.QK_HI, p_fmt=p_fmt, v_fmt=oracle.V_HI, q_hi=q16, k_hi=k16, v_hi=v16)


@pytest.mark.parametrize("causal", [False, True])
def test_reference_matches_torch_sdpa(causal):
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((2, 4, 70, 16)) for _ in range(3))
    ours = oracle.attention_ref(q, k, v, causal, 0.25)
    t = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                                         is_causal=causal, scale=0.25)
    assert np.max(np.abs(ours - t.numpy())) < 1e-13


@pytest.mark.parametrize("N", [200, 256, 100])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_passthrough_equals_reference(N, causal):
    w = I.workload("llm_int8", B=1, Hq=2, Hkv=2, N=N, D=32)
    q, k, v = I.make_qkv(w, 3)
    qb, kb, vb = I.bits16(q), I.bits16(k), I.bits16(v)
    sm = 1 / math.sqrt(32)
    out = oracle.attention(_hi_ops(qb, kb, vb), 1, 2, 2, N, 32, causal, sm)
    ref = oracle.attention_ref(_val(qb), _val(kb), _val(vb), causal, sm)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("causal", [False, True])
def test_int8_scores_are_dequantized_products(causal):
    w = I.workload("llm_int8", B=1, Hq=2, Hkv=2, N=192, D=64)
    q, k, v = I.make_qkv(w, 4)
    qb, kb, vb = I.bits16(q), I.bits16(k), I.bits16(v)
    qc, qs = oracle.quant_int8(qb, oracle.BF16, 128)
    kc, ks = oracle.quant_int8(kb, oracle.BF16, 64)
    ops = oracle.AttnOperands(qk_fmt=oracle.QK_INT8, p_fmt=oracle.P_EXACT, v_fmt=oracle.V_HI,
                              q_i8=qc, q_s=qs, k_i8=kc, k_s=ks, v_hi=vb)
    sm = 0.125
    out = oracle.attention(ops, 1, 2, 2, 192, 64, causal, sm)
    qd = qc * np.repeat(qs, 128, axis=2)[:, :, :192, None].astype(np.float64)
    kd = kc * np.repeat(ks, 64, axis=2)[:, :, :192, None].astype(np.float64)
    ref = oracle.attention_ref(qd, kd, _val(vb), causal, sm)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_mxfp4_and_fp8_operands_are_dequantized_products():
    w = I.workload("fp4_search", B=1, Hq=1, Hkv=1, N=160, D=64)
    q, k, v = I.make_qkv(w, 5)
    qb, kb, vb = I.bits16(q), I.bits16(k), I.bits16(v)
    qc, qe = oracle.quant_mxfp4(qb, oracle.BF16, 0)
    kc, ke = oracle.quant_mxfp4(kb, oracle.BF16, 0)
    vc, vs = oracle.quant_fp8_channel(vb, oracle.BF16)

    def dq(c, e):
        lo = oracle.e2m1_decode(c & 15); hi = oracle.e2m1_decode(c >> 4)
        d = np.stack([lo, hi], -1).reshape(c.shape[:-1] + (-1, 32))
        return (d * (2.0 ** (e.astype(np.int64) - 127))[..., None]).reshape(c.shape[:-1] + (-1,))

    ops = oracle.AttnOperands(qk_fmt=oracle.QK_MXFP4, p_fmt=oracle.P_EXACT, v_fmt=oracle.V_E4M3,
                              q_lp=qc, q_e8=qe, k_lp=kc, k_e8=ke, v_lp=vc, v_s=vs)
    out = oracle.attention(ops, 1, 1, 1, 160, 64, False, 0.125)
    vd = np.swapaxes(oracle.e4m3_decode(vc[..., :160]) * vs[..., None], 2, 3)
    ref = oracle.attention_ref(dq(qc, qe), dq(kc, ke), vd, False, 0.125)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


PFMTS = [oracle.P_BF16, oracle.P_E4M3, oracle.P_MXFP4, oracle.P_NVFP4_MXFP8]


@pytest.mark.parametrize("p_fmt", PFMTS)
@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_v(p_fmt, causal):
    # Q = 0: scores are 0, Ptilde = 1 exactly, and every P format represents 1 exactly,
    # so row i is the mean of V over the keys it may see.
    N, D = 200, 64
    w = I.workload("llm_int8", B=1, Hq=1, Hkv=1, N=N, D=D)
    _, k, v = I.make_qkv(w, 6)
    zq = np.zeros((1, 1, N, D), np.uint16)
    qc, qs = oracle.quant_int8(zq, oracle.BF16, 128)
    kc, ks = oracle.quant_int8(I.bits16(k), oracle.BF16, 64)
    assert np.all(qs == 0) and np.all(qc == 0)
    vb = I.bits16(v)
    ops = oracle.AttnOperands(qk_fmt=oracle.QK_INT8, p_fmt=p_fmt, v_fmt=oracle.V_HI,
                              q_i8=qc, q_s=qs, k_i8=kc, k_s=ks, v_hi=vb)
    out = oracle.attention(ops, 1, 1, 1, N, D, causal, 0.125)
    vv = _val(vb)[0, 0]
    want = np.cumsum(vv, 0) / np.arange(1, N + 1)[:, None] if causal else np.broadcast_to(vv.mean(0), (N, D))
    assert np.max(np.abs(out[0, 0] - want)) <= 1e-12


@pytest.mark.parametrize("p_fmt", PFMTS)
def test_causal_row0_is_v0(p_fmt):
    w = I.workload("llm_int8", B=1, Hq=1, Hkv=1, N=130, D=64)
    q, k, v = I.make_qkv(w, 7)
    qc, qs = oracle.quant_int8(I.bits16(q), oracle.BF16, 128)
    kc, ks = oracle.quant_int8(I.bits16(k), oracle.BF16, 64)
    vb = I.bits16(v)
    ops = oracle.AttnOperands(qk_fmt=oracle.QK_INT8, p_fmt=p_fmt, v_fmt=oracle.V_HI,
                              q_i8=qc, q_s=qs, k_i8=kc, k_s=ks, v_hi=vb)
    out = oracle.attention(ops, 1, 1, 1, 130, 64, True, 0.125)
    assert np.array_equal(out[0, 0, 0], _val(vb)[0, 0, 0])


def test_rows_sum_to_one():
    # V = 1: O = (sum of Phat) / l.  Exact P: 1 to rounding; bf16 P: within bf16's half-step.
    w = I.workload("llm_int8", B=1, Hq=2, Hkv=2, N=192, D=64)
    q, k, _ = I.make_qkv(w, 8)
    ones = _bf16(np.ones((1, 2, 192, 64)))
    for p_fmt, tol in ((oracle.P_EXACT, 1e-12), (oracle.P_BF16, 2.0 ** -8)):
        for causal in (False, True):
            out = oracle.attention(_hi_ops(I.bits16(q), I.bits16(k), ones, p_fmt), 1, 2, 2, 192, 64, causal, 0.125)
            assert np.max(np.abs(out - 1.0)) <= tol


def test_gqa_equals_repeated_kv():
    w = I.workload("thrift_long", B=1, Hq=4, Hkv=2, N=160, D=64)
    q, k, v = I.make_qkv(w, 9)
    qc, qs = oracle.quant_int8(I.bits16(q), oracle.BF16, 128)
    kc, ks = oracle.quant_int8(I.bits16(k), oracle.BF16, 64)
    vb = I.bits16(v)
    ops = oracle.AttnOperands(qk_fmt=oracle.QK_INT8, p_fmt=oracle.P_BF16, v_fmt=oracle.V_HI,
                              q_i8=qc, q_s=qs, k_i8=kc, k_s=ks, v_hi=vb)
    gqa = oracle.attention(ops, 1, 4, 2, 160, 64, True, 0.125)
    rep = lambda a: np.repeat(a, 2, axis=1)
    ops2 = oracle.AttnOperands(qk_fmt=oracle.QK_INT8, p_fmt=oracle.P_BF16, v_fmt=oracle.V_HI,
                               q_i8=qc, q_s=qs, k_i8=rep(kc), k_s=rep(ks), v_hi=rep(vb))
    mha = oracle.attention(ops2, 1, 4, 4, 160, 64, True, 0.125)
    assert np.array_equal(gqa, mha)


def test_subset_matches_full_run():
    w = I.workload("llm_int8", B=2, Hq=2, Hkv=2, N=384, D=64)
    q, k, v = I.make_qkv(w, 10)
    ops = _hi_ops(I.bits16(q), I.bits16(k), I.bits16(v), oracle.P_BF16)
    full = oracle.attention(ops, 2, 2, 2, 384, 64, True, 0.125)
    part = oracle.attention(ops, 2, 2, 2, 384, 64, True, 0.125, bh=(1, 3), qb=(1, 3))
    assert np.array_equal(part[0, 1, 128:], full[0, 1, 128:])
    assert np.isnan(part[0, 0]).all() and np.isnan(part[0, 1, :128]).all()
