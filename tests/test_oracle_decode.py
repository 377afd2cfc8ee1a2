"""Pins for the oracle's decode-shaped attention on an NVFP4 KV cache.

- The cache's values: a hand-built K row and V channel decode to E2M1 x UE4M3, low nibble
  first; V's along-token values agree with the rows quantizer's for on-grid inputs.
- Against torch's scaled_dot_product_attention in fp64 (a library routine) on the same
  dequantized values, with the bottom-right causal mask written out as a boolean mask.
- Closed forms: one key gives its V row; Q = 0 gives the mean of V over the visible keys
  (prefix means under causal masking); V rows all equal give that row.
"""
import numpy as np
import torch

import oracle
from bit_quantized_attention_03_amd import inputs as I


def _cache(x16, axis=0):
    c, s, _ = oracle.quant_nvfp4(x16, oracle.BF16, axis, 1)
    return c, s


def test_nvfp4_row_values_hand_example():
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 0] = 0x27          # element 0: code 7 (6.0); element 1: code 2 (1.0)
    codes[0, 8] = 0xF0          # element 16: 0; element 17: code 0xF (-6.0)
    scales = np.full((1, 8), 0x38, np.uint8)   # UE4M3 1.0
    scales[0, 1] = 0x40                         # 2.0 for elements 16..31
    v = oracle.nvfp4_rows_value(codes, scales)
    assert v[0, 0] == 6.0 and v[0, 1] == 1.0 and v[0, 16] == 0.0 and v[0, 17] == -12.0
    assert np.count_nonzero(v) == 3
    # along tokens: channel 0's tokens 0, 1 and channel 1's token 17
    vc = np.zeros((2, 32), np.uint8)            # D = 2 channels, Np = 64 tokens
    vc[0, 0] = 0x27
    vc[1, 8] = 0xF0
    vs = np.full((4, 2), 0x38, np.uint8)
    vs[1, 1] = 0x40                              # tokens 16..31 of channel 1: scale 2.0
    tv = oracle.nvfp4_tokens_value(vc, vs, 40)
    assert tv.shape == (40, 2)
    assert tv[0, 0] == 6.0 and tv[1, 0] == 1.0 and tv[17, 1] == -12.0 and np.count_nonzero(tv) == 3


def test_token_layout_values_match_row_layout_on_grid():
    """On-grid rows (each 16-block already a scale times E2M1 values, with the block max at 6 x
    scale along both axes) quantize exactly either way, so both layouts give the same values."""
    rng = np.random.default_rng(2)
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    v = rng.choice(e2m1, size=(1, 1, 64, 32)) * rng.choice([-1, 1], size=(1, 1, 64, 32))
    v[..., ::16, :] = 6.0                        # every 16-token group of every channel hits 6
    v[..., :, ::16] = 6.0                        # every 16-channel group of every row hits 6
    bf = lambda x: I.bits16(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
    c0, s0 = _cache(bf(v), 0)
    c1, s1 = _cache(bf(v), 1)
    assert np.array_equal(oracle.nvfp4_rows_value(c0, s0), v)
    assert np.array_equal(oracle.nvfp4_tokens_value(c1, s1, 64), v)


def _setup(B=1, Hq=4, Hkv=2, Nq=3, Nk=300, seed=0):
    rng = np.random.default_rng(seed)
    bf = lambda x: I.bits16(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
    q16 = bf(rng.standard_normal((B, Hq, Nq, 128)))
    k16 = bf(rng.standard_normal((B, Hkv, Nk, 128)))
    v16 = bf(rng.standard_normal((B, Hkv, Nk, 128)))
    return q16, _cache(k16), _cache(v16, 1)


def test_matches_library_sdpa():
    q16, (kc, ks), (vc, vs) = _setup()
    for causal in (False, True):
        got = oracle.decode_attention(q16, oracle.BF16, kc, ks, vc, vs, causal, 0.1)
        q = torch.from_numpy(oracle.decode16(q16, oracle.BF16).astype(np.float64))
        K = torch.from_numpy(oracle.nvfp4_rows_value(kc, ks)).repeat_interleave(2, dim=1)
        V = torch.from_numpy(oracle.nvfp4_tokens_value(vc, vs, K.shape[2])).repeat_interleave(2, dim=1)
        Nq, Nk = q.shape[2], K.shape[2]
        mask = (torch.arange(Nk)[None, :] <= (Nk - Nq + torch.arange(Nq))[:, None]) if causal else None
        want = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=0.1)
        assert np.allclose(got, want.numpy(), rtol=0, atol=1e-12)


def test_closed_forms():
    q16, (kc, ks), (vc, vs) = _setup(Nk=200)
    V = oracle.nvfp4_tokens_value(vc, vs, 200)
    # one key: a cache of one token (its V group padded with zero codes)
    vc1 = np.zeros_like(vc[..., :32]); vc1[..., 0] = vc[..., 0] & 15
    vs1 = vs[:, :, :4].copy()
    got = oracle.decode_attention(q16, oracle.BF16, kc[:, :, :1], ks[:, :, :1], vc1, vs1, False, 0.3)
    assert np.allclose(got, np.repeat(V[:, :, :1], 2, axis=1).repeat(3, axis=2), rtol=0, atol=1e-15)
    # Q = 0: uniform weights over the visible keys
    z = np.zeros_like(q16)
    got = oracle.decode_attention(z, oracle.BF16, kc, ks, vc, vs, True, 0.3)
    for i in range(3):
        n_vis = 200 - 3 + i + 1
        assert np.allclose(got[0, 0, i], V[0, 0, :n_vis].mean(axis=0), rtol=0, atol=1e-12)
    # all V rows equal: every token of a channel carries token 0's code and scale
    lo = vc[..., :1] & 15
    vce = np.broadcast_to(lo | (lo << 4), vc.shape).copy()
    vse = np.broadcast_to(vs[:, :, :1], vs.shape).copy()
    got = oracle.decode_attention(q16, oracle.BF16, kc, ks, vce, vse, False, 0.3)
    assert np.allclose(got, np.broadcast_to(np.repeat(V[:, :, :1], 2, axis=1), got.shape), rtol=0, atol=1e-12)
