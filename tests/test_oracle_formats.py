"""Pins for the oracle's number formats against brute force and library casts.

Each encoder is checked against an independent nearest-value search over the format's
enumerated value set (ties to the even code, saturation at the largest finite value), and
where a library cast exists (torch float8_e4m3fn / bfloat16, numpy float16) against it too.
"""
import math

import numpy as np
import pytest
import torch

import oracle

# ---------------------------------------------------------------- brute-force reference grids


def _e4m3_table():
    vals = []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue  # NaN
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append((c, -v if s else v))
    return vals


def _e2m1_table():
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    return [(c, -mags[c & 7] if c & 8 else mags[c & 7]) for c in range(16)]


def _nearest_code(x: np.ndarray, table, vmax: float) -> np.ndarray:
    """Nearest representable value (same sign), ties to the even code, saturating at vmax."""
    x = x.astype(np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), vmax)
    pos = [(c, v) for c, v in table if v >= 0 and not (c & (0x80 if vmax > 6 else 0x8))]
    codes = np.array([c for c, _ in pos]); vals = np.array([v for _, v in pos])
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = (d == best)
    # among tied candidates prefer the even code
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    out = codes[pick]
    signbit = 0x80 if vmax > 6 else 0x8
    return np.where(sign, out | signbit, out)


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


# ---------------------------------------------------------------- E4M3

def test_e4m3_exhaustive_over_bf16_vs_bruteforce():
    x = _all_bf16_values()
    got = oracle.e4m3_encode(x)
    want = _nearest_code(x, _e4m3_table(), 448.0)
    assert np.array_equal(got, want.astype(np.uint8))


def test_e4m3_vs_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * 10, rng.uniform(-448, 448, 200000),
                        rng.standard_normal(100000) * 1e-3, [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10]])
    x = x.astype(np.float32)
    ours = oracle.e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_decode_roundtrip_and_saturation():
    codes = np.array([c for c, _ in _e4m3_table()], np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), codes)
    assert oracle.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert oracle.e4m3_encode(np.array([1e9, -1e9, 465.0], np.float32)).tolist() == [0x7E, 0xFE, 0x7E]
    assert math.isnan(oracle.e4m3_decode(np.array([0x7F], np.uint8))[0])


# ---------------------------------------------------------------- E2M1

def test_e2m1_exhaustive_over_bf16_vs_bruteforce():
    x = _all_bf16_values()
    got = oracle.e2m1_encode(x)
    want = _nearest_code(x, _e2m1_table(), 6.0)
    assert np.array_equal(got, want.astype(np.uint8))


def test_e2m1_golden_ties():
    rows = [l.split() for l in open(__file__.replace("test_oracle_formats.py", "golden/e2m1_ties.txt"))
            if l.strip() and not l.startswith("#")]
    x = np.array([float(a) for a, _ in rows], np.float32)
    want = np.array([float(b) for _, b in rows])
    got = oracle.e2m1_decode(oracle.e2m1_encode(x))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


# ---------------------------------------------------------------- bf16 / fp16

def test_bf16_vs_torch_on_random_bit_patterns():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = oracle.bf16_encode(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(oracle.bf16_decode(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_f16_vs_numpy_on_random_values():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=500_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 1e6)]
    x = np.concatenate([x, (rng.standard_normal(500_000) * 3).astype(np.float32),
                        (rng.standard_normal(100_000) * 1e-6).astype(np.float32)])
    ours = oracle.f16_encode(x)
    with np.errstate(over="ignore"):   # |x| > 65504 overflows to inf on both sides
        theirs = x.astype(np.float16)
    assert np.array_equal(ours, theirs.view(np.uint16))
    assert np.array_equal(oracle.f16_decode(ours), theirs.astype(np.float32))


# ---------------------------------------------------------------- E8M0 exponent

@pytest.mark.parametrize("seed", [0, 1])
def test_mx_exponent_is_smallest_fitting(seed):
    rng = np.random.default_rng(seed)
    amax = np.concatenate([np.exp(rng.uniform(-20, 20, 2000)), [1.5, 3.0, 6.0, 6.0000001, 0.75, 12.0]])
    for a in amax:
        e = oracle.mx_exponent(a)
        assert 6.0 * 2.0 ** e >= a and 6.0 * 2.0 ** (e - 1) < a
        # closed form: amax = m * 2^k, m in [0.5, 1): e = k-3 if 6 * 2^(k-3) >= amax else k-2
        m, k = math.frexp(a)
        assert e == (k - 3 if 6.0 * 2.0 ** (k - 3) >= a else k - 2)
    assert oracle.mx_exponent(0.0) == -127
