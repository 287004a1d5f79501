"""Pins of the oracle's number formats and its exp against things other than itself.

Storage formats are the ones the pages name ("DeepSeek-V4: a million-token
context that agents can actually use", storage paragraph: FP8 KV entries,
BF16 RoPE dims, FP4 indexer); the exact variants (OCP E4M3FN, bfloat16,
OCP MX E2M1 with E8M0 block scales) are the readings stated in the oracle.
Each check below uses an independent route: torch's own casts, exhaustive
nearest-value search over the format's value set, exact rational
arithmetic, or libm.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch


def _fp8_values():
    """All finite E4M3FN values via torch's own decode (library routine)."""
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    return codes


def test_fp8_decode_matches_torch_all_codes(oracle):
    ref = _fp8_values()
    for c in range(256):
        d = oracle.fp8_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(d), c
        else:
            assert d == ref[c] and math.copysign(1, d) == math.copysign(1, ref[c]), (c, d, ref[c])
    assert oracle.fp8_decode(0x7E) == 448.0
    assert oracle.fp8_decode(0x01) == 2.0 ** -9


def test_fp8_roundtrip_every_finite_code(oracle):
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.fp8_encode(oracle.fp8_decode(c)) == c, hex(c)


def test_fp8_encode_matches_torch_random_and_ties(oracle):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(30.0),
        rng.standard_normal(5000).astype(np.float32) * np.float32(0.01),
        (rng.random(5000) * 463.0).astype(np.float32),
    ])
    # every midpoint between neighbouring positive values (ties to even)
    vals = sorted(set(v for v in _fp8_values() if not math.isnan(v) and v >= 0))
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    x = np.concatenate([x, np.array(mids, np.float32), -np.array(mids, np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_encode(float(v)) for v in x], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_fp8_encode_is_nearest_value_bruteforce(oracle):
    """Independent formulation: nearest value of the finite set, ties to even code; saturating."""
    vals = _fp8_values()
    finite = [(c, v) for c, v in enumerate(vals) if not math.isnan(v) and c < 128]
    rng = np.random.default_rng(2)
    for v in list(rng.standard_normal(3000) * 40.0) + [449.0, 1e6, 463.99, 464.0, 1e-300]:
        a = abs(v)
        best = min(finite, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
        code = best[0] if a < 448 else 0x7E
        code |= 0x80 if v < 0 else 0
        assert oracle.fp8_encode(v) == code, v


def _bf16_rne_fraction(v: float) -> float:
    """Exact RNE of a double to 8 significant bits by rational arithmetic."""
    if v == 0:
        return v
    a = Fraction(abs(v))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    n = a / q
    f = n.numerator // n.denominator
    r = n - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return math.copysign(float(f * q), v)


def test_bf16_encode_matches_torch_on_fp32_values(oracle):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 2 ** -130, -(2 ** -140)], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_encode(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_encode_from_fp64_rounds_once(oracle):
    """Values that fp32 cannot hold: direct RNE from fp64, no double rounding."""
    rng = np.random.default_rng(4)
    xs = list(rng.standard_normal(5000)) + [1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8 - 2 ** -40, 1 + 2 ** -8 + 2 ** -30]
    for v in xs:
        got = oracle.bf16_decode(oracle.bf16_encode(v))
        assert got == _bf16_rne_fraction(v), v
    # a double just above a bf16 midpoint whose fp32 rounding would land exactly on the midpoint
    v = 1 + 2 ** -8 + 2 ** -40
    assert oracle.bf16_encode(v) == 0x3F81


E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX v1.0 FP4 E2M1 magnitudes


def test_fp4_table_and_nearest_even(oracle):
    for c in range(16):
        v = oracle.fp4_decode(c)
        assert abs(v) == E2M1[c & 7] and (c < 8 or v <= 0)
    rng = np.random.default_rng(5)
    for v in list(rng.uniform(-9, 9, 4000)) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 6.5, 100.0]:
        a = abs(v)
        best = min(range(8), key=lambda c: (abs(E2M1[c] - a), c & 1))
        code = (best if a < 6 else 7) | (8 if v < 0 else 0)
        assert oracle.fp4_encode(v) == code, v
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, r in ties.items():
        assert oracle.fp4_decode(oracle.fp4_encode(v)) == r


def test_mxfp4_block_scale_rule(oracle):
    rng = np.random.default_rng(6)
    for trial in range(300):
        x = rng.standard_normal(64) * (10.0 ** rng.uniform(-6, 6))
        if trial % 17 == 0:
            x[:32] = 0.0
        codes, scales = oracle.mxfp4_quant(x)
        for b in range(2):
            blk = x[32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                assert scales[b] == 0 and not codes[32 * b:32 * b + 32].any()
                continue
            e = math.frexp(amax)[1] - 1          # floor(log2 amax)
            E = min(max(e - 2, -127), 127)
            assert scales[b] == E + 127
            for i in range(32):
                v = blk[i] * 2.0 ** -E
                a = abs(v)
                best = min(range(8), key=lambda c: (abs(E2M1[c] - a), c & 1))
                code = (best if a < 6 else 7) | (8 if v < 0 else 0)
                assert codes[32 * b + i] == code


def test_exp_constants_from_ln2():
    import oracle as O
    c = O.exp_consts()
    getcontext().prec = 80
    ln2 = Fraction(str(Decimal(2).ln()))
    assert c[0] == float(1 / ln2)
    hi, lo = Fraction(c[1]), Fraction(c[2])
    # head has at most 32 significant bits, so n * LN2_HI is exact for |n| < 2^21
    m, e = math.frexp(c[1])
    assert float(m * 2 ** 32).is_integer()
    assert abs(hi + lo - ln2) < Fraction(1, 2 ** 85)
    for i in range(14):
        assert c[3 + i] == float(Fraction(1, math.factorial(i)))


def test_exp_det_within_two_ulp_of_libm(oracle):
    rng = np.random.default_rng(7)
    xs = np.concatenate([-rng.random(200000) * 700.0, -rng.random(50000) * 2.0, [0.0, -1e-300, -700.0, -699.9]])
    worst = 0
    for x in xs[::5]:
        a = oracle.exp_det(float(x))
        b = math.exp(float(x))
        ulp = math.ulp(b)
        worst = max(worst, abs(a - b) / ulp)
    assert worst <= 2.0, worst
    assert oracle.exp_det(0.0) == 1.0
    assert oracle.exp_det(-701.0) == 0.0


def test_exp_det_against_high_precision(oracle):
    getcontext().prec = 60
    rng = np.random.default_rng(8)
    for x in -rng.random(300) * 50.0:
        exact = Decimal(float(x)).exp()
        a = oracle.exp_det(float(x))
        assert abs(Decimal(a) - exact) <= Decimal(math.ulp(a)) * 2
