"""Pins of the unfused-comparator oracle: exact rationals, agreement with
the fused oracle where no intermediate rounding happens, and a hand-worked
case where the stored AllReduce result rounds."""

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synthetic import f32_to_bf16_bits, integer_scaled_inputs


def _val(bits):
    return Fraction(float(oracle.bf16_bits_to_f64(np.array([bits], np.uint16))[0]))


def _rne_bf16_fraction(v: Fraction) -> Fraction:
    """Nearest bf16 of a positive or negative rational in the normal range,
    ties to even, from the definition (8 significant bits)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a))
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (e - 7)                 # spacing in [2^e, 2^(e+1))
    k = a / q
    fl = math.floor(k)
    r = k - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def test_unfused_oracle_exact_rational_bruteforce():
    getcontext().prec = 50
    rng = np.random.default_rng(2)
    N, T, h = 3, 3, 8
    parts = f32_to_bf16_bits(rng.standard_normal((N, T, h)).astype(np.float32))
    res = f32_to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    w = f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(h)).astype(np.float32))
    eps = 1e-5
    y, x, red = oracle.unfused_reduce_rmsnorm(list(parts), res, w, eps, "bf16")
    e32 = Fraction(float(np.float32(eps)))
    for t in range(T):
        red_q = [_rne_bf16_fraction(sum(_val(parts[i, t, j]) for i in range(N))) for j in range(h)]
        assert [_val(b) for b in red[t]] == red_q
        xq = [red_q[j] + _val(res[t, j]) for j in range(h)]
        q = sum(v * v for v in xq) / h + e32
        rs = 1 / (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()
        for j in range(h):
            st = _rne_bf16_fraction(xq[j])
            want = (Decimal(st.numerator) / Decimal(st.denominator)) * rs * \
                (Decimal(_val(w[j]).numerator) / Decimal(_val(w[j]).denominator))
            assert y[t, j] == pytest.approx(float(want), rel=1e-14)
            assert Fraction(float(x[t, j])) == xq[j]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unfused_equals_fused_when_nothing_rounds(dtype):
    # k/16 values with |k| <= 8: every partial sum and x is exact in bf16 and
    # float32 (|x| <= 4.5 needs at most 7 significant bits at spacing 1/16).
    d = integer_scaled_inputs(4, 6, 64, dtype, kmax=8, seed=9)
    d_fused = oracle.fused_reduce_rmsnorm(list(d["partials"]), d["residual"], d["weight"], 1e-5, dtype)
    y_u, x_u, _ = oracle.unfused_reduce_rmsnorm(list(d["partials"]), d["residual"], d["weight"], 1e-5, dtype)
    np.testing.assert_array_equal(y_u, d_fused[0])
    np.testing.assert_array_equal(x_u, d_fused[1])


def test_stored_reduction_rounds_before_the_residual_is_added():
    # bf16: P0 = 1, P1 = 2^-8 -> the reduced value 1 + 2^-8 is a tie and rounds
    # to the even 1.0; adding R = 2^-8 then gives x = 1 + 2^-8 (fused: 1 + 2^-7).
    h = 8
    parts = np.zeros((2, 1, h), np.float32)
    parts[0, 0, 0] = 1.0
    parts[1, 0, 0] = 2.0 ** -8
    res = np.zeros((1, h), np.float32)
    res[0, 0] = 2.0 ** -8
    pb, rb, wb = f32_to_bf16_bits(parts), f32_to_bf16_bits(res), f32_to_bf16_bits(np.ones(h, np.float32))
    y, x, red = oracle.unfused_reduce_rmsnorm(list(pb), rb, wb, 0.0, "bf16")
    assert red[0, 0] == 0x3F80                       # 1.0
    assert x[0, 0] == 1.0 + 2.0 ** -8
    rs = 1.0 / math.sqrt((1.0 + 2.0 ** -8) ** 2 / h)
    assert y[0, 0] == pytest.approx(1.0 * rs, rel=1e-15)   # scales the stored 1.0 (tie to even)
    yf, xf, _ = oracle.fused_reduce_rmsnorm(list(pb), rb, wb, 0.0, "bf16")
    assert xf[0, 0] == 1.0 + 2.0 ** -7
