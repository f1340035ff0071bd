"""Pins of the fp64 oracle of the fused reduce + residual-add + RMSNorm step.

Each test checks the oracle against something other than itself: exact
rational arithmetic, closed forms, a library special case, exact
bit-pattern enumeration, and invariants that the mathematics fixes.  Chosen so
that a dropped term (partial, residual, eps, weight), a wrong sign, index or
operand order, a sum instead of a mean, or a double rounding fails one of
them.
"""

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synthetic import integer_scaled_inputs, make_inputs, special_rows_inputs


# ---------------------------------------------------------------- helpers ----

def _bf16_value_exact(bits: int) -> Fraction:
    """Value of a finite bf16 bit pattern, from its fields."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        v = Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    else:
        v = (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))
    return sign * v


_POS_BF16 = None


def _positive_bf16_table():
    global _POS_BF16
    if _POS_BF16 is None:
        _POS_BF16 = [_bf16_value_exact(b) for b in range(0x7F80)]   # 0 .. max finite
    return _POS_BF16


def _rne_bf16_bruteforce(v: float) -> int:
    """Nearest bf16 by bisection over every finite bf16 value; ties to even."""
    import bisect
    if math.isnan(v):
        return 0x7FC0 | (0x8000 if math.copysign(1, v) < 0 else 0)
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    if math.isinf(v):
        return sign | 0x7F80
    a = abs(Fraction(v))
    tab = _positive_bf16_table()
    top = tab[-1]
    ulp_top = top - tab[-2]
    if a >= top + ulp_top / 2:          # tie at the top rounds to the even 2**128
        return sign | 0x7F80
    i = bisect.bisect_left(tab, a)
    if i < len(tab) and tab[i] == a:
        return sign | i
    lo, hi = i - 1, i
    if hi >= len(tab):
        return sign | lo
    dl, dh = a - tab[lo], tab[hi] - a
    if dl < dh:
        return sign | lo
    if dh < dl:
        return sign | hi
    return sign | (lo if lo % 2 == 0 else hi)


def _exact_row_reference(parts, res, w, eps32, dtype):
    """Brute force in exact rationals (sum and mean of squares) and 50-digit
    decimals (square root), element by element in pure Python."""
    getcontext().prec = 50
    widen = (lambda b: _bf16_value_exact(int(b))) if dtype == "bf16" else (lambda f: Fraction(float(f)))
    N, T, h = parts.shape
    eps = Fraction(float(np.float32(eps32)))
    ys, xs = [], []
    for t in range(T):
        x = [sum((widen(parts[i, t, j]) for i in range(N)), Fraction(0)) + widen(res[t, j])
             for j in range(h)]
        ms = sum((v * v for v in x), Fraction(0)) / h
        q = ms + eps
        rs = 1 / (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()
        y = [(Decimal(v.numerator) / Decimal(v.denominator)) * rs
             * (Decimal(widen(w[j]).numerator) / Decimal(widen(w[j]).denominator))
             for j, v in enumerate(x)]
        xs.append([float(v) for v in x])
        ys.append([float(v) for v in y])
    return np.array(ys), np.array(xs)


# ---------------------------------------------------- widening / rounding ----

def test_bf16_widening_exact_for_every_pattern():
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    for b in list(range(0, 0x7F80, 97)) + list(range(0x8000, 0xFF80, 101)) + [0x7F7F, 0x0001, 0x8001, 0x0080]:
        assert Fraction(float(vals[b])) == _bf16_value_exact(b), hex(b)
    assert np.isinf(vals[0x7F80]) and np.isnan(vals[0x7FC0])


def _rounding_edge_values():
    rng = np.random.default_rng(123)
    vals = [0.0, -0.0, 1.0, -1.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -126,
            2.0 ** -126 - 2.0 ** -134, 2.0 ** -126 - 2.0 ** -140, 1e-40, -1e-41,
            float(np.finfo(np.float32).max), 2.0 ** 128 - 2.0 ** 119,
            2.0 ** 128 - 2.0 ** 119 - 2.0 ** 70, 2.0 ** 128, 1e300, -1e300,
            math.inf, -math.inf]
    # exact bf16 midpoints (ties) and their fp64 neighbours
    for b in rng.integers(0, 0x7F7F, 300):
        lo, hi = _bf16_value_exact(int(b)), _bf16_value_exact(int(b) + 1)
        mid = float((lo + hi) / 2)
        vals += [mid, -mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    vals += list(rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, 300))
    vals += list(rng.standard_normal(50) * 2.0 ** -130)
    return np.array(vals, dtype=np.float64)


def test_round_f64_to_bf16_matches_exact_bruteforce():
    vals = _rounding_edge_values()
    got = oracle.round_f64_to_bf16_bits(vals)
    want = np.array([_rne_bf16_bruteforce(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(vals[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_round_nan_and_shape():
    x = np.array([[np.nan, -np.nan], [1.0, -2.0]])
    r = oracle.round_f64_to_bf16_bits(x)
    assert r.shape == (2, 2)
    assert r[0, 0] == 0x7FC0 and r[1, 0] == 0x3F80 and r[1, 1] == 0xC000


def test_direct_rounding_differs_from_double_rounding():
    # 1 + 2**-8 + 2**-30 is above the bf16 midpoint 1 + 2**-8, so it rounds
    # up; through float32 it first becomes exactly the midpoint and then rounds
    # to even (down).  The oracle must round once.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.round_f64_to_bf16_bits(np.array([v]))[0] == 0x3F81
    assert _rne_bf16_bruteforce(float(np.float32(v))) == 0x3F80


# --------------------------------------------------------- fused oracle ----

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_matches_exact_rational_bruteforce(dtype):
    rng = np.random.default_rng(7)
    N, T, h = 3, 4, 16
    parts = rng.standard_normal((N, T, h)).astype(np.float32)
    res = rng.standard_normal((T, h)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(h)).astype(np.float32)
    parts[1, 2] *= 1000.0          # a row with a large dynamic range
    res[3] *= 1e-3
    if dtype == "bf16":
        from synthetic import f32_to_bf16_bits
        parts, res, w = f32_to_bf16_bits(parts), f32_to_bf16_bits(res), f32_to_bf16_bits(w)
    eps = 1e-5
    y, x, rows = oracle.fused_reduce_rmsnorm(list(parts), res, w, eps, dtype)
    y_ref, x_ref = _exact_row_reference(parts, res, w, eps, dtype)
    assert list(rows) == list(range(T))
    np.testing.assert_allclose(x, x_ref, rtol=1e-15, atol=0)
    np.testing.assert_allclose(y, y_ref, rtol=1e-14, atol=0)


def test_oracle_uses_float32_eps_and_eps_inside_root():
    # A tiny row makes eps dominate, so its placement and value matter.
    N, T, h = 1, 1, 8
    parts = np.full((N, T, h), 2.0 ** -12, dtype=np.float32)
    res = np.zeros((T, h), dtype=np.float32)
    w = np.ones(h, dtype=np.float32)
    eps = 1e-5                       # not exactly representable in float32
    y, _, _ = oracle.fused_reduce_rmsnorm(list(parts), res, w, eps, "f32")
    e32 = Fraction(float(np.float32(eps)))
    c = Fraction(2) ** -12
    want = float(c) / math.sqrt(float(c * c + e32))
    assert y[0, 0] == pytest.approx(want, rel=1e-15)
    assert abs(y[0, 0] - float(c) / math.sqrt(float(c * c) + 1e-5)) > 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_closed_forms_constant_onehot_zero_rows(dtype):
    N, T, h = 3, 33, 64
    eps = 1e-5
    e64 = float(np.float32(eps))
    s = special_rows_inputs(N, T, h, dtype)
    parts, res = list(s["partials"]), s["residual"]
    # constant rows with weight 1: y = sign(c) / sqrt(1 + eps / c^2)
    y1, x1, _ = oracle.fused_reduce_rmsnorm(parts, res, s["weight_one"], eps, dtype)
    widen = oracle.bf16_bits_to_f64 if dtype == "bf16" else oracle.f32_to_f64
    w = widen(s["weight"])
    y, x, _ = oracle.fused_reduce_rmsnorm(parts, res, s["weight"], eps, dtype)
    for t in range(T):
        c = s["value"][t]
        if s["kind"][t] == 0:
            assert np.all(y[t] == 0) and np.all(x[t] == 0)
        elif s["kind"][t] == 1:
            want = math.copysign(1.0, c) / math.sqrt(1.0 + e64 / (c * c))
            np.testing.assert_allclose(y1[t], want, rtol=1e-15)
            np.testing.assert_array_equal(x1[t], c)
        else:
            j = s["hot"][t]
            want = c * w[j] / math.sqrt(c * c / h + e64)
            assert y[t, j] == pytest.approx(want, rel=1e-15)
            others = np.delete(y[t], j)
            assert np.all(others == 0)


def test_closed_form_example_value():
    # c = 2**-8 and eps = 1e-5: 1/sqrt(1 + 1e-5 * 2**16) = 1/sqrt(1.65536...)
    N, T, h = 1, 1, 16
    parts = np.full((N, T, h), 2.0 ** -8, dtype=np.float32)
    y, _, _ = oracle.fused_reduce_rmsnorm(list(parts), np.zeros((T, h), np.float32),
                                          np.ones(h, np.float32), 1e-5, "f32")
    assert y[0, 0] == pytest.approx(0.7772, abs=5e-5)


def test_library_special_case_torch_rms_norm():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    T, h = 17, 96
    p = rng.standard_normal((1, T, h)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(h)).astype(np.float32)
    eps = 1e-6
    y, x, _ = oracle.fused_reduce_rmsnorm(list(p), np.zeros((T, h), np.float32), w, eps, "f32")
    ref = torch.nn.functional.rms_norm(torch.from_numpy(p[0]).double(), (h,),
                                       torch.from_numpy(w).double(),
                                       eps=float(np.float32(eps))).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(x, p[0].astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_invariants_sign_weight_permutation(dtype):
    N, T, h = 4, 9, 32
    d = integer_scaled_inputs(N, T, h, dtype, kmax=8)
    parts, res, w = d["partials"], d["residual"], d["weight"]
    neg = (lambda a: a ^ np.uint16(0x8000)) if dtype == "bf16" else (lambda a: -a)
    y, x, _ = oracle.fused_reduce_rmsnorm(list(parts), res, w, 1e-5, dtype)
    yn, xn, _ = oracle.fused_reduce_rmsnorm([neg(p) for p in parts], neg(res), w, 1e-5, dtype)
    np.testing.assert_array_equal(yn, -y)
    np.testing.assert_array_equal(xn, -x)
    w2 = d["weight"].astype(np.float32) if dtype == "f32" else None
    if dtype == "f32":
        y2, _, _ = oracle.fused_reduce_rmsnorm(list(parts), res, w2 * 2, 1e-5, dtype)
        np.testing.assert_array_equal(y2, 2 * y)
    yp, xp, _ = oracle.fused_reduce_rmsnorm(list(parts[::-1]), res, w, 1e-5, dtype)
    np.testing.assert_array_equal(xp, x)
    np.testing.assert_array_equal(yp, y)


def test_partials_and_residual_all_enter_the_sum():
    # Changing any one partial or the residual changes x by exactly that amount.
    N, T, h = 3, 2, 8
    d = integer_scaled_inputs(N, T, h, "f32", kmax=8, seed=5)
    _, x0, _ = oracle.fused_reduce_rmsnorm(list(d["partials"]), d["residual"], d["weight"], 1e-5, "f32")
    for i in range(N + 1):
        parts = d["partials"].copy()
        res = d["residual"].copy()
        if i < N:
            parts[i, 1, 3] += 0.5
        else:
            res[1, 3] += 0.5
        _, x1, _ = oracle.fused_reduce_rmsnorm(list(parts), res, d["weight"], 1e-5, "f32")
        diff = x1 - x0
        assert diff[1, 3] == 0.5 and np.count_nonzero(diff) == 1


def test_shard_rows_partition_and_bounds():
    for T in (0, 1, 7, 8, 64, 100, 1023):
        for N in (1, 2, 3, 8, 16):
            seen = []
            for k in range(N):
                r = oracle.shard_rows(T, N, k)
                assert r.start == (k * T) // N and r.stop == ((k + 1) * T) // N
                seen += list(r)
            assert seen == list(range(T))
    assert list(oracle.shard_rows(10, 4, 1)) == [2, 3, 4]
    assert list(oracle.shard_rows(10, 4, 3)) == [7, 8, 9]
    with pytest.raises(ValueError):
        oracle.shard_rows(8, 2, 2)


def test_shard_oracle_equals_full_rows():
    d = make_inputs("tiny")
    y, x, _ = oracle.fused_reduce_rmsnorm(list(d["partials"]), d["residual"], d["weight"], d["eps"], "f32")
    for k in range(2):
        ys, xs, rows = oracle.shard_rmsnorm(list(d["partials"]), d["residual"], d["weight"], d["eps"], "f32", k)
        np.testing.assert_array_equal(ys, y[rows])
        np.testing.assert_array_equal(xs, x[rows])
