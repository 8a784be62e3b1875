"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin is a function ``pin(o)`` taking an oracle-like namespace ``o`` (the
real oracle package, or a copy with a planted mistake) and raising
AssertionError when ``o`` disagrees with the fact it checks.  The facts are:
hand-derived worked examples (tests/golden/worked_examples.json), exact
rational arithmetic (fractions.Fraction), one-operation-at-a-time binary64
routes that round once to binary32, brute force on tiny inputs, invariants
of the definitions (permutation, power-of-two scaling, sign symmetry, zero
rows), and the ternary zero fraction of Gaussian weights.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
    GOLD = json.load(f)

F32_EPS = float(np.float32(1e-5))


def f32(v):
    return float(np.float32(v))


# ---------------------------------------------------------------- worked examples

def pin_e1_ternarize(o):
    e = GOLD["E1_ternarize"]
    w = np.array(e["W"], np.float32)
    g = o.absmean_gamma(w)
    assert float(g) == e["gamma"]
    d = np.float32(g) + np.float32(1e-5)
    assert int(np.float32(d).view(np.uint32)) == int(e["d_bits"], 16)
    assert o.ternarize(w, g).tolist() == e["t"]


def pin_e2_epsilon(o):
    e = GOLD["E2_epsilon_moves_threshold"]
    w = np.array(e["W"], np.float32)
    assert o.ternarize(w, o.absmean_gamma(w)).tolist() == e["t"]


def pin_e3_layout(o):
    e = GOLD["E3_layout"]
    t = np.array([e["t_row"]], np.int8)
    assert o.pack_ternary(t)[0].tolist() == e["bytes"]


def pin_e4_act_quant(o):
    e = GOLD["E4_act_quant"]
    q, a, rs = o.quant_act(np.array(e["x"], np.float32))
    assert q.tolist() == e["q"]
    assert a.tolist() == e["absmax"]
    assert rs.tolist() == e["rowsum"]


def pin_e5_contract_rescale(o):
    e1, e4, e5 = GOLD["E1_ternarize"], GOLD["E4_act_quant"], GOLD["E5_contract_rescale"]
    t = np.array(e1["t"], np.int8)
    q = np.array(e4["q"], np.int8)
    acc = o.contract(q, t)
    assert acc.tolist() == e5["acc"]
    y = o.rescale(acc, np.float32(e1["gamma"]), np.array(e4["absmax"], np.float32))
    assert np.array_equal(np.asarray(y, np.float64), np.array(e5["y"]))


# ---------------------------------------------------------------- gamma

def _gamma_by_fractions(w):
    s = sum(Fraction(float(v)) for v in np.abs(w).ravel())
    mean = float(s) / float(w.size)          # float(Fraction) rounds to nearest
    return np.float32(mean)


def _awkward_weights(rng, n, k):
    """Magnitudes spread over many binades, including subnormals, so that any
    inexact or order-dependent sum shows up in the rounded result."""
    mant = rng.random((n, k)) + 0.5
    expo = rng.integers(-140, 90, size=(n, k))
    w = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    w *= np.where(rng.random((n, k)) < 0.5, -1, 1).astype(np.float32)
    w[rng.random((n, k)) < 0.1] = 0.0
    return w


def pin_gamma_exact_fraction(o):
    rng = np.random.default_rng(11)
    cases = [_awkward_weights(rng, 3, 16), _awkward_weights(rng, 7, 32),
             rng.standard_normal((5, 48)).astype(np.float32) * np.float32(0.02)]
    # one huge value beside many small ones: a naive float sum loses the small ones
    big = np.full((4, 64), 1.0, np.float32)
    big[0, 0] = np.float32(2.0 ** 60)
    cases.append(big)
    # S = 2**60 + 2**36 + 254: RN64(S) = 2**60 + 2**36 + 256, so the mean lies
    # just above a binary32 midpoint and rounds up; a running binary64 sum
    # drops every 1.0, lands on the midpoint itself and rounds to even (down).
    tie = np.ones((16, 16), np.float32)
    tie[0, 0] = np.float32(2.0 ** 60)
    tie[0, 1] = np.float32(2.0 ** 36)
    cases.append(tie)
    small = np.full((2, 16), np.float32(1e-3), np.float32)
    small[1, 3] = np.float32(3.0e7)
    cases.append(small)
    for w in cases:
        g = o.absmean_gamma(w)
        assert np.float32(g).view(np.uint32) == _gamma_by_fractions(w).view(np.uint32)


def pin_gamma_constant(o):
    for c in (0.02, -0.75, 3.0e-20, 1.0, 12345.678):
        for shape in ((1, 16), (3, 7), (64, 96)):
            w = np.full(shape, np.float32(c), np.float32)
            assert np.float32(o.absmean_gamma(w)) == np.float32(abs(np.float32(c)))


def pin_gamma_pow2_scaling(o):
    rng = np.random.default_rng(12)
    w = rng.standard_normal((33, 64)).astype(np.float32)
    g = np.float32(o.absmean_gamma(w))
    for k in (-7, -1, 3, 20):
        gk = np.float32(o.absmean_gamma(w * np.float32(2.0 ** k)))
        assert gk == g * np.float32(2.0 ** k)


def pin_gamma_permutation(o):
    rng = np.random.default_rng(13)
    w = _awkward_weights(rng, 16, 64)
    g = np.float32(o.absmean_gamma(w)).view(np.uint32)
    for _ in range(3):
        p = rng.permutation(w.ravel()).reshape(w.shape)
        assert np.float32(o.absmean_gamma(p)).view(np.uint32) == g
    # row and column reversal as well (a transposed reading of W)
    assert np.float32(o.absmean_gamma(np.ascontiguousarray(w.T))).view(np.uint32) == g


# ---------------------------------------------------------------- ternarize

def _ternarize_scalar(wv, gamma):
    d = f32(f32(gamma) + F32_EPS)            # one binary32 addition
    u = f32(float(wv) / d)                   # binary64 quotient, rounded once to binary32
    r = round(u)                             # Python rounds half to even
    return max(-1, min(1, r))


def pin_ternarize_independent(o):
    rng = np.random.default_rng(14)
    gamma = np.float32(0.0161)
    d = np.float32(gamma) + np.float32(1e-5)
    w = rng.standard_normal(2000).astype(np.float32) * np.float32(0.02)
    # exact ties and their neighbours: u = 0.5 and u = 1.5 exactly
    ties = np.array([0.5, 1.5, 2.5], np.float32) * d
    nbrs = np.concatenate([np.nextafter(ties, np.float32(1)), np.nextafter(ties, np.float32(0))])
    w = np.concatenate([w, ties, -ties, nbrs, -nbrs, [0.0, -0.0]]).astype(np.float32)
    t = o.ternarize(w.reshape(1, -1), gamma)[0]
    ref = [_ternarize_scalar(v, gamma) for v in w]
    assert t.tolist() == ref


def pin_ternarize_sign_symmetry(o):
    rng = np.random.default_rng(15)
    w = rng.standard_normal((8, 64)).astype(np.float32) * np.float32(0.02)
    g = o.absmean_gamma(w)
    assert np.array_equal(o.ternarize(-w, g), -o.ternarize(w, g))


def pin_zero_fraction(o):
    """For W ~ N(0, s) the absmean is s*sqrt(2/pi) and the threshold half of
    it, so P(t = 0) = erf(sqrt(2/pi) / (2 sqrt 2)) = 0.3101 (each sign 0.345)."""
    rng = np.random.default_rng(16)
    w = rng.standard_normal((512, 2048)).astype(np.float32) * np.float32(0.02)
    t = o.ternarize(w, o.absmean_gamma(w))
    p0 = math.erf(math.sqrt(2 / math.pi) / (2 * math.sqrt(2)))
    assert abs(float(np.mean(t == 0)) - p0) < 0.005
    assert abs(float(np.mean(t == 1)) - (1 - p0) / 2) < 0.005
    assert abs(float(np.mean(t == -1)) - (1 - p0) / 2) < 0.005


# ---------------------------------------------------------------- pack

def _decode_bytes(row_bytes, k):
    """Independent decoder: read each weight's two bits one by one."""
    out = []
    for kk in range(k):
        g, r = divmod(kk, 16)
        j, i = divmod(r, 4)
        byte = row_bytes[4 * g + i]
        code = (byte >> (2 * j)) & 3
        assert code != 3
        out.append(code - 1)
    return out


def pin_pack_roundtrip(o):
    rng = np.random.default_rng(17)
    t = rng.integers(-1, 2, size=(5, 96)).astype(np.int8)
    t[2] = 0
    p = o.pack_ternary(t)
    assert p.shape == (5, 24) and p.dtype == np.uint8
    for n in range(5):
        assert _decode_bytes(p[n].tolist(), 96) == t[n].tolist()
    assert p[2].tolist() == [0x55] * 24


# ---------------------------------------------------------------- act-quant

def _quant_scalar_row(row):
    a = max(abs(float(v)) for v in row)
    m = max(a, F32_EPS)
    s = f32(127.0 / m)                       # one binary32 division
    out = []
    for v in row:
        p = f32(float(v) * s)                # exact binary64 product, rounded once
        out.append(max(-127, min(127, round(p))))
    return out, a


def pin_quant_act_independent(o):
    rng = np.random.default_rng(18)
    x = rng.standard_normal((6, 4096)).astype(np.float32)
    x[1] = rng.standard_t(4, 4096).astype(np.float32)
    x[2] = 0.0
    x[3] *= np.float32(1e-4)
    # make ties: x * s = k + 0.5 exactly when absmax = 127
    x[4, :8] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -126.5, 126.5]
    x[4, 8:] = rng.uniform(-100, 100, 4088).astype(np.float32)
    q, a, rs = o.quant_act(x)
    for r in range(x.shape[0]):
        ref, ar = _quant_scalar_row(x[r])
        assert q[r].tolist() == ref
        assert float(a[r]) == ar
        assert int(rs[r]) == sum(ref)


def pin_quant_act_order_sensitive(o):
    """A case where 127/m is rounded before the product matters: the product
    x * RN32(127/m) and RN32(x*127)/m round to opposite sides of a half."""
    # absmax 15.317623 (0x417514FC) and x = 1.2664177 (0x3FA219FA):
    # x * RN32(127/m) = 10.5 exactly -> 10, while RN32(x*127)/m = 10.500001 -> 11;
    # absmax 12.734374 (0x414BBFFF), x = -2.25609 (0xC01063C7): -22.500002 -> -23
    # against -22.5 -> -22.
    bits = np.array([[0x417514FC, 0x3FA219FA, 0, 0],
                     [0xC14BBFFF, 0xC01063C7, 0x3F800000, 0]], np.uint32)
    x = np.tile(bits.view(np.float32), (1, 4))
    q, _, _ = o.quant_act(x)
    assert q[0, 1] == 10 and q[1, 1] == -23
    for r in range(x.shape[0]):
        ref, _ = _quant_scalar_row(x[r])
        assert q[r].tolist() == ref


def pin_quant_act_invariants(o):
    rng = np.random.default_rng(20)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    x[5] = 0.0
    q, a, _ = o.quant_act(x)
    for r in range(16):
        if r == 5:
            assert not q[r].any() and float(a[r]) == 0.0
        else:
            assert int(np.max(np.abs(q[r].astype(np.int32)))) == 127
    assert int(q.astype(np.int32).min()) >= -127
    qn, an, _ = o.quant_act(-x)
    assert np.array_equal(qn, -q) and np.array_equal(an, a)
    for k in (-10, 4):
        qk, _, _ = o.quant_act(x * np.float32(2.0 ** k))
        assert np.array_equal(qk, q)
    # one token per row: T rows quantise independently of each other
    q1, _, _ = o.quant_act(x[3:4])
    assert np.array_equal(q1[0], q[3])


def pin_widen_bf16(o):
    bits = np.array([[0x3F80, 0xC040, 0x0000, 0x8000, 0x4049, 0x0001]], np.uint16)
    x = o.widen_bf16(bits)
    assert x[0, :4].tolist() == [1.0, -3.0, 0.0, -0.0]
    assert x[0, 4] == np.float32(3.140625)
    assert x[0, 5] == np.float32(2.0 ** -133)


# ---------------------------------------------------------------- contraction

def pin_contract_bruteforce(o):
    rng = np.random.default_rng(21)
    k = 5
    rows = np.array(np.meshgrid(*[[-1, 0, 1]] * k, indexing="ij")).reshape(k, -1).T
    k16 = 16
    t = np.zeros((rows.shape[0], k16), np.int8)
    t[:, :k] = rows
    t[:, k:] = rng.integers(-1, 2, size=(rows.shape[0], k16 - k))
    q = rng.integers(-127, 128, size=(3, k16)).astype(np.int8)
    acc = o.contract(q, t)
    assert acc.shape == (3, rows.shape[0]) and acc.dtype == np.int32
    for a in range(3):
        for n in range(rows.shape[0]):
            s = 0
            for kk in range(k16):
                s += int(t[n, kk]) * int(q[a, kk])
            assert int(acc[a, n]) == s


def pin_contract_invariants(o):
    rng = np.random.default_rng(22)
    t = rng.integers(-1, 2, size=(9, 128)).astype(np.int8)
    t[4] = 0
    q = rng.integers(-127, 128, size=(7, 128)).astype(np.int8)
    q[:, :3] = 127
    acc = o.contract(q, t)
    assert not acc[:, 4].any()
    p = rng.permutation(128)
    assert np.array_equal(o.contract(q[:, p], t[:, p]), acc)
    assert np.array_equal(o.contract(q, -t), -acc)
    # a square, non-symmetric t checked against explicit loops
    ts = rng.integers(-1, 2, size=(16, 16)).astype(np.int8)
    qs = rng.integers(-127, 128, size=(3, 16)).astype(np.int8)
    accs = o.contract(qs, ts)
    for a in range(3):
        for n in range(16):
            assert int(accs[a, n]) == sum(int(ts[n, kk]) * int(qs[a, kk]) for kk in range(16))
    # extremes: all +127 against all +1 gives 127*K
    full = o.contract(np.full((1, 128), 127, np.int8), np.ones((1, 128), np.int8))
    assert int(full[0, 0]) == 127 * 128


def pin_contract_large_k(o):
    """K = 2**18: partial sums pass 2**24, where a binary32 accumulator would
    start to round; the int64 dot product is the independent route."""
    rng = np.random.default_rng(24)
    k = 1 << 18
    q = rng.integers(90, 128, size=(2, k)).astype(np.int8)
    q[1, ::3] = -127
    t = rng.integers(0, 2, size=(3, k)).astype(np.int8)
    t[2] = 1
    t[2, 7] = 0
    acc = o.contract(q, t)
    ref = q.astype(np.int64) @ t.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)


# ---------------------------------------------------------------- rescale

def pin_rescale(o):
    rng = np.random.default_rng(23)
    acc = rng.integers(-300000, 300000, size=(4, 6)).astype(np.int32)
    acc[1, 2] = 0
    gamma = np.float32(0.0159)
    absmax = np.array([3.5, 0.0, 1e-7, 17.25], np.float32)
    y = np.asarray(o.rescale(acc, gamma, absmax), np.float64)
    for t in range(4):
        m = Fraction(float(max(absmax[t], np.float32(1e-5))))
        for n in range(6):
            exact = Fraction(int(acc[t, n])) * Fraction(float(gamma)) * m / 127
            if exact == 0:
                assert y[t, n] == 0.0
            else:
                assert abs(Fraction(float(y[t, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
    assert y[1, 2] == 0.0


# ------------------------------------------------------------ SubLN + act-quant

def _rn(q, p, emin):
    """Round the rational q to p significant bits, nearest with ties to even,
    with the exponent floored at emin (gradual underflow); a Fraction."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1                               # now 2^e <= q < 2^(e + 1)
    e = max(e, emin)
    scale = Fraction(2) ** (p - 1 - e)
    n = q * scale
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * Fraction(fl) / scale


def _rn32(q):
    return _rn(q, 24, -126)


def _rn64(q):
    return _rn(q, 53, -1022)


def _sqrt_rn32(v):
    """RN32(sqrt(v)) for a non-negative rational v, from an integer square
    root with 200 fractional bits: the exact root lies in [X, X + 1) * 2^-200,
    and no binary32 rounding boundary of a root of a binary32 number falls
    strictly inside such an interval, so its midpoint rounds the same way."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    y = v * Fraction(4) ** 200
    x = math.isqrt(y.numerator // y.denominator)
    exact = Fraction(x * x) == y
    return _rn32(Fraction(x, 2 ** 200) if exact else Fraction(2 * x + 1, 2 ** 201))


def _rne_int(q):
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _subln_scalar(row, gain, eps_n):
    """SubLN + A1 of one token in exact rationals, each defined rounding
    applied by _rn32 / _rn64 above: returns (codes, a, rowsum, r) as Python
    numbers.  Shares nothing with the oracle but the definition."""
    xs = [Fraction(float(np.float32(v))) for v in row]
    gs = [Fraction(float(np.float32(v))) for v in gain]
    k = len(xs)
    s = _rn64(sum(v * v for v in xs))                  # exact sum, one rounding
    ms = _rn32(_rn64(s / k))
    v = _rn32(ms + Fraction(float(np.float32(eps_n))))
    r = _rn32(1 / _sqrt_rn32(v))
    xh = [_rn32(_rn32(x * g) * r) for x, g in zip(xs, gs)]
    a = max(abs(t) for t in xh)
    m = max(a, Fraction(F32_EPS))
    sc = _rn32(Fraction(127) / m)
    q = [max(-127, min(127, _rne_int(_rn32(t * sc)))) for t in xh]
    return q, float(a), sum(q), float(r)


def pin_e6_subln(o):
    e = GOLD["E6_subln"]
    x = np.array(e["x"], np.float32)
    q, a, rowsum, r = o.subln_quant_act(x, np.array(e["gain"], np.float32), e["eps_n"])
    assert q.tolist() == e["q"]
    assert rowsum.tolist() == e["rowsum"]
    assert np.asarray(a, np.float64).tolist() == e["a"]
    assert np.asarray(r, np.float64).tolist() == e["r"]


def pin_subln_scalar_route(o):
    # every output bit for bit against the exact-rational route above, on
    # rows of several kinds: heavy tails with negative gains, bf16-valued
    # activations, a wide range of magnitudes (subnormal to 1e18), a zero row
    rng = np.random.default_rng(64)
    k = 40
    x = (rng.standard_t(4, size=(6, k)) * 2).astype(np.float32)
    bf = rng.standard_normal(k).astype(np.float32).view(np.uint32)
    x[1] = ((bf + np.uint32(0x8000)) & np.uint32(0xFFFF0000)).view(np.float32)
    x[2] = (rng.standard_normal(k) * 10.0 ** rng.uniform(-44, 18, k)).astype(np.float32)
    x[3] = 0.0
    x[4, ::3] = 0.0
    g = (1.0 + 0.6 * rng.standard_normal(k)).astype(np.float32)
    # and 48 short rows, where the order of the two products shows in the
    # last bit of x_hat, hence of its absmax
    x16 = rng.standard_t(4, size=(48, 16)).astype(np.float32)
    g16 = (1.0 + 0.6 * rng.standard_normal(16)).astype(np.float32)
    for xx, gg in ((x, g), (x16, g16)):
        q, a, rowsum, r = o.subln_quant_act(xx, gg, 1e-5)
        for t in range(xx.shape[0]):
            qs, as_, rs, r_ = _subln_scalar(xx[t], gg, 1e-5)
            assert q[t].tolist() == qs, t
            assert float(a[t]) == as_ and int(rowsum[t]) == rs and float(r[t]) == r_, t


def pin_subln_exact_sum(o):
    # rows of one large value B (at each position k with k mod 128 < 8 in the
    # second row) and ones elsewhere, found by search: the exact sum of the
    # squares leads to one binary32 r, a running binary64 sum (first row:
    # every 1 is lost against B^2) or numpy's pairwise sum (second row) to
    # its neighbour; the exact-rational route fixes r
    for k, b, spaced in ((530, 142735360.0, False), (1026, 150822912.0, True)):
        x = np.ones((1, k), np.float32)
        if spaced:
            x[0, (np.arange(k) % 128) < 8] = b
        else:
            x[0, 0] = b
        _, _, _, r = o.subln_quant_act(x, np.ones(k, np.float32), 1e-5)
        assert float(r[0]) == _subln_scalar(x[0], np.ones(k), 1e-5)[3], k


def pin_subln_unit_gain_constant_rows(o):
    # g = 1 and a constant row c: x_hat is one value, every code is +-127,
    # and a = RN32(|c| * r) with r from the closed form S = K c^2
    cs = [1.0, -2.5, 3e-3, 1000.0, -0.0625]
    k = 64
    x = np.array([[c] * k for c in cs], np.float32)
    q, a, _, r = o.subln_quant_act(x, np.ones(k, np.float32), 1e-5)
    for i, c in enumerate(cs):
        c32 = Fraction(float(np.float32(c)))
        v = _rn32(_rn32(_rn64(k * c32 * c32) / k) + Fraction(F32_EPS))
        rr = _rn32(1 / _sqrt_rn32(v))
        assert set(q[i].tolist()) == {127 if c > 0 else -127}
        assert float(r[i]) == float(rr) and float(a[i]) == float(_rn32(abs(c32) * rr))


def pin_subln_zero_row(o):
    x = np.zeros((2, 32), np.float32)
    x[1, 3] = 1.0
    q, a, rowsum, r = o.subln_quant_act(x, np.full(32, 2.0, np.float32))
    assert not q[0].any() and float(a[0]) == 0.0 and int(rowsum[0]) == 0
    assert float(r[0]) == float(_rn32(1 / _sqrt_rn32(Fraction(F32_EPS))))
    # one non-zero entry: it is the absmax, so its code is 127 and the rest 0
    assert q[1].tolist() == [0, 0, 0, 127] + [0] * 28


def pin_subln_scale_invariance(o):
    # x * 2^j scales S by 4^j exactly; away from eps_n (large rows) r scales
    # by 2^-j and x_hat, its codes and absmax are unchanged
    rng = np.random.default_rng(65)
    x = (rng.standard_normal((3, 96)) * 40).astype(np.float32)
    g = (1.0 + 0.5 * rng.standard_normal(96)).astype(np.float32)
    q, a, rs, r = o.subln_quant_act(x, g, 1e-30)
    q2, a2, rs2, r2 = o.subln_quant_act(x * np.float32(8), g, 1e-30)
    assert np.array_equal(q, q2) and np.array_equal(a, a2) and np.array_equal(r, r2 * np.float32(8))


def pin_subln_near_binary64_norm(o):
    # the binary32 route against the norm in binary64 throughout: codes may
    # differ only where the two round a product to different sides of a .5
    # boundary (rare, and by one); absmax within a few binary32 roundings
    rng = np.random.default_rng(63)
    x = rng.standard_t(4, size=(64, 512)).astype(np.float32)
    g = (1.0 + 0.3 * rng.standard_normal(512)).astype(np.float32)
    q, a, _, _ = o.subln_quant_act(x, g)
    qp, mp = o.subln_plain(x, g)
    d = np.abs(q.astype(np.int32) - qp.astype(np.int32))
    assert d.max() <= 1 and np.count_nonzero(d) <= q.size // 1000
    assert np.allclose(a, mp, rtol=5e-7, atol=0.0)


# ------------------------------------------------------------ gated ReLU^2, bf16

def _bf16_torch(v):
    import torch   # an independent round-to-nearest-even to bfloat16
    t = torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _gated_scalar(ag, au, gg, gu, a):
    # the defined route in exact rationals: g and u are step A3's binary64
    # evaluation ((acc * gamma) * m) / 127, one rounding per operation,
    # rounded to binary32; then two binary32 products
    m = max(Fraction(float(np.float32(a))), Fraction(F32_EPS))
    def a3(acc, gamma):
        t = _rn64(_rn64(acc * Fraction(float(np.float32(gamma)))) * m)
        return _rn32(_rn64(t / 127))
    g, u = a3(int(ag), gg), a3(int(au), gu)
    r = max(g, Fraction(0))
    return float(_rn32(_rn32(r * r) * u))


def pin_e7_gated_relu2(o):
    e = GOLD["E7_gated_relu2"]
    h = o.gated_relu2(np.array(e["acc_gate"]), np.array(e["acc_up"]), e["gamma_gate"],
                      e["gamma_up"], np.array(e["absmax"], np.float32))
    assert [f"0x{v:04x}" for v in h.ravel().tolist()] == e["h_bf16"]


def pin_gated_route(o):
    # inputs where a binary32 output scale RN32(RN32(gamma * m) / 127), or
    # the other order of the two products, changes the bfloat16 bits (found
    # by search); expected values from the exact-rational route above and
    # torch's rounding
    gg, gu, a = 0.0173, 0.0291, 3.7
    ag = np.array([[3962, 9049, 15404, 7127, 8976, 2483, 320, 7, 0, 1000]])
    au = np.array([[-4705, 8931, 9021, -14946, 2615, -481, -905, 5, 100, -1]])
    h = o.gated_relu2(ag, au, gg, gu, np.array([a], np.float32))
    want = _bf16_torch([_gated_scalar(x, y, gg, gu, a) for x, y in zip(ag[0], au[0])])
    assert np.array_equal(h.ravel(), want)


def pin_bf16_rne(o):
    rng = np.random.default_rng(71)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    # exact halfway cases too: bit 15 set, lower bits clear, both parities
    halves = (rng.integers(0, 1 << 15, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, halves[np.isfinite(halves)], np.float32([0.0, -0.0, 1.0, 3.0e38])])
    assert np.array_equal(o.bf16_rne(v), _bf16_torch(v))


def pin_gated_invariants(o):
    rng = np.random.default_rng(72)
    ag = rng.integers(-5000, 5000, (4, 300))
    au = rng.integers(-5000, 5000, (4, 300))
    a = rng.uniform(0.1, 50, 4).astype(np.float32)
    h = o.gated_relu2(ag, au, 0.02, 0.03, a)
    # no output where the gate is not positive
    assert np.all((h[ag <= 0] & 0x7fff) == 0)
    # the up output's sign flips only the sign bit
    assert np.array_equal(o.gated_relu2(ag, -au, 0.02, 0.03, a), h ^ np.uint16(0x8000))
    # doubling the gate sums is exact and multiplies h by 4 (exponent + 2)
    h2 = o.gated_relu2(2 * ag, au, 0.02, 0.03, a)
    nz = (h & 0x7fff) != 0
    assert np.array_equal(h2[nz], h[nz] + np.uint16(0x0100))


def pin_gated_matches_binary64(o):
    # against ReLU(g)^2 * u in binary64 rounded once to bfloat16: the bits may
    # differ only at bfloat16 rounding boundaries, by one unit
    rng = np.random.default_rng(73)
    ag = rng.integers(-20000, 20000, (16, 2000))
    au = rng.integers(-20000, 20000, (16, 2000))
    a = rng.uniform(0.5, 20, 16).astype(np.float32)
    h = o.gated_relu2(ag, au, 0.0173, 0.0291, a).astype(np.int32)
    p = _bf16_torch(o.gated_relu2_plain(ag, au, 0.0173, 0.0291, a).astype(np.float32)).astype(np.int32)
    d = np.abs(h - p)
    assert d.max() <= 1 and np.count_nonzero(d) <= h.size // 500


# ------------------------------------------------------------ binary weights (W1A8)

def _decode_binary(packed, k):
    # read back bit by bit from the stated layout: weight k = 32g + 4j + i at
    # bit 8i + j of little-endian word g of its row; bit 1 means +1
    n = packed.shape[0]
    t = np.zeros((n, k), np.int8)
    for r in range(n):
        for kk in range(k):
            g, rem = divmod(kk, 32)
            j, i = divmod(rem, 4)
            byte = packed[r, 4 * g + i]
            t[r, kk] = 1 if (byte >> j) & 1 else -1
    return t


def pin_e8_binary(o):
    e = GOLD["E8_binary"]
    w = np.array(e["w"], np.float32)
    packed, gamma = o.pack_weights_binary(w)
    assert [[f"0x{b:02x}" for b in row] for row in packed] == e["packed"]
    assert float(gamma) == e["gamma"]


def pin_binary_decoder(o):
    rng = np.random.default_rng(81)
    w = rng.standard_normal((9, 96)).astype(np.float32)
    w[0, :5] = [0.0, -0.0, 1e-45, -1e-45, 0.0]
    t = o.binarize(w)
    assert set(np.unique(t)) <= {-1, 1}
    want = np.where(np.signbit(w) & (w != 0), -1, 1)     # zeros of either sign -> +1
    assert np.array_equal(t, want)
    assert np.array_equal(_decode_binary(o.pack_binary(t), 96), t)


def pin_binary_rows_and_symmetry(o):
    assert np.all(o.pack_binary(np.ones((2, 64), np.int8)) == 0xFF)
    assert np.all(o.pack_binary(-np.ones((2, 64), np.int8)) == 0x00)
    rng = np.random.default_rng(82)
    w = rng.standard_normal((5, 64)).astype(np.float32)
    w[w == 0] = 1.0
    p = o.pack_binary(o.binarize(w))
    assert np.array_equal(o.pack_binary(o.binarize(-w)), ~p)
    with pytest.raises(ValueError):
        o.pack_binary(np.ones((1, 48), np.int8))          # K % 32 != 0
    with pytest.raises(ValueError):
        o.pack_binary(np.zeros((1, 32), np.int8))         # 0 is not a binary level


def pin_binary_forward_by_hand(o):
    # tiny case against plain Python loops over the definitions
    rng = np.random.default_rng(83)
    w = (rng.standard_normal((3, 32)) * 0.02).astype(np.float32)
    x = rng.standard_normal((2, 32)).astype(np.float32)
    y, acc, _, gamma = o.forward_binary(w, x)
    q, a, _ = o.quant_act(x)
    assert float(gamma) == float(np.float32(math.fsum(abs(float(v)) for v in w.ravel()) / w.size))
    for tt in range(2):
        for n in range(3):
            s = sum((1 if w[n, k] >= 0 else -1) * int(q[tt, k]) for k in range(32))
            assert acc[tt, n] == s
            want = s * float(gamma) * max(float(a[tt]), float(np.float32(1e-5))) / 127
            assert abs(y[tt, n] - want) <= 1e-12 * max(1.0, abs(want))


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
