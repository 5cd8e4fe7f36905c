"""Pins of the oracle's fused-producer, calibration and KV-cache functions.

Each check ties an oracle function to something other than itself: exact
rational / high-precision decimal evaluation of the defining formula, closed
forms, brute force on small inputs, or an identity. Planted mistakes at the
end must each trip at least one check.
"""
import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle.fp8dq_oracle as O
import synth

pytestmark = []

BF16_MIN_SUB = Fraction(1, 2 ** 133)


def exact_bf16_bits(q: Fraction) -> int:
    """Round an exact rational to bf16 (nearest, ties to even), bit pattern.
    Overflow -> inf; the sign of an exact zero is not decided here."""
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # 2^e <= a < 2^(e+1)
    e = max(e, -126)                             # subnormal: fixed spacing 2^-133
    ulp = Fraction(2) ** (e - 7)
    n = a / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (k & 1)):
        k += 1
    val = k * ulp
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f32 = np.float32(float(val))                 # exact: val is a bf16 value
    return sign | int(f32.view(np.uint32) >> 16) & 0x7FFF


def dec(x: float) -> Decimal:
    return Decimal(float(x))                     # exact binary value


def silu_mul_exact_bits(g: float, u: float) -> int:
    """Exact bf16 rounding of silu(g) * u. For g > 0 as g*u - delta with
    delta = g*u*e^-g / (1 + e^-g) (small, taken to 60 digits relative, the
    difference then exact); for g <= 0 as g*u*e^g / (1 + e^g)."""
    neg_zero = (math.copysign(1, g) * math.copysign(1, u)) < 0
    with localcontext() as ctx:
        ctx.prec = 60
        gd, ud = dec(g), dec(u)
        try:
            if g > 0:
                e = (-gd).exp()
                q = Fraction(g) * Fraction(u) - Fraction(gd * ud * e / (1 + e))
            else:
                e = gd.exp()
                q = Fraction(gd * ud * e / (1 + e))
        except ArithmeticError:          # e^g far below any decimal exponent
            q = Fraction(0)
    if q == 0:
        return 0x8000 if neg_zero else 0
    return exact_bf16_bits(q)


def rmsnorm_exact_bits(x: np.ndarray, gam: np.ndarray, eps: float) -> np.ndarray:
    with localcontext() as ctx:
        ctx.prec = 60
        ms = sum(Fraction(float(v)) ** 2 for v in x) / len(x) + Fraction(eps)
        r = 1 / (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        out = []
        for xv, gv in zip(x, gam):
            h = Fraction(dec(gv) * dec(xv) * r)
            if h == 0:
                neg = (math.copysign(1, xv) * math.copysign(1, gv)) < 0
                out.append(0x8000 if neg else 0)
            else:
                out.append(exact_bf16_bits(h))
    return np.array(out, np.uint16)


def bits_of(v) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.asarray(v, np.float32))


# ----------------------------------------------------------------------------
def check_bf16_rounding(o):
    rng = np.random.default_rng(21)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000))
    mids = (o.bf16_to_f64(bits_of(rng.standard_normal(500))) *
            (1 + 2.0 ** -8))                     # exact bf16 midpoints (ties)
    extra = np.array([0.0, -0.0, 3.5e38, -3.5e38, 2.0 ** -134, -(2.0 ** -133) * 1.5,
                      o.BF16_MAX, o.BF16_MAX * (1 + 2.0 ** -9)])
    allv = np.concatenate([v, mids, extra])
    got = o.f64_to_bf16_bits(allv)
    for x, b in zip(allv, got):
        want = exact_bf16_bits(Fraction(float(x))) if x != 0 else (0x8000 if math.copysign(1, x) < 0 else 0)
        assert int(b) == want, (x, hex(int(b)), hex(want))


def check_silu_mul_highprec(o):
    rng = np.random.default_rng(22)
    g = np.concatenate([rng.standard_normal(400) * 3, rng.standard_normal(100) * 30,
                        [0.0, -0.0, 1e-30, -1e-30, 80.0, -80.0, 100.0, -100.0, 700.0,
                         -700.0, 1e4, -1e4, 3e38, -3e38]])
    u = rng.standard_normal(g.size) * np.exp2(rng.integers(-20, 20, g.size))
    gb, ub = bits_of(g), bits_of(u)
    got = o.silu_mul_bf16(np.concatenate([gb, ub])[None, :])[0]
    gf, uf = o.bf16_to_f64(gb), o.bf16_to_f64(ub)
    for i in range(g.size):
        want = silu_mul_exact_bits(gf[i], uf[i])
        assert int(got[i]) == want, (gf[i], uf[i], hex(int(got[i])), hex(want))


def check_silu_identities(o):
    rng = np.random.default_rng(23)
    u = o.bf16_to_f64(bits_of(rng.standard_normal(64)))
    ub = bits_of(u)
    # g = 0: silu(0) = 0, so h is a zero with the sign of 0 * u
    h0 = o.silu_mul_bf16(np.concatenate([bits_of(np.zeros(64)), ub])[None, :])[0]
    assert np.all((h0 & 0x7FFF) == 0) and np.all((h0 >> 15) == (u < 0))
    # g large: silu(g) = g to far below bf16 precision, so h = RN(g * u)
    g = np.full(64, 200.0)
    hg = o.silu_mul_bf16(np.concatenate([bits_of(g), ub])[None, :])[0]
    assert np.array_equal(hg, o.f64_to_bf16_bits(200.0 * u))
    # silu(g) - silu(-g) = g, checked on the exact-formula side with u = 1
    gs = o.bf16_to_f64(bits_of(rng.standard_normal(32) * 4))
    one = bits_of(np.ones(32))
    hp = o.bf16_to_f64(o.silu_mul_bf16(np.concatenate([bits_of(gs), one])[None, :])[0])
    hn = o.bf16_to_f64(o.silu_mul_bf16(np.concatenate([bits_of(-gs), one])[None, :])[0])
    assert np.all(np.abs((hp - hn) - gs) <= 2.0 ** -7 * (np.abs(hp) + np.abs(hn)) + 1e-30)


def check_silu_structural_ties(o):
    """g*u (huge g) or g*u/2 (tiny g) an exact bf16 midpoint. silu(g) < g for
    g > 0 puts |h| below the tie for huge g; silu(g) = g/2 + g^2/4 + ... puts
    it above for tiny g > 0 and below for tiny g < 0. The bf16 neighbour
    toward zero is the truncation of the midpoint's value."""
    U = np.arange(87, 171, 2, dtype=np.float64)          # 3 * U: odd, 9 bits
    trunc = lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for g, halve, away in ((3.0 * 2.0 ** 98, False, False), (3.0 * 2.0 ** 120, False, False),
                           (3.0 * 2.0 ** -102, True, True), (-3.0 * 2.0 ** -102, True, False)):
        for sgn in (1.0, -1.0):
            u = sgn * U * (2.0 ** -30 if not halve else 1.0)
            m = g * u / (2.0 if halve else 1.0)
            gu = bits_of(np.concatenate([np.full(U.size, g), u]))[None, :]
            assert np.array_equal(o.bf16_to_f64(gu[0, U.size:]), u)
            got = o.silu_mul_bf16(gu)[0]
            lo = trunc(m)
            want = lo + 1 if away else lo
            assert np.array_equal(got, want.astype(np.uint16)), (g, sgn, got, want)


def check_rmsnorm_highprec(o):
    rng = np.random.default_rng(24)
    rows = [rng.standard_normal(48), rng.standard_normal(48) * 1e-3,   # eps matters
            rng.standard_normal(48) * 50, rng.standard_normal(48) * 3e-3]
    gam = o.bf16_to_f64(bits_of(rng.standard_normal(48) * 0.5 + 1))
    xb = bits_of(np.stack(rows))
    got = o.rmsnorm_bf16(xb, bits_of(gam))
    xs = o.bf16_to_f64(xb)
    for r in range(xs.shape[0]):
        want = rmsnorm_exact_bits(xs[r], gam, o.RMS_EPS)
        assert np.array_equal(got[r], want), (r, np.nonzero(got[r] != want))


def check_rmsnorm_special(o):
    gam1 = bits_of(np.ones(16))
    z = o.rmsnorm_bf16(bits_of(np.zeros((1, 16))), gam1)
    assert np.all(z == 0)
    c = 0.375
    h = o.rmsnorm_bf16(bits_of(np.full((1, 16), c)), gam1)
    with localcontext() as ctx:
        ctx.prec = 60
        want = exact_bf16_bits(Fraction(dec(c) / (dec(c) ** 2 + dec(o.RMS_EPS)).sqrt()))
    assert np.all(h == want)


def check_nearest_rank_bruteforce(o):
    rng = np.random.default_rng(25)
    for trial in range(60):
        n = int(rng.integers(1, 80))
        x = rng.standard_normal(n) * np.exp2(rng.integers(-4, 4, n))
        xb = bits_of(x)
        vals = sorted(float(v) for v in o.bf16_to_f64(xb))
        for lo, hi in [(1, 999), (100, 900), (0, 1000), (500, 500)]:
            klo = max(1, min(n, math.ceil(Fraction(lo, 1000) * n)))
            khi = max(1, min(n, math.ceil(Fraction(hi, 1000) * n)))
            want = max(abs(vals[klo - 1]), abs(vals[khi - 1]))
            assert o.calib_amax(xb, lo, hi) == want, (trial, n, lo, hi)
    # 1..n: the nearest-rank P99.9 of the integers 1..n is ceil(0.999 n)
    for n in (1000, 2048, 4097, 12345):
        xb = bits_of(np.arange(1, n + 1) % 256 + 0.0)  # bf16-exact integers
        ints = np.sort(np.arange(1, n + 1) % 256)
        assert o.calib_amax(xb, 1, 999) == max(ints[math.ceil(0.999 * n) - 1],
                                              ints[max(1, math.ceil(0.001 * n)) - 1])


def check_static_quant(o):
    s = np.float32(1.0 / 448.0)
    xb = bits_of([500.0, -500.0, 1e30, -1e30, 0.5, -0.0, 0.0])
    q = o.quant_static(xb, s)
    assert q[0] == 0x7E and q[1] == 0xFE and q[2] == 0x7E and q[3] == 0xFE   # saturation
    assert q[5] == 0x80 and q[6] == 0x00
    # with s = amax/448 of the tensor, static = dynamic per-row quantization
    x = synth.activations(1, 256, 31, 32)
    qd, sd = o.quant_per_row(x)
    assert np.array_equal(o.quant_static(x, sd[0])[0], qd[0])
    # exact rationals on random values against a fixed scale
    rng = np.random.default_rng(26)
    xs = bits_of(rng.standard_normal(500) * 3)
    sc = np.float32(0.0071)
    q = o.quant_static(xs, sc)
    grid = [Fraction(float(v)) for v in o.E4M3_VALUES[:127]]
    for b, c in zip(xs, q):
        t = Fraction(float(o.bf16_to_f64(np.array([b]))[0])) / Fraction(float(sc))
        a = abs(t)
        if a >= 448:
            code = 126
        else:
            lo = max(i for i in range(127) if grid[i] <= a)
            hi = min(lo + 1, 126)
            d0, d1 = a - grid[lo], grid[hi] - a
            code = lo if (d0 < d1 or (d0 == d1 and lo % 2 == 0)) else hi
        code |= 0x80 if (t < 0 or (t == 0 and (int(b) >> 15))) else 0
        assert int(c) == code, (int(b), int(c), code)


def check_kv_scatter(o):
    rng = np.random.default_rng(27)
    T, width = 40, 256
    k = synth.activations(T, width, 41, 42)
    v = synth.activations(T, width, 43, 44)
    slots = rng.permutation(100)[:T]
    slots[::7] = -1                                 # skipped tokens
    out = o.kv_quant_scatter(k, v, slots)
    qk, sk = o.quant_per_row(k)
    qv, sv = o.quant_per_row(v)
    assert set(out) == set(int(s) for s in slots if s >= 0)
    for t, slot in enumerate(slots):
        if slot >= 0:
            a, b, c, d = out[int(slot)]
            assert np.array_equal(a, qk[t]) and b == sk[t]
            assert np.array_equal(c, qv[t]) and d == sv[t]


CHECKS = [check_bf16_rounding, check_silu_mul_highprec, check_silu_identities,
          check_silu_structural_ties,
          check_rmsnorm_highprec, check_rmsnorm_special, check_nearest_rank_bruteforce,
          check_static_quant, check_kv_scatter]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin_next(check):
    check(O)


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------
def _silu_wrong_sign(gu_bits):
    gu = O.bf16_to_f64(gu_bits)
    half = gu.shape[1] // 2
    g, u = gu[:, :half], gu[:, half:]
    with np.errstate(over="ignore"):
        return O.f64_to_bf16_bits(g / (1.0 + np.exp(g)) * u)


def _silu_swapped_halves(gu_bits):
    gu = np.asarray(gu_bits)
    half = gu.shape[1] // 2
    return _ORIG["silu_mul_bf16"](np.concatenate([gu[:, half:], gu[:, :half]], axis=1))


def _rms_no_eps(x_bits, gamma_bits, eps=O.RMS_EPS):
    return _ORIG["rmsnorm_bf16"](x_bits, gamma_bits, 0.0)


def _rms_sum(x_bits, gamma_bits, eps=O.RMS_EPS):
    x = O.bf16_to_f64(x_bits)
    gam = O.bf16_to_f64(gamma_bits)[None, :]
    return O.f64_to_bf16_bits(gam * x / np.sqrt(np.sum(x * x, 1, keepdims=True) + eps))


def _rank_floor(n, permille):
    return int(min(max((permille * n) // 1000, 1), n))


def _bf16_truncating(y):
    y = np.asarray(y, np.float64)
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _kv_off_by_one(k_bits, v_bits, slots):
    return _ORIG["kv_quant_scatter"](k_bits, v_bits, np.asarray(slots) + 1)


_ORIG = {n: getattr(O, n) for n in ("silu_mul_bf16", "rmsnorm_bf16", "kv_quant_scatter")}

MUTATIONS = {
    "silu_wrong_sign": ("silu_mul_bf16", _silu_wrong_sign),
    "silu_swapped_halves": ("silu_mul_bf16", _silu_swapped_halves),
    "rms_no_eps": ("rmsnorm_bf16", _rms_no_eps),
    "rms_sum_not_mean": ("rmsnorm_bf16", _rms_sum),
    "rank_floor": ("nearest_rank", _rank_floor),
    "bf16_truncating": ("f64_to_bf16_bits", _bf16_truncating),
    "kv_off_by_one": ("kv_quant_scatter", _kv_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_next_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    failed = []
    for check in CHECKS:
        try:
            check(O)
        except (AssertionError, ValueError, IndexError, KeyError):
            failed.append(check.__name__)
    assert failed, f"mutation {name} slipped past every pin"
