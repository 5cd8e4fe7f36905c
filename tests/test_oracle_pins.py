"""Pins of the CPU oracle against things other than itself (CPU only).

Each check is written as a function of the oracle module so that the
"planted mistake" tests at the bottom can run the same checks on a copy of
the oracle with one deliberate error and show that some check fails.

Independent sources used here:
* the format limits the pages print (tests/golden/fp8_format_limits.json);
* torch's float8_e4m3fn / float8_e5m2 conversions (a library routine,
  used only as a cross-check of the codec);
* exact rational arithmetic (fractions.Fraction / Python integers);
* closed forms and special cases (lossless inputs, block == per-channel);
* the 70B checkpoint figures printed on the pages (storage closed form).
"""
import bisect
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.fp8dq_oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# Independent helpers (exact arithmetic, library tables)
# ----------------------------------------------------------------------------
def torch_fp8_table(dtype) -> np.ndarray:
    b = torch.arange(256, dtype=torch.uint8).view(dtype)
    return b.to(torch.float64).numpy()


TORCH_E4M3 = torch_fp8_table(torch.float8_e4m3fn)
TORCH_E5M2 = torch_fp8_table(torch.float8_e5m2)
# non-negative finite E4M3 grid as exact rationals, from torch's decode
GRID_FR = [Fraction(float(v)) for v in TORCH_E4M3[:127]]


def exact_rne_code(q: Fraction) -> int:
    """Nearest E4M3 magnitude code to |q| (ties to even code, saturating)."""
    a = abs(q)
    if a >= GRID_FR[-1]:
        return 126
    lo = bisect.bisect_right(GRID_FR, a) - 1
    hi = lo + 1
    d_lo, d_hi = a - GRID_FR[lo], GRID_FR[hi] - a
    if d_lo < d_hi:
        return lo
    if d_hi < d_lo:
        return hi
    return lo if lo % 2 == 0 else hi


def exact_rn_f32(q: Fraction) -> float:
    """Round a non-negative rational to the nearest fp32 (ties to even)."""
    if q == 0:
        return 0.0
    # exponent e with 2**e <= q < 2**(e+1)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    e = max(e, -126)                    # below: fixed subnormal spacing
    ulp = Fraction(2) ** (e - 23)
    n, r = divmod(q, ulp)
    n = int(n)
    if r > ulp / 2 or (r == ulp / 2 and n % 2 == 1):
        n += 1
    return float(n * ulp)


def all_positive_finite_bf16() -> np.ndarray:
    bits = np.arange(1, 0x7F80, dtype=np.uint16)      # +denormals .. max
    return bits


# ----------------------------------------------------------------------------
# Checks (each returns normally or raises AssertionError)
# ----------------------------------------------------------------------------
def check_format_limits(o):
    g = json.load(open(os.path.join(GOLD, "fp8_format_limits.json")))
    e4 = o.fp8_decode_table(g["e4m3"]["exponent_bits"], g["e4m3"]["mantissa_bits"], True)
    e5 = o.fp8_decode_table(g["e5m2"]["exponent_bits"], g["e5m2"]["mantissa_bits"], False)
    assert np.nanmax(e4[np.isfinite(e4)]) == g["e4m3"]["max"]
    assert np.nanmax(e5[np.isfinite(e5)]) == g["e5m2"]["max"]
    assert o.E4M3_MAX == g["e4m3"]["max"]
    # the 448 maximum forces the variant with only S.1111.111 as NaN
    assert set(np.flatnonzero(np.isnan(o.E4M3_VALUES))) == {0x7F, 0xFF}
    assert o.E4M3_VALUES[0x08] == 2.0 ** -6 and o.E4M3_VALUES[0x01] == 2.0 ** -9


def check_decode_vs_torch(o):
    for mine, ref in ((o.E4M3_VALUES, TORCH_E4M3), (o.E5M2_VALUES, TORCH_E5M2)):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan)
        assert np.array_equal(mine[~nan], ref[~nan])
        assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def check_roundtrip(o):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert len(codes) == 254
    assert np.array_equal(o.e4m3_encode(o.e4m3_decode(codes)), codes)


def check_encode_vs_torch_all_bf16(o):
    """Every finite bf16 with |v| <= 448, both signs, vs torch's RNE cast."""
    pos = np.arange(0, 0x7F80, dtype=np.uint16)
    bits = np.concatenate([pos, pos | np.uint16(0x8000)])
    v = o.bf16_to_f64(bits)
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3_encode(v), ref)


def check_saturation(o):
    v = np.array([448.0, 463.99, 464.0, 1e6, 57344.0, -500.0, -1e30])
    got = o.e4m3_encode(v)
    assert np.array_equal(got, np.array([0x7E] * 5 + [0xFE] * 2, np.uint8))


def check_signed_zero(o):
    got = o.e4m3_encode(np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10)]))
    # 2**-10 is the tie between 0 and 2**-9: even code 0 wins
    assert np.array_equal(got, np.array([0x00, 0x80, 0x00, 0x80, 0x00, 0x80], np.uint8))


def check_quantizer_exact_rational(o, n=4000, seed=7):
    """x / s rounded exactly (Fraction) vs the oracle, random + near-tie."""
    rng = np.random.default_rng(seed)
    # random bf16 x and fp32 s with |x|/s inside the E4M3 range
    xb = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    x = synth.bf16_bits_to_f32(xb).astype(np.float64)
    s = (np.abs(x) / rng.uniform(1e-3, 448, n)).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1.0))
    # near ties: s = M' * 2**k * (1 + j*2**-23), x = bf16(M * s) for midpoints M
    mids = [(GRID_FR[i] + GRID_FR[i + 1]) / 2 for i in range(126)]
    xt, st = [], []
    for i in range(n // 2):
        mval = float(mids[rng.integers(0, 126)])
        k = int(rng.integers(-8, 8))
        base = np.float32(2.0 ** k)
        jj = int(rng.integers(-3, 4))
        s_ = np.float32(float(base) * (1 + jj * 2.0 ** -23))
        xv = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
            np.array([mval * float(s_)], np.float32)))[0]
        xt.append(float(xv) * (1 if rng.integers(0, 2) else -1))
        st.append(s_)
    x = np.concatenate([x, np.array(xt)])
    s = np.concatenate([s, np.array(st, np.float32)])
    got = o.quantize_with_scale(x, s)
    for xi, si, gi in zip(x, s, got):
        q = Fraction(float(xi)) / Fraction(float(si))
        code = exact_rne_code(q) | (0x80 if np.signbit(xi) else 0)
        assert gi == code, (xi, si, gi, code)


def check_scale_exhaustive(o):
    """RN_fp32(amax/448) for every positive finite bf16 amax, exactly."""
    bits = all_positive_finite_bf16()
    amax = o.bf16_to_f64(bits)
    got = o.scale_from_amax(amax)
    want = np.array([exact_rn_f32(Fraction(float(a)) / 448) for a in amax],
                    dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # and the fp32 IEEE division gives the same bits (used by the kernels'
    # readers as the plain definition of the step)
    f32div = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), f32div.view(np.uint32))


def check_row_invariants(o):
    """Properties any correct per-row quantizer has, on synthetic rows."""
    xb = synth.activations(64, 1024, 11, 12)
    xb[5] = 0                                       # an all-zero row
    xb[6, :] = synth.f32_to_bf16_bits(np.full(1024, -0.0, np.float32))
    q, s = o.quant_per_row(xb)
    x = o.bf16_to_f64(xb)
    amax = np.max(np.abs(x), axis=1)
    for r in range(64):
        if amax[r] == 0:
            assert s[r] == 0
            assert np.array_equal(q[r], np.where(np.signbit(x[r]), 0x80, 0).astype(np.uint8))
            continue
        a = int(np.argmax(np.abs(x[r])))
        assert q[r, a] & 0x7F == 0x7E                     # argmax -> 448
        assert abs(448.0 * float(s[r]) - amax[r]) <= 2.0 ** -24 * amax[r]
        v = o.e4m3_decode(q[r]) * float(s[r])
        # |val*s - x| <= half an E4M3 step of x/s, times s
        t = np.abs(x[r] / float(s[r]))
        e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
        half_step = 2.0 ** (e - 4) * float(s[r])
        assert np.all(np.abs(v - x[r]) <= half_step * (1 + 1e-12))
        order = np.argsort(x[r], kind="stable")
        assert np.all(np.diff(o.e4m3_decode(q[r])[order]) >= 0)   # monotone


def check_tiny_gemm_bruteforce(o, seed=3):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (8, 8, 8), (2, 3, 128)]:
        qx = rng.choice(finite, size=(M, K))
        qw = rng.choice(finite, size=(N, K))
        sx = rng.uniform(0.01, 2, M).astype(np.float32)
        sw = rng.uniform(0.01, 2, N).astype(np.float32)
        y = o.linear_per_channel(qx, sx, qw, sw)
        fx = [[Fraction(float(TORCH_E4M3[c])) for c in row] for row in qx]
        fw = [[Fraction(float(TORCH_E4M3[c])) for c in row] for row in qw]
        for m in range(M):
            for n in range(N):
                P = sum(a * b for a, b in zip(fx[m], fw[n]))
                want = P * Fraction(float(sx[m])) * Fraction(float(sw[n]))
                assert abs(Fraction(y[m, n]) - want) <= abs(want) * Fraction(1, 2 ** 50)


def check_block_bruteforce(o, seed=8):
    """Block epilogue with distinct per-group scales, exact rationals."""
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M, N, K = 3, 256, 384
    qx = rng.choice(finite, size=(M, K))
    qw = rng.choice(finite, size=(N, K))
    sx = rng.uniform(0.01, 2, (M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.01, 2, (N // 128, K // 128)).astype(np.float32)
    y = o.linear_block(qx, sx, qw, sw)
    for m, n in [(0, 0), (1, 127), (2, 128), (0, 255), (2, 200)]:
        want = Fraction(0)
        for g in range(K // 128):
            P = sum(Fraction(float(TORCH_E4M3[qx[m, k]])) * Fraction(float(TORCH_E4M3[qw[n, k]]))
                    for k in range(g * 128, (g + 1) * 128))
            want += P * Fraction(float(sx[m, g])) * Fraction(float(sw[n // 128, g]))
        assert abs(Fraction(y[m, n]) - want) <= abs(want) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 60)


def check_gemm_exact_int(o, seed=4):
    """Large K: P * 2**18 equals an int64 product of code values * 2**9."""
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    qx = rng.choice(finite, size=(4, 28672))
    qw = rng.choice(finite, size=(3, 28672))
    P = o.gemm_codes(qx, qw)
    ix = (TORCH_E4M3[qx] * 512).astype(np.int64)
    iw = (TORCH_E4M3[qw] * 512).astype(np.int64)
    assert np.array_equal((P * 2.0 ** 18).astype(np.int64), ix @ iw.T)


def check_lossless_linear(o, seed=5):
    """Rows built as 2**a * (E4M3 values) with one +-448: quantization is
    lossless, so the FP8 linear equals the plain product X W^T."""
    rng = np.random.default_rng(seed)
    finite = [c for c in range(127)]
    M, N, K = 6, 5, 256
    X = np.empty((M, K)); W = np.empty((N, K))
    for mat, R in ((X, M), (W, N)):
        for r in range(R):
            codes = rng.choice(finite, size=K) | (rng.integers(0, 2, K) << 7)
            codes[rng.integers(0, K)] = 0x7E if rng.integers(0, 2) else 0xFE
            mat[r] = TORCH_E4M3[codes.astype(np.uint8)] * 2.0 ** int(rng.integers(-12, 4))
    xb = synth.f32_to_bf16_bits(X.astype(np.float32))
    wb = synth.f32_to_bf16_bits(W.astype(np.float32))
    assert np.array_equal(o.bf16_to_f64(xb), X) and np.array_equal(o.bf16_to_f64(wb), W)
    y, qx, sx, qw, sw = o.fp8_linear(xb, wb)
    assert np.array_equal(o.e4m3_decode(qx) * sx[:, None].astype(np.float64), X)
    assert np.allclose(y, X @ W.T, rtol=1e-14, atol=0)


def check_block_equals_channel(o, seed=6):
    """Every 128-group of a row with the same amax and every 128x128 block
    of a 128-row band with the same amax: block == per-channel result."""
    rng = np.random.default_rng(seed)
    M, N, K = 4, 256, 384

    def build(R, band):
        a = rng.standard_normal((R, K)).astype(np.float32)
        peak = rng.uniform(0.5, 4, (R + band - 1) // band).astype(np.float32)
        for r in range(R):
            pk = np.float32(peak[r // band])
            for g in range(K // 128):
                seg = a[r, g * 128:(g + 1) * 128]
                np.clip(seg, -0.9 * pk, 0.9 * pk, out=seg)
                seg[rng.integers(0, 128)] = pk if rng.integers(0, 2) else -pk
        return synth.f32_to_bf16_bits(a)

    xb = build(M, 1)
    wb = build(N, 128)
    y_c, qx_c, sx_c, qw_c, sw_c = o.fp8_linear(xb, wb)
    y_b, qx_b, sx_b, qw_b, sw_b = o.fp8_linear_block(xb, wb)
    assert np.array_equal(qx_c, qx_b) and np.array_equal(qw_c, qw_b)
    assert np.array_equal(np.repeat(sx_c[:, None], K // 128, 1), sx_b)
    assert np.allclose(y_b, y_c, rtol=1e-13, atol=0)


def check_tolerance(o):
    """The comparison of bf16 outputs: |y - y_ref| <= 1e-3 + 1e-2 |y_ref|
    (spec tolerance), measured from the exact value y_ref. Values just
    inside the bound pass, values just outside fail; the bound scales with
    |y_ref|, not with the value under test."""
    cases = [  # (y_ref, y, expected)
        (0.0, 1e-3 * (1 - 1e-9), True), (0.0, -1e-3 * (1 - 1e-9), True),
        (0.0, 1e-3 * (1 + 1e-6), False), (0.0, 5e-3, False),
        (10.0, 10.101 - 1e-9, True), (10.0, 10.101 + 1e-6, False),
        (10.0, 9.899 + 1e-9, True), (10.0, 9.899 - 1e-6, False),
        (-3.0, -3.031 + 1e-9, True), (-3.0, -3.031 - 1e-6, False),
        # 0.98905 is 0.01095 from 1.0: inside 1e-3 + 1e-2 * |y_ref| = 0.011,
        # outside a bound taken from |y| (0.0108905)
        (1.0, 0.98905, True),
        (1e6, 1e6 * 1.01, True), (1e6, 1e6 * 1.0101, False),
    ]
    ref = np.array([c[0] for c in cases])
    got = np.array([c[1] for c in cases])
    want = np.array([c[2] for c in cases])
    res = o.within_tolerance(got, ref)
    assert res.dtype == bool and res.shape == ref.shape
    assert np.array_equal(res, want), np.argwhere(res != want).ravel()


def check_storage_closed_form(o):
    """Per-output-channel scales reproduce the 70B checkpoint figures."""
    g = json.load(open(os.path.join(GOLD, "llama31_70b_fp8_storage.json")))
    a = g["architecture"]
    h, I, L, V = a["hidden"], a["intermediate"], a["layers"], a["vocab"]
    kv = a["kv_heads"] * a["head_dim"]
    linears = [(h, h), (kv, h), (kv, h), (h, h), (I, h), (I, h), (h, I)]
    w_elems = L * sum(n * k for n, k in linears)
    # one scale per output channel (the rows of each W [N,K])
    s_elems = L * sum(n for n, _ in linears)
    other = L * 2 * h + h + 2 * V * h          # norms, embedding, lm_head
    params = w_elems + s_elems + other
    nbytes = w_elems * 1 + 2 * (s_elems + other)   # E4M3: one byte
    assert round(params / 1e9, 2) == g["params_billion_printed"]
    assert round(nbytes / 1e9, 2) == g["bytes_gb_printed"]
    assert round(nbytes / 2 ** 30, 1) == g["bytes_gib_printed"]
    assert L * len(linears) == g["weight_scale_tensors"]
    assert abs((2 * w_elems + 2 * other) / 1e9 - g["bf16_gb_approx"]) < 2


CHECKS = [check_format_limits, check_decode_vs_torch, check_roundtrip,
          check_encode_vs_torch_all_bf16, check_saturation, check_signed_zero,
          check_quantizer_exact_rational, check_scale_exhaustive,
          check_row_invariants, check_tiny_gemm_bruteforce,
          check_block_bruteforce, check_gemm_exact_int, check_lossless_linear,
          check_block_equals_channel, check_storage_closed_form, check_tolerance]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(O)


# ----------------------------------------------------------------------------
# Planted mistakes: each mutated oracle must fail at least one check.
# ----------------------------------------------------------------------------
def _ties_away(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    grid = O.E4M3_VALUES[:127]
    lo = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    mid = (grid[lo] + grid[hi]) / 2
    code = np.where(a < mid, lo, hi)
    code = np.where(a >= 448, 126, code)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def _truncating(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    grid = O.E4M3_VALUES[:127]
    lo = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 126)
    return (lo | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


_ORIG_ENC = O.e4m3_encode


def _no_sign_of_zero(v):
    c = _ORIG_ENC(v)
    return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)

MUTATIONS = {
    "tolerance_from_tested_value": ("within_tolerance",
                                    lambda g, r, rtol=1e-2, atol=1e-3: np.abs(np.asarray(g) - r)
                                    <= atol + rtol * np.abs(np.asarray(g))),
    "tolerance_rtol_atol_swapped": ("within_tolerance",
                                    lambda g, r, rtol=1e-2, atol=1e-3: np.abs(np.asarray(g) - r)
                                    <= rtol + atol * np.abs(np.asarray(r))),
    "tolerance_strict_relative": ("within_tolerance",
                                  lambda g, r, rtol=1e-2, atol=1e-3: np.abs(np.asarray(g) - r)
                                  <= rtol * np.abs(np.asarray(r))),
    "ties_away_from_zero": ("e4m3_encode", _ties_away),
    "truncation": ("e4m3_encode", _truncating),
    "drops_sign_of_zero": ("e4m3_encode", _no_sign_of_zero),
    "fnuz_max_240": ("scale_from_amax",
                     lambda a: (np.asarray(a, np.float64) / 240.0).astype(np.float32)),
    "scale_not_rounded_to_f32": ("quantize_with_scale",
                                 lambda x, s: _ORIG_ENC(np.asarray(x) / np.asarray(s, np.float64) * (1 + 2.0 ** -30))),
    "transposed_weight": ("gemm_codes",
                          lambda qx, qw: O.e4m3_decode(qx) @ O.e4m3_decode(qw)[:, ::-1].T),
    "missing_act_scale": ("linear_per_channel",
                          lambda qx, sx, qw, sw: O.gemm_codes(qx, qw) * np.asarray(sw, np.float64)[None, :]),
    "block_scale_after_sum": ("linear_block",
                              lambda qx, sx, qw, sw, block=128: O.gemm_codes(qx, qw)
                              * np.asarray(sx, np.float64).mean(1)[:, None]
                              * np.repeat(np.asarray(sw, np.float64), 128, 0).mean(1)[None, :]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    failed = []
    for check in CHECKS:
        try:
            check(O)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"mutation {name} slipped past every pin"
