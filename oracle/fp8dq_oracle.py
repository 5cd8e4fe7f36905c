"""CPU oracle of the FP8-Dynamic linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

It is plain numpy in float64, written to be checked by eye against the
definitions on the pages (cited per function as page title + section):

* E4M3 / E5M2 number formats -- "Llama 3 精读实录" page, §2.1 (two FP8
  formats): E4M3 has 4 exponent and 3 mantissa bits with largest value 448;
  E5M2 has 5 and 2 with largest value 57344.
* Weights: static FP8, one scale per output channel from a min/max
  observer -- Llama-3.1-8B-Instruct-FP8-Dynamic page, FP8 dynamic
  quantization table (weights row); Llama-3.1-70B-FP8-Dynamic page, §1.2.
* Activations: dynamic FP8, one scale per token computed at run time --
  same table (input activations row); Llama-3.1-70B-FP8-Dynamic page, §1.2.
* Block variant: one scale per 128x128 weight block, activations grouped by
  128 and quantized dynamically -- Llama-3.2-3B-Instruct-FP8-Block page,
  FP8 block quantization table (block_structure, input activations rows).
* lm_head is not quantized -- all three walk-through pages (ignore list).
  The oracle simply has no lm_head function.

Readings where the pages are silent (listed with reasons in the design
notes): the scale is fp32 ``RN(amax / 448)``; the rounded quotient is the
exact ``x / s`` with the stored fp32 scale; rounding is to nearest with
ties to the even code, saturating at +-448; the sign of zero is kept; an
all-zero unit has scale 0 and zero codes; the epilogue is
``acc * sx[m] * sw[n]`` with no bias.

Parity status: every function here is pinned by CPU tests against closed
forms, brute force with exact rationals, a library cross-check of the codec
and special cases (tests/test_oracle_pins.py). The pages print no worked
numeric example of the quantizer or the GEMM, so no pin comes from a
printed value of the method itself.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0      # largest finite E4M3 value (two-formats section)
E5M2_MAX = 57344.0    # largest finite E5M2 value (same section)
BLOCK = 128           # block edge / activation group width (block table)


# ----------------------------------------------------------------------------
# Inputs: bfloat16 bit patterns -> exact float64
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# FP8 formats, from their bit fields ("Llama 3 精读实录" page, §2.1)
# ----------------------------------------------------------------------------
def fp8_decode_table(exp_bits: int, man_bits: int, finite_top: bool) -> np.ndarray:
    """Value of each of the 256 codes of a sign/exponent/mantissa byte.

    bias = 2**(exp_bits-1) - 1. Exponent field 0 is subnormal
    (m / 2**man_bits * 2**(1-bias)). ``finite_top`` selects the variant
    whose all-ones exponent still holds finite numbers and only the
    all-ones mantissa there is NaN (the variant whose maximum is 448 for
    E4M3); otherwise the all-ones exponent is Inf (mantissa 0) or NaN, as
    in IEEE (the variant whose maximum is 57344 for E5M2).
    """
    bias = 2 ** (exp_bits - 1) - 1
    emax_field = 2 ** exp_bits - 1
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> man_bits) & emax_field
        m = code & (2 ** man_bits - 1)
        if e == emax_field and not finite_top:
            out[code] = sign * np.inf if m == 0 else np.nan
            continue
        if e == emax_field and finite_top and m == 2 ** man_bits - 1:
            out[code] = np.nan
            continue
        if e == 0:
            out[code] = sign * (m / 2.0 ** man_bits) * 2.0 ** (1 - bias)
        else:
            out[code] = sign * (1.0 + m / 2.0 ** man_bits) * 2.0 ** (e - bias)
    return out


E4M3_VALUES = fp8_decode_table(4, 3, finite_top=True)
E5M2_VALUES = fp8_decode_table(5, 2, finite_top=False)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each finite float64 ``v``.

    Round to nearest; a value exactly halfway between two neighbours takes
    the one whose code is even (mantissa LSB 0). Magnitudes at or above
    448 give 448 (saturation: this format has no infinity). The sign bit is
    copied from ``v``, so -0.0 and negative values that round to zero give
    0x80.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input is outside the contract")
    a = np.abs(v)
    grid = E4M3_VALUES[:127]            # codes 0x00..0x7E, increasing values
    lo = np.searchsorted(grid, a, side="right") - 1     # grid[lo] <= a
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    mid = (grid[lo] + grid[hi]) / 2.0   # exact: five significant bits
    code = np.where(a < mid, lo, np.where(a > mid, hi,
                                          np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= E4M3_MAX, 126, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


# ----------------------------------------------------------------------------
# Scale and quantization of one unit (a token row, a 128-group, a weight
# row or a 128x128 block)
# ----------------------------------------------------------------------------
def scale_from_amax(amax: np.ndarray) -> np.ndarray:
    """fp32 scale = RN_fp32(amax / 448); amax is the unit's largest |x|.

    The float64 quotient is rounded once more to float32 (numpy's cast is
    round-to-nearest-even). An all-zero unit gets scale 0.
    """
    return (np.asarray(amax, dtype=np.float64) / E4M3_MAX).astype(np.float32)


def quantize_with_scale(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E4M3 code of x / s, with ``s`` (fp32, broadcast to x) as stored.

    The quotient is formed in float64 from the fp32 scale. A unit with
    s == 0 is all zeros and keeps each element's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    s64 = np.broadcast_to(np.asarray(s, dtype=np.float32).astype(np.float64),
                          x.shape)
    safe = np.where(s64 > 0, s64, 1.0)
    q = np.where(s64 > 0, x / safe, np.copysign(0.0, x))
    return e4m3_encode(q)


def quant_per_row(x_bits: np.ndarray):
    """Per-token activations / per-output-channel weights.

    One unit per row of a [R, K] bf16 matrix: amax over the row (symmetric
    min/max: the larger of |min| and |max|), then scale, then codes.
    Returns (codes uint8 [R,K], scales fp32 [R]).
    """
    x = bf16_to_f64(x_bits)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0])
    s = scale_from_amax(amax)
    return quantize_with_scale(x, s[:, None]), s


def quant_per_group(x_bits: np.ndarray, group: int = BLOCK):
    """Activations of the block variant: one unit per row per 128 columns.

    Returns (codes uint8 [R,K], scales fp32 [R, K/group]).
    """
    x = bf16_to_f64(x_bits)
    R, K = x.shape
    if K % group:
        raise ValueError("K must be a multiple of the group width")
    g = x.reshape(R, K // group, group)
    s = scale_from_amax(np.max(np.abs(g), axis=2))
    q = quantize_with_scale(g, s[:, :, None])
    return q.reshape(R, K), s


def quant_weight_block(w_bits: np.ndarray, block: int = BLOCK):
    """Weights of the block variant: one unit per 128x128 block of W [N,K].

    Returns (codes uint8 [N,K], scales fp32 [N/block, K/block]).
    """
    w = bf16_to_f64(w_bits)
    N, K = w.shape
    if N % block or K % block:
        raise ValueError("N and K must be multiples of the block edge")
    b = w.reshape(N // block, block, K // block, block)
    s = scale_from_amax(np.max(np.abs(b), axis=(1, 3)))
    q = quantize_with_scale(b, s[:, None, :, None])
    return q.reshape(N, K), s


# ----------------------------------------------------------------------------
# GEMM core and epilogues
# ----------------------------------------------------------------------------
def gemm_codes(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """P[m,n] = sum_k val(qx[m,k]) * val(qw[n,k]), in float64.

    Every code value is a multiple of 2**-9 below 2**9, so every product is
    a multiple of 2**-18 below 2**18 and every partial sum is exact in
    float64 while K <= 2**17: P is exact, whatever order BLAS sums in.
    """
    if qx.shape[1] > 2 ** 17:
        raise ValueError("K beyond the exact-accumulation bound")
    a = e4m3_decode(qx)
    b = e4m3_decode(qw)
    return a @ b.T


def linear_per_channel(qx, sx, qw, sw) -> np.ndarray:
    """y[m,n] = P[m,n] * sx[m] * sw[n] (float64, not rounded to bf16)."""
    P = gemm_codes(qx, qw)
    return P * np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]


def linear_block(qx, sx, qw, sw, block: int = BLOCK) -> np.ndarray:
    """y[m,n] = sum_g P_g[m,n] * sx[m,g] * sw[n//128, g] (float64).

    P_g sums k over the g-th 128-wide group only: the scales differ per
    group, so they are applied before the groups are added.
    """
    M, K = qx.shape
    N = qw.shape[0]
    G = K // block
    y = np.zeros((M, N), dtype=np.float64)
    swn = np.repeat(np.asarray(sw, np.float64), block, axis=0)  # [N, G]
    for g in range(G):
        ks = slice(g * block, (g + 1) * block)
        Pg = gemm_codes(qx[:, ks], qw[:, ks])
        y += Pg * np.asarray(sx, np.float64)[:, g][:, None] * swn[:, g][None, :]
    return y


def fp8_linear(x_bits, w_bits):
    """The whole FP8-Dynamic linear from bf16 inputs (per-token / per-channel).

    Returns (y float64 [M,N], qx, sx, qw, sw).
    """
    qx, sx = quant_per_row(x_bits)
    qw, sw = quant_per_row(w_bits)
    return linear_per_channel(qx, sx, qw, sw), qx, sx, qw, sw


def fp8_linear_block(x_bits, w_bits):
    """The block variant from bf16 inputs. Returns (y, qx, sx, qw, sw)."""
    qx, sx = quant_per_group(x_bits)
    qw, sw = quant_weight_block(w_bits)
    return linear_block(qx, sx, qw, sw), qx, sx, qw, sw


# ----------------------------------------------------------------------------
# Comparison helpers
# ----------------------------------------------------------------------------
def f64_to_bf16_rne(y: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), as float64.

    Used only as a diagnostic (the fraction of outputs that equal the
    correctly rounded result); the tolerance test uses the float64 value.
    """
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)                 # y = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)            # below 2**-126: fixed spacing 2**-133
    scaled = np.ldexp(y, 8 - e)        # 8 significant bits above the point
    return np.ldexp(np.round(scaled), e - 8)   # np.round: ties to even


def within_tolerance(y_gpu, y_ref, rtol: float = 1e-2, atol: float = 1e-3):
    """Elementwise |y_gpu - y_ref| <= atol + rtol*|y_ref| (returns bool array)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    return np.abs(y_gpu - y_ref) <= atol + rtol * np.abs(y_ref)


# ----------------------------------------------------------------------------
# Producers of the quantizer's input, fused with it downstream ("next" rows).
# Each is defined as its exact real-valued formula, evaluated in float64 and
# rounded once to bfloat16 (the model's activation dtype); the FP8 per-token
# quantization then applies to that bf16 tensor exactly as above.
# ----------------------------------------------------------------------------
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
RMS_EPS = 1e-5   # RMSNorm epsilon ("Llama 3 精读实录" page, §1.3)


def f64_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit pattern: round to nearest, ties to even, sign
    of zero kept, magnitudes that round past the largest finite bf16 -> inf."""
    y = np.asarray(y, dtype=np.float64)
    r = f64_to_bf16_rne(y)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, y), r)
    r = np.copysign(r, y)                      # keep the sign of zero
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _near_bf16_midpoint(h: np.ndarray, rel: float = 2.0 ** -30) -> np.ndarray:
    """True where a float64 value lies within ``rel`` (relative) of a bf16
    rounding midpoint -- there the float64 evaluation error could decide the
    rounding, so the exact value has to."""
    h = np.asarray(h, np.float64)
    m, e = np.frexp(h)
    e = np.maximum(e, -125)
    scaled = np.ldexp(h, 8 - e)                # bf16 ulps above the point
    frac = np.abs(scaled - np.floor(scaled) - 0.5)
    return np.isfinite(h) & (h != 0) & (frac < rel * 256)


def _exact_round_bf16(value) -> int:
    """Exact round-to-nearest-even of a Decimal / Fraction to bf16 bits."""
    from fractions import Fraction
    q = Fraction(value)
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    n = a / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (k & 1)):
        k += 1
    val = k * ulp
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    return sign | (int(np.float32(float(val)).view(np.uint32)) >> 16) & 0x7FFF


def silu_mul_bf16(gu_bits: np.ndarray) -> np.ndarray:
    """SwiGLU's gated product h = bf16(silu(g) * u), silu(g) = g / (1 + e^-g).

    g is the first half of the columns of ``gu_bits`` [R, 2I] and u the
    second half: the gate and up branches of one fused gate_up GEMM, which
    the "Llama 3 精读实录" page (§1.3) says are computed separately and then
    multiplied elementwise. Returns bf16 bits [R, I].

    Evaluated in float64. Where the float64 value lies within 2^-30 of the
    midpoint m between two bf16 neighbours, the side of m is decided exactly
    (for g > 37 float64 rounds silu(g) to g and can turn h into an exact tie
    that the true value misses): with s = 1 / (1 + e^-g) > 0,
        h - m = s * ((g*u - m) - m * e^-g),
    where g*u - m is an exact rational and m * e^-g is taken to 60 digits.
    """
    from decimal import Decimal, localcontext
    from fractions import Fraction
    gu = bf16_to_f64(gu_bits)
    half = gu.shape[1] // 2
    g, u = gu[:, :half], gu[:, half:]
    with np.errstate(over="ignore"):
        sil = g / (1.0 + np.exp(-g))           # e^-g = inf -> silu = -0
    h = sil * u
    out = f64_to_bf16_bits(h)
    for r, c in zip(*np.nonzero(_near_bf16_midpoint(h))):
        gv, uv, hv = float(g[r, c]), float(u[r, c]), float(h[r, c])
        # the two bf16 neighbours of hv and their midpoint
        lo_bits = int(np.float32(hv).view(np.uint32)) >> 16     # truncation (|.| down)
        lo = float(np.uint32(lo_bits << 16).view(np.float32))
        hi = float(np.uint32((lo_bits + 1) << 16).view(np.float32))
        m = (Fraction(lo) + Fraction(hi)) / 2
        a = Fraction(gv) * Fraction(uv) - m
        with localcontext() as ctx:
            ctx.prec = 60
            try:
                b = Fraction(Decimal(m.numerator) / Decimal(m.denominator) * Decimal(-gv).exp())
            except ArithmeticError:   # e^-g beyond any decimal exponent: g < 0 huge
                b = None
        if b is None:
            side = -1 if hv > 0 else 1   # unreachable for near-midpoint values
        else:
            if b == 0 and m != 0:
                # e^-g below the decimal range (g > 2.3e6): m * e^-g is not
                # zero but smaller than any nonzero a, and has the sign of m
                d = a if a != 0 else -m
            else:
                d = a - b
            side = (d > 0) - (d < 0)     # sign of h - m
        up = side * (1 if hv > 0 else -1)            # sign of |h| - |m|
        if up > 0 or (up == 0 and (lo_bits & 1)):
            out[r, c] = lo_bits + 1
        else:
            out[r, c] = lo_bits
    return out


def silu_mul_quant(gu_bits: np.ndarray):
    """Per-token FP8 quantization of h = silu_mul_bf16(gu). (codes, scales)."""
    return quant_per_row(silu_mul_bf16(gu_bits))


def rmsnorm_bf16(x_bits: np.ndarray, gamma_bits: np.ndarray,
                 eps: float = RMS_EPS) -> np.ndarray:
    """RMSNorm h = bf16(gamma * x / sqrt(mean(x^2) + eps)) per row of x [R, H].

    eps = 1e-5 and the norm before attention and the MLP ("Llama 3 精读实录"
    page, §1.3); the page keeps RMSNorm itself in bf16 (§5.3), so its output
    is the bf16 tensor that the FP8 quantization then reads. Evaluated in
    float64; elements within 2^-30 of a bf16 rounding midpoint are evaluated
    again exactly (rational mean square, 60-digit square root).
    """
    from decimal import Decimal, localcontext
    from fractions import Fraction
    x = bf16_to_f64(x_bits)
    gam = bf16_to_f64(gamma_bits)[None, :]
    ms = np.mean(x * x, axis=1, keepdims=True)
    h = gam * x / np.sqrt(ms + eps)
    out = f64_to_bf16_bits(h)
    near = _near_bf16_midpoint(h)
    for r in np.unique(np.nonzero(near)[0]):   # exact evaluation near midpoints
        with localcontext() as ctx:
            ctx.prec = 60
            q = sum(Fraction(float(v)) ** 2 for v in x[r]) / x.shape[1] + Fraction(eps)
            rinv = 1 / (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()
            for c in np.nonzero(near[r])[0]:
                out[r, c] = _exact_round_bf16(Decimal(float(gam[0, c])) *
                                              Decimal(float(x[r, c])) * rinv)
    return out


def rmsnorm_quant(x_bits, gamma_bits, eps: float = RMS_EPS):
    """Per-token FP8 quantization of rmsnorm_bf16(x, gamma). (codes, scales)."""
    return quant_per_row(rmsnorm_bf16(x_bits, gamma_bits, eps))


def nearest_rank(n: int, permille: int) -> int:
    """1-based rank of the permille/1000 quantile of n values, nearest-rank
    method: ceil(p * n), kept inside [1, n]. Exact integer arithmetic."""
    k = -((-permille * n) // 1000)
    return int(min(max(k, 1), n))


def calib_amax(x_bits: np.ndarray, lo_permille: int = 1, hi_permille: int = 999) -> float:
    """Static calibration range of a tensor: the larger magnitude of its
    lo- and hi-quantiles (P0.1 and P99.9 by default), instead of max |x| --
    the "Llama 3 精读实录" page, §2.2 (percentiles as the dynamic range)."""
    v = np.sort(bf16_to_f64(x_bits).ravel())
    n = v.size
    if n == 0:
        return 0.0
    lo = v[nearest_rank(n, lo_permille) - 1]
    hi = v[nearest_rank(n, hi_permille) - 1]
    return float(max(abs(lo), abs(hi)))


def calib_scale(x_bits, lo_permille: int = 1, hi_permille: int = 999) -> np.float32:
    """fp32 static per-tensor scale RN(calib_amax / 448)."""
    return scale_from_amax(np.array([calib_amax(x_bits, lo_permille, hi_permille)]))[0]


def quant_static(x_bits: np.ndarray, s) -> np.ndarray:
    """E4M3 codes of x / s with one fixed (static) fp32 scale for the whole
    tensor. Values beyond 448 * s saturate to +-448 (codes 0x7E / 0xFE)."""
    return quantize_with_scale(bf16_to_f64(x_bits), np.float32(s))


def kv_quant_scatter(k_bits: np.ndarray, v_bits: np.ndarray, slots: np.ndarray):
    """FP8 KV cache write ("Llama 3 精读实录" page, §4.1: FP8 also compresses
    the KV cache): each token row of K and V [T, width] is quantized per
    token and lands in cache row slots[t] (negative: not written).

    Returns {slot: (k_codes, k_scale, v_codes, v_scale)} for the written rows.
    """
    qk, sk = quant_per_row(k_bits)
    qv, sv = quant_per_row(v_bits)
    out = {}
    for t, slot in enumerate(np.asarray(slots).tolist()):
        if slot >= 0:
            out[int(slot)] = (qk[t], sk[t], qv[t], sv[t])
    return out
