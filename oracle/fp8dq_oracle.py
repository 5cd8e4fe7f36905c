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
