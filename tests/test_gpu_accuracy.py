"""GPU accuracy of the FP8 GEMM against the exact sum and against the
measured accumulation law of the FP8 matrix instructions (tests/mfma_law.py).

* Constructed codes whose groups of 8 mix one large product with small ones:
  the prefill kernels (16x16x128 and 32x32x64 MFMAs, per-channel and block)
  must give exactly what the law predicts, and the decode kernels, which run
  the token row's large codes through their own MFMA, the exact sum.
* The longest rows the boundary accepts (K = FP8DQ_MAX_K = 131072): decode
  within the tolerance of the oracle; prefill within the tolerance of the
  law's prediction (and the nominal tolerance counted).
* Every output of the four 70B decode linears at 1, 8, 32 and 64 tokens
  within the tolerance of the oracle.
* Per-channel scales near both ends of the fp32 range on every kernel path:
  finite outputs, within the tolerance of the law's prediction.
"""
import numpy as np
import pytest
import torch

import oracle.fp8dq_oracle as O
import synth
from gpu_util import (RTOL, ATOL, assert_y_close, dev, dev_bf16, ensure_built,
                      host_bf16_f64, say)
from mfma_law import law_sum, law_sum_split

pytestmark = pytest.mark.gpu

MAX_K = 131072


@pytest.fixture(scope="module")
def F():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ensure_built()


def constructed(R: int, C: int, K: int, seed: int):
    """R token-row and C weight-row patterns of E4M3 values, K a multiple of
    16. Every group of 8 starts with a large product (x code 16..448 times a
    weight of 1..2) whose sign alternates by group, so the large products
    cancel in pairs; the other 7 products are small (2^-7 .. 2)."""
    rng = np.random.default_rng(seed)
    big = np.array([16.0, 24.0, 32.0, 64.0, 96.0, 192.0, 256.0, 448.0])
    small_x = np.array([2.0 ** -4, 0.09375, 0.125, 0.1875, 0.25, 0.375, 0.5, 0.75, 1.0])
    small_w = np.array([2.0 ** -3, 0.1875, 0.25, 0.375, 0.5, 0.625, 0.75, 1.0, 1.5, 2.0])
    G = K // 8
    vx = rng.choice(small_x, size=(R, K)) * rng.choice([-1.0, 1.0], size=(R, K))
    vw = rng.choice(small_w, size=(C, K)) * rng.choice([-1.0, 1.0], size=(C, K))
    sgn = np.where(np.arange(G) % 2 == 0, 1.0, -1.0)
    xb = rng.choice(big, size=(R, G // 2)).repeat(2, axis=1)       # same value in a pair
    wb = rng.choice(np.array([1.0, 1.25, 1.5, 2.0]), size=(C, G // 2)).repeat(2, axis=1)
    vx[:, 0::8] = xb
    vw[:, 0::8] = wb * sgn[None, :]
    return vx, vw


def tile(a: np.ndarray, rows: int) -> np.ndarray:
    return np.tile(a, (rows // a.shape[0], 1))


# (name, M, N, K, flags, block): which kernel runs follows from the shape
LAW_CASES = [
    ("decode_register", 4, 256, 512, 2, False),
    ("decode_register_block", 4, 256, 512, 2, True),
    ("decode_line_8_rows", 8, 4096, 512, 2, False),
    ("decode_line_16_rows", 16, 4096, 512, 2, False),
    ("decode_line", 48, 256, 512, 2, False),
    ("decode_block", 48, 256, 512, 2, True),
    ("decode_line_64_rows", 64, 256, 512, 2, False),
    ("decode_block_64_rows", 64, 256, 512, 2, True),
    ("prefill_small_tile", 64, 256, 512, 1, False),
    ("prefill_small_tile_block_k128", 64, 256, 128, 1, True),
    ("prefill_small_tile_k128_wide", 4096, 4096, 128, 1, False),
    ("prefill_line", 4096, 4096, 256, 1, False),
    ("prefill_line_192_wide", 4096, 6144, 256, 1, False),
    ("prefill_line_block", 4096, 4096, 512, 1, True),
    ("prefill_line_block_column_split", 8192, 3072, 512, 1, True),
]


@pytest.mark.parametrize("name,M,N,K,flags,block", LAW_CASES, ids=[c[0] for c in LAW_CASES])
def test_accumulation_law_constructed(F, name, M, N, K, flags, block):
    say(f"law {name} {M}x{N}x{K}")
    R, C = min(8, M), 8
    vx, vw = constructed(R, C, K, seed=K + M)
    exact = vx @ vw.T
    decode = flags == 2
    pred = law_sum_split(vx, vw) if decode else law_sum(vx, vw)
    assert not np.array_equal(law_sum(vx, vw), exact), "the case must exercise the cut"
    if decode:
        assert np.array_equal(pred, exact), "the split must restore the small products"
    qx = O.e4m3_encode(tile(vx, M))
    qw = O.e4m3_encode(tile(vw, N))
    assert np.array_equal(O.e4m3_decode(qx[:R]), vx) and np.array_equal(O.e4m3_decode(qw[:C]), vw)
    if block:
        sx = np.ones((M, K // 128), np.float32)
        sw = np.ones((N // 128, K // 128), np.float32)
        y = F.fp8_gemm_block(dev(qx), dev(sx), dev(qw), dev(sw), flags=flags)
    else:
        sx = np.ones(M, np.float32)
        sw = np.ones(N, np.float32)
        y = F.fp8_gemm(dev(qx), dev(sx), dev(qw), dev(sw), flags=flags)
    torch.cuda.synchronize()
    got = host_bf16_f64(y)
    want = O.f64_to_bf16_rne(np.tile(pred, (M // R, N // C)))
    bad = got != want
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: {bad.sum()} outputs off the law, first at {i}: "
                             f"got {got[i]!r} want {want[i]!r} (exact {exact[i[0] % R, i[1] % C]!r})")
    off = ~O.within_tolerance(np.tile(O.f64_to_bf16_rne(pred), (1, 1)), exact)
    say(f"  {name}: every output as the law predicts; {off.sum()} of {off.size} "
        f"patterns outside the tolerance of the exact sum")


@pytest.mark.parametrize("M,N,K", [(20, 100, 65536), (20, 100, MAX_K), (1, 96, MAX_K),
                                   (8, 64, 65536), (64, 128, MAX_K)])
def test_decode_long_rows(F, M, N, K):
    """The synthetic activations (1 % outlier channels x 20) at the longest
    rows: every output within tolerance of the exact sum."""
    say(f"decode long rows {M}x{N}x{K}")
    xb = synth.activations(M, K, 1200 + M, 1300 + K)
    wb = synth.weights(N, K, 1400 + N + K)
    qw_o, sw_o = O.quant_per_row(wb)
    qx_o, sx_o = O.quant_per_row(xb)
    y, qx, sx = F.fp8_linear(dev_bf16(xb), dev(qw_o), dev(sw_o))
    torch.cuda.synchronize()
    assert np.array_equal(qx.cpu().numpy(), qx_o)
    assert_y_close(host_bf16_f64(y), O.linear_per_channel(qx_o, sx_o, qw_o, sw_o), "y")


def periodic_codes(rows: int, K: int, period: int, seed: int) -> np.ndarray:
    """Codes of `period` distinct per-token-quantized rows (N(0,1) with 1 %
    outlier columns x 20, |value| = 448 |z| / max |z| rounded to E4M3),
    repeated to `rows` rows: row r equals row r % period."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((period, K))
    z[:, rng.permutation(K)[: K // 100]] *= 20
    v = 448.0 * z / np.abs(z).max(axis=1, keepdims=True)
    return np.tile(O.e4m3_encode(v), (rows // period, 1))


@pytest.mark.parametrize("block", [False, True])
def test_prefill_longest_rows_follow_law(F, block):
    """K = 131072 through the whole-line prefill kernels (a 4096 x 4096
    output, so the whole-line tiles run): sampled outputs within the
    tolerance of the law's prediction; the count outside the nominal
    tolerance of the exact sum is reported."""
    M = N = 4096
    K = MAX_K
    P = 32                                   # distinct rows of X and of W
    say(f"prefill longest rows block={block}")
    qx = periodic_codes(M, K, P, 5)
    qw = periodic_codes(N, K, P, 6)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 10, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 22, replace=False)]))
    vx, vw = O.e4m3_decode(qx[rows]), O.e4m3_decode(qw[cols])
    if block:
        G = K // 128
        sx = (2.0 ** rng.integers(-8, -4, size=(M, G))).astype(np.float32)
        sw = (2.0 ** rng.integers(-10, -6, size=(N // 128, G))).astype(np.float32)
        y = F.fp8_gemm_block(dev(qx), dev(sx), dev(qw), dev(sw), flags=1)
        torch.cuda.synchronize()
        pred = np.zeros((len(rows), len(cols)))
        ref = np.zeros((len(rows), len(cols)))
        for g in range(G):
            ks = slice(128 * g, 128 * g + 128)
            f = sx[rows, g].astype(np.float64)[:, None] * sw[cols // 128, g].astype(np.float64)[None, :]
            pred += law_sum(vx[:, ks], vw[:, ks]) * f
            ref += (vx[:, ks] @ vw[:, ks].T) * f
    else:
        sx = (2.0 ** rng.integers(-8, -4, size=M)).astype(np.float32)
        sw = (2.0 ** rng.integers(-10, -6, size=N)).astype(np.float32)
        y = F.fp8_gemm(dev(qx), dev(sx), dev(qw), dev(sw), flags=1)
        torch.cuda.synchronize()
        s = sx[rows].astype(np.float64)[:, None] * sw[cols].astype(np.float64)[None, :]
        pred = law_sum(vx, vw) * s
        ref = (vx @ vw.T) * s
    got = host_bf16_f64(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    assert_y_close(got, pred, "y against the law")
    off = ~O.within_tolerance(got, ref)
    say(f"  {off.sum()} of {off.size} sampled outputs outside the tolerance of the exact sum")


def test_decode_workspace_reuse(F):
    """One zero-filled workspace serves split-K calls of different shapes in
    a row (the tile counters are left zero by every call): each result is
    bit-identical to the same call with a fresh workspace."""
    shapes = [(20, 100, 65536), (1, 96, 131072), (64, 512, 28672), (5, 1024, 16384),
              (20, 100, 65536)]
    need = max(F.fp8_workspace_bytes(M, N, K) for M, N, K in shapes)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (M, N, K) in enumerate(shapes):
        say(f"  reuse {i}: {M}x{N}x{K}")
        xb = synth.activations(M, K, 40 + i, 50 + i)
        qw, sw = F.fp8_quant_act(dev_bf16(synth.weights(N, K, 60 + i)))
        x = dev_bf16(xb)
        y1, _, _ = F.fp8_linear(x, qw, sw, ws=ws)
        y2, _, _ = F.fp8_linear(x, qw, sw)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"call {i}"


@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_c3_every_output(F, j):
    """70B decode qkv, o, gate_up and down (j = 0..3) at 1, 8, 32 and 64
    tokens (both decode kernels, every token-row layout): every output of
    the linear within tolerance of the oracle."""
    d = synth.workload(3, j, 3)
    K, N = d["K"], d["N"]
    say(f"c3 every output {d['name']} {N}x{K}")
    qw_o, sw_o = O.quant_per_row(d["w"])
    vw = O.e4m3_decode(qw_o)
    qw_d, sw_d = dev(qw_o), dev(sw_o)
    for M in (1, 8, 32, 64):
        xb = d["x"][:M]
        qx_o, sx_o = O.quant_per_row(xb)
        y, qx, sx = F.fp8_linear(dev_bf16(xb), qw_d, sw_d)
        torch.cuda.synchronize()
        assert np.array_equal(qx.cpu().numpy(), qx_o)
        ref = (O.e4m3_decode(qx_o) @ vw.T) * sx_o.astype(np.float64)[:, None] \
            * sw_o.astype(np.float64)[None, :]
        assert_y_close(host_bf16_f64(y), ref, f"M={M}")


def _sample(n, k, seed):
    """The first and last 16 indices and k random ones, sorted, unique."""
    rng = np.random.default_rng(seed)
    edge = min(16, n)
    idx = np.concatenate([np.arange(edge), np.arange(n - edge, n),
                          rng.choice(n, size=min(k, n), replace=False)])
    return np.unique(idx)


@pytest.mark.parametrize("M,N,K,flags", [(4096, 4096, 1024, 1), (4096, 6144, 512, 1),
                                         (512, 512, 1024, 1), (512, 512, 128, 1),
                                         (3, 512, 1024, 2), (16, 512, 1024, 2),
                                         (64, 512, 1024, 2)],
                         ids=["wide_tiles", "tiles_192", "small_tiles", "k128", "decode_3_rows",
                              "decode_16_rows", "decode_64_rows"])
def test_per_channel_scale_extremes(F, M, N, K, flags):
    """Per-channel scales near both ends of the fp32 range: activation rows
    scaled by 2^90 to 2^118 (so acc * sx alone passes 2^128 while y stays
    finite) and by 2^-110 and 2^-120, weight rows by 2^-20 to 2^0. Every
    kernel path (256 x 256 and 256 x 192 whole-line tiles, the small-tile
    kernel and its K = 128 case, the register and whole-line decode kernels)
    gives finite outputs within tolerance of the matrix instruction's
    accumulation law (tests/mfma_law.py) times the scales, on sampled rows
    and columns. (Against the exact sum, the rows scaled up lose the
    absolute term of the tolerance that covers cancelling sums near zero,
    so the law's cut shows as a relative error there.)"""
    say(f"per-channel scale extremes {M}x{N}x{K} flags={flags}")
    rng = np.random.default_rng(M + N + K)
    xf = synth.bf16_bits_to_f32(synth.activations(M, K, 3400 + M, 3401)).astype(np.float64)
    ex = np.array([0, 90, 100, 110, 114, 118, -110, -120])[(5 + 3 * np.arange(M)) % 8]
    xb = synth.f32_to_bf16_bits((xf * 2.0 ** ex[:, None]).astype(np.float32))
    wf = synth.bf16_bits_to_f32(synth.weights(N, K, 3402 + N)).astype(np.float64)
    ew = rng.choice([-20, -10, -4, 0], N)
    wb = synth.f32_to_bf16_bits((wf * 2.0 ** ew[:, None]).astype(np.float32))
    qx, sx = O.quant_per_row(xb)
    qw, sw = O.quant_per_row(wb)
    rows = np.unique(np.concatenate([np.arange(min(16, M)), _sample(M, 48, 41)]))
    cols = np.unique(np.concatenate([np.arange(8), _sample(N, 40, 42)]))
    acc = O.gemm_codes(qx[rows], qw[cols])
    ref = O.linear_per_channel(qx[rows], sx[rows], qw[cols], sw[cols])
    assert np.all(np.abs(ref) < 2.0 ** 127), "test data must keep y finite in bf16"
    vx, vw = O.e4m3_decode(qx[rows]), O.e4m3_decode(qw[cols])
    law = law_sum_split(vx, vw) if flags == 2 else law_sum(vx, vw)
    pred = law * (sx[rows].astype(np.float64)[:, None] * sw[cols].astype(np.float64)[None, :])
    with np.errstate(over="ignore"):
        assert np.any(np.isinf(acc.astype(np.float32) * sx[rows, None])), \
            "the case must take acc * sx past fp32's range"
    y = F.fp8_gemm(dev(qx), dev(sx), dev(qw), dev(sw), flags=flags)
    torch.cuda.synchronize()
    got = host_bf16_f64(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    assert np.all(np.isfinite(got)), "non-finite outputs"
    assert_y_close(got, pred, "y against the law")
    off = ~O.within_tolerance(got, ref)
    say(f"  {off.sum()} of {off.size} sampled outputs outside the tolerance of the exact sum")
