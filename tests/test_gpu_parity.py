"""GPU parity: the HIP library (through the C-ABI) against the CPU oracle.

Codes and scales must match bit for bit; bf16 outputs must be within
1e-2 relative / 1e-3 absolute of the oracle's float64 value. Inputs are the
seeded synthetic workloads of `synth` (same bytes on both sides). At full
sizes the oracle computes sampled rows / columns; every expected value comes
from the oracle alone.
"""
import numpy as np
import pytest
import torch

import oracle.fp8dq_oracle as O
import synth
from gpu_util import (assert_codes_equal, assert_scales_equal, assert_y_close,
                      dev, dev_bf16, ensure_built, host_bf16_f64, host_bits, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ensure_built()


def sample_idx(n, k, seed):
    rng = np.random.default_rng(seed)
    edge = min(16, n)
    idx = np.concatenate([np.arange(edge), np.arange(n - edge, n),
                          rng.choice(n, size=min(k, n), replace=False)])
    return np.unique(idx)


# ----------------------------------------------------------------------------
# Quantizers
# ----------------------------------------------------------------------------
ROW_SHAPES = [(1, 8), (3, 40), (5, 512), (7, 520), (64, 4096), (33, 3072),
              (17, 8192), (9, 14336), (5, 28672), (3, 40960), (2, 65536),
              (130, 1024), (300, 2056), (129, 3000), (200, 4096), (140, 14336), (130, 16384),
              # the many-row ladder's other rungs (1 to 16 chunks per lane, 1 to 8
              # waves per row) and the two-pass kernel
              (129, 512), (131, 2048), (132, 6144), (133, 8192), (134, 12288),
              (135, 24576), (136, 32768), (137, 40960)]


@pytest.mark.parametrize("rows,K", ROW_SHAPES)
def test_quant_rows(F, rows, K):
    say(f"quant rows {rows}x{K}")
    xb = synth.activations(rows, K, 100 + K, 200 + K)
    if rows > 2:
        xb[1] = 0                                          # all-zero row
        xb[2, :] = 0x8000                                  # all -0.0 row
    q, s = F.fp8_quant_act(dev_bf16(xb))
    torch.cuda.synchronize()
    q_o, s_o = O.quant_per_row(xb)
    assert_scales_equal(s.cpu().numpy(), s_o, "scales")
    assert_codes_equal(q.cpu().numpy(), q_o, "codes")


def _near_tie_rows(amax_bits: np.ndarray, width: int, seed: int) -> np.ndarray:
    """Rows whose amax is each given bf16 value; the rest are values close to
    E4M3 rounding midpoints of x / s, plus random values below amax."""
    rng = np.random.default_rng(seed)
    R = len(amax_bits)
    amax = O.bf16_to_f64(amax_bits)
    s = O.scale_from_amax(amax).astype(np.float64)
    grid = O.E4M3_VALUES[:127]
    mids = (grid[:-1] + grid[1:]) / 2
    half = width // 2
    pick = mids[rng.integers(0, 125, size=(R, half))]          # below 440
    near = synth.f32_to_bf16_bits((pick * s[:, None]).astype(np.float32)).astype(np.int32)
    near = near + rng.integers(-1, 2, size=(R, half))           # +-1 ulp nudges
    rnd = rng.uniform(0, 1, size=(R, width - half)) * amax[:, None]
    far = synth.f32_to_bf16_bits(rnd.astype(np.float32)).astype(np.int32)
    mag = np.concatenate([near, far], axis=1)
    mag = np.clip(mag, 0, amax_bits.astype(np.int32)[:, None])  # |x| <= amax
    sign = rng.integers(0, 2, size=(R, width)).astype(np.int32) << 15
    x = (mag | sign).astype(np.uint16)
    x[:, 0] = amax_bits | (np.uint16(0x8000) * (rng.integers(0, 2, R) == 1)).astype(np.uint16)
    return x


@pytest.mark.parametrize("group", [0, 128])
def test_quant_every_bf16_amax_near_ties(F, group):
    """Every positive finite bf16 amax (incl. fp32-subnormal scales and the
    2^-64 pre-scale range), rows dense in near-midpoint quotients."""
    say(f"quant exhaustive amax, group={group}")
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint16)
    xb = _near_tie_rows(amax_bits, 128, seed=17 + group)
    q, s = F.fp8_quant_act(dev_bf16(xb), group=group)
    torch.cuda.synchronize()
    q_o, s_o = O.quant_per_row(xb)
    s_h = s.cpu().numpy().reshape(-1)
    assert_scales_equal(s_h, s_o, "scales")
    assert_codes_equal(q.cpu().numpy(), q_o, "codes")


@pytest.mark.parametrize("rows,K", [(1, 128), (5, 384), (64, 3072), (17, 8192), (300, 256)])
def test_quant_groups(F, rows, K):
    say(f"quant groups {rows}x{K}")
    xb = synth.activations(rows, K, 300 + K, 400 + K)
    if rows > 2:
        xb[1, 128:256] = 0                                 # one all-zero group
    q, s = F.fp8_quant_act(dev_bf16(xb), group=128)
    torch.cuda.synchronize()
    q_o, s_o = O.quant_per_group(xb)
    assert_scales_equal(s.cpu().numpy(), s_o, "group scales")
    assert_codes_equal(q.cpu().numpy(), q_o, "group codes")


@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (1024, 3072)])
def test_quant_weight_block(F, N, K):
    say(f"quant weight block {N}x{K}")
    wb = synth.weights(N, K, 500 + N + K)
    wb[0:128, 0:128] = 0                                   # an all-zero block
    q, s = F.fp8_quant_weight_block(dev_bf16(wb))
    torch.cuda.synchronize()
    q_o, s_o = O.quant_weight_block(wb)
    assert_scales_equal(s.cpu().numpy(), s_o, "block scales")
    assert_codes_equal(q.cpu().numpy(), q_o, "block codes")


# ----------------------------------------------------------------------------
# GEMM core
# ----------------------------------------------------------------------------
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


@pytest.mark.parametrize("flags", [1, 2])
def test_mfma_product_table(F, flags):
    """Every product of two finite E4M3 values is exact in bf16: with unit
    scales and one nonzero code per row the output is the exact table."""
    say(f"product table flags={flags}")
    K = 256
    qa = np.zeros((254, K), np.uint8)
    for r, c in enumerate(FINITE):
        qa[r, (r * 37) % K] = c
        qa[r, 200] = c                       # shared position: products land here
    qa_dev = dev(qa)
    ones = dev(np.ones(254, np.float32))
    y = F.fp8_gemm(qa_dev, ones, qa_dev, ones, flags=flags)
    torch.cuda.synchronize()
    want = O.linear_per_channel(qa, np.ones(254, np.float32), qa, np.ones(254, np.float32))
    got = host_bf16_f64(y)
    assert np.array_equal(O.f64_to_bf16_rne(want), want)     # exact in bf16
    diff = got != want
    assert not diff.any(), f"{diff.sum()} mismatches, first {np.argwhere(diff)[0]}"


GEMM_SHAPES = [(1, 16, 128), (16, 1024, 4096), (65, 130, 256), (300, 200, 384),
               (513, 1030, 1024), (256, 256, 128), (1000, 1000, 512), (64, 8192, 1024),
               (2048, 512, 640)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("flags", [0, 1, 2])
def test_gemm_parity(F, M, N, K, flags):
    say(f"gemm {M}x{N}x{K} flags={flags}")
    xb = synth.activations(M, K, 600 + M, 700 + K)
    wb = synth.weights(N, K, 800 + N + K)
    qx, sx = O.quant_per_row(xb)
    qw, sw = O.quant_per_row(wb)
    y = F.fp8_gemm(dev(qx), dev(sx), dev(qw), dev(sw), flags=flags)
    torch.cuda.synchronize()
    assert_y_close(host_bf16_f64(y), O.linear_per_channel(qx, sx, qw, sw), "y")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (16, 1024, 3072), (65, 256, 384),
                                   (300, 384, 1024), (1000, 640, 512)])
@pytest.mark.parametrize("flags", [0, 1, 2])
def test_gemm_block_parity(F, M, N, K, flags):
    say(f"gemm block {M}x{N}x{K} flags={flags}")
    xb = synth.activations(M, K, 900 + M, 1000 + K)
    wb = synth.weights(N, K, 1100 + N + K)
    qx, sx = O.quant_per_group(xb)
    qw, sw = O.quant_weight_block(wb)
    y = F.fp8_gemm_block(dev(qx), dev(sx), dev(qw), dev(sw), flags=flags)
    torch.cuda.synchronize()
    assert_y_close(host_bf16_f64(y), O.linear_block(qx, sx, qw, sw), "y")


def test_gemm_random_codes_small_k(F):
    """Uniformly random finite codes and scales (not only synthetic data)."""
    rng = np.random.default_rng(5)
    for (M, N, K, flags) in [(40, 48, 128, 0), (100, 64, 128, 1), (7, 33, 128, 2)]:
        qx = rng.choice(FINITE, size=(M, K))
        qw = rng.choice(FINITE, size=(N, K))
        sx = rng.uniform(1e-4, 1e-3, M).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
        y = F.fp8_gemm(dev(qx), dev(sx), dev(qw), dev(sw), flags=flags)
        torch.cuda.synchronize()
        assert_y_close(host_bf16_f64(y), O.linear_per_channel(qx, sx, qw, sw),
                       f"random codes {M}x{N}x{K} flags={flags}")


WIDE_RAGGED = [
    # 256 x 192 tiles (two full rounds of them against 1.1 - 1.5 rounds of 256-wide ones)
    (4173, 3853, 384), (4097, 4104, 256), (4352, 4096, 1152), (4352, 4790, 384),
    (4000, 6144, 256),
    # 256 x 256 tiles: one round; two rounds with two workgroups taking one tile
    (4000, 3990, 384), (4352, 7630, 256),
    # 256 x 256 tiles on line-aligned rows (N % 64 == 0): the full tiles store
    # whole 128-byte lines, the last tile row (M ragged) 16-byte pieces;
    # 510 tiles, so workgroups walk two tiles each (254 of them)
    (4300, 7680, 256)]


@pytest.mark.parametrize("M,N,K", WIDE_RAGGED)
def test_gemm_wide_tiles_ragged(F, M, N, K):
    """Shapes with at least 256 tiles of 256 x 256 (the whole-line kernel)
    and ragged edges: M and N off the tile grid, N % 8 != 0 (element
    stores), K = 256 (the shortest K loop), an odd number of 128-column
    groups. Every output is compared."""
    say(f"gemm wide {M}x{N}x{K}")
    rng = np.random.default_rng(M + N + K)
    qx = rng.choice(FINITE, size=(M, K))
    qw = rng.choice(FINITE, size=(N, K))
    sx = rng.uniform(1e-4, 1e-3, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    y = F.fp8_gemm(dev(qx), dev(sx), dev(qw), dev(sw), flags=1)
    torch.cuda.synchronize()
    assert_y_close(host_bf16_f64(y), O.linear_per_channel(qx, sx, qw, sw), "y")


@pytest.mark.parametrize("M,N,K", [(4352, 4096, 384), (4200, 2176, 1152), (2100, 4352, 512),
                                   (8192, 4096, 640), (6300, 4224, 384), (8192, 5120, 384)])
def test_gemm_block_wide_tiles(F, M, N, K):
    """Block-scaled GEMM with more tiles than CUs, ragged M, the shortest K
    of that mode (three groups), and group scales that differ by orders of
    magnitude between groups. On 256 CUs:
    - the first shape runs its first 2304 columns as 256 x 256 tiles and the
      rest as 256 x 128 tiles, in two launches;
    - the next four run 256 x 256 tiles only (8 waves). Two of them have a
      last tile column half past N (N = 2176, 4224). Two have more such
      tiles than CUs, so workgroups walk two tiles each (all of them, or 169
      of 256);
    - the last runs two rounds of 256 x 256 tiles (4096 columns), then one
      of 256 x 128."""
    say(f"gemm block wide {M}x{N}x{K}")
    G = K // 128
    rng = np.random.default_rng(M + 3 * N + K)
    qx = rng.choice(FINITE, size=(M, K))
    qw = rng.choice(FINITE, size=(N, K))
    sx = (rng.uniform(0.5, 1.0, (M, G)) * 10.0 ** rng.integers(-6, -2, (M, G))).astype(np.float32)
    sw = (rng.uniform(0.5, 1.0, (N // 128, G)) * 10.0 ** rng.integers(-5, -2, (N // 128, G))).astype(np.float32)
    qx[7, 128:256] = 0                                 # an all-zero activation group
    sx[7, 1] = 0.0
    y = F.fp8_gemm_block(dev(qx), dev(sx), dev(qw), dev(sw), flags=1)
    torch.cuda.synchronize()
    assert_y_close(host_bf16_f64(y), O.linear_block(qx, sx, qw, sw), "y")


def test_linear_x_beyond_4gib(F):
    """fp8_linear with M * K > 2^32 bytes of X codes: the prefill path runs
    row blocks so that each block's operand offsets fit 32 bits; rows on
    both sides of the block boundary, and the last rows, are compared."""
    M, N, K = 150000, 256, 28672
    rows_max = ((1 << 32) - 1) // K
    rows_max -= rows_max % 256
    assert M * K > (1 << 32) and rows_max < M
    say(f"linear {M}x{K}->{N}, row block {rows_max}")
    g = torch.Generator(device="cuda").manual_seed(77)
    x_d = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
    wb = synth.weights(N, K, 4242)
    w_d = dev_bf16(wb)
    qw_d, sw_d = F.fp8_quant_act(w_d)
    y_d, qx_d, sx_d = F.fp8_linear(x_d, qw_d, sw_d)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_idx(M, 24, 78),
                                     np.arange(rows_max - 3, rows_max + 3), np.arange(M - 3, M)]))
    rows_d = torch.from_numpy(rows).cuda()
    xb = host_bits(x_d[rows_d])
    del x_d
    qx_o, sx_o = O.quant_per_row(xb)
    assert_codes_equal(qx_d[rows_d].cpu().numpy(), qx_o, "act codes")
    assert_scales_equal(sx_d[rows_d].cpu().numpy(), sx_o, "act scales")
    qw_o, sw_o = O.quant_per_row(wb)
    assert_y_close(host_bf16_f64(y_d[rows_d]), O.linear_per_channel(qx_o, sx_o, qw_o, sw_o), "y")


# ----------------------------------------------------------------------------
# The whole linear on the workloads
# ----------------------------------------------------------------------------
def _linear_case(F, xb, wb, cols, flags=0, what=""):
    """GPU: W per-channel quantization + fp8_linear. Oracle: sampled W rows
    (output columns `cols`), all X rows."""
    x_d = dev_bf16(xb)
    w_d = dev_bf16(wb)
    qw_d, sw_d = F.fp8_quant_act(w_d)
    y_d, qx_d, sx_d = F.fp8_linear(x_d, qw_d, sw_d, flags=flags)
    torch.cuda.synchronize()
    qw_o, sw_o = O.quant_per_row(wb[cols])
    assert_scales_equal(sw_d.cpu().numpy()[cols], sw_o, f"{what} weight scales")
    assert_codes_equal(qw_d.cpu().numpy()[cols], qw_o, f"{what} weight codes")
    qx_o, sx_o = O.quant_per_row(xb)
    assert_scales_equal(sx_d.cpu().numpy(), sx_o, f"{what} act scales")
    assert_codes_equal(qx_d.cpu().numpy(), qx_o, f"{what} act codes")
    y_ref = O.linear_per_channel(qx_o, sx_o, qw_o, sw_o)
    assert_y_close(host_bf16_f64(y_d[:, torch.from_numpy(cols).cuda()]), y_ref, f"{what} y")


def test_c1_single_linear(F):
    d = synth.workload(1)
    say("c1 16x4096->1024")
    _linear_case(F, d["x"], d["w"], np.arange(d["N"]), what="c1")


@pytest.mark.parametrize("j", [0, 1, 2, 3])
@pytest.mark.parametrize("M", [64, 256])
def test_c2_prefill_shapes(F, j, M):
    d = synth.workload(2, j, M=M)
    say(f"c2 {d['name']} M={M} K={d['K']} N={d['N']}")
    _linear_case(F, d["x"], d["w"], sample_idx(d["N"], 256, j), what=f"c2 {d['name']}")


@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_c3_decode_shapes(F, j):
    name, K, N = synth.SHAPES["c3"][j]
    say(f"c3 {name} K={K} N={N}: weights")
    wb = synth.weights(N, K, synth.seed_of(3, j, 0, 1))
    w_d = dev_bf16(wb)
    qw_d, sw_d = F.fp8_quant_act(w_d)
    del w_d
    cols = sample_idx(N, 192, 10 + j)
    qw_o, sw_o = O.quant_per_row(wb[cols])
    del wb
    torch.cuda.synchronize()
    assert_scales_equal(sw_d.cpu().numpy()[cols], sw_o, "weight scales")
    assert_codes_equal(qw_d.cpu().numpy()[cols], qw_o, "weight codes")
    cols_d = torch.from_numpy(cols).cuda()
    for i, M in enumerate(synth.M_OF["c3"]):
        say(f"c3 {name} M={M}")
        xb = synth.workload(3, j, i, w=False)["x"]
        y_d, qx_d, sx_d = F.fp8_linear(dev_bf16(xb), qw_d, sw_d)
        torch.cuda.synchronize()
        qx_o, sx_o = O.quant_per_row(xb)
        assert_scales_equal(sx_d.cpu().numpy(), sx_o, "act scales")
        assert_codes_equal(qx_d.cpu().numpy(), qx_o, "act codes")
        assert_y_close(host_bf16_f64(y_d[:, cols_d]),
                       O.linear_per_channel(qx_o, sx_o, qw_o, sw_o), f"M={M} y")


@pytest.mark.parametrize("j", [0, 1, 2, 3])
@pytest.mark.parametrize("M", [64, 512])
def test_c4_block_shapes(F, j, M):
    d = synth.workload(4, j, M=M)
    N, K = d["N"], d["K"]
    say(f"c4 {d['name']} M={M} K={K} N={N}")
    x_d = dev_bf16(d["x"])
    w_d = dev_bf16(d["w"])
    qw_d, sw_d = F.fp8_quant_weight_block(w_d)
    y_d, qx_d, sx_d = F.fp8_linear_block(x_d, qw_d, sw_d)
    torch.cuda.synchronize()
    bands = np.unique([0, N // 128 - 1, (N // 128) // 2])
    rows = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in bands])
    qw_o, sw_o = O.quant_weight_block(d["w"][rows])
    assert_scales_equal(sw_d.cpu().numpy()[bands], sw_o, "block weight scales")
    assert_codes_equal(qw_d.cpu().numpy()[rows], qw_o, "block weight codes")
    qx_o, sx_o = O.quant_per_group(d["x"])
    assert_scales_equal(sx_d.cpu().numpy(), sx_o, "group act scales")
    assert_codes_equal(qx_d.cpu().numpy(), qx_o, "group act codes")
    y_ref = O.linear_block(qx_o, sx_o, qw_o, sw_o)
    assert_y_close(host_bf16_f64(y_d[:, torch.from_numpy(rows).cuda()]), y_ref, "y")


def block_ref_rows(qx, sx, qw, sw, rows, cols):
    """Oracle y of the block variant at sampled rows and columns (float64):
    sum over groups of the exact group product times sx[m,g] sw[n/128,g]."""
    G = qx.shape[1] // 128
    vx = O.e4m3_decode(qx[rows])
    vw = O.e4m3_decode(qw[cols])
    y = np.zeros((len(rows), len(cols)))
    for g in range(G):
        ks = slice(128 * g, 128 * g + 128)
        f = sx[rows, g].astype(np.float64)[:, None] * sw[cols // 128, g].astype(np.float64)[None, :]
        y += O.gemm_codes(qx[rows][:, ks], qw[cols][:, ks]) * f
    return y


@pytest.mark.parametrize("M,N,flags", [(8192, 8192, 1), (512, 512, 1), (64, 512, 1), (48, 512, 2),
                                       (8, 512, 2), (4, 512, 2), (64, 512, 2), (57, 512, 2)],
                         ids=["wide_tiles", "narrow_tiles", "narrow_m64", "decode", "decode_8_rows",
                              "decode_4_rows", "decode_64_rows", "decode_57_rows"])
def test_block_factor_extremes(F, M, N, flags):
    """Block factors sx * sw spanning the fp32 range, made by multiplying a
    row's own group scales (so y stays of order 1, as in real data): later
    groups 2^90 and 2^120 below the first (the largest carried ratio of a
    single accumulator would overflow fp32 at 2^120), the first group 2^120
    below the rest, two activation scales in the fp32 subnormals (1e-41,
    whose product with a weight scale of 2e-4 is subnormal; 1e-42, whose
    product underflows to 0), factors rising by 2^10 and falling by 2^12 per
    group, and unchanged rows. Codes are those of the synthetic activations;
    y within tolerance of the oracle on sampled rows and columns (8192 x 8192
    runs the 256 x 256 whole-line tiles, 512 x 512 the 256 x 128 ones; 57
    and 64 decode rows the layout where each wave owns 16 token rows, the
    last wave's partly past M at 57)."""
    K = 1024
    G = K // 128
    say(f"block factor extremes {M}x{N} flags={flags}")
    qx, sx = O.quant_per_group(synth.activations(M, K, 3100 + M, 3200))
    qw, sw = O.quant_weight_block(synth.weights(N, K, 3300 + N))
    g = np.arange(G)
    mult = {
        0: np.where(g >= 1, 2.0 ** -90, 1.0),      # later groups 2^90 below
        1: np.where(g >= 1, 2.0 ** -120, 1.0),     # 2^120 below
        2: np.where(g == 0, 2.0 ** -120, 1.0),     # the first group 2^120 below
        4: 2.0 ** (10.0 * g - 70),                 # rising by 2^10
        5: 2.0 ** (-12.0 * g),                     # falling by 2^12
    }
    sx = sx.copy()
    for r in range(M):
        k = r % 8
        if k in mult:
            sx[r] = (sx[r].astype(np.float64) * mult[k]).astype(np.float32)
        elif k == 3:   # a zero factor right after a normal one, then a subnormal one
            sx[r, 3], sx[r, 5] = np.float32(1e-42), np.float32(1e-41)
    sw = sw.copy()
    sw[:, 3] = sw[:, 5] = np.float32(2e-4)                          # with the subnormal sx
    # fp32 products: 1e-41 * 2e-4 is subnormal, 1e-42 * 2e-4 underflows to 0
    assert 0 < np.float32(1e-41) * np.float32(2e-4) < 2.0 ** -126
    assert np.float32(1e-42) * np.float32(2e-4) == 0
    y = F.fp8_gemm_block(dev(qx), dev(sx), dev(qw), dev(sw), flags=flags)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(min(16, M)), sample_idx(M, 48, 31)]))
    cols = np.unique(np.concatenate([np.arange(8), sample_idx(N, 40, 32)]))
    ref = block_ref_rows(qx, sx, qw, sw, rows, cols)
    got = host_bf16_f64(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    assert np.all(np.isfinite(got)), "non-finite outputs"
    assert_y_close(got, ref, "y")


@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_c4_full_size_sampled(F, j):
    """The Llama-3.2-3B block linears at M = 8192 through fp8_linear_block,
    in the launch configuration the benchmark times (256 x 256 whole-line
    tiles for gate_up, walking several tiles per workgroup; the wide-then-
    narrow column split for the others): codes and scales of sampled rows
    and weight blocks bit-exact, y within tolerance there."""
    d = synth.workload(4, j)
    M, N, K = d["M"], d["N"], d["K"]
    say(f"c4 full {d['name']} {M}x{K}->{N}")
    rows = sample_idx(M, 48, 90 + j)
    bands = np.unique([0, 1, N // 256, N // 128 - 2, N // 128 - 1])
    cols = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in bands])
    x_d = dev_bf16(d["x"])
    w_d = dev_bf16(d["w"])
    qw_d, sw_d = F.fp8_quant_weight_block(w_d)
    y_d, qx_d, sx_d = F.fp8_linear_block(x_d, qw_d, sw_d)
    torch.cuda.synchronize()
    qw_o, sw_o = O.quant_weight_block(d["w"][cols])
    qx_o, sx_o = O.quant_per_group(d["x"][rows])
    assert_codes_equal(qw_d.cpu().numpy()[cols], qw_o, "weight codes")
    assert_scales_equal(sw_d.cpu().numpy()[bands], sw_o, "weight block scales")
    assert_codes_equal(qx_d.cpu().numpy()[rows], qx_o, "act codes")
    assert_scales_equal(sx_d.cpu().numpy()[rows], sx_o, "act scales")
    ysub = y_d[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    assert_y_close(host_bf16_f64(ysub), O.linear_block(qx_o, sx_o, qw_o, sw_o), "y")


def test_c5_full_size_sampled(F):
    d = synth.workload(5)
    M, N = d["M"], d["N"]
    say(f"c5 full {M}x{d['K']}->{N} zero_rows={len(d['zero_rows'])}")
    planted_rows = [p[0] for p in d["planted"]]
    rows = np.unique(np.concatenate([sample_idx(M, 32, 90), d["zero_rows"][:4],
                                     planted_rows]))
    cols = sample_idx(N, 96, 91)
    x_d = dev_bf16(d["x"])
    w_d = dev_bf16(d["w"])
    qw_d, sw_d = F.fp8_quant_act(w_d)
    del w_d
    y_d, qx_d, sx_d = F.fp8_linear(x_d, qw_d, sw_d)
    torch.cuda.synchronize()
    qx_o, sx_o = O.quant_per_row(d["x"][rows])
    qw_o, sw_o = O.quant_per_row(d["w"][cols])
    assert_codes_equal(qx_d.cpu().numpy()[rows], qx_o, "act codes")
    assert_scales_equal(sx_d.cpu().numpy()[rows], sx_o, "act scales")
    assert_codes_equal(qw_d.cpu().numpy()[cols], qw_o, "weight codes")
    ysub = y_d[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    assert_y_close(host_bf16_f64(ysub), O.linear_per_channel(qx_o, sx_o, qw_o, sw_o), "y")
    # properties over every row: zero rows -> s = 0 and an all-zero y row
    sx_all = sx_d.cpu().numpy()
    zr = torch.from_numpy(d["zero_rows"]).cuda()
    assert np.all(sx_all[d["zero_rows"]] == 0)
    assert int((y_d[zr] != 0).sum()) == 0
    assert np.all(sx_all[np.setdiff1d(np.arange(M), d["zero_rows"])] > 0)


# ----------------------------------------------------------------------------
# Decode path (M <= 64): ragged shapes, split-K, the two-step equivalence
# ----------------------------------------------------------------------------
DECODE_CASES = [(1, 8192, 8192), (5, 100, 1664), (16, 1024, 4096), (17, 520, 3200),
                (33, 4096, 896), (64, 10240, 8192), (64, 33, 128), (2, 2048, 28672),
                (8, 57344, 8192), (48, 1000, 1152), (50, 130, 256),
                # few weight rows at one token, ragged N, 16 tokens, the
                # shortest K (unsplit: K < 16384), the longest K at one token
                (1, 64, 8192), (3, 100, 2048), (16, 200, 1920), (4, 32, 128),
                (1, 8192, 28672),
                # register kernel split on a long row at one token
                (1, 64, 16384),
                # whole-line kernel with one 16-row token block (5-16
                # tokens), in 2 and 8 K slices
                (9, 4500, 2560), (12, 4096, 16384),
                # whole-line kernel on long rows (8, 16 and 20 K slices; more
                # than 16 slices take the reduction's general loop)
                (64, 8192, 28672), (40, 3000, 16384), (20, 100, 20480)]


@pytest.mark.parametrize("M,N,K", DECODE_CASES)
def test_decode_linear_shapes(F, M, N, K):
    """fp8_linear at M <= 64 (the split-K decode path): codes and scales
    bit-exact, y within tolerance on sampled columns, y bit-identical to
    fp8_quant_act + fp8_gemm forced onto the decode path, and repeated calls
    reproduce the result."""
    say(f"decode {M}x{N}x{K}")
    xb = synth.activations(M, K, 1200 + M, 1300 + K)
    wb = synth.weights(N, K, 1400 + N + K)
    qw_d, sw_d = F.fp8_quant_act(dev_bf16(wb))
    cols = sample_idx(N, 256, M)
    qw_o, sw_o = O.quant_per_row(wb[cols])
    x_d = dev_bf16(xb)
    y, qx, sx = F.fp8_linear(x_d, qw_d, sw_d)
    y_again, _, _ = F.fp8_linear(x_d, qw_d, sw_d)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_again.view(torch.int16)), "repeat"
    qx_o, sx_o = O.quant_per_row(xb)
    assert_scales_equal(sx.cpu().numpy(), sx_o, "act scales")
    assert_codes_equal(qx.cpu().numpy(), qx_o, "act codes")
    cols_d = torch.from_numpy(cols).cuda()
    assert_y_close(host_bf16_f64(y[:, cols_d]),
                   O.linear_per_channel(qx_o, sx_o, qw_o, sw_o), "y")
    y2 = F.fp8_gemm(qx, sx, qw_d, sw_d, flags=F.FORCE_DECODE)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "linear vs two-step"


def test_decode_linear_special_rows(F):
    """fp8_linear on the decode path with an all-zero row (scale 0), a row
    whose scale needs the 2^64 pre-scale, a row of -0.0 and an ordinary row:
    codes and scales bit-exact, y as the two-step path."""
    M, N, K = 4, 300, 1024
    xb = synth.activations(M, K, 1500, 1501)
    xb[0] = 0
    xb[1] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(xb[1]) * np.float32(2.0 ** -100))
    xb[2] = 0x8000
    wb = synth.weights(N, K, 1502)
    qw_d, sw_d = F.fp8_quant_act(dev_bf16(wb))
    y, qx, sx = F.fp8_linear(dev_bf16(xb), qw_d, sw_d)
    torch.cuda.synchronize()
    qx_o, sx_o = O.quant_per_row(xb)
    assert sx_o[0] == 0 and 0 < sx_o[1] < 2.0 ** -64
    assert_scales_equal(sx.cpu().numpy(), sx_o, "act scales")
    assert_codes_equal(qx.cpu().numpy(), qx_o, "act codes")
    qw_o, sw_o = O.quant_per_row(wb)
    assert_y_close(host_bf16_f64(y), O.linear_per_channel(qx_o, sx_o, qw_o, sw_o), "y")
    y2 = F.fp8_gemm(qx, sx, qw_d, sw_d, flags=F.FORCE_DECODE)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "linear vs two-step"


# ----------------------------------------------------------------------------
# Determinism and guard bands
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,flags", [(4096, 4096, 4096, 0), (16, 1024, 4096, 0),
                                         (64, 8192, 8192, 0), (300, 1030, 1024, 2)])
def test_deterministic(F, M, N, K, flags):
    say(f"determinism {M}x{N}x{K} flags={flags}")
    xb = synth.activations(M, K, 1, 2)
    wb = synth.weights(N, K, 3)
    qw, sw = F.fp8_quant_act(dev_bf16(wb))
    x_d = dev_bf16(xb)
    y1, q1, s1 = F.fp8_linear(x_d, qw, sw, flags=flags)
    y2, q2, s2 = F.fp8_linear(x_d, qw, sw, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_guard_bands_untouched(F):
    """Outputs written through views of larger buffers: bytes around them keep
    their 0xA5 canary after quantization, GEMM (both paths) and linear."""
    M, N, K = 70, 1030, 384
    pad = 4096
    xb = synth.activations(M, K, 7, 8)
    wb = synth.weights(N, K, 9)
    x_d = dev_bf16(xb)
    qw, sw = F.fp8_quant_act(dev_bf16(wb))

    def canvas(nbytes):
        c = torch.full((nbytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
        return c

    for flags in (1, 2):
        cy = canvas(M * N * 2)
        cq = canvas(M * K)
        cs = canvas(M * 4)
        y = cy[pad:pad + M * N * 2].view(torch.bfloat16).view(M, N)
        q = cq[pad:pad + M * K].view(M, K)
        s = cs[pad:pad + M * 4].view(torch.float32)
        F.fp8_linear(x_d, qw, sw, y=y, qx_out=q, sx_out=s, flags=flags)
        torch.cuda.synchronize()
        for c, n in ((cy, M * N * 2), (cq, M * K), (cs, M * 4)):
            h = c.cpu().numpy()
            assert np.all(h[:pad] == 0xA5) and np.all(h[pad + n:] == 0xA5), flags


def test_empty_inputs(F):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = F.fp8_quant_act(x)
    assert q.shape == (0, 256) and s.shape == (0,)
    qw = torch.zeros((128, 256), dtype=torch.uint8, device="cuda")
    sw = torch.ones(128, dtype=torch.float32, device="cuda")
    y, qx, sx = F.fp8_linear(x, qw, sw)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


def test_binding_rejects_mismatched_tensors(F):
    """The binding checks every tensor's dtype, shape, layout and device
    before its pointer reaches the library (which sees only pointers and
    sizes): each mismatch raises ValueError and launches nothing."""
    d = "cuda"
    M, N, K = 8, 256, 512
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=d)
    qx = torch.zeros((M, K), dtype=torch.uint8, device=d)
    sx = torch.ones(M, dtype=torch.float32, device=d)
    qw = torch.zeros((N, K), dtype=torch.uint8, device=d)
    sw = torch.ones(N, dtype=torch.float32, device=d)
    bad = [
        lambda: F.fp8_gemm(qx, sx, qw[:, :256].contiguous(), sw),           # W rows of another K
        lambda: F.fp8_gemm(qx, sx, qw, sw[:128]),                            # too few channel scales
        lambda: F.fp8_gemm(qx, sx.double(), qw, sw),                         # wrong dtype
        lambda: F.fp8_gemm(qx, sx, qw.t().contiguous().t(), sw),             # not contiguous
        lambda: F.fp8_gemm(qx, sx, qw, sw, y=torch.empty((M, N + 1), dtype=torch.bfloat16, device=d)),
        lambda: F.fp8_gemm(qx, sx, qw, sw, ws=torch.zeros(1 << 20, dtype=torch.uint8)),  # host ws
        lambda: F.fp8_linear(x, qw, sw.cpu()),                               # host scales
        lambda: F.fp8_linear(x, qw, sw, qx_out=torch.empty((M, K + 8), dtype=torch.uint8, device=d)),
        lambda: F.fp8_linear_noalloc(x, qw[:128], sw),                       # W and scales disagree
        lambda: F.fp8_gemm_block(qx, torch.ones((M, 4), device=d), qw[:200].contiguous(),
                                 torch.ones((2, 4), device=d)),              # N not a multiple of 128
        lambda: F.fp8_linear_block(x, qw, torch.ones((2, 3), device=d)),    # wrong block-scale grid
        lambda: F.fp8_quant_act(x, group=64),
        lambda: F.fp8_quant_static(x, torch.ones(1)),                        # scale read on the device
        lambda: F.fp8_rmsnorm_quant(x, torch.ones(K + 8, dtype=torch.bfloat16, device=d)),
        lambda: F.fp8_kv_cache_quant(x, x, torch.zeros(M, dtype=torch.int32, device=d),
                                     torch.zeros((16, K), dtype=torch.uint8, device=d),
                                     torch.zeros((16, K), dtype=torch.uint8, device=d),
                                     torch.zeros(16, device=d), torch.zeros(16, device=d)),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(ValueError):
            f()
            pytest.fail(f"case {i} was not rejected")
    torch.cuda.synchronize()
