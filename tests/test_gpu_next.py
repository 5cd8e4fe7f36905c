"""GPU parity of the fused producers, static calibration and the FP8 KV-cache
write against the CPU oracle (codes and scales bit-exact)."""
import math

import numpy as np
import pytest
import torch

import oracle.fp8dq_oracle as O
import synth
from gpu_util import assert_codes_equal, assert_scales_equal, dev, dev_bf16, ensure_built, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ensure_built()


def bits_of(v):
    return synth.f32_to_bf16_bits(np.asarray(v, np.float32))


def gate_up(rows, inner, seed, extreme=True):
    """Synthetic gate_up output rows [rows, 2*inner] (bf16 bits): N(0, 2)
    gates and N(0, 1) ups with 1% outlier columns; a share of gates pushed to
    large magnitudes (fp64 path, exact ties where silu(g) rounds to g)."""
    gu = synth.activations(rows, 2 * inner, seed, seed + 1)
    if extreme:
        rng = np.random.default_rng(seed + 2)
        g = synth.bf16_bits_to_f32(gu[:, :inner]).copy()
        pick = rng.random(g.shape) < 0.02
        big = rng.choice([40.0, 48.0, 64.0, 65.0, 96.0, 200.0, -40.0, -90.0, -120.0,
                          1e4, -1e4, -3e38, 1e-30], size=g.shape)
        g = np.where(pick, big, g)
        gu[:, :inner] = bits_of(g)
    return gu


SILU_SHAPES = [(1, 8), (3, 136), (64, 1024), (17, 14336), (5, 28672), (130, 512), (2, 65536),
               # every rung of the row-team ladder (4 waves, 2 to 8 chunks per lane)
               (6, 4096), (7, 6144), (9, 8192), (4, 10240), (3, 12288), (5, 16384)]


@pytest.mark.parametrize("rows,inner", SILU_SHAPES)
def test_silu_mul_quant(F, rows, inner):
    say(f"silu_mul_quant {rows}x{inner}")
    gu = gate_up(rows, inner, 5000 + inner)
    q, s = F.fp8_silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    qo, so = O.silu_mul_quant(gu)
    assert_scales_equal(s.cpu().numpy(), so, "silu scales")
    assert_codes_equal(q.cpu().numpy(), qo, "silu codes")


def test_silu_mul_quant_full_size_sampled(F):
    """Llama-3.1-8B down_proj input: M = 4096 tokens, I = 14336 (gate_up
    output 4096 x 28672); the oracle checks sampled rows."""
    M, inner = 4096, 14336
    say(f"silu_mul_quant full {M}x{inner}")
    rows = np.unique(np.concatenate([[0, 1, M - 1], np.random.default_rng(9).choice(M, 24, replace=False)]))
    gu_rows = gate_up(M, inner, 777)
    q, s = F.fp8_silu_mul_quant(dev_bf16(gu_rows))
    torch.cuda.synchronize()
    qo, so = O.silu_mul_quant(gu_rows[rows])
    assert_scales_equal(s.cpu().numpy()[rows], so, "silu scales")
    assert_codes_equal(q.cpu().numpy()[rows], qo, "silu codes")


def norm_input(rows, hidden, seed):
    x = synth.activations(rows, hidden, seed, seed + 1)
    xf = synth.bf16_bits_to_f32(x).copy()
    if rows >= 3:
        xf[1] = 0.0                      # all-zero row: h = 0, scale 0
        xf[2] *= 1e-3                    # tiny row: eps matters
    gamma = bits_of(np.random.default_rng(seed + 2).normal(1.0, 0.3, hidden))
    return bits_of(xf), gamma


RMS_SHAPES = [(1, 8), (5, 4096), (64, 4096), (7, 8192), (3, 16384), (130, 512), (2, 65536),
              # the ladder's other rungs
              (6, 6144), (4, 10240), (3, 12288), (5, 14336), (2, 28672)]


@pytest.mark.parametrize("rows,hidden", RMS_SHAPES)
def test_rmsnorm_quant(F, rows, hidden):
    say(f"rmsnorm_quant {rows}x{hidden}")
    x, gamma = norm_input(rows, hidden, 6000 + hidden)
    q, s = F.fp8_rmsnorm_quant(dev_bf16(x), dev_bf16(gamma))
    torch.cuda.synchronize()
    qo, so = O.rmsnorm_quant(x, gamma)
    assert_scales_equal(s.cpu().numpy(), so, "rms scales")
    assert_codes_equal(q.cpu().numpy(), qo, "rms codes")


def test_rmsnorm_quant_full_size_sampled(F):
    M, hidden = 4096, 4096
    say(f"rmsnorm_quant full {M}x{hidden}")
    x, gamma = norm_input(M, hidden, 888)
    q, s = F.fp8_rmsnorm_quant(dev_bf16(x), dev_bf16(gamma))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 2, M - 1], np.random.default_rng(10).choice(M, 32, replace=False)]))
    qo, so = O.rmsnorm_quant(x[rows], gamma)
    assert_scales_equal(s.cpu().numpy()[rows], so, "rms scales")
    assert_codes_equal(q.cpu().numpy()[rows], qo, "rms codes")


@pytest.mark.parametrize("n", [0, 8, 1000, 4096 * 64, 1 << 22])
@pytest.mark.parametrize("lo,hi", [(1, 999), (0, 1000), (100, 900), (500, 500)])
def test_calib_scale(F, n, lo, hi):
    say(f"calib n={n} lo={lo} hi={hi}")
    x = synth.activations(max(-(-n // 256), 1), 256, 7000 + n, 7001).ravel()[:n]
    x = np.ascontiguousarray(x)
    xd = dev_bf16(x) if n else torch.empty((0,), dtype=torch.bfloat16, device="cuda")
    s = F.fp8_calib_scale(xd, lo, hi)
    torch.cuda.synchronize()
    want = O.calib_scale(x, lo, hi)
    assert_scales_equal(s.cpu().numpy(), np.array([want], np.float32), "calib scale")


@pytest.mark.parametrize("n_ext", [7, 8, 9])
def test_calib_scale_rank_at_bucket_edges(F, n_ext):
    """8000 values: n_ext of them -3.0, one -0.0 and one +0.0, the rest 1.0
    (one key, so one bucket holds nearly every value): the P0.1 rank (k = 8)
    lands inside, exactly at and just past the end of the -3.0 group, the
    P99.9 rank inside the 1.0 group."""
    n = 8000
    x = np.full(n, 0x3F80, np.uint16)                  # 1.0
    x[:n_ext] = 0xC040                                 # -3.0
    x[n_ext] = 0x8000                                  # -0.0
    x[n_ext + 1] = 0x0000                              # +0.0
    x = np.random.default_rng(n_ext).permutation(x)
    say(f"calib bucket edges n_ext={n_ext}")
    s = F.fp8_calib_scale(dev_bf16(x), 1, 999)
    torch.cuda.synchronize()
    want = O.calib_scale(x, 1, 999)
    assert_scales_equal(s.cpu().numpy(), np.array([want], np.float32), "calib scale")


@pytest.mark.parametrize("n", [1 << 28, (1 << 32) + 8000])
def test_calib_scale_closed_form_large(F, n):
    """n values cycling through 1000 distinct bf16 values: the nearest-rank
    order statistics follow from the counts, without sorting. The second size
    takes the ranks beyond 32 bits."""
    distinct = np.unique(synth.bf16_bits_to_f32(bits_of(
        np.random.default_rng(11).standard_normal(4000) * 4)))[:1000]
    assert distinct.size == 1000
    say(f"calib closed form n={n}")
    order = np.random.default_rng(12).permutation(1000)
    pattern = torch.from_numpy(bits_of(distinct[order]).view(np.int16)).cuda()
    x = pattern.repeat(n // 1000 + 1)[:n].contiguous().view(torch.bfloat16)
    s = F.fp8_calib_scale(x, 1, 999)
    torch.cuda.synchronize()
    # counts: value index j appears n // 1000 times, plus once more for the
    # first n % 1000 positions of the pattern
    cnt = np.full(1000, n // 1000, np.int64)
    cnt[order[: n % 1000]] += 1
    cum = np.cumsum(cnt)

    def stat(permille):
        k = max(1, min(n, -((-permille * n) // 1000)))
        return float(distinct[np.searchsorted(cum, k)])

    amax = max(abs(stat(1)), abs(stat(999)))
    want = O.scale_from_amax(np.array([amax]))
    assert_scales_equal(s.cpu().numpy(), want, "calib closed form")


@pytest.mark.parametrize("n,scale", [(4096, None), (8 * 1000, 0.001), (1 << 20, None),
                                     (64, 0.0), (4096, 2.0 ** -80)])
def test_quant_static(F, n, scale):
    """Static codes with the calibrated scale (and fixed scales: a small one
    makes saturation live, 0, and a tiny one that needs the pre-scale)."""
    say(f"quant_static n={n} scale={scale}")
    x = np.ascontiguousarray(synth.activations(n // 64, 64, 8000 + n, 8001).ravel())
    xd = dev_bf16(x)
    if scale is None:
        s_dev = F.fp8_calib_scale(xd, 1, 999)
        s_host = O.calib_scale(x, 1, 999)
        torch.cuda.synchronize()
        assert_scales_equal(s_dev.cpu().numpy(), np.array([s_host], np.float32), "scale")
    else:
        s_host = np.float32(scale)
        s_dev = dev(np.array([s_host], np.float32))
    q = F.fp8_quant_static(xd, s_dev)
    torch.cuda.synchronize()
    qo = O.quant_static(x, s_host)
    assert_codes_equal(q.cpu().numpy(), qo, "static codes")
    if scale == 0.001:
        assert np.any((qo & 0x7F) == 0x7E), "saturation not exercised"


@pytest.mark.parametrize("T,width,n_slots", [(37, 1024, 64), (5, 8, 8), (300, 1024, 512),
                                             (16, 8192, 20),
                                             # every rung of the row-team ladder
                                             (64, 2048, 100), (9, 4096, 12),
                                             (5, 16384, 7), (3, 65536, 8)])
def test_kv_cache_quant(F, T, width, n_slots):
    say(f"kv cache T={T} width={width} slots={n_slots}")
    k = synth.activations(T, width, 9000 + T, 9001)
    v = synth.activations(T, width, 9002 + T, 9003)
    rng = np.random.default_rng(T)
    slots = rng.permutation(n_slots)[:T] if T <= n_slots else rng.integers(0, n_slots, T)
    slots = slots.astype(np.int64)
    slots[::5] = -1                        # not written
    if T > 3:
        slots[3] = n_slots + 7             # beyond the cache: not written
    if T > n_slots:                        # keep the written slots distinct
        seen = set()
        for i in range(T):
            if 0 <= slots[i] < n_slots:
                if slots[i] in seen:
                    slots[i] = -1
                seen.add(int(slots[i]))
    kc = torch.full((n_slots, width), 0xA5, dtype=torch.uint8, device="cuda")
    vc = torch.full((n_slots, width), 0x5A, dtype=torch.uint8, device="cuda")
    ks = torch.full((n_slots,), -7.0, dtype=torch.float32, device="cuda")
    vs = torch.full((n_slots,), -9.0, dtype=torch.float32, device="cuda")
    F.fp8_kv_cache_quant(dev_bf16(k), dev_bf16(v), torch.from_numpy(slots).cuda(), kc, vc, ks, vs)
    torch.cuda.synchronize()
    valid = np.where((slots >= 0) & (slots < n_slots), slots, -1)
    want = O.kv_quant_scatter(k, v, valid)
    kc_h, vc_h, ks_h, vs_h = kc.cpu().numpy(), vc.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy()
    for slot in range(n_slots):
        if slot in want:
            a, b, c, d = want[slot]
            assert_codes_equal(kc_h[slot], a, f"k codes slot {slot}")
            assert_codes_equal(vc_h[slot], c, f"v codes slot {slot}")
            assert ks_h[slot].view(np.uint32) == np.float32(b).view(np.uint32)
            assert vs_h[slot].view(np.uint32) == np.float32(d).view(np.uint32)
        else:
            assert np.all(kc_h[slot] == 0xA5) and np.all(vc_h[slot] == 0x5A), slot
            assert ks_h[slot] == -7.0 and vs_h[slot] == -9.0, slot


def test_next_rows_empty(F):
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = F.fp8_silu_mul_quant(e)
    assert q.shape == (0, 32)
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    q, s = F.fp8_rmsnorm_quant(e, g)
    assert q.shape == (0, 64)
    s = F.fp8_calib_scale(torch.empty((0,), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert float(s.cpu()[0]) == 0.0


def test_silu_exact_ties_round_toward_zero(F):
    """g*u an exact bf16 midpoint with silu(g) < g: the true h is just below
    the tie (in magnitude) and rounds toward zero; g in the fp32 path's range
    (48), where e^-g is subnormal in fp64 (736) and where it underflows
    (9984). A product G*U of odd mantissa parts in [257, 511] is a 9-bit odd
    number: exactly a midpoint between two bf16 values."""
    rng = np.random.default_rng(31)
    gs, us = [], []
    for g, G in ((48.0, 3), (736.0, 23), (9984.0, 39)):
        odd_u = [U for U in range(1, 256, 2) if 257 <= G * U <= 511]
        for _ in range(64):
            U = int(rng.choice(odd_u))
            u = U * 2.0 ** -int(rng.integers(0, 20)) * (1 if rng.random() < 0.5 else -1)
            assert O._near_bf16_midpoint(np.array([g * u]), 2.0 ** -60)[0]
            gs.append(g)
            us.append(u)
    n = len(gs)
    pad = (-n) % 8
    gu = bits_of(np.concatenate([gs, [1.0] * pad, us, [1.0] * pad]))[None, :]
    q, s = F.fp8_silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    qo, so = O.silu_mul_quant(gu)
    assert_scales_equal(s.cpu().numpy(), so, "tie scales")
    assert_codes_equal(q.cpu().numpy(), qo, "tie codes")


@pytest.mark.parametrize("rows,inner", SILU_SHAPES)
def test_silu_mul_bf16(F, rows, inner):
    """The bf16 h itself, bit-exact (its rounding is otherwise seen only
    through the FP8 codes, which hide most one-ulp differences)."""
    say(f"silu_mul bf16 {rows}x{inner}")
    gu = gate_up(rows, inner, 5100 + inner)
    h = F.fp8_silu_mul(dev_bf16(gu))
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.silu_mul_bf16(gu)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} h mismatches, first at {bad[:5]}"


def every_bf16_gate(seed, rows):
    """Rows [rows, 2I] holding every finite bf16 g once per row, each with its
    own random u in [-1, 1] (so h stays finite)."""
    b = np.arange(65536, dtype=np.uint32)
    finite = (b & 0x7F80) != 0x7F80
    g = b[finite].astype(np.uint16)
    pad = (-g.size) % 8
    g = np.concatenate([g, np.zeros(pad, np.uint16)])
    rng = np.random.default_rng(seed)
    u = bits_of(rng.uniform(-1.0, 1.0, (rows, g.size)))
    return np.concatenate([np.broadcast_to(g, (rows, g.size)), u], axis=1).astype(np.uint16)


def test_silu_mul_bf16_every_gate(F):
    """All finite bf16 gate values, in the fast path's range (|g| <= 64) and
    beyond, against the oracle bit for bit."""
    gu = every_bf16_gate(41, 4)
    say(f"silu_mul bf16 every gate {gu.shape}")
    h = F.fp8_silu_mul(dev_bf16(gu))
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.silu_mul_bf16(gu)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} h mismatches, first at {bad[:5]}"


@pytest.mark.parametrize("rows,hidden", RMS_SHAPES)
def test_rmsnorm_bf16(F, rows, hidden):
    say(f"rmsnorm bf16 {rows}x{hidden}")
    x, gamma = norm_input(rows, hidden, 6100 + hidden)
    h = F.fp8_rmsnorm(dev_bf16(x), dev_bf16(gamma))
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.rmsnorm_bf16(x, gamma)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} h mismatches, first at {bad[:5]}"


def test_bf16_and_fp8_outputs_agree(F):
    """The quantizing entry points quantize exactly the h the bf16 ones give."""
    gu = gate_up(33, 1536, 91)
    h = F.fp8_silu_mul(dev_bf16(gu))
    q1, s1 = F.fp8_silu_mul_quant(dev_bf16(gu))
    q2, s2 = F.fp8_quant_act(h)
    x, gamma = norm_input(33, 2048, 92)
    hn = F.fp8_rmsnorm(dev_bf16(x), dev_bf16(gamma))
    q3, s3 = F.fp8_rmsnorm_quant(dev_bf16(x), dev_bf16(gamma))
    q4, s4 = F.fp8_quant_act(hn)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    assert torch.equal(q3, q4) and torch.equal(s3, s4)


def test_silu_structural_ties(F):
    """g*u/2 an exact midpoint with tiny g (the true h is above it for g > 0,
    below for g < 0), and g*u one with huge g (below it): bf16 h and codes."""
    U = np.arange(87, 171, 2, dtype=np.float64)
    gs, us = [], []
    for g, scale in ((3.0 * 2.0 ** -102, 1.0), (-3.0 * 2.0 ** -102, 1.0),
                     (3.0 * 2.0 ** -60, 1.0), (3.0 * 2.0 ** 98, 2.0 ** -30),
                     (3.0 * 2.0 ** 40, 2.0 ** -30)):
        for sgn in (1.0, -1.0):
            gs += [g] * U.size
            us += list(sgn * U * scale)
    n = len(gs)
    pad = (-n) % 8
    gu = bits_of(np.concatenate([gs, [1.0] * pad, us, [1.0] * pad]))[None, :]
    h = F.fp8_silu_mul(dev_bf16(gu))
    q, s = F.fp8_silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.silu_mul_bf16(gu)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} h mismatches, first at {bad[:5]}"
    qo, so = O.silu_mul_quant(gu)
    assert_scales_equal(s.cpu().numpy(), so, "structural tie scales")
    assert_codes_equal(q.cpu().numpy(), qo, "structural tie codes")


def silu_big_products(rows, inner, seed):
    """Gates with |g| <= 64 beside ups near the bf16 maximum, so that g*u
    passes 2^128 (fp32 overflow) while h = silu(g) * u stays a finite bf16:
    g in [1.06, 1.3] (silu(g) <= 1.03) or in [-60, -1.06] (|silu(g)| < 0.28)
    against |u| in [1.5, 1.9] * 2^127; the other half of the columns ordinary."""
    rng = np.random.default_rng(seed)
    g = np.where(rng.random((rows, inner)) < 0.5, rng.uniform(1.06, 1.3, (rows, inner)),
                 -rng.uniform(1.06, 60.0, (rows, inner)))
    u = rng.choice([-1.0, 1.0], (rows, inner)) * rng.uniform(1.5, 1.9, (rows, inner)) * 2.0 ** 127
    plain = rng.random((rows, inner)) < 0.5
    g = np.where(plain, rng.normal(0.0, 2.0, (rows, inner)), g)
    u = np.where(plain, rng.normal(0.0, 1.0, (rows, inner)), u)
    return np.concatenate([bits_of(g), bits_of(u)], axis=1)


def test_silu_mul_fp32_overflowing_products(F):
    """Elements whose fp32 product g*u overflows while h is finite take the
    exact path: bf16 h and codes bit-exact."""
    gu = silu_big_products(16, 1024, 4242)
    want = O.silu_mul_bf16(gu)
    assert not np.any((want & 0x7F80) == 0x7F80), "test data must keep h finite"
    g = synth.bf16_bits_to_f32(gu[:, :1024]).astype(np.float32)
    u = synth.bf16_bits_to_f32(gu[:, 1024:]).astype(np.float32)
    with np.errstate(over="ignore"):
        assert np.count_nonzero(np.isinf(g * u)) > 1000, "g*u must overflow fp32"
    say(f"silu_mul fp32-overflowing g*u {gu.shape}")
    h = F.fp8_silu_mul(dev_bf16(gu))
    q, s = F.fp8_silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} h mismatches, first at {bad[:5]}"
    qo, so = O.silu_mul_quant(gu)
    assert_scales_equal(s.cpu().numpy(), so, "overflowing-product scales")
    assert_codes_equal(q.cpu().numpy(), qo, "overflowing-product codes")


def rms_tiny_products(rows, hidden, seed):
    """Rows whose RMS is 1 to 2^23 (r = 1/RMS down to 2^-23) holding, in half
    of the columns, bf16-subnormal x (down to 2^-133) under gammas of 2^100 to
    2^127: x * r falls into (or below) fp32's subnormal range while
    gamma * x * r is an ordinary normal value (the other columns' gammas are
    scaled by 2^-40, so these values also decide the scales and codes)."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1.0, (rows, hidden)) * 2.0 ** rng.integers(0, 24, (rows, 1))
    gamma = rng.normal(1.0, 0.3, hidden) * 2.0 ** -40   # so the tiny-x columns set the amax
    cols = rng.random(hidden) < 0.5
    sub = rng.integers(1, 128, (rows, hidden)) * 2.0 ** -133 * rng.choice([-1.0, 1.0], (rows, hidden))
    x = np.where(cols[None, :], sub, x)
    gamma = np.where(cols, rng.choice([2.0 ** 100, 1.5 * 2.0 ** 110, 2.0 ** 120, 1.75 * 2.0 ** 126],
                                      hidden), gamma)
    return bits_of(x), bits_of(gamma)


def test_rmsnorm_subnormal_intermediate(F):
    """x * r in fp32's subnormal range under a large gamma takes the exact
    path: bf16 h and codes bit-exact."""
    x, gamma = rms_tiny_products(16, 1024, 4343)
    say(f"rmsnorm subnormal x*r {x.shape}")
    want = O.rmsnorm_bf16(x, gamma)
    h = F.fp8_rmsnorm(dev_bf16(x), dev_bf16(gamma))
    q, s = F.fp8_rmsnorm_quant(dev_bf16(x), dev_bf16(gamma))
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} h mismatches, first at {bad[:5]}"
    qo, so = O.rmsnorm_quant(x, gamma)
    assert_scales_equal(s.cpu().numpy(), so, "subnormal-intermediate scales")
    assert_codes_equal(q.cpu().numpy(), qo, "subnormal-intermediate codes")


@pytest.mark.parametrize("eps", [1e-30, 0.5, 1e30])
def test_rmsnorm_eps_range(F, eps):
    """eps at both ends of the accepted range [1e-30, 1e30] and between, on
    rows that make it matter: an all-zero row, rows of tiny and of
    bf16-subnormal values, an ordinary row and one near the bf16 maximum.
    bf16 h and codes bit-exact."""
    rows, hidden = 8, 1024
    rng = np.random.default_rng(int(np.log10(eps)) + 200)
    xf = rng.normal(0.0, 1.0, (rows, hidden))
    xf[1] = 0.0
    xf[2] *= 1e-36                                    # tiny normal values
    xf[3] = rng.integers(1, 128, hidden) * 2.0 ** -133 * rng.choice([-1.0, 1.0], hidden)
    xf[4] *= 1e35                                     # near the bf16 maximum
    x = bits_of(xf)
    gamma = bits_of(rng.normal(1.0, 0.3, hidden))
    say(f"rmsnorm eps={eps}")
    want = O.rmsnorm_bf16(x, gamma, eps)
    h = F.fp8_rmsnorm(dev_bf16(x), dev_bf16(gamma), eps=eps)
    q, s = F.fp8_rmsnorm_quant(dev_bf16(x), dev_bf16(gamma), eps=eps)
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} h mismatches, first at {bad[:5]}"
    qo, so = O.rmsnorm_quant(x, gamma, eps)
    assert_scales_equal(s.cpu().numpy(), so, "eps-range scales")
    assert_codes_equal(q.cpu().numpy(), qo, "eps-range codes")
