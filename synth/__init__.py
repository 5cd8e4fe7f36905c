"""Seeded synthetic inputs for the FP8-Dynamic linear workloads.

This module is shared by the tests, the benchmark and the smoke check. It
holds no part of the quantization method: it only draws random numbers and
rounds them to bfloat16 (the model's I/O dtype, per the
Llama-3.1-8B-Instruct-FP8-Dynamic page, architecture notes: the model is
bfloat16). Everything is returned as raw bf16 bit patterns (``uint16``) so
that the CPU oracle and the GPU path consume identical bytes.

Workloads (all synthetic; the pages name no dataset):

* ``c1`` single linear, M=16, 4096 -> 1024.
* ``c2`` Llama-3.1-8B prefill, M=4096: qkv 4096->6144, o 4096->4096,
  gate_up 4096->28672, down 14336->4096.
* ``c3`` Llama-3.1-70B decode, M in {1, 8, 32, 64}: qkv 8192->10240,
  o 8192->8192, gate_up 8192->57344, down 28672->8192.
* ``c4`` Llama-3.2-3B block variant, M=8192: qkv 3072->5120, o 3072->3072,
  gate_up 3072->16384, down 8192->3072.
* ``c5`` long context, M=32768, gate_up 4096->28672, Student-t(3)
  activations with 0.1 % all-zero rows and planted values beyond 448.

Activations are N(0, 1) with round(0.01*K) seeded "outlier" columns scaled
by 20 before rounding; weights are N(0, 0.02) (standard deviation 0.02).

Seed rule: ``seed = 1_000_000*c + 10_000*j + 100*i + t`` with ``c`` the
workload number, ``j`` the shape index (qkv 0, o 1, gate_up 2, down 3),
``i`` the M index (c3 only) and ``t`` the tensor (0 X, 1 W, 2 outlier
columns, 3 zero rows, 4 planted values).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "SHAPES", "M_OF", "seed_of", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "activations", "weights", "long_context_activations", "workload",
]

# (name, K, N) per workload, in listed order (index j of the seed rule).
SHAPES = {
    "c1": [("single", 4096, 1024)],
    "c2": [("qkv", 4096, 6144), ("o", 4096, 4096),
           ("gate_up", 4096, 28672), ("down", 14336, 4096)],
    "c3": [("qkv", 8192, 10240), ("o", 8192, 8192),
           ("gate_up", 8192, 57344), ("down", 28672, 8192)],
    "c4": [("qkv", 3072, 5120), ("o", 3072, 3072),
           ("gate_up", 3072, 16384), ("down", 8192, 3072)],
    "c5": [("gate_up", 4096, 28672)],
}
M_OF = {"c1": [16], "c2": [4096], "c3": [1, 8, 32, 64], "c4": [8192],
        "c5": [32768]}

PLANTED = (600.0, -1000.0, 5000.0, -60000.0)


def seed_of(c: int, j: int = 0, i: int = 0, t: int = 0) -> int:
    return 1_000_000 * c + 10_000 * j + 100 * i + t


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); finite only."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def activations(M: int, K: int, seed_x: int, seed_cols: int,
                outlier_frac: float = 0.01, outlier_gain: float = 20.0,
                rows: slice | None = None) -> np.ndarray:
    """N(0,1) activations [M,K] with round(frac*K) outlier columns x gain.

    ``rows`` draws the whole matrix's stream but returns only those rows
    (the stream is consumed in row order, so a row slice is cheap to skip).
    """
    rng = np.random.default_rng(seed_x)
    r0, r1 = (0, M) if rows is None else (rows.start or 0, rows.stop or M)
    if r0:
        rng.standard_normal(size=(r0, K), dtype=np.float32)  # skip
    x = rng.standard_normal(size=(r1 - r0, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    cols = np.random.default_rng(seed_cols).permutation(K)[:n_out]
    x[:, cols] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x)


def weights(N: int, K: int, seed_w: int, std: float = 0.02) -> np.ndarray:
    """N(0, std) weights [N,K] as bf16 bits."""
    rng = np.random.default_rng(seed_w)
    w = rng.standard_normal(size=(N, K), dtype=np.float32)
    w *= np.float32(std)
    return f32_to_bf16_bits(w)


def long_context_activations(M: int, K: int, c: int = 5, j: int = 0,
                             n_rows: int | None = None):
    """Student-t(3) activations with zero rows and planted large values.

    The zero rows and planted positions are fixed by the full ``M``; only the
    leading ``n_rows`` rows (default all) are drawn and returned.
    Returns (bits [n_rows,K] uint16, zero_rows, planted [(row, col, value)]),
    with zero_rows / planted restricted to the returned rows.
    """
    n = M if n_rows is None else n_rows
    rng = np.random.default_rng(seed_of(c, j, 0, 0))
    x = np.empty((n, K), dtype=np.float32)
    step = 2048
    for r in range(0, n, step):  # chunked draw bounds the fp64 temporary
        e = min(n, r + step)
        x[r:e] = rng.standard_t(3, size=(e - r, K))
    n_zero = max(1, int(round(0.001 * M)))
    zero_rows = np.sort(np.random.default_rng(seed_of(c, j, 0, 3))
                        .permutation(M)[:n_zero])
    prng = np.random.default_rng(seed_of(c, j, 0, 4))
    nonzero = np.setdiff1d(np.arange(M), zero_rows)
    prow = prng.choice(nonzero, size=len(PLANTED), replace=False)
    pcol = prng.integers(0, K, size=len(PLANTED))
    zero_rows = zero_rows[zero_rows < n]
    x[zero_rows, :] = 0.0
    planted = []
    for r, cc, v in zip(prow, pcol, PLANTED):
        if r < n:
            x[r, cc] = v
            vb = float(bf16_bits_to_f32(f32_to_bf16_bits(np.array([v], np.float32)))[0])
            planted.append((int(r), int(cc), vb))       # value after bf16 rounding
    return f32_to_bf16_bits(x), zero_rows, planted


def workload(c: int, j: int = 0, i: int = 0, M: int | None = None,
             x: bool = True, w: bool = True):
    """Inputs of workload ``c``, shape ``j``, M index ``i``.

    Returns dict(name, M, K, N, x (bf16 bits or None), w (bf16 bits or None),
    and for c5: zero_rows, planted). ``M`` overrides the workload's M:
    smaller N(0,1) instances draw the first rows of the same stream; a
    smaller c5 instance places its own zero rows (at least one) and the
    four planted values within its M rows.
    """
    key = f"c{c}"
    name, K, N = SHAPES[key][j]
    M_full = M_OF[key][i]
    Mx = M_full if M is None else M
    out = {"name": name, "M": Mx, "K": K, "N": N, "x": None, "w": None}
    if x:
        if c == 5:
            # a smaller instance carries its own zero rows / planted values
            bits, zr, planted = long_context_activations(Mx, K, c, j)
            out["x"] = bits
            out["zero_rows"] = zr
            out["planted"] = planted
        else:
            out["x"] = activations(M_full, K, seed_of(c, j, i, 0),
                                   seed_of(c, j, 0, 2), rows=slice(0, Mx))
    if w:
        out["w"] = weights(N, K, seed_of(c, j, 0, 1))
    return out
