"""Seeded input generators: determinism, shapes and the workloads' structure."""
import numpy as np

import synth


def test_bf16_rounding_is_rne():
    f = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5e-39, 3.0e38], np.float32)
    b = synth.f32_to_bf16_bits(f)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even mantissa
    assert back[2] == 1.0 + 2.0 ** -6          # tie -> even (up)
    assert np.signbit(back[3])
    assert np.isfinite(back[4])


def test_deterministic_and_row_prefix():
    a = synth.workload(2, 0, M=64, w=False)["x"]
    b = synth.workload(2, 0, M=64, w=False)["x"]
    assert np.array_equal(a, b)
    c = synth.workload(2, 0, M=16, w=False)["x"]
    assert np.array_equal(a[:16], c)


def test_outlier_columns():
    x = synth.bf16_bits_to_f32(synth.workload(1, w=False)["x"])
    col_rms = np.sqrt((x.astype(np.float64) ** 2).mean(0))
    assert (col_rms > 8).sum() == round(0.01 * 4096)


def test_weight_std():
    w = synth.bf16_bits_to_f32(synth.weights(256, 4096, 1))
    assert abs(w.std() - 0.02) < 5e-4


def test_long_context_structure():
    d = synth.workload(5, M=2048, w=False)
    x = synth.bf16_bits_to_f32(d["x"])
    assert len(d["zero_rows"]) == 2
    assert np.all(x[d["zero_rows"]] == 0)
    assert len(d["planted"]) == 4
    for r, c, v in d["planted"]:
        assert x[r, c] == v
    assert np.abs(x).max() > 448
