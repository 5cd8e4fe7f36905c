"""Helpers of the GPU parity tests (host <-> device marshalling, comparison)."""
import os
import sys

import numpy as np
import torch

import oracle.fp8dq_oracle as O


def ensure_built():
    from fp8_dynamic_quantized_amd import build as B
    if not os.path.exists(B.LIB):
        B.build()
    import fp8_dynamic_quantized_amd as F
    F.lib()
    return F


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_bf16_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f64(host_bits(t))


def assert_codes_equal(got: np.ndarray, want: np.ndarray, what: str):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} code mismatches, first at {i}: "
                             f"got 0x{int(got[i]):02x} want 0x{int(want[i]):02x}")


def assert_scales_equal(got: np.ndarray, want: np.ndarray, what: str):
    g = np.ascontiguousarray(got, np.float32).view(np.uint32)
    w = np.ascontiguousarray(want, np.float32).view(np.uint32)
    if not np.array_equal(g, w):
        bad = np.argwhere(g != w)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} scale mismatches, first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


# Output tolerance of the FP8-Dynamic linear: |y - y_ref| <= 1e-3 + 1e-2 |y_ref|
RTOL, ATOL = 1e-2, 1e-3


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray, what: str):
    ok = O.within_tolerance(y_gpu, y_ref, RTOL, ATOL)
    exact = np.mean(y_gpu == O.f64_to_bf16_rne(y_ref))
    err = np.abs(y_gpu - y_ref)
    rel = np.max(err / np.maximum(np.abs(y_ref), 1e-30)) if err.size else 0.0
    say(f"  {what}: n={y_ref.size} max_abs={err.max() if err.size else 0:.3g} "
        f"max_rel={rel:.3g} exact_bf16_frac={exact:.4f}")
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} outputs out of tolerance, first at {i}: "
                             f"got {y_gpu[i]!r} want {y_ref[i]!r}")
