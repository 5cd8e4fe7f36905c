"""The C-ABI library loads, exports what include/fp8dq.h declares and rejects
bad arguments on the host (no GPU needed: every case below returns before
anything would be enqueued)."""
import ctypes
import os

import pytest

import fp8_dynamic_quantized_amd as F
from fp8_dynamic_quantized_amd import build as B


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB):
        B.build()
    return F.lib()


P = ctypes.c_void_p
A = P(0x10000)          # a 16-byte aligned stand-in address (never dereferenced)
MIS = P(0x10004)        # misaligned stand-in


def test_exports_every_declared_symbol(L):
    names = F.header_functions()
    assert {"fp8_quant_act", "fp8_linear", "fp8_linear_block"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert F.fp8_status_string(code) not in ("", "unknown status")
    assert F.fp8_status_string(99) == "unknown status"
    assert F.fp8dq_version().count(".") == 2


def test_quant_act_errors(L):
    q = L.fp8_quant_act
    assert q(None, 4, 64, 0, A, A, None) == -1
    assert q(A, 4, 64, 0, None, A, None) == -1
    assert q(A, 4, 64, 0, A, None, None) == -1
    assert q(A, -1, 64, 0, A, A, None) == -2
    assert q(A, 4, 0, 0, A, A, None) == -2
    assert q(A, 4, 60, 0, A, A, None) == -2        # K % 8
    assert q(A, 4, 192, 128, A, A, None) == -2     # K % 128 for groups
    assert q(A, 4, 64, 64, A, A, None) == -5       # group must be 0 or 128
    assert q(MIS, 4, 64, 0, A, A, None) == -3
    assert q(A, 4, 64, 0, MIS, A, None) == -3
    assert q(None, 0, 64, 0, None, None, None) == 0  # empty: nothing to do


def test_quant_weight_block_errors(L):
    f = L.fp8_quant_weight_block
    assert f(None, 128, 128, A, A, None) == -1
    assert f(A, 100, 128, A, A, None) == -2
    assert f(A, 128, 100, A, A, None) == -2
    assert f(A, 128, 128, MIS, A, None) == -3
    assert f(None, 0, 128, None, None, None) == 0


@pytest.mark.parametrize("fn", ["fp8_gemm", "fp8_gemm_block"])
def test_gemm_errors(L, fn):
    g = getattr(L, fn)
    assert g(None, A, A, A, A, 16, 128, 128, 0, None, 0, None) == -1
    assert g(A, A, A, A, None, 16, 128, 128, 0, None, 0, None) == -1
    assert g(A, A, A, A, A, -1, 128, 128, 0, None, 0, None) == -2
    assert g(A, A, A, A, A, 16, 128, 100, 0, None, 0, None) == -2   # K % 128
    assert g(A, A, A, A, A, 16, 128, 0, 0, None, 0, None) == -2
    assert g(A, A, A, A, A, 16, 128, 128, 7, None, 0, None) == -5
    assert g(A, A, MIS, A, A, 100, 128, 128, 1, None, 0, None) == -3
    assert g(A, A, A, A, A, 0, 128, 128, 0, None, 0, None) == 0     # empty M
    assert g(None, None, None, None, None, 16, 0, 128, 0, None, 0, None) == 0
    # weight codes must stay under 4 GiB (32-bit offsets), on every path
    assert g(A, A, A, A, A, 128, 1 << 16, 1 << 16, 0, None, 0, None) == -2
    assert g(A, A, A, A, A, 16, 1 << 16, 1 << 16, 1, None, 0, None) == -2
    assert g(A, A, A, A, A, 32, 1 << 16, 1 << 16, 0, None, 0, None) == -2
    assert g(A, A, A, A, A, 1, 1 << 16, 1 << 16, 2, None, 0, None) == -2
    # K beyond FP8DQ_MAX_K = 2^17 (the range the accumulation error is
    # validated over) is rejected on every path; 2^17 itself is accepted
    for flags in (0, 1, 2):
        assert g(A, A, A, A, A, 65536, 128, 1 << 24, flags, None, 0, None) == -2
        assert g(A, A, A, A, A, 16, 128, (1 << 17) + 128, flags, None, 0, None) == -2
        assert g(A, A, A, A, A, 4096, 128, (1 << 17) + 128, flags, None, 0, None) == -2
    assert g(A, A, A, A, A, 16, 128, 1 << 17, 0, None, 0, None) != -2


def test_gemm_block_needs_n_multiple_of_128(L):
    assert L.fp8_gemm_block(A, A, A, A, A, 16, 200, 128, 0, None, 0, None) == -2
    assert L.fp8_linear_block(A, A, A, A, 16, 200, 128, A, A, 0, None, 0, None) == -2


def test_workspace_rules(L):
    # decode shapes whose row blocks leave the CUs short of work split K and
    # need a workspace: a zeroed counter area of 16 KiB, then fp32 partials
    # (splits x M x N); prefill needs none
    # (partial tiles of 16 x 16 floats, or 128 x 16*ceil(M/16) floats)
    for M, N, K in [(16, 1024, 16384), (1, 96, 131072), (64, 8192, 28672), (20, 100, 65536)]:
        need = F.fp8_workspace_bytes(M, N, K)
        assert need >= 16384 + 2 * 1024 and (need - 16384) % 1024 == 0, (M, N, K)
    # 16-row weight blocks (up to 4 tokens): no split with as many blocks as
    # CUs, nor on rows shorter than 16384
    assert F.fp8_workspace_bytes(1, 57344, 8192) == 0
    assert F.fp8_workspace_bytes(4, 10240, 8192) == 0
    assert F.fp8_workspace_bytes(4, 1024, 4096) == 0
    # 128-row weight blocks (5-64 tokens): fewer blocks than CUs split K
    assert F.fp8_workspace_bytes(8, 10240, 8192) > 0
    assert F.fp8_workspace_bytes(16, 1024, 4096) > 0
    assert F.fp8_workspace_bytes(32, 1024, 4096) > 0
    assert F.fp8_workspace_bytes(8, 57344, 8192) == 0      # 448 blocks: no split
    assert F.fp8_workspace_bytes(4096, 4096, 4096) == 0
    assert F.fp8_workspace_bytes(16, 1024, 16384, flags=F.FORCE_PREFILL) == 0
    assert F.fp8_workspace_bytes(16, 1024, 100) == 0       # invalid K -> 0
    assert F.fp8_workspace_bytes(16, 1024, (1 << 17) + 128) == 0   # K beyond the bound -> 0
    assert F.fp8_workspace_bytes(16, 1000, 4096, block=True) == 0  # invalid N
    need = F.fp8_workspace_bytes(16, 1024, 16384)
    g = L.fp8_gemm
    assert g(A, A, A, A, A, 16, 1024, 16384, 0, None, 0, None) == -1
    assert g(A, A, A, A, A, 16, 1024, 16384, 0, A, need - 4, None) == -4
    assert g(A, A, A, A, A, 16, 1024, 16384, 0, MIS, need, None) == -3
    # M beyond one decode slab (64 rows) takes the larger of a full slab's and
    # the last slab's workspace
    assert F.fp8_workspace_bytes(200, 1024, 16384, flags=F.FORCE_DECODE) == max(
        F.fp8_workspace_bytes(64, 1024, 16384), F.fp8_workspace_bytes(8, 1024, 16384))


@pytest.mark.parametrize("fn", ["fp8_linear", "fp8_linear_block"])
def test_linear_errors(L, fn):
    f = getattr(L, fn)
    assert f(None, A, A, A, 16, 128, 128, A, A, 0, None, 0, None) == -1
    assert f(A, A, A, A, 16, 128, 128, None, A, 0, None, 0, None) == -1
    assert f(MIS, A, A, A, 16, 128, 128, A, A, 0, None, 0, None) == -3
    assert f(A, A, A, A, 16, 128, 96, A, A, 0, None, 0, None) == -2
    assert f(A, A, A, A, 16, 128, 128, A, A, 9, None, 0, None) == -5
    assert f(None, None, None, None, 0, 128, 128, None, None, 0, None, 0, None) == 0


def test_fused_producer_errors(L):
    f = L.fp8_silu_mul_quant
    assert f(None, 4, 256, A, A, None) == -1
    assert f(A, 4, 100, A, A, None) == -2          # I % 8
    assert f(A, 4, 65536 + 8, A, A, None) == -2    # row too long
    assert f(A, -1, 256, A, A, None) == -2
    assert f(MIS, 4, 256, A, A, None) == -3
    assert f(None, 0, 256, None, None, None) == 0   # empty
    g = L.fp8_rmsnorm_quant
    assert g(A, None, 4, 256, 1e-5, A, A, None) == -1
    assert g(A, A, 4, 12, 1e-5, A, A, None) == -2
    assert g(A, A, 4, 256, -1.0, A, A, None) == -2    # negative eps
    assert g(A, A, 4, 256, 0.0, A, A, None) == -2     # eps below 1e-30
    assert g(A, A, 4, 256, 1e-31, A, A, None) == -2
    assert g(A, A, 4, 256, 1e31, A, A, None) == -2
    assert g(A, A, 4, 256, float("nan"), A, A, None) == -2
    assert g(A, MIS, 4, 256, 1e-5, A, A, None) == -3
    assert g(None, None, 0, 256, 1e-5, None, None, None) == 0
    f = L.fp8_silu_mul
    assert f(None, 4, 256, A, None) == -1
    assert f(A, 4, 100, A, None) == -2
    assert f(A, 4, 65536 + 8, A, None) == -2
    assert f(A, 4, 256, MIS, None) == -3
    assert f(None, 0, 256, None, None) == 0
    g = L.fp8_rmsnorm
    assert g(A, A, 4, 256, 1e-5, None, None) == -1
    assert g(A, A, 4, 12, 1e-5, A, None) == -2
    assert g(A, A, 4, 256, -1.0, A, None) == -2
    assert g(A, A, 4, 256, 0.0, A, None) == -2
    assert g(A, A, 4, 256, 1e-5, MIS, None) == -3
    assert g(None, None, 0, 256, 1e-5, None, None) == 0


def test_calibration_and_static_errors(L):
    need = F.fp8_calib_workspace_bytes(4096)
    assert need > 0
    c = L.fp8_calib_scale
    assert c(A, 4096, 1, 999, A, None, need, None) == -1
    assert c(A, 4096, 1, 999, A, A, need - 4, None) == -4
    assert c(A, 4095, 1, 999, A, A, need, None) == -2      # n % 8
    assert c(A, 4096, 999, 1, A, A, need, None) == -2      # lo > hi
    assert c(A, 4096, 1, 1001, A, A, need, None) == -2
    assert c(A, 1 << 40, 1, 999, A, A, need, None) == -2
    assert c(MIS, 4096, 1, 999, A, A, need, None) == -3
    s = L.fp8_quant_static
    assert s(A, 100, A, A, None) == -2
    assert s(None, 64, A, A, None) == -1
    assert s(A, 0, None, None, None) == 0


def test_kv_cache_errors(L):
    k = L.fp8_kv_cache_quant
    assert k(A, A, 8, 1024, None, 16, A, A, A, A, None) == -1
    assert k(A, A, 8, 1000 + 4, A, 16, A, A, A, A, None) == -2
    assert k(A, A, 8, 1024, A, -1, A, A, A, A, None) == -2
    assert k(A, MIS, 8, 1024, A, 16, A, A, A, A, None) == -3
    assert k(None, None, 0, 1024, None, 16, None, None, None, None, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from fp8_dynamic_quantized_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _binding.lib()


def test_binding_tensor_checks():
    """The binding's per-tensor check (before any pointer reaches the
    library): dtype, shape, layout and device; block shapes need N and K
    multiples of 128 (host logic only, so host tensors stand in)."""
    import torch
    from fp8_dynamic_quantized_amd import _binding
    need = _binding._need
    t = torch.zeros((4, 8), dtype=torch.uint8)
    with pytest.raises(ValueError, match="expected"):
        need(t, torch.float32, (4, 8), "t")                     # dtype
    with pytest.raises(ValueError, match="expected"):
        need(t, torch.uint8, (4, 16), "t")                      # shape
    with pytest.raises(ValueError, match="expected"):
        need(t.t(), torch.uint8, (8, 4), "t")                   # not contiguous
    with pytest.raises(ValueError, match="device memory"):
        need(t, torch.uint8, (4, 8), "t")                       # host memory
    with pytest.raises(ValueError, match="missing"):
        need(None, torch.uint8, (4, 8), "t")
    with pytest.raises(ValueError, match="multiples of 128"):
        _binding._need_blocks(200, 512)
    with pytest.raises(ValueError, match="multiples of 128"):
        _binding._need_blocks(256, 320)
    _binding._need_blocks(256, 512)
    with pytest.raises(ValueError, match="contiguous device memory"):
        _binding._need_ws(torch.zeros(16, dtype=torch.uint8), torch.device("cuda", 0))
    with pytest.raises(ValueError, match="multiples of 128"):
        F.fp8_gemm_block(torch.zeros((8, 512), dtype=torch.uint8), torch.ones((8, 4)),
                         torch.zeros((200, 512), dtype=torch.uint8), torch.ones((2, 4)))
