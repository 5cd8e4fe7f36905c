"""ctypes binding of libfp8dq.so: argument marshalling only.

Every function here has the name of a C entry point in include/fp8dq.h,
takes torch tensors (device memory) and passes their pointers, sizes and
the current HIP stream to the library. All arithmetic runs in the library's
HIP kernels; there is no other implementation to fall back to, and a missing
library raises.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp8dq.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "fp8dq.h")

AUTO, FORCE_PREFILL, FORCE_DECODE = 0, 1, 2
DECODE_MAX_M = 64
GROUP = 128

_c_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "fp8_quant_act": (ctypes.c_int, [_c_p, _i64, _i64, ctypes.c_int32, _c_p, _c_p, _c_p]),
    "fp8_quant_weight_block": (ctypes.c_int, [_c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "fp8_gemm": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64,
                                ctypes.c_uint32, _c_p, ctypes.c_size_t, _c_p]),
    "fp8_gemm_block": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64,
                                      ctypes.c_uint32, _c_p, ctypes.c_size_t, _c_p]),
    "fp8_linear": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _c_p, _c_p,
                                  ctypes.c_uint32, _c_p, ctypes.c_size_t, _c_p]),
    "fp8_linear_block": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _c_p,
                                        _c_p, ctypes.c_uint32, _c_p, ctypes.c_size_t, _c_p]),
    "fp8_linear_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _c_p,
                                          _c_p, ctypes.c_uint32, _c_p]),
    "fp8_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, ctypes.c_int32, ctypes.c_uint32]),
    "fp8_silu_mul_quant": (ctypes.c_int, [_c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "fp8_rmsnorm_quant": (ctypes.c_int, [_c_p, _c_p, _i64, _i64, ctypes.c_double, _c_p,
                                         _c_p, _c_p]),
    "fp8_silu_mul": (ctypes.c_int, [_c_p, _i64, _i64, _c_p, _c_p]),
    "fp8_rmsnorm": (ctypes.c_int, [_c_p, _c_p, _i64, _i64, ctypes.c_double, _c_p, _c_p]),
    "fp8_calib_workspace_bytes": (ctypes.c_size_t, [_i64]),
    "fp8_calib_scale": (ctypes.c_int, [_c_p, _i64, ctypes.c_int32, ctypes.c_int32, _c_p,
                                       _c_p, ctypes.c_size_t, _c_p]),
    "fp8_quant_static": (ctypes.c_int, [_c_p, _i64, _c_p, _c_p, _c_p]),
    "fp8_kv_cache_quant": (ctypes.c_int, [_c_p, _c_p, _i64, _i64, _c_p, _i64, _c_p, _c_p,
                                          _c_p, _c_p, _c_p]),
    "fp8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8dq_version": (ctypes.c_char_p, []),
}

_lib = None


class Fp8dqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_text(status)})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m fp8_dynamic_quantized_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/fp8dq.h declares."""
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)


def status_text(status: int) -> str:
    return lib().fp8_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp8dqError(fn, status)


def _ptr(t):
    # a plain int: the argtypes (c_void_p) convert it, with no object per call
    return None if t is None else t.data_ptr()


def _stream(t, stream):
    """The HIP stream to enqueue on: the one given, else torch's current
    stream of t's device (read through torch's raw-stream accessor where it
    has one: a small call matters when a decode linear takes 15 us)."""
    import torch
    if stream is not None:
        return stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, shape, name, dev=None):
    """Check one tensor argument before its pointer reaches the library: the
    library sees only pointers and sizes, so a wrong shape, dtype, layout or
    device here would become an out-of-bounds access on the GPU."""
    if t is None:
        raise ValueError(f"{name}: missing")
    if t.dtype is not dtype or t.shape != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be device memory")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name}: on {t.device}, the other operands on {dev}")


def _need_ws(ws, dev):
    """A caller's workspace: contiguous device memory on the operands' device
    (its size is checked by the library)."""
    if ws is None:
        return
    if not ws.is_contiguous() or not ws.is_cuda or ws.device != dev:
        raise ValueError(f"ws: expected contiguous device memory on {dev}")


def _need_blocks(N, K):
    if N % GROUP or K % GROUP:
        raise ValueError(f"block scales need N and K multiples of {GROUP}, got N={N}, K={K}")


def fp8_workspace_bytes(M: int, N: int, K: int, block: bool = False,
                        flags: int = AUTO) -> int:
    return int(lib().fp8_workspace_bytes(M, N, K, int(block), flags))


def fp8_status_string(status: int) -> str:
    return status_text(status)


def fp8dq_version() -> str:
    return lib().fp8dq_version().decode()


def fp8_quant_act(x, group: int = 0, q=None, scale=None, stream=None):
    """Quantize bf16 x [rows, K] -> (codes uint8 [rows, K], scales fp32)."""
    import torch
    rows, K = x.shape
    _need(x, torch.bfloat16, (rows, K), "x")
    if group not in (0, GROUP):
        raise ValueError(f"group: 0 or {GROUP}, got {group}")
    if group and K % GROUP:
        raise ValueError(f"group {GROUP} needs K a multiple of {GROUP}, got {K}")
    sshape = (rows,) if group == 0 else (rows, K // GROUP)
    q = torch.empty((rows, K), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty(sshape, dtype=torch.float32, device=x.device) if scale is None else scale
    _need(q, torch.uint8, (rows, K), "q", x.device)
    _need(scale, torch.float32, sshape, "scale", x.device)
    _check("fp8_quant_act", lib().fp8_quant_act(
        _ptr(x), rows, K, group, _ptr(q), _ptr(scale), _stream(x, stream)))
    return q, scale


def fp8_quant_weight_block(w, qw=None, sw=None, stream=None):
    """128x128 block quantization of bf16 w [N, K] -> (codes, sw [N/128, K/128])."""
    import torch
    N, K = w.shape
    _need(w, torch.bfloat16, (N, K), "w")
    _need_blocks(N, K)
    qw = torch.empty((N, K), dtype=torch.uint8, device=w.device) if qw is None else qw
    sw = torch.empty((N // GROUP, K // GROUP), dtype=torch.float32,
                     device=w.device) if sw is None else sw
    _need(qw, torch.uint8, (N, K), "qw", w.device)
    _need(sw, torch.float32, (N // GROUP, K // GROUP), "sw", w.device)
    _check("fp8_quant_weight_block", lib().fp8_quant_weight_block(
        _ptr(w), N, K, _ptr(qw), _ptr(sw), _stream(w, stream)))
    return qw, sw


def _workspace(M, N, K, block, flags, ws, device):
    """The caller's workspace and its size in bytes, or a zero-filled one of
    the size the call needs (the library checks the size either way)."""
    import torch
    if ws is None:
        need = fp8_workspace_bytes(M, N, K, block, flags)
        if need:
            ws = torch.zeros(need, dtype=torch.uint8, device=device)   # counters start at zero
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return ws, nbytes


def fp8_gemm(qx, sx, qw, sw, y=None, flags: int = AUTO, ws=None, stream=None):
    """y = bf16((qx qw^T) * sx[m] * sw[n]); codes uint8, scales fp32."""
    import torch
    M, K = qx.shape
    N = qw.shape[0]
    dev = qx.device
    _need(qx, torch.uint8, (M, K), "qx", dev)
    _need(sx, torch.float32, (M,), "sx", dev)
    _need(qw, torch.uint8, (N, K), "qw", dev)
    _need(sw, torch.float32, (N,), "sw", dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, torch.bfloat16, (M, N), "y", dev)
    _need_ws(ws, dev)
    ws, nb = _workspace(M, N, K, False, flags, ws, dev)
    _check("fp8_gemm", lib().fp8_gemm(
        _ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(y), M, N, K, flags,
        _ptr(ws), nb, _stream(qx, stream)))
    return y


def fp8_gemm_block(qx, sx, qw, sw, y=None, flags: int = AUTO, ws=None, stream=None):
    """Block-scaled GEMM: sx [M, K/128], sw [N/128, K/128]."""
    import torch
    M, K = qx.shape
    N = qw.shape[0]
    dev = qx.device
    _need_blocks(N, K)
    _need(qx, torch.uint8, (M, K), "qx", dev)
    _need(sx, torch.float32, (M, K // GROUP), "sx", dev)
    _need(qw, torch.uint8, (N, K), "qw", dev)
    _need(sw, torch.float32, (N // GROUP, K // GROUP), "sw", dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, torch.bfloat16, (M, N), "y", dev)
    _need_ws(ws, dev)
    ws, nb = _workspace(M, N, K, True, flags, ws, dev)
    _check("fp8_gemm_block", lib().fp8_gemm_block(
        _ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(y), M, N, K, flags,
        _ptr(ws), nb, _stream(qx, stream)))
    return y


def fp8_linear(x, qw, sw, y=None, qx_out=None, sx_out=None, flags: int = AUTO,
               ws=None, stream=None):
    """FP8-Dynamic linear: per-token quantization of x, then the FP8 GEMM.

    Returns (y bf16 [M, N], qx uint8 [M, K], sx fp32 [M]).
    """
    import torch
    M, K = x.shape
    N = qw.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    dev = x.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    qx_out = torch.empty((M, K), dtype=torch.uint8, device=dev) if qx_out is None else qx_out
    sx_out = torch.empty((M,), dtype=torch.float32, device=dev) if sx_out is None else sx_out
    _need(qw, torch.uint8, (N, K), "qw", dev)
    _need(sw, torch.float32, (N,), "sw", dev)
    _need(y, torch.bfloat16, (M, N), "y", dev)
    _need(qx_out, torch.uint8, (M, K), "qx_out", dev)
    _need(sx_out, torch.float32, (M,), "sx_out", dev)
    _need_ws(ws, dev)
    ws, nb = _workspace(M, N, K, False, flags, ws, dev)
    _check("fp8_linear", lib().fp8_linear(
        _ptr(x), _ptr(qw), _ptr(sw), _ptr(y), M, N, K, _ptr(qx_out), _ptr(sx_out),
        flags, _ptr(ws), nb, _stream(x, stream)))
    return y, qx_out, sx_out


def fp8_linear_noalloc(x, qw, sw, y=None, qx_out=None, sx_out=None, flags: int = AUTO,
                       stream=None):
    """fp8_linear without a workspace (the library's static device scratch).

    Returns (y bf16 [M, N], qx uint8 [M, K], sx fp32 [M]); outputs not passed
    are allocated here, by torch, before the call.
    """
    import torch
    M, K = x.shape
    N = qw.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    dev = x.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    qx_out = torch.empty((M, K), dtype=torch.uint8, device=dev) if qx_out is None else qx_out
    sx_out = torch.empty((M,), dtype=torch.float32, device=dev) if sx_out is None else sx_out
    _need(qw, torch.uint8, (N, K), "qw", dev)
    _need(sw, torch.float32, (N,), "sw", dev)
    _need(y, torch.bfloat16, (M, N), "y", dev)
    _need(qx_out, torch.uint8, (M, K), "qx_out", dev)
    _need(sx_out, torch.float32, (M,), "sx_out", dev)
    _check("fp8_linear_noalloc", lib().fp8_linear_noalloc(
        _ptr(x), _ptr(qw), _ptr(sw), _ptr(y), M, N, K, _ptr(qx_out), _ptr(sx_out),
        flags, _stream(x, stream)))
    return y, qx_out, sx_out


def fp8_linear_block(x, qw, sw, y=None, qx_out=None, sx_out=None,
                     flags: int = AUTO, ws=None, stream=None):
    """Block variant: group-128 activation quantization, block-scaled GEMM.

    Returns (y bf16 [M, N], qx uint8 [M, K], sx fp32 [M, K/128]).
    """
    import torch
    M, K = x.shape
    N = qw.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need_blocks(N, K)
    dev = x.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    qx_out = torch.empty((M, K), dtype=torch.uint8, device=dev) if qx_out is None else qx_out
    sx_out = (torch.empty((M, K // GROUP), dtype=torch.float32, device=dev)
              if sx_out is None else sx_out)
    _need(qw, torch.uint8, (N, K), "qw", dev)
    _need(sw, torch.float32, (N // GROUP, K // GROUP), "sw", dev)
    _need(y, torch.bfloat16, (M, N), "y", dev)
    _need(qx_out, torch.uint8, (M, K), "qx_out", dev)
    _need(sx_out, torch.float32, (M, K // GROUP), "sx_out", dev)
    _need_ws(ws, dev)
    ws, nb = _workspace(M, N, K, True, flags, ws, dev)
    _check("fp8_linear_block", lib().fp8_linear_block(
        _ptr(x), _ptr(qw), _ptr(sw), _ptr(y), M, N, K, _ptr(qx_out), _ptr(sx_out),
        flags, _ptr(ws), nb, _stream(x, stream)))
    return y, qx_out, sx_out


# ----------------------------------------------------------------------------
# Fused producers, static calibration, FP8 KV cache
# ----------------------------------------------------------------------------
RMS_EPS = 1e-5


def fp8_silu_mul_quant(gu, q=None, scale=None, stream=None):
    """gu bf16 [rows, 2I] = (gate | up) -> per-token FP8 of bf16(silu(gate) * up).

    Returns (codes uint8 [rows, I], scales fp32 [rows])."""
    import torch
    rows, two_i = gu.shape
    _need(gu, torch.bfloat16, (rows, two_i), "gu")
    if two_i % 2:
        raise ValueError("gu: the column count must be even (gate | up)")
    inner = two_i // 2
    q = torch.empty((rows, inner), dtype=torch.uint8, device=gu.device) if q is None else q
    scale = torch.empty((rows,), dtype=torch.float32, device=gu.device) if scale is None else scale
    _need(q, torch.uint8, (rows, inner), "q", gu.device)
    _need(scale, torch.float32, (rows,), "scale", gu.device)
    _check("fp8_silu_mul_quant", lib().fp8_silu_mul_quant(
        _ptr(gu), rows, inner, _ptr(q), _ptr(scale), _stream(gu, stream)))
    return q, scale


def fp8_rmsnorm_quant(x, gamma, eps: float = RMS_EPS, q=None, scale=None, stream=None):
    """x bf16 [rows, H], gamma bf16 [H] -> per-token FP8 of
    bf16(gamma * x / sqrt(mean(x^2) + eps)). Returns (codes, scales)."""
    import torch
    rows, hidden = x.shape
    _need(x, torch.bfloat16, (rows, hidden), "x")
    _need(gamma, torch.bfloat16, (hidden,), "gamma", x.device)
    q = torch.empty((rows, hidden), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((rows,), dtype=torch.float32, device=x.device) if scale is None else scale
    _need(q, torch.uint8, (rows, hidden), "q", x.device)
    _need(scale, torch.float32, (rows,), "scale", x.device)
    _check("fp8_rmsnorm_quant", lib().fp8_rmsnorm_quant(
        _ptr(x), _ptr(gamma), rows, hidden, float(eps), _ptr(q), _ptr(scale),
        _stream(x, stream)))
    return q, scale


def fp8_silu_mul(gu, out=None, stream=None):
    """gu bf16 [rows, 2I] = (gate | up) -> bf16(silu(gate) * up) [rows, I]."""
    import torch
    rows, two_i = gu.shape
    _need(gu, torch.bfloat16, (rows, two_i), "gu")
    if two_i % 2:
        raise ValueError("gu: the column count must be even (gate | up)")
    inner = two_i // 2
    out = torch.empty((rows, inner), dtype=torch.bfloat16, device=gu.device) if out is None else out
    _need(out, torch.bfloat16, (rows, inner), "out", gu.device)
    _check("fp8_silu_mul", lib().fp8_silu_mul(_ptr(gu), rows, inner, _ptr(out),
                                              _stream(gu, stream)))
    return out


def fp8_rmsnorm(x, gamma, eps: float = RMS_EPS, out=None, stream=None):
    """x bf16 [rows, H], gamma bf16 [H] -> bf16(gamma * x / sqrt(mean(x^2) + eps))."""
    import torch
    rows, hidden = x.shape
    _need(x, torch.bfloat16, (rows, hidden), "x")
    _need(gamma, torch.bfloat16, (hidden,), "gamma", x.device)
    out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(out, torch.bfloat16, (rows, hidden), "out", x.device)
    _check("fp8_rmsnorm", lib().fp8_rmsnorm(_ptr(x), _ptr(gamma), rows, hidden, float(eps),
                                            _ptr(out), _stream(x, stream)))
    return out


def fp8_calib_workspace_bytes(n: int) -> int:
    return int(lib().fp8_calib_workspace_bytes(n))


def fp8_calib_scale(x, lo_permille: int = 1, hi_permille: int = 999, scale=None,
                    ws=None, stream=None):
    """Static per-tensor scale RN(max(|P_lo|, |P_hi|) / 448) of a bf16 tensor
    (nearest-rank percentiles, per mille). Returns a device fp32 [1] tensor."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x: contiguous bf16 device tensor expected")
    n = x.numel()
    scale = torch.empty((1,), dtype=torch.float32, device=x.device) if scale is None else scale
    _need(scale, torch.float32, (1,), "scale", x.device)
    need = fp8_calib_workspace_bytes(n)
    ws = torch.empty(need, dtype=torch.uint8, device=x.device) if ws is None else ws
    _need_ws(ws, x.device)
    _check("fp8_calib_scale", lib().fp8_calib_scale(
        _ptr(x), n, lo_permille, hi_permille, _ptr(scale), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(x, stream)))
    return scale


def fp8_quant_static(x, scale, q=None, stream=None):
    """E4M3 codes of a bf16 tensor with one static device-resident fp32 scale
    (saturating at +-448). Returns codes with x's shape."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x: contiguous bf16 device tensor expected")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    _need(scale, torch.float32, (1,), "scale", x.device)   # read on the device
    _need(q, torch.uint8, tuple(x.shape), "q", x.device)
    _check("fp8_quant_static", lib().fp8_quant_static(
        _ptr(x), x.numel(), _ptr(scale), _ptr(q), _stream(x, stream)))
    return q


def fp8_kv_cache_quant(k, v, slots, k_cache, v_cache, k_scale, v_scale, stream=None):
    """Per-token FP8 quantization of K and V [T, width] (bf16) into cache rows
    slots[t] (int64; negative or >= the cache's rows: not written)."""
    import torch
    T, width = k.shape
    _need(k, torch.bfloat16, (T, width), "k")
    dev = k.device
    _need(v, torch.bfloat16, (T, width), "v", dev)
    _need(slots, torch.int64, (T,), "slots", dev)
    n_slots = k_cache.shape[0]
    _need(k_cache, torch.uint8, (n_slots, width), "k_cache", dev)
    _need(v_cache, torch.uint8, (n_slots, width), "v_cache", dev)
    _need(k_scale, torch.float32, (n_slots,), "k_scale", dev)
    _need(v_scale, torch.float32, (n_slots,), "v_scale", dev)
    _check("fp8_kv_cache_quant", lib().fp8_kv_cache_quant(
        _ptr(k), _ptr(v), T, width, _ptr(slots), n_slots, _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _stream(k, stream)))
