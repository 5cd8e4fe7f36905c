// C-ABI boundary of the FP8-Dynamic linear library (see include/fp8dq.h).
// Every argument is checked here, on the host, before anything is enqueued.
#include "fp8dq.h"

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace {

using fp8dq::DecodePlan;

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8DQ_OK : FP8DQ_ERR_HIP;
}

inline bool known_flags(uint32_t f) {
  return f == FP8DQ_AUTO || f == FP8DQ_FORCE_PREFILL || f == FP8DQ_FORCE_DECODE;
}

inline bool use_decode(int64_t M, uint32_t flags) {
  if (flags == FP8DQ_FORCE_DECODE) return true;
  if (flags == FP8DQ_FORCE_PREFILL) return false;
  return M <= FP8DQ_DECODE_MAX_M;
}

// Workspace for a GEMM call: the decode path processes M in slabs of at
// most 64 rows (one after another on the stream), so the larger of a full
// slab's and the last slab's needs.
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, uint32_t flags,
                     size_t cap = SIZE_MAX) {
  if (M <= 0 || N <= 0 || K <= 0 || (K % 128) != 0 || K > FP8DQ_MAX_K) return 0;
  if (!use_decode(M, flags)) return 0;
  size_t need = 0;
  const int64_t slabs[2] = {M < FP8DQ_DECODE_MAX_M ? M : FP8DQ_DECODE_MAX_M,
                            M % FP8DQ_DECODE_MAX_M};
  for (int64_t slab : slabs) {
    if (slab <= 0) continue;
    const DecodePlan p = fp8dq::plan_decode(slab, N, K, cap);
    const size_t b = fp8dq::decode_workspace_bytes(slab, N, p);
    if (b > need) need = b;
  }
  return need;
}

int check_gemm_args(const uint8_t* qx, const float* sx, const uint8_t* qw,
                    const float* sw, const void* y, int64_t M, int64_t N,
                    int64_t K, uint32_t flags, const void* ws, size_t ws_bytes,
                    bool block, bool check_ws = true) {
  if (M < 0 || N < 0 || K <= 0 || (K % 128) != 0) return FP8DQ_ERR_SHAPE;
  if (block && (N % 128) != 0) return FP8DQ_ERR_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return FP8DQ_ERR_SHAPE;
  if (!known_flags(flags)) return FP8DQ_ERR_FLAGS;
  // the prefill and whole-line decode kernels address the weight operand
  // with 32-bit byte offsets (N * K < 2^32), and the prefill path runs X in
  // blocks of whole 256-row tiles that fit them; K is at most
  // FP8DQ_MAX_K, the range over which the accumulation error is validated
  // (and the block kernel keeps a tile's weight-block scales in LDS)
  if (N * K >= (int64_t(1) << 32) || K > FP8DQ_MAX_K) return FP8DQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8DQ_OK;
  if (!qx || !sx || !qw || !sw || !y) return FP8DQ_ERR_NULL;
  if (!aligned16(qx) || !aligned16(sx) || !aligned16(qw) || !aligned16(sw) ||
      !aligned16(y))
    return FP8DQ_ERR_ALIGN;
  const size_t need = check_ws ? gemm_ws_bytes(M, N, K, flags) : 0;
  if (need > 0) {
    if (!ws) return FP8DQ_ERR_NULL;
    if (!aligned16(ws)) return FP8DQ_ERR_ALIGN;
    if (ws_bytes < need) return FP8DQ_ERR_WORKSPACE;
  }
  return FP8DQ_OK;
}

// Launch a validated GEMM (M, N > 0).
// ws_cap: the workspace the decode plans may use (the caller's workspace was
// checked against the uncapped need; the no-allocation entry point caps the
// plans at its static scratch).
int run_gemm(const uint8_t* qx, const float* sx, const uint8_t* qw,
             const float* sw, void* y, int64_t M, int64_t N, int64_t K,
             uint32_t flags, void* ws, bool block, hipStream_t st,
             size_t ws_cap = SIZE_MAX) {
  if (!use_decode(M, flags)) {
    // The prefill kernels address an operand with 32-bit byte offsets: run
    // row blocks of X small enough for that (W itself must stay below 4 GiB,
    // checked with the arguments).
    const int64_t G = K / 128;
    int64_t rows_max = ((int64_t(1) << 32) - 1) / K;
    rows_max -= rows_max % 256;
    if (rows_max <= 0) return FP8DQ_ERR_SHAPE;   // excluded by the size rules
    for (int64_t m0 = 0; m0 < M; m0 += rows_max) {
      const int64_t rows = (M - m0) < rows_max ? (M - m0) : rows_max;
      fp8dq::launch_gemm_prefill(qx + m0 * K, sx + (block ? m0 * G : m0), qw, sw,
                                 static_cast<uint16_t*>(y) + m0 * N, rows, N, K, block, st);
      const int s = launch_status();
      if (s != FP8DQ_OK) return s;
    }
    return FP8DQ_OK;
  }
  const int64_t G = K / 128;
  for (int64_t m0 = 0; m0 < M; m0 += FP8DQ_DECODE_MAX_M) {
    const int64_t rows = (M - m0) < FP8DQ_DECODE_MAX_M ? (M - m0) : FP8DQ_DECODE_MAX_M;
    const DecodePlan p = fp8dq::plan_decode(rows, N, K, ws_cap);
    const float* sxs = sx + (block ? m0 * G : m0);
    fp8dq::launch_gemm_decode(qx + m0 * K, sxs, qw, sw,
                              static_cast<uint16_t*>(y) + m0 * N, ws, rows, N, K,
                              block, p, st);
    const int s = launch_status();
    if (s != FP8DQ_OK) return s;
  }
  return FP8DQ_OK;
}

}  // namespace

extern "C" {

int fp8_quant_act(const void* x_bf16, int64_t rows, int64_t K, int32_t group,
                  uint8_t* q, float* scale, void* stream) {
  if (group != 0 && group != 128) return FP8DQ_ERR_FLAGS;
  if (rows < 0 || K <= 0 || (K % (group ? 128 : 8)) != 0) return FP8DQ_ERR_SHAPE;
  if (rows > INT32_MAX || K > INT32_MAX) return FP8DQ_ERR_SHAPE;
  if (rows == 0) return FP8DQ_OK;
  if (!x_bf16 || !q || !scale) return FP8DQ_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(q) || !aligned16(scale)) return FP8DQ_ERR_ALIGN;
  if (group == 0)
    fp8dq::launch_quant_rows(x_bf16, rows, K, q, scale, as_stream(stream));
  else
    fp8dq::launch_quant_groups(x_bf16, rows, K, q, scale, as_stream(stream));
  return launch_status();
}

int fp8_quant_weight_block(const void* w_bf16, int64_t N, int64_t K, uint8_t* qw,
                           float* sw, void* stream) {
  if (N < 0 || K <= 0 || (N % 128) != 0 || (K % 128) != 0) return FP8DQ_ERR_SHAPE;
  if (N > INT32_MAX || K > INT32_MAX) return FP8DQ_ERR_SHAPE;
  if (N == 0) return FP8DQ_OK;
  if (!w_bf16 || !qw || !sw) return FP8DQ_ERR_NULL;
  if (!aligned16(w_bf16) || !aligned16(qw) || !aligned16(sw)) return FP8DQ_ERR_ALIGN;
  fp8dq::launch_quant_wblock(w_bf16, N, K, qw, sw, as_stream(stream));
  return launch_status();
}

int fp8_gemm(const uint8_t* qx, const float* sx, const uint8_t* qw,
             const float* sw, void* y_bf16, int64_t M, int64_t N, int64_t K,
             uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  int s = check_gemm_args(qx, sx, qw, sw, y_bf16, M, N, K, flags, ws, ws_bytes, false);
  if (s != FP8DQ_OK || M == 0 || N == 0) return s;
  return run_gemm(qx, sx, qw, sw, y_bf16, M, N, K, flags, ws, false, as_stream(stream));
}

int fp8_gemm_block(const uint8_t* qx, const float* sx, const uint8_t* qw,
                   const float* sw, void* y_bf16, int64_t M, int64_t N,
                   int64_t K, uint32_t flags, void* ws, size_t ws_bytes,
                   void* stream) {
  int s = check_gemm_args(qx, sx, qw, sw, y_bf16, M, N, K, flags, ws, ws_bytes, true);
  if (s != FP8DQ_OK || M == 0 || N == 0) return s;
  return run_gemm(qx, sx, qw, sw, y_bf16, M, N, K, flags, ws, true, as_stream(stream));
}

static int linear_common(const void* x_bf16, const uint8_t* qw, const float* sw,
                         void* y_bf16, int64_t M, int64_t N, int64_t K,
                         uint8_t* qx_out, float* sx_out, uint32_t flags, void* ws,
                         size_t ws_bytes, void* stream, bool block) {
  int s = check_gemm_args(qx_out, sx_out, qw, sw, y_bf16, M, N, K, flags, ws,
                          ws_bytes, block);
  if (s != FP8DQ_OK || M == 0 || N == 0) return s;
  if (!x_bf16) return FP8DQ_ERR_NULL;
  if (!aligned16(x_bf16)) return FP8DQ_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  if (block) fp8dq::launch_quant_groups(x_bf16, M, K, qx_out, sx_out, st);
  else fp8dq::launch_quant_rows(x_bf16, M, K, qx_out, sx_out, st);
  s = launch_status();
  if (s != FP8DQ_OK) return s;
  return run_gemm(qx_out, sx_out, qw, sw, y_bf16, M, N, K, flags, ws, block, st);
}

int fp8_linear(const void* x_bf16, const uint8_t* qw, const float* sw,
               void* y_bf16, int64_t M, int64_t N, int64_t K, uint8_t* qx_out,
               float* sx_out, uint32_t flags, void* ws, size_t ws_bytes,
               void* stream) {
  return linear_common(x_bf16, qw, sw, y_bf16, M, N, K, qx_out, sx_out, flags,
                       ws, ws_bytes, stream, false);
}

int fp8_linear_noalloc(const void* x_bf16, const uint8_t* qw, const float* sw,
                       void* y_bf16, int64_t M, int64_t N, int64_t K,
                       uint8_t* qx_out, float* sx_out, uint32_t flags, void* stream) {
  int s = check_gemm_args(qx_out, sx_out, qw, sw, y_bf16, M, N, K, flags, nullptr, 0,
                          false, /*check_ws=*/false);
  if (s != FP8DQ_OK || M == 0 || N == 0) return s;
  if (!x_bf16) return FP8DQ_ERR_NULL;
  if (!aligned16(x_bf16)) return FP8DQ_ERR_ALIGN;
  // the decode plans are capped at the static scratch, so the need never
  // exceeds it; checked all the same before anything is enqueued
  const size_t need = gemm_ws_bytes(M, N, K, flags, fp8dq::kScratchBytes);
  if (need > fp8dq::kScratchBytes) return FP8DQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = fp8dq::scratch_for_current_device();
    if (!ws) return FP8DQ_ERR_HIP;
  }
  hipStream_t st = as_stream(stream);
  fp8dq::launch_quant_rows(x_bf16, M, K, qx_out, sx_out, st);
  s = launch_status();
  if (s != FP8DQ_OK) return s;
  return run_gemm(qx_out, sx_out, qw, sw, y_bf16, M, N, K, flags, ws, false, st,
                  fp8dq::kScratchBytes);
}

int fp8_linear_block(const void* x_bf16, const uint8_t* qw, const float* sw,
                     void* y_bf16, int64_t M, int64_t N, int64_t K,
                     uint8_t* qx_out, float* sx_out, uint32_t flags, void* ws,
                     size_t ws_bytes, void* stream) {
  return linear_common(x_bf16, qw, sw, y_bf16, M, N, K, qx_out, sx_out, flags,
                       ws, ws_bytes, stream, true);
}

// ---- fused producers, static calibration, KV cache ------------------------
static constexpr int64_t kMaxFusedRow = 65536;  // values per row of the row kernels

int fp8_silu_mul_quant(const void* gu_bf16, int64_t rows, int64_t I, uint8_t* q,
                       float* scale, void* stream) {
  if (rows < 0 || I <= 0 || (I % 8) != 0 || I > kMaxFusedRow) return FP8DQ_ERR_SHAPE;
  if (rows > INT32_MAX) return FP8DQ_ERR_SHAPE;
  if (rows == 0) return FP8DQ_OK;
  if (!gu_bf16 || !q || !scale) return FP8DQ_ERR_NULL;
  if (!aligned16(gu_bf16) || !aligned16(q) || !aligned16(scale)) return FP8DQ_ERR_ALIGN;
  if (fp8dq::launch_silu_mul_quant(gu_bf16, rows, I, q, scale, as_stream(stream)) != 0)
    return FP8DQ_ERR_SHAPE;
  return launch_status();
}

int fp8_rmsnorm_quant(const void* x_bf16, const void* gamma_bf16, int64_t rows, int64_t H,
                      double eps, uint8_t* q, float* scale, void* stream) {
  if (rows < 0 || H <= 0 || (H % 8) != 0 || H > kMaxFusedRow) return FP8DQ_ERR_SHAPE;
  if (rows > INT32_MAX) return FP8DQ_ERR_SHAPE;
  // eps in [1e-30, 1e30] (NaN fails too): 1 / sqrt(mean + eps) then stays
  // below 1e15, inside fp32's range, whatever the row
  if (!(eps >= 1.0e-30) || eps > 1.0e30) return FP8DQ_ERR_SHAPE;
  if (rows == 0) return FP8DQ_OK;
  if (!x_bf16 || !gamma_bf16 || !q || !scale) return FP8DQ_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(gamma_bf16) || !aligned16(q) || !aligned16(scale))
    return FP8DQ_ERR_ALIGN;
  if (fp8dq::launch_rmsnorm_quant(x_bf16, gamma_bf16, rows, H, eps, q, scale,
                                  as_stream(stream)) != 0)
    return FP8DQ_ERR_SHAPE;
  return launch_status();
}

int fp8_silu_mul(const void* gu_bf16, int64_t rows, int64_t I, void* h_bf16, void* stream) {
  if (rows < 0 || I <= 0 || (I % 8) != 0 || I > kMaxFusedRow) return FP8DQ_ERR_SHAPE;
  if (rows > INT32_MAX) return FP8DQ_ERR_SHAPE;
  if (rows == 0) return FP8DQ_OK;
  if (!gu_bf16 || !h_bf16) return FP8DQ_ERR_NULL;
  if (!aligned16(gu_bf16) || !aligned16(h_bf16)) return FP8DQ_ERR_ALIGN;
  if (fp8dq::launch_silu_mul(gu_bf16, rows, I, h_bf16, as_stream(stream)) != 0)
    return FP8DQ_ERR_SHAPE;
  return launch_status();
}

int fp8_rmsnorm(const void* x_bf16, const void* gamma_bf16, int64_t rows, int64_t H, double eps,
                void* h_bf16, void* stream) {
  if (rows < 0 || H <= 0 || (H % 8) != 0 || H > kMaxFusedRow) return FP8DQ_ERR_SHAPE;
  if (rows > INT32_MAX) return FP8DQ_ERR_SHAPE;
  if (!(eps >= 1.0e-30) || eps > 1.0e30) return FP8DQ_ERR_SHAPE;   // as fp8_rmsnorm_quant
  if (rows == 0) return FP8DQ_OK;
  if (!x_bf16 || !gamma_bf16 || !h_bf16) return FP8DQ_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(gamma_bf16) || !aligned16(h_bf16)) return FP8DQ_ERR_ALIGN;
  if (fp8dq::launch_rmsnorm(x_bf16, gamma_bf16, rows, H, eps, h_bf16, as_stream(stream)) != 0)
    return FP8DQ_ERR_SHAPE;
  return launch_status();
}

size_t fp8_calib_workspace_bytes(int64_t n) {
  return n < 0 ? 0 : fp8dq::calib_workspace_bytes();
}

int fp8_calib_scale(const void* x_bf16, int64_t n, int32_t lo_permille, int32_t hi_permille,
                    float* scale_out, void* ws, size_t ws_bytes, void* stream) {
  if (n < 0 || (n % 8) != 0 || n >= (int64_t(1) << 40)) return FP8DQ_ERR_SHAPE;
  if (lo_permille < 0 || hi_permille > 1000 || lo_permille > hi_permille)
    return FP8DQ_ERR_SHAPE;
  if ((n > 0 && !x_bf16) || !scale_out || !ws) return FP8DQ_ERR_NULL;
  if ((n > 0 && !aligned16(x_bf16)) || !aligned16(ws)) return FP8DQ_ERR_ALIGN;
  if (ws_bytes < fp8dq::calib_workspace_bytes()) return FP8DQ_ERR_WORKSPACE;
  // nearest-rank order statistics: k = ceil(p * n), kept in [1, n]
  auto rank = [n](int64_t pm) {
    int64_t k = (pm * n + 999) / 1000;
    if (k < 1) k = 1;
    if (k > n) k = n;
    return n == 0 ? int64_t(0) : k;
  };
  fp8dq::launch_calib_scale(x_bf16, n, rank(lo_permille), rank(hi_permille), scale_out, ws,
                            as_stream(stream));
  return launch_status();
}

int fp8_quant_static(const void* x_bf16, int64_t n, const float* scale, uint8_t* q,
                     void* stream) {
  if (n < 0 || (n % 8) != 0) return FP8DQ_ERR_SHAPE;
  if (n == 0) return FP8DQ_OK;
  if (!x_bf16 || !scale || !q) return FP8DQ_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(q) || (reinterpret_cast<uintptr_t>(scale) & 3u))
    return FP8DQ_ERR_ALIGN;
  fp8dq::launch_quant_static(x_bf16, n, scale, q, as_stream(stream));
  return launch_status();
}

int fp8_kv_cache_quant(const void* k_bf16, const void* v_bf16, int64_t T, int64_t width,
                       const int64_t* slots, int64_t n_slots, uint8_t* k_cache,
                       uint8_t* v_cache, float* k_scale, float* v_scale, void* stream) {
  if (T < 0 || width <= 0 || (width % 8) != 0 || width > kMaxFusedRow || n_slots < 0)
    return FP8DQ_ERR_SHAPE;
  if (T > INT32_MAX) return FP8DQ_ERR_SHAPE;
  if (T == 0) return FP8DQ_OK;
  if (!k_bf16 || !v_bf16 || !slots || !k_cache || !v_cache || !k_scale || !v_scale)
    return FP8DQ_ERR_NULL;
  if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(k_cache) ||
      !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(slots) & 7u) ||
      (reinterpret_cast<uintptr_t>(k_scale) & 3u) || (reinterpret_cast<uintptr_t>(v_scale) & 3u))
    return FP8DQ_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  if (fp8dq::launch_kv_quant(k_bf16, v_bf16, T, width, slots, n_slots, k_cache, v_cache,
                             k_scale, v_scale, st) != 0)
    return FP8DQ_ERR_SHAPE;
  return launch_status();
}

size_t fp8_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t block,
                           uint32_t flags) {
  if (!known_flags(flags)) return 0;
  if (block && (N % 128) != 0) return 0;
  return gemm_ws_bytes(M, N, K, flags);
}

const char* fp8_status_string(int status) {
  switch (status) {
    case FP8DQ_OK: return "ok";
    case FP8DQ_ERR_NULL: return "null pointer";
    case FP8DQ_ERR_SHAPE: return "bad shape";
    case FP8DQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FP8DQ_ERR_WORKSPACE: return "workspace too small";
    case FP8DQ_ERR_FLAGS: return "unsupported flags or group";
    case FP8DQ_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* fp8dq_version(void) { return "0.1.0"; }

}  // extern "C"
