// Host-side launchers of the gfx950 kernels. Arguments are validated by the
// C-ABI layer (api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8dq {

// Dynamic quantization (quant.hip).
void launch_quant_rows(const void* x, int64_t rows, int64_t K, uint8_t* q,
                       float* scale, hipStream_t st);
void launch_quant_groups(const void* x, int64_t rows, int64_t K, uint8_t* q,
                         float* scale, hipStream_t st);
void launch_quant_wblock(const void* w, int64_t N, int64_t K, uint8_t* q,
                         float* scale, hipStream_t st);

// Prefill GEMM (gemm_prefill.hip): LDS-tiled MFMA, fused epilogue.
// block = false: per-channel scales sx[M], sw[N];
// block = true : sx[M, K/128], sw[N/128, K/128].
// Whole-line block-scaled prefill GEMM (gemm_block.hip); K >= 256,
// K <= 131072, 32-bit operand and scale offsets.
void launch_gemm_line_block(const uint8_t* qx, const float* sx, const uint8_t* qw,
                            const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                            hipStream_t st);
void launch_gemm_prefill(const uint8_t* qx, const float* sx, const uint8_t* qw,
                         const float* sw, void* y, int64_t M, int64_t N,
                         int64_t K, bool block, hipStream_t st);

// Decode GEMM (gemm_decode.hip): small-M, HBM-streaming, split-K with the
// reduction done by the last slice of each output tile.
struct DecodePlan {
  int mb;            // 16-row blocks of M covered (M <= 16 * mb)
  int splits;        // K slices across the grid (1: no partials)
  int kt_per_split;  // 128-wide K steps per slice
  int line;          // 1: whole-line kernel (LDS ring), 0: register-loading kernel
};
// Split workspaces: [tile counters: kDecodeCounterBytes][fp32 partials
// splits x M x N]. The counters must be zero before a call and every call
// leaves them zero; K is split only while a launch has at most
// kDecodeMaxSplitTiles output tiles, so the counter area never moves.
constexpr int64_t kDecodeMaxSplitTiles = 4096;
constexpr size_t kDecodeCounterBytes = (size_t)kDecodeMaxSplitTiles * 4;
// ws_cap: largest workspace the plan may use (split counts needing more are
// not considered; one slice needs none).
DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, size_t ws_cap = SIZE_MAX);
size_t decode_workspace_bytes(int64_t M, int64_t N, const DecodePlan& p);
void launch_gemm_decode(const uint8_t* qx, const float* sx, const uint8_t* qw,
                        const float* sw, void* y, void* ws, int64_t M,
                        int64_t N, int64_t K, bool block, const DecodePlan& p,
                        hipStream_t st);

// Fused producers, static calibration, KV cache (fused_quant.hip). The row
// launchers return -1 when a row is longer than 65536 values.
int launch_silu_mul_quant(const void* gu, int64_t rows, int64_t I, uint8_t* q,
                          float* scale, hipStream_t st);
int launch_rmsnorm_quant(const void* x, const void* gamma, int64_t rows, int64_t H,
                         double eps, uint8_t* q, float* scale, hipStream_t st);
int launch_silu_mul(const void* gu, int64_t rows, int64_t I, void* h, hipStream_t st);
int launch_rmsnorm(const void* x, const void* gamma, int64_t rows, int64_t H, double eps,
                   void* h, hipStream_t st);
int launch_kv_quant(const void* k, const void* v, int64_t T, int64_t width,
                    const int64_t* slots, int64_t n_slots, uint8_t* kc, uint8_t* vc,
                    float* ks, float* vs, hipStream_t st);
size_t calib_workspace_bytes();
void launch_calib_scale(const void* x, int64_t n, int64_t k_lo, int64_t k_hi,
                        float* scale_out, void* ws, hipStream_t st);
void launch_quant_static(const void* x, int64_t n, const float* scale, uint8_t* q,
                         hipStream_t st);

// Static device scratch of the no-allocation entry point (noalloc.hip):
// this device's copy of the array (its address from hipGetSymbolAddress,
// taken once per device) and its size; nullptr if the address could not be
// obtained.
constexpr size_t kScratchBytes = kDecodeCounterBytes + ((size_t)16 << 20);
void* scratch_for_current_device();

}  // namespace fp8dq
