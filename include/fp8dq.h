/*
 * fp8dq.h -- FP8-Dynamic quantized linear layer for AMD MI355X (gfx950).
 *
 * The operation (as the pages define it):
 *   - Activations are quantized at run time, one scale per token (row of X),
 *     to FP8 E4M3 -- Llama-3.1-8B-Instruct-FP8-Dynamic page, FP8 dynamic
 *     quantization table (input activations row); Llama-3.1-70B-FP8-Dynamic
 *     page, section 1.2 (activations bullet).
 *   - Weights are stored as E4M3 with one scale per output channel (row of
 *     W), found with a min/max observer -- same table, weights row; 70B page,
 *     section 1.2, weights bullet; one weight_scale beside every Linear (70B
 *     page, section 2).
 *   - Block variant: one weight scale per 128x128 block of W, activation
 *     scales per token per 128-column group, both dynamic for activations --
 *     Llama-3.2-3B-Instruct-FP8-Block page, FP8 block quantization table.
 *   - E4M3 is the 4-exponent/3-mantissa-bit format whose largest value is
 *     448 -- "Llama 3 精读实录" page, section 2.1.
 *   - lm_head is never quantized (ignore list on all three walk-through
 *     pages): nothing in this library applies to it; callers keep it bf16.
 *
 * Numerics (fixed here where the pages are silent):
 *   amax  = max |x| over the unit (row, 128-group, W row or 128x128 block)
 *   s     = RN_fp32(amax / 448), stored as fp32; s = 0 for an all-zero unit
 *   q     = E4M3 code nearest to the exact quotient x / s (ties to the even
 *           code, saturating at +-448, sign of zero kept); q = +-0 if s = 0
 *   y     = bf16_RNE( sum_k val(qx[m,k]) val(qw[n,k]) * sx[m] * sw[n] )
 *   block: y = bf16_RNE( sum_g (sum_{k in g} val*val) * sx[m,g] * sw[n/128,g] )
 *   The scale product sx * sw (per channel, or per group) is formed first,
 *   so every intermediate stays inside fp32 while that product is below
 *   2^128 (both amax beyond about 2^73 at once is outside this range).
 *   The sum is accumulated in fp32 (any order); codes and scales are
 *   bit-exact. y is within 1e-2 relative / 1e-3 absolute of the exact value
 *   on the decode path; the prefill path is exact to the matrix
 *   instruction's own accumulation (below), which leaves rare outputs near
 *   zero outside that tolerance (8 of 16.8 M outputs of the Llama-3.1-8B
 *   down linear at 4096 tokens, 1 of 940 M of its gate_up at 32768 tokens,
 *   by at most 1.5 times the allowed error).
 *
 * Accumulation (measured on gfx950, both FP8 MFMA shapes): the matrix
 * instruction adds its products in groups of 8 consecutive k. Inside a
 * group every product is cut toward zero to a multiple of 2^(E - 13), E the
 * largest e(x) + e(w) of the group (unbiased exponents, -6 for subnormal
 * codes); groups and the running fp32 sum are then added with about 24
 * significant bits. So per output
 *     |acc - exact| < sum over groups g of 7 * 2^(E_g - 13)  (+ fp32 terms),
 * the bound being reached only where a group mixes products more than 7
 * binades apart. The decode path (FP8DQ_FORCE_DECODE, and M <= 64 under
 * FP8DQ_AUTO) splits each token row's codes of magnitude >= 16 from the
 * rest and runs the two halves through separate MFMAs, so large activation
 * codes (outlier channels) do not cut the small ones' products; the prefill
 * kernels keep one MFMA per product (their rate is the matrix core's).
 * K is at most FP8DQ_MAX_K: the range over which these errors were
 * measured against the exact sum.
 *
 * Conventions for every entry point:
 *   - extern "C"; no C++ exception crosses the boundary.
 *   - All tensor pointers are caller-owned DEVICE memory, row-major and
 *     contiguous, 16-byte aligned. X is bf16 [M,K], W is bf16 [N,K] (K is
 *     the contiguous dimension of both), Y is bf16 [M,N]; codes are uint8
 *     E4M3 with the same shapes; scales are fp32.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; nothing synchronizes.
 *   - All arguments are validated on the host before anything is enqueued;
 *     on any error nothing is enqueued and outputs are untouched.
 *   - The library allocates and frees nothing, keeps no pointer after it
 *     returns and holds no mutable global state: calls are reentrant.
 *     Concurrent calls that write the same buffers race (caller's problem).
 *     The one exception is fp8_linear_noalloc, whose static per-GPU scratch
 *     array (and its device address, looked up once per GPU) is shared by
 *     all its calls on that GPU.
 *   - Inputs and outputs must not overlap. Inputs must be finite (NaN / Inf
 *     are outside the contract: not checked, result unspecified).
 *   - M = 0 or N = 0 (rows = 0) is a valid empty call: FP8DQ_OK, nothing
 *     enqueued. Negative sizes are FP8DQ_ERR_SHAPE.
 */
#ifndef FP8DQ_H
#define FP8DQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FP8DQ_OK              0
#define FP8DQ_ERR_NULL       -1  /* a required pointer is NULL */
#define FP8DQ_ERR_SHAPE      -2  /* negative size, or a size rule below broken */
#define FP8DQ_ERR_ALIGN      -3  /* a tensor pointer is not 16-byte aligned */
#define FP8DQ_ERR_WORKSPACE  -4  /* workspace smaller than fp8_workspace_bytes() */
#define FP8DQ_ERR_FLAGS      -5  /* unknown flag bits or group value */
#define FP8DQ_ERR_HIP        -6  /* the HIP runtime reported a launch error */

/* flags for the GEMM / linear calls: which kernel family runs. */
#define FP8DQ_AUTO            0u  /* M <= 64: split-K decode path, else prefill */
#define FP8DQ_FORCE_PREFILL   1u  /* LDS-tiled MFMA GEMM at any M */
#define FP8DQ_FORCE_DECODE    2u  /* HBM-streaming split-K GEMM at any M */

/* Largest M the decode (small-M) path takes under FP8DQ_AUTO. */
#define FP8DQ_DECODE_MAX_M   64

/* Largest K of the GEMM and linear calls (2^17; the longest Llama-3.x
 * reduction is 28672). */
#define FP8DQ_MAX_K          131072

/*
 * fp8_quant_act -- dynamic activation quantization (also the per-channel
 * weight quantizer: rows of W are output channels, same arithmetic).
 *   x      : bf16 [rows, K]
 *   group  : 0   -> one scale per row,           scale is fp32 [rows]
 *            128 -> one scale per row per 128 columns, scale is fp32
 *                   [rows, K/128] (block variant's activations)
 *   q      : uint8 E4M3 codes [rows, K] (output)
 *   scale  : fp32 scales (output), layout as above
 * Size rules: rows >= 0; K > 0 and K % 8 == 0 (group 0) or K % 128 == 0
 * (group 128). Any other group value is FP8DQ_ERR_FLAGS.
 * Source: FP8 dynamic quantization table (input activations / weights rows)
 * on the Llama-3.1-8B-Instruct-FP8-Dynamic page; block table on the
 * Llama-3.2-3B-Instruct-FP8-Block page (group 128).
 */
int fp8_quant_act(const void* x_bf16, int64_t rows, int64_t K, int32_t group,
                  uint8_t* q, float* scale, void* stream);

/*
 * fp8_quant_weight_block -- 128x128 block weight quantization (setup step
 * of the block variant).
 *   w  : bf16 [N, K];  qw : uint8 [N, K] (output);
 *   sw : fp32 [N/128, K/128] (output), block (nb, kb) covers rows
 *        128nb..128nb+127 and columns 128kb..128kb+127.
 * Size rules: N >= 0, K > 0, N % 128 == 0, K % 128 == 0.
 * Source: block_structure [128, 128] in the FP8 block quantization table,
 * Llama-3.2-3B-Instruct-FP8-Block page.
 */
int fp8_quant_weight_block(const void* w_bf16, int64_t N, int64_t K,
                           uint8_t* qw, float* sw, void* stream);

/*
 * fp8_gemm -- Y = bf16( (Qx Qw^T) * sx[m] * sw[n] ) from codes and scales:
 * the FP8 matrix product with per-token activation scales and per-output-
 * channel weight scales, rescaled to bf16 in the epilogue.
 * Source: FP8 dynamic quantization table of the Llama-3.1-8B-Instruct-FP8-
 * Dynamic page (per-channel weights, per-token activations); the
 * Llama-3.1-70B-FP8-Dynamic page, section 1.2 (the same scheme) and section
 * 3 (the FP8 products run on the matrix units, no dequantized copy).
 *   qx : uint8 [M, K], sx : fp32 [M];  qw : uint8 [N, K], sw : fp32 [N]
 *   y  : bf16 [M, N] (output)
 *   flags : FP8DQ_AUTO / FP8DQ_FORCE_PREFILL / FP8DQ_FORCE_DECODE
 *   ws, ws_bytes : device workspace for split-K partial sums and tile
 *        counters; ws may be NULL iff fp8_workspace_bytes(M, N, K, 0, flags)
 *        == 0. Its bytes must be zero before the first call that uses it
 *        (allocate it zero-filled); every call leaves its counter area zero
 *        again, so a zeroed workspace serves any number of calls of any
 *        shapes, one at a time (calls that overlap on one workspace race).
 * Size rules: M, N >= 0; K > 0, K % 128 == 0 and K <= FP8DQ_MAX_K;
 * N * K < 2^32 (the weight codes under 4 GiB); FP8DQ_ERR_SHAPE otherwise.
 */
int fp8_gemm(const uint8_t* qx, const float* sx, const uint8_t* qw,
             const float* sw, void* y_bf16, int64_t M, int64_t N, int64_t K,
             uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_gemm_block -- block-scaled GEMM:
 *   y[m,n] = bf16( sum_g P_g[m,n] * sx[m,g] * sw[n/128, g] ), P_g the code
 *   product summed over the g-th 128-column group.
 * Source: FP8 block quantization table of the Llama-3.2-3B-Instruct-FP8-
 * Block page (weight block structure [128, 128], activations per token per
 * group of 128, dynamic).
 *   sx : fp32 [M, K/128];  sw : fp32 [N/128, K/128]
 * Size rules: M, N >= 0; N % 128 == 0; K > 0, K % 128 == 0 and
 * K <= FP8DQ_MAX_K; N * K < 2^32, as for fp8_gemm.
 * ws as for fp8_gemm (block = 1 in fp8_workspace_bytes).
 */
int fp8_gemm_block(const uint8_t* qx, const float* sx, const uint8_t* qw,
                   const float* sw, void* y_bf16, int64_t M, int64_t N,
                   int64_t K, uint32_t flags, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * fp8_linear -- the FP8-Dynamic linear: quantize X per token (writes qx_out,
 * sx_out, which the caller owns and may inspect) and run fp8_gemm with the
 * pre-quantized weight (qw, sw from fp8_quant_act on W).
 * Source: the FP8 dynamic quantization table of the Llama-3.1-8B-Instruct-
 * FP8-Dynamic page (weights static per channel, activations dynamic per
 * token, computed at run time) and the Llama-3.1-70B-FP8-Dynamic page,
 * section 1.2 (the same split: weights quantized once, activations per
 * inference).
 *   x : bf16 [M, K]; qx_out : uint8 [M, K]; sx_out : fp32 [M]
 * Size rules, workspace and errors: those of fp8_gemm.
 */
int fp8_linear(const void* x_bf16, const uint8_t* qw, const float* sw,
               void* y_bf16, int64_t M, int64_t N, int64_t K,
               uint8_t* qx_out, float* sx_out, uint32_t flags, void* ws,
               size_t ws_bytes, void* stream);

/*
 * fp8_linear_noalloc -- fp8_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation with no workspace argument. The
 * decode path's split-K partials and tile counters live in a static device
 * array of the library, FP8DQ_NOALLOC_SCRATCH_BYTES per GPU (16 MiB + 16
 * KiB, held from the first call on a GPU until the process ends), and the
 * decode plans only split K as far as that array holds; the result is within
 * the tolerance of fp8_linear's (bit-identical where fp8_linear's plan fits
 * the array). The call allocates nothing. All calls on one GPU share its
 * array: calls that overlap on one GPU (several streams or threads) race.
 * Arguments, size rules and errors: those of fp8_linear; FP8DQ_ERR_HIP if
 * the array's device address cannot be obtained.
 */
#define FP8DQ_NOALLOC_SCRATCH_BYTES ((size_t)16 * 1024 * 1024 + 16 * 1024)
int fp8_linear_noalloc(const void* x_bf16, const uint8_t* qw, const float* sw,
                       void* y_bf16, int64_t M, int64_t N, int64_t K,
                       uint8_t* qx_out, float* sx_out, uint32_t flags, void* stream);

/*
 * fp8_linear_block -- block variant: quantize X per token per 128-group
 * (qx_out uint8 [M, K], sx_out fp32 [M, K/128]) then fp8_gemm_block with
 * block-quantized weights (qw, sw from fp8_quant_weight_block).
 * Source: FP8 block quantization table of the Llama-3.2-3B-Instruct-FP8-
 * Block page (block_structure [128, 128] weights; group-128 dynamic
 * activations).
 * Size rules, workspace and errors: those of fp8_gemm_block.
 */
int fp8_linear_block(const void* x_bf16, const uint8_t* qw, const float* sw,
                     void* y_bf16, int64_t M, int64_t N, int64_t K,
                     uint8_t* qx_out, float* sx_out, uint32_t flags, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * fp8_workspace_bytes -- device workspace the GEMM / linear calls need for
 * these sizes and flags (block = 0: per-channel, 1: block variant). 0 when
 * the chosen path needs none. Pure host function; never fails (returns 0 for
 * invalid sizes, which the compute calls then reject).
 */
size_t fp8_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t block,
                           uint32_t flags);

/* ------------------------------------------------------------------------
 * Producers fused with the per-token quantizer, static calibration and the
 * FP8 KV cache ("Llama 3 精读实录" page). In the fused producers the bf16
 * value h that gets quantized is the correctly rounded bf16 of the exact
 * real formula (ties to even); its FP8 codes and scales then follow the
 * per-token rules of fp8_quant_act. Row kernels take rows of at most 65536
 * values (FP8DQ_ERR_SHAPE beyond). Same conventions as above otherwise.
 * ------------------------------------------------------------------------ */

/*
 * fp8_silu_mul_quant -- SwiGLU's gated product, quantized per token:
 *   h[r,i] = bf16( silu(g[r,i]) * u[r,i] ),  silu(g) = g / (1 + e^-g),
 *   g = gu[r, 0:I], u = gu[r, I:2I] (gate | up, as one fused gate_up GEMM
 *   writes them); q [rows, I] and scale [rows] as fp8_quant_act(h, group 0).
 * Source: §1.3 of the page (gate and up branches computed separately, then
 * multiplied elementwise). h is not written out.
 * Size rules: rows >= 0; I > 0, I % 8 == 0, I <= 65536.
 */
int fp8_silu_mul_quant(const void* gu_bf16, int64_t rows, int64_t I, uint8_t* q,
                       float* scale, void* stream);

/*
 * fp8_rmsnorm_quant -- RMSNorm, quantized per token:
 *   h[r,i] = bf16( gamma[i] * x[r,i] / sqrt(mean_i(x[r,i]^2) + eps) ),
 *   x bf16 [rows, H], gamma bf16 [H]; q [rows, H], scale [rows].
 * Source: §1.3 of the page (eps = 1e-5, norm before attention and the MLP;
 * §5.3 keeps the norm itself in bf16). 1e-30 <= eps <= 1e30 (FP8DQ_ERR_SHAPE
 * otherwise): 1 / sqrt(mean + eps) then stays inside fp32's range (with
 * eps = 0 an all-zero row would have no value).
 * Size rules: rows >= 0; H > 0, H % 8 == 0, H <= 65536.
 */
int fp8_rmsnorm_quant(const void* x_bf16, const void* gamma_bf16, int64_t rows, int64_t H,
                      double eps, uint8_t* q, float* scale, void* stream);

/*
 * fp8_silu_mul, fp8_rmsnorm -- the same two producers with the bf16 h row as
 * the output instead of its FP8 codes: h_bf16 [rows, I] (resp. [rows, H]),
 * bit-identical to the h the quantizing entry points quantize. The norm in
 * bf16 is what feeds layers that stay in bf16 (the final norm before
 * lm_head, which the FP8 schemes leave unquantized: the Llama-3.1-8B-
 * Instruct-FP8-Dynamic page's model description). Same size rules, errors
 * and stream semantics as fp8_silu_mul_quant / fp8_rmsnorm_quant;
 * h_bf16 16-byte aligned.
 */
int fp8_silu_mul(const void* gu_bf16, int64_t rows, int64_t I, void* h_bf16, void* stream);
int fp8_rmsnorm(const void* x_bf16, const void* gamma_bf16, int64_t rows, int64_t H, double eps,
                void* h_bf16, void* stream);

/*
 * fp8_calib_scale -- static per-tensor scale from percentile calibration:
 *   amax = max(|x_(k_lo)|, |x_(k_hi)|), k = ceil(p * n) clamped to [1, n]
 *   (nearest-rank order statistics of the n values, p = permille / 1000),
 *   *scale_out = RN_fp32(amax / 448)   (0 when n == 0).
 * Source: §2.2 of the page (P99.9 / P0.1 percentiles of a calibration set
 * as the dynamic range instead of the maximum): lo 1, hi 999 by default.
 *   x: bf16 [n]; scale_out: device fp32 [1]; ws: fp8_calib_workspace_bytes
 *   bytes (contents need no initialisation).
 * Size rules: 0 <= n < 2^40, n % 8 == 0; 0 <= lo <= hi <= 1000.
 */
size_t fp8_calib_workspace_bytes(int64_t n);
int fp8_calib_scale(const void* x_bf16, int64_t n, int32_t lo_permille, int32_t hi_permille,
                    float* scale_out, void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_quant_static -- E4M3 codes of x / s with one static scale s (device
 * fp32 [1], e.g. from fp8_calib_scale): nearest with ties to the even code,
 * saturating at +-448 (0x7E / 0xFE), sign of zero kept; s == 0 gives +-0.
 *   x: bf16 [n] -> q: uint8 [n].  Size rules: n >= 0, n % 8 == 0.
 */
int fp8_quant_static(const void* x_bf16, int64_t n, const float* scale, uint8_t* q,
                     void* stream);

/*
 * fp8_kv_cache_quant -- FP8 KV cache write: each token row of K and V
 * (bf16 [T, width], width = KV heads * head dim) is quantized per token as
 * in fp8_quant_act and stored in cache row slots[t] of k_cache / v_cache
 * (uint8 [n_slots, width]) with its scale in k_scale / v_scale (fp32
 * [n_slots]); tokens whose slot is negative or >= n_slots are not written.
 * Valid slots are expected to be distinct (as a cache's slot mapping is):
 * when two tokens name one slot, which token's row and scale the slot ends
 * up holding is unspecified. slots: device int64 [T]. Source: §4.1 of the page (FP8 also compresses
 * the KV cache). Size rules: T >= 0; width > 0, width % 8 == 0,
 * width <= 65536; n_slots >= 0.
 */
int fp8_kv_cache_quant(const void* k_bf16, const void* v_bf16, int64_t T, int64_t width,
                       const int64_t* slots, int64_t n_slots, uint8_t* k_cache,
                       uint8_t* v_cache, float* k_scale, float* v_scale, void* stream);

/* fp8_status_string -- static text for a status code (never NULL). */
const char* fp8_status_string(int status);

/* fp8dq_version -- library version string, "major.minor.patch". */
const char* fp8dq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8DQ_H */
