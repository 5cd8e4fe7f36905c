// Dynamic FP8 (E4M3) quantization kernels for gfx950.
//
// What is computed (Llama-3.1-8B-Instruct-FP8-Dynamic page, FP8 dynamic
// quantization table; Llama-3.2-3B-Instruct-FP8-Block page, FP8 block
// quantization table; E4M3 limits from the "Llama 3 精读实录" page, §2.1):
//   per unit (a row, a 128-column group of a row, or a 128x128 block):
//     amax = max |x|;  s = RN_fp32(amax / 448);  q = E4M3_RNE(x / s)
// with the exact quotient x / s (s as stored), ties to the even code and the
// sign of zero kept; an all-zero unit has s = 0 and codes +-0.
//
// Design (HBM-bound: 2 bytes in, 1 byte + scales out per element):
//  * each lane owns 8-element (16-byte) chunks of the unit, loaded once and
//    kept in registers between the amax pass and the quantize pass;
//  * amax is an integer max over the bf16 bit patterns with the sign bit
//    cleared (exact for finite inputs), reduced across the wave with DPP
//    moves and permlane swaps (registers only) and across waves through LDS;
//  * the quotient is formed as y = x * RN(1/s) in fp32 and rounded by the
//    hardware fp32->E4M3 conversion (round to nearest even). y is within
//    2^-23 (relative) of x / s, so it can land on the wrong side of an E4M3
//    rounding midpoint only when it is within a couple of fp32 ulps of one.
//    Such lanes -- and lanes in the E4M3 subnormal range, where the midpoint
//    test below does not apply -- take an exact fix-up: the sign of
//    (midpoint * s - |x|) from one fused multiply-add decides the side (and
//    exactly zero means a tie, resolved to the even code). bf16 inputs make
//    exact ties common (a row whose amax has a short mantissa puts many x / s
//    exactly on midpoints), so the fix-up is inline and branch-free.
//  * exact quotients never exceed 448.9 for bf16 inputs (the scale rounding
//    moves them by at most a few parts per thousand, in the fp32-subnormal
//    scale range), so y stays below 464, where the hardware conversion still
//    rounds to 448; no clamp is needed.
//  * scales below 2^-64 are handled by scaling x and s by 2^64 (exact), which
//    keeps 1/s finite and the fix-up's product away from fp32 underflow.
#include "device_common.hpp"
#include "kernels.hpp"
#include "quant_codec.hpp"

namespace fp8dq {
namespace {

using namespace codec;

// ---------------------------------------------------------------------------
// Per-row quantization: one scale per row of [rows, K].
// A team of TEAM_WAVES waves owns a row; each lane holds CH chunks of the row
// in registers. Block = 256 threads (4 / TEAM_WAVES rows per block).
// SPLIT (few long rows): CH blocks per row (blockIdx.y), each loading the
// whole row for its amax but encoding and storing only its lanes' chunk y,
// so the encoding of one row runs on CH CUs (the extra reads of the row hit
// L2; the amax, a maximum, is the same in every block).
// ---------------------------------------------------------------------------
template <int CH, int TEAM_WAVES, bool SPLIT = false>
__global__ __launch_bounds__(TEAM_WAVES >= 4 ? 64 * TEAM_WAVES : 256) void quant_rows_kernel(
    const uint4* __restrict__ x, int64_t rows, int64_t K, uint2* __restrict__ q,
    float* __restrict__ scale) {
  constexpr int TEAM = 64 * TEAM_WAVES;
  constexpr int ROWS_PER_BLOCK = TEAM_WAVES >= 4 ? 1 : 4 / TEAM_WAVES;
  __shared__ uint32_t red[TEAM_WAVES >= 4 ? TEAM_WAVES : 4];
  const int tid = threadIdx.x;
  const int team = tid / TEAM;
  const int tl = tid % TEAM;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + team;
  const int64_t nch = K >> 3;  // chunks per row
  const bool row_ok = row < rows;
  const uint4* xr = x + (row_ok ? row : 0) * nch;

  uint4 v[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * TEAM + tl;
    v[i] = ld16_if<true>(xr, c, row_ok && c < nch);
  }
  us2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < CH; ++i) m2 = chunk_amax(v[i], m2);
  uint32_t m = m2.x > m2.y ? m2.x : m2.y;
  m = wave64_max(m);
  if (TEAM_WAVES > 1) {   // the team's waves meet in red[team * TEAM_WAVES ...]
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    const uint32_t* tr = red + team * TEAM_WAVES;
    m = tr[0];
#pragma unroll
    for (int w = 1; w < TEAM_WAVES; ++w) m = m > tr[w] ? m : tr[w];
  }
  if (!row_ok) return;
  float s, r, p;
  bool tiny;
  unit_scale(m, s, r, p, tiny);
  if (tl == 0 && (!SPLIT || blockIdx.y == 0)) scale[row] = s;
  uint2* qr = q + row * nch;
  if (!tiny) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t c = (int64_t)i * TEAM + tl;
      if (c < nch && (!SPLIT || i == (int)blockIdx.y)) qr[c] = quant8<false>(v[i], s, r, p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t c = (int64_t)i * TEAM + tl;
      if (c < nch && (!SPLIT || i == (int)blockIdx.y)) qr[c] = quant8<true>(v[i], s, r, p);
    }
  }
}

// Rows longer than the register-resident kernels take (K > 32768): two
// passes over the row, one block of 256 threads per row.
__global__ __launch_bounds__(256) void quant_rows_2pass_kernel(
    const uint4* __restrict__ x, int64_t rows, int64_t K, uint2* __restrict__ q,
    float* __restrict__ scale) {
  __shared__ uint32_t red[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t nch = K >> 3;
  const uint4* xr = x + row * nch;
  us2 m2 = {0, 0};
  for (int64_t c = tid; c < nch; c += 256) m2 = chunk_amax(xr[c], m2);
  uint32_t m = m2.x > m2.y ? m2.x : m2.y;
  m = wave64_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < 4; ++w) m = m > red[w] ? m : red[w];
  float s, r, p;
  bool tiny;
  unit_scale(m, s, r, p, tiny);
  if (tid == 0) scale[row] = s;
  uint2* qr = q + row * nch;
  for (int64_t c = tid; c < nch; c += 256)
    qr[c] = tiny ? quant8<true>(xr[c], s, r, p) : quant8<false>(xr[c], s, r, p);
}

// ---------------------------------------------------------------------------
// Group-128 quantization (block variant's activations): 16 lanes per group,
// one chunk each; each thread handles UNROLL chunks spaced by the block size.
// ---------------------------------------------------------------------------
template <int UNROLL>
__global__ __launch_bounds__(256) void quant_groups_kernel(
    const uint4* __restrict__ x, int64_t total_chunks, uint2* __restrict__ q,
    float* __restrict__ scale) {
  const int64_t base = (int64_t)blockIdx.x * 256 * UNROLL + threadIdx.x;
  uint4 v[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t c = base + (int64_t)u * 256;
    v[u] = c < total_chunks ? ld16_nt(x + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t c = base + (int64_t)u * 256;
    us2 m2 = chunk_amax(v[u], us2{0, 0});
    uint32_t m = m2.x > m2.y ? m2.x : m2.y;
    m = row16_max(m);
    float s, r, p;
    bool tiny;
    unit_scale(m, s, r, p, tiny);
    if (c < total_chunks) {
      if ((threadIdx.x & 15) == 0) scale[c >> 4] = s;
    }
    uint2 out;
    if (__builtin_expect(__any(tiny), 0)) {
      out = quant8<true>(v[u], s, r, p);
    } else {
      out = quant8<false>(v[u], s, r, p);
    }
    if (c < total_chunks) q[c] = out;
  }
}

// ---------------------------------------------------------------------------
// 128x128 block weight quantization: one 256-thread block per weight block.
// Thread t covers rows (t / 16) + 16 i, i = 0..7, chunk t % 16 of the block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_wblock_kernel(
    const uint4* __restrict__ w, int64_t N, int64_t K, uint2* __restrict__ q,
    float* __restrict__ scale) {
  __shared__ uint32_t red[4];
  const int tid = threadIdx.x;
  const int64_t kb = blockIdx.x, nb = blockIdx.y;
  const int64_t nch = K >> 3;
  const int64_t col = kb * 16 + (tid & 15);
  uint4 v[8];
  us2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = nb * 128 + (tid >> 4) + 16 * i;
    v[i] = w[r * nch + col];
    m2 = chunk_amax(v[i], m2);
  }
  uint32_t m = m2.x > m2.y ? m2.x : m2.y;
  m = wave64_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int i = 1; i < 4; ++i) m = m > red[i] ? m : red[i];
  float s, r, p;
  bool tiny;
  unit_scale(m, s, r, p, tiny);
  if (tid == 0) scale[nb * (K >> 7) + kb] = s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t rr = nb * 128 + (tid >> 4) + 16 * i;
    q[rr * nch + col] = tiny ? quant8<true>(v[i], s, r, p)
                             : quant8<false>(v[i], s, r, p);
  }
}

template <int CH, int TW, bool SPLIT = false>
void launch_rows(const void* x, int64_t rows, int64_t K, uint8_t* q,
                 float* scale, hipStream_t st) {
  constexpr int RPB = TW >= 4 ? 1 : 4 / TW;
  constexpr int THREADS = TW >= 4 ? 64 * TW : 256;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((quant_rows_kernel<CH, TW, SPLIT>), dim3((unsigned)blocks, SPLIT ? CH : 1),
                     dim3(THREADS), 0, st, (const uint4*)x, rows, K, (uint2*)q,
                     scale);
}

}  // namespace

// Host launchers (validated arguments only).
void launch_quant_rows(const void* x, int64_t rows, int64_t K, uint8_t* q,
                       float* scale, hipStream_t st) {
  const int64_t nch = K / 8;
  // Few rows (decode): 1024-thread blocks, each thread 1-4 chunks, so the
  // load -> amax -> quantize chain of one row is short; with 2 or 4 chunks,
  // as many blocks per row, each encoding one chunk per lane (the encoding
  // dominates: on one CU, a 28672-wide row took 5.2 us, 64 of them 8.8 us).
  if (rows <= 128 && nch > 64 && nch <= 1024 * 4) {
    if (nch <= 1024) launch_rows<1, 16>(x, rows, K, q, scale, st);
    else if (nch <= 2048) launch_rows<2, 16, true>(x, rows, K, q, scale, st);
    else launch_rows<4, 16, true>(x, rows, K, q, scale, st);
    return;
  }
  // One wave per row for short rows, else a team of 4 (or 8) waves. At
  // K = 4096 (512 chunks) the team is faster than one wave with 8 chunks per
  // lane: 16.7 against 21.0 us on 4096 rows from HBM (the row's loads spread
  // over 4 waves, and its amax / codes chain is 4 times shorter per lane);
  // at K = 14336, 8 waves with 4 chunks each: 38 against 40 us.
  if (nch <= 64 * 1) launch_rows<1, 1>(x, rows, K, q, scale, st);
  else if (nch <= 64 * 2) launch_rows<2, 1>(x, rows, K, q, scale, st);
  else if (nch <= 64 * 4) launch_rows<4, 1>(x, rows, K, q, scale, st);
  else if (nch <= 256 * 2) launch_rows<2, 4>(x, rows, K, q, scale, st);
  else if (nch <= 256 * 3) launch_rows<3, 4>(x, rows, K, q, scale, st);
  else if (nch <= 256 * 4) launch_rows<4, 4>(x, rows, K, q, scale, st);
  else if (nch <= 256 * 6) launch_rows<6, 4>(x, rows, K, q, scale, st);
  else if (nch <= 256 * 8) launch_rows<4, 8>(x, rows, K, q, scale, st);
  else if (nch <= 256 * 12) launch_rows<12, 4>(x, rows, K, q, scale, st);
  else if (nch <= 256 * 16) launch_rows<16, 4>(x, rows, K, q, scale, st);
  else
    hipLaunchKernelGGL(quant_rows_2pass_kernel, dim3((unsigned)rows), dim3(256),
                       0, st, (const uint4*)x, rows, K, (uint2*)q, scale);
}

void launch_quant_groups(const void* x, int64_t rows, int64_t K, uint8_t* q,
                         float* scale, hipStream_t st) {
  // 2 chunks per thread: on the Llama-3.2-3B inputs (8192 x 3072 and x 8192)
  // 18.0-18.1 and 40.1-40.7 us, against 19.0-19.3 and 40.8-40.9 with 4 and
  // 19.0 and 45-47 with 1 (alternating builds on one box)
  constexpr int U = 2;
  const int64_t total = rows * (K / 8);
  const int64_t blocks = (total + 256 * U - 1) / (256 * U);
  hipLaunchKernelGGL((quant_groups_kernel<U>), dim3((unsigned)blocks),
                     dim3(256), 0, st, (const uint4*)x, total, (uint2*)q,
                     scale);
}

void launch_quant_wblock(const void* w, int64_t N, int64_t K, uint8_t* q,
                         float* scale, hipStream_t st) {
  hipLaunchKernelGGL(quant_wblock_kernel, dim3((unsigned)(K / 128), (unsigned)(N / 128)),
                     dim3(256), 0, st, (const uint4*)w, N, K, (uint2*)q, scale);
}

}  // namespace fp8dq
