// Decode (small-M) FP8 GEMM for gfx950: the weight stream is the cost.
//
// Same contraction and epilogue as the prefill kernel (FP8 dynamic
// quantization table on the Llama-3.1-8B-Instruct-FP8-Dynamic page; block
// table on the Llama-3.2-3B-Instruct-FP8-Block page), for M <= 64 tokens,
// where every weight byte is used by at most 64 rows and the layer is bound
// by reading W from HBM (the 70B page's section 3 notes that the FP8 gain
// comes from moving half the bytes).
//
// Structure:
//  * a workgroup owns 16*NB weight rows; its 4 waves take interleaved
//    128-byte K steps of those rows (wave w: steps w, w+4, ...), so the
//    workgroup streams contiguous K and no two waves load the same bytes;
//  * each wave keeps D K-steps of fragments in flight (loads for step t+D
//    issue right after step t's MFMAs); weight loads are plain loads
//    (non-temporal hints measured slower);
//  * MFMA operand A = 16 weight rows, B = 16 token rows (rows past M read
//    zeros through a bounds-checked load, with no memory access; their
//    outputs are dropped);
//  * the 4 waves' partial sums are added in a fixed order through LDS;
//  * when N alone gives too few workgroups and the rows are long (K >=
//    16384), K is also split across the grid (grid.y): fp32 partials go to a
//    workspace and a second kernel adds them in split order and applies the
//    epilogue -- deterministic.
#include "device_common.hpp"
#include "kernels.hpp"

#include <mutex>

namespace fp8dq {
namespace {

constexpr int BK = 128;

// Compile-time tunables (defaults are the tuned values).
#ifndef FP8DQ_DEC_D
#define FP8DQ_DEC_D 4      // K steps of fragments in flight per wave
#endif
#ifndef FP8DQ_DEC_NT
#define FP8DQ_DEC_NT 0     // non-temporal weight loads (measured slower)
#endif

__device__ __forceinline__ v8i gload_frag_nt(const uint8_t* p) {
  const uint4 lo = ld16_nt(p);
  const uint4 hi = ld16_nt(p + 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

__device__ __forceinline__ v8i gload_frag(const uint8_t* p) {
  const uint4 lo = ld16(p);
  const uint4 hi = ld16(p + 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Token-row fragment through a bounds-checked buffer load: a lane whose
// offset lies past the buffer's size reads zeros without a memory access.
// (Raw buffer resource, word 3 = 0x00020000 on gfx9-family parts.)
__device__ __forceinline__ v8i bload_frag(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16u), 0, 0);
  v8i res;
  res[0] = (int)lo.x; res[1] = (int)lo.y; res[2] = (int)lo.z; res[3] = (int)lo.w;
  res[4] = (int)hi.x; res[5] = (int)hi.y; res[6] = (int)hi.z; res[7] = (int)hi.w;
  return res;
}

template <int MB, int NB, int D, bool BLOCK>
__global__ __launch_bounds__(256) void gemm_decode_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K,
    int kt_per_split) {
  __shared__ v4f red[4][NB * MB][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kg = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB;
  const int split = blockIdx.y;
  const int KT = K / BK;
  const int G = KT;
  const int kt0 = split * kt_per_split;
  const int kt1 = min(KT, kt0 + kt_per_split);

  const uint8_t* wp[NB];
  int xrow[MB];
  // Token rows: lanes of MFMA padding rows (16 j + lr >= M) get an offset past
  // the buffer and load nothing. Their outputs are dropped; loads repeating a
  // real row cost the load path as much as distinct ones (at M = 1, 15 of 16
  // token rows are padding). M * K < 2^30 on this path (M <= 64, K < 2^24).
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)qx, (short)0, M * K, 0x00020000);
  uint32_t xoff[MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    wp[i] = qw + (int64_t)min(n0 + 16 * i + lr, N - 1) * K + kg * 32;
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    xrow[j] = min(16 * j + lr, M - 1);
    xoff[j] = 16 * j + lr < M ? (uint32_t)(16 * j + lr) * (uint32_t)K + (uint32_t)(kg * 32)
                              : 0x80000000u;
  }

  v4f acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // K steps of this wave: kt0 + wave + 4 t, t = 0 .. cnt-1
  const int first = kt0 + wave;
  const int cnt = first < kt1 ? (kt1 - first + 3) / 4 : 0;

  v8i a[D][NB], b[D][MB];
  float sxr[D][MB], swr[D][NB];   // block: the step's group scales, loaded with it
  // (a step index past the row's end is clamped: the prologue loads D steps
  // without conditions, so the loop starts with a known number in flight)
  auto load = [&](int d, int t) {
    const int kt = min(first + 4 * t, KT - 1);
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      a[d][i] = FP8DQ_DEC_NT ? gload_frag_nt(wp[i] + k0) : gload_frag(wp[i] + k0);
#pragma unroll
    for (int j = 0; j < MB; ++j) b[d][j] = bload_frag(xrs, xoff[j] + (uint32_t)k0);
    if (BLOCK) {
      const int g = kt;
#pragma unroll
      for (int j = 0; j < MB; ++j) sxr[d][j] = sx[(int64_t)xrow[j] * G + g];
#pragma unroll
      for (int i = 0; i < NB; ++i) swr[d][i] = sw[(int64_t)((n0 + 16 * i) >> 7) * G + g];
    }
  };
  auto compute = [&](int d) {
    if (BLOCK) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          const v4f p = mfma_e4m3_16x16x128(a[d][i], b[d][j], v4f{0.f, 0.f, 0.f, 0.f});
          const float sc = sxr[d][j] * swr[d][i];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sc, acc[i][j][r]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = mfma_e4m3_16x16x128(a[d][i], b[d][j], acc[i][j]);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
  // Steady state: every step of a batch has a step D ahead to load, so the
  // body has no conditions and each step waits only for its own loads (the
  // compiler cannot count loads across the tail's conditions and waits for
  // all of them there, draining the D steps in flight).
  int t0 = 0;
  for (; t0 + 2 * D <= cnt; t0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(d);
      load(d, t0 + d + D);
    }
  }
  for (; t0 < cnt; t0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int t = t0 + d;
      if (t < cnt) {
        compute(d);
        if (t + D < cnt) load(d, t + D);
      }
    }
  }

  // ---- fixed-order reduction of the 4 waves' partial sums ----
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) red[wave][i * MB + j][lane] = acc[i][j];
  __syncthreads();
  if (wave != 0) return;
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + 16 * i + 4 * kg;
    if (n >= N) continue;
    float s4[4] = {1.f, 1.f, 1.f, 1.f};
    if (!BLOCK && ws == nullptr) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s4[r] = (n + r < N) ? sw[n + r] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int m = 16 * j + lr;
      if (m >= M) continue;
      v4f s = red[0][i * MB + j][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const v4f o = red[w][i * MB + j][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] += o[r];
      }
      if (ws != nullptr) {  // split-K partial (already block-scaled if BLOCK)
        float* out = ws + ((int64_t)split * M + m) * N + n;
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<float4*>(out) = make_float4(s[0], s[1], s[2], s[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) out[r] = s[r];
        }
      } else {
        const float sm = BLOCK ? 1.0f : sx[m];
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = BLOCK ? s[r] : s[r] * sm * s4[r];
        uint16_t* out = y + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(out) = pk;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) out[r] = (uint16_t)f32_to_bf16_rne(v[r]);
        }
      }
    }
  }
}

// y[m,n] = bf16( (sum over splits, in order, of ws[s,m,n]) * scales )
// S > 0: the number of slices is a compile-time constant, so all S partials
// of an output are loaded before the first add (one memory latency instead of
// S); S = 0: any number, one partial at a time. Either way the partials are
// added in slice order.
template <bool BLOCK, int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ ws, const float* __restrict__ sx,
    const float* __restrict__ sw, uint16_t* __restrict__ y, int M, int N,
    int splits) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)M * N;
  if (idx >= total) return;
  const int64_t m = idx / N, n = idx % N;
  float s;
  if constexpr (S > 0) {
    float p[S];
#pragma unroll
    for (int k = 0; k < S; ++k) p[k] = ws[(int64_t)k * total + idx];
    s = p[0];
#pragma unroll
    for (int k = 1; k < S; ++k) s += p[k];
  } else {
    s = ws[idx];
    for (int k = 1; k < splits; ++k) s += ws[(int64_t)k * total + idx];
  }
  const float v = BLOCK ? s : s * sx[m] * sw[n];
  y[idx] = (uint16_t)f32_to_bf16_rne(v);
}

template <bool BLOCK, int S = 2>
void launch_reduce(const float* ws, const float* sx, const float* sw, uint16_t* y,
                   int64_t M, int64_t N, int splits, hipStream_t st) {
  if constexpr (S <= 16) {
    if (splits != S) {
      launch_reduce<BLOCK, S + 1>(ws, sx, sw, y, M, N, splits, st);
      return;
    }
  }
  constexpr int SK = S <= 16 ? S : 0;
  const int64_t total = M * N;
  hipLaunchKernelGGL((splitk_reduce_kernel<BLOCK, SK>), dim3((unsigned)((total + 255) / 256)),
                     dim3(256), 0, st, ws, sx, sw, y, (int)M, (int)N, splits);
}

// ---------------------------------------------------------------------------
// Whole-line decode kernel: 128 weight rows x (16 MB) token rows per
// workgroup, one 128-byte K step (a pair of 64-byte halves, or one scale
// group) per step, v_mfma_f32_16x16x128_f8f6f4.
//  * Weights and the token rows' codes move HBM/L2 -> LDS with whole-line
//    loads (8 rows x 128 bytes per instruction) into an LDS ring; the
//    codes of the token rows are loaded once per workgroup and shared by the
//    4 waves (each wave takes 32 weight rows), where the register-loading
//    kernel had every wave fetch them again.
//  * Rows of 128 bytes with 16-byte chunks XOR-permuted by row bits 0-3
//    (conflict-free 16-row fragment reads; every 16-row fragment has the
//    same permutation).
//  * Step p: wait for pair p (the newer ones may stay in flight), barrier,
//    refill the slot of pair p-1, read pair p, run its MFMAs. The
//    barrier also proves that every wave's reads of pair p-1 are done (their
//    MFMAs waited for them).
//  * Per-channel: fp32 accumulation; block: each 128-wide step is one scale
//    group, accumulated with its factor sx[m,g] * sw[n/128,g]; the group's
//    scales ride with its pair into the slot (one 4-byte-per-lane load).
//  * One K slice per grid row; more than one slice writes fp32 partials for
//    splitk_reduce_kernel.
// ---------------------------------------------------------------------------
constexpr int DL_BN = 128;               // weight rows per workgroup
#ifndef FP8DQ_DL_NSL
#define FP8DQ_DL_NSL 3
#endif
constexpr int DL_NSL = FP8DQ_DL_NSL;     // ring slots

__device__ __forceinline__ int dswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// s_waitcnt immediate: at most n vector-memory operations outstanding
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

template <int MB, bool BLOCK>
__global__ __launch_bounds__(256, 2) void gemm_decode_line_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K,
    int kp_per_split) {
  constexpr int BMR = 16 * MB;                       // token rows (padded)
  constexpr int SLOT = (BMR + DL_BN) * BK + (BLOCK ? 512 : 0);  // + block scales
  constexpr int XB = BMR * BK;                       // weight part of a slot
  constexpr int SB = (BMR + DL_BN) * BK;             // block: sx [64] then sw [64]
  constexpr int XI = (2 * MB + 3) / 4;               // token-row loads per wave (>= 1)
  constexpr int WI = DL_BN / 32;                     // weight loads per wave
  constexpr int L = XI + WI + (BLOCK ? 1 : 0);
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * DL_BN;
  const int split = blockIdx.y;
  const int KP = K / BK;
  const int p0 = split * kp_per_split;
  const int p1 = min(KP, p0 + kp_per_split);
  const int np = p1 - p0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;

  // loads: lane l covers row 8g + l/8, chunk slot l%8 <- global chunk
  // (l%8) ^ dswz(row) = (l%8) ^ (l/8) ^ (g & 1)
  const int rl = lane >> 3;
  uint32_t xoff[XI], woff[WI];
  int xg[XI];
#pragma unroll
  for (int u = 0; u < XI; ++u) {
    // token-row groups 0 .. 2MB-1; with fewer groups than waves, the extra
    // waves load a copy of group (wave % 2MB) (identical bytes, same place)
    const int g = (4 * u + wave) % (2 * MB);
    xg[u] = g;
    const int row = min(8 * g + rl, M - 1);
    xoff[u] = (uint32_t)row * (uint32_t)K + (uint32_t)(((lane & 7) ^ rl ^ (g & 1)) << 4);
  }
#pragma unroll
  for (int u = 0; u < WI; ++u) {
    const int g = 4 * u + wave;
    const int row = min(n0 + 8 * g + rl, N - 1);
    woff[u] = (uint32_t)row * (uint32_t)K + (uint32_t)(((lane & 7) ^ rl ^ (g & 1)) << 4);
  }
  const int KPall = K / BK;
  // block: wave 1 loads the weight-block scale of the group (every lane the
  // same value), the other waves the token rows' activation scales (the
  // same 64 values each)
  const uint32_t scoff = BLOCK
      ? (wave == 1 ? (uint32_t)(n0 >> 7) * (uint32_t)KPall * 4u
                   : (uint32_t)min(lane, M - 1) * (uint32_t)KPall * 4u)
      : 0u;
  auto issue = [&](int p) {   // pair p of this slice (clamped) into slot p % DL_NSL
    const int pc = p0 + min(p, np - 1);
    const uint32_t sb = lds0 + (uint32_t)((p % DL_NSL) * SLOT);
    const size_t koff = (size_t)pc * BK;
#pragma unroll
    for (int u = 0; u < XI; ++u) dma16(qx + koff, xoff[u], sb + (uint32_t)(xg[u] * 1024));
#pragma unroll
    for (int u = 0; u < WI; ++u)
      dma16(qw + koff, woff[u], sb + XB + (uint32_t)((4 * u + wave) * 1024));
    if constexpr (BLOCK)
      dma4(wave == 1 ? (const void*)sw : (const void*)sx, scoff + (uint32_t)pc * 4u,
           sb + SB + (wave == 1 ? 256u : 0u));
  };

  // fragments (16 x 128 bytes): lane l reads row 16 f + l % 16, chunks
  // 2 (l / 16) and 2 (l / 16) + 1
  const int fr = lane & 15, kq = lane >> 4;
  const uint32_t o0 = (uint32_t)(fr * BK + (((2 * kq) ^ dswz(fr)) << 4));
  const uint32_t o1 = (uint32_t)(fr * BK + (((2 * kq + 1) ^ dswz(fr)) << 4));
  auto rd = [&](const uint8_t* base) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + o0);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + o1);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
  };

  v4f acc[2][MB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int q = 0; q < DL_NSL - 1; ++q) issue(q);
  for (int p = 0; p < np; ++p) {
    // pair p landed; the DL_NSL-2 newer pairs may still be in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((DL_NSL - 2) * L));
    asm volatile("s_barrier" ::: "memory");
    issue(p + DL_NSL - 1);
    const uint8_t* sb = smem + (p % DL_NSL) * SLOT;
    v8i a[2], b[MB];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = rd(sb + XB + (32 * wave + 16 * i) * BK);
#pragma unroll
    for (int j = 0; j < MB; ++j) b[j] = rd(sb + 16 * j * BK);
    if constexpr (BLOCK) {   // the group's scales from the slot
      const float* scl = reinterpret_cast<const float*>(sb + SB);
      const float swg = scl[64];
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const float f = scl[16 * j + fr] * swg;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const v4f pr = mfma_e4m3_16x16x128(a[i], b[j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], f, acc[i][j][r]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = mfma_e4m3_16x16x128(a[i], b[j], acc[i][j]);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may still target LDS

  // D[n, m]: lane l holds n = 16 i + 4 (l / 16) + r of the wave's rows, m = 16 j + l % 16
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = n0 + 32 * wave + 16 * i + 4 * kq;
    if (n >= N) continue;
    float s4[4] = {1.f, 1.f, 1.f, 1.f};
    if (!BLOCK && ws == nullptr) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s4[r] = sw[min(n + r, N - 1)];
    }
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int m = 16 * j + fr;
      if (m >= M) continue;
      const v4f s = acc[i][j];
      if (ws != nullptr) {  // split-K partial (already block-scaled if BLOCK)
        float* out = ws + ((int64_t)split * M + m) * N + n;
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<float4*>(out) = make_float4(s[0], s[1], s[2], s[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) out[r] = s[r];
        }
      } else {
        const float sm = BLOCK ? 1.0f : sx[m];
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = BLOCK ? s[r] : s[r] * sm * s4[r];
        uint16_t* out = y + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(out) = pk;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) out[r] = (uint16_t)f32_to_bf16_rne(v[r]);
        }
      }
    }
  }
}

template <int MB, bool BLOCK>
void launch_line_dec(const uint8_t* qx, const float* sx, const uint8_t* qw,
                     const float* sw, void* y, float* ws, int64_t M, int64_t N,
                     int64_t K, const DecodePlan& p, hipStream_t st) {
  constexpr int smem = DL_NSL * ((16 * MB + DL_BN) * BK + (BLOCK ? 512 : 0));
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_decode_line_kernel<MB, BLOCK>),
        hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  });
  const unsigned gx = (unsigned)((N + DL_BN - 1) / DL_BN);
  float* part = p.splits > 1 ? ws : nullptr;
  hipLaunchKernelGGL((gemm_decode_line_kernel<MB, BLOCK>), dim3(gx, (unsigned)p.splits),
                     dim3(256), smem, st, qx, sx, qw, sw, (uint16_t*)y, part, (int)M, (int)N,
                     (int)K, p.kt_per_split);
  if (p.splits > 1) launch_reduce<BLOCK>(ws, sx, sw, (uint16_t*)y, M, N, p.splits, st);
}

template <int MB, int NB, int D, bool BLOCK>
void launch_cfg(const uint8_t* qx, const float* sx, const uint8_t* qw,
                const float* sw, void* y, float* ws, int64_t M, int64_t N,
                int64_t K, const DecodePlan& p, hipStream_t st) {
  const unsigned gx = (unsigned)((N + 16 * NB - 1) / (16 * NB));
  float* part = p.splits > 1 ? ws : nullptr;
  hipLaunchKernelGGL((gemm_decode_kernel<MB, NB, D, BLOCK>),
                     dim3(gx, (unsigned)p.splits), dim3(256), 0, st, qx, sx, qw,
                     sw, (uint16_t*)y, part, (int)M, (int)N, (int)K,
                     p.kt_per_split);
  if (p.splits > 1) launch_reduce<BLOCK>(ws, sx, sw, (uint16_t*)y, M, N, p.splits, st);
}

template <int MB, bool BLOCK>
void launch_mb(const uint8_t* qx, const float* sx, const uint8_t* qw,
               const float* sw, void* y, float* ws, int64_t M, int64_t N,
               int64_t K, const DecodePlan& p, hipStream_t st) {
  if (p.nb == 1) launch_cfg<MB, 1, FP8DQ_DEC_D, BLOCK>(qx, sx, qw, sw, y, ws, M, N, K, p, st);
  else if (p.nb == 2) launch_cfg<MB, 2, FP8DQ_DEC_D, BLOCK>(qx, sx, qw, sw, y, ws, M, N, K, p, st);
  else launch_cfg<MB, 4, FP8DQ_DEC_D, BLOCK>(qx, sx, qw, sw, y, ws, M, N, K, p, st);
}

}  // namespace

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K) {
  DecodePlan p;
  p.mb = (int)((M + 15) / 16);
  if (p.mb < 1) p.mb = 1;
  if (p.mb > 4) p.mb = 4;  // callers guarantee M <= 64 on this path
  const int64_t KT = K / BK;
#ifdef FP8DQ_DEC_NB
  p.nb = FP8DQ_DEC_NB;
#else
#ifdef FP8DQ_DEC_NB_WIDE
  p.nb = (M > 16 || N / 32 >= 1024) ? 2 : 1;
#else
  // Two weight row-blocks per workgroup halve the activation re-reads per
  // weight byte, which pays from M > 16; below, single blocks stream better.
  p.nb = M > 16 ? 2 : 1;
#endif
#endif
#ifdef FP8DQ_DEC_TARGET
  const int64_t target = FP8DQ_DEC_TARGET;
#else
  const int64_t target = 512;
#endif
  // Up to 16 token rows the register-loading kernel streams the weights
  // faster (its loads in flight are not bounded by LDS); above, re-reading
  // the token rows per 16-32 weight rows costs more than the whole-line
  // kernel's shared copy in LDS.
#ifdef FP8DQ_DEC_LINE
  p.line = FP8DQ_DEC_LINE;
#else
  p.line = M > 16 ? 1 : 0;
#endif
  // the whole-line kernel addresses token rows with 32-bit byte offsets
  if ((int64_t)M * K >= (int64_t(1) << 32)) p.line = 0;
  if (p.line) {
    // Whole-line kernel: 128 weight rows per workgroup, two workgroups per
    // CU. Split K until there are >= 384 workgroups (1.5 per CU), keeping at
    // least 8 K steps per slice. Long rows with fewer row blocks than CUs
    // split to 512 workgroups (two on every CU): there the slices' fp32
    // partials are small next to the weights. Measured on the 70B down
    // (K = 28672) at 32 and 64 tokens: 8 slices 59.4 / 63.9 us against 6
    // slices 63.7 / 68.3 us; on K = 8192 shapes 512 workgroups were no faster
    // (o) or slower (qkv, gate_up).
    const int64_t wg0 = (N + DL_BN - 1) / DL_BN;
    const int64_t target = (K >= 16384 && wg0 < 256) ? 512 : 384;
    int64_t s = (target + wg0 - 1) / wg0;
    if (s > KT / 8) s = KT / 8;
    if (s < 1) s = 1;
    p.kt_per_split = (int)((KT + s - 1) / s);
    p.splits = (int)((KT + p.kt_per_split - 1) / p.kt_per_split);
    return p;
  }
  const int64_t wgs = (N + 16 * p.nb - 1) / (16 * p.nb);
  // Split K across the grid until there are >= target workgroups, keeping
  // at least 8 K steps (2 per wave) in each slice -- for long rows only:
  // below K = 16384 a workgroup streams its whole row block in less time
  // than the split's second launch (the reduce) costs. Measured at 16
  // tokens, 4096 -> 1024: 12.0 us unsplit against 15.1 us in 4 slices;
  // 8 tokens, 8192 -> 2048: 12.7 against 15.2 us.
  int64_t splits = 1;
  while (K >= 16384 && wgs * splits < target && KT / (splits * 2) >= 8) splits *= 2;
  p.kt_per_split = (int)((KT + splits - 1) / splits);
  p.splits = (int)((KT + p.kt_per_split - 1) / p.kt_per_split);
  return p;
}

size_t decode_workspace_bytes(int64_t M, int64_t N, const DecodePlan& p) {
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

void launch_gemm_decode(const uint8_t* qx, const float* sx, const uint8_t* qw,
                        const float* sw, void* y, float* ws, int64_t M,
                        int64_t N, int64_t K, bool block, const DecodePlan& p,
                        hipStream_t st) {
  if (p.line) {
    switch (p.mb) {
      case 1: block ? launch_line_dec<1, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                    : launch_line_dec<1, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
      case 2: block ? launch_line_dec<2, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                    : launch_line_dec<2, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
      case 3: block ? launch_line_dec<3, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                    : launch_line_dec<3, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
      default: block ? launch_line_dec<4, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                     : launch_line_dec<4, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
    }
    return;
  }
  switch (p.mb) {
    case 1: block ? launch_mb<1, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                  : launch_mb<1, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
    case 2: block ? launch_mb<2, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                  : launch_mb<2, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
    case 3: block ? launch_mb<3, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                  : launch_mb<3, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
    default: block ? launch_mb<4, true>(qx, sx, qw, sw, y, ws, M, N, K, p, st)
                   : launch_mb<4, false>(qx, sx, qw, sw, y, ws, M, N, K, p, st); break;
  }
}

}  // namespace fp8dq
