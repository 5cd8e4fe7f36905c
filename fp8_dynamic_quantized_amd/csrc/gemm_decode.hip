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
//  * MFMA operand A = 16 weight rows, B = 16 token rows (M padded by
//    clamping the row index; the padded outputs are dropped);
//  * the 4 waves' partial sums are added in a fixed order through LDS;
//  * when N alone gives too few workgroups, K is also split across the grid
//    (grid.y): fp32 partials go to a workspace and a second kernel adds them
//    in split order and applies the epilogue -- deterministic.
#include "device_common.hpp"
#include "kernels.hpp"

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
  const uint8_t* xp[MB];
  int xrow[MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    wp[i] = qw + (int64_t)min(n0 + 16 * i + lr, N - 1) * K + kg * 32;
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    xrow[j] = min(16 * j + lr, M - 1);
    xp[j] = qx + (int64_t)xrow[j] * K + kg * 32;
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
  auto load = [&](int d, int t) {
    const int64_t k0 = (int64_t)(first + 4 * t) * BK;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      a[d][i] = FP8DQ_DEC_NT ? gload_frag_nt(wp[i] + k0) : gload_frag(wp[i] + k0);
#pragma unroll
    for (int j = 0; j < MB; ++j) b[d][j] = gload_frag(xp[j] + k0);
  };
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < cnt) load(d, d);

  for (int t0 = 0; t0 < cnt; t0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int t = t0 + d;
      if (t < cnt) {
        if (BLOCK) {
          const int g = first + 4 * t;
          float sxg[MB];
#pragma unroll
          for (int j = 0; j < MB; ++j) sxg[j] = sx[(int64_t)xrow[j] * G + g];
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            const float swg = sw[(int64_t)((n0 + 16 * i) >> 7) * G + g];
#pragma unroll
            for (int j = 0; j < MB; ++j) {
              const v4f p = mfma_e4m3_16x16x128(a[d][i], b[d][j], v4f{0.f, 0.f, 0.f, 0.f});
              const float sc = sxg[j] * swg;
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sc, acc[i][j][r]);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < MB; ++j)
              acc[i][j] = mfma_e4m3_16x16x128(a[d][i], b[d][j], acc[i][j]);
        }
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
template <bool BLOCK>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ ws, const float* __restrict__ sx,
    const float* __restrict__ sw, uint16_t* __restrict__ y, int M, int N,
    int splits) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)M * N;
  if (idx >= total) return;
  const int64_t m = idx / N, n = idx % N;
  float s = ws[idx];
  for (int k = 1; k < splits; ++k) s += ws[(int64_t)k * total + idx];
  const float v = BLOCK ? s : s * sx[m] * sw[n];
  y[idx] = (uint16_t)f32_to_bf16_rne(v);
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
  if (p.splits > 1) {
    const int64_t total = M * N;
    hipLaunchKernelGGL((splitk_reduce_kernel<BLOCK>),
                       dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       ws, sx, sw, (uint16_t*)y, (int)M, (int)N, p.splits);
  }
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
  const int64_t wgs = (N + 16 * p.nb - 1) / (16 * p.nb);
  // Split K across the grid until there are >= target workgroups, keeping
  // at least 8 K steps (2 per wave) in each slice.
  int64_t splits = 1;
  while (wgs * splits < target && KT / (splits * 2) >= 8) splits *= 2;
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
