// Prefill (large-M) FP8 GEMM with fused scale epilogue, gfx950.
//
// Computes Y[m,n] = bf16( sum_k val(qx[m,k]) val(qw[n,k]) * scales ), the
// FP8-Dynamic linear's contraction: E4M3 activations (dynamic, per token)
// times E4M3 weights (per output channel), fp32 accumulation, rescaled to
// bf16 (Llama-3.1-8B-Instruct-FP8-Dynamic page, FP8 dynamic quantization
// table); block variant with one weight scale per 128x128 block and one
// activation scale per 128-wide group (Llama-3.2-3B-Instruct-FP8-Block page,
// FP8 block quantization table).
//
// Structure:
//  * workgroup = 4 waves (2 x 2), output tile BM x BN, wave tile
//    (BM/2) x (BN/2); K advances 128 bytes per step, which is exactly one
//    v_mfma_f32_16x16x128_f8f6f4 and, in the block variant, one scale group;
//  * the MFMA "A" operand is the weight tile and "B" the activation tile, so
//    each lane's four results are four consecutive n of one row m and the
//    epilogue stores 8 contiguous bytes per lane;
//  * A/B tiles are staged global -> registers -> LDS, double buffered: the
//    next K step's global loads are in flight while the current step's MFMAs
//    run, one barrier per K step;
//  * LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by the row so
//    that the fragment reads (16 rows x one chunk per 16 lanes) hit distinct
//    banks;
//  * workgroup ids are remapped so that tiles sharing A/B panels run on the
//    same XCD (ids are dealt round-robin over the 8 XCDs) and, within an
//    XCD, in groups of GM tile rows for L2 reuse.
#include "device_common.hpp"
#include "kernels.hpp"

#include <mutex>

namespace fp8dq {
namespace {

constexpr int BK = 128;
constexpr int GM = 8;  // tile rows per L2 group

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// LDS byte offset of 16-byte chunk c of tile row `row`.
__device__ __forceinline__ int lds_off(int row, int c) {
  return row * BK + ((c ^ swz(row)) << 4);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int kg) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + lds_off(row, 2 * kg));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + lds_off(row, 2 * kg + 1));
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <int BM, int BN, bool BLOCK>
__global__ __launch_bounds__(256, 1) void gemm_prefill_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int TM = BM / 2, TN = BN / 2;
  constexpr int MJ = TM / 16, NI = TN / 16;
  constexpr int XL = BM / 32, WL = BN / 32;  // 16-byte loads per thread
  constexpr int STAGE = (BM + BN) * BK;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- tile selection: XCD-aware remap, then grouped row-major order ----
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int group = GM * tiles_n;
  const int first_m = (bid / group) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_g = bid % group;
  const int tm = first_m + in_g % gm;
  const int tn = in_g / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kg = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- global load addressing: thread -> (row, chunk) of each tile ----
  const uint8_t* gx[XL];
  const uint8_t* gw[WL];
  int lx[XL], lw[WL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int id = tid + 256 * i, row = id >> 3, c = id & 7;
    const int gr = min(m0 + row, M - 1);
    gx[i] = qx + (int64_t)gr * K + c * 16;
    lx[i] = lds_off(row, c);
  }
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int id = tid + 256 * i, row = id >> 3, c = id & 7;
    const int gr = min(n0 + row, N - 1);
    gw[i] = qw + (int64_t)gr * K + c * 16;
    lw[i] = BM * BK + lds_off(row, c);
  }

  uint4 rx[XL], rw[WL];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < XL; ++i) rx[i] = *reinterpret_cast<const uint4*>(gx[i] + k0);
#pragma unroll
    for (int i = 0; i < WL; ++i) rw[i] = *reinterpret_cast<const uint4*>(gw[i] + k0);
  };
  auto lstore = [&](int stage) {
    uint8_t* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < XL; ++i) *reinterpret_cast<uint4*>(base + lx[i]) = rx[i];
#pragma unroll
    for (int i = 0; i < WL; ++i) *reinterpret_cast<uint4*>(base + lw[i]) = rw[i];
  };

  v4f acc[NI][MJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // block-variant scale addressing
  const int G = K / BK;
  int mrow[MJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j) mrow[j] = min(m0 + wm * TM + 16 * j + lr, M - 1);
  const int wblk = (n0 + wn * TN) / 128;  // weight block row of this wave

  const int KT = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    float sxg[MJ];
    float swg = 0.f;
    if (BLOCK) {
#pragma unroll
      for (int j = 0; j < MJ; ++j) sxg[j] = sx[(int64_t)mrow[j] * G + kt];
      swg = sw[(int64_t)wblk * G + kt];
    }
    if (kt + 1 < KT) gload(kt + 1);

    const uint8_t* sX = smem + (kt & 1) * STAGE;
    const uint8_t* sW = sX + BM * BK;
    v8i b[MJ];
#pragma unroll
    for (int j = 0; j < MJ; ++j) b[j] = lds_frag(sX, wm * TM + 16 * j + lr, kg);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const v8i a = lds_frag(sW, wn * TN + 16 * i + lr, kg);
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if (BLOCK) {
          const v4f t = mfma_e4m3_16x16x128(a, b[j], v4f{0.f, 0.f, 0.f, 0.f});
          const float sc = sxg[j] * swg;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(t[r], sc, acc[i][j][r]);
        } else {
          acc[i][j] = mfma_e4m3_16x16x128(a, b[j], acc[i][j]);
        }
      }
    }
    if (kt + 1 < KT) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: scale, round to bf16, store 4 consecutive n per lane ----
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int m = m0 + wm * TM + 16 * j + lr;
    if (m >= M) continue;
    const float sm = BLOCK ? 1.0f : sx[m];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = n0 + wn * TN + 16 * i + 4 * kg;
      float v[4];
      if (BLOCK) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r];
      } else {
        float s4[4];
        if (vec_ok && n + 3 < N) {
          const float4 t = *reinterpret_cast<const float4*>(sw + n);
          s4[0] = t.x; s4[1] = t.y; s4[2] = t.z; s4[3] = t.w;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) s4[r] = (n + r < N) ? sw[n + r] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] * sm * s4[r];
      }
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

template <int BM, int BN, bool BLOCK>
void launch_cfg(const uint8_t* qx, const float* sx, const uint8_t* qw,
                const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                hipStream_t st) {
  constexpr int smem = 2 * (BM + BN) * BK;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_prefill_kernel<BM, BN, BLOCK>),
        hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  });
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_prefill_kernel<BM, BN, BLOCK>),
                     dim3((unsigned)(tiles_m * tiles_n)), dim3(256), smem, st,
                     qx, sx, qw, sw, (uint16_t*)y, (int)M, (int)N, (int)K,
                     tiles_m, tiles_n);
}

}  // namespace

void launch_gemm_prefill(const uint8_t* qx, const float* sx, const uint8_t* qw,
                         const float* sw, void* y, int64_t M, int64_t N,
                         int64_t K, bool block, hipStream_t st) {
  // 256 x 256 tiles halve the L2->CU traffic per flop against 256 x 128; use
  // them when they still give at least two full waves of tiles on 256 CUs.
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  const bool use_big = big >= 512;
  if (block) {
    if (use_big) launch_cfg<256, 256, true>(qx, sx, qw, sw, y, M, N, K, st);
    else launch_cfg<256, 128, true>(qx, sx, qw, sw, y, M, N, K, st);
  } else {
    if (use_big) launch_cfg<256, 256, false>(qx, sx, qw, sw, y, M, N, K, st);
    else launch_cfg<256, 128, false>(qx, sx, qw, sw, y, M, N, K, st);
  }
}

}  // namespace fp8dq
