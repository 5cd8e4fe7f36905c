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
//  * A/B tiles go straight from global memory to LDS (global_load_lds, 16 B
//    per lane, no staging registers), double buffered: the next K step's
//    loads are in flight while the current step's MFMAs run; each wave waits
//    for its own loads (vmcnt) and one barrier per K step publishes them;
//  * LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by the row so
//    that the fragment reads (16 rows x one chunk per 16 lanes) hit distinct
//    banks;
//  * workgroup ids are remapped so that tiles sharing A/B panels run on the
//    same XCD (ids are dealt round-robin over the 8 XCDs) and, within an
//    XCD, in groups of GM tile rows for L2 reuse.
#include "device_common.hpp"
#include "gemm_line.hpp"
#include "kernels.hpp"

#include <mutex>
#include <type_traits>

namespace fp8dq {
namespace {

constexpr int BK = 128;
constexpr int GM = 8;  // tile rows per L2 group
// s_waitcnt immediate (gfx9 encoding): wait until at most n vector-memory
// operations of this wave are outstanding (expcnt / lgkmcnt not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kVmcnt0 = vmcnt_imm(0);

typedef __attribute__((address_space(1))) void* gbl_ptr;

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
  constexpr int XQ = BM / 32, WQ = BN / 32;  // 8-row groups per wave per stage
  constexpr int STAGE = (BM + BN) * BK;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lr = lane & 15, kg = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- direct global->LDS loads: a wave writes 1 KB = 8 tile rows per
  // instruction, lane l to byte 16*l; lane l therefore fetches row l/8 of
  // its group and the logical chunk whose swizzled slot is l % 8 ----
  uint32_t xoff[XQ], woff[WQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int g = q * 4 + wave, row = 8 * g + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    xoff[q] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)K + (uint32_t)(c * 16);
  }
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int g = q * 4 + wave, row = 8 * g + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    woff[q] = (uint32_t)min(n0 + row, N - 1) * (uint32_t)K + (uint32_t)(c * 16);
  }
  auto issue = [&](int kt, int stage) {
    const uint8_t* xk = qx + (size_t)kt * BK;
    const uint8_t* wk = qw + (size_t)kt * BK;
    uint8_t* sb = smem + stage * STAGE;
#pragma unroll
    for (int q = 0; q < XQ; ++q)
      __builtin_amdgcn_global_load_lds((gbl_ptr)(xk + xoff[q]),
                                       (lds_ptr)(sb + (q * 4 + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < WQ; ++q)
      __builtin_amdgcn_global_load_lds((gbl_ptr)(wk + woff[q]),
                                       (lds_ptr)(sb + BM * BK + (q * 4 + wave) * 1024), 16, 0, 0);
  };

  v4f acc[NI][MJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // block-variant scales: row pointers of sx, weight-block row of this wave
  const int G = K / BK;
  const float* sxr[MJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j)
    sxr[j] = sx + (size_t)min(m0 + wm * TM + 16 * j + lr, M - 1) * (BLOCK ? G : 1);
  const float* swr = sw + (size_t)((n0 + wn * TN) / 128) * (BLOCK ? G : 1);
  float sxc[MJ], sxn[MJ];
  float swc = 0.f, swn = 0.f;

  const int KT = K / BK;
  if (BLOCK) {
#pragma unroll
    for (int j = 0; j < MJ; ++j) sxc[j] = sxr[j][0];
    swc = swr[0];
  }
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) {
      if (BLOCK) {  // next step's scales, issued before the tile loads
#pragma unroll
        for (int j = 0; j < MJ; ++j) sxn[j] = sxr[j][kt + 1];
        swn = swr[kt + 1];
      }
      issue(kt + 1, (kt + 1) & 1);
    }

    const uint8_t* sX = smem + (kt & 1) * STAGE;
    const uint8_t* sW = sX + BM * BK;
    // Fragment schedule (pinned with scheduling barriers): A(0), then all B,
    // then for each A block i: read A(i+1), run the MFMAs of A(i). Each
    // MFMA group waits only for its own operands, and the next A fragment's
    // LDS latency hides under the current group's MFMAs.
    v8i a[2];
    a[0] = lds_frag(sW, wn * TN + lr, kg);
    v8i b[MJ];
#pragma unroll
    for (int j = 0; j < MJ; ++j) b[j] = lds_frag(sX, wm * TM + 16 * j + lr, kg);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + 1 < NI) a[(i + 1) & 1] = lds_frag(sW, wn * TN + 16 * (i + 1) + lr, kg);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if (BLOCK) {
          const v4f t = mfma_e4m3_16x16x128(a[i & 1], b[j], v4f{0.f, 0.f, 0.f, 0.f});
          const float sc = sxc[j] * swc;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(t[r], sc, acc[i][j][r]);
        } else {
          acc[i][j] = mfma_e4m3_16x16x128(a[i & 1], b[j], acc[i][j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // this wave's loads of step kt+1 landed
    __syncthreads();                      // everyone's landed; step kt fully read
    if (BLOCK) {
#pragma unroll
      for (int j = 0; j < MJ; ++j) sxc[j] = sxn[j];
      swc = swn;
    }
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
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] * (sm * s4[r]);   // scales first
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
  // The whole-line kernels need at least two 128-byte K pairs (K >= 256) and,
  // per-channel, at least one round of 256 x 256 tiles on the CUs (fewer
  // tiles leave CUs idle with one workgroup per CU); everything else runs on
  // the 256 x 128 small-tile kernel.
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  if (block) {
    if (K >= 256) launch_gemm_line_block(qx, sx, qw, sw, y, M, N, K, st);
    else launch_cfg<256, 128, true>(qx, sx, qw, sw, y, M, N, K, st);
    return;
  }
  if (big >= 256 && K >= 256) {
    // 256 x 192 tiles when they fill the last round of tiles on the CUs
    // better: the time goes as (rounds of tiles) x (tile width), and a
    // shape like 4096 x 6144 has 1.5 rounds of 256-wide tiles but two full
    // rounds of 192-wide ones
    const int ncu = line::cu_count();
    const int64_t tm = (M + 255) / 256;
    const int64_t t256 = tm * ((N + 255) / 256), t192 = tm * ((N + 191) / 192);
    bool narrow = false;
    if (ncu > 0) {
      const int64_t r256 = (t256 + ncu - 1) / ncu, r192 = (t192 + ncu - 1) / ncu;
      narrow = r192 * 192 * 10 < r256 * 256 * 9;   // at least 10 % less
    }
    if (narrow) line::launch_line<false, 192>(qx, sx, qw, sw, y, M, N, K, st);
    else line::launch_line<false, 256>(qx, sx, qw, sw, y, M, N, K, st);
  } else {
    launch_cfg<256, 128, false>(qx, sx, qw, sw, y, M, N, K, st);
  }
}

}  // namespace fp8dq
