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


// ---------------------------------------------------------------------------
// Deep-pipelined per-channel kernel: 256 x 256 tile, 64-byte K stages held in
// an S-slot LDS ring (S * 32 KB), v_mfma_f32_32x32x64_f8f6f4.
//  * loads for K step s are issued S-1 steps ahead with global_load_lds; a
//    wave waits only for the oldest step it needs (partial vmcnt), so S-2
//    steps of L2/MALL latency are covered;
//  * the fragments of step kt+1 are read from LDS while step kt's 16 MFMAs
//    run (two register sets); one barrier per step publishes step kt+1 and
//    frees the slot that step kt+S-1 is loaded into;
//  * the LDS loads are issued by a small asm helper (see dma16): the
//    compiler then does not add its own all-loads wait before every LDS read
//    (it cannot tell the ring slots apart), and the explicit vmcnt + barrier
//    are the synchronization.
// ---------------------------------------------------------------------------
constexpr int DBK = 64;           // K bytes per stage
constexpr int DEPI = 264;         // LDS row stride (bytes) of the epilogue staging

// LDS layout of a stage tile (rows x four 16-byte K chunks), in 1 KB groups
// of 16 rows. Inside a group, row r takes the 64-byte quad dq(r) (a fixed
// permutation of the 16 rows) and chunk c the slot c ^ dh(r) of that quad.
// Two properties follow:
//  * a global_load_lds lane quad (4 consecutive lanes, 64 LDS bytes) holds
//    the 4 chunks of one row: each quad fetches 64 contiguous global bytes;
//  * the 16 pieces of every 16-lane phase of a 32x32x64 fragment read land
//    on 16 different 16-byte bank slots (for each lane-phase grouping that
//    the bank-conflict counter is consistent with), so reads are
//    conflict-free.
__device__ __forceinline__ int dq(int r) {   // row -> quad (local bits)
  return (r & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 3);
}
__device__ __forceinline__ int dq_inv(int q) {  // quad -> local row
  return (q & 1) | (((q >> 2) & 1) << 1) | (((q >> 3) & 1) << 2) | (((q >> 1) & 1) << 3);
}
__device__ __forceinline__ int dh(int r) {   // chunk permutation of row r
  return (((r >> 1) ^ (r >> 4)) & 1) | (((r >> 2) & 1) << 1);
}
__device__ __forceinline__ int dlds_off(int row, int c) {
  return (row >> 4) * 1024 + ((dq(row & 15) << 2) + (c ^ dh(row))) * 16;
}


// BN: tile width (256 or 128); S: ring slots; WPC: workgroups per CU the
// register / LDS budget is sized for (two let one workgroup's MFMAs cover the
// other's barrier and memory waits).
// BLOCK (block variant, S odd): two 64-byte stages make one 128-wide scale
// group g, whose products count with the factor f_g = sx[m, g] * sw[nb, g]
// (nb = the wave's 128-row weight block). One accumulator carries the sum
// in units of the latest factor: before group g's first MFMAs the
// accumulator of row m is multiplied by f_{g-1} / f_g, and the epilogue
// multiplies by the last factor, so y = sum_g f_g P_g up to fp32 rounding
// (one rounding per group; a zero factor -- an all-zero group, whose codes
// and products are zero -- leaves the accumulator as it is). The
// activation scales of a group (256 tile rows) come into a 4-slot LDS ring
// with one 4-byte direct load per wave, issued on even steps two groups
// ahead (the same explicit wait counts cover them); the workgroup's weight
// block scales are copied to LDS once.
template <int BN, int S, int WPC, bool BLOCK>
__global__ __launch_bounds__(256, WPC) void gemm_prefill_deep_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int BM = 256;
  constexpr int DTM = 128, DTN = BN / 2;          // wave tile (m, n)
  constexpr int DMJ = DTM / 32, DNI = DTN / 32;   // 32x32 blocks per wave
  constexpr int DXQ = BM / 64, DWQ = BN / 64;     // 16-row load groups / wave / stage
  constexpr int DLPS = DXQ + DWQ;                 // loads per wave per stage
  constexpr int STAGE = (BM + BN) * DBK;
  constexpr int XB = BM * DBK;  // W tile offset inside a stage
  constexpr int RING = S * STAGE;                 // block variant: scale areas follow
  constexpr int EPI = DTN * 2 + 8;                // LDS row stride of the epilogue staging
  static_assert(!BLOCK || (S & 1) == 1, "block variant: S odd");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int group = GM * tiles_n;
  const int first_m = (bid / group) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_g = bid % group;
  const int m0 = (first_m + in_g % gm) * BM;
  const int n0 = (in_g / gm) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, kh = lane >> 5;

  // lane l of a load writes LDS byte 16*l of 1 KB group g (rows 16g..16g+15):
  // quad l / 4 = row 16g + dq_inv(l / 4), slot l % 4 = chunk (l % 4) ^ dh(row)
  uint32_t goff[DLPS];  // X groups first, then W groups
#pragma unroll
  for (int q = 0; q < DLPS; ++q) {
    const bool isx = q < DXQ;
    const int g = (isx ? q : q - DXQ) * 4 + wave;
    const int row = 16 * g + dq_inv(lane >> 2);
    const int c = (lane & 3) ^ dh(row);
    const int grow = isx ? min(m0 + row, M - 1) : min(n0 + row, N - 1);
    goff[q] = (uint32_t)grow * (uint32_t)K + (uint32_t)(c * 16);
  }
  const int KT = K / DBK;  // even: K is a multiple of 128
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;
  const int G = K / 128;                          // scale groups
  float* sxs = reinterpret_cast<float*>(smem + RING);          // [4][256]
  float* sws = reinterpret_cast<float*>(smem + RING + 4096);   // [BN/128][G]
  // activation scales of group g (tile rows 64*wave .. +63) -> slot g & 3
  const uint32_t sxoff =
      (uint32_t)min(m0 + 64 * wave + lane, M - 1) * (uint32_t)G * 4u;
  auto issue_sx = [&](int g) {
    g = min(max(g, 0), G - 1);
    dma4(sx, sxoff + (uint32_t)g * 4u,
         lds0 + (uint32_t)(RING + (g & 3) * 1024 + 256 * wave));
  };
  if constexpr (BLOCK) {  // the tile's BN/128 weight blocks (N % 128 == 0)
    const float* swr = sw + (int64_t)(n0 / 128) * G;
    for (int g = tid; g < (BN / 128) * G; g += 256) sws[g] = swr[g];  // published by the prologue barrier
  }
  // Load q (0 .. DLPS-1) of K step min(kt, KT-1) into ring slot kt % S. Past
  // the end the last step is loaded again into a slot that is never read,
  // which keeps the number of loads in flight (and so every wait count)
  // constant.
  auto issue_at = [&](uint32_t slot, int kt, int q) {
    const bool isx = q < DXQ;
    const uint32_t sb = lds0 + slot + (isx ? 0 : XB) + ((isx ? q : q - DXQ) * 4 + wave) * 1024;
    const uint8_t* base = (isx ? qx : qw) + (size_t)min(kt, KT - 1) * DBK;
    dma16(base, goff[q], sb);
  };
  // byte offsets of the slot step kt+1 is read from and of the slot step
  // kt+S-1 is loaded into, advanced by one slot per step (no division)
  uint32_t rslot = (uint32_t)STAGE, wslot = (uint32_t)((S - 1) * STAGE);
  const int arow0 = wn * DTN + lr, brow0 = wm * DTM + lr;
  // one 16-byte half (h = 0: chunk 2*kh, 1: chunk 2*kh+1) of a fragment
  // Fragment f of a step sits at a per-lane base + 2048 * f: rows 32 apart
  // share their low 5 bits, so the in-group permutation is the same. One
  // address add per operand half and step; the rest are immediate offsets.
  const uint32_t oA0 = XB + dlds_off(arow0, 2 * kh), oA1 = XB + dlds_off(arow0, 2 * kh + 1);
  const uint32_t oB0 = dlds_off(brow0, 2 * kh), oB1 = dlds_off(brow0, 2 * kh + 1);
  auto rd_at = [&](v8i& f, const uint8_t* p, int h) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    f[4 * h + 0] = v.x; f[4 * h + 1] = v.y; f[4 * h + 2] = v.z; f[4 * h + 3] = v.w;
  };
  // Read order of a step's fragments: A0, B0 .. B(DMJ-1), A1 .. A(DNI-1),
  // the order in which the next step's MFMAs first use them, so that every
  // fragment has many MFMAs between its read and its use.
  auto frag_of = [](int o) { return o == 0 ? 0 : (o <= DMJ ? DNI + o - 1 : o - DMJ); };
  auto read_frag = [&](v8i (&Af)[DNI], v8i (&Bf)[DMJ], uint32_t slot, int f, int h) {
    if (f < DNI) rd_at(Af[f], smem + slot + (h ? oA1 : oA0) + 2048 * f, h);
    else rd_at(Bf[f - DNI], smem + slot + (h ? oB1 : oB0) + 2048 * (f - DNI), h);
  };

  v16f acc[DNI][DMJ];
#pragma unroll
  for (int i = 0; i < DNI; ++i)
#pragma unroll
    for (int j = 0; j < DMJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  float fcur[DMJ];  // block variant: factor the accumulator is counted in
#pragma unroll
  for (int j = 0; j < DMJ; ++j) fcur[j] = 0.f;

  // prologue: steps 0 .. S-2 in flight; step 0 published and read. In the
  // block variant, the load issues of the prologue's steps stand for issue
  // steps -(S-1) .. -1; the even ones carry a scale load too (group 0), so
  // that every steady-state wait count below holds from the first step.
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    if constexpr (BLOCK) {  // virtual even issue steps -4, -2: groups 0, 1
      if (((s - (S - 1)) & 1) == 0) issue_sx((s - (S - 1)) / 2 + 2);
    }
#pragma unroll
    for (int q = 0; q < DLPS; ++q) issue_at((uint32_t)(s * STAGE), s, q);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * DLPS));
  __syncthreads();
  v8i A[2][DNI], B[2][DMJ];
#pragma unroll
  for (int r = 0; r < 2 * (DNI + DMJ); ++r) read_frag(A[0], B[0], 0u, frag_of(r >> 1), r & 1);

  // Step kt: wait until step kt+1 has landed (S-3 newer steps may still be
  // in flight), publish it with the barrier (which also frees the slot step
  // kt-1 used), then issue step kt's MFMAs in a fixed order, each paired
  // with one 16-byte fragment read of step kt+1 and the first ones with one
  // refill load of step kt+S-1. Scheduling barriers keep that interleave:
  // the LDS latency of every read hides under the MFMAs of the current step.
  constexpr int NM = DNI * DMJ;          // MFMAs per step
  constexpr int NR = 2 * (DNI + DMJ);    // fragment halves per step
  constexpr int RPM = (NR + NM - 1) / NM;  // fragment reads per MFMA slot
  static_assert(RPM <= 2 && DLPS <= NM, "at most two reads / one load per MFMA");
  // loads issued after step kt+1's: S-3 steps, plus (block) one scale load
  // for every even step among them
  constexpr int WAITN = (S - 3) * DLPS + (BLOCK ? (S - 3) / 2 : 0);
  // Per-channel variant (S = 5): the loads go out in pairs on odd steps kt,
  // for steps kt+3 and kt+4, each 16-row group's two 64-byte halves of the
  // same 128-byte lines back to back, so that the second request of a line
  // meets the first one in flight instead of fetching the line again. Wait
  // counts: at even kt the pair issued at kt-1 (2*DLPS loads) may still be
  // in flight; at odd kt only the last load of the pair holding kt+1.
  constexpr bool PAIRED = !BLOCK && S == 5;
  constexpr int WAIT_EVEN = PAIRED ? 2 * DLPS : WAITN;
  constexpr int WAIT_ODD = PAIRED ? 1 : WAITN;
  // block variant: factor of group g for this lane's rows, and the rescale
  // of the accumulator from the previous factor to it
  auto group_rescale = [&](int g, float (&rho)[DMJ]) {
    const float* sl = sxs + (g & 3) * 256 + wm * DTM + lr;
    const float swg = sws[wn * (DTN / 128) * G + g];
#pragma unroll
    for (int j = 0; j < DMJ; ++j) {
      const float f = sl[32 * j] * swg;
      const bool live = f != 0.0f;
      rho[j] = live ? fcur[j] / f : 1.0f;
      fcur[j] = live ? f : fcur[j];
    }
  };
  auto step = [&](int kt, auto cur_c, auto more_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool more = decltype(more_c)::value;
    if (more) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(cur == 0 ? WAIT_EVEN : WAIT_ODD));
      // A bare barrier: the LDS data is published by each wave's own vmcnt
      // wait, and every wave has waited (lgkmcnt) for its reads of the slot
      // about to be refilled before the MFMAs that used them, so the
      // lgkmcnt(0) of __syncthreads() would only stall the matrix core.
      asm volatile("s_barrier" ::: "memory");
    }
    // block variant, first stage of group g = kt/2: rescale to f_g
    float rho[DMJ];
    if constexpr (BLOCK && cur == 0) {
      group_rescale(kt / 2, rho);
      if (more) issue_sx(kt / 2 + 2);   // two groups ahead of its first stage
    }
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      if (more) {
#pragma unroll
        for (int u = 0; u < RPM; ++u) {
          const int r = t * RPM + u;
          if (r < NR) read_frag(A[cur ^ 1], B[cur ^ 1], rslot, frag_of(r >> 1), r & 1);
        }
        if constexpr (PAIRED) {
          if (cur == 1 && t < 2 * DLPS) {
            const uint32_t ws3 = wslot == 0u ? (uint32_t)((S - 1) * STAGE) : wslot - STAGE;
            if ((t & 1) == 0) issue_at(ws3, kt + 3, t >> 1);
            else issue_at(wslot, kt + 4, t >> 1);
          }
        } else {
          if (t < DLPS) issue_at(wslot, kt + S - 1, t);
        }
      }
      const int i = t / DMJ, j = t % DMJ;
      if constexpr (BLOCK && cur == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= rho[j];
      }
      acc[i][j] = mfma_e4m3_32x32x64(A[cur][i], B[cur][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    rslot = rslot + STAGE == (uint32_t)(S * STAGE) ? 0u : rslot + STAGE;
    wslot = wslot + STAGE == (uint32_t)(S * STAGE) ? 0u : wslot + STAGE;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // The first two steps are peeled: the loop is then entered only from code
  // identical to its own back edge, and the compiler keeps its LDS waits at
  // the loop head partial instead of draining every read.
  if (KT >= 4) {
    step(0, I0(), std::true_type());
    step(1, I1(), std::true_type());
    for (int kt = 2; kt < KT - 2; kt += 2) {
      step(kt, I0(), std::true_type());
      step(kt + 1, I1(), std::true_type());
    }
  }
  step(KT - 2, I0(), std::true_type());
  step(KT - 1, I1(), std::false_type());
  // no load may still be writing this workgroup's LDS when it retires
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // ---- epilogue: scale, round to bf16, stage through LDS, coalesced store --
  // Each wave writes its DTM x DTN bf16 block to its own LDS area (row stride
  // DEPI bytes: 8-byte writes from 32 consecutive rows fall on distinct
  // banks), then stores it row-wise, 16 bytes per lane: every store
  // instruction covers whole 256-byte row segments.
  // The per-channel epilogue's scales: one sx row and one sw column per
  // thread, loaded here (their latency overlaps the drain above and the
  // barrier below), then shared through LDS past the staging area; a global
  // load per column group with a wait after each would cost a memory round
  // trip each.
  constexpr int SCL = 4 * DTM * EPI;   // byte offset of the scale area
  static_assert(SCL + 4 * (BM + BN) <= RING, "scale area inside the ring");
  float sxv = 0.f, swv = 0.f;
  if constexpr (!BLOCK) {
    sxv = sx[min(m0 + tid, M - 1)];
    if (tid < BN) swv = sw[min(n0 + tid, N - 1)];
  }
  __syncthreads();  // every wave is done reading the ring
  float* scl = reinterpret_cast<float*>(smem + SCL);   // sx [BM] then sw [BN]
  if constexpr (!BLOCK) {
    scl[tid] = sxv;
    if (tid < BN) scl[BM + tid] = swv;
    __syncthreads();
  }
  uint8_t* ep = smem + wave * (DTM * EPI);
#pragma unroll
  for (int j = 0; j < DMJ; ++j) {
    const int ml = 32 * j + lr;
    const float sm = BLOCK ? fcur[j] : scl[wm * DTM + ml];
#pragma unroll
    for (int i = 0; i < DNI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 32 * i + 8 * q + 4 * kh;
        uint2 pk;
        if constexpr (BLOCK) {  // sum counted in units of the last factor
          pk.x = pack_bf16x2(acc[i][j][4 * q + 0] * sm, acc[i][j][4 * q + 1] * sm);
          pk.y = pack_bf16x2(acc[i][j][4 * q + 2] * sm, acc[i][j][4 * q + 3] * sm);
        } else {
          const float4 s4 = *reinterpret_cast<const float4*>(scl + BM + wn * DTN + nl);
          pk.x = pack_bf16x2(acc[i][j][4 * q + 0] * sm * s4.x, acc[i][j][4 * q + 1] * sm * s4.y);
          pk.y = pack_bf16x2(acc[i][j][4 * q + 2] * sm * s4.z, acc[i][j][4 * q + 3] * sm * s4.w);
        }
        *reinterpret_cast<uint2*>(ep + ml * EPI + nl * 2) = pk;
      }
    }
  }
  constexpr int SEGS = DTN / 8;                  // 16-byte segments per row
  constexpr int RPI = 64 / SEGS;                 // rows per store instruction
  const int rsub = lane / SEGS, cseg = lane % SEGS;
  const int nbase = n0 + wn * DTN + 8 * cseg;
  const bool vec_ok = (N & 7) == 0 && nbase + 7 < N;
#pragma unroll 4
  for (int t = 0; t < DTM / RPI; ++t) {
    const int ml = RPI * t + rsub;
    const int m = m0 + wm * DTM + ml;
    const uint8_t* src = ep + ml * EPI + cseg * 16;
    const uint2 lo = *reinterpret_cast<const uint2*>(src);
    const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
    if (m < M) {
      uint16_t* out = y + (int64_t)m * N + nbase;
      if (vec_ok) {
        *reinterpret_cast<uint4*>(out) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        const uint32_t w4[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (nbase + e < N) out[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

template <int BN, int S, int WPC, bool BLOCK = false>
void launch_deep(const uint8_t* qx, const float* sx, const uint8_t* qw,
                 const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                 hipStream_t st) {
  constexpr int ring = S * (256 + BN) * DBK;
  constexpr int stage_out = 4 * 128 * (BN + 8);  // epilogue staging, 4 waves
  constexpr int smem_max = (BLOCK ? ring + 4096 + 4 * 1024 * (BN / 128) : ring);
  constexpr int smem_cap = smem_max > stage_out ? smem_max : stage_out;
  static_assert(smem_cap * WPC <= 160 * 1024, "LDS budget");
  // block variant: + activation-scale ring (4 KB) + the weight block scales
  const int smem_need = BLOCK ? ring + 4096 + (int)((K / 128) * 4 * (BN / 128)) : ring;
  const int smem = smem_need > stage_out ? smem_need : stage_out;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_prefill_deep_kernel<BN, S, WPC, BLOCK>),
        hipFuncAttributeMaxDynamicSharedMemorySize, smem_cap);
  });
  const int tiles_m = (int)((M + 255) / 256);
  const int tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_prefill_deep_kernel<BN, S, WPC, BLOCK>),
                     dim3((unsigned)(tiles_m * tiles_n)), dim3(256), smem, st, qx, sx, qw,
                     sw, (uint16_t*)y, (int)M, (int)N, (int)K, tiles_m, tiles_n);
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
  // them when they still fill the 256 CUs at least once.
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
#if defined(FP8DQ_TILE_OVERRIDE) && FP8DQ_TILE_OVERRIDE == 1
  const bool use_big = true;
#elif defined(FP8DQ_TILE_OVERRIDE) && FP8DQ_TILE_OVERRIDE == 2
  const bool use_big = false;
#else
  const bool use_big = big >= 256;
#endif
  if (block) {
    // deep kernel: 32-bit scale offsets and at most 1024 scale groups
    const bool deep_ok = K <= 131072 && (uint64_t)M * (uint64_t)(K / 128) * 4u < (1ull << 32);
#if defined(FP8DQ_BLOCK_OLD)
    const bool deep = false;
#else
    const bool deep = deep_ok;
#endif
    if (deep && K >= 256) {
      launch_gemm_line_block(qx, sx, qw, sw, y, M, N, K, st);
    } else if (deep) {
      launch_deep<128, 5, 1, true>(qx, sx, qw, sw, y, M, N, K, st);
    }
    else if (use_big) launch_cfg<256, 256, true>(qx, sx, qw, sw, y, M, N, K, st);
    else launch_cfg<256, 128, true>(qx, sx, qw, sw, y, M, N, K, st);
  } else {
#if defined(FP8DQ_TILE_OVERRIDE) && FP8DQ_TILE_OVERRIDE == 3
    launch_deep<128, 4, 1>(qx, sx, qw, sw, y, M, N, K, st);
#elif defined(FP8DQ_TILE_OVERRIDE) && FP8DQ_TILE_OVERRIDE == 4
    launch_deep<128, 6, 1>(qx, sx, qw, sw, y, M, N, K, st);
#elif defined(FP8DQ_TILE_OVERRIDE) && FP8DQ_TILE_OVERRIDE == 5
    launch_deep<256, 4, 1>(qx, sx, qw, sw, y, M, N, K, st);
#else
    if (use_big && K >= 256) {
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
    }
    else if (use_big) launch_deep<256, 5, 1>(qx, sx, qw, sw, y, M, N, K, st);
    else launch_cfg<256, 128, false>(qx, sx, qw, sw, y, M, N, K, st);
#endif
  }
}

}  // namespace fp8dq
