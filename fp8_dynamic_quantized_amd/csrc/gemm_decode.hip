// Decode (small-M) FP8 GEMM for gfx950: the weight stream is the cost.
//
// Same contraction and epilogue as the prefill kernels (FP8 dynamic
// quantization table on the Llama-3.1-8B-Instruct-FP8-Dynamic page; block
// table on the Llama-3.2-3B-Instruct-FP8-Block page), for M <= 64 tokens,
// where every weight byte is used by at most 64 rows and the layer is bound
// by reading W from HBM (the 70B page's section 3 notes that the FP8 gain
// comes from moving half the bytes).
//
// Two kernels, by token count:
//  * up to 4 rows, gemm_decode_kernel: a workgroup owns 16 weight rows and
//    one K slice; its 4 waves take interleaved 128-byte K steps with a 4-deep
//    register prefetch of weight and token-row fragments (plain 16-byte
//    loads, bounded only by registers), and add their partial sums in a
//    fixed order through LDS;
//  * 5-64 rows, gemm_decode_line_kernel: 128 weight rows per workgroup
//    (32 per wave against every token row; at 49-64 rows each wave instead
//    takes its own 16 token rows against all 128 weight rows, which splits
//    a token fragment once per step instead of four times and cut the 70B
//    qkv linear at 64 tokens from 29.7 to 25.2 us); weights and the token
//    rows' codes move L2 -> LDS with
//    whole-line loads into a 3-slot ring, the token rows loaded once per
//    workgroup and shared by its waves. Every token row then costs 1/128 of
//    the weight bytes, against 1/16 in the register kernel, whose token-row
//    loads added 14-37 % to its time at 16 rows on the 70B linears. Each
//    workgroup starts its K slice at its own pair (a rotation by 7 pairs per
//    workgroup index) and wraps around.
//
// Accuracy. The FP8 matrix instruction adds its products in groups of 8
// consecutive K; inside a group every product is cut (toward zero) to a
// multiple of 2^(E-13), E the group's largest exponent sum e(x) + e(w). A
// token row's few large codes (outlier channels) then cut the other products
// of their groups. Here each token-row fragment is split into its codes of
// magnitude >= 16 and the rest, and the two halves go through two MFMAs into
// the same accumulator: a group's small products are then cut relative to
// small ones only. The split is exact (the halves have disjoint support) and
// costs one more MFMA and a few bit operations per step, which the weight
// stream mostly hides.
//
// Split K. When the row blocks alone leave the CUs short of work, K is
// split across the grid (grid.y). Each slice writes its fp32 partial tile to
// the workspace and counts itself on the tile's counter; the last slice to
// arrive adds all partials in slice order (so the result does not depend on
// the arrival order) and applies the epilogue, then clears the counter. The
// partials are written and read with the sc1 cache policy (as agent-scope
// atomic accesses are), so they reach the memory side of the per-XCD L2s,
// and every store has completed before its slice is counted (a relaxed
// agent-scope atomic add on the counter).
#include "device_common.hpp"
#include "kernels.hpp"

#include <atomic>
#include <mutex>

namespace fp8dq {
namespace {

constexpr int BK = 128;
constexpr int kDecD = 4;   // K steps of fragments in flight per wave (register kernel)

// s_waitcnt immediate: at most n vector-memory operations outstanding
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Token-row codes of magnitude >= 16 (exponent field >= 11, 0x58 with the
// sign cleared) go to `hi`, the others to `lo`; 4 codes per dword, no carry
// between bytes.
__device__ __forceinline__ void split_big(const v8i& b, v8i& lo, v8i& hi) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t v = (uint32_t)b[r];
    const uint32_t t = ((v & 0x7F7F7F7Fu) + 0x28282828u) & 0x80808080u;
    const uint32_t m = t | (t - (t >> 7));
    hi[r] = (int)(v & m);
    lo[r] = (int)(v ^ (v & m));
  }
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

__device__ __forceinline__ v8i gload_frag(const uint8_t* p) {
  const uint4 lo = ld16(p);
  const uint4 hi = ld16(p + 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Split-K partial tiles: every (tile, slice) owns a contiguous block of the
// workspace in the lanes' own order (16 bytes per lane and fragment), so a
// wave's store or load of a fragment is one coalesced 1 KB access. Stores and
// loads carry the sc1 cache policy (as agent-scope atomic accesses do): they
// reach the memory side of the per-XCD L2s, where another XCD's slice reads
// them.
constexpr int kSc1 = 16;   // cache-policy operand bit: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st_part(__amdgpu_buffer_rsrc_t r, uint32_t off, const v4f& v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)off, 0, kSc1);
}
__device__ __forceinline__ v4f ld_part(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSc1));
}

// y[m, n..n+3] = bf16(v * scales) (per-channel: v * (sx[m] * sw[n+r]), the
// scale product first, since v * sx[m] alone could pass fp32's range while y
// stays finite; block: v is already scaled); columns past N are not written.
template <bool BLOCK>
__device__ __forceinline__ void store_out(uint16_t* __restrict__ y, const float* __restrict__ sx,
                                          const float* __restrict__ sw, int m, int n, int N,
                                          const float (&s)[4]) {
  float v[4];
  const float sm = BLOCK ? 1.0f : sx[m];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = BLOCK ? s[r] : s[r] * (sm * sw[min(n + r, N - 1)]);
  uint16_t* out = y + (int64_t)m * N + n;
  if ((N & 3) == 0 && n + 3 < N) {
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

// ---------------------------------------------------------------------------
// Register-loading kernel (up to 4 token rows).
// ---------------------------------------------------------------------------
template <bool BLOCK>
__global__ __launch_bounds__(256) void gemm_decode_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, float* __restrict__ part, unsigned* __restrict__ cnt,
    int M, int N, int K, int kt_per_split) {
  constexpr int D = kDecD;
  __shared__ v4f red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int split = blockIdx.y, splits = gridDim.y;
  const int KT = K / BK;
  const int G = KT;
  const int kt0 = split * kt_per_split;
  const int kt1 = min(KT, kt0 + kt_per_split);

  // MFMA operand A: 16 weight rows; B: 16 token rows. Lanes of padding token
  // rows (lr >= M) get an offset past the buffer and load nothing; their
  // outputs are dropped. M * K < 2^31 on this path (M <= 4, K <= 2^17).
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)qx, (short)0, M * K, 0x00020000);
  const uint8_t* wp = qw + (int64_t)min(n0 + lr, N - 1) * K + kg * 32;
  const int xrow = min(lr, M - 1);
  const uint32_t xoff = lr < M ? (uint32_t)lr * (uint32_t)K + (uint32_t)(kg * 32) : 0x80000000u;

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  // K steps of this wave: kt0 + wave + 4 t, t = 0 .. cnt-1
  const int first = kt0 + wave;
  const int cntw = first < kt1 ? (kt1 - first + 3) / 4 : 0;

  v8i a[D], b[D];
  float sxr[D], swr[D];   // block: the step's group scales, loaded with it
  // (a step index past the row's end is clamped: the prologue loads D steps
  // without conditions, so the loop starts with a known number in flight)
  auto load = [&](int d, int t) {
    const int kt = min(first + 4 * t, KT - 1);
    const int64_t k0 = (int64_t)kt * BK;
    a[d] = gload_frag(wp + k0);
    b[d] = bload_frag(xrs, xoff + (uint32_t)k0);
    if (BLOCK) {
      sxr[d] = sx[(int64_t)xrow * G + kt];
      swr[d] = sw[(int64_t)(n0 >> 7) * G + kt];
    }
  };
  auto compute = [&](int d) {
    v8i lo, hi;
    split_big(b[d], lo, hi);
    if (BLOCK) {
      v4f p = mfma_e4m3_16x16x128(a[d], lo, v4f{0.f, 0.f, 0.f, 0.f});
      p = mfma_e4m3_16x16x128(a[d], hi, p);
      const float sc = sxr[d] * swr[d];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], sc, acc[r]);
    } else {
      acc = mfma_e4m3_16x16x128(a[d], lo, acc);
      acc = mfma_e4m3_16x16x128(a[d], hi, acc);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
  // Steady state: every step of a batch has a step D ahead to load, so the
  // body has no conditions and each step waits only for its own loads (the
  // compiler cannot count loads across the tail's conditions and waits for
  // all of them there, draining the D steps in flight).
  int t0 = 0;
  if (cntw >= D && cntw % D == 0) {
    // whole batches: the last one loads nothing, so its waits stay exact
    const int nb = cntw / D;
    for (int bt = 0; bt + 1 < nb; ++bt) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        compute(d);
        load(d, (bt + 1) * D + d);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) compute(d);
    t0 = cntw;
  }
  for (; t0 + 2 * D <= cntw; t0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(d);
      load(d, t0 + d + D);
    }
  }
  for (; t0 < cntw; t0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int t = t0 + d;
      if (t < cntw) {
        compute(d);
        if (t + D < cntw) load(d, t + D);
      }
    }
  }

  // ---- fixed-order reduction of the 4 waves' partial sums ----
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  v4f s = red[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const v4f o = red[w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] += o[r];
  }
  // D[n, m]: lane l holds n = n0 + 4 (l / 16) + r, m = l % 16
  const int n = n0 + 4 * kg, m = lr;
  const bool live = n < N && m < M;
  if (splits == 1) {
    if (live) {
      const float v[4] = {s[0], s[1], s[2], s[3]};
      store_out<BLOCK>(y, sx, sw, m, n, N, v);
    }
    return;
  }
  // split K: publish this slice's partial tile (1 KB, lane order), count it;
  // the last slice adds all slices' tiles in slice order
  float* tile = part + (int64_t)blockIdx.x * splits * 256;
  const __amdgpu_buffer_rsrc_t pr = part_rsrc(tile, (uint32_t)splits * 1024u);
  st_part(pr, (uint32_t)split * 1024u + (uint32_t)lane * 16u, s);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the partial's stores have completed
  unsigned old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__shfl(old, 0) != (unsigned)(splits - 1)) return;
  v4f t = ld_part(pr, (uint32_t)lane * 16u);
  for (int k = 1; k < splits; ++k) {
    const v4f o = ld_part(pr, (uint32_t)k * 1024u + (uint32_t)lane * 16u);
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] += o[r];
  }
  if (live) {
    const float v[4] = {t[0], t[1], t[2], t[3]};
    store_out<BLOCK>(y, sx, sw, m, n, N, v);
  }
  if (lane == 0)
    __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Whole-line decode kernel: 128 weight rows x (16 MB) token rows per
// workgroup, one 128-byte K step (a pair of 64-byte halves, or one scale
// group) per step, v_mfma_f32_16x16x128_f8f6f4.
//  * Weights and the token rows' codes move HBM/L2 -> LDS with whole-line
//    loads (8 rows x 128 bytes per instruction) into an LDS ring; the
//    codes of the token rows are loaded once per workgroup and shared by the
//    4 waves (each wave takes 32 weight rows).
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
// ---------------------------------------------------------------------------
constexpr int DL_BN = 128;               // weight rows per workgroup
constexpr int DL_NSL = 3;                // ring slots

__device__ __forceinline__ int dswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int MB, bool BLOCK, bool TW>
__global__ __launch_bounds__(256, 2) void gemm_decode_line_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, float* __restrict__ part, unsigned* __restrict__ cnt,
    int M, int N, int K, int kp_per_split) {
  constexpr int BMR = 16 * MB;                       // token rows (padded)
  constexpr int SLOT = (BMR + DL_BN) * BK + (BLOCK ? 512 : 0);  // + block scales
  constexpr int XB = BMR * BK;                       // weight part of a slot
  constexpr int SB = (BMR + DL_BN) * BK;             // block: sx [64] then sw [64]
  constexpr int XI = (2 * MB + 3) / 4;               // token-row loads per wave (>= 1)
  constexpr int WI = DL_BN / 32;                     // weight loads per wave
  constexpr int L = XI + WI + (BLOCK ? 1 : 0);
  // The WG's MFMA blocks: 8 weight fragments x MB token fragments (16 rows
  // each). A wave takes NWF weight fragments from W0 and NTF token fragments
  // from T0: two weight fragments against every token fragment, or (TW, 64
  // token rows) every weight fragment against its own token fragment, so
  // that each wave splits one token fragment a step instead of all four.
  static_assert(!TW || MB == 4, "token-row waves need 4 token fragments");
  constexpr int NWF = TW ? 8 : 2;
  constexpr int NTF = TW ? 1 : MB;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ unsigned last_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * DL_BN;
  const int W0 = TW ? 0 : 2 * wave, T0 = TW ? wave : 0;
  const int split = blockIdx.y, splits = gridDim.y;
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
  // block: wave 1 loads the weight-block scale of the group (every lane the
  // same value), the other waves the token rows' activation scales (the
  // same 64 values each)
  const uint32_t scoff = BLOCK
      ? (wave == 1 ? (uint32_t)(n0 >> 7) * (uint32_t)KP * 4u
                   : (uint32_t)min(lane, M - 1) * (uint32_t)KP * 4u)
      : 0u;
  // Pair p of the slice is its pair (p + rot) mod np. Workgroups that start
  // together on the same K offset read their 128 rows at addresses a
  // multiple of K apart at the same moment; spreading the starting offsets
  // over the slice measured 3-16 % faster on the 70B linears at 16-64
  // tokens (the multiplier 7 was the best of 1, 7 and 29 at 64 tokens).
  const int rot = (int)((blockIdx.x * 7u) % (unsigned)np);
  auto issue = [&](int p) {   // pair p of this slice (clamped) into slot p % DL_NSL
    int pq = min(p, np - 1) + rot;
    pq -= pq >= np ? np : 0;
    const int pc = p0 + pq;
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

  v4f acc[NWF][NTF];
#pragma unroll
  for (int i = 0; i < NWF; ++i)
#pragma unroll
    for (int j = 0; j < NTF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int q = 0; q < DL_NSL - 1; ++q) issue(q);
  for (int p = 0; p < np; ++p) {
    // pair p landed; the DL_NSL-2 newer pairs may still be in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((DL_NSL - 2) * L));
    asm volatile("s_barrier" ::: "memory");
    issue(p + DL_NSL - 1);
    const uint8_t* sb = smem + (p % DL_NSL) * SLOT;
    v8i a[NWF], bl[NTF], bh[NTF];
#pragma unroll
    for (int i = 0; i < NWF; ++i) a[i] = rd(sb + XB + 16 * (W0 + i) * BK);
#pragma unroll
    for (int j = 0; j < NTF; ++j) split_big(rd(sb + 16 * (T0 + j) * BK), bl[j], bh[j]);
    if constexpr (BLOCK) {   // the group's scales from the slot
      const float* scl = reinterpret_cast<const float*>(sb + SB);
      const float swg = scl[64];
#pragma unroll
      for (int j = 0; j < NTF; ++j) {
        const float f = scl[16 * (T0 + j) + fr] * swg;
#pragma unroll
        for (int i = 0; i < NWF; ++i) {
          v4f pr = mfma_e4m3_16x16x128(a[i], bl[j], v4f{0.f, 0.f, 0.f, 0.f});
          pr = mfma_e4m3_16x16x128(a[i], bh[j], pr);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], f, acc[i][j][r]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NWF; ++i)
#pragma unroll
        for (int j = 0; j < NTF; ++j) {
          acc[i][j] = mfma_e4m3_16x16x128(a[i], bl[j], acc[i][j]);
          acc[i][j] = mfma_e4m3_16x16x128(a[i], bh[j], acc[i][j]);
        }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may still target LDS

  // D[n, m]: lane l holds n = 16 i + 4 (l / 16) + r of the wave's rows, m = 16 j + l % 16
  if (splits == 1) {
#pragma unroll
    for (int i = 0; i < NWF; ++i) {
      const int n = n0 + 16 * (W0 + i) + 4 * kq;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < NTF; ++j) {
        const int m = 16 * (T0 + j) + fr;
        if (m >= M) continue;
        const float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        store_out<BLOCK>(y, sx, sw, m, n, N, v);
      }
    }
    return;
  }
  // split K: publish this slice's partial tile (lane order: [wave][i][j]
  // [lane] x 16 bytes), count it; the last slice adds all slices' tiles in
  // slice order
  constexpr uint32_t TILE_B = 4u * NWF * NTF * 1024u;   // bytes of one slice's tile
  float* tile = part + (int64_t)blockIdx.x * splits * (TILE_B / 4);
  const __amdgpu_buffer_rsrc_t pr = part_rsrc(tile, (uint32_t)splits * TILE_B);
  const uint32_t lo_off = (uint32_t)wave * NWF * NTF * 1024u + (uint32_t)lane * 16u;
#pragma unroll
  for (int i = 0; i < NWF; ++i)
#pragma unroll
    for (int j = 0; j < NTF; ++j)
      st_part(pr, (uint32_t)split * TILE_B + lo_off + (uint32_t)(i * NTF + j) * 1024u, acc[i][j]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's stores have completed
  __syncthreads();                            // ... and every other wave's
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(splits - 1);
  __syncthreads();
  if (!last_flag) return;
  // slice by slice, all of a slice's fragments in flight together (and the
  // next slice's issued before this one's adds): about one memory latency
  // per slice
  v4f nxt[NWF][NTF];
#pragma unroll
  for (int i = 0; i < NWF; ++i)
#pragma unroll
    for (int j = 0; j < NTF; ++j) acc[i][j] = ld_part(pr, lo_off + (uint32_t)(i * NTF + j) * 1024u);
  for (int k = 1; k < splits; ++k) {
#pragma unroll
    for (int i = 0; i < NWF; ++i)
#pragma unroll
      for (int j = 0; j < NTF; ++j)
        nxt[i][j] = ld_part(pr, (uint32_t)k * TILE_B + lo_off + (uint32_t)(i * NTF + j) * 1024u);
#pragma unroll
    for (int i = 0; i < NWF; ++i)
#pragma unroll
      for (int j = 0; j < NTF; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] += nxt[i][j][r];
  }
#pragma unroll
  for (int i = 0; i < NWF; ++i) {
    const int n = n0 + 16 * (W0 + i) + 4 * kq;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < NTF; ++j) {
      const int m = 16 * (T0 + j) + fr;
      if (m >= M) continue;
      const float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      store_out<BLOCK>(y, sx, sw, m, n, N, v);
    }
  }
  if (tid == 0)
    __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB, bool BLOCK, bool TW = false>
void launch_line_dec(const uint8_t* qx, const float* sx, const uint8_t* qw,
                     const float* sw, void* y, float* part, unsigned* cnt, int64_t M,
                     int64_t N, int64_t K, const DecodePlan& p, hipStream_t st) {
  constexpr int smem = DL_NSL * ((16 * MB + DL_BN) * BK + (BLOCK ? 512 : 0));
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_decode_line_kernel<MB, BLOCK, TW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  });
  const unsigned gx = (unsigned)((N + DL_BN - 1) / DL_BN);
  hipLaunchKernelGGL((gemm_decode_line_kernel<MB, BLOCK, TW>), dim3(gx, (unsigned)p.splits),
                     dim3(256), smem, st, qx, sx, qw, sw, (uint16_t*)y, part, cnt, (int)M,
                     (int)N, (int)K, p.kt_per_split);
}

template <bool BLOCK>
void launch_reg_dec(const uint8_t* qx, const float* sx, const uint8_t* qw,
                    const float* sw, void* y, float* part, unsigned* cnt, int64_t M,
                    int64_t N, int64_t K, const DecodePlan& p, hipStream_t st) {
  const unsigned gx = (unsigned)((N + 15) / 16);
  hipLaunchKernelGGL((gemm_decode_kernel<BLOCK>), dim3(gx, (unsigned)p.splits), dim3(256), 0,
                     st, qx, sx, qw, sw, (uint16_t*)y, part, cnt, (int)M, (int)N, (int)K,
                     p.kt_per_split);
}

// CUs of the current device, asked once per device (the plan runs on every
// call, and a decode linear takes 15-20 us)
int decode_cu_count() {
  constexpr int kDevs = 64;
  static std::atomic<int> cached[kDevs];   // 0: not asked yet
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kDevs) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu <= 0)
    return 256;
  if (dev >= 0 && dev < kDevs) cached[dev].store(ncu, std::memory_order_relaxed);
  return ncu;
}

}  // namespace

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, size_t ws_cap) {
  DecodePlan p;
  p.mb = (int)((M + 15) / 16);
  if (p.mb < 1) p.mb = 1;
  if (p.mb > 4) p.mb = 4;  // callers guarantee M <= 64 on this path

  const int64_t KT = K / BK;
  const int64_t ncu = decode_cu_count();
  // above 4 token rows, the whole-line kernel: on the 70B linears at 5-8
  // rows it was 1-11 % faster than the register kernel on qkv, gate_up and
  // down and 2-4 % slower on o; at 3 rows mixed (o 8 % slower); at 16 rows
  // 11-20 % faster (the register kernel's token-row loads grow with the rows)
  p.line = M > 4 ? 1 : 0;
  if (p.line) {
    // Whole-line kernel: 128 weight rows per workgroup (wg0 row blocks). K
    // is split so that the slices fill the CUs once: floor(CUs / wg0)
    // slices; up to 32 tokens on rows shorter than 16384, at most 3 where 3
    // already reach half the CUs; long rows (K >= 16384) with more than 32
    // tokens take two workgroups per CU. Measured on the 70B linears at
    // 12-64 tokens, forcing 1-12 slices: this picks the fastest count or one
    // within 2 % for qkv, o and down. A grid a little over one workgroup per
    // CU (qkv in 4 slices: 320) was the slowest after an unsplit K; o in 4
    // slices (16 K steps each) was 13 % slower than in 3 up to 32 tokens and
    // 6-12 % faster above; the 16 x 4096 -> 1024 linear (8 row blocks) was
    // 3 % slower in 3 slices than in 4.
    const int64_t wg0 = (N + DL_BN - 1) / DL_BN;
    int64_t sp = ncu / wg0;
    if (K >= 16384 && M > 32) sp = (2 * ncu) / wg0;
    if (K < 16384 && M <= 32 && sp > 3 && 3 * wg0 >= ncu / 2) sp = 3;
    if (sp < 1) sp = 1;
    if (sp > KT / 8) sp = KT / 8;
    if (sp < 1) sp = 1;
    const size_t tile_b = (size_t)DL_BN * 16 * p.mb * 4;
    while (sp > 1 && (wg0 > kDecodeMaxSplitTiles ||
                      kDecodeCounterBytes + (size_t)sp * (size_t)wg0 * tile_b > ws_cap))
      --sp;
    p.kt_per_split = (int)((KT + sp - 1) / sp);
    p.splits = (int)((KT + p.kt_per_split - 1) / p.kt_per_split);
    return p;
  }
  // Register kernel: 16 weight rows per workgroup. K is split only for long
  // rows (K >= 16384) with fewer row blocks than CUs, into the fewest slices
  // that give every CU one (at least 8 K steps each). Measured: on the 70B
  // linears at 1 and 8 tokens (512 to 3584 row blocks) 2 or 4 slices were
  // 0-13 % slower than none, and the 16-token 4096 -> 1024 linear (64 row
  // blocks, 32 K steps) took 12.6 us in 4 slices against 11.1 us unsplit.
  const int64_t RB = (N + 15) / 16;
  int64_t best_s = 1;
  while (K >= 16384 && RB * best_s < ncu && KT / (best_s * 2) >= 8 &&
         RB <= kDecodeMaxSplitTiles &&
         kDecodeCounterBytes + (size_t)(best_s * 2) * (size_t)RB * 1024u <= ws_cap)
    best_s *= 2;
  p.kt_per_split = (int)((KT + best_s - 1) / best_s);
  p.splits = (int)((KT + p.kt_per_split - 1) / p.kt_per_split);
  return p;
}

size_t decode_workspace_bytes(int64_t M, int64_t N, const DecodePlan& p) {
  if (p.splits <= 1) return 0;
  (void)M;
  // one partial tile per (tile, slice): 16 x 16 floats (register kernel) or
  // 128 x 16 mb floats (whole-line kernel)
  const size_t tiles = p.line ? (size_t)((N + DL_BN - 1) / DL_BN) : (size_t)((N + 15) / 16);
  const size_t tile_b = p.line ? (size_t)DL_BN * 16 * p.mb * 4 : (size_t)16 * 16 * 4;
  return kDecodeCounterBytes + (size_t)p.splits * tiles * tile_b;
}

void launch_gemm_decode(const uint8_t* qx, const float* sx, const uint8_t* qw,
                        const float* sw, void* y, void* ws, int64_t M,
                        int64_t N, int64_t K, bool block, const DecodePlan& p,
                        hipStream_t st) {
  unsigned* cnt = p.splits > 1 ? static_cast<unsigned*>(ws) : nullptr;
  float* part = p.splits > 1
      ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kDecodeCounterBytes)
      : nullptr;
  if (!p.line) {
    block ? launch_reg_dec<true>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st)
          : launch_reg_dec<false>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st);
    return;
  }
  switch (p.mb) {
    case 1: block ? launch_line_dec<1, true>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st)
                  : launch_line_dec<1, false>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st); break;
    case 2: block ? launch_line_dec<2, true>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st)
                  : launch_line_dec<2, false>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st); break;
    case 3: block ? launch_line_dec<3, true>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st)
                  : launch_line_dec<3, false>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st); break;
    default: block ? launch_line_dec<4, true, true>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st)
                   : launch_line_dec<4, false, true>(qx, sx, qw, sw, y, part, cnt, M, N, K, p, st); break;
  }
}

}  // namespace fp8dq
