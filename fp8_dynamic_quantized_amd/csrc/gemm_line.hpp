// Whole-line prefill GEMM kernels (gfx950), shared by the per-channel
// instantiation (gemm_prefill.hip) and the block instantiation
// (gemm_block.hip, built with the MFMA accumulators in ordinary VGPRs so the
// per-group rescale is a plain multiply).
//
// What is computed: Y[m,n] = bf16( sum_k val(qx[m,k]) val(qw[n,k]) * scales )
// (Y's rows ldy elements apart),
// per-token x per-channel scales (Llama-3.1-8B-Instruct-FP8-Dynamic page, FP8
// dynamic quantization table) or 128-wide activation groups x 128 x 128
// weight blocks (Llama-3.2-3B-Instruct-FP8-Block page, FP8 block
// quantization table).
#pragma once
#include "device_common.hpp"

#include <mutex>
#include <type_traits>

namespace fp8dq {
namespace line {
namespace {

// Tile rows per L2 band (see the tile order below). Fewer rows keep a band's
// X blocks in the XCD's 4 MB L2 while its W blocks stream through; measured
// against 8 rows, alternating builds on one box: per-channel with 4 rows, 8B
// o +6 %, down +3 %, gate_up +2 %; block with 2 rows, 3B gate_up +30 %
// (4 rows: +19 %; 1 row: +25 %), the other shapes within 1-3 %. With 64 or
// more tile rows (M >= 16384) per-channel bands of 3 rows: the 8B gate_up at
// M = 32768 +5 % against 4 rows (at M = 4096, 3 rows cost o 3 %).
template <bool BLOCK>
__device__ __forceinline__ int band_rows(int tiles_m) {
  return BLOCK ? 2 : (tiles_m >= 64 ? 3 : 4);
}
// block: odd-step MFMA slot at which the next group's factor is formed
constexpr int kGroupFactorAt = 2;
// s_waitcnt immediate (gfx9 encoding): at most n vector-memory operations of
// this wave outstanding (expcnt / lgkmcnt not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// ---------------------------------------------------------------------------
// Whole-line kernels: 256 x BN tiles (BN = 256 or 192 per-channel, 128 or 256
// block), v_mfma_f32_32x32x64_f8f6f4, 4 waves (2 x 2); 256 x 256 block tiles
// take 8 waves (2 x 4, two per SIMD), each with a 128 x 64 part.
//  * A load instruction moves 8 rows x 128 bytes (two 64-byte MFMA K steps of
//    each row): every request is a whole 128-byte line. The L2 -> LDS path
//    costs the same per line touched, so 64-byte row pieces (16 rows per
//    instruction) reached only half the bytes per cycle.
//  * LDS: NSL pair slots [X: 256 rows | W: BN rows], rows of 128 bytes whose
//    16-byte chunks are XOR-permuted by row bits 0-4 (conflict-free fragment
//    reads; fragments 32 rows apart sit at a constant distance); then the
//    scale areas, filled by 4-byte-per-lane direct loads.
//  * Step kt runs the MFMAs of K step kt while reading the fragments of step
//    kt+1 from LDS. Pairs are issued on odd steps: at step 2P+1 pair P+NSL
//    goes into the slot of pair P. Every wave has waited (lgkmcnt) for its
//    reads of that slot -- issued during step 2P, at the front of the step --
//    before the barrier of step 2P+1, so the refill never races a read. Odd
//    steps wait for the pair read next and hold the only barrier; even steps
//    read the second half of a pair that has already landed.
//  * Per-channel: NSL = 2 (two 64 KB slots), the tile's sx / sw in LDS.
//  * Block (128 x 128 weight blocks, 128-wide activation groups): NSL = 3
//    48 KB slots for 256 x 128 tiles, 2 x 64 KB for 256 x 256 ones; a pair
//    is exactly one scale group g, whose 256 activation
//    scales ride with the pair into a per-slot LDS ring, and the tile's
//    weight-block scales for every g are loaded once. One accumulator carries
//    the sum in units of the current factor f_g = sx[m,g] * sw[nb,g] (held
//    above 2^-64 of the largest factor so far and above 2^-126, so it never
//    overflows): it is multiplied by u_{g-1} / u_g before group g's first
//    MFMAs and by the last units at the end.
//    The next group's scales are read right after the odd step's barrier and
//    its factor is formed a few MFMAs later, so the matrix core does not
//    wait for those reads.
//  * Epilogue from registers: scale, round to bf16, and pair lanes l and l+32
//    with v_permlane32_swap so each lane holds 16 contiguous bytes. In a tile
//    with no ragged edge, v_permlane16_swap and a DPP row rotation then
//    regroup two 32-column fragments so that each store instruction writes
//    8 rows x 128 bytes (whole lines) with the non-temporal hint: Y (a round
//    of tiles writes about one L2 of it per XCD) then streams past the L2
//    instead of evicting X and W. Whole lines without the hint, or the hint
//    on 32-byte row pieces, gained nothing or lost.
//  * A workgroup may walk several tiles (blockIdx.x, + gridDim.x, ...): after
//    a tile's last step and one barrier, the next tile's scales (other
//    buffer) and first NSL pairs are issued, so they load during this tile's
//    epilogue. Values derived from the lane index are re-derived where a tile
//    starts and in the epilogue rather than kept in registers across it: the
//    epilogue needs nearly all of them, and a spilled value would bring
//    scratch loads (and the compiler's waits for them) into the load pipeline.
//    The fragment offsets live from a tile's start to its last step
//    (per-channel; the 8-wave block kernel re-derives them per step, where
//    keeping them made it spill): that took the K loop from 39 to 8 VALU
//    instructions per pair, and 8B qkv, gate_up and down 3-5 % faster.
// ---------------------------------------------------------------------------
constexpr int LBK = 128;                 // K bytes per pair (two MFMA steps)

template <bool BLOCK, int BNP>
struct LineCfg {
  static constexpr int BM = 256, BN = BNP;
  // waves: 2 x 2; 256-wide block tiles take 2 x 4 (two waves per SIMD, each
  // with the same 128 x 64 part as in a 256 x 128 tile)
  static constexpr int NW = (BLOCK && BNP == 256) ? 8 : 4;
  static constexpr int NSL = (BLOCK && BNP == 128) ? 3 : 2; // pair slots
  static constexpr int SLOT = (BM + BN) * LBK;
  static constexpr int XQ = BM / (8 * NW), WQ = BN / (8 * NW);  // loads per wave per pair
  static constexpr int NLD = XQ + WQ;
  static constexpr int NBLK = BLOCK ? BN / 128 : 0;         // weight blocks across a tile
  static constexpr int SC = NSL * SLOT;                     // scale areas
  // per-channel: two tile-scale buffers [sx 256 | sw 256] (this tile's and
  // the next one's); block: the sx ring NSL x [256], then two buffers of a
  // tile's weight-block scales [NBLK][G], loaded in 64-entry chunks
  static constexpr int SWB = SC + (BLOCK ? NSL * 1024 : 2 * 2048);
  __host__ __device__ static int swsz(int K) {
    return BLOCK ? NBLK * ((K / 128 + 63) / 64) * 256 : 0;
  }
  static size_t smem(int64_t K) { return (size_t)SWB + 2 * (size_t)swsz((int)K); }
};

__device__ __forceinline__ int lswz(int row) { return (row & 7) ^ ((row >> 3) & 3); }

__device__ __forceinline__ uint32_t pk_bf16_rne(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <bool BLOCK, int BNP>
__global__ __launch_bounds__((64 * LineCfg<BLOCK, BNP>::NW), 1) void gemm_prefill_line_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K, int ldy, int tiles_m, int tiles_n) {
  using C = LineCfg<BLOCK, BNP>;
  static_assert(BLOCK ? (BNP == 128 || BNP == 256) : (BNP == 256 || BNP == 192),
                "tile widths built");
  constexpr int BM = C::BM, BN = C::BN, NSL = C::NSL, SLOT = C::SLOT, NW = C::NW;
  constexpr int XQ = C::XQ, WQ = C::WQ, NLD = C::NLD;
  constexpr int DTM = 128, DTN = BN / (NW / 2);
  constexpr int DMJ = DTM / 32, DNI = DTN / 32;   // 32-row fragments per wave (m, n)
  constexpr int NM = DNI * DMJ;                   // MFMAs per step
  constexpr int NR = 2 * (DNI + DMJ);             // fragment halves per step
  constexpr int RPE = (NR + NM - 1) / NM;         // reads per MFMA slot, odd steps
  constexpr int NSC = BLOCK ? 1 : 0;              // scale loads per pair
  constexpr int XB = BM * LBK;                    // W part of a slot
  static_assert(2 * NM >= NR, "even steps read two halves per MFMA");
  constexpr int IPS = (NLD + NSC + NM - 1) / NM;  // loads issued per MFMA slot, odd steps
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int ntiles = tiles_m * tiles_n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;
  const int G = K / 128;                          // pairs = scale groups
  const int SWSZ = C::swsz(K);

  // Tile v -> origin. Consecutive workgroup ids go to the 8 XCDs in turn;
  // v is remapped so that XCD x works through one contiguous range of tiles,
  // ordered in bands of GM tile rows that share X and W in its L2. A
  // workgroup takes tiles blockIdx.x, + gridDim.x, ... (gridDim.x a multiple
  // of 8 or the tile count), so round k of every workgroup covers the same
  // tiles as a one-tile-per-workgroup launch would.
  auto lane_now = []() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  auto origin = [&](int v, int& m0, int& n0) {
    int bid = v;
    if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
    const int GM = band_rows<BLOCK>(tiles_m);
    const int group = GM * tiles_n;
    const int first_m = (bid / group) * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_g = bid % group;
    m0 = (first_m + in_g % gm) * BM;
    n0 = (in_g / gm) * BN;
  };

  // Loads: groups of 8 rows; wave w takes groups NW q + w. Lane l covers row
  // 8g + l/8 and LDS chunk slot l%8, i.e. global chunk (l%8) ^ lswz(row)
  // = (l%8) ^ (l/8) ^ (w%4) (independent of q).
  // operand offsets of the current tile
  uint32_t rowX[XQ], rowW[WQ];
  uint32_t sxoff = 0u;   // block: this wave's 64 rows of activation scales
  int m0, n0;
  // (the lane index is re-derived where a tile starts and in the epilogue,
  // so nothing derived from it stays in registers across the K loop)
  auto set_tile = [&](int v) {
    origin(v, m0, n0);
    const int ln = lane_now();
    const int r8 = 8 * wave + (ln >> 3);
    const uint32_t cc = (uint32_t)(((ln & 7) ^ (ln >> 3) ^ (wave & 3)) << 4);
    // 24-bit multiplies (rows and K are below 2^24: K by the size rules,
    // rows because rows x K stays below 2^32 with K >= 256): 32-bit results,
    // where a full multiply-add would hold a 64-bit register pair
#pragma unroll
    for (int q = 0; q < XQ; ++q)
      rowX[q] = __umul24((uint32_t)min(m0 + 8 * NW * q + r8, M - 1), (uint32_t)K) + cc;
#pragma unroll
    for (int q = 0; q < WQ; ++q)
      rowW[q] = __umul24((uint32_t)min(n0 + 8 * NW * q + r8, N - 1), (uint32_t)K) + cc;
    // block: 64 rows of activation scales per wave (waves 4-7 repeat 0-3)
    sxoff = BLOCK ? (uint32_t)min(m0 + 64 * (wave & 3) + ln, M - 1) * (uint32_t)G * 4u : 0u;
  };
  int v = blockIdx.x;
  set_tile(v);
  int par = 0;   // tile-scale buffer of the current tile

  // tile-level scales of the tile at (tm0, tn0) into buffer b
  auto tile_scales = [&](int tm0, int tn0, int b) {
    const int lane = lane_now();
    if constexpr (BLOCK) {
      // the scales of the tile's NBLK weight blocks for every group, in
      // chunks of 64 groups (a block past N, in a ragged last tile, repeats
      // the last one; its columns are not stored)
      const int nch = (G + 63) / 64;
      for (int c = wave; c < C::NBLK * nch; c += NW) {
        const int blk = min(tn0 / 128 + c / nch, N / 128 - 1);
        dma4(sw, (uint32_t)(blk * G + min(64 * (c % nch) + lane, G - 1)) * 4u,
             lds0 + C::SWB + (uint32_t)(b * SWSZ + 256 * c));
      }
    } else {
      // 64 sx (rows) and 64 sw (columns) per wave
      const uint32_t sb = lds0 + C::SC + (uint32_t)(b * 2048);
      dma4(sx, (uint32_t)min(tm0 + 64 * wave + lane, M - 1) * 4u, sb + 256 * wave);
      dma4(sw, (uint32_t)min(tn0 + 64 * wave + lane, N - 1) * 4u, sb + 1024 + 256 * wave);
    }
  };
  // load u of pair p (clamped to the last one: past the end the re-load
  // keeps every wait count constant) into slot index si
  auto issue = [&](int si, int p, int u) {
    const int pc = min(p, G - 1);
    if (u < NLD) {
      const size_t koff = (size_t)pc * LBK;
      const uint32_t sb = lds0 + (uint32_t)(si * SLOT);
      if (u < XQ) dma16(qx + koff, rowX[u], sb + (uint32_t)((NW * u + wave) * 1024));
      else dma16(qw + koff, rowW[u - XQ], sb + XB + (uint32_t)((NW * (u - XQ) + wave) * 1024));
    } else if (BLOCK && u == NLD) {
      dma4(sx, sxoff + (uint32_t)pc * 4u, lds0 + C::SC + (uint32_t)(si * 1024 + 256 * (wave & 3)));
    }
  };
  // a tile's scales and pairs 0 .. NSL-1 into slots s0, s0+1, ...
  auto prologue = [&](int s0) {
    tile_scales(m0, n0, par);
#pragma unroll
    for (int pp = 0; pp < NSL; ++pp) {
      const int si = (s0 + pp) % NSL;
#pragma unroll
      for (int u = 0; u < NLD + NSC; ++u) issue(si, pp, u);
    }
  };

  // fragment offsets within a slot: row r = base + 32 f, chunk c =
  // 4 par + 2 kh + h (formed where they are used: a few instructions per
  // step, no registers held across a tile's epilogue)
  using Offs = uint32_t[2][2];
  auto frag_offsets = [&](Offs& oA, Offs& oB) {
    const int ln = lane_now();
    const int flr = ln & 31, fkh = ln >> 5;
    const int arow0 = wn * DTN + flr, brow0 = wm * DTM + flr;
    const int sz = lswz(flr);
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = (4 * pr + 2 * fkh + h) ^ sz;
        oA[pr][h] = (uint32_t)(XB + arow0 * LBK + (c << 4));
        oB[pr][h] = (uint32_t)(brow0 * LBK + (c << 4));
      }
  };
  auto rd_at = [&](v8i& f, const uint8_t* p, int h) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    f[4 * h + 0] = q.x; f[4 * h + 1] = q.y; f[4 * h + 2] = q.z; f[4 * h + 3] = q.w;
  };
  // read order A0, B0 .. B(DMJ-1), A1 .. : the order of first use
  auto frag_of = [](int o) { return o == 0 ? 0 : (o <= DMJ ? DNI + o - 1 : o - DMJ); };
  auto read_frag = [&](const Offs& oA, const Offs& oB, v8i (&Af)[DNI], v8i (&Bf)[DMJ],
                       int si, int pr, int f, int h) {
    const uint8_t* base = smem + si * SLOT;
    if (f < DNI) rd_at(Af[f], base + oA[pr][h] + 4096 * f, h);
    else rd_at(Bf[f - DNI], base + oB[pr][h] + 4096 * (f - DNI), h);
  };

  v16f acc[DNI][DMJ];
  // block: factor the accumulator is counted in, per row j, the largest
  // factor so far, and the rescale for the next group (formed one step ahead)
  float fcur[DMJ], fmax[DMJ], rho[DMJ];
#pragma unroll
  for (int j = 0; j < DMJ; ++j) { fcur[j] = 0.f; fmax[j] = 0.f; rho[j] = 1.f; }
  // group g's scales of this lane's rows, read from LDS (gsx, gsw) ...
  float gsx[DMJ], gsw = 0.f;
  auto group_scales = [&](int g, int si) {
    const int lr = lane_now() & 31;
    const float* sxs = reinterpret_cast<const float*>(smem + C::SC + si * 1024);
    // this wave's 64 columns lie in weight block (wn * DTN) / 128 of the tile
    const int blk = (wn * DTN) / 128;
    gsw = reinterpret_cast<const float*>(smem + C::SWB + par * SWSZ)[blk * ((G + 63) / 64) * 64 +
                                                                     min(g, G - 1)];
#pragma unroll
    for (int j = 0; j < DMJ; ++j) gsx[j] = sxs[wm * DTM + 32 * j + lr];
  };
  // ... and f_g -> rho and the next units (formed later, so the reads'
  // latency is hidden). The accumulator counts in units
  //   u_g = max(f_g, 2^-64 * (largest factor so far), 2^-126):
  // the ratio u_{g-1} / u_g then stays below 2^65 and rcp never sees a
  // subnormal, so the carried sum stays below 2^98 whatever the scales
  // (zero groups, factors below the fp32 range, drops of any size). A group
  // whose factor lies below the floor is weighted by u_g instead of f_g; its
  // share of y then errs by at most 2^24 * 2^-64 of the largest factor, far
  // below the fp32 rounding of the largest group's own share. gsx[j] is
  // replaced by u_g.
  auto group_factor = [&]() {
#pragma unroll
    for (int j = 0; j < DMJ; ++j) {
      const float f = gsx[j] * gsw;
      fmax[j] = __builtin_fmaxf(fmax[j], f);
      const float u = __builtin_fmaxf(__builtin_fmaxf(f, fmax[j] * 0x1p-64f), 0x1p-126f);
      rho[j] = fcur[j] * __builtin_amdgcn_rcpf(u);
      gsx[j] = u;
    }
  };

  int cs = 0;  // slot index of the pair the current step belongs to
  v8i A[2][DNI], B[2][DMJ];
  // wait for a tile's pair 0 (and its scales), read its first fragments;
  // block: the accumulator starts in units of group 0's factor
  // per-channel: the tile's fragment offsets, formed once per tile (block
  // kernels form them per step: kept, they push the 8-wave kernel to spill)
  Offs toA, toB;
  auto start_tile = [&]() {
    // fragments are filled a half at a time: start each from an arbitrary
    // value so the previous tile's are not kept alive through the epilogue
#pragma unroll
    for (int f = 0; f < DNI; ++f) {
      A[0][f] = __builtin_nondeterministic_value(A[0][f]);
      A[1][f] = __builtin_nondeterministic_value(A[1][f]);
    }
#pragma unroll
    for (int f = 0; f < DMJ; ++f) {
      B[0][f] = __builtin_nondeterministic_value(B[0][f]);
      B[1][f] = __builtin_nondeterministic_value(B[1][f]);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSL - 1) * (NLD + NSC)));
    __syncthreads();
    Offs oA, oB;
    frag_offsets(oA, oB);
    if constexpr (!BLOCK) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) { toA[a][b] = oA[a][b]; toB[a][b] = oB[a][b]; }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(oA, oB, A[0], B[0], cs, 0, frag_of(r >> 1), r & 1);
    if constexpr (BLOCK) {
#pragma unroll
      for (int j = 0; j < DMJ; ++j) { fcur[j] = 0.f; fmax[j] = 0.f; rho[j] = 1.f; }
      group_scales(0, cs);
      group_factor();
#pragma unroll
      for (int j = 0; j < DMJ; ++j) fcur[j] = gsx[j];   // rho of group 0 is unused
    }
  };
  prologue(0);
  start_tile();
  // Step kt (cur = kt & 1). Even: read step kt+1 (same pair, second half),
  // two reads per MFMA at the front of the step; block: rescale each
  // accumulator block before its first MFMA of the group. Odd: wait for the
  // next pair, barrier, read step kt+1 from the next slot, refill this
  // pair's slot with pair kt/2 + NSL; block: form the next group's rescale.
  // The first step of a tile starts its accumulators from zero.
  //
  // 256 x 192 tiles (EARLY): the refill moves to the middle of the even step
  // and the wait for the next pair to the middle of the odd step, so a pair
  // is issued about three K steps before it is read instead of two (waiting
  // for the ring is the loop's largest stall). Even step: reads of the
  // pair's second half, then (this wave's reads done, barrier: every wave's
  // reads of the slot done) the refill of the pair's own slot with pair
  // kt/2 + NSL. Odd step: the first half of the MFMAs, then the wait for
  // the next pair (the pair issued after it may stay in flight), a barrier
  // (every wave's part of it landed), and its first-half reads. Measured:
  // 8B qkv 96 against 101 us; with 256-wide tiles the second barrier per
  // pair costs more than the earlier refill gains (gate_up 400 against 388).
  constexpr bool EARLY = !BLOCK && BNP == 192;
  constexpr int TB = (NR + 1) / 2;                          // even: reads before the barrier
  constexpr int IPE = (NLD + NSC + (NM - TB) - 1) / (NM - TB);  // loads per slot after it
  constexpr int TW = NM / 2;                                // odd: MFMAs before the wait
  constexpr int RPO = (NR + (NM - TW) - 1) / (NM - TW);     // reads per slot after it
  static_assert(TB < NM && TW < NM, "mid-step points inside the step");
  auto step = [&](int kt, auto cur_c, auto more_c, auto first_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool more = decltype(more_c)::value;
    constexpr bool first = decltype(first_c)::value;
    const int ns = cs + 1 == NSL ? 0 : cs + 1;
    if (!EARLY && cur == 1 && more) {
      // vmcnt: the NSL-2 newer pairs may stay in flight; lgkmcnt(0): this
      // wave's reads of the slot refilled below are done
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSL - 2) * (NLD + NSC)) & ~0x0F00);
      asm volatile("s_barrier" ::: "memory");
      if constexpr (BLOCK) {
        group_scales(kt / 2 + 1, ns);
      }
    }
    const int rs = cur == 0 ? cs : ns;
    Offs oA, oB;
    if constexpr (!BLOCK) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) { oA[a][b] = toA[a][b]; oB[a][b] = toB[a][b]; }
    } else {
      if (more) frag_offsets(oA, oB);
    }
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      if (more) {
        if (cur == 0) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 2 * t + u;
            if (r < NR) read_frag(oA, oB, A[1], B[1], rs, 1, frag_of(r >> 1), r & 1);
          }
          if constexpr (EARLY) {
            if (t == TB) {
              __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
              asm volatile("s_barrier" ::: "memory");
            }
            if (t >= TB) {
#pragma unroll
              for (int u = 0; u < IPE; ++u) {
                const int w = IPE * (t - TB) + u;
                if (w < NLD + NSC) issue(cs, kt / 2 + NSL, w);
              }
            }
          }
        } else if constexpr (EARLY) {
          if (t == TW) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSL - 1) * (NLD + NSC)));
            asm volatile("s_barrier" ::: "memory");
          }
          if (t >= TW) {
#pragma unroll
            for (int u = 0; u < RPO; ++u) {
              const int r = RPO * (t - TW) + u;
              if (r < NR) read_frag(oA, oB, A[0], B[0], rs, 0, frag_of(r >> 1), r & 1);
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < RPE; ++u) {
            const int r = RPE * t + u;
            if (r < NR) read_frag(oA, oB, A[0], B[0], rs, 0, frag_of(r >> 1), r & 1);
          }
#pragma unroll
          for (int u = 0; u < IPS; ++u) {
            const int w = IPS * t + u;
            if (w < NLD + NSC) issue(cs, kt / 2 + NSL, w);
          }
        }
      }
      if constexpr (BLOCK && cur == 1) {
        if (more && t == kGroupFactorAt) group_factor();
      }
      const int i = t / DMJ, j = t % DMJ;
      if constexpr (first) {
        acc[i][j] = mfma_e4m3_32x32x64(A[cur][i], B[cur][j], v16f{});
      } else {
        if constexpr (BLOCK && cur == 0) {   // rho = 1 before group 1
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] *= rho[j];
        }
        acc[i][j] = mfma_e4m3_32x32x64(A[cur][i], B[cur][j], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (BLOCK && cur == 1) {
      if (more) {
#pragma unroll
        for (int j = 0; j < DMJ; ++j) fcur[j] = gsx[j];
      }
    }
    if (cur == 1) cs = ns;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  const int KT = K / 64;   // even, >= 4
  const bool vec = ((N | ldy) & 7) == 0;

  for (;;) {
    step(0, I0(), T(), T());
    step(1, I1(), T(), F());
    for (int kt = 2; kt < KT - 2; kt += 2) {
      step(kt, I0(), T(), F());
      step(kt + 1, I1(), T(), F());
    }
    step(KT - 2, I0(), T(), F());
    step(KT - 1, I1(), F(), F());
    const int vn = v + (int)gridDim.x;
    const bool has_next = vn < ntiles;   // uniform
    const int em0 = m0, en0 = n0, epar = par;
    if (has_next) {
      // every wave is done reading the slots (lgkmcnt, barrier): the next
      // tile's scales and first pairs load under this tile's epilogue
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      v = vn;
      par ^= 1;
      set_tile(v);
      prologue(cs);
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may still target LDS
    }

    // ---- epilogue ----
    const int eln = lane_now();
    const int elr = eln & 31, ekh = eln >> 5;
    const float* scl = reinterpret_cast<const float*>(smem + C::SC + epar * 2048);
    float smv[DMJ];
#pragma unroll
    for (int j = 0; j < DMJ; ++j) smv[j] = BLOCK ? fcur[j] : scl[wm * DTM + 32 * j + elr];
    // A tile inside Y (no ragged edge, rows starting on 128-byte lines)
    // stores whole lines with the non-temporal hint, two 32-column fragments
    // (64 columns, one line of a row) at a time; other tiles, and a fragment
    // left without a line-aligned partner (256 x 192 tiles: the wave's third),
    // store 16-byte pieces, masked per element at the edges.
    const bool full = em0 + BM <= M && en0 + BN <= N && (ldy & 63) == 0 &&
                      ((uintptr_t)y & 127) == 0;   // uniform
    const int fo = (wn * DNI) & 1;   // fragment i starts a line when (i + fo) is even
    // (i, qp) -> 16 bytes of this lane's row: bf16 of the scaled
    // accumulators, lanes l and l+32 exchanging halves with
    // v_permlane32_swap so lane l holds n = 32 i + 16 qp + 8 (l / 32) + 0..7
    // of row m = 32 j + l % 32
    auto pack16 = [&](int i, int j, int qp, float sm, const float4 (&s4)[4], uint32_t (&o)[4]) {
      uint32_t w[2][2];   // [q of the pair][dword]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int q = 2 * qp + u;
        // the scale product first: acc * sx alone could pass fp32's range
        // (activation rows near the bf16 maximum) while y stays finite
        w[u][0] = pk_bf16_rne(acc[i][j][4 * q + 0] * (sm * s4[q].x), acc[i][j][4 * q + 1] * (sm * s4[q].y));
        w[u][1] = pk_bf16_rne(acc[i][j][4 * q + 2] * (sm * s4[q].z), acc[i][j][4 * q + 3] * (sm * s4[q].w));
      }
      // lane l (kh 0) keeps its q = 2qp values and takes lane l+32's; lane
      // l+32 keeps its q = 2qp+1 values and takes lane l's
      const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
      o[0] = s0[0]; o[1] = s1[0]; o[2] = s0[1]; o[3] = s1[1];
    };
    auto col_scales = [&](int i, float4 (&s4)[4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s4[q] = BLOCK ? make_float4(1.f, 1.f, 1.f, 1.f)
                      : *reinterpret_cast<const float4*>(scl + 256 + wn * DTN + 32 * i + 8 * q + 4 * ekh);
    };
    // j outer, then i and qp: a lane's stores of one row (the wave's
    // 2 * DTN bytes of it) go out back to back
#pragma unroll
    for (int j = 0; j < DMJ; ++j) {
      const int m = em0 + wm * DTM + 32 * j + elr;
      const float sm = smv[j];
#pragma unroll
      for (int i = 0; i < DNI; ++i) {
        const bool lead = ((i + fo) & 1) == 0;
        if (full && lead && i + 1 < DNI) {
          // Fragments i and i+1 (64 columns) of rows 32 j .. 32 j + 31 as 4
          // stores of 8 rows x 128 bytes. After pack16, lane bits 0-4 are
          // row bits 0-4 and lane bit 5 is column bit 3; qp is column bit 4
          // and i & 1 column bit 5. v_permlane16_swap exchanges lane bit 4
          // with qp, a row_ror:8 DPP move lane bit 3 with i & 1: the slot
          // [a][b] then holds rows 16 b + 8 a + (l & 7) and lane l columns
          // 32 (l>>3 & 1) + 16 (l>>4 & 1) + 8 (l>>5) + 0..7.
          uint32_t r[2][2][4];   // [i & 1 -> row bit 3][qp -> row bit 4][dword]
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            float4 s4[4];
            col_scales(i + a, s4);
#pragma unroll
            for (int qp = 0; qp < 2; ++qp) pack16(i + a, j, qp, sm, s4, r[a][qp]);
          }
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const auto t = __builtin_amdgcn_permlane16_swap(r[a][0][d], r[a][1][d], false, false);
              r[a][0][d] = t[0];
              r[a][1][d] = t[1];
            }
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint32_t x = r[0][b][d], z = r[1][b][d];
              // r[0]: lanes with bit 3 set take z from lane ^ 8, the others
              // keep x; r[1]: lanes with bit 3 clear take x from lane ^ 8,
              // the others keep z
              r[0][b][d] = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)z, 0x128, 0xF, 0xC, false);
              r[1][b][d] = (uint32_t)__builtin_amdgcn_update_dpp((int)z, (int)x, 0x128, 0xF, 0x3, false);
            }
          const int cn = en0 + wn * DTN + 32 * i + 32 * ((eln >> 3) & 1) + 16 * ((eln >> 4) & 1) +
                         8 * (eln >> 5);
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              const int rm = em0 + wm * DTM + 32 * j + 16 * b + 8 * a + (eln & 7);
              const u32x4 v = {r[a][b][0], r[a][b][1], r[a][b][2], r[a][b][3]};
              __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y + (int64_t)rm * ldy + cn));
            }
        } else if (!full || (lead && i + 1 == DNI) || (!lead && i == 0)) {
          float4 s4[4];
          col_scales(i, s4);
#pragma unroll
          for (int qp = 0; qp < 2; ++qp) {
            uint32_t o[4];
            pack16(i, j, qp, sm, s4, o);
            const int n = en0 + wn * DTN + 32 * i + 16 * qp + 8 * ekh;
            if (m < M) {
              uint16_t* out = y + (int64_t)m * ldy + n;
              if (vec && n + 7 < N) {
                *reinterpret_cast<uint4*>(out) = make_uint4(o[0], o[1], o[2], o[3]);
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                  if (n + e < N) out[e] = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
              }
            }
          }
        }
      }
    }
    if (!has_next) break;
    set_tile(v);   // recomputed rather than kept in registers across the epilogue
    start_tile();
  }
}

// Compute units of the current device (0 when the runtime does not say).
inline int cu_count() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return ncu;
}

// y: rows of ldy elements (0: N), of which the first N are written.
template <bool BLOCK, int BNP>
void launch_line(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                 void* y, int64_t M, int64_t N, int64_t K, hipStream_t st, int64_t ldy = 0) {
  using C = LineCfg<BLOCK, BNP>;
  if (ldy == 0) ldy = N;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_prefill_line_kernel<BLOCK, BNP>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  const int tiles_m = (int)((M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((N + C::BN - 1) / C::BN);
  const int ntiles = tiles_m * tiles_n;
  // Persistent when there are more tiles than CUs (one workgroup per CU
  // walks its tiles; the next tile's scales and first pairs load under the
  // current one's epilogue): per-channel measured 1.5-3.5 % faster on the 8B
  // and long-context gate_up shapes, block 256 x 256 tiles 1-5 % faster on
  // the 3B qkv and gate_up shapes. 256 x 128 block tiles (16 per CU on the
  // 3B gate_up) keep one tile per workgroup: there the dispatcher's dynamic
  // assignment balanced the CUs better than a fixed one (6 % slower
  // persistent).
  int grid = ntiles;
  if (!BLOCK || BNP == 256) {
    const int ncu = cu_count();
    if (ncu > 0 && ncu % 8 == 0 && ntiles > ncu) grid = ncu;
  }
  hipLaunchKernelGGL((gemm_prefill_line_kernel<BLOCK, BNP>), dim3((unsigned)grid), dim3(64 * C::NW),
                     C::smem(K), st, qx, sx, qw, sw, (uint16_t*)y, (int)M, (int)N, (int)K,
                     (int)ldy, tiles_m, tiles_n);
}

}  // namespace
}  // namespace line
}  // namespace fp8dq
