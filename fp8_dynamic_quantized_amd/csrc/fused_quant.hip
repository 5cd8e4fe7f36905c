// Producers fused with the dynamic FP8 quantizer, static calibration and the
// FP8 KV-cache write (gfx950).
//
// What is computed ("Llama 3 精读实录" page):
//  * SwiGLU product, §1.3 (gate and up computed separately, then multiplied
//    elementwise): h = bf16(silu(g) * u), silu(g) = g / (1 + e^-g), g and u
//    the two halves of the fused gate_up output row; then per-token FP8.
//  * RMSNorm, §1.3 (eps 1e-5, before attention and the MLP; kept in bf16,
//    §5.3): h = bf16(gamma * x / sqrt(mean(x^2) + eps)); then per-token FP8.
//  * Static calibration, §2.2 (P99.9 / P0.1 percentiles as the dynamic
//    range instead of max): amax = max(|x_(k_lo)|, |x_(k_hi)|) over the
//    whole tensor (nearest-rank order statistics), s = RN(amax / 448); and
//    the static quantization x -> E4M3(x / s) with saturation at +-448.
//  * FP8 KV cache, §4.1: per-token quantization of K and V rows written to
//    the cache rows a slot mapping names.
//
// The bf16 rounding of h is exact (the correctly rounded value of the real
// formula): h is formed in fp32 with a few ulps of error and rounded to bf16
// directly unless it lies within 8 fp32 ulps of a bf16 rounding midpoint,
// is tiny, or an fp32 intermediate left its normal range (SwiGLU: |g| > 64
// or |g*u| > 2^127; RMSNorm: x * r tiny); those elements are formed again in fp64,
// where a near-midpoint SwiGLU value is decided by the exact identity
//   h - m = s * ((g*u - m) - m * e^-g),  s = 1 / (1 + e^-g) > 0,
// in which g*u - m is exact in fp64. The quantization that follows is the
// exact codec of the other quantization kernels.
#include "device_common.hpp"
#include "kernels.hpp"
#include "quant_codec.hpp"

namespace fp8dq {
namespace {

using namespace codec;

constexpr uint32_t kMidTol = 8;  // fp32 ulps around a bf16 rounding midpoint

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ bool near_mid16(float h) {
  const uint32_t low = __float_as_uint(h) & 0xFFFFu;
  return (low - (0x8000u - kMidTol)) <= 2u * kMidTol;
}

__device__ __forceinline__ bool tiny32(float h) {  // |h| < 2^-100 (one compare, |h| operand)
  return __builtin_fabsf(h) < 0x1p-100f;
}

// Value of bf16 bit pattern b (sign included) as a double; b's magnitude may
// be one past the largest finite bf16, which stands for 2^128.
__device__ __forceinline__ double bf16_val(uint32_t b) {
  if ((b & 0x7FFFu) == 0x7F80u) return (b & 0x8000u) ? -0x1p128 : 0x1p128;
  return (double)__uint_as_float(b << 16);
}

// Correctly rounded bf16 of a finite double h (ties to even). Within 2^-30
// of the midpoint m between h's bf16 neighbours, `tie_side(m, d)` gives the
// sign of |h| - |m| (d is the fp64 difference |h| - |m|, which a caller
// without an exact identity returns as is). inf for magnitudes that round
// past the largest bf16.
template <typename TieSide>
__device__ __forceinline__ uint32_t f64_to_bf16(double h, TieSide tie_side) {
  if (h == 0.0) return (__double_as_longlong(h) < 0) ? 0x8000u : 0u;
  const float t = __double2float_rz(h);          // truncation toward zero
  uint32_t lo = __float_as_uint(t) >> 16;        // bf16 neighbour toward zero
  if ((lo & 0x7FFFu) >= 0x7F80u) return lo & 0xFF80u;  // beyond fp32 range: inf
  const double m = 0.5 * (bf16_val(lo) + bf16_val(lo + 1));
  double d = fabs(h) - fabs(m);                  // > 0: round away from zero
  if (fabs(d) <= 0x1p-30 * fabs(m)) d = tie_side(m, d);
  if (d > 0.0 || (d == 0.0 && (lo & 1u))) lo += 1;
  return lo;
}

// ---- SwiGLU ---------------------------------------------------------------
__device__ __noinline__ uint32_t silu_mul_slow(float gf, float uf) {
  const double g = gf, u = uf;
  const double e = exp(-g);                      // inf for g < -709: h = -0 * u
  const double h = g / (1.0 + e) * u;
  return f64_to_bf16(h, [&](double m, double) {
    // sign(|h| - |m|) = sign(h - m) * sign(m), with
    //   h - m = s * (g*u - m*(1 + e^-g)) = s * ((g*u - 2m) - m*expm1(-g)).
    // g*u - 2m is exact (g*u has 16 bits and m 9, within 44 binades of each
    // other whenever h is within 2^-36 of g*u), and expm1 keeps the small-g
    // ties exact: there m = g*u/2 and h - m ~ m*g/2.
    const double a = fma(g, u, -2.0 * m);
    const double side = a - m * expm1(-g);
    // zero when e^-g < 2^-54 (g > 37) and g*u = m: silu(g) < g for g > 0,
    // so |h| < |m| then.
    if (side == 0.0) return g > 0.0 ? -1.0 : 0.0;
    return m > 0.0 ? side : -side;
  });
}

// e^-g for |g| <= 64 from the hardware base-2 exponential: -g * log2(e) is
// split into p = RN(-g * L) and its remainder d (L = log2(e) as a head and a
// tail), and 2^(p + d) is taken as 2^p * (1 + d ln 2) (|d| < 2^-17, so the
// dropped second-order term is below 2^-35).
__device__ __forceinline__ float exp_neg(float g) {
  constexpr float kL = 0x1.715476p+0f;      // log2(e), head
  constexpr float kLlo = 0x1.4ae0bep-26f;   // log2(e) - kL
  constexpr float kLn2 = 0x1.62e430p-1f;
  const float x = -g;
  const float p = x * kL;
  const float d = fmaf(x, kLlo, fmaf(x, kL, -p));
  const float e2 = __builtin_amdgcn_exp2f(p);
  return fmaf(e2 * kLn2, d, e2);
}

// 1 / (1 + e^-g), |g| <= 64, from the hardware reciprocal. Its relative error
// over every bf16 g with |g| <= 64 stays below kSiluRecipErr (checked over
// all of them), so h = RN(g*u * r), with g*u exact, is within
// kSiluRecipErr + 2^-24 of the real value: under 4 fp32 ulps of h.
__device__ __forceinline__ float silu_recip(float g) {
  return __builtin_amdgcn_rcpf(1.0f + exp_neg(g));
}

// Elements the fast value cannot decide: |g| > 64, g*u past 2^127 (it may
// have overflowed fp32 while h = silu(g) * u is still a finite bf16), h near
// a bf16 rounding midpoint, or h tiny while g*u is not zero.
__device__ __forceinline__ bool silu_flag(float g, float gu, float h) {
  return (__builtin_fabsf(g) > 64.0f) | (__builtin_fabsf(gu) > 0x1p127f) | near_mid16(h) |
         (tiny32(h) & (gu != 0.0f));
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {   // RNE, two values
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8 gate and 8 up values (one 16-byte chunk each) -> 8 h values (bf16). The
// fast value is formed for all 8 without a branch; a lane with a flagged
// element forms those again in the exact path.
__device__ __forceinline__ uint4 silu_mul8(uint4 gv, uint4 uv) {
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
  const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
  float g[8], u[8], h[8];
  bool any = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    g[2 * i] = bf16lo(gw[i]);
    g[2 * i + 1] = bf16hi(gw[i]);
    u[2 * i] = bf16lo(uw[i]);
    u[2 * i + 1] = bf16hi(uw[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float gu = g[i] * u[i];
    h[i] = gu * silu_recip(g[i]);
    any |= silu_flag(g[i], gu, h[i]);
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pk_bf16(h[2 * i], h[2 * i + 1]);
  if (__builtin_expect(any, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (silu_flag(g[i], g[i] * u[i], h[i])) {
        const uint32_t b = silu_mul_slow(g[i], u[i]);
        o[i >> 1] = (i & 1) ? ((o[i >> 1] & 0xFFFFu) | (b << 16)) : ((o[i >> 1] & 0xFFFF0000u) | b);
      }
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---- RMSNorm --------------------------------------------------------------
__device__ __noinline__ uint32_t rms_slow(float xf, float gf, double r) {
  const double h = (double)xf * r * (double)gf;
  return f64_to_bf16(h, [](double, double d) { return d; });  // fp64 decides
}

// Elements the fast value (t = x * r32, then h = t * gamma: within 3 fp32
// ulps of the real value while both stay normal) cannot decide: h near a
// bf16 rounding midpoint, or t or h tiny while x and gamma are not zero (a
// t in fp32's subnormal range has lost bits that a large gamma would carry
// into a normal h).
__device__ __forceinline__ bool rms_flag(float x, float gm, float t, float h) {
  return near_mid16(h) | ((tiny32(t) | tiny32(h)) & (x != 0.0f) & (gm != 0.0f));
}

// 8 values and their 8 gamma entries -> 8 normalized values (bf16).
__device__ __forceinline__ uint4 rms8(uint4 xv, uint4 gv, float r32, double r64) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
  float x[8], gm[8], t[8], h[8];
  bool any = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16lo(xw[i]);
    x[2 * i + 1] = bf16hi(xw[i]);
    gm[2 * i] = bf16lo(gw[i]);
    gm[2 * i + 1] = bf16hi(gw[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t[i] = x[i] * r32;
    h[i] = t[i] * gm[i];
    any |= rms_flag(x[i], gm[i], t[i], h[i]);
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pk_bf16(h[2 * i], h[2 * i + 1]);
  if (__builtin_expect(any, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (rms_flag(x[i], gm[i], t[i], h[i])) {
        const uint32_t b = rms_slow(x[i], gm[i], r64);
        o[i >> 1] = (i & 1) ? ((o[i >> 1] & 0xFFFFu) | (b << 16)) : ((o[i >> 1] & 0xFFFF0000u) | b);
      }
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ double chunk_sumsq(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double a = bf16lo(w[i]), b = bf16hi(w[i]);
    s = fma(a, a, s);
    s = fma(b, b, s);
  }
  return s;
}

// Sum over the wave's 64 lanes, in every lane, by the same lane pairings
// as wave64_max (both 32-bit halves of each value moved); the pairs add in
// either order to the same bits, so every lane ends with one value.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_mov<CTRL>((uint32_t)b), hi = dpp_mov<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ double join_f64(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);   // row_half_mirror
  v += dpp_f64<0x140>(v);   // row_mirror
  uint64_t b = (uint64_t)__double_as_longlong(v);
  const auto l16 = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  v = join_f64(l16[0], h16[0]) + join_f64(l16[1], h16[1]);
  b = (uint64_t)__double_as_longlong(v);
  const auto l32 = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  return join_f64(l32[0], h32[0]) + join_f64(l32[1], h32[1]);
}

// ---- shared per-row tail: amax of the h chunks, scale, codes ---------------
template <int CH, int TW>
__device__ __forceinline__ void quantize_team(const uint4 (&h)[CH], bool row_ok, int64_t row,
                                              int64_t nch, int team_lane, uint32_t* red,
                                              uint2* __restrict__ q, float* __restrict__ scale) {
  constexpr int TEAM = 64 * TW;
  // chunks past the row end hold arbitrary values (their loads were not
  // zeroed) and are left out here and at the store
  us2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const us2 a = chunk_amax(h[i], m2);
    if ((int64_t)i * TEAM + team_lane < nch) m2 = a;
  }
  uint32_t m = m2.x > m2.y ? m2.x : m2.y;
  m = wave64_max(m);
  if (TW > 1) {   // the team's waves meet in red[team * TW ...]
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    const uint32_t* tr = red + (threadIdx.x / TEAM) * TW;
    m = tr[0];
#pragma unroll
    for (int w = 1; w < TW; ++w) m = m > tr[w] ? m : tr[w];
  }
  if (!row_ok) return;
  float s, r, p;
  bool tiny;
  unit_scale(m, s, r, p, tiny);
  if (team_lane == 0) scale[row] = s;
  uint2* qr = q + row * nch;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * TEAM + team_lane;
    if (c < nch) qr[c] = tiny ? quant8<true>(h[i], s, r, p) : quant8<false>(h[i], s, r, p);
  }
}

// Stores the team's bf16 h chunks of one row (the unquantized outputs).
template <int CH, int TW>
__device__ __forceinline__ void store_team(const uint4 (&h)[CH], bool row_ok, int64_t row,
                                           int64_t nch, int team_lane, uint4* __restrict__ out) {
  if (!row_ok) return;
  uint4* orow = out + row * nch;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * 64 * TW + team_lane;
    if (c < nch) orow[c] = h[i];
  }
}

// One team of TW waves per row (TW = 1: four rows per 256-thread block).
// Q: per-token FP8 codes and scales; else the bf16 h row itself.
template <int CH, int TW, bool Q>
__global__ __launch_bounds__(TW >= 4 ? 64 * TW : 256) void silu_mul_kernel(
    const uint4* __restrict__ gu, int64_t rows, int64_t I, void* __restrict__ out,
    float* __restrict__ scale) {
  constexpr int TEAM = 64 * TW;
  constexpr int RPB = TW >= 4 ? 1 : 4 / TW;
  __shared__ uint32_t red[TW >= 4 ? TW : 4];
  const int tid = threadIdx.x, tl = tid % TEAM;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TEAM;
  const int64_t nch = I >> 3;
  const bool row_ok = row < rows;
  const uint4* gr = gu + (row_ok ? row : 0) * 2 * nch;
  uint4 gv[CH], uv[CH], h[CH];
  // every lane loads (chunk 0 past the row end, a valid address) and nothing
  // is zeroed: the team's amax and stores leave those chunks out
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * TEAM + tl;
    const int64_t cc = (row_ok && c < nch) ? c : 0;
    gv[i] = ld16(gr + cc);
    uv[i] = ld16(gr + nch + cc);
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) h[i] = silu_mul8(gv[i], uv[i]);   // silu(0) * 0 = +0
  if (Q)
    quantize_team<CH, TW>(h, row_ok, row, nch, tl, red, static_cast<uint2*>(out), scale);
  else
    store_team<CH, TW>(h, row_ok, row, nch, tl, static_cast<uint4*>(out));
}

template <int CH, int TW, bool Q>
__global__ __launch_bounds__(TW >= 4 ? 64 * TW : 256) void rmsnorm_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ gamma, int64_t rows,
    int64_t H, double eps, void* __restrict__ out, float* __restrict__ scale) {
  constexpr int TEAM = 64 * TW;
  constexpr int RPB = TW >= 4 ? 1 : 4 / TW;
  __shared__ uint32_t red[TW >= 4 ? TW : 4];
  __shared__ double reds[TW >= 4 ? TW : 4];
  const int tid = threadIdx.x, tl = tid % TEAM;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TEAM;
  const int64_t nch = H >> 3;
  const bool row_ok = row < rows;
  const uint4* xr = x + (row_ok ? row : 0) * nch;
  uint4 h[CH], gv[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * TEAM + tl;
    h[i] = ld16_if(xr, c, row_ok && c < nch);
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * TEAM + tl;
    gv[i] = ld16_if(gamma, c, c < nch);
  }
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < CH; ++i) ss += chunk_sumsq(h[i]);
  ss = wave_sum_f64(ss);
  if (TW > 1) {
    if ((tid & 63) == 0) reds[tid >> 6] = ss;
    __syncthreads();
    const double* tr = reds + (tid / TEAM) * TW;
    ss = tr[0];
#pragma unroll
    for (int w = 1; w < TW; ++w) ss += tr[w];   // fixed order
  }
  const double r64 = 1.0 / sqrt(ss / (double)H + eps);
  const float r32 = (float)r64;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * TEAM + tl;
    if (row_ok && c < nch) h[i] = rms8(h[i], gv[i], r32, r64);
  }
  if (Q)
    quantize_team<CH, TW>(h, row_ok, row, nch, tl, red, static_cast<uint2*>(out), scale);
  else
    store_team<CH, TW>(h, row_ok, row, nch, tl, static_cast<uint4*>(out));
}

// ---- static calibration: exact order statistics by two radix passes -------
// bf16 bits -> 16-bit key with the same order as the values (-0 below +0).
__device__ __forceinline__ uint32_t okey(uint32_t b) {
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
__device__ __forceinline__ uint32_t okey_inv(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
}

constexpr int kHistBlocks = 1024;
constexpr int kSub = 16;   // sub-histograms per block, by lane % 16

// The two global histograms (256 high-byte, 512 low-byte counters) start at 0.
__global__ __launch_bounds__(256) void calib_zero_kernel(unsigned long long* __restrict__ hist) {
  for (int i = threadIdx.x; i < 768; i += 256) hist[i] = 0ull;
}

// Pass 1: histogram of the key's high byte. Pass 2: histograms of the low
// byte of the keys whose high byte is sel[0] / sel[2]. Each block counts
// into kSub sub-histograms laid out [bin][sub]: the lanes of one wave that
// hit the same bin use different banks (at most 4 lanes share a sub), where
// one histogram serialised up to 64 lanes on the few populated buckets of
// real data. Blocks then add their counts to the global histogram (integer
// atomics: the sums are exact and order-free).
template <bool SECOND>
__global__ __launch_bounds__(256) void calib_hist_kernel(const uint4* __restrict__ x,
                                                         int64_t nch, const int64_t* sel,
                                                         unsigned long long* __restrict__ hist) {
  constexpr int NB = SECOND ? 512 : 256;
  __shared__ uint32_t hst[NB * kSub];
  const int tid = threadIdx.x;
  const uint32_t sub = (uint32_t)tid & (kSub - 1);
  for (int b = tid; b < NB * kSub; b += 256) hst[b] = 0;
  uint32_t hb_lo = 0, hb_hi = 0;
  if (SECOND) { hb_lo = (uint32_t)sel[0]; hb_hi = (uint32_t)sel[2]; }
  __syncthreads();
  auto count = [&](const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t k = okey((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      if (!SECOND) {
        atomicAdd(&hst[(k >> 8) * kSub + sub], 1u);
      } else {
        if ((k >> 8) == hb_lo) atomicAdd(&hst[(k & 255u) * kSub + sub], 1u);
        if ((k >> 8) == hb_hi) atomicAdd(&hst[(256 + (k & 255u)) * kSub + sub], 1u);
      }
    }
  };
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t c = (int64_t)blockIdx.x * 256 + tid;
  for (; c + 3 * stride < nch; c += 4 * stride) {   // four loads in flight
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ld16(x + c + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) count(v[u]);
  }
  for (; c < nch; c += stride) count(ld16(x + c));
  __syncthreads();
  for (int b = tid; b < NB; b += 256) {
    uint32_t t = 0;   // a block counts below 2^30 values (n < 2^40, 1024 blocks)
#pragma unroll
    for (int u = 0; u < kSub; ++u) t += hst[b * kSub + u];
    if (t) atomicAdd(&hist[(SECOND ? 256 : 0) + b], (unsigned long long)t);
  }
}

// For ranks k_lo and k_hi (1-based), the bucket holding the rank and the
// rank inside it, from inclusive prefix sums of the histogram. One block of
// 256. SECOND: the buckets are low bytes; write the scale.
template <bool SECOND>
__global__ __launch_bounds__(256) void calib_select_kernel(const unsigned long long* __restrict__ hist,
                                                           int64_t k_lo, int64_t k_hi,
                                                           int64_t* sel, float* scale_out) {
  constexpr int H = SECOND ? 2 : 1;
  __shared__ int64_t cnt[H][256], inc[H][256];
  __shared__ int64_t res[4];
  const int tid = threadIdx.x;
  for (int h = 0; h < H; ++h) {
    const int64_t c = (int64_t)hist[(SECOND ? 256 : 0) + h * 256 + tid];
    cnt[h][tid] = c;
    inc[h][tid] = c;
  }
  const int64_t ranks[2] = {SECOND ? sel[1] : k_lo, SECOND ? sel[3] : k_hi};
  if (tid < 4) res[tid] = (tid & 1) ? ranks[tid >> 1] : 0;   // k = 0: bucket 0, rank 0
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    int64_t t[H];
#pragma unroll
    for (int h = 0; h < H; ++h) t[h] = tid >= d ? inc[h][tid - d] : 0;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < H; ++h) inc[h][tid] += t[h];
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int h = SECOND ? j : 0;
    const int64_t k = ranks[j];
    const int64_t before = inc[h][tid] - cnt[h][tid];
    if (k >= 1 && before < k && k <= inc[h][tid]) {   // exactly one bucket
      res[2 * j] = tid;
      res[2 * j + 1] = k - before;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (!SECOND) {
      for (int j = 0; j < 4; ++j) sel[j] = res[j];
    } else {
      const uint32_t key_lo = ((uint32_t)sel[0] << 8) | (uint32_t)res[0];
      const uint32_t key_hi = ((uint32_t)sel[2] << 8) | (uint32_t)res[2];
      const float vlo = fabsf(__uint_as_float(okey_inv(key_lo) << 16));
      const float vhi = fabsf(__uint_as_float(okey_inv(key_hi) << 16));
      const float amax = (k_hi > 0) ? fmaxf(vlo, vhi) : 0.0f;
      scale_out[0] = amax / kE4M3Max;            // correctly rounded: RN(amax/448)
    }
  }
}

// Static quantization with one fp32 scale for the whole tensor: codes of
// x / s, saturating at +-448 (clamped before the hardware conversion, whose
// own saturation does not reach beyond 464).
template <bool PRE>
__device__ __forceinline__ uint2 quant8_sat(uint4 raw, float s, float r, float p) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8], y[8], yc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[i] = (PRE ? x[i] * p : x[i]) * r;
    yc[i] = __builtin_fminf(__builtin_fmaxf(y[i], -460.0f), 460.0f);
  }
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(yc[0], yc[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(yc[2], yc[3], lo, true);
  uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(yc[4], yc[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(yc[6], yc[7], hi, true);
  bool any = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) any |= needs_fixup(y[i]);
  if (__builtin_expect(any, 0)) {
    const float sp = PRE ? s * p : s;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (needs_fixup(y[i])) {
        uint32_t& word = (i < 4) ? lo : hi;
        const int sh = 8 * (i & 3);
        const float ax = __builtin_fabsf(PRE ? x[i] * p : x[i]);
        const uint32_t mag = exact_mag(ax, sp, __builtin_fabsf(y[i]));
        const uint32_t code = mag | ((__float_as_uint(x[i]) >> 24) & 0x80u);
        word = (word & ~(0xFFu << sh)) | (code << sh);
      }
    }
  }
  return make_uint2(lo, hi);
}

__global__ __launch_bounds__(256) void quant_static_kernel(const uint4* __restrict__ x,
                                                           int64_t nch, const float* sptr,
                                                           uint2* __restrict__ q) {
  const float s = *sptr;
  const bool tiny = s < kTinyScale && s > 0.0f;
  const float p = tiny ? kPreScale : 1.0f;
  const float r = s > 0.0f ? 1.0f / (s * p) : 0.0f;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nch;
       c += (int64_t)gridDim.x * 256)
    q[c] = tiny ? quant8_sat<true>(ld16(x + c), s, r, p) : quant8_sat<false>(ld16(x + c), s, r, p);
}

// ---- FP8 KV cache: per-token quantization, rows scattered by slot ---------
// One launch for K and V: rows 0 .. T-1 of the grid are K's tokens, T .. 2T-1
// V's (a team takes one row).
template <int CH, int TW>
__global__ __launch_bounds__(TW >= 4 ? 64 * TW : 256) void kv_quant_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, int64_t T, int64_t width,
    const int64_t* __restrict__ slots, int64_t n_slots, uint2* __restrict__ kc,
    uint2* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs) {
  constexpr int TEAM = 64 * TW;
  constexpr int RPB = TW >= 4 ? 1 : 4 / TW;
  __shared__ uint32_t red[TW >= 4 ? TW : 4];
  const int tid = threadIdx.x, tl = tid % TEAM;
  const int64_t t2 = (int64_t)blockIdx.x * RPB + tid / TEAM;
  const bool is_v = t2 >= T;
  const int64_t t = is_v ? t2 - T : t2;
  const uint4* x = is_v ? v : k;
  uint2* cache = is_v ? vc : kc;
  float* cscale = is_v ? vs : ks;
  const int64_t nch = width >> 3;
  const bool tok = t < T;
  // the row's loads do not wait for its slot: they go out together with the
  // slot's load, and the slot only decides the store (rows of skipped slots
  // are read and dropped)
  const int64_t slot = tok ? slots[t] : -1;
  const uint4* xr = x + (tok ? t : 0) * nch;
  uint4 h[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = (int64_t)i * TEAM + tl;
    h[i] = ld16_if<true>(xr, c, tok && c < nch);
  }
  const bool row_ok = slot >= 0 && slot < n_slots;   // out-of-range slots are skipped
  quantize_team<CH, TW>(h, row_ok, row_ok ? slot : 0, nch, tl, red, cache, cscale);
}

// Row-team launch ladders: CH chunks per lane, TW waves per row. The wide
// ladder starts at teams of 4 waves (one row per block), with CH the fewest
// chunks per lane that cover the row, so no lane of a 14336-wide row idles.
template <template <int, int> class Launch, typename... A>
int launch_ladder(int64_t nch, A... a) {
  if (nch <= 64) { Launch<1, 1>::go(a...); return 0; }
  if (nch <= 128) { Launch<2, 1>::go(a...); return 0; }
  if (nch <= 256) { Launch<4, 1>::go(a...); return 0; }
  if (nch <= 512) { Launch<8, 1>::go(a...); return 0; }
  if (nch <= 1024) { Launch<4, 4>::go(a...); return 0; }
  if (nch <= 2048) { Launch<8, 4>::go(a...); return 0; }
  if (nch <= 4096) { Launch<4, 16>::go(a...); return 0; }
  if (nch <= 8192) { Launch<8, 16>::go(a...); return 0; }
  return -1;
}

template <template <int, int> class Launch, typename... A>
int launch_ladder_wide(int64_t nch, A... a) {
  if (nch <= 256) { Launch<1, 4>::go(a...); return 0; }
  if (nch <= 512) { Launch<2, 4>::go(a...); return 0; }
  if (nch <= 768) { Launch<3, 4>::go(a...); return 0; }
  if (nch <= 1024) { Launch<4, 4>::go(a...); return 0; }
  if (nch <= 1280) { Launch<5, 4>::go(a...); return 0; }
  if (nch <= 1536) { Launch<6, 4>::go(a...); return 0; }
  if (nch <= 1792) { Launch<7, 4>::go(a...); return 0; }
  if (nch <= 2048) { Launch<8, 4>::go(a...); return 0; }
  if (nch <= 4096) { Launch<4, 16>::go(a...); return 0; }
  if (nch <= 8192) { Launch<8, 16>::go(a...); return 0; }
  return -1;
}

template <int CH, int TW>
struct RowsGrid {
  static dim3 blocks(int64_t rows) {
    constexpr int RPB = TW >= 4 ? 1 : 4 / TW;
    return dim3((unsigned)((rows + RPB - 1) / RPB));
  }
  static dim3 threads() { return dim3(TW >= 4 ? 64 * TW : 256); }
};

template <bool Q>
struct SiluLaunch {
  template <int CH, int TW>
  struct L {
    static void go(const void* gu, int64_t rows, int64_t I, void* out, float* s,
                   hipStream_t st) {
      hipLaunchKernelGGL((silu_mul_kernel<CH, TW, Q>), (RowsGrid<CH, TW>::blocks(rows)),
                         (RowsGrid<CH, TW>::threads()), 0, st, (const uint4*)gu, rows, I, out,
                         s);
    }
  };
};
template <bool Q>
struct RmsLaunch {
  template <int CH, int TW>
  struct L {
    static void go(const void* x, const void* g, int64_t rows, int64_t H, double eps,
                   void* out, float* s, hipStream_t st) {
      hipLaunchKernelGGL((rmsnorm_kernel<CH, TW, Q>), (RowsGrid<CH, TW>::blocks(rows)),
                         (RowsGrid<CH, TW>::threads()), 0, st, (const uint4*)x,
                         (const uint4*)g, rows, H, eps, out, s);
    }
  };
};
template <int CH, int TW>
struct KvLaunch {
  static void go(const void* k, const void* v, int64_t T, int64_t width, const int64_t* slots,
                 int64_t n_slots, uint8_t* kc, uint8_t* vc, float* ks, float* vs,
                 hipStream_t st) {
    hipLaunchKernelGGL((kv_quant_kernel<CH, TW>), (RowsGrid<CH, TW>::blocks(2 * T)),
                       (RowsGrid<CH, TW>::threads()), 0, st, (const uint4*)k,
                       (const uint4*)v, T, width, slots, n_slots, (uint2*)kc, (uint2*)vc, ks,
                       vs);
  }
};

}  // namespace

int launch_silu_mul_quant(const void* gu, int64_t rows, int64_t I, uint8_t* q,
                          float* scale, hipStream_t st) {
  return launch_ladder_wide<SiluLaunch<true>::template L>(I / 8, gu, rows, I, (void*)q,
                                                          scale, st);
}

int launch_silu_mul(const void* gu, int64_t rows, int64_t I, void* h, hipStream_t st) {
  // bf16 h out, rows of 1537-2048 chunks (the Llama-3.1-8B I = 14336): teams
  // of 16 waves with 2 chunks per lane, 61.3-61.5 against 65.9 us for 4
  // waves with 7 (the quantizing variant, which waits for the row's amax
  // before its stores, was 2-4 % slower that way and keeps the ladder)
  const int64_t nch = I / 8;
  if (nch > 1536 && nch <= 2048) {
    SiluLaunch<false>::template L<2, 16>::go(gu, rows, I, h, (float*)nullptr, st);
    return 0;
  }
  return launch_ladder_wide<SiluLaunch<false>::template L>(nch, gu, rows, I, h,
                                                           (float*)nullptr, st);
}

int launch_rmsnorm_quant(const void* x, const void* gamma, int64_t rows, int64_t H,
                         double eps, uint8_t* q, float* scale, hipStream_t st) {
  return launch_ladder_wide<RmsLaunch<true>::template L>(H / 8, x, gamma, rows, H, eps,
                                                         (void*)q, scale, st);
}

int launch_rmsnorm(const void* x, const void* gamma, int64_t rows, int64_t H, double eps,
                   void* h, hipStream_t st) {
  return launch_ladder_wide<RmsLaunch<false>::template L>(H / 8, x, gamma, rows, H, eps, h,
                                                          (float*)nullptr, st);
}

int launch_kv_quant(const void* k, const void* v, int64_t T, int64_t width,
                    const int64_t* slots, int64_t n_slots, uint8_t* kc, uint8_t* vc,
                    float* ks, float* vs, hipStream_t st) {
  return launch_ladder<KvLaunch>(width / 8, k, v, T, width, slots, n_slots, kc, vc, ks, vs,
                                 st);
}

size_t calib_workspace_bytes() {
  return 768 * sizeof(unsigned long long) + 4 * sizeof(int64_t);
}

void launch_calib_scale(const void* x, int64_t n, int64_t k_lo, int64_t k_hi,
                        float* scale_out, void* ws, hipStream_t st) {
  const int64_t nch = n / 8;
  int nblk = (int)((nch + 255) / 256);
  if (nblk > kHistBlocks) nblk = kHistBlocks;
  if (nblk < 1) nblk = 1;
  unsigned long long* hist = static_cast<unsigned long long*>(ws);
  int64_t* sel = reinterpret_cast<int64_t*>(hist + 768);
  hipLaunchKernelGGL(calib_zero_kernel, dim3(1), dim3(256), 0, st, hist);
  hipLaunchKernelGGL((calib_hist_kernel<false>), dim3(nblk), dim3(256), 0, st,
                     (const uint4*)x, nch, (const int64_t*)sel, hist);
  hipLaunchKernelGGL((calib_select_kernel<false>), dim3(1), dim3(256), 0, st,
                     (const unsigned long long*)hist, k_lo, k_hi, sel, scale_out);
  hipLaunchKernelGGL((calib_hist_kernel<true>), dim3(nblk), dim3(256), 0, st,
                     (const uint4*)x, nch, (const int64_t*)sel, hist);
  hipLaunchKernelGGL((calib_select_kernel<true>), dim3(1), dim3(256), 0, st,
                     (const unsigned long long*)hist, k_lo, k_hi, sel, scale_out);
}

void launch_quant_static(const void* x, int64_t n, const float* scale, uint8_t* q,
                         hipStream_t st) {
  const int64_t nch = n / 8;
  int64_t blocks = (nch + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(quant_static_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint4*)x, nch, scale, (uint2*)q);
}

}  // namespace fp8dq
