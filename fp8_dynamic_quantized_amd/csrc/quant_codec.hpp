// Exact dynamic E4M3 codec shared by the quantization kernels and the fused
// producers (same arithmetic everywhere, so codes agree bit for bit).
//
// What is computed (Llama-3.1-8B-Instruct-FP8-Dynamic page, FP8 dynamic
// quantization table; E4M3 limits from the "Llama 3 精读实录" page, §2.1):
//   s = RN_fp32(amax / 448);  q = E4M3_RNE(x / s) with the exact quotient,
//   ties to the even code, the sign of zero kept, +-0 when s = 0.
// How: y = x * RN(1/s) in fp32, converted by the hardware (round to nearest
// even); lanes whose y sits within a couple of fp32 ulps of an E4M3 midpoint,
// or in the E4M3 subnormal range, take an exact fix-up from the sign of one
// fused multiply-add (midpoint * s - |x|). Scales below 2^-64 are handled by
// scaling x and s by 2^64 (exact).
#pragma once
#include "device_common.hpp"

namespace fp8dq {
namespace codec {

constexpr uint32_t kNearTol = 2;          // fp32 ulps of slack around a midpoint
constexpr float kTinyScale = 0x1p-64f;    // scales below this are pre-scaled
constexpr float kPreScale = 0x1p64f;

// Exact E4M3 magnitude code of |x| / s, given its fp32 estimate ay = |y|
// (within 2 fp32 ulps). The exact quotient lies in the E4M3 interval that
// truncation of ay selects, or just across its midpoint; one fused
// multiply-add gives the exact sign of (midpoint * s - |x|): positive keeps
// the lower code, negative takes the upper one, zero is a tie that goes to
// the even code. Normal range: the interval comes from ay's bits; E4M3
// subnormal range (ay < 2^-6): the spacing is 2^-9.
//   ax = |x| (times the pre-scale p), sp = s * p.
__device__ __forceinline__ uint32_t exact_mag(float ax, float sp, float ay) {
  const uint32_t yb = __float_as_uint(ay);
  uint32_t trunc;
  float mid;
  if (ay >= 0x1p-6f) {
    trunc = (yb >> 20) - (120u << 3);  // exponent rebias 127 -> 7, 3 bits kept
    mid = __uint_as_float((yb & 0xFFF00000u) | 0x80000u);
  } else {
    trunc = (uint32_t)(ay * 512.0f);   // floor: ay >= 0
    mid = __builtin_fmaf((float)trunc, 0x1p-9f, 0x1p-10f);
  }
  const float t = __builtin_fmaf(mid, sp, -ax);
  const uint32_t up = (t < 0.0f) | ((t == 0.0f) & (trunc & 1u));
  const uint32_t code = trunc + up;
  return code < 126u ? code : 126u;  // beyond 448: saturate
}

// True when y needs the exact fix-up: its low 20 mantissa bits are within
// kNearTol of the E4M3 normal-range midpoint pattern, or 0 < |y| < 2^-6.
__device__ __forceinline__ bool needs_fixup(float y) {
  uint32_t b = __float_as_uint(y);
  bool near_mid = ((b + (kNearTol - 0x80000u)) << 12) <= ((2u * kNearTol) << 12);
  bool small = ((b << 1) - 2u) < ((0x3C800000u << 1) - 2u);
  return near_mid || small;
}

// Quantize 8 bf16 values (one 16-byte chunk) with scale s.
// r = 1/(s*p) (0 when s == 0), p the pre-scale (1 or 2^64, PRE only).
template <bool PRE>
__device__ __forceinline__ uint2 quant8(uint4 raw, float s, float r, float p) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8], y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (PRE ? x[i] * p : x[i]) * r;
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  // the 8 tests without a branch, then one branch for the chunk
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
        float ax = __builtin_fabsf(PRE ? x[i] * p : x[i]);
        uint32_t mag = exact_mag(ax, sp, __builtin_fabsf(y[i]));
        uint32_t code = mag | ((__float_as_uint(x[i]) >> 24) & 0x80u);
        word = (word & ~(0xFFu << sh)) | (code << sh);
      }
    }
  }
  return make_uint2(lo, hi);
}

// Largest |bf16| bit pattern (sign cleared) over a chunk, per 16-bit half.
__device__ __forceinline__ us2 chunk_amax(uint4 v, us2 acc) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a = w[i] & 0x7FFF7FFFu;
    us2 h = __builtin_bit_cast(us2, a);
    acc = __builtin_elementwise_max(acc, h);
  }
  return acc;
}

// Lane reductions without LDS, for a unit's amax: DPP moves inside rows of
// 16 lanes (swap neighbours, swap pairs, half-row mirror, row mirror: after
// each step a quad, an 8-lane half-row, then the row hold one value), then
// v_permlane16_swap (rows 0 and 1, 2 and 3) and v_permlane32_swap (the two
// halves). Each step pairs lanes, so every lane ends with the same value.
// All 64 lanes must be active. (Generic lane shuffles compile to
// ds_bpermute, an LDS round trip per step on the row's critical chain; these
// stay in registers, which made the per-token quantizers 2-4 % faster.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// maximum over each row of 16 lanes, in every lane of the row
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = umax32(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]
  v = umax32(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]
  v = umax32(v, dpp_mov<0x141>(v));   // row_half_mirror
  v = umax32(v, dpp_mov<0x140>(v));   // row_mirror
  return v;
}

// maximum over the wave's 64 lanes, in every lane
__device__ __forceinline__ uint32_t wave64_max(uint32_t v) {
  v = row16_max(v);
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umax32(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax32(b[0], b[1]);
}

__device__ __forceinline__ void unit_scale(uint32_t amax_bits, float& s,
                                           float& r, float& p, bool& tiny) {
  float amax = __uint_as_float(amax_bits << 16);
  s = amax / kE4M3Max;  // IEEE division, correctly rounded
  tiny = s < kTinyScale && s > 0.0f;
  p = tiny ? kPreScale : 1.0f;
  r = s > 0.0f ? 1.0f / (s * p) : 0.0f;
}

}  // namespace codec
}  // namespace fp8dq
