// Device-side helpers shared by the FP8-Dynamic kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8dq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads (plain and non-temporal) returning HIP's uint4.
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Chunk c of p when ok, else zeros. The load is issued in every lane (from
// chunk 0 when !ok, so p[0] must be readable), with no branch around it:
// a lane's loads then all go out before the first of them is waited for,
// where a branch per load makes the compiler wait for each before the next.
template <bool NT = false>
__device__ __forceinline__ uint4 ld16_if(const uint4* p, int64_t c, bool ok) {
  const uint4* a = p + (ok ? c : 0);
  const uint4 v = NT ? ld16_nt(a) : ld16(a);
  return ok ? v : make_uint4(0, 0, 0, 0);
}

constexpr float kE4M3Max = 448.0f;  // largest finite E4M3 magnitude

// 16x16 output tile, K = 128 E4M3 x E4M3 products per MFMA, fp32 accumulate.
// Operand layout (both A and B): lane l holds row (l % 16) of its operand
// and 32 consecutive K-bytes of that row; the four lane groups l / 16 hold
// the four 32-byte K slices. A and B use the same lane->K mapping, so any
// consistent assignment of K bytes to (lane group, byte) gives the same sum.
// Output: lane l holds C[4*(l/16) + r][l % 16], r = 0..3, where the first
// index runs over A's rows and the second over B's rows.
// Scale operands 0 select the unscaled instruction (plain E4M3 products).
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i& a, const v8i& b,
                                                   const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0,
                                                          0, 0);
}

typedef float v16f __attribute__((ext_vector_type(16)));

// 32x32 output tile, K = 64 E4M3 x E4M3 products per MFMA, fp32 accumulate.
// Operands: lane l holds row (l % 32) and 32 consecutive K-bytes, the two
// lane halves l / 32 holding the two 32-byte K slices (same mapping for A
// and B). Output: lane l holds C[8*(v/4) + 4*(l/32) + (v%4)][l % 32] in
// element v = 0..15 (first index: A's rows, second: B's rows).
__device__ __forceinline__ v16f mfma_e4m3_32x32x64(const v8i& a, const v8i& b,
                                                   const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0,
                                                          0, 0);
}

// fp32 -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}


// LDS (address space 3) pointer, for taking the 32-bit LDS address of a
// shared array.
typedef __attribute__((address_space(3))) void* lds_ptr;

// One global_load_lds_dwordx4: 16 bytes from base + off (off per lane, base
// wave-uniform) to LDS byte address lds + 16 * lane (lds wave-uniform). It
// has no result registers; completion is observed with vmcnt, which callers
// wait for explicitly (issued from asm so that the compiler adds no waits of
// its own before LDS reads). M0 carries the LDS base and needs one wait
// state before the load reads it.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory", "m0");
}

// One global_load_lds_dword: 4 bytes from base + off (off per lane) to LDS
// byte address lds + 4 * lane (M0 = lds). Completion is observed with vmcnt.
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory", "m0");
}

}  // namespace fp8dq
