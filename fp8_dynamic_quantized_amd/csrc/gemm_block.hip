// Block-scaled instantiations of the whole-line prefill GEMM (gemm_line.hpp).
// Built with the MFMA destination / accumulator operands in ordinary VGPRs
// (each wave's 128 x 64 part of a tile holds 128 accumulator registers), so
// that the per-group rescale of the accumulator is one multiply per element
// instead of an AGPR read, multiply and write.
#include "gemm_line.hpp"
#include "kernels.hpp"

namespace fp8dq {

void launch_gemm_line_block(const uint8_t* qx, const float* sx, const uint8_t* qw,
                            const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                            hipStream_t st) {
  // 256 x 256 tiles (8 waves, two per SIMD: one wave's rescale runs beside
  // the other's MFMAs, and each pair load and barrier serves twice the MFMAs)
  // or 256 x 128 tiles (4 waves), whichever finishes the tiles in less time.
  // Measured on the Llama-3.2-3B linears at M = 8192, a 256-wide tile takes
  // about 1.6 times as long as a 128-wide one (gate_up, qkv: 4-9 % faster
  // wide; o and down, whose 256-wide tiles fill 1.5 rounds of the CUs, 4-5 %
  // slower wide).
  const int ncu = line::cu_count();
  const int64_t tm = (M + 255) / 256;
  const int64_t t256 = tm * ((N + 255) / 256), t128 = tm * ((N + 127) / 128);
  bool wide = false;
  if (ncu > 0) {
    const int64_t r256 = (t256 + ncu - 1) / ncu, r128 = (t128 + ncu - 1) / ncu;
    wide = r256 * 8 < r128 * 5;
  }
  if (wide) line::launch_line<true, 256>(qx, sx, qw, sw, y, M, N, K, st);
  else line::launch_line<true, 128>(qx, sx, qw, sw, y, M, N, K, st);
}

}  // namespace fp8dq
