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
  // Tiles: 256 x 256 (8 waves, two per SIMD: one wave's rescale runs beside
  // the other's MFMAs, and each pair load and barrier serves twice the MFMAs)
  // or 256 x 128 (4 waves). Measured on the Llama-3.2-3B linears at M = 8192,
  // a round of 256-wide tiles on the CUs takes about 1.6 times a round of
  // 128-wide ones. The launch that finishes the tiles in the fewest such
  // units is chosen: all wide, all narrow, or the first nw 256-column blocks
  // wide and the rest narrow in a second launch (costed one tenth of a
  // narrow round more). The split fills whole rounds where one width alone
  // leaves a round half empty: N = 3072 at M = 8192 takes one wide round
  // and one narrow one (2.6) instead of 1.5 wide rounds (3.2) or three
  // narrow ones (3.0).
  const int ncu = line::cu_count();
  if (ncu <= 0) {
    line::launch_line<true, 128>(qx, sx, qw, sw, y, M, N, K, st);
    return;
  }
  const int64_t tm = (M + 255) / 256;
  auto rounds = [&](int64_t tiles) { return (tiles + ncu - 1) / ncu; };
  // costs in tenths of a round of 128-wide tiles
  int64_t best = rounds(tm * ((N + 127) / 128)) * 10;
  int64_t nw_best = 0;   // 0: all narrow; -1: all wide; else the split
  const int64_t all_wide = rounds(tm * ((N + 255) / 256)) * 16;
  if (all_wide < best) { best = all_wide; nw_best = -1; }
  for (int64_t nw = 1; 256 * nw < N; ++nw) {
    const int64_t c = rounds(tm * nw) * 16 + rounds(tm * ((N - 256 * nw + 127) / 128)) * 10 + 1;
    if (c < best) { best = c; nw_best = nw; }
  }
  if (nw_best < 0) {
    line::launch_line<true, 256>(qx, sx, qw, sw, y, M, N, K, st);
  } else if (nw_best == 0) {
    line::launch_line<true, 128>(qx, sx, qw, sw, y, M, N, K, st);
  } else {
    // columns [0, n1) wide, [n1, N) narrow; Y rows stay N elements apart
    const int64_t n1 = 256 * nw_best, G = K / 128;
    line::launch_line<true, 256>(qx, sx, qw, sw, y, M, n1, K, st, N);
    line::launch_line<true, 128>(qx, sx, qw + n1 * K, sw + (n1 / 128) * G,
                                 static_cast<uint16_t*>(y) + n1, M, N - n1, K, st, N);
  }
}

}  // namespace fp8dq
