// Block-scaled instantiation of the whole-line prefill GEMM (gemm_line.hpp).
// Built with the MFMA destination / accumulator operands in ordinary VGPRs
// (the 256 x 128 tile's 128 accumulator registers fit), so that the
// per-group rescale of the accumulator is one multiply per element instead
// of an AGPR read, multiply and write.
#include "gemm_line.hpp"
#include "kernels.hpp"

namespace fp8dq {

void launch_gemm_line_block(const uint8_t* qx, const float* sx, const uint8_t* qw,
                            const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                            hipStream_t st) {
  line::launch_line<true, 128>(qx, sx, qw, sw, y, M, N, K, st);
}

}  // namespace fp8dq
