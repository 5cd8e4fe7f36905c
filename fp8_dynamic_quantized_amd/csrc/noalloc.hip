// Device scratch of fp8_linear_noalloc: one file-scope array per GPU, so the
// entry point needs no allocation (for callers that cannot allocate: code
// under HIP graph capture, serving loops, harnesses that forbid it).
//
// Layout (as the decode path's caller workspace): 16 KiB of split-K tile
// counters, zero when the library loads and left zero by every call, then
// 16 MiB of fp32 partial sums. Every call on a GPU shares that GPU's array;
// calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace fp8dq {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_ptr[kMaxDevices];          // per device: the array's device address
std::once_flag g_once[kMaxDevices];

}  // namespace

void* scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  // with this device current: its own copy of the array, at its own address
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_ptr[dev] = p;
  });
  return g_ptr[dev];
}

}  // namespace fp8dq
