// W12 GEMM for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// GEMM's scratch (packed activations, argmax key slots, the K-slice sums of
// remaining channel groups) lives in one file-scope device array instead of
// a caller workspace.  Each GPU the library runs on holds its own copy of
// the array until the process ends.
#include <mutex>

#include "internal.h"

namespace tvp {
constexpr size_t kNoAllocScratchBytes = TVP_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocMaxDevices = 64;
}  // namespace tvp

// The array itself.  In host code this name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[tvp::kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[tvp::kNoAllocMaxDevices];  // device address of `scratch` on each device
}  // namespace

using namespace tvp;

extern "C" {

int w12_gemm_ex_noalloc(const uint16_t* x, int64_t m, int64_t ldx, const tvp_w12_packed* w,
                        const tvp_gemm_epilogue* epi, hipStream_t stream) {
  if (!w || !epi) return TVP_ERR_ARG;
  if (m < 1 || m > 192) return TVP_ERR_SHAPE;
  const size_t need = w12_gemm_workspace(m, w);
  if (need == 0 || need > kNoAllocScratchBytes) return TVP_ERR_WORKSPACE;
  int dev = -1;
  TVP_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kNoAllocMaxDevices) return TVP_ERR_ARG;
  if (stream) {
    hipDevice_t sd = -1;
    TVP_CHECK_HIP(hipStreamGetDevice(stream, &sd));
    if (sd != dev) return TVP_ERR_ARG;  // the array's address is per device
  }
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TVP_ERR_HIP;
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  // Nothing in the scratch needs to start at zero: every kernel writes what
  // it later reads within the call.
  return w12_gemm_ex(x, m, ldx, w, epi, ptr, kNoAllocScratchBytes, stream);
}

}  // extern "C"
