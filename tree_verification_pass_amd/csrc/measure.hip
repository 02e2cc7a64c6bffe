// Streaming-read probe: the HBM read rate this GPU sustains for a plain
// sequential stream, the practical ceiling the weight stream of the pass is
// compared against.  Every thread keeps eight 16-byte loads in flight over
// a grid-stride walk, XOR-folds what it read and the workgroup writes one
// word, so no load can be dropped.  The loads carry the non-temporal hint,
// as the GEMM's weight loads do (measured on MI355X: 6.97 TB/s, against
// 6.2-6.4 TB/s for the same stream with ordinary loads).
#include "internal.h"

namespace tvp {

constexpr int kProbeUnroll = 8;
constexpr int kProbeGroups = 4096;

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * kProbeUnroll;
  for (size_t base = (size_t)blockIdx.x * 256 * kProbeUnroll + threadIdx.x; base < n16; base += stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t i = base + (size_t)u * 256;
      v[u] = i < n16 ? load_nt(src + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s[256];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int i = 0; i < 256; ++i) a ^= s[i];
    sink[blockIdx.x] = a;
  }
}

}  // namespace tvp

using namespace tvp;

extern "C" {

int tvp_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes < 16 || ((uintptr_t)src) % 16 != 0) return TVP_ERR_ARG;
  read_probe_kernel<<<dim3(kProbeGroups), dim3(256), 0, stream>>>((const uint4*)src, bytes / 16, sink);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

}  // extern "C"
