// probe.hip -- a plain streaming read, for measuring the read rate that a
// kernel of this library reaches on the current GPU (the scale against which
// the weight-streaming kernels' HBM rooflines are read).  Not part of the
// layer.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;

// Each thread reads 16-byte pieces grid-stride, four in flight per turn, and
// writes the XOR of every word it read (so no load can be dropped).
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4 *__restrict__ p, int64_t n,
                                                                    uint32_t *__restrict__ out) {
  const int64_t stride = int64_t(gridDim.x) * kProbeThreads;
  int64_t i = int64_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[int64_t(blockIdx.x) * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace moe

extern "C" int moe_stream_read(const void *src, size_t bytes, uint32_t *out, int32_t blocks, void *stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65536 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return MOE_E_INVALID;
  moe::launch(moe::stream_read_kernel, dim3(unsigned(blocks)), dim3(moe::kProbeThreads), 0,
              static_cast<hipStream_t>(stream), static_cast<const uint4 *>(src), int64_t(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}
