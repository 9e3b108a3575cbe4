// Attainable HBM read bandwidth, as context for the decode kernels' roofline
// fractions: a streaming read of a caller buffer with nothing written back
// (the decode kernels read far more than they write).
#include <hip/hip_runtime.h>

#include "abi_internal.h"

namespace {

// Each thread keeps four independent 16-byte loads in flight per round
// (grid-stride over whole rounds, then the tail), folds them with XOR and
// stores only if the fold hits a value no input here produces, so the loads
// cannot be removed and nothing is written.
__global__ __launch_bounds__(512) void read_probe_kernel(const uint4* __restrict__ p, size_t n_vec, uint32_t* sink) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n_vec; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" {

oscar_status oscar_bw_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  oscar::clear_error();
  if (!buf || !sink) return oscar::fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return oscar::fail(OSCAR_ERR_INVALID_ARG, "buffer and size must be multiples of 16 bytes");
  if (bytes == 0) return OSCAR_OK;
  const unsigned blocks = unsigned(8 * oscar::device_cu_count());
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return oscar::hip_status(hipGetLastError(), "read probe launch");
}

}  // extern "C"
