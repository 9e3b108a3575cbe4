// Decode attention without a caller workspace: the arrival counters and the
// per-segment records live in one statically sized device array of the
// library, for callers that cannot allocate device memory (code under graph
// capture, serving loops that must not call the allocator).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "abi_internal.h"

using oscar::fail;

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;        // the whole array
constexpr size_t kCounterBytes = size_t(256) << 10;       // counters of up to 65536 (sequence, KV head) units
constexpr size_t kRecordBytes = kScratchBytes - kCounterBytes;

}  // namespace

// One copy per device the library runs on, held until the process ends.  Host
// code never uses this name as an address: kernels get the device address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

__global__ void scratch_zero_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words; i += size_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint8_t* g_ptr[kMaxDevices] = {};

// The array's address on the current device, looked up once per device; the
// first call also clears the counters (stream-ordered before the decode).
oscar_status scratch_for_device(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return oscar::hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(OSCAR_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return oscar::hip_status(e, "hipGetSymbolAddress(scratch)");
    hipLaunchKernelGGL(scratch_zero_kernel, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(p), kCounterBytes / 4);
    if (hipError_t e = hipGetLastError()) return oscar::hip_status(e, "scratch counter clear launch");
    g_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_ptr[dev];
  return OSCAR_OK;
}

}  // namespace

extern "C" {

oscar_status oscar_paged_decode_attn_noalloc(const oscar_cache* cache, const void* q, int32_t batch,
                                             int32_t n_q_heads, const int32_t* seq_lens, int32_t max_seq_len,
                                             const int32_t* bt_q, const int32_t* bt_h, int32_t max_pages,
                                             const float* r_k, const float* r_v, float sm_scale,
                                             int32_t split_pages, void* out, void* stream) {
  oscar::clear_error();
  oscar::DecodePlan plan;
  if (oscar_status s = oscar::decode_validate(false, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h,
                                              max_pages, r_k, r_v, sm_scale, split_pages, out, &plan))
    return s;
  if (batch == 0) return OSCAR_OK;
  if (plan.counter_bytes > kCounterBytes || plan.bytes - plan.counter_bytes > kRecordBytes)
    return fail(OSCAR_ERR_WORKSPACE,
                "call needs more than the built-in 32 MiB decode scratch (65536 (sequence, KV head) units, "
                "32512 KiB of records); use oscar_paged_decode_attn with a workspace");
  uint8_t* base = nullptr;
  if (oscar_status s = scratch_for_device(static_cast<hipStream_t>(stream), &base)) return s;
  return oscar::decode_launch(false, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h, max_pages, r_k,
                              r_v, sm_scale, plan, reinterpret_cast<int32_t*>(base),
                              reinterpret_cast<float*>(base + kCounterBytes), out, stream);
}

}  // extern "C"
