// liboscar C ABI: argument validation, workspace planning and launches.  The
// semantics of every entry point are specified in include/oscar.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "abi_internal.h"
#include "kernels.h"

namespace oscar {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = '\0'; }

}  // namespace oscar

using oscar::fail;

namespace {

bool supported_d(int32_t d) { return d == 64 || d == 128; }

}  // namespace

namespace oscar {

oscar_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return OSCAR_OK;
  oscar::set_error("OSCAR_ERR_HIP: %s: %s", what, hipGetErrorString(e));
  return OSCAR_ERR_HIP;
}

oscar_status check_cache(const oscar_cache* c, bool need_int2, bool need_bf16) {
  if (!c) return fail(OSCAR_ERR_INVALID_ARG, "cache is NULL");
  if (!supported_d(c->d)) return fail(OSCAR_ERR_UNSUPPORTED, "cache d must be 64 or 128");
  if (c->n_kv_heads < 1) return fail(OSCAR_ERR_INVALID_ARG, "cache n_kv_heads < 1");
  if (c->n_sink < 0 || c->n_recent < 0) return fail(OSCAR_ERR_INVALID_ARG, "negative n_sink or n_recent");
  if (need_int2 && (!c->int2_pool || c->n_int2_pages < 1)) return fail(OSCAR_ERR_INVALID_ARG, "INT2 pool missing");
  if (need_bf16 && (!c->bf16_pool || c->n_bf16_pages < 1)) return fail(OSCAR_ERR_INVALID_ARG, "BF16 pool missing");
  return OSCAR_OK;
}

}  // namespace oscar

namespace {

using oscar::check_cache;
using oscar::hip_status;

}  // namespace

namespace oscar {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// The grid (one 8-wave workgroup fits a CU).
// * split_pages > 0: per-unit items of split_pages pages each.
// * Automatic, few units (at most a quarter of the CUs): per-unit items sized
//   so that one round fills the CUs: one BF16 item per unit and the INT2
//   pages of all units spread over the remaining CUs (for the longest
//   possible lengths).  One segment per workgroup keeps the latency chain
//   short.
// * Automatic, many units: one workgroup per CU, each taking an even share
//   of all units' pages (balanced slices), whatever the device-side lengths;
//   about three record slots per workgroup a unit could span, at least 8 (the
//   kernel widens the slices where a unit would need more).
// A sequence covers at most n_pages + 2 pages of work (the pages at the two
// ends of the INT2 range also hold BF16 tokens), plus the per-range overhead
// positions of balanced slices.
oscar_status plan_decode(int32_t batch, int32_t n_kv, int32_t n_q, int32_t d, int32_t max_seq_len,
                         int32_t split_pages, bool all_raw, DecodePlan* plan) {
  if (batch < 0 || max_seq_len < 0) return fail(OSCAR_ERR_INVALID_ARG, "negative batch or max_seq_len");
  if (!supported_d(d)) return fail(OSCAR_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (n_kv < 1 || n_q < 1 || n_q % n_kv) return fail(OSCAR_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q / n_kv;
  if (G > 16) return fail(OSCAR_ERR_UNSUPPORTED, "query group size above 16");
  if (split_pages != 0 && (split_pages < 8 || split_pages > 1 << 20 || split_pages % 8))
    return fail(OSCAR_ERR_INVALID_ARG, "split_pages must be 0 or a multiple of 8 in [8, 2^20]");
  const long long units = (long long)batch * n_kv;
  const long long max_pages = (max_seq_len + 15LL) / 16;
  const long long max_cost = max_pages + 2 + 2LL * oscar_launch::decode_seg_pages() + oscar_launch::decode_own_pages();
  if (units * max_cost >= (1LL << 31)) return fail(OSCAR_ERR_UNSUPPORTED, "2^31 or more pages of work in one call; split the batch");
  const int max_rec = oscar_launch::decode_max_records();
  const long long cus = device_cu_count();
  plan->per_unit = split_pages != 0 || 4 * units <= cus;
  plan->first_int2 = 0;
  if (plan->per_unit) {
    long long split = split_pages, first = 0;
    if (!split) {
      // With long INT2 items the BF16 pages join item 0, which then takes
      // `first` INT2 pages fewer than a full item, the BF16 segment's cost
      // (its fixed cost plus its pages, in INT2 pages: about seg_pages(G) +
      // 64), so that every workgroup of the round holds INT2 work; kept when
      // that first chunk is at least 64 pages (not for short histories, whose
      // items are mostly fixed cost).
      const long long per = all_raw || units == 0 ? 0 : cus / units;
      const long long c0 = oscar_launch::decode_seg_pages_of(G) + 64;
      if (per >= 2) {
        const long long sp = ((max_pages + c0 + per - 1) / per + 7) / 8 * 8;
        if (sp - c0 >= 64 && sp >= (max_pages + max_rec - 3) / (max_rec - 2)) {
          split = sp;
          first = (sp - c0) / 8 * 8;
        }
      }
      if (!split) {
        const long long items = std::max(1LL, all_raw ? cus : cus - units);
        split = std::max<long long>(oscar_launch::decode_min_slice(), (units * max_pages + items - 1) / items);
        split = std::max(split, (max_pages + max_rec - 2) / (max_rec - 1));
        split = (split + 7) / 8 * 8;  // measured: fewer, slightly larger items beat an uneven last pair round
      }
    }
    // workgroups per unit: item 0 (BF16 pages and `first` INT2 pages), then
    // the INT2 items; records: one per segment
    const long long n_items = 1 + (std::max(0LL, max_pages - first) + split - 1) / split;
    const long long n_rec = n_items + (first > 0 ? 1 : 0);
    if (n_rec > max_rec) return fail(OSCAR_ERR_UNSUPPORTED, "more chunks per (sequence, KV head) than one merge takes; use a larger split_pages");
    if (units * n_items > (1LL << 31) - 1) return fail(OSCAR_ERR_UNSUPPORTED, "grid too large; use a larger split_pages");
    plan->fixed_ppw = int(split);
    plan->first_int2 = int(first);
    plan->unit_items = int(n_items);
    plan->cap = int(n_rec);
    plan->n_wg = int(std::max(1LL, units * n_items));
  } else {
    plan->fixed_ppw = 0;
    plan->unit_items = 0;
    plan->n_wg = int(cus);
    const long long per = (3 * cus + units - 1) / units + 3;
    plan->cap = int(std::min<long long>(max_rec, std::max(8LL, per)));
  }
  plan->rec_floats = (2 * G + G * d + 1 + 3) / 4 * 4;  // [max G][sum G][value sums G d][basis flag]
  plan->counter_bytes = (size_t(units) * 4 + 255) / 256 * 256;
  plan->bytes = plan->counter_bytes + size_t(units) * plan->cap * plan->rec_floats * 4;
  return OSCAR_OK;
}

}  // namespace oscar

namespace {

using oscar::DecodePlan;
using oscar::device_cu_count;
using oscar::plan_decode;

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words; i += size_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// BF16 rows into BF16 pages: K token-major [16][d], V channel-major [d][16].
__global__ void write_bf16_kernel(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                                  const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
                                  const int32_t* __restrict__ bt_h, int32_t max_pages, uint16_t* __restrict__ pool,
                                  int32_t n_kv, int32_t d) {
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y;
  const int c = threadIdx.x;
  const int32_t pos = row_pos[row];
  const int64_t page = bt_h[int64_t(row_seq[row]) * max_pages + (pos >> 4)];
  const int slot = pos & 15;
  uint16_t* base = pool + (page * n_kv + h) * int64_t(32) * d;
  const int64_t src = (row * n_kv + h) * d + c;
  base[slot * d + c] = k_new[src];
  base[16 * d + c * 16 + slot] = v_new[src];
}

}  // namespace

extern "C" {

const char* oscar_status_string(oscar_status s) {
  switch (s) {
    case OSCAR_OK: return "OSCAR_OK";
    case OSCAR_ERR_INVALID_ARG: return "OSCAR_ERR_INVALID_ARG";
    case OSCAR_ERR_UNSUPPORTED: return "OSCAR_ERR_UNSUPPORTED";
    case OSCAR_ERR_NUMERIC: return "OSCAR_ERR_NUMERIC";
    case OSCAR_ERR_WORKSPACE: return "OSCAR_ERR_WORKSPACE";
    case OSCAR_ERR_HIP: return "OSCAR_ERR_HIP";
  }
  return "OSCAR_ERR_UNKNOWN";
}

const char* oscar_last_error(void) { return oscar::g_err; }

int32_t oscar_version(void) { return OSCAR_VERSION; }

size_t oscar_int2_page_bytes(int32_t d, int32_t n_kv_heads) {
  if (!supported_d(d) || n_kv_heads < 1) return 0;
  return size_t(12) * d * n_kv_heads;
}

size_t oscar_bf16_page_bytes(int32_t d, int32_t n_kv_heads) {
  if (!supported_d(d) || n_kv_heads < 1) return 0;
  return size_t(64) * d * n_kv_heads;
}

static oscar_status quantize_append_common(int bits, const oscar_cache* cache, const void* k_new, const void* v_new,
                                           int64_t n_rows, const int32_t* row_seq, const int32_t* row_pos,
                                           const int32_t* bt_q, int32_t max_pages, const float* r_k, const float* r_v,
                                           float tau_k, float tau_v, void* stream) {
  oscar::clear_error();
  if (oscar_status s = check_cache(cache, true, false)) return s;
  if (n_rows < 0) return fail(OSCAR_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows == 0) return OSCAR_OK;
  if (!k_new || !v_new || !row_seq || !row_pos || !bt_q || !r_k || !r_v)
    return fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (max_pages < 1) return fail(OSCAR_ERR_INVALID_ARG, "max_pages < 1");
  if (!(tau_k > 0.f) || !(tau_v > 0.f) || !std::isfinite(tau_k) || !std::isfinite(tau_v))
    return fail(OSCAR_ERR_INVALID_ARG, "clip thresholds must be finite and positive");
  if ((n_rows + 15) / 16 > int64_t(0x7FFFFFFF)) return fail(OSCAR_ERR_UNSUPPORTED, "n_rows too large");
  return hip_status(oscar_launch::quantize_append(cache->d, bits, cache->n_kv_heads, cache->int2_pool, k_new, v_new, n_rows,
                                                  row_seq, row_pos, bt_q, max_pages, r_k, r_v, tau_k, tau_v,
                                                  device_cu_count(), static_cast<hipStream_t>(stream)),
                    "quantize_append launch");
}

oscar_status oscar_quantize_append(const oscar_cache* cache, const void* k_new, const void* v_new, int64_t n_rows,
                                   const int32_t* row_seq, const int32_t* row_pos, const int32_t* bt_q,
                                   int32_t max_pages, const float* r_k, const float* r_v, float tau_k, float tau_v,
                                   void* stream) {
  return quantize_append_common(2, cache, k_new, v_new, n_rows, row_seq, row_pos, bt_q, max_pages, r_k, r_v, tau_k,
                                tau_v, stream);
}

oscar_status oscar_quantize_append_int4(const oscar_cache* cache, const void* k_new, const void* v_new, int64_t n_rows,
                                        const int32_t* row_seq, const int32_t* row_pos, const int32_t* bt_q,
                                        int32_t max_pages, const float* r_k, const float* r_v, float tau_k,
                                        float tau_v, void* stream) {
  return quantize_append_common(4, cache, k_new, v_new, n_rows, row_seq, row_pos, bt_q, max_pages, r_k, r_v, tau_k,
                                tau_v, stream);
}

size_t oscar_int4_page_bytes(int32_t d, int32_t n_kv_heads) {
  if (!supported_d(d) || n_kv_heads < 1) return 0;
  return size_t(20) * d * n_kv_heads;
}

oscar_status oscar_write_bf16(const oscar_cache* cache, const void* k_new, const void* v_new, int64_t n_rows,
                              const int32_t* row_seq, const int32_t* row_pos, const int32_t* bt_h, int32_t max_pages,
                              void* stream) {
  oscar::clear_error();
  if (oscar_status s = check_cache(cache, false, true)) return s;
  if (n_rows < 0) return fail(OSCAR_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows == 0) return OSCAR_OK;
  if (!k_new || !v_new || !row_seq || !row_pos || !bt_h) return fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (max_pages < 1) return fail(OSCAR_ERR_INVALID_ARG, "max_pages < 1");
  if (n_rows > int64_t(0x7FFFFFFF)) return fail(OSCAR_ERR_UNSUPPORTED, "n_rows too large");
  hipLaunchKernelGGL(write_bf16_kernel, dim3(unsigned(n_rows), unsigned(cache->n_kv_heads)), dim3(cache->d), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), row_seq, row_pos, bt_h, max_pages,
                     static_cast<uint16_t*>(cache->bf16_pool), cache->n_kv_heads, cache->d);
  return hip_status(hipGetLastError(), "write_bf16 launch");
}

oscar_status oscar_decode_step_update(const oscar_cache* cache, const void* k_new, const void* v_new, int32_t batch,
                                     const int32_t* seq_lens, const int32_t* bt_q, const int32_t* bt_h,
                                     int32_t max_pages, const float* r_k, const float* r_v, float tau_k, float tau_v,
                                     void* stream) {
  oscar::clear_error();
  if (oscar_status s = check_cache(cache, true, true)) return s;
  if (batch < 0) return fail(OSCAR_ERR_INVALID_ARG, "batch < 0");
  if (batch == 0) return OSCAR_OK;
  if (!k_new || !v_new || !seq_lens || !bt_q || !bt_h || !r_k || !r_v)
    return fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (max_pages < 1) return fail(OSCAR_ERR_INVALID_ARG, "max_pages < 1");
  if (!(tau_k > 0.f) || !(tau_v > 0.f) || !std::isfinite(tau_k) || !std::isfinite(tau_v))
    return fail(OSCAR_ERR_INVALID_ARG, "clip thresholds must be finite and positive");
  return hip_status(oscar_launch::decode_step_update(cache->d, cache->n_kv_heads, cache->n_sink, cache->n_recent,
                                                     cache->int2_pool, cache->bf16_pool, k_new, v_new, batch,
                                                     seq_lens, bt_q, bt_h, max_pages, r_k, r_v, tau_k, tau_v,
                                                     static_cast<hipStream_t>(stream)),
                    "decode_step_update launch");
}

oscar_status oscar_calib_gram(const void* x, int64_t n_rows, int32_t n_x_heads, int32_t n_kv_heads, int32_t d,
                              double* out, void* stream) {
  oscar::clear_error();
  if (!x || !out) return fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (!supported_d(d)) return fail(OSCAR_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (n_rows < 1 || n_kv_heads < 1) return fail(OSCAR_ERR_INVALID_ARG, "n_rows < 1 or n_kv_heads < 1");
  if (n_x_heads < n_kv_heads || n_x_heads % n_kv_heads) return fail(OSCAR_ERR_INVALID_ARG, "n_x_heads not a multiple of n_kv_heads");
  if (n_x_heads / n_kv_heads > 16) return fail(OSCAR_ERR_UNSUPPORTED, "more than 16 heads per KV group");
  if (reinterpret_cast<uintptr_t>(x) % 16) return fail(OSCAR_ERR_INVALID_ARG, "x not 16-byte aligned");
  const int64_t pooled = n_rows * (n_x_heads / n_kv_heads);
  if (pooled / 256 >= int64_t(0x7FFFFFFF) || n_rows > (int64_t(1) << 40)) return fail(OSCAR_ERR_UNSUPPORTED, "too many rows");
  return hip_status(oscar_launch::calib_gram(d, x, n_rows, n_x_heads, n_kv_heads, out, static_cast<hipStream_t>(stream)),
                    "calib_gram launch");
}

oscar_status oscar_decode_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads, int32_t d,
                                          int32_t max_seq_len, int32_t split_pages, size_t* bytes) {
  oscar::clear_error();
  if (!bytes) return fail(OSCAR_ERR_INVALID_ARG, "bytes is NULL");
  DecodePlan plan, plan_raw;  // valid for the mixed cache and the all-BF16 decode
  if (oscar_status s = plan_decode(batch, n_kv_heads, n_q_heads, d, max_seq_len, split_pages, false, &plan))
    return s;
  if (oscar_status s = plan_decode(batch, n_kv_heads, n_q_heads, d, max_seq_len, split_pages, true, &plan_raw))
    return s;
  *bytes = std::max(plan.bytes, plan_raw.bytes);
  return OSCAR_OK;
}

oscar_status oscar_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  oscar::clear_error();
  if (!workspace) return fail(OSCAR_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes % 4) return fail(OSCAR_ERR_INVALID_ARG, "workspace_bytes not a multiple of 4");
  if (workspace_bytes == 0) return OSCAR_OK;
  const size_t words = workspace_bytes / 4;
  const unsigned blocks = unsigned(std::min<size_t>(4096, (words + 255) / 256));
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(workspace), words);
  return hip_status(hipGetLastError(), "workspace init launch");
}

}  // extern "C"

namespace oscar {

oscar_status decode_validate(bool all_raw, const oscar_cache* cache, const void* q, int32_t batch,
                             int32_t n_q_heads, const int32_t* seq_lens, int32_t max_seq_len, const int32_t* bt_q,
                             const int32_t* bt_h, int32_t max_pages, const float* r_k, const float* r_v,
                             float sm_scale, int32_t split_pages, const void* out, DecodePlan* plan) {
  if (oscar_status s = check_cache(cache, !all_raw, true)) return s;
  if (oscar_status s = plan_decode(batch, cache->n_kv_heads, n_q_heads, cache->d, max_seq_len, split_pages, all_raw, plan))
    return s;
  if (batch == 0) return OSCAR_OK;
  if (!q || !seq_lens || !bt_h || !out || (!all_raw && (!bt_q || !r_k || !r_v)))
    return fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (max_pages < 1 || int64_t(max_seq_len) > int64_t(max_pages) * 16)
    return fail(OSCAR_ERR_INVALID_ARG, "max_seq_len exceeds 16 * max_pages");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f)) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  if (batch > 65535) return fail(OSCAR_ERR_UNSUPPORTED, "batch above 65535");
  return OSCAR_OK;
}

oscar_status decode_launch(bool all_raw, const oscar_cache* cache, const void* q, int32_t batch, int32_t n_q_heads,
                           const int32_t* seq_lens, int32_t max_seq_len, const int32_t* bt_q, const int32_t* bt_h,
                           int32_t max_pages, const float* r_k, const float* r_v, float sm_scale,
                           const DecodePlan& plan, int32_t* counters, float* partials, void* out, void* stream,
                           const void* k_new, const void* v_new, float tau_k, float tau_v) {
  const int G = n_q_heads / cache->n_kv_heads;
  return hip_status(
      oscar_launch::paged_decode(cache->d, all_raw, cache->int2_pool, cache->n_int2_pages, cache->bf16_pool, cache->n_kv_heads, G,
                                 cache->n_sink, cache->n_recent, n_q_heads, q, batch, seq_lens, all_raw ? bt_h : bt_q,
                                 bt_h, max_pages, r_k, r_v, sm_scale, plan.per_unit, plan.unit_items, plan.first_int2, plan.fixed_ppw,
                                 plan.n_wg, plan.cap, max_seq_len, partials, counters, plan.rec_floats, out,
                                 4LL * batch * cache->n_kv_heads < device_cu_count(), k_new, v_new, tau_k, tau_v,
                                 static_cast<hipStream_t>(stream)),
      "decode launch");
}

}  // namespace oscar

static oscar_status decode_common(bool all_raw, const oscar_cache* cache, const void* q, int32_t batch,
                                  int32_t n_q_heads, const int32_t* seq_lens, int32_t max_seq_len,
                                  const int32_t* bt_q, const int32_t* bt_h, int32_t max_pages, const float* r_k,
                                  const float* r_v, float sm_scale, int32_t split_pages, void* workspace,
                                  size_t workspace_bytes, void* out, void* stream) {
  oscar::clear_error();
  DecodePlan plan;
  if (oscar_status s = oscar::decode_validate(all_raw, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h,
                                              max_pages, r_k, r_v, sm_scale, split_pages, out, &plan))
    return s;
  if (batch == 0) return OSCAR_OK;
  if (!workspace) return fail(OSCAR_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < plan.bytes) return fail(OSCAR_ERR_WORKSPACE, "workspace smaller than oscar_decode_workspace_bytes");
  int32_t* counters = static_cast<int32_t*>(workspace);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.counter_bytes);
  return oscar::decode_launch(all_raw, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h, max_pages, r_k,
                              r_v, sm_scale, plan, counters, partials, out, stream);
}

namespace {

// Work plan of the many-column attention (chunked prefill, INT4 decode): a
// workgroup takes one tile of 16 NWV query columns of one (sequence, KV
// head) and one chunk of `spc` steps of 32 tokens (BF16 page pairs,
// quantized page pairs, tiles of new rows); with more than one chunk per
// tile, records of 2 + 2d floats per column and chunk go to the workspace
// and a second launch merges them.  Automatic: about 2 (extend) or 3 (decode,
// one-wave workgroups) workgroups per compute unit, at least 8 (16) steps a
// chunk, which amortizes a chunk's query rotation and record.
struct AttendPlan {
  int n_ct, n_chunks, spc;
  size_t bytes;
};

oscar_status plan_attend(bool extend, int32_t batch, int32_t n_kv, int32_t n_q, int32_t d, int32_t S, int32_t W,
                         int32_t max_cache_len, int32_t max_new, int32_t split_steps, AttendPlan* plan) {
  if (batch < 0 || max_cache_len < 0 || max_new < 0) return fail(OSCAR_ERR_INVALID_ARG, "negative batch or lengths");
  if (!supported_d(d)) return fail(OSCAR_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (n_kv < 1 || n_q < 1 || n_q % n_kv) return fail(OSCAR_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if (S < 0 || W < 0) return fail(OSCAR_ERR_INVALID_ARG, "negative n_sink or n_recent");
  const int G = n_q / n_kv;
  if (G > 16) return fail(OSCAR_ERR_UNSUPPORTED, "query group size above 16");
  if (split_steps < 0) return fail(OSCAR_ERR_INVALID_ARG, "split_steps < 0");
  const int nct = oscar_launch::attend_cols(extend, d);  // query columns of a workgroup tile
  const long long cols = extend ? (long long)max_new * G : G;
  plan->n_ct = int(std::max(1LL, (cols + nct - 1) / nct));
  const long long pages = (max_cache_len + 15LL) / 16;
  const long long raw = std::min(pages, (S + 15LL) / 16 + (W + 15LL) / 16 + 2);
  const long long qsteps = (pages + 2) / 2, osteps = (raw + 1) / 2 + (extend ? (max_new + 31LL) / 32 : 0);
  const long long steps = qsteps + osteps;
  const long long units = (long long)batch * n_kv;
  if (units * plan->n_ct > (1LL << 30)) return fail(OSCAR_ERR_UNSUPPORTED, "grid too large; split the batch");
  // several chunks: quantized steps and the others in chunks of their own
  auto chunks_of = [&](long long sp) { return steps <= sp ? 1 : (qsteps + sp - 1) / sp + (osteps + sp - 1) / sp; };
  long long spc = split_steps;
  if (!spc) {
    // as many workgroups as fit on the device at once (the decode kernel
    // holds three per CU; extend is measured best at two) and no more
    // (measured: a few workgroups past a whole round cost more than longer
    // chunks), the steps spread evenly
    const long long target = (extend ? 2LL : 3LL) * device_cu_count();
    const long long base = std::max(1LL, units * plan->n_ct);
    const long long chunks = std::max(1LL, target / base);
    spc = std::max(8LL, (steps + chunks - 1) / chunks);
    if (chunks_of(spc) > chunks) {  // the smallest larger spc that fits (chunks_of does not grow with spc)
      long long lo = spc, hi = std::max(spc, steps);
      while (lo < hi) {
        const long long mid = lo + (hi - lo) / 2;
        if (chunks_of(mid) > chunks) lo = mid + 1;
        else hi = mid;
      }
      spc = lo;
    }
  }
  const long long n_chunks = chunks_of(spc);
  if (units * plan->n_ct * n_chunks > (1LL << 31) - 1) return fail(OSCAR_ERR_UNSUPPORTED, "grid too large; use a larger split_steps");
  if (n_chunks > 8192) return fail(OSCAR_ERR_UNSUPPORTED, "more than 8192 chunks per unit; use a larger split_steps");
  plan->spc = int(std::min<long long>(spc, 1 << 30));
  plan->n_chunks = int(n_chunks);
  plan->bytes = plan->n_chunks > 1 ? size_t(units) * plan->n_ct * plan->n_chunks * nct * (4 + 2 * size_t(d)) * 4 : 0;
  return OSCAR_OK;
}

oscar_status attend_common(bool extend, int bits, const oscar_cache* cache, const void* q, const void* k_new,
                           const void* v_new, int32_t batch, int32_t n_q_heads, const int32_t* cu,
                           const int32_t* clen, int32_t max_cache_len, int32_t max_new, const int32_t* bt_q,
                           const int32_t* bt_h, int32_t max_pages, const float* r_k, const float* r_v, float sm_scale,
                           int32_t split_steps, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  oscar::clear_error();
  if (oscar_status s = check_cache(cache, true, true)) return s;
  if (bits != 2 && bits != 4) return fail(OSCAR_ERR_UNSUPPORTED, "code_bits must be 2 or 4");
  AttendPlan plan;
  if (oscar_status s = plan_attend(extend, batch, cache->n_kv_heads, n_q_heads, cache->d, cache->n_sink,
                                   cache->n_recent, max_cache_len, max_new, split_steps, &plan))
    return s;
  if (batch == 0 || (extend && max_new == 0)) return OSCAR_OK;
  if (!q || !clen || !bt_q || !bt_h || !r_k || !r_v || !out || (extend && (!k_new || !v_new || !cu)))
    return fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (max_pages < 1 || int64_t(max_cache_len) > int64_t(max_pages) * 16)
    return fail(OSCAR_ERR_INVALID_ARG, "max cache length exceeds 16 * max_pages");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f)) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  if (plan.bytes && (!workspace || workspace_bytes < plan.bytes))
    return fail(OSCAR_ERR_WORKSPACE, "workspace missing or smaller than the workspace query's size");
  const int G = n_q_heads / cache->n_kv_heads;
  return hip_status(oscar_launch::paged_attend(cache->d, bits, extend, cache->int2_pool, int(std::min<int64_t>(cache->n_int2_pages, 0x7FFFFFFF)),
                                               cache->bf16_pool, int(std::min<int64_t>(cache->n_bf16_pages, 0x7FFFFFFF)),
                                               cache->n_kv_heads, G, cache->n_sink, cache->n_recent, n_q_heads, q,
                                               k_new, v_new, cu, clen, batch, bt_q, bt_h, max_pages, r_k, r_v,
                                               sm_scale, plan.n_ct, plan.n_chunks, plan.spc,
                                               static_cast<float*>(workspace), out, static_cast<hipStream_t>(stream)),
                    "attention launch");
}

}  // namespace

extern "C" {

oscar_status oscar_extend_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads, int32_t d,
                                          int32_t n_sink, int32_t n_recent, int32_t max_cache_len, int32_t max_new,
                                          int32_t split_steps, size_t* bytes) {
  oscar::clear_error();
  if (!bytes) return fail(OSCAR_ERR_INVALID_ARG, "bytes is NULL");
  AttendPlan plan;
  if (oscar_status s = plan_attend(true, batch, n_kv_heads, n_q_heads, d, n_sink, n_recent, max_cache_len, max_new,
                                   split_steps, &plan))
    return s;
  *bytes = plan.bytes;
  return OSCAR_OK;
}

oscar_status oscar_paged_extend_attn(const oscar_cache* cache, int32_t code_bits, const void* q, const void* k_new,
                                     const void* v_new, int32_t batch, int32_t n_q_heads, const int32_t* cu_rows,
                                     const int32_t* cache_lens, int32_t max_cache_len, int32_t max_new,
                                     const int32_t* bt_q, const int32_t* bt_h, int32_t max_pages, const float* r_k,
                                     const float* r_v, float sm_scale, int32_t split_steps, void* workspace,
                                     size_t workspace_bytes, void* out, void* stream) {
  return attend_common(true, code_bits, cache, q, k_new, v_new, batch, n_q_heads, cu_rows, cache_lens, max_cache_len,
                       max_new, bt_q, bt_h, max_pages, r_k, r_v, sm_scale, split_steps, workspace, workspace_bytes,
                       out, stream);
}

oscar_status oscar_decode_int4_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads, int32_t d,
                                               int32_t n_sink, int32_t n_recent, int32_t max_seq_len,
                                               int32_t split_steps, size_t* bytes) {
  oscar::clear_error();
  if (!bytes) return fail(OSCAR_ERR_INVALID_ARG, "bytes is NULL");
  AttendPlan plan;
  if (oscar_status s = plan_attend(false, batch, n_kv_heads, n_q_heads, d, n_sink, n_recent, max_seq_len, 0,
                                   split_steps, &plan))
    return s;
  *bytes = plan.bytes;
  return OSCAR_OK;
}

oscar_status oscar_paged_decode_attn_int4(const oscar_cache* cache, const void* q, int32_t batch, int32_t n_q_heads,
                                          const int32_t* seq_lens, int32_t max_seq_len, const int32_t* bt_q,
                                          const int32_t* bt_h, int32_t max_pages, const float* r_k, const float* r_v,
                                          float sm_scale, int32_t split_steps, void* workspace,
                                          size_t workspace_bytes, void* out, void* stream) {
  return attend_common(false, 4, cache, q, nullptr, nullptr, batch, n_q_heads, nullptr, seq_lens, max_seq_len, 0,
                       bt_q, bt_h, max_pages, r_k, r_v, sm_scale, split_steps, workspace, workspace_bytes, out,
                       stream);
}

oscar_status oscar_paged_decode_attn(const oscar_cache* cache, const void* q, int32_t batch, int32_t n_q_heads,
                                     const int32_t* seq_lens, int32_t max_seq_len, const int32_t* bt_q,
                                     const int32_t* bt_h, int32_t max_pages, const float* r_k, const float* r_v,
                                     float sm_scale, int32_t split_pages, void* workspace, size_t workspace_bytes,
                                     void* out, void* stream) {
  return decode_common(false, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h, max_pages, r_k, r_v,
                       sm_scale, split_pages, workspace, workspace_bytes, out, stream);
}

oscar_status oscar_decode_step(const oscar_cache* cache, const void* k_new, const void* v_new, const void* q,
                               int32_t batch, int32_t n_q_heads, const int32_t* seq_lens, int32_t max_seq_len,
                               const int32_t* bt_q, const int32_t* bt_h, int32_t max_pages, const float* r_k,
                               const float* r_v, float tau_k, float tau_v, float sm_scale, int32_t split_pages,
                               void* workspace, size_t workspace_bytes, void* out, void* stream) {
  oscar::clear_error();
  DecodePlan plan;
  if (oscar_status s = oscar::decode_validate(false, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h,
                                              max_pages, r_k, r_v, sm_scale, split_pages, out, &plan))
    return s;
  if (batch == 0) return OSCAR_OK;
  if (!k_new || !v_new) return fail(OSCAR_ERR_INVALID_ARG, "null device pointer");
  if (!(tau_k > 0.f) || !(tau_v > 0.f) || !std::isfinite(tau_k) || !std::isfinite(tau_v))
    return fail(OSCAR_ERR_INVALID_ARG, "clip thresholds must be finite and positive");
  if (!workspace) return fail(OSCAR_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < plan.bytes) return fail(OSCAR_ERR_WORKSPACE, "workspace smaller than oscar_decode_workspace_bytes");
  int32_t* counters = static_cast<int32_t*>(workspace);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.counter_bytes);
  if (!plan.per_unit && (long long)batch * cache->n_kv_heads > device_cu_count()) {
    // Balanced slices over more units than CUs: a fused launch would give
    // every workgroup several quantized tokens, each a chain of round trips
    // to memory inside the workgroup; the few-row update kernel does them all
    // in parallel first (measured faster from 512 units on), then the decode.
    if (oscar_status s = hip_status(
            oscar_launch::decode_step_update(cache->d, cache->n_kv_heads, cache->n_sink, cache->n_recent,
                                             cache->int2_pool, cache->bf16_pool, k_new, v_new, batch, seq_lens,
                                             bt_q, bt_h, max_pages, r_k, r_v, tau_k, tau_v,
                                             static_cast<hipStream_t>(stream)),
            "decode_step_update launch"))
      return s;
    return oscar::decode_launch(false, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h, max_pages,
                                r_k, r_v, sm_scale, plan, counters, partials, out, stream);
  }
  // one launch (per-unit items, or balanced slices that count each unit's
  // quantized token in its row)
  return oscar::decode_launch(false, cache, q, batch, n_q_heads, seq_lens, max_seq_len, bt_q, bt_h, max_pages, r_k,
                              r_v, sm_scale, plan, counters, partials, out, stream, k_new, v_new, tau_k, tau_v);
}

oscar_status oscar_paged_decode_attn_bf16(const oscar_cache* cache, const void* q, int32_t batch, int32_t n_q_heads,
                                          const int32_t* seq_lens, int32_t max_seq_len, const int32_t* bt_h,
                                          int32_t max_pages, float sm_scale, int32_t split_pages, void* workspace,
                                          size_t workspace_bytes, void* out, void* stream) {
  return decode_common(true, cache, q, batch, n_q_heads, seq_lens, max_seq_len, nullptr, bt_h, max_pages, nullptr,
                       nullptr, sm_scale, split_pages, workspace, workspace_bytes, out, stream);
}

}  // extern "C"
