// Internal declarations shared by the HIP translation units of liboscar
// (argument checks, decode planning and the decode launch); not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace oscar {

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Decode work planning shared by the workspace query and the decode calls.
struct DecodePlan {
  bool per_unit;    // per-unit items, or balanced slices over all units
  int unit_items;   // per-unit items: workgroups per (sequence, KV head)
  int first_int2;   // per-unit items: INT2 pages item 0 takes after the BF16 pages (0: none)
  int fixed_ppw;    // per-unit items: pages per item; slices: pages per slice (0: spread evenly)
  int n_wg;         // workgroups in the grid
  int cap;          // record slots per (sequence, KV head)
  int rec_floats;
  size_t counter_bytes;
  size_t bytes;     // counters, then cap records per (sequence, KV head)
};

oscar_status plan_decode(int32_t batch, int32_t n_kv, int32_t n_q, int32_t d, int32_t max_seq_len,
                         int32_t split_pages, bool all_raw, DecodePlan* plan);

// OSCAR_ERR_HIP with detail for a failed HIP call, else OSCAR_OK.
oscar_status hip_status(hipError_t e, const char* what);
// Validates a cache description (geometry, the pools the call needs).
oscar_status check_cache(const oscar_cache* c, bool need_int2, bool need_bf16);

// Host-visible checks of a decode call (everything but the workspace) and
// its work plan.
oscar_status decode_validate(bool all_raw, const oscar_cache* cache, const void* q, int32_t batch,
                             int32_t n_q_heads, const int32_t* seq_lens, int32_t max_seq_len, const int32_t* bt_q,
                             const int32_t* bt_h, int32_t max_pages, const float* r_k, const float* r_v,
                             float sm_scale, int32_t split_pages, const void* out, DecodePlan* plan);
// The decode launch with its arrival counters and records at the given device addresses.
oscar_status decode_launch(bool all_raw, const oscar_cache* cache, const void* q, int32_t batch, int32_t n_q_heads,
                           const int32_t* seq_lens, int32_t max_seq_len, const int32_t* bt_q, const int32_t* bt_h,
                           int32_t max_pages, const float* r_k, const float* r_v, float sm_scale,
                           const DecodePlan& plan, int32_t* counters, float* partials, void* out, void* stream,
                           const void* k_new = nullptr, const void* v_new = nullptr, float tau_k = 0.f,
                           float tau_v = 0.f);

}  // namespace oscar
