// Launch functions of the liboscar kernels (internal; called by abi.hip after
// argument validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar_launch {

hipError_t quantize_append(int d, int bits, int n_kv, void* pool, const void* k_new, const void* v_new, int64_t n_rows,
                           const int32_t* row_seq, const int32_t* row_pos, const int32_t* bt_q,
                           int32_t max_pages, const float* r_k, const float* r_v, float tau_k, float tau_v,
                           int n_cus, hipStream_t stream);

// one decode step's cache update: new tokens to BF16 slots, the token
// leaving each recent window to INT2
hipError_t decode_step_update(int d, int n_kv, int n_sink, int n_recent, void* int2_pool, void* bf16_pool,
                              const void* k_new, const void* v_new, int batch, const int32_t* seq_lens,
                              const int32_t* bt_q, const int32_t* bt_h, int32_t max_pages, const float* r_k,
                              const float* r_v, float tau_k, float tau_v, hipStream_t stream);

// calibration second moments C(h) = (1 / (N G)) sum x^T x over the G heads of
// each KV group (float64 out, zeroed first)
hipError_t calib_gram(int d, const void* x, int64_t n_rows, int n_x_heads, int n_kv, void* out, hipStream_t stream);

size_t decode_lds_bytes(int d, int G, bool all_raw);
int decode_max_records();  // record slots per (sequence, KV head) the merge can hold
int decode_min_slice();    // pages per workgroup slice at least
int decode_seg_pages();    // extra positions per nonempty page range in balanced slices (at most)
int decode_seg_pages_of(int G);  // the same for query group G
int decode_own_pages();    // extra positions of a unit whose fused step quantizes a token

// k_new != nullptr: the fused decode step (the step's cache update in the same launch)
hipError_t paged_decode(int d, bool all_raw, const void* int2_pool, int n_int2_pages, const void* bf16_pool, int n_kv, int G, int S,
                        int W, int Hq, const void* q, int batch, const int32_t* seq_lens, const int32_t* bt_q,
                        const int32_t* bt_h, int max_pages, const float* r_k, const float* r_v, float sm_scale,
                        bool per_unit, int unit_items, int first_int2, int fixed_ppw, int n_wg, int cap, int max_seq_len,
                        float* partials, int32_t* counters, int rec_floats, void* out, bool speculate,
                        const void* k_new, const void* v_new, float tau_k, float tau_v, hipStream_t stream);

// paged attention with many query columns (extend: chunked prefill over
// INT2/INT4 pages; otherwise decode over an INT4 cache), and its merge
size_t attend_lds_bytes(int d, bool extend);
int attend_waves(bool extend, int d);
int attend_cols(bool extend, int d);
hipError_t paged_attend(int d, int bits, bool extend, const void* qpool, int n_qpages, const void* bf16_pool,
                        int n_bpages, int n_kv, int G, int S, int W, int Hq, const void* q, const void* k_new,
                        const void* v_new, const int32_t* cu, const int32_t* clen, int batch, const int32_t* bt_q,
                        const int32_t* bt_h, int max_pages, const float* r_k, const float* r_v, float sm_scale,
                        int n_ct, int n_chunks, int spc, float* rec, void* out, hipStream_t stream);

}  // namespace oscar_launch
