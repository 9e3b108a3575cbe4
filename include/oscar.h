/*
 * oscar.h — C ABI of liboscar: the online hot path of OSCAR (Offline Spectral
 * Covariance-Aware Rotation for 2-bit KV cache quantization) on AMD Instinct
 * MI355X (gfx950).
 *
 * Sources cited in this header (the method is described in prose only):
 *   [TS]  "Technical Summary: OSCAR - Offline Spectral Covariance-Aware Rotation
 *         for 2-bit KV Cache Quantization" (gist.science), sections 2.1, 2.2.A
 *         (Offline Calibration Phase), 2.2.B (Online Serving Phase), 4.
 *   [AB]  the arXiv abstract of "OSCAR: Offline Spectral Covariance-Aware
 *         Rotation for 2-bit KV Cache Quantization" (mlsanity.com paper page,
 *         section "Abstract (arXiv)").
 * Where the sources are silent, the reading taken is stated next to the
 * definition ("Reading:").
 *
 * Conventions used everywhere below
 *   d          head dimension, 64 or 128.
 *   H_kv, H_q  key/value heads and query heads; G = H_q / H_kv, 1 <= G <= 16.
 *              Query head i reads KV head floor(i / G).
 *   page       16 consecutive token positions [16p, 16p + 16) of one sequence.
 *   group      32 consecutive rotated channels [32g, 32g + 32); n_g = d / 32.
 *   rows       vectors are row vectors; a rotation acts as y = x . R, with R
 *              stored row-major as R[k][c] (k = input channel, c = output).
 *   bf16, f16  IEEE-754 binary16 ("f16") and bfloat16 ("bf16") bit patterns,
 *              little-endian, stored as uint16.
 *
 * Ownership and execution
 *   The caller owns every buffer.  The library never allocates device memory,
 *   never synchronises a stream and keeps no state apart from a thread-local
 *   error string.  Device calls are asynchronous on the given stream
 *   (hipStream_t passed as void*; NULL = the null stream).  No call throws.
 *
 * Errors
 *   Every call validates its host-visible arguments (pointers, geometry,
 *   sizes) before launching anything; on a violation it launches nothing and
 *   returns OSCAR_ERR_INVALID_ARG, OSCAR_ERR_UNSUPPORTED or
 *   OSCAR_ERR_WORKSPACE.  A failed launch returns OSCAR_ERR_HIP.  Device-side
 *   contents (page ids inside block tables, sequence lengths, row positions)
 *   are preconditions stated per call; they are not checked.
 *   oscar_last_error() returns a readable detail for the last non-OK status of
 *   the calling thread.
 */
#ifndef OSCAR_H_
#define OSCAR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OSCAR_OK = 0,
  OSCAR_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shape   */
  OSCAR_ERR_UNSUPPORTED = 2, /* geometry outside d in {64,128}, G in [1,16], ...  */
  OSCAR_ERR_NUMERIC = 3,     /* non-finite input or eigensolver non-convergence   */
  OSCAR_ERR_WORKSPACE = 4,   /* workspace pointer null or smaller than required   */
  OSCAR_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed        */
} oscar_status;

#define OSCAR_PAGE_TOKENS 16
#define OSCAR_GROUP_CHANNELS 32
#define OSCAR_VERSION 1

/* Name of a status code ("OSCAR_OK", ...). Never NULL. */
const char* oscar_status_string(oscar_status s);
/* Detail for the calling thread's last non-OK status; "" if none. */
const char* oscar_last_error(void);
/* OSCAR_VERSION of the built library. */
int32_t oscar_version(void);

/* ------------------------------------------------------------------------ *
 * Offline calibration (host, synchronous, float64 arithmetic inside).
 *
 * Computes, per KV head h with query group Q(h) = {hG, ..., hG + G - 1}
 * ([TS] 2.1 and 2.2.A steps 1-4; [AB]):
 *   C_Q(h) = 1/(N G) sum_{i in Q(h)} Q_i^T Q_i              (query-aware key
 *            target; Q_i is the [N, d] matrix of query head i's rows)
 *   C_S(h) = 1/(N G) sum_{i in Q(h)} O_i^T O_i,  O_i = S_i V_h (score-aware value
 *            target V^T S^T S V / N; S_i is the attention-score matrix)
 *   U = eigenvectors of C, ordered by descending eigenvalue
 *   R = U . H . P_br  with H = H_d / sqrt(d) (Sylvester Hadamard, H_1 = [1],
 *            H_2n = [[H_n, H_n], [H_n, -H_n]]) and P_br[r][c] = 1 iff r is the
 *            log2(d)-bit reversal of c (an involution).
 *   R_K uses U_Q (of C_Q), R_V uses U_S (of C_S).
 *   tau_K (tau_V) = the clip_quantile quantile of |K_h . R_K(h)| (|V_h . R_V(h)|)
 *            pooled over all N rows, all KV heads and all d channels ([TS] 2.2.A
 *            step 4: one threshold per layer).
 * Readings:
 *   - S_i = row-softmax(Q_i K_h^T / sqrt(d) + causal mask), i.e. calibration
 *     row r attends to rows 0..r.  If o_calib is given it is used as O_i
 *     directly (a model run can capture S V itself).
 *   - Eigenvector sign: each column of U is negated if needed so that its
 *     entry of largest magnitude is positive (lowest index on ties).
 *   - Quantile: the M values |y| sorted ascending a[0..M-1]; rr = q (M - 1);
 *     tau = a[floor(rr)] + (rr - floor(rr)) (a[floor(rr)+1] - a[floor(rr)]).
 * Eigen-decomposition is a cyclic Jacobi iteration in float64 that stops
 * when every off-diagonal entry is at most 1e-14 * ||C||_F, after at most
 * max_sweeps sweeps (0 selects 64); not reaching that returns
 * OSCAR_ERR_NUMERIC.
 * n_threads: host worker threads for the calibration attention (0 = all).
 * Inputs (host, row-major float32): q_calib [n_rows][H_kv*G][d],
 * k_calib and v_calib [n_rows][H_kv][d], o_calib NULL or [n_rows][H_kv*G][d].
 * Outputs (host, float64): r_k, r_v [H_kv][d][d]; *tau_k, *tau_v;
 * eig_k, eig_v NULL or [H_kv][d] (descending).
 * Errors: INVALID_ARG for null required pointers, n_rows < 2, H_kv < 1 or
 * clip_quantile outside (0, 1]; UNSUPPORTED for d not in {64, 128} or G
 * outside [1, 16]; NUMERIC for a non-finite input value or non-convergence.
 * ------------------------------------------------------------------------ */
oscar_status oscar_build_rotation(int32_t d, int32_t n_kv_heads, int32_t group_q,
                                  int64_t n_rows, const float* q_calib,
                                  const float* k_calib, const float* v_calib,
                                  const float* o_calib, double clip_quantile,
                                  int32_t max_sweeps, int32_t n_threads,
                                  double* r_k, double* r_v, double* tau_k,
                                  double* tau_v, double* eig_k, double* eig_v);

/* ------------------------------------------------------------------------ *
 * Calibration targets on the GPU ([TS] 2.1 and 2.2.A step 1: the key target
 * is the query second moment Q^T Q / N and the value target V^T S^T S V / N =
 * O^T O / N with O = S V, each pooled over the query heads of a KV group).
 * For x the Q rows (or the O rows) of a calibration forward pass:
 *   out[h] = (1 / (N G)) sum_{n < N} sum_{i = hG}^{hG+G-1} x[n][i]^T x[n][i]
 * with G = n_x_heads / n_kv_heads (x[n][i] a row vector, so out[h] is d x d).
 * The Gram products run on the bf16 matrix cores (exact products, float32
 * sums over blocks of 256 pooled rows, float64 sums of the blocks by atomic
 * adds, so the last bits may differ from run to run).
 * x: device bf16 [n_rows][n_x_heads][d], 16-byte aligned.  out: device
 * float64 [n_kv_heads][d][d], overwritten (the call zeroes it, accumulates
 * into it with atomic adds, then fills the lower triangle; three launches on
 * the stream), not overlapping x.
 * Errors: INVALID_ARG for null pointers, n_rows < 1, n_kv_heads < 1,
 * n_x_heads not a positive multiple of n_kv_heads or x not 16-byte aligned;
 * UNSUPPORTED for d not in {64, 128}, G > 16 or more than 2^39 pooled rows. */
oscar_status oscar_calib_gram(const void* x, int64_t n_rows, int32_t n_x_heads,
                              int32_t n_kv_heads, int32_t d, double* out, void* stream);

/* oscar_build_rotation's steps 2-4 from given targets (host, float64
 * [n_kv_heads][d][d], e.g. copied back from oscar_calib_gram): each target is
 * symmetrised ((C + C^T) / 2), decomposed and composed exactly as there; the
 * clip thresholds come from k_calib, v_calib (host float32
 * [n_rows][n_kv_heads][d]).  Outputs and errors as oscar_build_rotation
 * (NUMERIC also for a non-finite target entry). */
oscar_status oscar_build_rotation_from_targets(int32_t d, int32_t n_kv_heads,
                                               const double* c_q, const double* c_s,
                                               int64_t n_rows, const float* k_calib,
                                               const float* v_calib, double clip_quantile,
                                               int32_t max_sweeps, int32_t n_threads,
                                               double* r_k, double* r_v, double* tau_k,
                                               double* tau_v, double* eig_k, double* eig_v);

/* ------------------------------------------------------------------------ *
 * Comparison rotations through the same cache path ([TS] 1: Hadamard
 * transforms are the data-oblivious rotations OSCAR improves on; [TS] 4,
 * "Accuracy Preservation": naive INT2 and Hadamard-only are the baselines).
 *   OSCAR_ROTATION_HADAMARD: R_K = R_V = H . P_br for every KV head, the
 *       fixed factor of the composite rotation above (U = I);
 *   OSCAR_ROTATION_IDENTITY: R_K = R_V = I (no rotation).
 * tau_K, tau_V: the clip_quantile quantiles of |K_h . R| and |V_h . R| as in
 * oscar_build_rotation.  The results feed oscar_quantize_append and
 * oscar_paged_decode_attn unchanged.
 * Inputs (host, row-major float32): k_calib, v_calib [n_rows][H_kv][d].
 * Outputs (host, float64): r_k, r_v [H_kv][d][d]; *tau_k, *tau_v.
 * n_threads: host worker threads (0 = all).
 * Errors: INVALID_ARG for an unknown variant, null pointers, n_rows < 2,
 * H_kv < 1 or clip_quantile outside (0, 1]; UNSUPPORTED for d not in
 * {64, 128}; NUMERIC for a non-finite input value.
 * ------------------------------------------------------------------------ */
typedef enum {
  OSCAR_ROTATION_HADAMARD = 1,
  OSCAR_ROTATION_IDENTITY = 2
} oscar_rotation_variant;

oscar_status oscar_build_fixed_rotation(int32_t variant, int32_t d, int32_t n_kv_heads,
                                        int64_t n_rows, const float* k_calib,
                                        const float* v_calib, double clip_quantile,
                                        int32_t n_threads, double* r_k, double* r_v,
                                        double* tau_k, double* tau_v);

/* ------------------------------------------------------------------------ *
 * Paged cache geometry ([TS] 2.2.B: sink and recent tokens in BF16, the
 * middle history in INT2 after rotation and clipping, paged and compatible
 * with prefix caching; [AB]: paged KV-cache serving).
 *
 * Regions of a sequence of length L (L counts the token being decoded):
 *   sink   = [0, min(S, L))
 *   recent = [max(S, L - W), L)
 *   middle = [S, L - W) when L - W > S, else empty
 * with S = n_sink and W = n_recent.  Sink and recent tokens live raw
 * (unrotated) in BF16 pages; middle tokens live rotated, clipped and
 * quantized in INT2 pages.
 *
 * Block tables bt_q and bt_h are int32 [B][max_pages] (row stride
 * max_pages).  Entry [b][p] names the physical INT2 (resp. BF16) page that
 * holds logical page p = floor(t / 16) of sequence b.  bt_q[b][p] is read
 * only when page p holds a middle token, bt_h[b][p] only when it holds a sink
 * or recent token; other entries may hold any value (e.g. -1).  Several
 * sequences may name the same physical page (a shared prefix); pages are
 * only read by the decode call.
 *
 * INT2 page.  A physical INT2 page holds all H_kv heads; head h of page P
 * starts at byte (P * H_kv + h) * B_q, B_q = 12 d  (1536 B at d = 128, 768 B
 * at d = 64).  Inside it, six areas follow each other:
 *   KC  K codes    4d bytes = (16 d / 64) uint32 words
 *   VC  V codes    4d bytes
 *   KS  K scales   f16 [16 slots][n_g]
 *   KZ  K zeros    f16 [16 slots][n_g]
 *   VS  V scales   f16 [4][n_g][4]   index (q n_g + g) 4 + r, slot = 4q + r
 *   VZ  V zeros    f16 [4][n_g][4]   same index
 * A code is a 2-bit unsigned integer c in {0,1,2,3} at bit positions
 * [b, b+1] of a little-endian uint32 word.  With n_w = d / 64:
 *   KC: the code of slot m, channel c lives in word (quad * 16 + m) * n_w + w,
 *       where g = c / 32, hb = (c / 16) % 2, quad = (c / 4) % 4, r = c % 4,
 *       w = g / 2, and bit b = 16 (r % 2) + 8 (g % 2) + 4 hb + 2 (r / 2).
 *   VC: the code of slot t = 4q + r (q, r in 0..3), channel c lives in word
 *       (q * 16 + c16) * n_w + w, where c16 = c % 16, blk = c / 16,
 *       w = blk / 4, bb = blk % 4, and bit b = 16 (r % 2) + 8 (r / 2) + 2 bb.
 * Slots of a page that hold no middle token are never read.
 * The decoded (dequantized) value of a code is c * s + z, with s, z the f16
 * scale and zero of that slot's channel group.
 *
 * BF16 page.  Head h of physical BF16 page P starts at element
 * (P * H_kv + h) * 32 d of a bf16 array and holds
 *   K  [16 slots][d]    (token-major)
 *   V  [d][16 slots]    (channel-major)
 * ------------------------------------------------------------------------ */
size_t oscar_int2_page_bytes(int32_t d, int32_t n_kv_heads); /* per physical page */
size_t oscar_bf16_page_bytes(int32_t d, int32_t n_kv_heads); /* per physical page */

typedef struct {
  int32_t d;            /* 64 or 128                                          */
  int32_t n_kv_heads;   /* H_kv >= 1                                          */
  int32_t n_sink;       /* S >= 0                                             */
  int32_t n_recent;     /* W >= 0                                             */
  void* int2_pool;      /* device, n_int2_pages * oscar_int2_page_bytes bytes */
  int64_t n_int2_pages;
  void* bf16_pool;      /* device, n_bf16_pages * oscar_bf16_page_bytes bytes */
  int64_t n_bf16_pages;
} oscar_cache;

/* ------------------------------------------------------------------------ *
 * Quantize-append ([TS] 2.2.B: the middle history is stored in INT2 after the
 * fixed rotation and clipping; 2.2.A step 4 for the clip).
 * For every row j < n_rows, every KV head h, and X in {K, V}:
 *   y = x_j,h . R_X(h)                       (R_K or R_V, float32 [H_kv][d][d])
 *   y = min(max(y, -tau_X), tau_X)
 *   per group g: mn = min, mx = max of its 32 values;
 *       s = f16_rne((mx - mn) / 3), z = f16_rne(mn)
 *   code = clamp(rne((y - z) / s), 0, 3); code = 0 where s == 0
 * and the codes, s and z are written to slot row_pos[j] % 16 of INT2 page
 * bt_q[row_seq[j]][row_pos[j] / 16] in the layout above.  Other slots of the
 * page are left unchanged.
 * Readings: asymmetric INT2 with z = group minimum and s = range / 3, groups
 * of 32 consecutive rotated channels per token, codes taken against the
 * stored f16 s and z, round-half-to-even, symmetric clip.
 * k_new, v_new: device bf16 [n_rows][H_kv][d].  row_seq, row_pos: device
 * int32 [n_rows].  bt_q: device int32 [B][max_pages].  r_k, r_v: device
 * float32 [H_kv][d][d].
 * Preconditions (device contents): 0 <= row_pos[j] < 16 max_pages, the named
 * page is valid and not shared with another sequence, and no two rows name
 * the same (sequence, position).
 * Arithmetic: y is accumulated in float32, from float32 products for up to
 * 64 rows per call and, for more rows, on the matrix cores from an f16
 * hi + lo split of 256 R (22 significant bits) and an exact f16 copy of x,
 * so a code can differ from exact arithmetic only when (y - z) / s lies
 * within about 1e-5 of a rounding boundary.  Up to 64 rows, values of
 * magnitude beyond 2^120 may overflow the float32 products.
 * n_rows == 0 returns OSCAR_OK and launches nothing.
 * ------------------------------------------------------------------------ */
oscar_status oscar_quantize_append(const oscar_cache* cache, const void* k_new,
                                   const void* v_new, int64_t n_rows,
                                   const int32_t* row_seq, const int32_t* row_pos,
                                   const int32_t* bt_q, int32_t max_pages,
                                   const float* r_k, const float* r_v,
                                   float tau_k, float tau_v, void* stream);

/* Raw BF16 rows into BF16 pages (the sink and recent store of [TS] 2.2.B):
 * row j, head h goes to slot row_pos[j] % 16 of BF16 page
 * bt_h[row_seq[j]][row_pos[j] / 16], K token-major and V channel-major.
 * Same argument conventions and preconditions as oscar_quantize_append. */
oscar_status oscar_write_bf16(const oscar_cache* cache, const void* k_new,
                              const void* v_new, int64_t n_rows,
                              const int32_t* row_seq, const int32_t* row_pos,
                              const int32_t* bt_h, int32_t max_pages, void* stream);

/* One decode step's cache update in one launch ([TS] 2.2.B "Mixed-Precision
 * Layout": sink and recent tokens stay in BF16, the middle history is INT2
 * after the fixed rotation and clip).  For every sequence b < batch with
 * L = seq_lens[b] >= 1 (the length the step decodes, its new token at
 * position L - 1 included), with S = n_sink and W = n_recent of the cache:
 *   - the new token (row b of k_new, v_new) is written to slot (L - 1) % 16 of
 *     BF16 page bt_h[b][(L - 1) / 16] when it is a sink or recent token
 *     (W >= 1, or L - 1 < S);
 *   - the token entering the middle history, t = L - 1 - W (t = L - 1 when
 *     W = 0), if t >= S, is quantized exactly as oscar_quantize_append does
 *     into slot t % 16 of INT2 page bt_q[b][t / 16]; with W >= 1 its raw row
 *     is read from its BF16 slot (bt_h[b][t / 16], t % 16), where the
 *     previous steps left it.
 * Sequences with L <= 0 are skipped.  Nothing else is written.
 * k_new, v_new: device bf16 [batch][H_kv][d].  seq_lens: device int32 [batch].
 * bt_q, bt_h: device int32 [B][max_pages] with B >= batch.  r_k, r_v: device
 * float32 [H_kv][d][d].
 * Preconditions (device contents): the named pages are valid and not shared
 * with another sequence; the BF16 slot of token t still holds its row and is
 * not the BF16 slot the new token goes to.
 * Arithmetic: float32 products, as oscar_quantize_append uses for up to 64
 * rows, whatever the batch.
 * Errors: as oscar_quantize_append; both pools of the cache are required.
 * batch == 0 returns OSCAR_OK and launches nothing. */
oscar_status oscar_decode_step_update(const oscar_cache* cache, const void* k_new,
                                      const void* v_new, int32_t batch,
                                      const int32_t* seq_lens, const int32_t* bt_q,
                                      const int32_t* bt_h, int32_t max_pages,
                                      const float* r_k, const float* r_v,
                                      float tau_k, float tau_v, void* stream);

/* ------------------------------------------------------------------------ *
 * Paged decode attention over the mixed cache ([TS] 2.2.B "kernel
 * integration": unpacking, dequantization, inverse rotation and attention for
 * the INT2 history in one fused kernel, paged and prefix-cache compatible;
 * [AB]).  For sequence b, query head i, h = floor(i / G), scale sm_scale:
 *   logit_j = sm_scale * q_i . k_j                  j in sink or recent (raw)
 *   logit_j = sm_scale * (q_i . R_K(h)) . kh_j      j in middle, kh_j the
 *                                                   decoded rotated key
 *   p = softmax(logit) over j in [0, L_b)
 *   out_i = sum_{raw j} p_j v_j + (sum_{middle j} p_j vh_j) . R_V(h)^T
 * Because R is orthogonal this is attention over the decoded cache mapped
 * back to the original basis (the "inverse rotation").  Output is bf16.
 * The kernel splits the pages of each (sequence, KV head) over workgroups
 * and merges the partial results with a log-sum-exp reduction in the same
 * launch.
 * q: device bf16 [B][H_q][d].  seq_lens: device int32 [B].  bt_q, bt_h:
 * device int32 [B][max_pages].  r_k, r_v: device float32 [H_kv][d][d].
 * max_seq_len: host-known upper bound of seq_lens, <= 16 max_pages (sizes the
 * grid).  split_pages: pages per workgroup item of one (sequence, KV head),
 * a multiple of 8 in [8, 2^20] with at most 255 INT2 items per sequence, or 0
 * for automatic (per-(sequence, KV head) items sized to the device's compute
 * units for small batches, equal page slices over the whole batch for large
 * ones).  workspace: device memory of at least
 * oscar_decode_workspace_bytes(...) bytes, prepared once with
 * oscar_decode_workspace_init.  It holds one arrival counter per (sequence,
 * KV head), which the call counts up and its last workgroup of that pair
 * resets to zero, and the per-workgroup partial results; every completed call
 * leaves it prepared.  A call that does not complete (a launch error, a
 * device fault) can leave counters non-zero, and a later call on that
 * workspace then merges at the wrong time and returns wrong values:
 * oscar_decode_workspace_init restores it.
 * out: device bf16 [B][H_q][d].
 * Preconditions (device contents): 0 <= seq_lens[b] <= max_seq_len, valid
 * page ids wherever they are read.  A sequence with seq_lens[b] == 0 gets a
 * zero output.  Two calls sharing one workspace must not overlap in time.
 * Arithmetic: the rotated query is rounded to f16 once; probabilities enter
 * the value products as f16; accumulation is float32.
 * batch == 0 returns OSCAR_OK and launches nothing.
 * ------------------------------------------------------------------------ */
oscar_status oscar_decode_workspace_bytes(int32_t batch, int32_t n_kv_heads,
                                          int32_t n_q_heads, int32_t d,
                                          int32_t max_seq_len, int32_t split_pages,
                                          size_t* bytes);
oscar_status oscar_decode_workspace_init(void* workspace, size_t workspace_bytes,
                                         void* stream);
oscar_status oscar_paged_decode_attn(const oscar_cache* cache, const void* q,
                                     int32_t batch, int32_t n_q_heads,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     const int32_t* bt_q, const int32_t* bt_h,
                                     int32_t max_pages, const float* r_k,
                                     const float* r_v, float sm_scale,
                                     int32_t split_pages, void* workspace,
                                     size_t workspace_bytes, void* out, void* stream);

/* One decode step in one launch ([TS] 2.2.B: the middle history is stored in
 * INT2 after the fixed rotation and clip, sink and recent tokens stay BF16,
 * and the fused kernel attends over that cache): exactly
 * oscar_decode_step_update(cache, k_new, v_new, batch, seq_lens, bt_q, bt_h,
 * max_pages, r_k, r_v, tau_k, tau_v) followed by
 * oscar_paged_decode_attn(cache, q, ...) with the same arguments, so the
 * cache afterwards holds the same bytes and the output meets the same
 * definition.  With at most as many (sequence, KV head) units as compute
 * units it is one launch: the workgroup that reads the new token's BF16 page
 * writes it there first, and the workgroup that reads the last middle page
 * quantizes the token entering the middle history, writes it to its INT2
 * slot and attends to it from the decoded values (its slot in the page is
 * not read).  With more units it launches the update kernel, then the
 * decode, on the same stream.  Arguments, workspace rules, preconditions and
 * errors as the two calls. */
oscar_status oscar_decode_step(const oscar_cache* cache, const void* k_new, const void* v_new,
                               const void* q, int32_t batch, int32_t n_q_heads,
                               const int32_t* seq_lens, int32_t max_seq_len,
                               const int32_t* bt_q, const int32_t* bt_h, int32_t max_pages,
                               const float* r_k, const float* r_v, float tau_k, float tau_v,
                               float sm_scale, int32_t split_pages, void* workspace,
                               size_t workspace_bytes, void* out, void* stream);

/* The same decode with every token in BF16 pages (bt_h for all positions,
 * no rotation): the uncompressed baseline the INT2 cache is compared with
 * ([TS] 4 and [AB] compare OSCAR's decode against BF16).  Same arguments and
 * workspace rules minus the INT2 table and rotations; the cache's n_sink and
 * n_recent are ignored. */
oscar_status oscar_paged_decode_attn_bf16(const oscar_cache* cache, const void* q,
                                          int32_t batch, int32_t n_q_heads,
                                          const int32_t* seq_lens, int32_t max_seq_len,
                                          const int32_t* bt_h, int32_t max_pages,
                                          float sm_scale, int32_t split_pages,
                                          void* workspace, size_t workspace_bytes,
                                          void* out, void* stream);

/* ------------------------------------------------------------------------ *
 * INT4 cache variant ([TS] 4 "Scalability": the INT4 KV cache OSCAR's
 * capacity is compared with).  The same rotation, clip and per-token group-32
 * asymmetric quantizer with 16 levels: s = f16_rne((mx - mn) / 15),
 * z = f16_rne(mn), code = clamp(rne((y - z) / s), 0, 15), code 0 where
 * s == 0.  Sink and recent tokens stay in the BF16 pages as for INT2.
 *
 * INT4 page.  Head h of physical page P starts at byte (P * H_kv + h) * B_4,
 * B_4 = 20 d (2560 B at d = 128, 1280 B at d = 64), and holds, one after the
 * other: K codes [16 slots][d / 2] bytes, V codes [16][d / 2] (channel 2i in
 * the low nibble of byte i, channel 2i + 1 in the high nibble), then f16 K
 * scales [16 slots][n_g], K zeros [16][n_g], V scales [16][n_g], V zeros
 * [16][n_g].  Every slot owns its bytes.
 * The oscar_cache fields int2_pool / n_int2_pages describe the INT4 pool for
 * the calls below.
 * ------------------------------------------------------------------------ */
size_t oscar_int4_page_bytes(int32_t d, int32_t n_kv_heads); /* per physical page */

/* Quantize-append into INT4 pages: oscar_quantize_append with 16 levels and
 * the INT4 page layout; same arguments, preconditions, arithmetic and errors. */
oscar_status oscar_quantize_append_int4(const oscar_cache* cache, const void* k_new,
                                        const void* v_new, int64_t n_rows,
                                        const int32_t* row_seq, const int32_t* row_pos,
                                        const int32_t* bt_q, int32_t max_pages,
                                        const float* r_k, const float* r_v,
                                        float tau_k, float tau_v, void* stream);

/* ------------------------------------------------------------------------ *
 * Chunked-prefill ("extend") attention over the mixed cache ([TS] 2.2.B
 * "Kernel Integration" and [TS] 3: paged KV layouts with prefix caching, so
 * a request whose prefix is cached prefills only its new tokens, which attend
 * the cached pages).  For sequence b with P = cache_lens[b] cached tokens
 * and new rows r = cu_rows[b] .. cu_rows[b+1] - 1 (row i = r - cu_rows[b] at
 * position P + i), query head j of row r, h = floor(j / G):
 *   keys/values: the cached tokens [0, P) under the regions of a length-P
 *     cache (sink and recent raw from BF16 pages via bt_h; the middle decoded
 *     from the INT2 (code_bits 2) or INT4 (code_bits 4) pages via bt_q and
 *     attended in the rotated basis, as the decode does), and the new rows
 *     0 .. i of the sequence, raw (causal);
 *   out[r][j] = softmax attention of q[r][j] over them, scale sm_scale, with
 *     the middle's value sum rotated back by R_V(h)^T.
 * The call only reads the cache: writing the new rows into it (BF16 for the
 * recent window, quantize-append for the rest) is a separate step.
 * q: device bf16 [T][H_q][d]; k_new, v_new: device bf16 [T][H_kv][d] (T =
 * cu_rows[batch]); cu_rows: device int32 [batch + 1], non-decreasing from 0;
 * cache_lens: device int32 [batch]; bt_q, bt_h: device int32
 * [batch][max_pages]; r_k, r_v: device float32 [H_kv][d][d]; out: device
 * bf16 [T][H_q][d].  max_cache_len, max_new: host bounds of cache_lens[b]
 * and of the rows per sequence (they size the grid); max_cache_len <=
 * 16 max_pages.  split_steps: steps of 32 tokens per workgroup chunk (0:
 * automatic); with more than one chunk per (sequence, KV head, column tile)
 * the call writes chunk records to `workspace` (at least
 * oscar_extend_workspace_bytes bytes, no preparation needed; 0 bytes when a
 * single chunk suffices) and merges them in a second launch.
 * Preconditions (device contents): 0 <= cache_lens[b] <= max_cache_len, at
 * most max_new rows per sequence, valid page ids wherever they are read.
 * Arithmetic: middle keys and values decoded to f16, the rotated query f16,
 * their probabilities f16; raw keys, values and queries as bf16 (exact
 * products), their probabilities as bf16 hi + lo; float32 sums.
 * Errors: as oscar_paged_decode_attn; UNSUPPORTED for code_bits other than
 * 2 or 4.  batch == 0 or max_new == 0 returns OSCAR_OK and launches nothing.
 * ------------------------------------------------------------------------ */
oscar_status oscar_extend_workspace_bytes(int32_t batch, int32_t n_kv_heads,
                                          int32_t n_q_heads, int32_t d, int32_t n_sink,
                                          int32_t n_recent, int32_t max_cache_len,
                                          int32_t max_new, int32_t split_steps,
                                          size_t* bytes);
oscar_status oscar_paged_extend_attn(const oscar_cache* cache, int32_t code_bits,
                                     const void* q, const void* k_new, const void* v_new,
                                     int32_t batch, int32_t n_q_heads,
                                     const int32_t* cu_rows, const int32_t* cache_lens,
                                     int32_t max_cache_len, int32_t max_new,
                                     const int32_t* bt_q, const int32_t* bt_h,
                                     int32_t max_pages, const float* r_k, const float* r_v,
                                     float sm_scale, int32_t split_steps, void* workspace,
                                     size_t workspace_bytes, void* out, void* stream);

/* Decode attention over a cache whose middle is INT4: the definition of
 * oscar_paged_decode_attn with INT4 pages (seq_lens[b] = L counts the token
 * being decoded; regions of a length-L cache).  The work is cut into chunks
 * of split_steps steps of 32 tokens (0: automatic); the chunk records need
 * oscar_decode_int4_workspace_bytes bytes of workspace (no preparation;
 * 0 bytes when a single chunk suffices) and are merged in a second launch.
 * Arithmetic as oscar_paged_extend_attn.  Errors as oscar_paged_decode_attn. */
oscar_status oscar_decode_int4_workspace_bytes(int32_t batch, int32_t n_kv_heads,
                                               int32_t n_q_heads, int32_t d, int32_t n_sink,
                                               int32_t n_recent, int32_t max_seq_len,
                                               int32_t split_steps, size_t* bytes);
oscar_status oscar_paged_decode_attn_int4(const oscar_cache* cache, const void* q,
                                          int32_t batch, int32_t n_q_heads,
                                          const int32_t* seq_lens, int32_t max_seq_len,
                                          const int32_t* bt_q, const int32_t* bt_h,
                                          int32_t max_pages, const float* r_k,
                                          const float* r_v, float sm_scale,
                                          int32_t split_steps, void* workspace,
                                          size_t workspace_bytes, void* out, void* stream);

/* The same decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that must not call the allocator,
 * harnesses that forbid it): no workspace argument; the arrival counters and
 * per-workgroup records live in one 32 MiB array inside the library, one copy
 * per device, held until the process ends.  The first call on a device looks
 * the array up and clears its counters with a kernel on `stream`.
 * Limits: at most 65536 (sequence, KV head) units and 32512 KiB of records
 * (oscar_decode_workspace_bytes minus its counter part, for the same
 * arguments); beyond that OSCAR_ERR_WORKSPACE, nothing launched.  Every call
 * on a device shares that array: calls that overlap in time on one device
 * (two streams, two threads) race and return wrong values; a call that does
 * not complete can leave counters non-zero for the rest of the process.
 * Outputs are bit-identical to oscar_paged_decode_attn for the same
 * arguments.  No hipMalloc or other allocation is made. */
oscar_status oscar_paged_decode_attn_noalloc(const oscar_cache* cache, const void* q,
                                             int32_t batch, int32_t n_q_heads,
                                             const int32_t* seq_lens, int32_t max_seq_len,
                                             const int32_t* bt_q, const int32_t* bt_h,
                                             int32_t max_pages, const float* r_k,
                                             const float* r_v, float sm_scale,
                                             int32_t split_pages, void* out, void* stream);

/* ------------------------------------------------------------------------ *
 * Measurement context (not part of the method): reads `bytes` bytes of the
 * device buffer `buf` once, streaming, and writes nothing back (`sink`, a
 * device uint32, is written only if the data fold to one particular value),
 * so that timing it gives the attainable HBM read bandwidth the decode
 * kernels, which read far more than they write, can be compared with ([TS] 4
 * attributes the batch-1 decode speedup to reduced memory traffic).
 * buf and bytes: multiples of 16 bytes.  Asynchronous on `stream`.
 * Errors: INVALID_ARG for null pointers or unaligned buf or bytes.
 * ------------------------------------------------------------------------ */
oscar_status oscar_bw_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* OSCAR_H_ */
