// Kernel B — fused paged decode attention over the mixed cache ([TS] 2.2.B
// "kernel integration": unpacking, dequantization, inverse rotation and
// attention for the INT2 history in one kernel, paged and prefix-cache
// compatible; [AB]).  Also the all-BF16 baseline the INT2 cache is compared
// with ([TS] 4).
//
// Work split.  Grid (chunk, KV head, sequence).  The pages of a sequence are
// cut into chunks of one kind: INT2 chunks (split_pages pages of the middle
// history) and BF16 chunks (the sink and recent pages).  A workgroup of 8
// waves takes one chunk of one (sequence, KV head); each wave takes page
// pairs.  The G query heads of the group are the 16 columns of every MFMA
// tile.  INT2 page pairs stream through registers with whole-wave coalesced
// loads four pairs ahead of the compute, and are re-read per lane from a
// private LDS slot in the layout the MFMA operands need.
//
// INT2 tokens are never dequantized.  A 2-bit code c masked in place inside a
// 16-bit half is the f16 subnormal c * 4^p * 2^-24 (p = its 2-bit position),
// exact, and the MFMA multiplies it exactly.  The group affine map is
// factored out of the dot products:
//   q~ . (c s + z) = s (q~ . c) + z sum(q~)                          (keys)
//   sum_t p_t (c_t s_t + z_t) = sum_t (p_t s_t) c_t + sum_t p_t z_t   (values)
// so scales multiply either the 16x16 logit tile or the f16 probabilities,
// and the zero terms are one extra small MFMA each.  The position factors
// 4^p are folded into the query (keys) or applied once at the end (values).
// Logits are kept in log2 units (q~ pre-scaled by sm_scale * log2 e).
//
// Each chunk's result (max, sum, value sum in the rotated or the raw basis)
// goes to the workspace with device-coherent stores; the last workgroup of a
// (sequence, KV head) merges them by log-sum-exp and applies the output
// rotation R_V^T on the MFMA.
#include <algorithm>
#include <type_traits>

#include "device_utils.h"
#include "layout.h"
#include "kernels.h"

using namespace oscar_dev;

namespace {

struct DecParams {
  const uint8_t* int2_pool;
  int32_t n_int2_pages;
  const uint16_t* bf16_pool;
  int32_t n_kv, G, S, W, Hq;
  const uint16_t* q;
  const int32_t* seq_lens;
  const int32_t* bt_q;
  const int32_t* bt_h;
  int32_t max_pages;
  const float* r_k;
  const float* r_v;
  float sm_scale;
  int32_t fixed_ppw;  // per-unit items: pages per item; balanced slices: pages per slice (0: spread evenly)
  float* partials;
  int32_t* counters;
  int32_t rec_floats;
  int32_t cap;        // record slots per (sequence, KV head)
  uint16_t* out;
  int32_t speculate;  // issue the first INT2 requests before reading the sequence lengths
  int32_t max_seq_len;
  int32_t batch;
  int32_t per_unit;    // per-unit items (1) or balanced slices (0)
  int32_t unit_items;  // per-unit items: workgroups per (sequence, KV head)
  int32_t first_int2;  // per-unit items: INT2 pages item 0 takes after the BF16 pages (0: none)
  // fused decode step: the step's new tokens (bf16 [B][n_kv][D]) and the clip
  // thresholds of the token entering the middle history
  const uint16_t* k_new;
  const uint16_t* v_new;
  float tau_k, tau_v;
};

// Waves per workgroup: 8 (one workgroup per CU, two waves per SIMD, four page
// pairs in flight per wave), 12 (three per SIMD, at most 168 VGPRs each, two
// pairs in flight) or 4 (two workgroups per CU, each wave rotating and merging
// two channel blocks).  Twelve passes the same tests but measured 10-15%
// slower on every decode workload; four (balanced slices over twice the
// workgroups) was faster on ragged batches of many units but up to 26% slower
// on uniform long ones, and the better slice costs below made it unnecessary:
// eight is the build.
#ifndef OSCAR_DECODE_WAVES
#define OSCAR_DECODE_WAVES 8
#endif
constexpr int kWaves = OSCAR_DECODE_WAVES;
static_assert(kWaves == 4 || kWaves == 8 || kWaves == 12, "4, 8 or 12 waves per workgroup");
constexpr int kThreads = 64 * kWaves;
constexpr int kMergeBatch = kThreads / 16;  // chunk records loaded per merge round
constexpr int kMaxChunks = 8 * kMergeBatch; // records (segments) per (sequence, KV head)
constexpr int kMinSlice = 2 * kWaves;       // pages per workgroup slice at least (a page pair per wave)
// LDS floats before the page-id blocks: per-wave max [kWaves][16], per-wave
// sum [kWaves][16], flags [16], per-block query sums [8][16]
constexpr int kMisc = 32 * kWaves + 16 + 128;
// Balanced slices count each nonempty page range (a unit's BF16 pages, its
// INT2 pages) as seg_pages(G) extra pages: the fixed cost of a segment
// (requests, query rotation, record, arrival, the unit's merge), in INT2 pages
// a CU streams meanwhile.  It grows with the query group (the rotation, the
// per-wave results, the record and the merge scale with G); fitted to
// per-workgroup timestamps of ragged batches: about 160 pages at G = 4 and
// 224 at G = 12.  Slices crossing many short units get fewer pages.
__host__ __device__ constexpr int seg_pages(int G) { return 128 + 8 * G; }
constexpr int kSegPagesMax = seg_pages(16);
// In a fused decode step the segment holding a unit's last middle page also
// quantizes the token entering the middle history (its rotation slices, raw
// row and INT2 slot: about two round trips to memory): that unit's row
// counts this many more positions.
constexpr int kOwnPages = 80;
static_assert(kMaxChunks * 16 % kThreads == 0, "merge: (record, query row) slots split evenly over threads");
constexpr float kTwo24 = 16777216.0f;
constexpr float kSlack = 4.0f;    // log2 units
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ bool overlaps(int a0, int a1, int b0, int b1) { return max(a0, b0) < min(a1, b1); }

// device-coherent (write-through / L2-bypassing) 32-bit accesses for the
// chunk records exchanged between workgroups on different XCDs
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (a, b) = hi + lo, each a bf16 pair (element 0 in the low half), to 16
// significant bits: the packed hardware conversion rounds to nearest even, as
// the scalar split does, in one instruction per pair and part.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ void split2x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = bf16x2_rne(a, b);
  lo = bf16x2_rne(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// Keep-mask of an f16/bf16 pair for tokens (t, t+1): stale bytes in slots
// outside the region must not reach the value sums (0 * NaN is NaN).
__device__ __forceinline__ uint32_t pair_keep(bool k0, bool k1) {
  return (k0 ? 0x0000FFFFu : 0u) | (k1 ? 0xFFFF0000u : 0u);
}

// Page plan of one sequence: BF16 page ranges A and B (sink, recent; one
// range when they meet) and the INT2 page range.  Its work, in pages, is the
// BF16 pages (A then B) followed by the INT2 pages.
struct SeqPlan {
  int L, n_pages, s1, m0, m1, r0;
  int ra0, ra1, rb0, rb1, q0, q1;
  int n_raw, real, cost;  // BF16 pages; BF16 + INT2 pages; with the per-range overhead
};

template <bool ALL_RAW>
__device__ __forceinline__ SeqPlan make_plan(const DecParams& p, int L) {
  SeqPlan sp;
  sp.L = L;
  sp.n_pages = (L + 15) >> 4;
  sp.s1 = ALL_RAW ? L : min(p.S, L);
  sp.m0 = p.S;
  sp.m1 = ALL_RAW ? 0 : L - p.W;
  sp.r0 = ALL_RAW ? L : max(p.S, L - p.W);
  if (ALL_RAW) {
    sp.ra0 = 0; sp.ra1 = sp.n_pages; sp.rb0 = sp.rb1 = 0; sp.q0 = sp.q1 = 0;
  } else {
    const int hs1 = (sp.s1 + 15) >> 4;                       // pages holding sink tokens
    const int hr0 = sp.r0 < L ? (sp.r0 >> 4) : sp.n_pages;   // first page holding a recent token
    if (hs1 >= hr0) {
      sp.ra0 = 0; sp.ra1 = sp.n_pages; sp.rb0 = sp.rb1 = 0;
    } else {
      sp.ra0 = 0; sp.ra1 = hs1; sp.rb0 = hr0; sp.rb1 = sp.n_pages;
    }
    if (sp.m1 > sp.m0) { sp.q0 = sp.m0 >> 4; sp.q1 = (sp.m1 + 15) >> 4; }
    else { sp.q0 = sp.q1 = 0; }
  }
  sp.n_raw = (sp.ra1 - sp.ra0) + (sp.rb1 - sp.rb0);
  sp.real = sp.n_raw + (sp.q1 - sp.q0);
  sp.cost = sp.real + seg_pages(p.G) * ((sp.n_raw > 0 ? 1 : 0) + (sp.q1 > sp.q0 ? 1 : 0)) +
            (p.k_new != nullptr && sp.m1 > sp.m0 ? kOwnPages : 0);
  return sp;
}

// Pages per workgroup slice: the total spread evenly over the grid, but
// large enough that no unit is cut into more than cap - 3 slices (its
// records then fit in cap slots) and that every wave gets a page pair.
// Positions stay below 2^31 (the host bounds the work of one call).
__device__ __forceinline__ int slice_pages(const DecParams& p, int total, int max_cost) {
  if (p.fixed_ppw) return p.fixed_ppw;
  const int even = int((static_cast<long long>(total) + gridDim.x - 1) / gridDim.x);
  const int fit = (max_cost + p.cap - 4) / (p.cap - 3);
  return max(max(even, fit), kMinSlice);
}

// Operands one lane needs from one INT2 page-head image (global or LDS).
template <int D>
struct PageOps {
  static constexpr int NG = D / 32, NW = D / 64;
  uint32_t kc[NW];      // KC words: token l16, K-slots of this quad
  uint32_t ks[2 * NG];  // K scales of tokens 4quad..4quad+3, all groups ([slot][g] f16)
  uint32_t kz[2];       // K zeros of token l16 (quads 0, 1 only)
  uint32_t vc[NW];      // VC words: channel l16 of each block, tokens of this quad
  uint32_t vs[2 * NG];  // V scales [quad][g][4 tokens]
  uint32_t vz[2];       // V zeros of group l16, tokens 4quad..4quad+3 (meaningful for l16 < NG)

  __device__ __forceinline__ void read_k(const uint8_t* base, int l16, int quad) {
    using GG = Geo<D>;
    const uint32_t* kcp = reinterpret_cast<const uint32_t*>(base + GG::KC) + (quad * 16 + l16) * NW;
    const uint32_t* ksp = reinterpret_cast<const uint32_t*>(base + GG::KS) + quad * 2 * NG;
#pragma unroll
    for (int i = 0; i < NW; ++i) kc[i] = kcp[i];
#pragma unroll
    for (int i = 0; i < 2 * NG; ++i) ks[i] = ksp[i];
    // every lane reads (the zero-term operand's rows for quads 2 and 3 are
    // zero, so what those lanes hold does not reach a sum that is kept)
    const uint32_t* kzp = reinterpret_cast<const uint32_t*>(base + GG::KZ) + l16 * (NG / 2);
    kz[0] = kzp[0];
    kz[1] = NG == 4 ? kzp[1] : 0u;
  }
  // CS > 1 (CS column slots per query): only the V scales of the NGV groups
  // this lane's column stands for, group min(CS h + l16 % CS, NG - 1) in
  // vs[2h], vs[2h + 1]; CS = 1: every group's
  template <int CS = 1>
  __device__ __forceinline__ void read_v(const uint8_t* base, int l16, int quad) {
    using GG = Geo<D>;
    constexpr int NGV = NG / CS > 0 ? NG / CS : 1;
    const uint32_t* vcp = reinterpret_cast<const uint32_t*>(base + GG::VC) + (quad * 16 + l16) * NW;
    const uint32_t* vsp = reinterpret_cast<const uint32_t*>(base + GG::VS) + quad * 2 * NG;
#pragma unroll
    for (int i = 0; i < NW; ++i) vc[i] = vcp[i];
    if (CS == 1) {
#pragma unroll
      for (int i = 0; i < 2 * NG; ++i) vs[i] = vsp[i];
    } else {
#pragma unroll
      for (int hh = 0; hh < NGV; ++hh) {
        const int g = min(CS * hh + l16 % CS, NG - 1);
        vs[2 * hh] = vsp[2 * g];
        vs[2 * hh + 1] = vsp[2 * g + 1];
      }
    }
    // every lane reads a valid slot (group min(l16, NG - 1)); rows l16 >= NG
    // of the zero-term operand are cleared by the caller's lane mask
    const uint32_t* vzp = reinterpret_cast<const uint32_t*>(base + GG::VZ) + (quad * NG + min(l16, NG - 1)) * 2;
    vz[0] = vzp[0];
    vz[1] = vzp[1];
  }
};

// A page pair goes from HBM straight into an LDS ring slot of its wave with
// global_load_lds_dwordx4: LOADS whole-wave loads of 1024 B, lane l of load i
// carrying pair bytes [1024 i + 16 l, +16) (page A, then page B; for d = 64
// the last 512 B of the slot are padding, filled from page B's last bytes).
// No registers hold pages in flight.
template <int D>
struct PairDma {
  static constexpr int HB = Geo<D>::HEAD_BYTES;  // 1536 or 768
  static constexpr int LOADS = (2 * HB + 1023) / 1024;
  static constexpr int SLOT = LOADS * 1024;
};
// page pairs requested ahead of the step being computed, and ring slots per
// wave (the two pairs being computed and those in flight)
constexpr int kDepth = kWaves <= 8 ? 4 : 2;
constexpr int kRing = kDepth + 2;


// SLICES: balanced slices over all units (several segments per workgroup),
// else per-unit items (one segment per workgroup, early requests).  Separate
// kernels keep each one's code to a single instance of the segment.
// CS (column slots per query: 4 for G <= 4, 2 for G <= 8, else 1): MFMA
// column n carries query n/CS, and in the value products its h-th B operand
// (probability times a V scale) stands for channel group CS h + n%CS, so
// that NG/CS operands (at least one) serve every channel block instead of NG.
// UPD (fused decode step): the launch also does the step's cache update.  The
// segment whose BF16 pages include the new token's page writes the new token
// to its slot before reading it; the INT2 segment holding the last middle
// page quantizes the token entering the middle history (exactly as the
// few-row quantize-append does), writes it to its INT2 slot for later steps,
// leaves that slot out of its own page loop and adds the token to its record
// from the decoded values.  Launched with per-unit items only: balanced
// slices leave no workgroup the slack to absorb the update's round trips.
template <int D, bool ALL_RAW, bool SLICES, int CS, bool UPD>
__global__ __launch_bounds__(kThreads, kWaves == 4 ? 2 : 1) void decode_kernel(DecParams p) {
  using GG = Geo<D>;
  constexpr int NG = GG::NG, NCB = GG::NCB, NKB = GG::NKB, HB = GG::HEAD_BYTES;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int G = p.G;
  // LDS: q-hat B operands [NG][64][4] u32 | misc kMisc floats | page-id
  // blocks | page rings [kWaves][kRing][SLOT], which the per-wave results and
  // the merge reuse once the page loop is over
  uint32_t* s_qhat = reinterpret_cast<uint32_t*>(smem);
  float* s_misc = reinterpret_cast<float*>(s_qhat + NG * 256);
  float* s_m = s_misc;                // [kWaves][16] per-wave max
  float* s_l = s_misc + 16 * kWaves;  // [kWaves][16] per-wave sum
  int* s_flag = reinterpret_cast<int*>(s_misc + 32 * kWaves);  // [16]
  uint32_t* s_tabs = reinterpret_cast<uint32_t*>(s_misc + kMisc);  // [kWaves][2][64] page-id blocks
  uint8_t* s_slots = reinterpret_cast<uint8_t*>(s_tabs + kWaves * 2 * 64);
  float* s_res = reinterpret_cast<float*>(s_slots);
  // s_res: per-wave results [kWaves][G][D]; in the last workgroup: merged [G][D] rot
  // and [G][D] raw

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  // wave index in a scalar register: page-table lookups become scalar loads,
  // which the vector-memory counter does not wait on
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x;
  const int qrow = min(l16, G - 1);  // per-query rows of the merge
  // query of MFMA column l16 (columns past the group repeat a real head;
  // their results are dropped)
  const int qcol = min(l16 / CS, G - 1);
  const float qscale = p.sm_scale * kLog2e;

  // the (sequence, KV head) unit of the current segment
  int b = 0, h = 0;
  const uint16_t* qb = p.q;
  const int32_t* btq = p.bt_q;
  const int32_t* bth = p.bt_h;
  auto set_unit = [&](int bb, int hh) {
    b = bb;
    h = hh;
    qb = p.q + (size_t(b) * p.Hq + h * G) * D;
    btq = p.bt_q + size_t(b) * p.max_pages;
    bth = p.bt_h + size_t(b) * p.max_pages;
  };

  // ---- requests of an INT2 segment starting at page sc0: the query-rotation
  // operands, the query, this wave's page ids and its first kDepth page pairs
  // (into ring slots 0..kDepth-1).  Entries past the segment may be anything:
  // table reads stay inside the row and page ids are clamped into the pool;
  // such pages are never used unmasked. ----
  using PD = PairDma<D>;
  uint8_t* const ring = s_slots + wave * kRing * PD::SLOT;
  // 16-channel blocks of the query rotation and of the merge's R_V^T: block
  // cb = wave + kWaves j (j < NB) when there are fewer waves than blocks;
  // with more waves, waves past NCB repeat a block and keep no result
  constexpr int NB = NCB > kWaves ? NCB / kWaves : 1;
  static_assert(NB * kWaves >= NCB && (NCB <= kWaves || NCB % kWaves == 0), "blocks over waves");
  const bool rot_wave = wave < NCB;
  float rvals[NB][NKB][8];
  u32x4 bqv[NKB];
  int sc0 = 0;  // first page of the segment the requests are for
  // Page ids of this wave's pairs, 32 pairs per register block: lane L holds
  // page sc0 + 2(wave + 8k) + L%2 of pair k = 32 blk + L/2.  Reading them with
  // readlane keeps memory waits out of the prefetch issue.  Block 0 is a
  // plain load; later blocks come through the wave's LDS table area (block
  // blk in area blk % 2), requested a whole block of pairs before they are
  // read: page loads that land in LDS are invisible to the compiler's wait
  // counting, so a plain load consumed mid-loop would drain them all.
  uint32_t* const my_tabs = s_tabs + wave * 2 * 64;
  auto tab_entry = [&](int blk) {
    const int k = 32 * blk + (lane >> 1);
    return btq + min(sc0 + 2 * (wave + kWaves * k) + (lane & 1), p.max_pages - 1);
  };
  auto clamp_page = [&](int v) { return min(max(v, 0), p.n_int2_pages - 1); };
  auto tab_dma = [&](int blk) {
    __builtin_amdgcn_global_load_lds(tab_entry(blk), my_tabs + 64 * (blk & 1), 4, 0, 0);
  };
  int tab = 0, tab_blk = 0;
  auto pair_pages = [&](int k, const uint8_t*& pa, const uint8_t*& pb) {
    const int i = 2 * (max(k, 0) & 31);
    pa = p.int2_pool + (size_t(__builtin_amdgcn_readlane(tab, i)) * p.n_kv + h) * HB;
    pb = p.int2_pool + (size_t(__builtin_amdgcn_readlane(tab, i + 1)) * p.n_kv + h) * HB;
  };
  // pair j (clamped to this wave's pairs) -> ring slot dst
  auto pair_dma = [&](int j, uint8_t* dst) {
    const uint8_t *pa, *pb;
    pair_pages(j, pa, pb);
#pragma unroll
    for (int i = 0; i < PD::LOADS; ++i) {
      const int o = 1024 * i + 16 * lane;
      const uint8_t* src = o < HB ? pa + o : pb + min(o - HB, HB - 16);
      __builtin_amdgcn_global_load_lds(src, dst + 1024 * i, 16, 0, 0);
    }
  };
  auto int2_requests = [&]() {
    tab_blk = 0;
    tab = clamp_page(*tab_entry(0));
    {  // every wave loads (waves past NCB repeat a block) so that no path leaves them unset
      const float* rk = p.r_k + size_t(h) * D * D;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            rvals[j][kb][i] = rk[size_t(32 * kb + 8 * quad + i) * D + 16 * ((wave + kWaves * j) & (NCB - 1)) + l16];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) bqv[kb] = *reinterpret_cast<const u32x4*>(qb + size_t(qcol) * D + 32 * kb + 8 * quad);
    }
    // The page requests go out as soon as the page ids are in, behind the
    // rotation operands (older requests: the compiler may not move loads
    // across this point), so that the rotation later waits with
    // vmcnt(kDepth LOADS + 1) for exactly those operands while the pages and
    // the page-id block stay in flight.
    asm volatile("" ::: "memory");
    // page loads are issued unconditionally (a wave short of pairs loads
    // unused pages) so that every wait counts exactly the loads issued after
    // the pair it waits for
#pragma unroll
    for (int u = 0; u < kDepth; ++u) pair_dma(u, ring + u * PD::SLOT);
    tab_dma(1);
  };

  // ---- work layout ----
  bool spec_issued = false;  // INT2 requests issued before the lengths were known
  int spec_b = 0, spec_h = 0;
  auto speculate_at = [&](int bb, int hh, int page) {
    set_unit(bb, hh);
    sc0 = page;
    int2_requests();
    spec_issued = true;
    spec_b = bb;
    spec_h = hh;
  };
  SeqPlan sp;
  // ---------------- one segment of unit (b, h) ----------------
  // INT2 (!is_raw): pages [c0, c1).  BF16: positions [c0, c1) in the list of
  // the sequence's BF16 pages (range A, then range B).  The segment leaves
  // record kseg of the unit's nseg.  The first segment of a workgroup is a
  // separate instance: only it can use the early requests, so no request
  // registers stay live from one segment to the next.
  auto segment = [&](auto first_tag, const bool is_raw, const int c0, const int c1, const int nseg,
                     const int kseg) __attribute__((always_inline)) {
  constexpr bool FIRST = decltype(first_tag)::value;
  // lane indices re-derived per segment through an opaque copy: addresses
  // built from them are then computed where they are used instead of being
  // hoisted out of the segment loop and kept live through the page loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  const int qcol = min(l16 / CS, G - 1);
  const int n_pairs = (c1 - c0 + 1) >> 1;
  // fused step: this INT2 segment holds the last middle token (the one that
  // enters the middle history this step) and handles it apart from its loop
  const bool owner = UPD && !is_raw && sp.m1 > sp.m0 && ((sp.m1 - 1) >> 4) >= c0 && ((sp.m1 - 1) >> 4) < c1;
  const int m0 = sp.m0, m1 = owner ? sp.m1 - 1 : sp.m1, s1 = sp.s1, r0 = sp.r0;
  float qf4[NB][4] = {};  // fused step: this lane's q~ blocks (log2 units)
  // Owner scratch past the per-wave results (kWaves x 16 queries x D floats)
  // in the ring area, free once the page loop is over: slice partials
  // [2][16][D], raw rows [2][D], decoded rotated k~, v~ [2][D], q~ [16][D],
  // then [16] logits of the token, [16] and [16] rescale factors, codes and
  // f16 scale/zero words
  float* const own_s = reinterpret_cast<float*>(s_slots) + kWaves * 16 * D;
  float* const own_part = own_s;
  float* const own_x = own_part + 2 * 16 * D;
  float* const own_kv = own_x + 2 * D;
  float* const own_q = own_kv + 2 * D;
  float* const own_l = own_q + 16 * D;
  uint8_t* const own_code = reinterpret_cast<uint8_t*>(own_l + 48);
  uint16_t* const own_sz = reinterpret_cast<uint16_t*>(own_code + 2 * D);  // [tensor][g][scale, zero]
  auto own_token = [&](const float (&qv)[NB][4]) __attribute__((always_inline)) {
    const int t = sp.m1 - 1;           // the token entering the middle history
    const int slot = t & 15;
    const size_t row = (size_t(b) * p.n_kv + h) * D;
    // y = x R as the few-row kernel sums it: 16 slices of D/16 inputs, each a
    // float32 multiply-add chain from zero, then the slices in order.  Thread
    // task (tensor T, slice ks, channel quad c4); its R values are requested
    // first, together with the raw row, so that the token costs one round
    // trip to memory
    constexpr int KS = D / 16, C4 = D / 4, NTASK = 2 * 16 * C4, NT = (NTASK + kThreads - 1) / kThreads;
    f32x4 rr[NT][KS];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int task = min(tid + n * kThreads, NTASK - 1), T = task / (16 * C4), ks = (task / C4) % 16, c4 = task % C4;
      const float* R = (T ? p.r_v : p.r_k) + size_t(h) * D * D;
#pragma unroll
      for (int j = 0; j < KS; ++j) rr[n][j] = *reinterpret_cast<const f32x4*>(R + size_t(ks * KS + j) * D + 4 * c4);
    }
    // its raw K and V rows: from its BF16 slot (W >= 1), or the new token (W = 0)
    uint16_t xb = 0;
    if (tid < 2 * D) {
      const int T = tid / D, c = tid % D;
      if (p.W >= 1) {
        const uint16_t* hp = p.bf16_pool + (size_t(bth[t >> 4]) * p.n_kv + h) * GG::BF16_HEAD_ELEMS;
        xb = T == 0 ? hp[slot * D + c] : hp[16 * D + c * 16 + slot];
      } else {
        xb = (T == 0 ? p.k_new : p.v_new)[row + c];
      }
    }
    // the scratch lies in the page rings: every wave is done reading its ring
    lds_barrier();
    if (tid < 2 * D) own_x[tid] = bf16_to_f32(xb);
    // q~ of the group's queries (the columns that hold each query once)
    if (rot_wave && l16 % CS == 0 && l16 / CS < G) {
      const int qi = l16 / CS;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) own_q[qi * D + 16 * (wave + kWaves * j) + 4 * quad + r] = qv[j][r];
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int task = tid + n * kThreads, T = task / (16 * C4), ks = (task / C4) % 16, c4 = task % C4;
      if (task >= NTASK) break;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const float x = own_x[T * D + ks * KS + j];
#pragma unroll
        for (int c = 0; c < 4; ++c) a[c] = __builtin_fmaf(x, rr[n][j][c], a[c]);
      }
      *reinterpret_cast<f32x4*>(own_part + (T * 16 + ks) * D + 4 * c4) = a;
    }
    __syncthreads();
    if (tid < 2 * D) {  // whole waves: a 32-channel group is half a wave
      const int T = tid / D, c = tid % D;
      float y = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) y += own_part[(T * 16 + k) * D + c];
      const float tau = T ? p.tau_v : p.tau_k;
      y = __builtin_amdgcn_fmed3f(y, -tau, tau);
      float mn = y, mx = y;
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m, 64));
        mx = fmaxf(mx, __shfl_xor(mx, m, 64));
      }
      const uint32_t s16 = f16_bits(div3(mx - mn));
      const uint32_t z16 = f16_bits(mn);
      const float sf = f16_to_f32(s16), zf = f16_to_f32(z16);
      int code = 0;
      if (sf != 0.0f) code = min(max(int(__builtin_rintf((y - zf) / sf)), 0), 3);
      own_code[T * D + c] = uint8_t(code);
      if ((c & 31) == 0) {
        own_sz[(T * NG + (c >> 5)) * 2] = uint16_t(s16);
        own_sz[(T * NG + (c >> 5)) * 2 + 1] = uint16_t(z16);
      }
      own_kv[T * D + c] = __builtin_fmaf(float(code), sf, zf);
    }
    __syncthreads();
    // the token's codes, scales and zeros into its INT2 slot (the layout the
    // few-row quantize-append writes: whole K words, whole V bytes)
    uint8_t* base = const_cast<uint8_t*>(p.int2_pool) + (size_t(btq[t >> 4]) * p.n_kv + h) * HB;
    if (tid < 4 * GG::NW) {
      const int quad2 = tid / GG::NW, w = tid % GG::NW;
      uint32_t wd = 0;
#pragma unroll
      for (int gp = 0; gp < 2; ++gp)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            wd |= uint32_t(own_code[64 * w + 32 * gp + 16 * hb + 4 * quad2 + r]) << (16 * (r & 1) + 8 * gp + 4 * hb + 2 * (r >> 1));
      reinterpret_cast<uint32_t*>(base + GG::KC)[(quad2 * 16 + slot) * GG::NW + w] = wd;
    } else if (tid >= 64 && tid < 64 + 16 * GG::NW) {
      const int i = tid - 64, c16 = i & 15, w = i >> 4;
      const int q4 = slot >> 2, r = slot & 3;
      uint32_t bits = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) bits |= uint32_t(own_code[D + 64 * w + 16 * bb + c16]) << (2 * bb);
      base[GG::VC + ((q4 * 16 + c16) * GG::NW + w) * 4 + 2 * (r & 1) + (r >> 1)] = uint8_t(bits);
    } else if (tid >= 128 && tid < 128 + 2 * NG) {
      const int T = (tid - 128) / NG, g = (tid - 128) % NG;
      const int iu = T == 0 ? slot * NG + g : ((slot >> 2) * NG + g) * 4 + (slot & 3);
      reinterpret_cast<uint16_t*>(base + (T == 0 ? GG::KS : GG::VS))[iu] = own_sz[(T * NG + g) * 2];
      reinterpret_cast<uint16_t*>(base + (T == 0 ? GG::KZ : GG::VZ))[iu] = own_sz[(T * NG + g) * 2 + 1];
    }
    // the token's logit for each query of the group (log2 units, as the loop's)
    for (int qi = wave; qi < G; qi += kWaves) {
      float a = 0.f;
      for (int c = lane; c < D; c += 64) a = __builtin_fmaf(own_q[qi * D + c], own_kv[c], a);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
      if (lane == 0) own_l[qi] = a;
    }
  };

  float m_run = kNegInf, l_part = 0.f;
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc_z = {0.f, 0.f, 0.f, 0.f};

  // online-softmax step shared by both chunk kinds: logits lg (log2 units,
  // -inf = masked) -> probabilities pv, accumulators rescaled as needed
  auto softmax_step = [&](auto& lg, auto& pv) {
    constexpr int NP = sizeof(lg) / sizeof(lg[0]);  // pages of logits
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < NP; ++j)
      mx = fmaxf(mx, fmaxf(fmaxf(lg[j][0], lg[j][1]), fmaxf(lg[j][2], lg[j][3])));
    mx = wave_max16(mx);
    // lazy rescaling: the reference max moves only when a logit exceeds it
    // by more than kSlack (probabilities stay <= 2^kSlack, safe in f16)
    const float m_new = fmaxf(m_run, mx);
    if (__any(mx > m_run + kSlack)) {
      const float f = (m_run == kNegInf) ? 0.f : exp2f(m_run - m_new);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] *= f;
      acc_z *= f;
      l_part *= f;
      m_run = m_new;
    }
    // every page pair holds at least one unmasked token, so m_run is finite
    // here unless the logits themselves are not; masked logits (-inf) give 0
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[j][r] = __builtin_amdgcn_exp2f(lg[j][r] - m_use);
  };

  // INT2 steps: the logits arrive already offset by -m_off (m_off = m_run,
  // or 0 before the first step), folded into the zero-term MFMA's
  // accumulator, so the exponent needs no subtraction unless the reference
  // max moves
  auto softmax_step_off = [&](auto& lg, auto& pv, float m_off) {
    constexpr int NP = sizeof(lg) / sizeof(lg[0]);
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < NP; ++j)
      mx = fmaxf(mx, fmaxf(fmaxf(lg[j][0], lg[j][1]), fmaxf(lg[j][2], lg[j][3])));
    mx = wave_max16(mx);
    if (__any(mx > kSlack || m_run == kNegInf)) {  // rare: everything rescaled in place
      const float m_new = fmaxf(m_run, mx + m_off);
      const float f = (m_run == kNegInf) ? 0.f : exp2f(m_run - m_new);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] *= f;
      acc_z *= f;
      l_part *= f;
      m_run = m_new;
      const float dl = (m_new == kNegInf) ? 0.f : m_new - m_off;
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[j][r] -= dl;
    }
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[j][r] = __builtin_amdgcn_exp2f(lg[j][r]);
  };

  if (is_raw) {
    // ---------------- BF16 chunk: raw q . k, raw-basis value sums ----------------
    if (UPD && (p.W >= 1 || sp.L - 1 < p.S)) {
      // fused step: the new token (position L - 1) to its BF16 slot, if this
      // segment reads that page, before the page is read
      const int pg = (sp.L - 1) >> 4, n_a = sp.ra1 - sp.ra0;
      const int li = pg < sp.ra1 ? pg - sp.ra0 : n_a + (pg - sp.rb0);
      if (li >= c0 && li < c1) {
        uint16_t* hp = const_cast<uint16_t*>(p.bf16_pool) + (size_t(bth[pg]) * p.n_kv + h) * GG::BF16_HEAD_ELEMS;
        const size_t src = (size_t(b) * p.n_kv + h) * D;
        const int slot = (sp.L - 1) & 15;
        if (tid < D) hp[slot * D + tid] = p.k_new[src + tid];
        else if (tid < 2 * D) hp[16 * D + (tid - D) * 16 + slot] = p.v_new[src + tid - D];
        __syncthreads();  // stores done and visible to this workgroup's page loads
      }
    }
    u32x4 bqr[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) bqr[kb] = *reinterpret_cast<const u32x4*>(qb + size_t(qcol) * D + 32 * kb + 8 * quad);
    const int n_a = sp.ra1 - sp.ra0;
    for (int pr = wave; pr < n_pairs; pr += kWaves) {
      float lg[2][4];
      uint32_t vraw[2][NCB][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int vi = c0 + 2 * pr + j;
        const int pg = vi < n_a ? sp.ra0 + vi : sp.rb0 + (vi - n_a);
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[j][r] = kNegInf;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) vraw[j][cb][0] = vraw[j][cb][1] = 0;
        if (vi >= c1) continue;
        const uint16_t* hbase = p.bf16_pool + (size_t(bth[pg]) * p.n_kv + h) * GG::BF16_HEAD_ELEMS;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          d = mfma_bf16(*reinterpret_cast<const u32x4*>(hbase + l16 * D + 32 * kb + 8 * quad), bqr[kb], d);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {  // V^T rows: channel 16cb + l16, tokens 4quad .. 4quad+3
          const u32x2 v = *reinterpret_cast<const u32x2*>(hbase + 16 * D + (16 * cb + l16) * 16 + 4 * quad);
          vraw[j][cb][0] = v[0];
          vraw[j][cb][1] = v[1];
        }
        bool keep[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * pg + 4 * quad + r;
          keep[r] = t < s1 || (t >= r0 && t < sp.L);
          if (keep[r]) lg[j][r] = d[r] * qscale;
        }
        const uint32_t k01 = pair_keep(keep[0], keep[1]), k23 = pair_keep(keep[2], keep[3]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) { vraw[j][cb][0] &= k01; vraw[j][cb][1] &= k23; }
      }
      float pv[2][4];
      softmax_step(lg, pv);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) l_part += pv[j][r];
      if (ALL_RAW) {
        // baseline: bf16 probabilities against bf16 values
        const u32x4 bpr = {bf16x2_rne(pv[0][0], pv[0][1]), bf16x2_rne(pv[0][2], pv[0][3]),
                           bf16x2_rne(pv[1][0], pv[1][1]), bf16x2_rne(pv[1][2], pv[1][3])};
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[cb] = mfma_bf16(u32x4{vraw[0][cb][0], vraw[0][cb][1], vraw[1][cb][0], vraw[1][cb][1]}, bpr, acc[cb]);
      } else {
        // sink/recent tokens of the mixed cache: the raw bf16 values (any
        // bf16 magnitude) against the probabilities split into bf16 hi + lo
        // (16 significant bits), two products per block
        uint32_t ph[4], pl[4];
        split2x2(pv[0][0], pv[0][1], ph[0], pl[0]);
        split2x2(pv[0][2], pv[0][3], ph[1], pl[1]);
        split2x2(pv[1][0], pv[1][1], ph[2], pl[2]);
        split2x2(pv[1][2], pv[1][3], ph[3], pl[3]);
        const u32x4 bph = {ph[0], ph[1], ph[2], ph[3]}, bpl = {pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const u32x4 a = {vraw[0][cb][0], vraw[0][cb][1], vraw[1][cb][0], vraw[1][cb][1]};
          acc[cb] = mfma_bf16(a, bpl, acc[cb]);
          acc[cb] = mfma_bf16(a, bph, acc[cb]);
        }
      }
    }
  } else if (!ALL_RAW) {
    // ---------------- INT2 segment ----------------
    if (!(FIRST && spec_issued && spec_b == b && spec_h == h && sc0 == c0)) {
      sc0 = c0;
      int2_requests();
    }
    const int n_mine = n_pairs > wave ? (n_pairs - wave + kWaves - 1) / kWaves : 0;
    // the rotation of the query runs while the first page pairs are in flight:
    // the wave of 16-channel block cb (group cb/2, half cb%2) rotates it with a
    // bf16 hi/lo split of R_K (16 significant bits; q~ is rounded to f16 afterwards)
    float* s_qsp = s_misc + 32 * kWaves + 16;  // [NCB][16] per-block query sums
    wait_vm<kDepth * PD::LOADS + 1>();  // the rotation operands (older than the page-id block and pages)
    if (rot_wave) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int cb = wave + kWaves * j, g = cb >> 1, hb = cb & 1;
        f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          uint32_t ph[4], pl[4];
#pragma unroll
          for (int i = 0; i < 8; i += 2) split2x2(rvals[j][kb][i], rvals[j][kb][i + 1], ph[i / 2], pl[i / 2]);
          a4 = mfma_bf16(u32x4{pl[0], pl[1], pl[2], pl[3]}, bqv[kb], a4);
          a4 = mfma_bf16(u32x4{ph[0], ph[1], ph[2], ph[3]}, bqv[kb], a4);
        }
        // a4[r] = q~[n = l16][c = 32g + 16hb + 4quad + r]; K-slot (e = 2hb + r/2, half r%2)
        const float v0 = a4[0] * qscale, v1 = a4[1] * qscale, v2 = a4[2] * qscale, v3 = a4[3] * qscale;
        if (UPD) {
          qf4[j][0] = v0; qf4[j][1] = v1; qf4[j][2] = v2; qf4[j][3] = v3;
        }
        const float f0 = hb ? 1.f / 16.f : 1.f, f1 = hb ? 1.f / 64.f : 1.f / 4.f;
        s_qhat[(g * 64 + lane) * 4 + 2 * hb] = pack_f16x2(v0 * f0, v1 * f0);
        s_qhat[(g * 64 + lane) * 4 + 2 * hb + 1] = pack_f16x2(v2 * f1, v3 * f1);
        const float qs = wave_sum16((v0 + v1) + (v2 + v3));
        if (quad == 0) s_qsp[cb * 16 + l16] = qs;
      }
    }
    lds_barrier();
    // zero-term B operand: K-slots of quad 0 carry the per-group query sums
    // (f16 hi), quad 1 their f16 remainders, the rest zero
    u32x4 bz = {0, 0, 0, 0};
    if (quad < 2) {
      uint32_t hv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float qsum = s_qsp[(2 * g) * 16 + l16] + s_qsp[(2 * g + 1) * 16 + l16];
        const uint32_t hi = f16_bits(qsum);
        hv[g] = quad == 0 ? hi : f16_bits(qsum - f16_to_f32(hi));
      }
      bz = u32x4{pack2(hv[0], hv[1]), pack2(hv[2], hv[3]), pack2(hv[4], hv[5]), pack2(hv[6], hv[7])};
    }
    const uint32_t ones = l16 == NG ? 0x3C003C00u : 0u;  // f16 1.0 pairs in A row NG
    const uint32_t zrow = l16 < NG ? 0xFFFFFFFFu : 0u;    // A rows that carry V zeros
    constexpr int NGV = NG / CS > 0 ? NG / CS : 1;         // V-scale B operands per pair
    // one page pair: logits, softmax, value sums
    // Two page pairs per step (pair k from slot A, pair k+1 from slot B): K
    // operands and logits of the four pages, one softmax step over their 64
    // tokens, then V operands and value sums pair by pair.  INTERIOR: all four
    // pages present and wholly inside the middle region (no per-token masking).
    auto page_of = [&](int k, int j) { return c0 + 2 * (wave + kWaves * k) + j; };
    auto page_live = [&](int pg) { return pg < c1; };
    auto do_two = [&](int k, const uint8_t* sa, const uint8_t* sb, bool has_b, auto interior_tag) {
      constexpr bool INTERIOR = decltype(interior_tag)::value;
      const float m_off = (m_run == kNegInf) ? 0.f : m_run;
      const f32x4 zinit = {-m_off, -m_off, -m_off, -m_off};
      float lg[4][4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int pg = page_of(k + (jj >> 1), jj & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[jj][r] = kNegInf;
        if (jj >= 2 && !has_b) continue;
        if (!INTERIOR && !page_live(pg)) continue;
        PageOps<D> P;
        P.read_k((jj < 2 ? sa : sb) + (jj & 1) * HB, l16, quad);
        const f32x4 dz = mfma_f16(u32x4{P.kz[0], P.kz[1], 0u, 0u}, bz, zinit);
        float lk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const uint32_t src = (g & 1) ? shr8_halves(P.kc[g >> 1]) : P.kc[g >> 1];
          const u32x4 a = {src & 0x00030003u, src & 0x000C000Cu, src & 0x00300030u, src & 0x00C000C0u};
          // q~ operand of group g, read from LDS at each use (measured: a little
          // faster than holding the NG operands in registers)
          const u32x4 bqg = *reinterpret_cast<const u32x4*>(s_qhat + (g * 64 + lane) * 4);
          const f32x4 dg = mfma_f16(a, bqg, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int idx = r * NG + g;  // scale of token 4quad + r, group g
            lk[r] = fmaf(dg[r], f16_to_f32(P.ks[idx >> 1] >> (16 * (idx & 1))), lk[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * pg + 4 * quad + r;
          if (INTERIOR || (t >= m0 && t < m1)) lg[jj][r] = fmaf(lk[r], kTwo24, dz[r]);
        }
      }
      float pv[4][4];
      softmax_step_off(lg, pv, m_off);
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        if (pr == 1 && !has_b) break;
        const uint8_t* slot = pr ? sb : sa;
        PageOps<D> P[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          P[j].template read_v<CS>(slot + j * HB, l16, quad);
          const int pg = page_of(k + pr, j);
          if (!INTERIOR && (!page_live(pg) || 16 * pg < m0 || 16 * pg + 16 > m1)) {
            // boundary (or absent) page: clear scale/zero of slots outside the middle
            bool keep[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 16 * pg + 4 * quad + r;
              keep[r] = page_live(pg) && t >= m0 && t < m1;
            }
            const uint32_t k01 = pair_keep(keep[0], keep[1]), k23 = pair_keep(keep[2], keep[3]);
#pragma unroll
            for (int g = 0; g < NGV; ++g) { P[j].vs[2 * g] &= k01; P[j].vs[2 * g + 1] &= k23; }
            P[j].vz[0] &= k01;
            P[j].vz[1] &= k23;
          }
        }
        // K-slot e = 2 page + token pair, half = token parity
        const uint32_t bp[4] = {pack_f16x2_rtz(pv[2 * pr][0], pv[2 * pr][1]), pack_f16x2_rtz(pv[2 * pr][2], pv[2 * pr][3]),
                                pack_f16x2_rtz(pv[2 * pr + 1][0], pv[2 * pr + 1][1]),
                                pack_f16x2_rtz(pv[2 * pr + 1][2], pv[2 * pr + 1][3])};
        // zero terms (rows g < NG) and the softmax denominator (row NG: ones),
        // both from the same f16 probabilities the value sums use
        acc_z = mfma_f16(u32x4{(P[0].vz[0] & zrow) | ones, (P[0].vz[1] & zrow) | ones, (P[1].vz[0] & zrow) | ones,
                               (P[1].vz[1] & zrow) | ones},
                         u32x4{bp[0], bp[1], bp[2], bp[3]}, acc_z);
        // B operands: probabilities times V scales, NGV of them (CS = 1: one
        // per group; else operand h holds column n's group CS h + n%CS)
        u32x4 bs[NGV];
#pragma unroll
        for (int g = 0; g < NGV; ++g)
          bs[g] = u32x4{hmul2(bp[0], P[0].vs[2 * g]), hmul2(bp[1], P[0].vs[2 * g + 1]),
                        hmul2(bp[2], P[1].vs[2 * g]), hmul2(bp[3], P[1].vs[2 * g + 1])};
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int w = cb >> 2, bb = cb & 3;
          const uint32_t m = 0x00030003u << (2 * bb);
          const u32x4 a = {P[0].vc[w] & m, shr8_halves(P[0].vc[w]) & m, P[1].vc[w] & m, shr8_halves(P[1].vc[w]) & m};
          acc[cb] = mfma_f16(a, bs[(cb >> 1) / CS], acc[cb]);
        }
      }
    };

    // Ring of kRing pair slots per wave, pair j in slot j % kRing.  kDepth
    // pairs per iteration, in steps of two: before each step the next two
    // pairs are requested (into the slots the previous step read) and the
    // step's own pairs are waited for.  The loads after a step's pairs are
    // the kDepth pairs requested since, hence vmcnt(kDepth LOADS).
    // Loads run unconditionally, past the last pair too (clamped), so that
    // the count holds; only the compute is skipped.
    // (A page-id block request between them only makes the wait stronger.)
    static_assert(32 % kDepth == 0 && kDepth % 2 == 0, "page-id blocks and pair steps");
    constexpr int kAfter = kDepth * PD::LOADS;
    for (int k = 0; k < n_mine; k += kDepth) {
      // page-id block of this group's prefetch targets (advances one block at
      // a time; its LDS copy was requested a whole block of pairs ago)
      const int jb = min(k + kDepth, n_mine - 1) >> 5;
      if (jb != tab_blk) {
        tab = clamp_page(int(my_tabs[64 * (jb & 1) + lane]));
        tab_blk = jb;
        tab_dma(jb + 1);
      }
      const int s0 = k % kRing;
      auto slot = [&](int i) {
        const int t = s0 + i;
        return ring + (t >= kRing ? t - kRing : t) * PD::SLOT;
      };
      auto step = [&](int kk) {
        if (kk < n_mine) {
          const bool has_b = kk + 1 < n_mine;
          const int pg0 = page_of(kk, 0), pg3 = page_of(kk + 1, 1);
          const bool interior = has_b && pg3 + 1 <= c1 && 16 * pg0 >= m0 && 16 * pg3 + 16 <= m1 &&
                                page_of(kk, 1) + 1 <= c1 && 16 * page_of(kk + 1, 0) >= m0;
          uint8_t* sa = slot(kk - k);
          uint8_t* sb = slot(kk - k + 1);
          if (interior) do_two(kk, sa, sb, true, std::true_type{});
          else do_two(kk, sa, sb, has_b, std::false_type{});
        }
      };
#pragma unroll
      for (int st = 0; st < kDepth; st += 2) {
        pair_dma(min(k + kDepth + st, n_mine - 1), slot(kDepth + st));
        pair_dma(min(k + kDepth + st + 1, n_mine - 1), slot(kDepth + st + 1));
        wait_vm<kAfter>();
        step(k + st);
      }
    }
    wait_vm<0>();  // no ring load lands after the results reuse the ring
    if (UPD && owner) own_token(qf4);
  }

  // ---- per-wave results -> LDS, merged over the 8 waves ----
  // row NG of the zero-term tile (lane (n, NG/4), element NG%4) holds an INT2
  // chunk's denominator; BF16 chunks summed theirs per lane
  const float l_w = is_raw ? wave_sum16(l_part) : __shfl(acc_z[NG & 3], l16 + 16 * (NG >> 2), 64);
  float zg[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) zg[g] = __shfl(acc_z[g], l16, 64);  // Z[g][n] lives in lane (n, quad 0)
  if (quad == 0) {
    s_m[wave * 16 + l16] = m_run;
    s_l[wave * 16 + l16] = l_w;
  }
  lds_barrier();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w * 16 + l16]);
  const float sc = (m_run == kNegInf) ? 0.f : exp2f(m_run - M);
  {
    // the column holding query qi's value sums of block cb: CS qi + (group
    // of cb) % CS for INT2 chunks, CS qi for BF16 chunks
    const int qi = l16 / CS;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const bool mine = qi < G && (CS == 1 || l16 % CS == (is_raw ? 0 : (cb >> 1) % CS));
      if (!mine) continue;
      f32x4 v;
      if (is_raw) {
        v = acc[cb] * sc;
      } else {
        const float fpos = kTwo24 / float(1 << (2 * (cb & 3)));
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = sc * (acc[cb][r] * fpos + zg[cb >> 1]);
      }
      *reinterpret_cast<f32x4*>(s_res + (wave * G + qi) * D + 16 * cb + 4 * quad) = v;
    }
  }
  lds_barrier();

  // ---- workgroup record [m G][l G][value sums G D][basis flag] -> workspace ----
  float* rec = p.partials + ((size_t(b) * p.n_kv + h) * p.cap + kseg) * size_t(p.rec_floats);
  if (tid < G) {
    const int cq = CS * tid;  // a column of query tid
    float mm = kNegInf;
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, s_m[w * 16 + cq]);
    float ll = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w * 16 + cq];
      if (mw != kNegInf) ll += exp2f(mw - mm) * s_l[w * 16 + cq];
    }
    if (UPD && owner) {  // fused step: the token handled apart joins the record
      const float lt = own_l[tid];
      const float mn = fmaxf(mm, lt);
      const float f1 = (mm == kNegInf) ? 0.f : exp2f(mm - mn), f2 = exp2f(lt - mn);
      ll = __builtin_fmaf(ll, f1, f2);
      mm = mn;
      own_l[16 + tid] = f1;
      own_l[32 + tid] = f2;
    }
    st_dev(rec + tid, mm);
    st_dev(rec + G + tid, ll);
  }
  if (UPD && owner) lds_barrier();
  if (tid == 0) st_dev(rec + 2 * G + G * D, is_raw ? 1.f : 0.f);
  for (int e = tid; e < G * D; e += kThreads) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) a += s_res[w * G * D + e];
    if (UPD && owner) a = __builtin_fmaf(a, own_l[16 + e / D], own_l[32 + e / D] * own_kv[D + e % D]);
    st_dev(rec + 2 * G + e, a);
  }
  // Hand-off to the unit's last workgroup: every thread's record stores are
  // ordered before the barrier, the barrier before thread 0's arrival, a
  // release at device scope; the last arrival acquires at device scope and
  // its barrier orders the acquire before every thread's record loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(p.counters + b * p.n_kv + h, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_flag[0] = (old == nseg - 1) ? 1 : 0;
  }
  __syncthreads();
  if (s_flag[0]) {

  // ---- last workgroup: log-sum-exp merge of the chunk records ----
  // The weights w_s[n] = 2^(m_s[n] - M[n]) come first, from every record's
  // max and sum, so the value sums are added without rescaling:
  //   out = (R_V^T-rotated sum_s w_s v_s over INT2 chunks + sum_s w_s v_s over
  //          BF16 chunks) / sum_s w_s l_s
  // Loads of maxima, sums, flags and the first values go out together, then R_V.
  const int n_s = nseg;
  const float* recs = p.partials + (size_t(b) * p.n_kv + h) * p.cap * size_t(p.rec_floats);
  float* s_wr = s_res;                       // [kMaxChunks][16] weights of INT2 records
  float* s_wu = s_wr + kMaxChunks * 16;      // [kMaxChunks][16] weights of BF16 records
  float* s_red = s_wu + kMaxChunks * 16;     // [2][8 waves][16] partial max / sum
  float* m_rot = s_red + 2 * kWaves * 16;    // [G][D] merged, rotated basis
  float* m_raw = m_rot + G * D;              // [G][D] merged, model basis
  constexpr int kPass = kMaxChunks * 16 / kThreads;  // (record, row) slots per thread
  const int ms_n = tid & 15;
  const int n_pass = (n_s * 16 + kThreads - 1) / kThreads;  // passes holding real records
  float cm[kPass], cl[kPass], cf[kPass];
#pragma unroll
  for (int i = 0; i < kPass; ++i) {  // clamped addresses: every load is in bounds
    cm[i] = kNegInf;
    cl[i] = cf[i] = 0.f;
    if (i < n_pass) {
      const int s = min((tid >> 4) + i * (kThreads / 16), n_s - 1), n = min(ms_n, G - 1);
      cm[i] = ld_dev(recs + size_t(s) * p.rec_floats + n);
      cl[i] = ld_dev(recs + size_t(s) * p.rec_floats + G + n);
      cf[i] = ld_dev(recs + size_t(s) * p.rec_floats + 2 * G + G * D);
    }
  }
  // Balanced slices, up to half a batch of records (the usual case) and more
  // than one round of elements (G D > kThreads): one batch holds the values
  // of two element rounds, [e0, e0 + kThreads) and the next, so that one wait
  // serves both (measured: 96q/8kv batch 64, 2% faster).  CS column slots
  // hold at most 16 / CS queries, so the four-slot kernel at d = 128 and the
  // two- and four-slot ones at d = 64 never pair.  The per-unit kernels inline
  // the merge at several segment sites and keep the single-round form: the
  // second form's code cost them what its wait saved.
  constexpr int kHalf = kMergeBatch / 2;
  constexpr bool kCanPair = SLICES && !ALL_RAW && (16 / CS) * D > kThreads;
  const bool paired = kCanPair && n_s <= kHalf && G * D > kThreads;
  float vv[kMergeBatch];
  auto load_batch = [&](int e0, int s0) {
    if (paired) {
      const size_t ea = size_t(2 * G + min(e0 + tid, G * D - 1));
      const size_t eb = size_t(2 * G + min(e0 + kThreads + tid, G * D - 1));
#pragma unroll
      for (int k = 0; k < kHalf; ++k) vv[k] = ld_dev(recs + size_t(min(k, n_s - 1)) * p.rec_floats + ea);
      if (e0 + kThreads < G * D)
#pragma unroll
        for (int k = 0; k < kHalf; ++k) vv[kHalf + k] = ld_dev(recs + size_t(min(k, n_s - 1)) * p.rec_floats + eb);
    } else {
      const size_t e = size_t(2 * G + min(e0 + tid, G * D - 1));
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) vv[k] = ld_dev(recs + size_t(min(s0 + k, n_s - 1)) * p.rec_floats + e);
    }
  };
  load_batch(0, 0);
  // R_V rows of output block cb = wave, requested after the records (the
  // weights wait only for the records; R_V is needed last)
  const float* rv = p.r_v + size_t(h) * D * D;
  f32x4 rva[NB][NKB][2];
  if (!ALL_RAW && wave < NCB) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const float* src = rv + size_t(16 * (wave + kWaves * j) + l16) * D + 32 * kb + 8 * quad;
        rva[j][kb][0] = *reinterpret_cast<const f32x4*>(src);
        rva[j][kb][1] = *reinterpret_cast<const f32x4*>(src + 4);
      }
  }
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < kPass; ++i) {
    const int s = (tid >> 4) + i * (kThreads / 16);
    if (s < n_s && ms_n < G) mx = fmaxf(mx, cm[i]);
  }
  mx = wave_max16(mx);
  if (quad == 0) s_red[wave * 16 + ms_n] = mx;
  lds_barrier();
  float Mn = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) Mn = fmaxf(Mn, s_red[w * 16 + ms_n]);
  float lsum = 0.f;
  // pass i holds records [32 i, 32 i + 32), the value rounds below read the
  // weights of records [0, 32 n_pass): later passes are neither read nor written
  static_assert(kMergeBatch == kThreads / 16, "a merge round reads the records of one pass");
#pragma unroll
  for (int i = 0; i < kPass; ++i) {
    if (i >= n_pass) break;
    const int s = (tid >> 4) + i * (kThreads / 16);
    const bool ok = s < n_s && ms_n < G && cm[i] != kNegInf;
    const float wgt = ok ? exp2f(cm[i] - Mn) : 0.f;
    lsum = fmaf(wgt, cl[i], lsum);
    s_wr[s * 16 + ms_n] = cf[i] != 0.f ? 0.f : wgt;  // every slot read is written: zero past n_s
    s_wu[s * 16 + ms_n] = cf[i] != 0.f ? wgt : 0.f;
  }
  lsum = wave_sum16(lsum);
  if (quad == 0) s_red[16 * kWaves + wave * 16 + ms_n] = lsum;
  lds_barrier();
  auto store_merged = [&](int e, int n, float orot, float oraw) {
    if (e < G * D) {
      float Ln = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) Ln += s_red[16 * kWaves + w * 16 + n];
      const float inv = 1.f / Ln;
      m_rot[e] = orot * inv;
      m_raw[e] = oraw * inv;
    }
  };
  if (paired) {
    // weights of records [n_s, kHalf) are zero
    for (int e0 = 0; e0 < G * D; e0 += 2 * kThreads) {
      if (e0 > 0) load_batch(e0, 0);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (e0 + r * kThreads >= G * D) break;  // uniform: the second round's values were not loaded
        const int e = e0 + r * kThreads + tid;
        const int n = min(e / D, 15);
        float orot = 0.f, oraw = 0.f;
#pragma unroll
        for (int k = 0; k < kHalf; ++k) {
          orot = fmaf(s_wr[k * 16 + n], vv[r * kHalf + k], orot);
          oraw = fmaf(s_wu[k * 16 + n], vv[r * kHalf + k], oraw);
        }
        store_merged(e, n, orot, oraw);
      }
    }
  } else {
    for (int e0 = 0; e0 < G * D; e0 += kThreads) {
      const int e = e0 + tid;
      const int n = min(e / D, 15);
      float orot = 0.f, oraw = 0.f;
      for (int s0 = 0; s0 < n_s; s0 += kMergeBatch) {
        if (e0 > 0 || s0 > 0) load_batch(e0, s0);
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          orot = fmaf(s_wr[(s0 + k) * 16 + n], vv[k], orot);
          oraw = fmaf(s_wu[(s0 + k) * 16 + n], vv[k], oraw);
        }
      }
      store_merged(e, n, orot, oraw);
    }
  }
  lds_barrier();
  // out^T[c][n] = raw[n][c] + sum_k R_V[c][k] rot[n][k]   (bf16 hi/lo splits, 3 MFMAs)
  if (wave < NCB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int cb = wave + kWaves * j;
      f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
      if (!ALL_RAW) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          uint32_t ah[4], al[4], bh[4], bl[4];
          const float* rot_row = m_rot + qrow * D + 32 * kb + 8 * quad;
#pragma unroll
          for (int k = 0; k < 8; k += 2) {
            split2x2(rva[j][kb][k / 4][k % 4], rva[j][kb][(k + 1) / 4][(k + 1) % 4], ah[k / 2], al[k / 2]);
            split2x2(rot_row[k], rot_row[k + 1], bh[k / 2], bl[k / 2]);
          }
          const u32x4 AH{ah[0], ah[1], ah[2], ah[3]}, AL{al[0], al[1], al[2], al[3]};
          const u32x4 BH{bh[0], bh[1], bh[2], bh[3]}, BL{bl[0], bl[1], bl[2], bl[3]};
          a4 = mfma_bf16(AL, BH, a4);
          a4 = mfma_bf16(AH, BL, a4);
          a4 = mfma_bf16(AH, BH, a4);
        }
      }
      if (l16 < G) {
        uint16_t* o = p.out + (size_t(b) * p.Hq + h * G + l16) * D + 16 * cb + 4 * quad;
        const float* rw = m_raw + l16 * D + 16 * cb + 4 * quad;
        u32x2 ov;
        ov[0] = bf16x2_rne(a4[0] + rw[0], a4[1] + rw[1]);
        ov[1] = bf16x2_rne(a4[2] + rw[2], a4[3] + rw[3]);
        *reinterpret_cast<u32x2*>(o) = ov;
      }
    }
  }
  if (tid == 0) __hip_atomic_store(p.counters + b * p.n_kv + h, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }  // merge
  };

  if constexpr (!SLICES) {
    // Per-unit items (few units): workgroup wg is item x of unit (b, h).  Item 0
    // takes the unit's BF16 pages and the first f0 INT2 pages (f0 = 0 for
    // short items), item x >= 1 INT2 pages [q0 + f0 + (x-1) split, + split)
    // (for the all-BF16 cache: item x takes BF16 positions
    // [x split, (x+1) split)).  INT2 items x >= 1 do not depend on the length,
    // so their requests go out before it is read.
    // The KV head varies fastest over the workgroup index: the workgroups
    // dispatched together read the same pages' head images (one page holds
    // every head of its 16 tokens), which keeps HBM rows open.
    const int per = p.unit_items, split = p.fixed_ppw, f0 = p.first_int2;
    const int hw = wg % p.n_kv, bx = wg / p.n_kv, x = bx % per;
    set_unit(bx / per, hw);
    // the length is requested first: waiting for it then leaves the early
    // page requests in flight
    const int L = p.seq_lens[b];
    if (!ALL_RAW && p.speculate && x >= 1) speculate_at(b, h, (p.S >> 4) + f0 + (x - 1) * split);
    if (L <= 0) {
      if (x == 0 && h == 0)
        for (int e = tid; e < p.Hq * D; e += kThreads) p.out[size_t(b) * p.Hq * D + e] = 0;
      return;
    }
    sp = make_plan<ALL_RAW>(p, L);
    if (ALL_RAW) {
      const int nseg = (sp.n_raw + split - 1) / split;
      if (x >= nseg) return;
      segment(std::true_type{}, true, x * split, min(sp.n_raw, (x + 1) * split), nseg, x);
      return;
    }
    // item 0: the BF16 pages, then the first c0n INT2 pages (a second segment
    // in the same workgroup); item x >= 1: INT2 pages [q0 + c0n + (x-1) split, + split)
    const int has_raw = sp.n_raw > 0 ? 1 : 0, nmid = sp.q1 - sp.q0, c0n = min(nmid, f0);
    const int head = c0n > 0 ? 1 : 0;
    const int nq = head + (nmid - c0n + split - 1) / split;
    if (x == 0) {
      if (has_raw) segment(std::true_type{}, true, 0, sp.n_raw, has_raw + nq, 0);
      if (head) {
        if (has_raw) lds_barrier();  // LDS of that segment's merge is rewritten by this one
        segment(std::false_type{}, false, sp.q0, sp.q0 + c0n, has_raw + nq, has_raw);
      }
      return;
    }
    if (x - 1 >= nq - head) return;
    const int q0 = sp.q0 + c0n + (x - 1) * split;
    segment(std::true_type{}, false, q0, min(sp.q1, q0 + split), has_raw + nq, has_raw + head + x - 1);
  } else {
  // Balanced slices (many units): the units, sequence-major, put their work
  // (BF16 sink and recent pages, INT2 pages, then seg_pages(G) positions per
  // nonempty range that hold no pages) in one row; workgroup wg takes the
  // slice [wg ppw, wg ppw + ppw) of it.  A segment is the part of a slice
  // inside one unit and one page kind; each leaves one record, and the unit's
  // last segment to finish merges its records.
  // Work of the sequences: thread t sums a block of them; a block scan gives
  // each block's first position.
  int* s_scan = reinterpret_cast<int*>(s_res);  // [kWaves] wave totals, [kWaves] owner's first position
  int* s_scani = s_scan + 32;                   // [kWaves] wave max cost, [kWaves] owner
  const int seq_blk = (p.batch + kThreads - 1) / kThreads;
  int v = 0, cmax = 0;
  {
    const int b0 = tid * seq_blk, b1 = min(p.batch, b0 + seq_blk);
    for (int bb = b0; bb < b1; ++bb) {
      const int L = p.seq_lens[bb];
      const int c = make_plan<ALL_RAW>(p, max(L, 0)).cost;
      v += p.n_kv * c;
      cmax = max(cmax, c);
      if (L <= 0 && wg == 0) {  // no tokens: zero output
        u32x4* o = reinterpret_cast<u32x4*>(p.out + size_t(bb) * p.Hq * D);
        for (int e = 0; e < p.Hq * D / 8; ++e) o[e] = u32x4{0, 0, 0, 0};
      }
    }
  }
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  int wmax = cmax;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wmax = max(wmax, __shfl_xor(wmax, o, 64));
  if (lane == 63) s_scan[wave] = inc;
  if (lane == 0) s_scani[wave] = wmax;
  lds_barrier();
  int total = 0, woff = 0, max_cost = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = s_scan[w];
    woff += w < wave ? t : 0;
    total += t;
    max_cost = max(max_cost, s_scani[w]);
  }
  // workgroup-uniform values read from LDS: scalar registers from here on
  total = __builtin_amdgcn_readfirstlane(total);
  max_cost = __builtin_amdgcn_readfirstlane(max_cost);
  const int ppw = slice_pages(p, total, max_cost);
  if ((long long)wg * ppw >= total) return;
  const int lo = wg * ppw;
  const int hi = int(min((long long)total, (long long)lo + ppw));
  const int excl = woff + inc - v;  // first position of this thread's sequences
  if (v > 0 && excl <= lo && lo < excl + v) {
    s_scan[kWaves] = excl;
    s_scani[kWaves] = tid;
  }
  lds_barrier();
  // walk the owner's block to the unit holding position lo
  int Cu = __builtin_amdgcn_readfirstlane(s_scan[kWaves]);
  {
    int bb = __builtin_amdgcn_readfirstlane(s_scani[kWaves]) * seq_blk;
    sp = make_plan<ALL_RAW>(p, max(p.seq_lens[bb], 0));
    while (Cu + p.n_kv * sp.cost <= lo) {
      Cu += p.n_kv * sp.cost;
      ++bb;
      sp = make_plan<ALL_RAW>(p, max(p.seq_lens[bb], 0));
    }
    const int hh = (lo - Cu) / sp.cost;
    Cu += hh * sp.cost;
    set_unit(bb, hh);
  }
  int pos = lo;
  // move pos onto pages of this or a later unit; false if none before hi
  auto settle = [&]() -> bool {
    for (;;) {
      if (pos < Cu + sp.real) return pos < hi;
      const int nxt = Cu + sp.cost;
      if (nxt >= hi) return false;
      pos = Cu = nxt;
      if (h + 1 < p.n_kv) {
        set_unit(b, h + 1);
      } else {
        int bb = b;
        do {
          ++bb;
          sp = make_plan<ALL_RAW>(p, max(p.seq_lens[bb], 0));
        } while (sp.cost == 0);
        set_unit(bb, 0);
      }
    }
  };
  if (!settle()) return;
  auto run = [&](auto first_tag) __attribute__((always_inline)) {
    const int raw_end = Cu + sp.n_raw, real_end = Cu + sp.real;
    const bool is_raw = pos < raw_end;
    const int seg_end = min(hi, is_raw ? raw_end : real_end);
    const int n_raw_seg = sp.n_raw > 0 ? (raw_end - 1) / ppw - Cu / ppw + 1 : 0;
    const int nseg = n_raw_seg + (sp.real > sp.n_raw ? (real_end - 1) / ppw - raw_end / ppw + 1 : 0);
    const int kseg = is_raw ? wg - Cu / ppw : n_raw_seg + wg - raw_end / ppw;
    segment(first_tag, is_raw, is_raw ? pos - Cu : sp.q0 + (pos - raw_end),
            is_raw ? seg_end - Cu : sp.q0 + (seg_end - raw_end), nseg, kseg);
    pos = seg_end;
    if (!settle()) return false;
    lds_barrier();  // LDS of this segment's merge is rewritten by the next segment
    return true;
  };
  while (run(std::false_type{})) {
  }
  }  // balanced slices
}

}  // namespace

namespace oscar_launch {

int decode_max_records() { return kMaxChunks; }

int decode_min_slice() { return kMinSlice; }

int decode_seg_pages() { return kSegPagesMax; }

int decode_seg_pages_of(int G) { return seg_pages(G); }

int decode_own_pages() { return kOwnPages; }

size_t decode_lds_bytes(int d, int G, bool all_raw) {
  const int ng = d / 32;
  const size_t slot = d == 128 ? PairDma<128>::SLOT : PairDma<64>::SLOT;
  const size_t rings = all_raw ? 0 : size_t(kWaves) * kRing * slot;
  size_t res = size_t(kWaves) * G * d;                              // per-wave results
  res = std::max(res, size_t(kMaxChunks) * 32 + 2 * kWaves * 16 + size_t(2) * G * d);  // merge
  return (size_t(ng) * 256 + kMisc + kWaves * 2 * 64) * 4 + std::max(rings, res * 4);
}

hipError_t paged_decode(int d, bool all_raw, const void* int2_pool, int n_int2_pages, const void* bf16_pool, int n_kv, int G, int S,
                        int W, int Hq, const void* q, int batch, const int32_t* seq_lens, const int32_t* bt_q,
                        const int32_t* bt_h, int max_pages, const float* r_k, const float* r_v, float sm_scale,
                        bool per_unit, int unit_items, int first_int2, int fixed_ppw, int n_wg, int cap, int max_seq_len,
                        float* partials, int32_t* counters, int rec_floats, void* out, bool speculate,
                        const void* k_new, const void* v_new, float tau_k, float tau_v, hipStream_t stream) {
  DecParams p{static_cast<const uint8_t*>(int2_pool), std::max(1, n_int2_pages), static_cast<const uint16_t*>(bf16_pool), n_kv, G, S, W, Hq,
              static_cast<const uint16_t*>(q), seq_lens, bt_q, bt_h, max_pages, r_k, r_v, sm_scale, fixed_ppw,
              partials, counters, rec_floats, cap, static_cast<uint16_t*>(out), speculate ? 1 : 0, max_seq_len, batch,
              per_unit ? 1 : 0, unit_items, first_int2, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
              tau_k, tau_v};
  const bool upd = k_new != nullptr;
  const dim3 grid(static_cast<unsigned>(n_wg));
  const size_t lds = decode_lds_bytes(d, G, all_raw);
  // column slots per query: as many as the 16 MFMA columns give every query
  const int cs = all_raw ? 1 : G <= 4 ? 4 : G <= 8 ? 2 : 1;
#define OSCAR_DECODE_LAUNCH(DD, RAW, GCOL)                                                                              \
  do {                                                                                                                 \
    if (upd && !RAW) {                                                                                                 \
      if (per_unit) hipLaunchKernelGGL((decode_kernel<DD, RAW, false, GCOL, !RAW>), grid, dim3(kThreads), lds, stream, p); \
      else hipLaunchKernelGGL((decode_kernel<DD, RAW, true, GCOL, !RAW>), grid, dim3(kThreads), lds, stream, p);           \
    } else {                                                                                                           \
      if (per_unit) hipLaunchKernelGGL((decode_kernel<DD, RAW, false, GCOL, false>), grid, dim3(kThreads), lds, stream, p); \
      else hipLaunchKernelGGL((decode_kernel<DD, RAW, true, GCOL, false>), grid, dim3(kThreads), lds, stream, p);           \
    }                                                                                                                  \
  } while (0)
  if (d == 128) {
    if (all_raw) OSCAR_DECODE_LAUNCH(128, true, 1);
    else if (cs == 4) OSCAR_DECODE_LAUNCH(128, false, 4);
    else if (cs == 2) OSCAR_DECODE_LAUNCH(128, false, 2);
    else OSCAR_DECODE_LAUNCH(128, false, 1);
  } else {
    if (all_raw) OSCAR_DECODE_LAUNCH(64, true, 1);
    else if (cs == 4) OSCAR_DECODE_LAUNCH(64, false, 4);
    else if (cs == 2) OSCAR_DECODE_LAUNCH(64, false, 2);
    else OSCAR_DECODE_LAUNCH(64, false, 1);
  }
#undef OSCAR_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace oscar_launch
