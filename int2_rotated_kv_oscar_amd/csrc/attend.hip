// Paged attention over the mixed cache with many query columns: chunked
// prefill ("extend") over INT2 or INT4 pages, and the INT4 cache's decode
// ([TS] 2.2.B "Kernel Integration": paged attention, prefix caching; [TS] 3:
// serving with paged KV layouts and prefix caching; [TS] 4 "Scalability": the
// INT4 KV cache OSCAR is compared with).
//
// A workgroup of NWV waves owns 16 NCW CB query columns of one (sequence, KV
// head): a column is one (new row, query head of the group) pair, taken
// row-major, so the G heads of a row sit side by side.  Extend: every wave
// holds CB = 2 blocks of 16 columns.  The decode (at most 16 query heads per
// KV head): wave 0 holds the one block, the other waves help decode steps.  It walks a chunk of
// the unit's work, 32 tokens per step: page pairs of the BF16 sink/recent
// pages, page pairs of the quantized middle pages, then (extend) tiles of 32
// new rows.  Each step is decoded once into an LDS tile shared by the waves:
// keys token-major and values channel-major, as f16 (quantized tokens: c s + z
// in the rotated basis) or as the raw bf16 bits (BF16 pages, new rows).  Tokens
// outside their region (stale slots of recycled pages, rows past the end) are
// written as zeros and their logits masked, so nothing stale reaches a sum.
// Every column-holding wave then runs, for its columns, the transposed products of
// flash attention on the matrix cores: logits^T = K Q^T (16x16x32, tokens x
// columns) and out^T += V^T P^T, with the online softmax over the tokens of a
// column in between.  Quantized tokens use the rotated query q~ = q R_K and
// a value sum in the rotated basis; raw tokens use q and a second value sum;
// out = raw + rot R_V^T at the end.  With more than one chunk per unit the
// chunks' states (max, sum, both value sums) go to a workspace and a second
// kernel merges them by log-sum-exp.
#include <algorithm>

#include "device_utils.h"
#include "kernels.h"
#include "layout.h"

using namespace oscar_dev;

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 pair of (a, b), element 0 in the low half, rounded to nearest even by
// the packed hardware conversion (one instruction per pair; the same bits as
// the scalar rounding for finite values)
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// (a, b) = hi + lo, each a bf16 pair, to 16 significant bits
__device__ __forceinline__ void split2x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = bf16x2_rne(a, b);
  lo = bf16x2_rne(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

constexpr float kNegInfA = -__builtin_inff();
constexpr float kSlackA = 4.0f;  // log2 units

struct AttParams {
  const uint8_t* qpool;    // INT2 or INT4 pool
  int32_t n_qpages;
  const uint16_t* bf16_pool;
  int32_t n_bpages;
  int32_t n_kv, G, S, W, Hq;
  const uint16_t* q;       // bf16 [rows][Hq][D]
  const uint16_t* k_new;   // bf16 [rows][n_kv][D] (extend)
  const uint16_t* v_new;
  const int32_t* cu;       // extend: [B + 1] row offsets
  const int32_t* clen;     // cached length per sequence (decode: the length)
  const int32_t* bt_q;
  const int32_t* bt_h;
  int32_t max_pages;
  const float* r_k;
  const float* r_v;
  float sm_scale;
  int32_t n_ct;            // column tiles per unit in the grid
  int32_t n_chunks;        // chunks per (unit, column tile)
  int32_t spc;             // steps per chunk
  float* rec;              // [unit][tile][chunk][column][2 + 2D] when n_chunks > 1
  uint16_t* out;           // bf16 [rows][Hq][D]
};

// Geometry of the quantized page-heads (INT2: the MFMA-shaped layout; INT4:
// row-owned nibbles).
template <int D, int BITS>
struct QGeo : QLayout<D, BITS> {
  static constexpr int BYTES = QLayout<D, BITS>::HEAD_BYTES;
};

// LDS tile of one step: keys [32 tokens][KROW], values [D][VROW] (u16 bits).
template <int D>
struct Tile {
  static constexpr int KROW = D + 8;   // padded rows: the lanes of an operand read hit distinct banks
  // 18 words: the 16 rows of an 8-byte value-operand read fall on distinct
  // bank pairs (rows are 8-byte aligned, not 16)
  static constexpr int VROW = 32 + 4;
  static constexpr int ELEMS = 32 * KROW + D * VROW;
};

__device__ __forceinline__ uint32_t f16pair(float a, float b) { return pack_f16x2(a, b); }
// Dequantized f16 pair (c0 s0 + z0, c1 s1 + z1) from a code pair held as f16
// subnormals (c 2^-24 in each half of x, from one mask of the code word):
// with S = s 2^24 the products c s are exact, and each half is one mixed-
// precision FMA rounded once to f16, as fma(float(c), s, z) then to f16.
constexpr float kTwo24 = 16777216.0f;
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t dq_pair(uint32_t x, float S0, float z0, float S1, float z1) {
  const h16x2 c = __builtin_bit_cast(h16x2, x);
  const h16x2 v = {(_Float16)__builtin_fmaf((float)c[0], S0, z0), (_Float16)__builtin_fmaf((float)c[1], S1, z1)};
  return __builtin_bit_cast(uint32_t, v);
}

// Region plan of a length-P cache: BF16 pages (range A = sink, range B =
// recent; one range when they meet) and the quantized pages [q0, q1).
struct Regions {
  int P, s1, m0, m1, r0;
  int ra1, rb0, rb1, q0, q1, n_raw;
  __device__ __forceinline__ int raw_page(int i) const { return i < ra1 ? i : rb0 + (i - ra1); }
};
__device__ __forceinline__ Regions make_regions(int P, int S, int W) {
  Regions g;
  g.P = P;
  const int n_pages = (P + 15) >> 4;
  g.s1 = min(S, P);
  g.m0 = S;
  g.m1 = P - W;
  g.r0 = max(S, P - W);
  const int hs1 = (g.s1 + 15) >> 4;
  const int hr0 = g.r0 < P ? (g.r0 >> 4) : n_pages;
  if (hs1 >= hr0) {
    g.ra1 = n_pages; g.rb0 = g.rb1 = n_pages;
  } else {
    g.ra1 = hs1; g.rb0 = hr0; g.rb1 = n_pages;
  }
  g.n_raw = g.ra1 + (g.rb1 - g.rb0);
  if (g.m1 > g.m0) { g.q0 = g.m0 >> 4; g.q1 = (g.m1 + 15) >> 4; }
  else { g.q0 = g.q1 = 0; }
  return g;
}

// ---- step fill: one 32-token step into the LDS tile ----
// Each thread loads its share of a quantized step's bytes into registers
// (issued two steps ahead, so that the loads overlap the products of the
// steps before) and then decodes them into the tile.  Shares: INT2 page pairs
// 2D items (a key code word, a value code word, their scales and zeros), INT4
// page pairs 2D items (a token's 16 channels: two key and two value code words
// of 8 nibbles, their scales and zeros).  Raw steps (BF16 page pairs: 4D key and
// 4D value chunks of 16 B; tiles of 32 new rows likewise) are few per unit
// and are loaded when stored.
template <int D, int BITS, int NTH>
struct Stage {
  static constexpr int NR = (4 * D + NTH - 1) / NTH;       // raw chunks per tensor per thread
  static constexpr int NQ = (2 * D + NTH - 1) / NTH;       // quantized items per thread
  static constexpr int QW = BITS == 2 ? 12 : 8;            // registers per item
  uint32_t qw[NQ][QW];
};

struct StepInfo {
  int kind;  // 0 BF16 page pair, 1 quantized page pair, 2 new rows
  int i0;    // first list position (pages) or first new row
};

__device__ __forceinline__ bool raw_token(const Regions& rg, int pos) {
  return pos < rg.s1 || (pos >= rg.r0 && pos < rg.P);
}

// The raw chunk e (< 4D) of a raw step: its key chunk and its value chunk.
template <int D>
__device__ __forceinline__ void raw_chunk_load(const AttParams& p, const Regions& rg, const int32_t* bth, int h,
                                               int row0, int n_rows, const StepInfo& si, int e, u32x4& kv, u32x4& vv) {
  constexpr int KCH = D / 8;
  kv = u32x4{0, 0, 0, 0};
  vv = u32x4{0, 0, 0, 0};
  if (e >= 4 * D) return;
  if (si.kind == 0) {
    const int j = e / (16 * KCH), tok = (e / KCH) % 16, ch = e % KCH;
    const int li = si.i0 + j;
    if (li < rg.n_raw) {
      const int pg = rg.raw_page(li);
      const uint16_t* base = p.bf16_pool + (size_t(min(max(bth[pg], 0), p.n_bpages - 1)) * p.n_kv + h) * Geo<D>::BF16_HEAD_ELEMS;
      kv = *reinterpret_cast<const u32x4*>(base + tok * D + 8 * ch);
    }
    const int jv = e / (2 * D), c = (e / 2) % D, half = e % 2;
    const int lv = si.i0 + jv;
    if (lv < rg.n_raw) {
      const int pg = rg.raw_page(lv);
      const uint16_t* base = p.bf16_pool + (size_t(min(max(bth[pg], 0), p.n_bpages - 1)) * p.n_kv + h) * Geo<D>::BF16_HEAD_ELEMS;
      vv = *reinterpret_cast<const u32x4*>(base + 16 * D + c * 16 + 8 * half);
    }
  } else {
    const int tok = e / KCH, ch = e % KCH;
    if (si.i0 + tok < n_rows) {
      const size_t off = (size_t(row0 + si.i0 + tok) * p.n_kv + h) * D + 8 * ch;
      kv = *reinterpret_cast<const u32x4*>(p.k_new + off);
      vv = *reinterpret_cast<const u32x4*>(p.v_new + off);
    }
  }
}

template <int D, int BITS, int NTH>
__device__ __forceinline__ void step_load(const AttParams& p, const Regions& rg, const int32_t* btq, const int32_t* bth,
                                          int h, int row0, int n_rows, const StepInfo& si, Stage<D, BITS, NTH>& st,
                                          int t) {
  using SG = Stage<D, BITS, NTH>;
  constexpr int NG = D / 32;
  if (si.kind != 1) {
    return;  // raw steps are loaded when stored
  } else if constexpr (BITS == 2) {
    using QG = QGeo<D, 2>;
    constexpr int NW = D / 64;
#pragma unroll
    for (int it = 0; it < SG::NQ; ++it) {
      const int e0 = t + it * NTH;
      if (NTH > 2 * D && e0 >= 2 * D) break;  // whole waves without an item (wide workgroups)
      const int e = e0 < 2 * D ? e0 : 0;
      const int j = e / D, wi = e % D;
      const int pg = min(rg.q0 + si.i0 + j, rg.q1 - 1);
      const uint8_t* base = p.qpool + (size_t(min(max(btq[pg], 0), p.n_qpages - 1)) * p.n_kv + h) * QG::BYTES;
      const int m = (wi / NW) % 16, w = wi % NW, q = wi / (16 * NW);
      st.qw[it][0] = reinterpret_cast<const uint32_t*>(base + QG::KC)[wi];
      st.qw[it][1] = reinterpret_cast<const uint32_t*>(base + QG::KS)[(m * NG + 2 * w) / 2];
      st.qw[it][2] = reinterpret_cast<const uint32_t*>(base + QG::KZ)[(m * NG + 2 * w) / 2];
      st.qw[it][3] = reinterpret_cast<const uint32_t*>(base + QG::VC)[wi];
      const u32x4 vs = *reinterpret_cast<const u32x4*>(base + QG::VS + 8 * (q * NG + 2 * w));
      const u32x4 vz = *reinterpret_cast<const u32x4*>(base + QG::VZ + 8 * (q * NG + 2 * w));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        st.qw[it][4 + k] = vs[k];
        st.qw[it][8 + k] = vz[k];
      }
    }
  } else {
    using QG = QGeo<D, 4>;
    constexpr int IPP = 16 * (D / 16);  // items per page: (token, 16-channel half group)
#pragma unroll
    for (int it = 0; it < SG::NQ; ++it) {
      const int e0 = t + it * NTH;
      if (NTH > 2 * IPP && e0 >= 2 * IPP) break;  // whole waves without an item
      const int e = e0 < 2 * IPP ? e0 : 0;
      const int j = e / IPP, wi = e % IPP;
      const int pg = min(rg.q0 + si.i0 + j, rg.q1 - 1);
      const uint8_t* base = p.qpool + (size_t(min(max(btq[pg], 0), p.n_qpages - 1)) * p.n_kv + h) * QG::BYTES;
      // token m = wi % 16 (consecutive lanes take consecutive tokens: the
      // value tile's channel rows are then written contiguously), channels
      // 16 hc .. 16 hc + 15 (8 bytes of codes), group hc / 2
      const int m = wi % 16, hc = wi / 16, g = hc / 2;
      const u32x2 kc = *reinterpret_cast<const u32x2*>(base + QG::KC + m * (D / 2) + 8 * hc);
      const u32x2 vc = *reinterpret_cast<const u32x2*>(base + QG::VC + m * (D / 2) + 8 * hc);
      st.qw[it][0] = kc[0];
      st.qw[it][1] = kc[1];
      st.qw[it][2] = vc[0];
      st.qw[it][3] = vc[1];
      st.qw[it][4] = reinterpret_cast<const uint16_t*>(base + QG::KS)[m * NG + g];
      st.qw[it][5] = reinterpret_cast<const uint16_t*>(base + QG::KZ)[m * NG + g];
      st.qw[it][6] = reinterpret_cast<const uint16_t*>(base + QG::VS)[m * NG + g];
      st.qw[it][7] = reinterpret_cast<const uint16_t*>(base + QG::VZ)[m * NG + g];
    }
  }
}

template <int D, int BITS, int NTH>
__device__ __forceinline__ void step_store(const AttParams& p, const Regions& rg, const int32_t* bth, int h, int row0,
                                           int n_rows, const StepInfo& si, const Stage<D, BITS, NTH>& st,
                                           uint16_t* tile, int t) {
  using T = Tile<D>;
  using SG = Stage<D, BITS, NTH>;
  uint16_t* vt = tile + 32 * T::KROW;
  if (si.kind != 1) {
    constexpr int KCH = D / 8;
#pragma unroll
    for (int it = 0; it < SG::NR; ++it) {
      const int e = t + it * NTH;
      if (e >= 4 * D) break;
      u32x4 kv, vv;
      raw_chunk_load<D>(p, rg, bth, h, row0, n_rows, si, e, kv, vv);
      uint32_t vw[4] = {vv[0], vv[1], vv[2], vv[3]};
      if (si.kind == 0) {
        const int j = e / (16 * KCH), tok = (e / KCH) % 16, ch = e % KCH;
        const int li = si.i0 + j;
        if (!(li < rg.n_raw && raw_token(rg, 16 * rg.raw_page(li) + tok))) kv = u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(tile + (16 * j + tok) * T::KROW + 8 * ch) = kv;
        const int jv = e / (2 * D), c = (e / 2) % D, half = e % 2;
        const int lv = si.i0 + jv;
        const int pg = lv < rg.n_raw ? rg.raw_page(lv) : -1;
#pragma unroll
        for (int k = 0; k < 8; ++k) {  // tokens outside the BF16 regions: zero (their bytes may be stale)
          const int pos = 16 * pg + 8 * half + k;
          if (pg < 0 || !raw_token(rg, pos)) vw[k / 2] &= (k & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        *reinterpret_cast<u32x2*>(vt + c * T::VROW + 16 * jv + 8 * half) = u32x2{vw[0], vw[1]};
        *reinterpret_cast<u32x2*>(vt + c * T::VROW + 16 * jv + 8 * half + 4) = u32x2{vw[2], vw[3]};
      } else {
        const int tok = e / KCH, ch = e % KCH;
        *reinterpret_cast<u32x4*>(tile + tok * T::KROW + 8 * ch) = kv;
#pragma unroll
        for (int k = 0; k < 8; ++k) vt[(8 * ch + k) * T::VROW + tok] = uint16_t(vw[k / 2] >> (16 * (k & 1)));
      }
    }
  } else if constexpr (BITS == 2) {
    constexpr int NW = D / 64;
#pragma unroll
    for (int it = 0; it < SG::NQ; ++it) {
      const int e = t + it * NTH;
      if (e >= 2 * D) break;
      const int j = e / D, wi = e % D;
      const int pg = rg.q0 + si.i0 + j;
      auto live = [&](int slot) {
        const int pos = 16 * pg + slot;
        return pg < rg.q1 && pos >= rg.m0 && pos < rg.m1;
      };
      // Key codes r and r + 1 of a word (one token, one group) sit 16 bits
      // apart (the MFMA-shaped page layout), so one shift and mask gives a
      // pair as f16 subnormals.  A slot outside the middle region gets scale
      // and zero 0: its value is 0 whatever stale bytes it holds.
      {  // K word: token m, channels 32 g + 16 hb + 4 quad + r, g in {2w, 2w + 1}
        const int quad = wi / (16 * NW), m = (wi / NW) % 16, w = wi % NW;
        const bool ok = live(m);
        const uint32_t word = st.qw[it][0], ks = st.qw[it][1], kz = st.qw[it][2];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const float S = ok ? f16_to_f32(ks >> (16 * gg)) * kTwo24 : 0.f, z = ok ? f16_to_f32(kz >> (16 * gg)) : 0.f;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const int b = 8 * gg + 4 * hb;  // codes r = 0, 1 at b, b + 16; r = 2, 3 at b + 2, b + 18
            const int c = 32 * (2 * w + gg) + 16 * hb + 4 * quad;
            *reinterpret_cast<u32x2*>(tile + (16 * j + m) * T::KROW + c) =
                u32x2{dq_pair((word >> b) & 0x00030003u, S, z, S, z), dq_pair((word >> (b + 2)) & 0x00030003u, S, z, S, z)};
          }
        }
      }
      {  // V word: tokens 4 q + r, channels c16 + 16 (4 w + bb), group 2 w + bb / 2
        // (each code of a pair has its own token's scale: one code at a time,
        // the f16 scale and zero going into the FMA as they are)
        const int q = wi / (16 * NW), c16 = (wi / NW) % 16, w = wi % NW;
        const uint32_t word = st.qw[it][3];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int c = c16 + 16 * (4 * w + bb), gg = bb >> 1;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int bit = 16 * (r & 1) + 8 * (r >> 1) + 2 * bb;
            const int hidx = 4 * gg + r;  // f16 index in the 16-byte scale/zero loads
            const float s = f16_to_f32(st.qw[it][4 + hidx / 2] >> (16 * (hidx & 1)));
            const float z = f16_to_f32(st.qw[it][8 + hidx / 2] >> (16 * (hidx & 1)));
            v[r] = live(4 * q + r) ? __builtin_fmaf(float((word >> bit) & 3u), s, z) : 0.f;
          }
          *reinterpret_cast<u32x2*>(vt + c * T::VROW + 16 * j + 4 * q) = u32x2{f16pair(v[0], v[1]), f16pair(v[2], v[3])};
        }
      }
    }
  } else {
    constexpr int IPP = 16 * (D / 16);
#pragma unroll
    for (int it = 0; it < SG::NQ; ++it) {
      const int e = t + it * NTH;
      if (e >= 2 * IPP) break;
      const int j = e / IPP, wi = e % IPP;
      const int pg = rg.q0 + si.i0 + j;
      const int m = wi % 16, c0 = 16 * (wi / 16);  // as in step_load
      const int pos = 16 * pg + m;
      const bool ok = pg < rg.q1 && pos >= rg.m0 && pos < rg.m1;
      // codes as f16 subnormals (c 2^-24) with S = s 2^24, as in the INT2
      // case; a key code pair is the two nibbles of one byte: the byte is
      // placed in both halves of a word and masked to its low nibble (low
      // half) and its high nibble (high half, 16 c 2^-24: scale S / 16)
      const float KS = ok ? f16_to_f32(st.qw[it][4]) * kTwo24 : 0.f, kz = ok ? f16_to_f32(st.qw[it][5]) : 0.f;
      const float VS = ok ? f16_to_f32(st.qw[it][6]) * kTwo24 : 0.f, vz = ok ? f16_to_f32(st.qw[it][7]) : 0.f;
#pragma unroll
      for (int hw = 0; hw < 2; ++hw) {
        const uint32_t kw = st.qw[it][hw], vw = st.qw[it][2 + hw];
        uint32_t kp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // byte i of kw into bytes 0 and 2 (selector 0x0C: a zero byte)
          const uint32_t x = __builtin_amdgcn_perm(0u, kw, uint32_t(i) | 0x0C00u | (uint32_t(i) << 16) | 0x0C000000u);
          kp[i] = dq_pair(x & 0x00F0000Fu, KS, kz, KS * 0.0625f, kz);
        }
        *reinterpret_cast<u32x4*>(tile + (16 * j + m) * T::KROW + c0 + 8 * hw) = u32x4{kp[0], kp[1], kp[2], kp[3]};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float x = __builtin_fmaf(f16_to_f32((vw >> (4 * k)) & 15u), VS, vz);
          vt[(c0 + 8 * hw + k) * T::VROW + 16 * j + m] = uint16_t(f16_bits(x));
        }
      }
    }
  }
}

// Unit of a workgroup and the rows of its sequence.
struct UnitRows {
  int b, h, row0, n_rows, P;
};
template <int MODE>
__device__ __forceinline__ UnitRows unit_rows(const AttParams& p, int unit) {
  UnitRows u;
  u.b = unit / p.n_kv;
  u.h = unit % p.n_kv;
  if (MODE == 0) {
    u.row0 = p.cu[u.b];
    u.n_rows = p.cu[u.b + 1] - u.row0;
  } else {
    u.row0 = u.b;
    u.n_rows = 1;
  }
  u.P = p.clen[u.b];
  return u;
}

// ---- the kernel ----
// MODE 0: extend (rows of new tokens at positions P + i, causal over them);
// MODE 1: decode (one query row per sequence at position L - 1, over the
// whole length-L cache).  A wave owns CB blocks of 16 columns (CB = 2 for
// extend), so every decoded step feeds CB times the products.  The steps of
// a unit are listed quantized page pairs first, then BF16 page pairs, then
// (extend) tiles of new rows.  A chunk runs its quantized steps with the
// value sums in the rotated basis, turns them into the model basis (times
// R_V^T on the MFMA) before its first raw step, so one accumulator set
// serves both kinds.
template <int D, int BITS, int NWV, int CB, int MODE>
__global__ __launch_bounds__(64 * NWV, 2) void attend_kernel(AttParams p) {
  using T = Tile<D>;
  constexpr int NCB = D / 16, NKB = D / 32, NTH = 64 * NWV;
  constexpr int NBUF = NWV > 1 ? 2 : 1;
  // waves that own columns: every wave for extend; for the decode (at most
  // 16 query heads per KV head) wave 0, the others decode steps only
  constexpr int NCW = MODE == 1 ? 1 : NWV;
  constexpr int NC = 16 * NCW * CB;  // columns of a tile
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* tiles = lds;                                               // [NBUF][T::ELEMS]
  float* fbuf = reinterpret_cast<float*>(lds + NBUF * T::ELEMS);       // [NCW][16][D] per-wave staging

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int chunk = blockIdx.x % p.n_chunks;
  const int ct = (blockIdx.x / p.n_chunks) % p.n_ct;
  const int unit = blockIdx.x / (p.n_chunks * p.n_ct);
  const UnitRows u = unit_rows<MODE>(p, unit);
  const int b = u.b, h = u.h, row0 = u.row0, n_rows = u.n_rows, P = u.P;

  if (MODE == 1 && P <= 0) {  // no tokens: a zero output (written once per sequence)
    if (h == 0 && ct == 0 && chunk == 0)
      for (int e = tid; e < p.Hq * D; e += NTH) p.out[size_t(b) * p.Hq * D + e] = 0;
    return;
  }
  const int col0 = ct * NC;                        // first column of the tile
  const int n_cols = n_rows * G;                   // columns of the unit
  if (col0 >= n_cols) return;
  // this lane's columns: block c of the wave holds columns col0 + 16 (CB wave + c) + l16
  bool col_ok[CB];
  int ri[CB], hi[CB], qpos[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int col = col0 + 16 * (CB * wave + c) + l16;
    col_ok[c] = wave < NCW && col < n_cols;
    ri[c] = col_ok[c] ? col / G : 0;
    hi[c] = col_ok[c] ? col % G : 0;
    qpos[c] = MODE == 0 ? P + ri[c] : P - 1;       // the column's query position
  }
  const int last_row = min(n_rows, (col0 + NC + G - 1) / G) - 1;  // last row with a column in the tile
  const bool wave_cols = wave < NCW && col0 + 16 * CB * wave < n_cols;  // this wave has columns (uniform)
  auto qrow_of = [&](int c) { return p.q + (size_t(row0 + ri[c]) * p.Hq + h * G + hi[c]) * D; };
  const float qscale = p.sm_scale * kLog2e;

  // ---- work of the unit: quantized page pairs, BF16 page pairs, new-row tiles ----
  const Regions rg = make_regions(max(P, 0), p.S, p.W);
  const int32_t* btq = p.bt_q + size_t(b) * p.max_pages;
  const int32_t* bth = p.bt_h + size_t(b) * p.max_pages;
  const int n_rp = (rg.n_raw + 1) >> 1;
  const int n_qp = (rg.q1 - rg.q0 + 1) >> 1;
  const int n_nt = MODE == 0 ? (last_row + 1 + 31) / 32 : 0;
  const int total = n_qp + n_rp + n_nt;
  // one chunk: every step; several: the quantized steps in chunks of spc,
  // then the raw steps in chunks of their own (no chunk mixes the bases, and
  // the raw steps, loaded without prefetch, run beside the quantized chunks)
  const int nqc = (n_qp + p.spc - 1) / p.spc;
  int s_begin = 0, s_end = total;
  if (p.n_chunks > 1) {
    s_begin = chunk < nqc ? chunk * p.spc : n_qp + (chunk - nqc) * p.spc;
    s_end = min(chunk < nqc ? n_qp : total, s_begin + p.spc);
  }
  // the chunk's quantized steps [qa, qb) and raw steps [ra, s_end) (global step numbers)
  const int qa = s_begin, qb = min(s_end, n_qp), ra = max(s_begin, n_qp);
  const bool has_q = qa < qb;
  constexpr int DEPTH = 2;  // quantized steps whose loads are in flight
  Stage<D, BITS, NTH> stq[DEPTH];
  auto qinfo = [&](int s) {  // steps past the chunk load a valid pair of it, never used
    StepInfo si;
    si.kind = 1;
    si.i0 = 2 * min(s, max(qb - 1, 0));
    return si;
  };
#pragma unroll
  for (int k = 0; k < DEPTH; ++k)
    if (has_q) step_load<D, BITS, NTH>(p, rg, btq, bth, h, row0, n_rows, qinfo(qa + k), stq[k], tid);

  // ---- query operands: q~ = q R_K (f16, pre-scaled by qscale) for the
  // quantized steps, computed for all the tile's columns in CB rounds, wave
  // w computing channel blocks w, w + NWV, ... of the round's column blocks
  // from the R_K values of its A operands (loaded once, straight into
  // registers); q~ goes through LDS to the waves that own the columns.  The
  // raw steps take the raw q (bf16). ----
  u32x4 bq[CB][NKB];
  if (MODE == 1)  // the waves without columns never set bq (nor use it)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) bq[0][kb] = u32x4{0u, 0u, 0u, 0u};
  auto load_raw_q = [&]() {
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const uint16_t* qr = qrow_of(c);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) bq[c][kb] = *reinterpret_cast<const u32x4*>(qr + 32 * kb + 8 * quad);
    }
  };
  if (has_q) {
    constexpr int CPW = NCB / NWV;  // channel blocks per wave
    static_assert(CPW >= 1 && NCB % NWV == 0, "channel blocks split over the waves");
    const float* rk = p.r_k + size_t(h) * D * D;
    // A operands of channel block cb = wave + NWV j, slice kb: lane (l16,
    // quad) holds R_K[32 kb + 8 quad + i][16 cb + l16], i < 8, as bf16 hi + lo
    u32x4 rah[CPW][NKB], ral[CPW][NKB];
    {
      float rv[CPW][NKB][8];
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 8; ++i) rv[j][kb][i] = rk[size_t(32 * kb + 8 * quad + i) * D + 16 * (wave + NWV * j) + l16];
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          uint32_t ph[4], pl[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) split2x2(rv[j][kb][2 * i], rv[j][kb][2 * i + 1], ph[i], pl[i]);
          rah[j][kb] = u32x4{ph[0], ph[1], ph[2], ph[3]};
          ral[j][kb] = u32x4{pl[0], pl[1], pl[2], pl[3]};
        }
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) {  // unrolled: bq[c] needs a constant index
      const uint16_t* qcols[NCW];  // the q rows of the round's column blocks (lane l16's column)
#pragma unroll
      for (int cbk = 0; cbk < NCW; ++cbk) {
        const int col = col0 + 16 * (CB * cbk + c) + l16;
        const int rr = col < n_cols ? col / G : 0, hh = col < n_cols ? col % G : 0;
        qcols[cbk] = p.q + (size_t(row0 + rr) * p.Hq + h * G + hh) * D;
      }
      f32x4 qacc[CPW][NCW];
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int cbk = 0; cbk < NCW; ++cbk) qacc[j][cbk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        u32x4 qk[NCW];  // B operands: the q slice kb of every column block
#pragma unroll
        for (int cbk = 0; cbk < NCW; ++cbk) qk[cbk] = *reinterpret_cast<const u32x4*>(qcols[cbk] + 32 * kb + 8 * quad);
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
          for (int cbk = 0; cbk < NCW; ++cbk) {
            qacc[j][cbk] = mfma_bf16(ral[j][kb], qk[cbk], qacc[j][cbk]);
            qacc[j][cbk] = mfma_bf16(rah[j][kb], qk[cbk], qacc[j][cbk]);
          }
      }
      // qacc[j][cbk][r] = q~[column block (CB cbk + c), column l16][channel 16 (wave + NWV j) + 4 quad + r]
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int cbk = 0; cbk < NCW; ++cbk)
          *reinterpret_cast<f32x4*>(fbuf + (16 * cbk + l16) * D + 16 * (wave + NWV * j) + 4 * quad) = qacc[j][cbk] * qscale;
      lds_barrier();
      if (MODE == 0 || wave < NCW) {  // the waves that own columns
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const float* src = fbuf + (16 * wave + l16) * D + 32 * kb + 8 * quad;
          bq[c][kb] = u32x4{f16pair(src[0], src[1]), f16pair(src[2], src[3]), f16pair(src[4], src[5]), f16pair(src[6], src[7])};
        }
      }
      lds_barrier();  // fbuf and the tiles are reused
    }
  } else {
    load_raw_q();
  }

  float m_run[CB], l_part[CB];
  f32x4 acc[CB][NCB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    m_run[c] = kNegInfA;
    l_part[c] = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[c][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool rotated = has_q;  // the accumulators hold rotated-basis value sums

  // products and online softmax of one step over the tile.  full: a
  // quantized step whose 32 tokens all lie in the middle region (no
  // per-token masks; columns past the unit's last carry finite values that
  // are never written)
  auto compute = [&](const uint16_t* tile, const StepInfo& si, const bool full) __attribute__((always_inline)) {
    if (!wave_cols) return;  // a wave without columns only decodes steps
    const bool quantized = si.kind == 1;
    f32x4 sc[CB][2];
#pragma unroll
    for (int c = 0; c < CB; ++c) sc[c][0] = sc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(tile + (16 * j + l16) * T::KROW + 32 * kb + 8 * quad);
#pragma unroll
        for (int c = 0; c < CB; ++c)
          sc[c][j] = quantized ? mfma_f16(a, bq[c][kb], sc[c][j]) : mfma_bf16(a, bq[c][kb], sc[c][j]);
      }
    // logits of tokens 16 j + 4 quad + r for column l16 of block c (log2 units), masked
    u32x4 bph[CB], bpl[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      float lg[2][4];
      float mx = kNegInfA;
      if (full) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lg[j][r] = sc[c][j][r];
            mx = fmaxf(mx, lg[j][r]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tk = 16 * j + 4 * quad + r;
            bool ok = col_ok[c];
            if (si.kind == 0) {
              const int li = si.i0 + j;
              ok = ok && li < rg.n_raw && raw_token(rg, 16 * rg.raw_page(li) + (tk & 15));
            } else if (quantized) {
              const int pg = rg.q0 + si.i0 + j, pos = 16 * pg + (tk & 15);
              ok = ok && pg < rg.q1 && pos >= rg.m0 && pos < rg.m1;
            } else {
              const int i = si.i0 + tk;  // new row index
              ok = ok && i < n_rows && P + i <= qpos[c];
            }
            lg[j][r] = ok ? (quantized ? sc[c][j][r] : sc[c][j][r] * qscale) : kNegInfA;
            mx = fmaxf(mx, lg[j][r]);
          }
      }
      mx = wave_max16(mx);
      // lazy rescale: the reference max moves only when a logit exceeds it by
      // more than kSlackA (probabilities stay <= 2^kSlackA, exact enough in f16)
      if (__any(mx > m_run[c] + kSlackA)) {
        const float m_new = fmaxf(m_run[c], mx);
        const float f = (m_run[c] == kNegInfA) ? 0.f : exp2f(m_run[c] - m_new);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[c][cb] *= f;
        l_part[c] *= f;
        m_run[c] = m_new;
      }
      const float m_use = (m_run[c] == kNegInfA) ? 0.f : m_run[c];
      float pv[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[j][r] = __builtin_amdgcn_exp2f(lg[j][r] - m_use);
          l_part[c] += pv[j][r];
        }
      if (quantized) {
        bph[c] = u32x4{f16pair(pv[0][0], pv[0][1]), f16pair(pv[0][2], pv[0][3]), f16pair(pv[1][0], pv[1][1]),
                       f16pair(pv[1][2], pv[1][3])};
      } else {
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split2x2(pv[i >> 1][2 * (i & 1)], pv[i >> 1][2 * (i & 1) + 1], ph[i], pl[i]);
        bph[c] = u32x4{ph[0], ph[1], ph[2], ph[3]};
        bpl[c] = u32x4{pl[0], pl[1], pl[2], pl[3]};
      }
    }
    // values: A = V^T rows (channel 16 cb + l16), K-slot 4 j + r = token 16 j + 4 quad + r
    const uint16_t* vt = tile + 32 * T::KROW;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const uint16_t* vr = vt + (16 * cb + l16) * T::VROW + 4 * quad;
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(vr), a1 = *reinterpret_cast<const u32x2*>(vr + 16);
      const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        if (quantized) {
          acc[c][cb] = mfma_f16(a, bph[c], acc[c][cb]);
        } else {
          acc[c][cb] = mfma_bf16(a, bpl[c], acc[c][cb]);
          acc[c][cb] = mfma_bf16(a, bph[c], acc[c][cb]);
        }
      }
    }
  };
  // rotated-basis value sums of block c -> model basis: acc^T[ch][n] = sum_k R_V[ch][k] rot[n][k]
  // (R_V rows and rot split into bf16 hi + lo, three products per block)
  float* wstage = fbuf + wave * 16 * D;
  const float* rvh = p.r_v + size_t(h) * D * D;
  auto rotate_back = [&]() {
    rotated = false;
    if (!wave_cols) return;
#pragma unroll
    for (int c = 0; c < CB; ++c) {  // unrolled: acc[c] needs a constant index
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) *reinterpret_cast<f32x4*>(wstage + l16 * D + 16 * cb + 4 * quad) = acc[c][cb];
      // the other lanes of the wave read these values: no LDS access may move
      // across this point, and the writes complete first
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const f32x4 ra0 = *reinterpret_cast<const f32x4*>(rvh + size_t(16 * cb + l16) * D + 32 * kb + 8 * quad);
          const f32x4 ra1 = *reinterpret_cast<const f32x4*>(rvh + size_t(16 * cb + l16) * D + 32 * kb + 8 * quad + 4);
          const float* rb = wstage + l16 * D + 32 * kb + 8 * quad;
          const float rav[8] = {ra0[0], ra0[1], ra0[2], ra0[3], ra1[0], ra1[1], ra1[2], ra1[3]};
          uint32_t ah[4], al[4], bh[4], bl[4];
#pragma unroll
          // scalar splits here: with the packed conversion the register
          // allocator spills the extend kernel (measured 5x slower)
          for (int i = 0; i < 4; ++i) {
            ah[i] = pack2(bf16_rne(rav[2 * i]), bf16_rne(rav[2 * i + 1]));
            al[i] = pack2(bf16_rne(rav[2 * i] - bf16_to_f32(ah[i] & 0xFFFFu)), bf16_rne(rav[2 * i + 1] - bf16_to_f32(ah[i] >> 16)));
            bh[i] = pack2(bf16_rne(rb[2 * i]), bf16_rne(rb[2 * i + 1]));
            bl[i] = pack2(bf16_rne(rb[2 * i] - bf16_to_f32(bh[i] & 0xFFFFu)), bf16_rne(rb[2 * i + 1] - bf16_to_f32(bh[i] >> 16)));
          }
          const u32x4 AH{ah[0], ah[1], ah[2], ah[3]}, AL{al[0], al[1], al[2], al[3]};
          const u32x4 BH{bh[0], bh[1], bh[2], bh[3]}, BL{bl[0], bl[1], bl[2], bl[3]};
          a4 = mfma_bf16(AL, BH, a4);
          a4 = mfma_bf16(AH, BL, a4);
          a4 = mfma_bf16(AH, BH, a4);
        }
        acc[c][cb] = a4;
      }
      // the next block's values overwrite the staging area only after every
      // lane has read this block's
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);
      asm volatile("" ::: "memory");
    }
  };
  auto tile_of = [&](int s) { return tiles + (NBUF == 2 ? (s & 1) : 0) * T::ELEMS; };

  // quantized steps: the loads of the next DEPTH steps stay in flight (every
  // step reloads its stage right after decoding it)
#pragma unroll 1
  for (int s = qa; s < qb; s += DEPTH) {
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      if (s + k < qb) {
        const StepInfo si = qinfo(s + k);
        uint16_t* tile = tile_of(s + k);
        step_store<D, BITS, NTH>(p, rg, bth, h, row0, n_rows, si, stq[k], tile, tid);
        step_load<D, BITS, NTH>(p, rg, btq, bth, h, row0, n_rows, qinfo(s + k + DEPTH), stq[k], tid);
        lds_barrier();  // the tile is complete; the loads just issued stay in flight
        const int pg0 = rg.q0 + si.i0;
        const bool full = pg0 + 1 < rg.q1 && 16 * pg0 >= rg.m0 && 16 * (pg0 + 2) <= rg.m1;
        compute(tile, si, full);
        if (NBUF == 1) lds_barrier();
      }
    }
  }
  // raw steps (BF16 pages, new rows): few per unit, loaded when stored
  if (ra < s_end && rotated) {
    rotate_back();
    load_raw_q();
  }
#pragma unroll 1
  for (int s = ra; s < s_end; ++s) {
    StepInfo si;
    if (s < n_qp + n_rp) {
      si.kind = 0;
      si.i0 = 2 * (s - n_qp);
    } else {
      si.kind = 2;
      si.i0 = 32 * (s - n_qp - n_rp);
    }
    uint16_t* tile = tile_of(s);
    step_store<D, BITS, NTH>(p, rg, bth, h, row0, n_rows, si, stq[0], tile, tid);
    lds_barrier();
    compute(tile, si, false);
    if (NBUF == 1) lds_barrier();
  }

  constexpr int RF = 4 + 2 * D;
  if (p.n_chunks > 1) {
    // record of this chunk: [m][l][2 unused][raw D][rot D] per column (the
    // value sums 16-byte aligned), the sums in the
    // field of their basis and zeros in the other (columns past the unit's
    // last are never merged: no record)
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const float l_tot = wave_sum16(l_part[c]);
      if (!col_ok[c]) continue;
      float* rec = p.rec + (((size_t(unit) * p.n_ct + ct) * p.n_chunks + chunk) * size_t(NC) + 16 * (CB * wave + c) + l16) * RF;
      if (quad == 0) {
        rec[0] = m_run[c];
        rec[1] = l_tot;
      }
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        *reinterpret_cast<f32x4*>(rec + 4 + 16 * cb + 4 * quad) = rotated ? zero : acc[c][cb];
        *reinterpret_cast<f32x4*>(rec + 4 + D + 16 * cb + 4 * quad) = rotated ? acc[c][cb] : zero;
      }
    }
    return;
  }
  // ---- single chunk: out = model-basis sums / l ----
  if (rotated) rotate_back();
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const float l_tot = wave_sum16(l_part[c]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (!col_ok[c]) continue;
    uint16_t* orow = p.out + (size_t(row0 + ri[c]) * p.Hq + h * G + hi[c]) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      u32x2 ov;
      ov[0] = bf16x2_rne(acc[c][cb][0] * inv, acc[c][cb][1] * inv);
      ov[1] = bf16x2_rne(acc[c][cb][2] * inv, acc[c][cb][3] * inv);
      *reinterpret_cast<u32x2*>(orow + 16 * cb + 4 * quad) = ov;
    }
  }
}

// Log-sum-exp merge of the chunk records of one column, then the output
// rotation: M = max_k m_k, w_k = 2^(m_k - M),
// out = (sum_k w_k raw_k + (sum_k w_k rot_k) R_V^T) / sum_k w_k l_k.
// One workgroup per (unit, column tile, column).  The chunk maxima and sums
// are requested first, then its R_V entries (output channel c = tid / TPC, a
// KPT-long run of k) and the first LB records' values of each wave, which
// arrive while the maxima and sums are reduced; the four waves take every fourth chunk (a lane holds
// FPL of the 2d value sums, LB chunks' loads in flight) and meet in LDS.
// LB = 32 for the decode (about 3 CUs of chunks per column: one batch per
// wave), 16 for extend (many more merge workgroups, fewer registers).
template <int D, int NC, int MODE>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttParams p) {
  constexpr int RF = 4 + 2 * D, NWM = 4, FPL = 2 * D / 64;  // waves, value floats per lane
  constexpr int TPC = 256 / D, KPT = D / TPC;                // threads per output channel, R_V entries each
  static_assert(FPL == 4 || FPL == 2, "d = 64 or 128");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int nk = p.n_chunks;
  float* s_w = reinterpret_cast<float*>(lds);  // [n_chunks] weights
  float* s_part = s_w + nk;                     // [NWM][2 D] per-wave value sums
  float* s_v = s_part + NWM * 2 * D;            // [2 D] merged raw, rot
  float* s_red = s_v + 2 * D;                   // [2 NWM] per-wave max, sum
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = blockIdx.y, ct = blockIdx.x % p.n_ct, unit = blockIdx.x / p.n_ct;
  const UnitRows u = unit_rows<MODE>(p, unit);
  if (MODE == 1 && u.P <= 0) return;
  const int G = p.G, col = ct * NC + cl;
  if (col >= u.n_rows * G) return;
  const int ri = col / G, hi = col % G;
  const size_t cstride = size_t(NC) * RF;
  const float* rec0 = p.rec + ((size_t(unit) * p.n_ct + ct) * nk * NC + cl) * RF;
  // maxima and sums first: thread k holds chunk k's (first 256 chunks); the
  // loads below are requested behind them, so the reduction waits only for
  // these two (load counters retire in order)
  float m0 = kNegInfA, l0 = 0.f;
  if (tid < nk) {
    m0 = rec0[tid * cstride];
    l0 = rec0[tid * cstride + 1];
  }
  const int c = tid / TPC, k0 = KPT * (tid % TPC);
  const float* rrow = p.r_v + size_t(u.h) * D * D + size_t(c) * D + k0;
  f32x4 rr[KPT / 4];
#pragma unroll
  for (int i = 0; i < KPT / 4; ++i) rr[i] = *reinterpret_cast<const f32x4*>(rrow + 4 * i);
  // this wave's chunks k = wave + NWM t, t < nt, LB at a time (indices
  // clamped into the records; the first LB requested before the weights,
  // which they do not need)
  constexpr int LB = MODE == 1 ? 32 : 16;
  const float* vb = rec0 + 4 + FPL * lane;
  const int nt = (nk - wave + NWM - 1) / NWM;
  float v[LB][FPL];
  auto load_batch = [&](int t0) {
#pragma unroll
    for (int t = 0; t < LB; ++t) {
      const int kk = min(wave + NWM * (t0 + t), nk - 1);
      if constexpr (FPL == 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(vb + kk * cstride);
#pragma unroll
        for (int f = 0; f < 4; ++f) v[t][f] = x[f];
      } else {
        const f32x2 x = *reinterpret_cast<const f32x2*>(vb + kk * cstride);
        v[t][0] = x[0];
        v[t][1] = x[1];
      }
    }
  };
  load_batch(0);
  float mx = m0;
  for (int k = tid + 256; k < nk; k += 256) mx = fmaxf(mx, rec0[k * cstride]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float l = 0.f;
  if (tid < nk) {
    const float w = m0 == kNegInfA ? 0.f : exp2f(m0 - mx);
    s_w[tid] = w;
    l = w * l0;
  }
  for (int k = tid + 256; k < nk; k += 256) {
    const float mk = rec0[k * cstride];
    const float w = mk == kNegInfA ? 0.f : exp2f(mk - mx);
    s_w[k] = w;
    l = __builtin_fmaf(w, rec0[k * cstride + 1], l);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  if (lane == 0) s_red[NWM + wave] = l;
  __syncthreads();  // the weights and the sums are visible to every wave
  l = (s_red[NWM] + s_red[NWM + 1]) + (s_red[NWM + 2] + s_red[NWM + 3]);
  float a[FPL];
#pragma unroll
  for (int f = 0; f < FPL; ++f) a[f] = 0.f;
  for (int t0 = 0; t0 < nt; t0 += LB) {
    if (t0 > 0) load_batch(t0);
#pragma unroll
    for (int t = 0; t < LB; ++t)
      if (t0 + t < nt)
#pragma unroll
        for (int f = 0; f < FPL; ++f) a[f] = __builtin_fmaf(s_w[wave + NWM * (t0 + t)], v[t][f], a[f]);
  }
#pragma unroll
  for (int f = 0; f < FPL; ++f) s_part[wave * 2 * D + FPL * lane + f] = a[f];
  __syncthreads();
  for (int j = tid; j < 2 * D; j += 256)
    s_v[j] = (s_part[j] + s_part[2 * D + j]) + (s_part[4 * D + j] + s_part[6 * D + j]);
  __syncthreads();
  // out[c] = (raw[c] + sum_k rot[k] R_V[c][k]) / L: each thread a KPT-long
  // run of k, the TPC runs of a channel summed over neighbouring lanes
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < KPT / 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) o = __builtin_fmaf(s_v[D + k0 + 4 * i + e], rr[i][e], o);
#pragma unroll
  for (int m = 1; m < TPC; m <<= 1) o += __shfl_xor(o, m, 64);
  if (tid % TPC == 0)
    p.out[(size_t(u.row0 + ri) * p.Hq + u.h * G + hi) * D + c] = uint16_t(bf16_rne(l > 0.f ? (s_v[c] + o) / l : 0.f));
}

}  // namespace

namespace oscar_launch {

// Waves per workgroup and 16-column blocks per wave: extend at d = 128 takes 8
// waves of 2 blocks (256 query columns), at d = 64 4 waves (the query
// rotation's d/16 = 4 channel blocks are split over the waves) of 2 blocks;
// the decode 4 waves that share each step's decoding, one of them holding
// the 16 columns.
int attend_waves(bool extend, int d) { return extend ? (d == 128 ? 8 : 4) : 4; }
int attend_cols(bool extend, int d) { return extend ? 16 * attend_waves(extend, d) * 2 : 16; }

size_t attend_lds_bytes(int d, bool extend) {
  const int nwv = attend_waves(extend, d), nbuf = nwv > 1 ? 2 : 1;
  const int ncw = extend ? nwv : 1;  // waves that own columns (per-wave staging)
  const size_t elems = d == 128 ? Tile<128>::ELEMS : Tile<64>::ELEMS;
  return size_t(nbuf) * elems * 2 + size_t(ncw) * 16 * d * 4;
}



hipError_t paged_attend(int d, int bits, bool extend, const void* qpool, int n_qpages, const void* bf16_pool,
                        int n_bpages, int n_kv, int G, int S, int W, int Hq, const void* q, const void* k_new,
                        const void* v_new, const int32_t* cu, const int32_t* clen, int batch, const int32_t* bt_q,
                        const int32_t* bt_h, int max_pages, const float* r_k, const float* r_v, float sm_scale,
                        int n_ct, int n_chunks, int spc, float* rec, void* out, hipStream_t stream) {
  AttParams p{static_cast<const uint8_t*>(qpool), std::max(1, n_qpages), static_cast<const uint16_t*>(bf16_pool),
              std::max(1, n_bpages), n_kv, G, S, W, Hq, static_cast<const uint16_t*>(q),
              static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), cu, clen, bt_q, bt_h,
              max_pages, r_k, r_v, sm_scale, n_ct, n_chunks, spc, rec, static_cast<uint16_t*>(out)};
  const unsigned units = unsigned(batch) * unsigned(n_kv);
  const dim3 grid(units * unsigned(n_ct) * unsigned(n_chunks));
  const int ncols = extend ? attend_cols(true, d) : std::min(G, 16);  // merge workgroups per column tile
  const dim3 mgrid(units * unsigned(n_ct), unsigned(ncols));
  const size_t lds = attend_lds_bytes(d, extend);
  const size_t mlds = (size_t(n_chunks) + 10 * size_t(d) + 8) * 4;
#define OSCAR_ATTEND(DD, BB, NW, MM)                                                                        \
  do {                                                                                                      \
    constexpr int CB_ = MM == 0 ? 2 : 1;                                                                    \
    hipLaunchKernelGGL((attend_kernel<DD, BB, NW, CB_, MM>), grid, dim3(64 * NW), lds, stream, p);          \
    if (n_chunks > 1)                                                                                       \
      hipLaunchKernelGGL((attend_merge_kernel<DD, MM == 0 ? 16 * NW * CB_ : 16, MM>), mgrid, dim3(256), mlds, stream, p); \
  } while (0)
  if (d == 128) {
    if (extend) { if (bits == 2) OSCAR_ATTEND(128, 2, 8, 0); else OSCAR_ATTEND(128, 4, 8, 0); }
    else { if (bits == 2) OSCAR_ATTEND(128, 2, 4, 1); else OSCAR_ATTEND(128, 4, 4, 1); }
  } else {
    if (extend) { if (bits == 2) OSCAR_ATTEND(64, 2, 4, 0); else OSCAR_ATTEND(64, 4, 4, 0); }
    else { if (bits == 2) OSCAR_ATTEND(64, 2, 4, 1); else OSCAR_ATTEND(64, 4, 4, 1); }
  }
#undef OSCAR_ATTEND
  return hipGetLastError();
}

}  // namespace oscar_launch
