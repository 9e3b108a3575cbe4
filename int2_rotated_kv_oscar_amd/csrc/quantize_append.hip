// Kernel A — quantize-append: rotate new K/V rows by the fixed rotation,
// clip, quantize per token in 32-channel groups to asymmetric INT2 and pack
// the codes into INT2 pages ([TS] 2.2.B online serving: the middle history is
// stored in INT2 after the fixed OSCAR rotation and clipping; [TS] 2.2.A
// step 4 for the per-layer clip).
//
// A workgroup takes one (KV head, tensor) and loops over tiles of 16 rows,
// one wave per 32-channel group (so group statistics stay inside a wave).  The
// rotation y = x . R is a dense 16 x d x d product per tile and runs on the
// 16x16x32 f16 MFMA: x is converted exactly from bf16 to f16, 256 R (float32)
// is split into f16 hi + lo parts (22 significant bits), so y is accurate to
// about 2^-22 relative.  Tiles use the transposed product y^T = R^T x^T,
// whose output lane layout (one row per lane, 4 consecutive channels per
// 16-channel block) keeps a 32-channel group inside one wave over its 4 lane
// quads: group min/max take three lane swaps.  Each wave's code bits go to
// LDS and are OR-combined into the page's words when stored; a tile that is
// one whole page is written with plain coalesced stores, scattered rows with
// per-field atomic updates.
#include <algorithm>

#include "device_utils.h"
#include "layout.h"
#include "kernels.h"

using namespace oscar_dev;

namespace {

struct QAParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t n_rows;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const int32_t* bt_q;
  int32_t max_pages;
  const float* r_k;
  const float* r_v;
  float tau_k, tau_v;
  uint8_t* pool;
  int32_t n_kv;
  // decode-step update only: lengths, BF16 tables and pool, regions
  const int32_t* seq_lens;
  const int32_t* bt_h;
  uint16_t* bf16_pool;
  int32_t n_sink, n_recent;
};

// Per-tile row metadata: lane l16 describes row tile*16 + l16 (all quads hold
// the same).
struct TileMeta {
  int32_t page, slot;
  bool valid;    // the row exists (page is meaningful only then)
  bool aligned;  // 16 consecutive positions of one sequence starting on a page boundary
};

// Codes through the float adder: t + 1.5 * 2^23 rounds t = (v - z) / s to
// the nearest integer (ties to even) in the low mantissa bits, so the clamp
// to [0, 3] is an integer med3 on the bit pattern (monotone for every finite
// value, negative ones included) and the packing adds the pattern shifted into
// place; the shifted copies of the constant part are removed by starting each
// word from minus their sum (all modulo 2^32).  The quotient is t0 = (v - z)
// inv refined once with its exact residual, t = t0 + (v - z - t0 s) inv,
// which is the exact quotient whenever that is a representable number: an
// exact midpoint k + 1/2 (frequent when the rotated values are themselves
// coarse, as without rotation) then rounds to even instead of to the side
// the reciprocal's error happens to fall on.  s = 0 gives inv = 0 and code 0.
constexpr float kMagic = 12582912.0f;
constexpr uint32_t kMagicBits = 0x4B400000u;
template <int TOP = 3>
__device__ __forceinline__ uint32_t code_bits(float v, float z, float inv, float s) {
  const float d = v - z;
  const float t0 = d * inv;
  const float t = __builtin_fmaf(__builtin_fmaf(-t0, s, d), inv, t0);
  const int b = __float_as_int(t + kMagic);
  return uint32_t(min(max(b, int(kMagicBits)), int(kMagicBits + uint32_t(TOP))));
}

// Reduction over the four lanes l16 + 16q of a row: the minimum of mn and the
// maximum of mx, both computed in every lane with three lane swaps (the lower
// half of the wave carries the minima, the upper half the negated maxima).
__device__ __forceinline__ void row_min_max(float& mn, float& mx) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(-mx), false, false);
  const float c = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(c), __float_as_uint(c), false, false);
  const float e = fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  auto f = __builtin_amdgcn_permlane32_swap(__float_as_uint(e), __float_as_uint(e), false, false);
  mn = __uint_as_float(f[0]);
  mx = -__uint_as_float(f[1]);
}

// LDS of a workgroup (shared by the K and V instances of the tile loop).
template <int D, bool ONE>
struct QAShared {
  static constexpr int NG = D / 32;
  // tiles in flight per workgroup: x and page ids of kX tiles, positions of kS
  static constexpr int kX = ONE ? 1 : 4, kS = ONE ? 1 : 8;
  static constexpr int kRowBytes = 2 * D + 16;  // padded LDS row of the x tile (conflict-free operand reads)
  // Rings filled by global_load_lds (no registers hold requests in flight):
  // wave g's quarter of the raw bf16 x tile (rows 4g .. 4g+3 for d = 128,
  // 1 KB), its copy of the tile's row_seq (lanes 0-15) and row_pos (lanes
  // 16-31) and of the rows' page ids (lanes 0-15).  Each wave reads only what
  // it requested itself.
  __attribute__((aligned(16))) uint8_t raw[kX][NG][1024];
  int32_t sp[kS][NG][64];
  int32_t pg[kX][NG][64];
  // x tiles in f16, each wave's code bits of a tile (by word lane) and its
  // f16 scales/zeros in page-area order; double-buffered
  __attribute__((aligned(16))) uint8_t x[2][16 * kRowBytes];
  uint32_t part[2][NG][64];
  uint32_t sz[2][16 * NG];  // [scale area | zero area] as u32 pairs of f16
  int32_t rexp[2][16];      // per-row power-of-two prescale of the x tile
};

// ONE: every workgroup has exactly one tile (a decode step's appends).
// BITS: 2 (the INT2 cache, MFMA-shaped code words) or 4 (the INT4 variant,
// row-owned nibbles: each wave stores its group's codes of a row directly).
template <int D, int TENSOR, bool ONE, int BITS>
__device__ void qa_tiles(const QAParams& p, int h, QAShared<D, ONE>& sh) {
  using GG = Geo<D>;
  using QL = QLayout<D, BITS>;
  constexpr int TOP = (1 << BITS) - 1;
  constexpr int NG = GG::NG, NKB = GG::NKB, NW = GG::NW;
  constexpr int kX = QAShared<D, ONE>::kX, kS = QAShared<D, ONE>::kS;
  constexpr int kRowBytes = QAShared<D, ONE>::kRowBytes;
  constexpr float kRScale = 256.0f;
  auto& s_raw = sh.raw;
  auto& s_sp = sh.sp;
  auto& s_pg = sh.pg;
  auto& s_x = sh.x;
  auto& s_part = sh.part;
  auto& s_sz = sh.sz;
  auto& s_rexp = sh.rexp;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* X = TENSOR ? p.v_new : p.k_new;
  const float* R = (TENSOR ? p.r_v : p.r_k) + size_t(h) * D * D;
  const float tau = TENSOR ? p.tau_v : p.tau_k;
  const int64_t n_tiles = (p.n_rows + 15) / 16;
  const int64_t n_mine = (n_tiles - blockIdx.x + gridDim.x - 1) / gridDim.x;  // >= 1 by the grid size

  // The i-th tile of this workgroup (clamped: past the end repeats the last).
  auto tile_of = [&](int64_t i) { return int64_t(blockIdx.x) + (i < n_mine ? i : n_mine - 1) * int64_t(gridDim.x); };
  // rows of tile t (1 .. 16)
  auto rows_of = [&](int64_t t) { const int64_t rem = p.n_rows - t * 16; return rem < 16 ? int(rem) : 16; };
  // Requests of the ring: lane l of wave g loads 16 B of row 4g + l/16 (for
  // d = 128) of the tile; rows past n_rows re-read the last row, tiles past
  // the workgroup's last re-read that tile (their results are never stored).
  constexpr int kQuarterRows = 16 / NG;        // rows of a tile per wave
  constexpr int kChunks = 2 * D / 16;          // 16-byte chunks per row
  static_assert(kQuarterRows * kChunks == 64, "one 16-byte chunk per lane");
  const int xrow = kQuarterRows * g + lane / kChunks;
  const uint32_t xcol = 8u * uint32_t(lane % kChunks);
  const uint32_t row_elems = uint32_t(p.n_kv) * D;
  auto issue_x = [&](int64_t i) {  // x quarter of tile i
    const int64_t t = tile_of(i);
    const uint16_t* xb = X + (t * 16 * p.n_kv + h) * D;
    __builtin_amdgcn_global_load_lds(xb + (uint32_t(min(xrow, rows_of(t) - 1)) * row_elems + xcol),
                                     &s_raw[i % kX][g][0], 16, 0, 0);
  };
  auto issue_sp = [&](int64_t i) {  // positions of tile i
    const int64_t t = tile_of(i);
    const int32_t* sp = ((lane & 16) ? p.row_pos : p.row_seq) + t * 16;
    __builtin_amdgcn_global_load_lds(sp + min(lane & 15, rows_of(t) - 1), &s_sp[i % kS][g][0], 4, 0, 0);
  };
  auto issue_pages = [&](int64_t i) {  // page ids of tile i's rows (its positions have landed)
    const int32_t seq = s_sp[i % kS][g][l16], pos = s_sp[i % kS][g][16 + l16];
    __builtin_amdgcn_global_load_lds(p.bt_q + (int64_t(seq) * p.max_pages + (pos >> 4)), &s_pg[i % kX][g][0], 4, 0, 0);
  };
  // positions first: the page ids need them
#pragma unroll
  for (int u = 0; u < kS; ++u) issue_sp(u);
  wait_vm<0>();
#pragma unroll
  for (int u = 0; u < kX; ++u) {
    issue_pages(u);
    issue_x(u);
  }

  // R operands of this group, split once: 256 R (a power of two keeps the
  // low parts out of the f16 subnormal range) as f16 hi + lo, 22 significant
  // bits; lane (c16 = l16, quad) holds R[32kb + 8quad + i][16cb + l16], cb = 2g + hb
  u32x4 rop[2][NKB][2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float rv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[i] = kRScale * R[size_t(32 * kb + 8 * quad + i) * D + 16 * (2 * g + hb) + l16];
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t h0 = f16_bits(rv[i]), h1 = f16_bits(rv[i + 1]);
        ph[i / 2] = pack2(h0, h1);
        pl[i / 2] = pack2(f16_bits(rv[i] - f16_to_f32(h0)), f16_bits(rv[i + 1] - f16_to_f32(h1)));
      }
      rop[hb][kb][0] = u32x4{ph[0], ph[1], ph[2], ph[3]};
      rop[hb][kb][1] = u32x4{pl[0], pl[1], pl[2], pl[3]};
    }

  // Where this lane's code bits go.  K: word (quad*16 + m)*NW + g/2 of row
  // m = l16 is lane `lane`'s, its fields at 16(r%2) + 8(g%2) + 4hb + 2(r/2).
  // V: after combining the four rows of a word across the lane quartet, lane
  // m writes word ((m/4)*16 + 4quad + m%4)*NW + g/2, its fields at
  // sh + 2((2g + hb)%4) with sh = 16(m%2) + 8((m/2)%2).
  const int pidx = TENSOR == 0 ? lane : ((l16 >> 2) * 16 + 4 * quad + (l16 & 3));
  const uint32_t vsh = 16u * (l16 & 1) + 8u * ((l16 >> 1) & 1);
  const uint32_t vsh0 = vsh + 2u * ((2 * g) & 3), vsh1 = vsh + 2u * ((2 * g + 1) & 3);
  uint32_t word0;  // minus the sum of the shifted constant parts of one word's fields
  if (TENSOR == 0) {
    uint32_t c = 0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) c += kMagicBits << (16 * (r & 1) + 8 * (g & 1) + 4 * hb + 2 * (r >> 1));
    word0 = 0u - c;
  } else {
    word0 = 0u - ((kMagicBits << vsh0) + (kMagicBits << vsh1));
  }

  // f16 index of the scale/zero of (slot m, group gg) inside its area: K
  // (and every INT4 area) [16][NG], INT2 V in token-quad order [4][NG][4]
  auto sz_index = [](int m, int gg) {
    return (TENSOR == 0 || BITS == 4) ? m * NG + gg : ((m >> 2) * NG + gg) * 4 + (m & 3);
  };
  // stores of a finished tile: wave 0 the INT2 codes, wave 1 the scales/zeros
  auto store_tile = [&](const TileMeta& mc, int buf) {
    if (g > 1) return;
    if (g == 1) {
      if (mc.aligned) {
        // scale and zero areas of the page are contiguous: 2 x 32 NG bytes
        const int page0 = __builtin_amdgcn_readfirstlane(mc.page);
        uint8_t* base = p.pool + (int64_t(page0) * p.n_kv + h) * int64_t(QL::HEAD_BYTES);
        uint32_t* dst = reinterpret_cast<uint32_t*>(base + (TENSOR == 0 ? QL::KS : QL::VS));
        if (lane < 16 * NG) dst[lane] = s_sz[buf][lane];
      } else {
        // lane j: row m = j / NG, group gg = j % NG, to that row's page and slot
        const int m = min(lane / NG, 15), gg = lane % NG;
        const int page = __shfl(mc.page, m, 64), slot = __shfl(mc.slot, m, 64);
        const bool valid = __shfl(int(mc.valid), m, 64) != 0;
        if (lane < 16 * NG && valid) {
          const uint16_t* sz16 = reinterpret_cast<const uint16_t*>(s_sz[buf]);
          const int ia = sz_index(m, gg), iu = sz_index(slot, gg);
          uint8_t* base = p.pool + (int64_t(page) * p.n_kv + h) * int64_t(QL::HEAD_BYTES);
          reinterpret_cast<uint16_t*>(base + (TENSOR == 0 ? QL::KS : QL::VS))[iu] = sz16[ia];
          reinterpret_cast<uint16_t*>(base + (TENSOR == 0 ? QL::KZ : QL::VZ))[iu] = sz16[16 * NG + ia];
        }
      }
      return;
    }
    if (BITS == 4) return;  // INT4 codes were stored by their waves
    uint32_t wd[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) wd[w] = s_part[buf][2 * w][lane] | s_part[buf][2 * w + 1][lane];
    if (mc.aligned) {
      // 16 rows = slots 0..15 of one page: the words are the page's code words
      const int page0 = __builtin_amdgcn_readfirstlane(mc.page);
      uint8_t* base = p.pool + (int64_t(page0) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
      uint32_t* dst = reinterpret_cast<uint32_t*>(base + (TENSOR == 0 ? GG::KC : GG::VC)) + lane * NW;
#pragma unroll
      for (int w = 0; w < NW; ++w) dst[w] = wd[w];
    } else if (TENSOR == 0) {
      if (mc.valid) {  // K code words hold a single token: plain stores
        uint8_t* base = p.pool + (int64_t(mc.page) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
        uint32_t* kc = reinterpret_cast<uint32_t*>(base + GG::KC) + (quad * 16 + mc.slot) * NW;
#pragma unroll
        for (int w = 0; w < NW; ++w) kc[w] = wd[w];
      }
    } else {
      // rows of different pages/slots: replace this row's 2-bit fields with
      // an atomic and (clear) and an atomic or (set); other rows may update
      // other fields of the same word meanwhile
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vpage = __shfl(mc.valid ? mc.page : -1, 4 * quad + r, 64), vslot = __shfl(mc.slot, 4 * quad + r, 64);
        if (vpage < 0) continue;
        uint8_t* base = p.pool + (int64_t(vpage) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
        const int sh = 16 * (vslot & 1) + 8 * ((vslot >> 1) & 1);
        uint32_t* vc = reinterpret_cast<uint32_t*>(base + GG::VC) + ((vslot >> 2) * 16 + l16) * NW;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t bits = ((wd[w] >> (16 * (r & 1) + 8 * (r >> 1))) & 0xFFu) << sh;
          atomicAnd(vc + w, ~(0xFFu << sh));
          atomicOr(vc + w, bits);
        }
      }
    }
  };

  auto epilogue = [&](const f32x4 (&acc)[2], int rexp, int buf, const TileMeta& mc) {
    // ---- group g of row m = l16: acc[hb][r] = y / F for channel
    // 32g + 16hb + 4quad + r, F = 2^(e - 8) (R scale and row prescale); the
    // clip, the statistics and the codes run on acc with F folded in ----
    const float F = __builtin_ldexpf(1.0f, rexp - 8), iF = __builtin_ldexpf(1.0f, 8 - rexp);
    const float tc = tau * iF;
    float y[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[hb][r] = __builtin_amdgcn_fmed3f(acc[hb][r], -tc, tc);
    float mn = fminf(fminf(fminf(y[0][0], y[0][1]), y[0][2]), fminf(fminf(y[0][3], y[1][0]), y[1][1]));
    mn = fminf(mn, fminf(y[1][2], y[1][3]));
    float mx = fmaxf(fmaxf(fmaxf(y[0][0], y[0][1]), y[0][2]), fmaxf(fmaxf(y[0][3], y[1][0]), y[1][1]));
    mx = fmaxf(mx, fmaxf(y[1][2], y[1][3]));
    row_min_max(mn, mx);
    // s = (max - min) / 3 and z = min in true units (F is a power of two:
    // the scalings are exact), rounded to f16; codes against the f16 values
    const uint32_t s16 = f16_bits(div3<TOP>(mx - mn) * F);
    const uint32_t z16 = f16_bits(mn * F);
    const float sf = f16_to_f32(s16);
    const float inv = sf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sf);  // s16 = 0: every code is 0
    const float zr = f16_to_f32(z16) * iF;  // (y - z) / s = (acc - z/F) / (s/F)
    const float invr = inv * F, sr = sf * iF;
    const int m = l16;
    uint32_t bits = 0;
    if (BITS == 4) {
      // row m owns bytes [16 g, 16 g + 16) of its code row: channels
      // 32g + 16hb + 4quad + r as nibbles r of the 16-bit word at byte 16g + 8hb + 2quad
      if (mc.valid) {
        uint8_t* base = p.pool + (int64_t(mc.page) * p.n_kv + h) * int64_t(QL::HEAD_BYTES) +
                        (TENSOR == 0 ? QL::KC : QL::VC) + mc.slot * (D / 2) + 16 * g + 2 * quad;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          uint32_t w16 = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) w16 |= (code_bits<TOP>(y[hb][r], zr, invr, sr) - kMagicBits) << (4 * r);
          *reinterpret_cast<uint16_t*>(base + 8 * hb) = uint16_t(w16);
        }
      }
    } else if (TENSOR == 0) {
      bits = word0;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bits += code_bits(y[hb][r], zr, invr, sr) << (16 * (r & 1) + 8 * (g & 1) + 4 * hb + 2 * (r >> 1));
    } else {
      // the four rows m = 4j..4j+3 (consecutive lanes) share these words:
      // their fields are OR-combined across the lane quartet, then lane m
      // keeps word r = m%4, one writer per word and wave
      bits = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t wr = (code_bits(y[0][r], zr, invr, sr) << vsh0) + word0;
        wr += code_bits(y[1][r], zr, invr, sr) << vsh1;
        wr |= uint32_t(__builtin_amdgcn_mov_dpp(int(wr), 0xB1, 0xF, 0xF, false));  // lanes ^1
        wr |= uint32_t(__builtin_amdgcn_mov_dpp(int(wr), 0x4E, 0xF, 0xF, false));  // lanes ^2
        bits = (m & 3) == r ? wr : bits;
      }
    }
    if (BITS == 2) s_part[buf][g][pidx] = bits;
    if (quad == 0) {  // in the page-area order of an aligned tile (slot = m)
      const int ia = sz_index(m, g);
      uint16_t* sz16 = reinterpret_cast<uint16_t*>(s_sz[buf]);
      sz16[ia] = uint16_t(s16);
      sz16[16 * NG + ia] = uint16_t(z16);
    }
  };

  // bf16 -> f16 is exact for 2^-17 <= |x| < 2^15; smaller values are cut
  // to the 2^-24 grid.  Rows of ordinary magnitude (every value of a lane
  // below 2^15, and some value of every lane at least 2^-3) are converted as
  // they are: a cut value then errs by at most 2^-21 of the row's largest.
  // Otherwise every row of this wave's quarter is scaled by the power of two
  // 2^-e that brings its largest magnitude into [2^14, 2^15) (e recorded per
  // row and undone in the epilogue; e >= -118 keeps the epilogue's factors
  // finite), so small rows keep their precision as large ones do.
  auto stage_x = [&](const u32x4& v, int buf) {
    const int row = kQuarterRows * g + lane / kChunks;
    // largest bf16 magnitude of each half over the lane's 8 values
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 mm = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(us2, v[0] & 0x7FFF7FFFu), __builtin_bit_cast(us2, v[1] & 0x7FFF7FFFu)),
        __builtin_elementwise_max(__builtin_bit_cast(us2, v[2] & 0x7FFF7FFFu), __builtin_bit_cast(us2, v[3] & 0x7FFF7FFFu)));
    const uint32_t mb = __builtin_bit_cast(uint32_t, mm);
    const uint32_t lo = mb & 0xFFFFu, hi = mb >> 16;
    const bool big = lo >= (142u << 7) || hi >= (142u << 7);
    const bool small = lo < (124u << 7) && hi < (124u << 7);
    u32x4 o;
    int e = 0;
    if (__builtin_expect(__any(big || small), 0)) {
      // exponent of the row's largest value, over the row's kChunks lanes
      int ex = int(max(lo, hi) >> 7);
#pragma unroll
      for (int msk = 1; msk < kChunks; msk <<= 1) ex = max(ex, __shfl_xor(ex, msk, 64));
      e = max(-118, ex - 141);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = pack_f16x2_rtz(__builtin_ldexpf(bf16_to_f32(v[i] & 0xFFFFu), -e), __builtin_ldexpf(bf16_to_f32(v[i] >> 16), -e));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_f16x2_rtz(bf16_to_f32(v[i] & 0xFFFFu), bf16_to_f32(v[i] >> 16));
    }
    *reinterpret_cast<u32x4*>(&s_x[buf][row * kRowBytes + 16 * (lane % kChunks)]) = o;
    if (lane % kChunks == 0) s_rexp[buf][row] = e;
  };

  // tile i's rows: page, slot, alignment (a uniform decision)
  auto meta = [&](int64_t i) {
    TileMeta mc;
    const int rl = rows_of(tile_of(i));
    const int32_t seq = s_sp[i % kS][g][l16], pos = s_sp[i % kS][g][16 + l16];
    mc.valid = l16 < rl;
    mc.page = s_pg[i % kX][g][l16];
    mc.slot = pos & 15;
    const int32_t seq0 = __builtin_amdgcn_readfirstlane(seq), pos0 = __builtin_amdgcn_readfirstlane(pos);
    const bool ok = seq == seq0 && pos == pos0 + l16;
    mc.aligned = rl == 16 && (pos0 & 15) == 0 && (__ballot(ok) & 0xFFFFull) == 0xFFFFull;
    return mc;
  };

  wait_vm<0>();  // the first tiles' requests (R's plain loads drained them already)

  // One barrier per tile: step i stages tile i, stores tile i-1 (its words
  // completed before the barrier), then runs tile i's MFMAs and epilogue.
  // After its stores every step issues the same three requests: positions of
  // tile i+8, x and page ids of tile i+4 (from positions that landed four
  // steps before).  A step waits for the requests of four steps before (at
  // most nine requests younger), never for stores of the last three steps.
  // Steps past the last tile re-request the clamped last tile and only store.
  TileMeta mprev = {0, 0, false, false};
  for (int64_t i = 0; i < n_mine + 1; ++i) {
    const int buf = int(i & 1);
    if (!ONE) wait_vm<9>();
    stage_x(*reinterpret_cast<const u32x4*>(&s_raw[i % kX][g][16 * lane]), buf);
    const TileMeta mc = meta(i);
    lds_barrier_keep_dma();
    if (i >= 1) store_tile(mprev, buf ^ 1);
    if (!ONE) {
      asm volatile("" ::: "memory");  // this step's ring reads are done before the refills are requested
      issue_sp(i + kS);
      issue_x(i + kX);
      issue_pages(i + kX);
    }
    if (i < n_mine) {
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      u32x4 xc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        xc[kb] = *reinterpret_cast<const u32x4*>(&s_x[buf][l16 * kRowBytes + 64 * kb + 16 * quad]);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int j = 1; j >= 0; --j)  // lo, then hi
            acc[hb] = mfma_f16(rop[hb][kb][j], xc[kb], acc[hb]);
      epilogue(acc, s_rexp[buf][l16], buf, mc);
    }
    mprev = mc;
  }
  wait_vm<0>();  // no ring request lands after the workgroup ends
}

template <int D, bool ONE, int BITS>
__global__ __launch_bounds__(64 * (D / 32), 4) void quantize_append_kernel(QAParams p) {
  __shared__ QAShared<D, ONE> sh;
  const int h = blockIdx.y;
  if (blockIdx.z == 0)
    qa_tiles<D, 0, ONE, BITS>(p, h, sh);
  else
    qa_tiles<D, 1, ONE, BITS>(p, h, sh);
}

// ---------------------------------------------------------------------------
// Few rows (a decode step's appends): the rotation is a handful of d x d
// vector-matrix products, too small for the tile pipeline above, whose time
// goes to fetching and splitting all of R per workgroup.  Here a workgroup
// takes one (KV head, tensor), one pair of channel groups (64 rotated
// channels, a slice of R of d x 64 float32) and up to kRowsPerWg rows, and
// computes y in plain float32 fused multiply-adds.  A group pair owns whole
// code words of a K row and whole code bytes of a V row in the page layout,
// so every field is written with a plain store: no atomics, whatever other
// rows share the words.
//
// STEP (a decode step's cache update, one row per sequence): for sequence b
// of length L (the new token at position L - 1 included) the row entering the
// middle history is the token L - 1 - W leaving the recent window, read from
// its BF16 slot (with W = 0, the new token itself, from k_new/v_new), if it
// lies at or past the sink; and the new token is written to its BF16 slot
// when it is a sink or recent token.
constexpr int kRowsPerWg = 8;
constexpr int kRowThreads = 256;
constexpr int64_t kFewRows = 64;  // row counts up to this take the few-row kernel

template <int D, bool STEP, int BITS>
__global__ __launch_bounds__(kRowThreads) void quantize_rows_kernel(QAParams p) {
  using GG = Geo<D>;
  using QL = QLayout<D, BITS>;
  constexpr int TOP = (1 << BITS) - 1;
  constexpr int NG = GG::NG, NW = GG::NW;
  constexpr int KS_PER = D / 16;  // reduction length of one k-slice (16 slices)
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int tensor = blockIdx.z & 1, pair = blockIdx.z >> 1;
  const uint16_t* X = tensor ? p.v_new : p.k_new;
  const float* R = (tensor ? p.r_v : p.r_k) + size_t(h) * D * D;
  const float tau = tensor ? p.tau_v : p.tau_k;
  const int64_t row0 = int64_t(blockIdx.x) * kRowsPerWg;
  const int nr = int(min<int64_t>(kRowsPerWg, p.n_rows - row0));  // >= 1 by the grid size

  __shared__ float s_part[kRowsPerWg][16][64];  // [row][k-slice][channel of the pair]
  __shared__ uint16_t s_x[kRowsPerWg][D];
  __shared__ uint8_t s_code[kRowsPerWg][64];
  __shared__ int32_t s_page[kRowsPerWg], s_slot[kRowsPerWg];  // INT2 destination (-1: none)
  __shared__ int32_t s_valid[kRowsPerWg];                      // the row is quantized and stored
  __shared__ int32_t s_src[kRowsPerWg];                        // STEP: BF16 page of the row (-1: k_new/v_new)
  __shared__ int32_t s_new[kRowsPerWg], s_newslot[kRowsPerWg];  // STEP: BF16 slot of the new token (-1: none)
  __shared__ uint16_t s_sz[kRowsPerWg][2][2];                  // f16 scale, zero per (row, group of the pair)

  // Row metadata.  The INT2 page id (a dependent load from the block table)
  // is needed only by the stores: it stays in a register of thread `tid`
  // and goes to LDS just before them, so its round trip overlaps the
  // products, statistics and codes (the barriers below order LDS only).
  int32_t my_page = -1, my_slot = 0;
  if (!STEP) {
    // every thread loads (threads past the chunk: its last row), so that the
    // compiler's wait counts are the same on every path
    const int rq = min(tid, nr - 1);
    my_page = p.row_seq[row0 + rq];  // the sequence, until the page id is looked up below
    my_slot = p.row_pos[row0 + rq];  // the position, likewise
    if (tid < nr) s_valid[tid] = 1;
  } else if (tid < nr) {
    {
      const int64_t b = row0 + tid;
      const int32_t L = p.seq_lens[b];
      int32_t t = -1, src = -1, nw = -1;
      if (L >= 1) {
        if (p.n_recent >= 1 || L - 1 < p.n_sink) nw = p.bt_h[b * p.max_pages + ((L - 1) >> 4)];
        t = p.n_recent >= 1 ? L - 1 - p.n_recent : L - 1;
        if (t < p.n_sink) t = -1;
        else if (p.n_recent >= 1) src = p.bt_h[b * p.max_pages + (t >> 4)];
      }
      if (t >= 0) my_page = p.bt_q[b * p.max_pages + (t >> 4)];
      my_slot = t & 15;
      s_valid[tid] = t >= 0 ? 1 : 0;
      s_slot[tid] = my_slot;  // the BF16 gather reads the same slot
      s_src[tid] = src;
      s_new[tid] = nw;
      s_newslot[tid] = (L - 1) & 15;
    }
  }
  if (STEP) lds_barrier();
  // the chunk's x rows (rows past the chunk re-read its last row; their
  // results are never stored) and this thread's slice of R, loaded before the
  // page id so that waiting for them does not wait for it (loads complete in
  // order)
  constexpr int kXPer = kRowsPerWg * D / kRowThreads;
  uint16_t xv[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int e = tid * kXPer + i, r = e / D, c = e % D, rr = min(r, nr - 1);
    xv[i] = 0;
    if (!STEP) {
      xv[i] = X[((row0 + rr) * p.n_kv + h) * D + c];
    } else if (s_src[rr] >= 0) {  // K token-major, V channel-major in the BF16 page
      const uint16_t* hp = p.bf16_pool + (int64_t(s_src[rr]) * p.n_kv + h) * GG::BF16_HEAD_ELEMS;
      xv[i] = tensor == 0 ? hp[s_slot[rr] * D + c] : hp[16 * D + c * 16 + s_slot[rr]];
    } else if (s_valid[rr]) {
      xv[i] = X[((row0 + rr) * p.n_kv + h) * D + c];
    }
  }
  // products: thread (k-slice ks, channel quad c4) over the rows
  const int c4 = tid & 15, ks = tid >> 4;
  f32x4 rr[KS_PER];
#pragma unroll
  for (int j = 0; j < KS_PER; ++j)
    rr[j] = *reinterpret_cast<const f32x4*>(R + size_t(ks * KS_PER + j) * D + 64 * pair + 4 * c4);
  asm volatile("" ::: "memory");  // the page-id load stays behind the x and R loads
  if (!STEP) {
    const int32_t seq = my_page, pos = my_slot;
    my_page = p.bt_q[int64_t(seq) * p.max_pages + (pos >> 4)];
    my_slot = pos & 15;
  }
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int e = tid * kXPer + i;
    s_x[e / D][e % D] = xv[i];
  }
  lds_barrier();
#pragma unroll
  for (int r = 0; r < kRowsPerWg; ++r) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS_PER; ++j) {
      const float x = bf16_to_f32(s_x[r][ks * KS_PER + j]);
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = __builtin_fmaf(x, rr[j][c], a[c]);
    }
    *reinterpret_cast<f32x4*>(&s_part[r][ks][4 * c4]) = a;
  }
  lds_barrier();

  // statistics and codes: thread (row rw, channel cc) holds channel cc of the
  // pair's first group and channel cc of its second, a row's 32 lanes being
  // one half of a wave
  const int rw = tid >> 5, cc = tid & 31;
  float y[2] = {0.f, 0.f};
#pragma unroll
  for (int gp = 0; gp < 2; ++gp) {
#pragma unroll
    for (int k = 0; k < 16; ++k) y[gp] += s_part[rw][k][32 * gp + cc];
    y[gp] = __builtin_amdgcn_fmed3f(y[gp], -tau, tau);
  }
#pragma unroll
  for (int gp = 0; gp < 2; ++gp) {
    float mn = y[gp], mx = y[gp];
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, m, 64));
      mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    }
    const uint32_t s16 = f16_bits(div3<TOP>(mx - mn));
    const uint32_t z16 = f16_bits(mn);
    const float sf = f16_to_f32(s16), zf = f16_to_f32(z16);
    int code = 0;
    if (sf != 0.0f) code = min(max(int(__builtin_rintf((y[gp] - zf) / sf)), 0), TOP);
    s_code[rw][32 * gp + cc] = uint8_t(code);
    if (cc == 0) {
      s_sz[rw][gp][0] = uint16_t(s16);
      s_sz[rw][gp][1] = uint16_t(z16);
    }
  }
  if (tid < nr) {  // the page ids, now needed (their round trip overlapped the work above)
    s_page[tid] = my_page;
    s_slot[tid] = my_slot;
  }
  lds_barrier();

  // f16 scale and zero of each (row, group of the pair)
  if (tid < 2 * nr && s_page[tid >> 1] >= 0) {
    const int row = tid >> 1, gp = tid & 1, g = 2 * pair + gp, slot = s_slot[row];
    uint8_t* base = p.pool + (int64_t(s_page[row]) * p.n_kv + h) * int64_t(QL::HEAD_BYTES);
    const int iu = (tensor == 0 || BITS == 4) ? slot * NG + g : ((slot >> 2) * NG + g) * 4 + (slot & 3);
    reinterpret_cast<uint16_t*>(base + (tensor == 0 ? QL::KS : QL::VS))[iu] = s_sz[row][gp][0];
    reinterpret_cast<uint16_t*>(base + (tensor == 0 ? QL::KZ : QL::VZ))[iu] = s_sz[row][gp][1];
  }

  // code fields of the page layout.  K, row slot m: word (quad 16 + m) NW + pair
  // holds channel 32 gp + 16 hb + 4 quad + r of the pair at bit
  // 16 (r % 2) + 8 gp + 4 hb + 2 (r / 2).  V, row slot t = 4q + r: the byte
  // 2 (r % 2) + r / 2 of word (q 16 + c16) NW + pair holds channel 16 bb + c16
  // of the pair at bit 2 bb.
  if (BITS == 4) {
    // INT4: the pair's 64 channels are bytes [32 pair, 32 pair + 32) of the row
    // (channel 2i in the low nibble of byte i)
    if (tid < 32 * nr && s_page[tid >> 5] >= 0) {
      const int row = tid >> 5, bi = tid & 31, slot = s_slot[row];
      uint8_t* base = p.pool + (int64_t(s_page[row]) * p.n_kv + h) * int64_t(QL::HEAD_BYTES);
      base[(tensor == 0 ? QL::KC : QL::VC) + slot * (D / 2) + 32 * pair + bi] =
          uint8_t(s_code[row][2 * bi] | (s_code[row][2 * bi + 1] << 4));
    }
  } else if (tensor == 0) {
    if (tid < 4 * nr && s_page[tid >> 2] >= 0) {
      const int row = tid >> 2, quad = tid & 3, slot = s_slot[row];
      uint32_t w = 0;
#pragma unroll
      for (int gp = 0; gp < 2; ++gp)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            w |= uint32_t(s_code[row][32 * gp + 16 * hb + 4 * quad + r]) << (16 * (r & 1) + 8 * gp + 4 * hb + 2 * (r >> 1));
      uint8_t* base = p.pool + (int64_t(s_page[row]) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
      reinterpret_cast<uint32_t*>(base + GG::KC)[(quad * 16 + slot) * NW + pair] = w;
    }
  } else {
    if (tid < 16 * nr && s_page[tid >> 4] >= 0) {
      const int row = tid >> 4, c16 = tid & 15, slot = s_slot[row];
      const int q = slot >> 2, r = slot & 3;
      uint32_t bits = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) bits |= uint32_t(s_code[row][16 * bb + c16]) << (2 * bb);
      uint8_t* base = p.pool + (int64_t(s_page[row]) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
      base[GG::VC + ((q * 16 + c16) * NW + pair) * 4 + 2 * (r & 1) + (r >> 1)] = uint8_t(bits);
    }
  }
  if (STEP && BITS == 2 && pair == 0) {
    // the new tokens to their BF16 slots (the first group pair's workgroups)
    const int rw2 = tid >> 5;
    if (rw2 < nr && s_new[rw2] >= 0) {
      uint16_t* hp = p.bf16_pool + (int64_t(s_new[rw2]) * p.n_kv + h) * GG::BF16_HEAD_ELEMS;
      const uint16_t* xr = X + ((row0 + rw2) * p.n_kv + h) * D;
      const int slot = s_newslot[rw2];
      for (int c = tid & 31; c < D; c += 32) {
        if (tensor == 0) hp[slot * D + c] = xr[c];
        else hp[16 * D + c * 16 + slot] = xr[c];
      }
    }
  }
}

}  // namespace

namespace oscar_launch {

hipError_t quantize_append(int d, int bits, int n_kv, void* pool, const void* k_new, const void* v_new, int64_t n_rows,
                           const int32_t* row_seq, const int32_t* row_pos, const int32_t* bt_q,
                           int32_t max_pages, const float* r_k, const float* r_v, float tau_k, float tau_v,
                           int n_cus, hipStream_t stream) {
  QAParams p{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), n_rows, row_seq, row_pos,
             bt_q, max_pages, r_k, r_v, tau_k, tau_v, static_cast<uint8_t*>(pool), n_kv};
  // workgroups loop over tiles of 16 rows (the split rotation stays in
  // registers); about three workgroups per CU over all (head, tensor) pairs
  if (n_rows <= kFewRows) {
    // few rows: plain float32 products, a slice of R per workgroup
    const dim3 grid(static_cast<unsigned>((n_rows + kRowsPerWg - 1) / kRowsPerWg), static_cast<unsigned>(n_kv),
                    static_cast<unsigned>(d / 32));  // (tensor, group pair)
    if (bits == 4) {
      if (d == 128) hipLaunchKernelGGL((quantize_rows_kernel<128, false, 4>), grid, dim3(kRowThreads), 0, stream, p);
      else hipLaunchKernelGGL((quantize_rows_kernel<64, false, 4>), grid, dim3(kRowThreads), 0, stream, p);
    } else {
      if (d == 128) hipLaunchKernelGGL((quantize_rows_kernel<128, false, 2>), grid, dim3(kRowThreads), 0, stream, p);
      else hipLaunchKernelGGL((quantize_rows_kernel<64, false, 2>), grid, dim3(kRowThreads), 0, stream, p);
    }
    return hipGetLastError();
  }
  const int64_t tiles = (n_rows + 15) / 16;
  const int64_t per_pair = std::max<int64_t>(1, (4 * int64_t(n_cus) + 2 * n_kv - 1) / (2 * n_kv));
  const dim3 grid(static_cast<unsigned>(std::min(tiles, per_pair)), static_cast<unsigned>(n_kv), 2u);
  // one tile per workgroup (few rows, as in a decode step): the unpipelined variant
  const bool one = tiles <= per_pair;
#define OSCAR_QA(DD, ONE_, BB) hipLaunchKernelGGL((quantize_append_kernel<DD, ONE_, BB>), grid, dim3(2 * DD), 0, stream, p)
  if (bits == 4) {
    if (d == 128) { if (one) OSCAR_QA(128, true, 4); else OSCAR_QA(128, false, 4); }
    else { if (one) OSCAR_QA(64, true, 4); else OSCAR_QA(64, false, 4); }
  } else {
    if (d == 128) { if (one) OSCAR_QA(128, true, 2); else OSCAR_QA(128, false, 2); }
    else { if (one) OSCAR_QA(64, true, 2); else OSCAR_QA(64, false, 2); }
  }
#undef OSCAR_QA
  return hipGetLastError();
}

hipError_t decode_step_update(int d, int n_kv, int n_sink, int n_recent, void* int2_pool, void* bf16_pool,
                              const void* k_new, const void* v_new, int batch, const int32_t* seq_lens,
                              const int32_t* bt_q, const int32_t* bt_h, int32_t max_pages, const float* r_k,
                              const float* r_v, float tau_k, float tau_v, hipStream_t stream) {
  QAParams p{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), batch, nullptr, nullptr,
             bt_q, max_pages, r_k, r_v, tau_k, tau_v, static_cast<uint8_t*>(int2_pool), n_kv,
             seq_lens, bt_h, static_cast<uint16_t*>(bf16_pool), n_sink, n_recent};
  const dim3 grid(static_cast<unsigned>((batch + kRowsPerWg - 1) / kRowsPerWg), static_cast<unsigned>(n_kv),
                  static_cast<unsigned>(d / 32));
  if (d == 128) hipLaunchKernelGGL((quantize_rows_kernel<128, true, 2>), grid, dim3(kRowThreads), 0, stream, p);
  else hipLaunchKernelGGL((quantize_rows_kernel<64, true, 2>), grid, dim3(kRowThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace oscar_launch
