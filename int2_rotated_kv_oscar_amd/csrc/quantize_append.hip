// Kernel A — quantize-append: rotate new K/V rows by the fixed rotation,
// clip, quantize per token in 32-channel groups to asymmetric INT2 and pack
// the codes into INT2 pages ([TS] 2.2.B online serving: the middle history is
// stored in INT2 after the fixed OSCAR rotation and clipping; [TS] 2.2.A
// step 4 for the per-layer clip).
//
// A workgroup takes one (KV head, tensor) and loops over tiles of 16 rows,
// one wave per 32-channel group (so group statistics stay inside a wave).  The
// rotation y = x . R is a dense 16 x d x d product per tile and runs on the
// 16x16x32 bf16 MFMA: x is exact in bf16, R (float32) is split exactly into
// three bf16 parts, so y is float32-accurate.  Tiles use the transposed
// product y^T = R^T x^T, whose output lane layout (one row per lane, 4
// consecutive channels per 16-channel block) keeps a 32-channel group inside
// one wave over its 4 lane quads: group min/max take two cross-lane steps.
// Codes are OR-combined into the page's word layout in LDS; a tile that is
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
};

// Group statistics -> f16 scale/zero (RNE) and a code generator.  s is
// (max - min) / 3 taken as a product with fp32(1/3) and the reciprocal of the
// stored f16 scale is the hardware approximation: both stay far inside the
// agreement windows (1e-6 of the group range for s, 1e-5 of a step for codes).
struct GroupQ {
  float zf, inv;
  uint32_t s16, z16;
  __device__ __forceinline__ void make(float mn, float mx) {
    s16 = f16_bits((mx - mn) * (1.0f / 3.0f));
    z16 = f16_bits(mn);
    const float sf = f16_to_f32(s16);
    zf = f16_to_f32(z16);
    inv = sf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sf);  // s16 = 0: every code is 0
  }
  __device__ __forceinline__ uint32_t code(float y) const {
    const float t = __builtin_rintf((y - zf) * inv);
    return uint32_t(__builtin_amdgcn_fmed3f(t, 0.0f, 3.0f));
  }
};

// Per-tile row metadata: lane l16 describes row tile*16 + l16 (all quads hold
// the same), page -1 for rows past n_rows.
struct TileMeta {
  int32_t page, slot;
  bool valid;    // the row exists (page is meaningful only then)
  bool aligned;  // 16 consecutive positions of one sequence starting on a page boundary
};

// ONE: every workgroup has exactly one tile (a decode step's appends)
template <int D, int TENSOR, bool ONE>
__device__ void qa_tiles(const QAParams& p, int h) {
  using GG = Geo<D>;
  constexpr int NG = GG::NG, NKB = GG::NKB, NW = GG::NW;
  constexpr int kDepth = 4;              // tiles in flight per workgroup
  constexpr float kRScale = 256.0f;
  constexpr int kRowBytes = 2 * D + 16;  // padded LDS row of the x tile (conflict-free operand reads)
  // x tiles (double-buffered), code words of a tile (one slot per lane,
  // OR-combined by the NG waves) and its f16 scales/zeros in page-area order
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][16 * kRowBytes];
  __shared__ uint32_t s_words[2][64][NW];
  __shared__ uint32_t s_sz[2][16 * NG];  // [scale area | zero area] as u32 pairs of f16
  __shared__ int32_t s_rexp[2][16];       // per-row power-of-two prescale of the x tile
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* X = TENSOR ? p.v_new : p.k_new;
  const float* R = (TENSOR ? p.r_v : p.r_k) + size_t(h) * D * D;
  const float tau = TENSOR ? p.tau_v : p.tau_k;
  const int64_t n_tiles = (p.n_rows + 15) / 16;
  const int64_t n_mine = (n_tiles - blockIdx.x + gridDim.x - 1) / gridDim.x;  // >= 1 by the grid size

  for (int i = tid; i < 2 * 64 * NW; i += 64 * NG) (&s_words[0][0][0])[i] = 0u;

  // The i-th tile of this workgroup (clamped: past the end repeats the last).
  auto tile_of = [&](int64_t i) { return int64_t(blockIdx.x) + min(i, n_mine - 1) * int64_t(gridDim.x); };
  // Ring of tiles in flight: wave g holds rows 4g .. 4g+3 of a tile (16 B per
  // lane), every lane the position of row l16.  Rows past n_rows re-read the
  // last row; their results are never stored.
  constexpr int kQuarterRows = 16 / NG;        // rows of a tile per wave
  constexpr int kChunks = 2 * D / 16;          // 16-byte chunks per row
  static_assert(kQuarterRows * kChunks == 64, "one 16-byte chunk per lane");
  u32x4 xr[kDepth];
  int32_t sr[kDepth], pr[kDepth];
  auto issue = [&](int u, int64_t i) {
    const int64_t t = tile_of(i);
    const int64_t xrow = min(t * 16 + kQuarterRows * g + lane / kChunks, p.n_rows - 1);
    xr[u] = *reinterpret_cast<const u32x4*>(X + (xrow * p.n_kv + h) * D + 8 * (lane % kChunks));
    const int64_t row = min(t * 16 + l16, p.n_rows - 1);
    sr[u] = p.row_seq[row];
    pr[u] = p.row_pos[row];
  };
#pragma unroll
  for (int u = 0; u < (ONE ? 1 : kDepth); ++u) issue(u, u);  // requested before R: the latencies overlap

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


  // stores of a finished tile: wave 0 the codes (then clears its word buffer),
  // wave 1 the scale/zero areas of an aligned tile
  auto store_tile = [&](const TileMeta& mc, int buf) {
    if (g == 0) {
      if (TENSOR == 0) {
        if (mc.valid) {  // K code words hold a single token: plain stores
          uint8_t* base = p.pool + (int64_t(mc.page) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
          uint32_t* kc = reinterpret_cast<uint32_t*>(base + GG::KC) + (quad * 16 + mc.slot) * NW;
#pragma unroll
          for (int w = 0; w < NW; ++w) kc[w] = s_words[buf][lane][w];
        }
      } else if (mc.aligned) {
        // 16 rows = slots 0..15 of one page: the words are the page's VC words
        const int page0 = __shfl(mc.page, 0, 64);
        uint8_t* base = p.pool + (int64_t(page0) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
        uint32_t* vc = reinterpret_cast<uint32_t*>(base + GG::VC) + lane * NW;
#pragma unroll
        for (int w = 0; w < NW; ++w) vc[w] = s_words[buf][lane][w];
      } else {
        // rows of different pages/slots: replace this row's 2-bit fields with
        // an atomic xor (other rows may update other fields of the same word)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int vpage = __shfl(mc.valid ? mc.page : -1, 4 * quad + r, 64), vslot = __shfl(mc.slot, 4 * quad + r, 64);
          if (vpage < 0) continue;
          uint8_t* base = p.pool + (int64_t(vpage) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
          const int sh = 16 * (vslot & 1) + 8 * ((vslot >> 1) & 1);
          uint32_t* vc = reinterpret_cast<uint32_t*>(base + GG::VC) + ((vslot >> 2) * 16 + l16) * NW;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t bits = ((s_words[buf][lane][w] >> (16 * (r & 1) + 8 * (r >> 1))) & 0xFFu) << sh;
            const uint32_t mask = 0xFFu << sh;
            const uint32_t old = __hip_atomic_load(vc + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t delta = (old & mask) ^ bits;
            if (delta) atomicXor(vc + w, delta);
          }
        }
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) s_words[buf][lane][w] = 0u;
    } else if (g == 1 && mc.aligned) {
      // scale and zero areas of the page are contiguous: 2 x 32 NG bytes
      const int page0 = __shfl(mc.page, 0, 64);
      uint8_t* base = p.pool + (int64_t(page0) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
      uint32_t* dst = reinterpret_cast<uint32_t*>(base + (TENSOR == 0 ? GG::KS : GG::VS));
      for (int i = lane; i < 16 * NG; i += 64) dst[i] = s_sz[buf][i];
    }
  };

  // Three-stage software pipeline over tiles: at step i the MFMAs of tile i run
  // while the epilogue of tile i-1 (codes, scales into LDS) executes, and the
  // words of tile i-2 are stored.  One barrier per step.
  auto epilogue = [&](const f32x4 (&acc)[2], const TileMeta& mc, int rexp, int buf) {
    // ---- epilogue for group g: acc[hb][r] = y / F for row m = l16, channel
    // 32g + 16hb + 4quad + r, F = 2^(e - 8) (R scale and row prescale); the
    // clip, the codes and the statistics run on acc with F folded into them ----
    const float F = __builtin_ldexpf(1.0f, rexp - 8), iF = __builtin_ldexpf(1.0f, 8 - rexp);
    const float tc = tau * iF;
    float y[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[hb][r] = __builtin_amdgcn_fmed3f(acc[hb][r], -tc, tc);
    float mn = fminf(fminf(fminf(y[0][0], y[0][1]), fminf(y[0][2], y[0][3])),
                     fminf(fminf(y[1][0], y[1][1]), fminf(y[1][2], y[1][3])));
    float mx = fmaxf(fmaxf(fmaxf(y[0][0], y[0][1]), fmaxf(y[0][2], y[0][3])),
                     fmaxf(fmaxf(y[1][0], y[1][1]), fmaxf(y[1][2], y[1][3])));
    GroupQ q; q.make(wave_min16(mn) * F, wave_max16(mx) * F);
    q.zf *= iF;   // codes from acc directly: (y - z) / s = (acc - z/F) / (s/F)
    q.inv *= F;
    uint16_t* sz16 = reinterpret_cast<uint16_t*>(s_sz[buf]);
    const int m = l16;
    if (TENSOR == 0) {
      // KC word (quad*16 + m)*NW + g/2 belongs to this lane
      uint32_t bits = 0;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) bits |= q.code(y[hb][r]) << (16 * (r & 1) + 8 * (g & 1) + 4 * hb + 2 * (r >> 1));
      atomicOr(&s_words[buf][lane][g / 2], bits);
    } else {
      // VC word ((m/4)*16 + c16)*NW + w, c16 = 4quad + r, w = g/2; tile row m
      // at bit 16(m%2) + 8((m/2)%2), block bb = (2g + hb)%4 at 2bb
      // the four rows m = 4j..4j+3 (consecutive lanes) share these words: their
      // fields are OR-combined across the lane quartet first, then lane m
      // writes word r = m%4, one writer per word and wave
      const int sh = 16 * (m & 1) + 8 * ((m >> 1) & 1);
      uint32_t mine = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t bits = (q.code(y[0][r]) << (sh + 2 * ((2 * g) & 3))) |
                        (q.code(y[1][r]) << (sh + 2 * ((2 * g + 1) & 3)));
        bits |= uint32_t(__builtin_amdgcn_mov_dpp(int(bits), 0xB1, 0xF, 0xF, false));  // lanes ^1
        bits |= uint32_t(__builtin_amdgcn_mov_dpp(int(bits), 0x4E, 0xF, 0xF, false));  // lanes ^2
        if ((m & 3) == r) mine = bits;
      }
      atomicOr(&s_words[buf][(m >> 2) * 16 + 4 * quad + (m & 3)][g / 2], mine);
    }
    if (quad == 0) {
      const int ia = TENSOR == 0 ? m * NG + g : ((m >> 2) * NG + g) * 4 + (m & 3);  // aligned: slot = m
      if (mc.aligned) {
        sz16[ia] = uint16_t(q.s16);
        sz16[16 * NG + ia] = uint16_t(q.z16);
      } else if (mc.valid) {
        uint8_t* base = p.pool + (int64_t(mc.page) * p.n_kv + h) * int64_t(GG::HEAD_BYTES);
        const int s = mc.slot;
        const int iu = TENSOR == 0 ? s * NG + g : ((s >> 2) * NG + g) * 4 + (s & 3);
        reinterpret_cast<uint16_t*>(base + (TENSOR == 0 ? GG::KS : GG::VS))[iu] = uint16_t(q.s16);
        reinterpret_cast<uint16_t*>(base + (TENSOR == 0 ? GG::KZ : GG::VZ))[iu] = uint16_t(q.z16);
      }
    }
  };

  // bf16 -> f16 is exact for |x| < 2^15 (down to 2^-17; smaller values round
  // at 2^-25).  A row holding a larger value is scaled by a power of two
  // 2^-e (e recorded per row and undone in the epilogue) before conversion.
  auto stage_x = [&](const u32x4& v, int buf) {
    const int row = kQuarterRows * g + lane / kChunks;
    bool big = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      big |= ((v[i] & 0x7F80u) >= (142u << 7)) | (((v[i] >> 16) & 0x7F80u) >= (142u << 7));
    u32x4 o;
    int e = 0;
    if (__builtin_expect(__any(big), 0)) {
      // exponent of the row's largest value, over the row's kChunks lanes
      int ex = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) ex = max(ex, int(max(v[i] & 0x7F80u, (v[i] >> 16) & 0x7F80u) >> 7));
#pragma unroll
      for (int msk = 1; msk < kChunks; msk <<= 1) ex = max(ex, __shfl_xor(ex, msk, 64));
      e = max(0, ex - 141);
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

  TileMeta m1 = {0, 0, false, false}, m2 = m1;
  int rep = 0;  // row prescale of the tile whose epilogue runs next
  f32x4 accp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  __syncthreads();  // s_words zeroed
  if constexpr (ONE) {
    // one tile for this workgroup: the same steps without the pipeline, two
    // barriers instead of three rounds
    stage_x(xr[0], 0);
    TileMeta mc;
    {
      const int64_t t = tile_of(0);
      const int32_t seq = sr[0], pos = pr[0];
      mc.page = p.bt_q[int64_t(seq) * p.max_pages + (pos >> 4)];
      mc.valid = t * 16 + l16 < p.n_rows;
      mc.slot = pos & 15;
      const int32_t seq0 = __shfl(seq, 0, 64), pos0 = __shfl(pos, 0, 64);
      const bool ok = mc.valid && seq == seq0 && pos == pos0 + l16 && (pos0 & 15) == 0;
      mc.aligned = (__ballot(ok) & 0xFFFFull) == 0xFFFFull;
    }
    lds_barrier();
    f32x4 acc1[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      u32x4 xc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) xc[kb] = *reinterpret_cast<const u32x4*>(&s_x[0][l16 * kRowBytes + 64 * kb + 16 * quad]);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int j = 1; j >= 0; --j) acc1[hb] = mfma_f16(rop[hb][kb][j], xc[kb], acc1[hb]);
    }
    epilogue(acc1, mc, s_rexp[0][l16], 0);
    lds_barrier();
    store_tile(mc, 0);
  } else {
  for (int64_t i0 = 0; i0 < n_mine + 2; i0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int64_t i = i0 + u;
      const int buf = int(i & 1);
      // tile i: x quarter -> f16 in LDS, positions -> page, slot, alignment
      stage_x(xr[u], buf);
      TileMeta mc;
      {
        const int64_t t = tile_of(i);
        const int32_t seq = sr[u], pos = pr[u];
        const bool valid = i < n_mine && t * 16 + l16 < p.n_rows;
        mc.page = p.bt_q[int64_t(seq) * p.max_pages + (pos >> 4)];  // seq/pos of a real row
        mc.valid = valid;
        mc.slot = pos & 15;
        const int32_t seq0 = __shfl(seq, 0, 64), pos0 = __shfl(pos, 0, 64);
        const bool ok = valid && seq == seq0 && pos == pos0 + l16 && (pos0 & 15) == 0;
        mc.aligned = (__ballot(ok) & 0xFFFFull) == 0xFFFFull;
      }
      // refill the ring slot kDepth tiles ahead (clamped: always issued)
      issue(u, i + kDepth);
      lds_barrier();
      // tile i-2: its LDS words are complete (buffer i&1)
      if (i >= 2 && i - 2 < n_mine) store_tile(m2, buf);
      f32x4 accn[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if (i < n_mine) {
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
              accn[hb] = mfma_f16(rop[hb][kb][j], xc[kb], accn[hb]);
      }
      const int ren = s_rexp[buf][l16];  // read now: the buffer is rewritten two steps on
      // tile i-1: codes and scales into LDS buffer (i-1)&1
      if (i >= 1 && i - 1 < n_mine) epilogue(accp, m1, rep, buf ^ 1);
      accp[0] = accn[0];
      accp[1] = accn[1];
      rep = ren;
      m2 = m1;
      m1 = mc;
    }
  }
  }  // pipelined tiles
}

template <int D, bool ONE>
__global__ __launch_bounds__(64 * (D / 32)) void quantize_append_kernel(QAParams p) {
  const int h = blockIdx.y;
  if (blockIdx.z == 0)
    qa_tiles<D, 0, ONE>(p, h);
  else
    qa_tiles<D, 1, ONE>(p, h);
}

}  // namespace

namespace oscar_launch {

hipError_t quantize_append(int d, int n_kv, void* pool, const void* k_new, const void* v_new, int64_t n_rows,
                           const int32_t* row_seq, const int32_t* row_pos, const int32_t* bt_q,
                           int32_t max_pages, const float* r_k, const float* r_v, float tau_k, float tau_v,
                           int n_cus, hipStream_t stream) {
  QAParams p{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), n_rows, row_seq, row_pos,
             bt_q, max_pages, r_k, r_v, tau_k, tau_v, static_cast<uint8_t*>(pool), n_kv};
  // workgroups loop over tiles of 16 rows (the split rotation stays in
  // registers); about three workgroups per CU over all (head, tensor) pairs
  const int64_t tiles = (n_rows + 15) / 16;
  const int64_t per_pair = std::max<int64_t>(1, (3 * int64_t(n_cus) + 2 * n_kv - 1) / (2 * n_kv));
  const dim3 grid(static_cast<unsigned>(std::min(tiles, per_pair)), static_cast<unsigned>(n_kv), 2u);
  // one tile per workgroup (few rows, as in a decode step): the unpipelined variant
  const bool one = tiles <= per_pair;
  if (d == 128) {
    if (one) hipLaunchKernelGGL((quantize_append_kernel<128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((quantize_append_kernel<128, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (one) hipLaunchKernelGGL((quantize_append_kernel<64, true>), grid, dim3(128), 0, stream, p);
    else hipLaunchKernelGGL((quantize_append_kernel<64, false>), grid, dim3(128), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace oscar_launch
