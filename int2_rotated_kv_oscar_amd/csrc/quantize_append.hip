// Kernel A — quantize-append: rotate new K/V rows by the fixed rotation,
// clip, quantize per token in 32-channel groups to asymmetric INT2 and pack
// the codes into INT2 pages ([TS] 2.2.B online serving: the middle history is
// stored in INT2 after the fixed OSCAR rotation and clipping; [TS] 2.2.A
// step 4 for the per-layer clip).
//
// One workgroup handles T tiles of 16 rows for one (KV head, tensor), one
// wave per 32-channel group (so group statistics stay inside a wave).  The
// rotation y = x . R is a dense 16 x d x d product per tile and runs on the
// 16x16x32 bf16 MFMA: x is exact in bf16, R (float32) is split exactly into
// three bf16 parts, so y is float32-accurate.  K tiles use the transposed
// product y^T = R^T x^T, whose output lane layout (one row per lane, 4
// consecutive channels per 16-channel block) is exactly the KC word layout;
// V tiles use y = x R, whose layout (4 rows per lane, one channel per block)
// is exactly the VC word layout.  Group statistics are cross-lane min/max.
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

template <int D>
__device__ __forceinline__ uint8_t* head_base(const QAParams& p, int64_t row, int h, int& slot) {
  const int32_t s = p.row_seq[row], pos = p.row_pos[row];
  slot = pos & 15;
  const int64_t page = p.bt_q[int64_t(s) * p.max_pages + (pos >> 4)];
  return p.pool + (page * p.n_kv + h) * int64_t(Geo<D>::HEAD_BYTES);
}

// Group statistics -> f16 scale/zero (RNE) and a code generator.
struct GroupQ {
  float zf, inv;
  bool zero_scale;
  uint32_t s16, z16;
  __device__ __forceinline__ void make(float mn, float mx) {
    const float s = (mx - mn) / 3.0f;
    s16 = f16_bits(s);
    z16 = f16_bits(mn);
    const float sf = f16_to_f32(s16);
    zf = f16_to_f32(z16);
    zero_scale = (sf == 0.0f);
    inv = zero_scale ? 0.0f : 1.0f / sf;
  }
  __device__ __forceinline__ uint32_t code(float y) const {
    if (zero_scale) return 0u;
    const float t = __builtin_rintf((y - zf) * inv);
    return uint32_t(fminf(fmaxf(t, 0.0f), 3.0f));
  }
};

template <int D, int T, int TENSOR>
__device__ void qa_body(const QAParams& p, int h, int64_t tile0) {
  using GG = Geo<D>;
  constexpr int NG = GG::NG, NKB = GG::NKB, NW = GG::NW;
  // one wave per channel group; code words are OR-combined in LDS
  __shared__ uint32_t s_words[T][64][NW];
  const int tid = threadIdx.x, g = tid >> 6, lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  const uint16_t* X = TENSOR ? p.v_new : p.k_new;
  const float* R = (TENSOR ? p.r_v : p.r_k) + size_t(h) * D * D;
  const float tau = TENSOR ? p.tau_v : p.tau_k;

  for (int i = tid; i < T * 64 * NW; i += 64 * NG) (&s_words[0][0][0])[i] = 0u;

  // R operand values of this group, all issued at once: lane (c16 = l16, quad)
  // holds R[32kb + 8quad + i][16cb + l16] for cb = 2g + hb
  float rv[2][NKB][8];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[hb][kb][i] = R[size_t(32 * kb + 8 * quad + i) * D + 16 * (2 * g + hb) + l16];

  // x operands: lane (row l16, quad) holds channels 32kb + 8quad .. +7 of its row;
  // the same registers serve as the B operand (K) and the A operand (V).
  u32x4 xop[T][NKB];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t row = (tile0 + t) * 16 + l16;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (row < p.n_rows)
        xop[t][kb] = *reinterpret_cast<const u32x4*>(X + (row * p.n_kv + h) * D + 32 * kb + 8 * quad);
      else
        xop[t][kb] = u32x4{0, 0, 0, 0};
    }
  }

  // Row metadata.  K: the lane's row is l16.  V: the lane's rows are 4quad + r.
  uint8_t* kbase[T];
  int kslot[T];
  uint8_t* vbase[T][4];
  int vslot[T][4];
  bool aligned[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (TENSOR == 0) {
      const int64_t row = (tile0 + t) * 16 + l16;
      kslot[t] = 0;
      kbase[t] = row < p.n_rows ? head_base<D>(p, row, h, kslot[t]) : nullptr;
    } else {
      const int64_t row0 = (tile0 + t) * 16;
      bool ok = true;
      if (lane < 16) {
        const int64_t row = row0 + lane;
        ok = row < p.n_rows && p.row_seq[row] == p.row_seq[row0] && p.row_pos[row] == p.row_pos[row0] + lane &&
             (p.row_pos[row0] & 15) == 0;
      }
      aligned[t] = __ballot(ok) == ~0ull;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + 4 * quad + r;
        vslot[t][r] = 0;
        vbase[t][r] = row < p.n_rows ? head_base<D>(p, row, h, vslot[t][r]) : nullptr;
      }
    }
  }

  f32x4 acc[T][2];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      uint32_t ph[4], pm[4], pl[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const Split3 a = split3(rv[hb][kb][i]);
        const Split3 b = split3(rv[hb][kb][i + 1]);
        ph[i / 2] = pack2(a.hi, b.hi);
        pm[i / 2] = pack2(a.mid, b.mid);
        pl[i / 2] = pack2(a.lo, b.lo);
      }
      const u32x4 rh{ph[0], ph[1], ph[2], ph[3]}, rm{pm[0], pm[1], pm[2], pm[3]}, rl{pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if (TENSOR == 0) {
          acc[t][hb] = mfma_bf16(rl, xop[t][kb], acc[t][hb]);
          acc[t][hb] = mfma_bf16(rm, xop[t][kb], acc[t][hb]);
          acc[t][hb] = mfma_bf16(rh, xop[t][kb], acc[t][hb]);
        } else {
          acc[t][hb] = mfma_bf16(xop[t][kb], rl, acc[t][hb]);
          acc[t][hb] = mfma_bf16(xop[t][kb], rm, acc[t][hb]);
          acc[t][hb] = mfma_bf16(xop[t][kb], rh, acc[t][hb]);
        }
      }
    }
  }
  __syncthreads();  // s_words zeroed

  // ---- epilogue for group g ----
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float y[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[hb][r] = fminf(fmaxf(acc[t][hb][r], -tau), tau);
    if (TENSOR == 0) {
      // y[hb][r] = row l16, channel 32g + 16hb + 4quad + r; the group spans the 4 quads
      float mn = y[0][0], mx = y[0][0];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) { mn = fminf(mn, y[hb][r]); mx = fmaxf(mx, y[hb][r]); }
      mn = fminf(mn, __shfl_xor(mn, 16, 64)); mn = fminf(mn, __shfl_xor(mn, 32, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64)); mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      GroupQ q; q.make(mn, mx);
      uint32_t bits = 0;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) bits |= q.code(y[hb][r]) << (16 * (r & 1) + 8 * (g & 1) + 4 * hb + 2 * (r >> 1));
      atomicOr(&s_words[t][lane][g / 2], bits);
      if (quad == 0 && kbase[t]) {
        reinterpret_cast<uint16_t*>(kbase[t] + GG::KS)[kslot[t] * NG + g] = uint16_t(q.s16);
        reinterpret_cast<uint16_t*>(kbase[t] + GG::KZ)[kslot[t] * NG + g] = uint16_t(q.z16);
      }
    } else {
      // y[hb][r] = row 4quad + r, channel 32g + 16hb + l16; the group spans the 16 lanes
      uint32_t bits = 0;  // 8 bits per row r: code of block bb at 2bb
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mn = fminf(y[0][r], y[1][r]), mx = fmaxf(y[0][r], y[1][r]);
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          mn = fminf(mn, __shfl_xor(mn, m, 64));
          mx = fmaxf(mx, __shfl_xor(mx, m, 64));
        }
        GroupQ q; q.make(mn, mx);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) bits |= q.code(y[hb][r]) << (8 * r + 2 * (2 * (g & 1) + hb));
        if (l16 == 0 && vbase[t][r]) {
          const int s = vslot[t][r];
          const int idx = ((s >> 2) * NG + g) * 4 + (s & 3);
          reinterpret_cast<uint16_t*>(vbase[t][r] + GG::VS)[idx] = uint16_t(q.s16);
          reinterpret_cast<uint16_t*>(vbase[t][r] + GG::VZ)[idx] = uint16_t(q.z16);
        }
      }
      atomicOr(&s_words[t][lane][g / 2], bits);
    }
  }
  __syncthreads();
  if (g != 0) return;

  // ---- code stores (wave 0) ----
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (TENSOR == 0) {
      if (kbase[t]) {
        uint32_t* kc = reinterpret_cast<uint32_t*>(kbase[t] + GG::KC) + (quad * 16 + kslot[t]) * NW;
#pragma unroll
        for (int w = 0; w < NW; ++w) kc[w] = s_words[t][lane][w];
      }
    } else if (aligned[t]) {
      // 16 rows = slots 0..15 of one page: the lane owns whole VC words
      uint32_t* vc = reinterpret_cast<uint32_t*>(vbase[t][0] + GG::VC) + (quad * 16 + l16) * NW;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t b = s_words[t][lane][w];
        uint32_t out = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) out |= ((b >> (8 * r)) & 0xFFu) << (16 * (r & 1) + 8 * (r >> 1));
        vc[w] = out;
      }
    } else {
      // rows of different pages/slots: replace this row's 2-bit fields with
      // an atomic xor (other rows may update other fields of the same word)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!vbase[t][r]) continue;
        const int s = vslot[t][r];
        const int sh = 16 * (s & 1) + 8 * ((s >> 1) & 1);
        uint32_t* vc = reinterpret_cast<uint32_t*>(vbase[t][r] + GG::VC) + ((s >> 2) * 16 + l16) * NW;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t bits = ((s_words[t][lane][w] >> (8 * r)) & 0xFFu) << sh;
          const uint32_t mask = 0xFFu << sh;
          const uint32_t old = __hip_atomic_load(vc + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t delta = (old & mask) ^ bits;
          if (delta) atomicXor(vc + w, delta);
        }
      }
    }
  }
}

template <int D, int T>
__global__ __launch_bounds__(64 * (D / 32)) void quantize_append_kernel(QAParams p) {
  const int h = blockIdx.y;
  const int64_t tile0 = int64_t(blockIdx.x) * T;
  if (blockIdx.z == 0)
    qa_body<D, T, 0>(p, h, tile0);
  else
    qa_body<D, T, 1>(p, h, tile0);
}

}  // namespace

namespace oscar_launch {

hipError_t quantize_append(int d, int n_kv, void* pool, const void* k_new, const void* v_new, int64_t n_rows,
                           const int32_t* row_seq, const int32_t* row_pos, const int32_t* bt_q,
                           int32_t max_pages, const float* r_k, const float* r_v, float tau_k, float tau_v,
                           hipStream_t stream) {
  QAParams p{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), n_rows, row_seq, row_pos,
             bt_q, max_pages, r_k, r_v, tau_k, tau_v, static_cast<uint8_t*>(pool), n_kv};
  const int64_t tiles = (n_rows + 15) / 16;
  const bool big = tiles >= 4 * 256;
  const int T = big ? 4 : 1;
  const dim3 grid(static_cast<unsigned>((tiles + T - 1) / T), static_cast<unsigned>(n_kv), 2u);
  if (d == 128) {
    if (big) hipLaunchKernelGGL((quantize_append_kernel<128, 4>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((quantize_append_kernel<128, 1>), grid, dim3(256), 0, stream, p);
  } else {
    if (big) hipLaunchKernelGGL((quantize_append_kernel<64, 4>), grid, dim3(128), 0, stream, p);
    else hipLaunchKernelGGL((quantize_append_kernel<64, 1>), grid, dim3(128), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace oscar_launch
