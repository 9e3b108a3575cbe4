// GPU calibration statistics ([TS] 2.1 and 2.2.A step 1: the key target is
// the query covariance Q^T Q / N, the value target V^T S^T S V / N = O^T O / N
// with O = S V the attention output; both pooled over the query heads of a KV
// group).  One kernel computes C(h) = (1 / (N G)) sum_n sum_{i in group h}
// x_{n,i}^T x_{n,i} for bf16 rows x (Q or O as a calibration forward pass
// produces them).  The eigendecomposition of C stays on the host in float64.
//
// The Gram matrix is a dense contraction over the N G pooled rows and runs on
// the 16x16x32 bf16 MFMA: bf16 x bf16 products are exact in float32, each
// workgroup sums blocks of 256 rows in float32, adds the blocks in float64
// and its partial, scaled by 1 / (N G), into the float64 result with
// float64 atomics; only the blocks on and above the diagonal are formed and
// the rest is mirrored.
#include <algorithm>

#include "device_utils.h"
#include "kernels.h"

using namespace oscar_dev;

namespace {

constexpr int kGramRows = 1024;  // pooled rows per workgroup
constexpr int kGramBlock = 256;  // rows per float32 block (then added into float64 registers)
constexpr int kGramStage = 128;  // rows staged in LDS per barrier pair
constexpr int kGramThreads = 512;

struct GramParams {
  const uint16_t* x;   // bf16 [N][Hx][D]
  int64_t n_rows;      // N
  int32_t n_x_heads;   // Hx = H_kv G
  int32_t group;       // G
  double* out;         // float64 [H_kv][D][D]
  double scale;        // 1 / (N G)
};

// Workgroup (chunk of 1024 pooled rows r = n G + j, KV head h).  Wave w owns
// the output rows 16 w .. 16 w + 15 (D = 128: all eight waves; D = 64: waves
// 0-3) against every column block.  Rows are loaded coalesced (16 lanes per
// 256-byte row) and staged transposed in LDS (channel-major), so both MFMA
// operands are 16-byte reads: A[i][k] = x[row k][16 ti + i], B[k][j] =
// x[row k][16 tj + j].  Row r of channel ch sits at position r ^ swz(ch),
// swz(ch) = 8 ((ch ^ (ch >> 3)) mod 16): a bijection over the 16 channels one
// write instruction touches (8 c + e, c = 0..15) and over the 16 one operand
// read touches (16 t + i, i = 0..15), so the 2-byte writes and the 16-byte
// reads fall in distinct banks, and every aligned 8-row group stays contiguous.
// Each block of 256 rows is summed in float32 (exact products) and then
// added into float64 registers; the workgroup's float64 partial, scaled by
// 1 / (N G), goes to the result with float64 atomic adds.
template <int D>
__global__ __launch_bounds__(kGramThreads) void calib_gram_kernel(GramParams p) {
  constexpr int NB = D / 16;             // channel blocks
  __shared__ __attribute__((aligned(16))) uint16_t s_xt[D][kGramStage];
  auto swz = [](int ch) { return 8 * ((ch ^ (ch >> 3)) & 15); };
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile choices are scalar branches
  const int h = blockIdx.y;
  const int64_t pooled = p.n_rows * p.group;
  const int64_t r0 = int64_t(blockIdx.x) * kGramRows;
  const int ti = wave;                   // output row block of this wave (used when < NB)
  double acc64[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc64[j][r] = 0.0;
  f32x4 acc[NB];
  // staging: load i of lane l in wave w is the 16-byte channel chunk l % NC of
  // stage row 16 w + (64 / NC) i + l / NC (NC = D / 8 chunks per row)
  constexpr int NC = D / 8;
  constexpr int kLoads = kGramStage * NC / kGramThreads;  // 4 (D = 128) or 2 (D = 64)
  static_assert(kGramStage == 128 && kGramBlock % (2 * kGramStage) == 0 && kGramThreads == 512, "staging map");
  auto srow = [&](int i) { return 16 * wave + (64 / NC) * i + lane / NC; };
  const int c8 = 8 * (lane % NC);
  // the rows of stage `st` (kGramStage rows from r0 + st kGramStage) into v;
  // rows past the end read as zeros.  Pooled row r = n G + j sits at element
  // (n H_x + h G + j) D: one scalar division per stage gives the stage's
  // first (n, j), and a lane's offset t = j0 + row (< 128 + 16) splits as
  // t = q G + j with q = floor((t + 1/2) / G) from a float reciprocal (exact:
  // (t + 1/2) / G is at least 1/32 away from an integer for G <= 16)
  const float inv_g = 1.0f / float(p.group);
  const uint16_t* xh = p.x + int64_t(h) * p.group * D;
  auto load_stage = [&](u32x4 (&v)[kLoads], int st) {
    const int64_t rb = r0 + int64_t(st) * kGramStage;
    const int64_t nb = rb / p.group;
    const int j0 = int(rb - nb * p.group);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int rr = srow(i);
      const int t = j0 + rr;
      const int q = int((float(t) + 0.5f) * inv_g);
      const int j = t - q * p.group;
      const bool live = rb + rr < pooled;
      const int64_t n = live ? nb + q : 0;  // rows past the end read row 0 (and are zeroed)
      const u32x4 w = *reinterpret_cast<const u32x4*>(xh + (n * p.n_x_heads + (live ? j : 0)) * D + c8);
      v[i] = live ? w : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // stages past the end of the rows are skipped (a uniform decision); stages
  // come in pairs, each with its own registers, loaded two stages ahead
  const int n_stages = int(std::min<int64_t>(kGramRows, pooled - r0) + kGramStage - 1) / kGramStage;
  u32x4 va[kLoads], vb[kLoads];
  load_stage(va, 0);
  load_stage(vb, 1);
  auto stage = [&](u32x4 (&v)[kLoads], int st) {
    if (st % (kGramBlock / kGramStage) == 0) {
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();  // the previous stage's operand reads are done
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int rr = srow(i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_xt[c8 + 2 * e][rr ^ swz(c8 + 2 * e)] = uint16_t(v[i][e] & 0xFFFFu);
        s_xt[c8 + 2 * e + 1][rr ^ swz(c8 + 2 * e + 1)] = uint16_t(v[i][e] >> 16);
      }
    }
    __syncthreads();
    if (st + 2 < n_stages) load_stage(v, st + 2);  // in flight during the next two stages
    // upper-triangle tiles only (tj >= ti): C is symmetric, the lower
    // triangle is mirrored afterwards
    if (ti < NB) {
#pragma unroll
      for (int k0 = 0; k0 < kGramStage; k0 += 32) {
        const int ca = 16 * ti + l16;
        const u32x4 a = *reinterpret_cast<const u32x4*>(&s_xt[ca][(k0 + 8 * quad) ^ swz(ca)]);
#pragma unroll
        for (int tj = 0; tj < NB; ++tj) {
          if (tj < ti) continue;
          const int cb = 16 * tj + l16;
          const u32x4 b = *reinterpret_cast<const u32x4*>(&s_xt[cb][(k0 + 8 * quad) ^ swz(cb)]);
          acc[tj] = mfma_bf16(a, b, acc[tj]);
        }
      }
    }
    if ((st + 1) % (kGramBlock / kGramStage) == 0 || st + 1 == n_stages) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc64[j][r] += double(acc[j][r]);
    }
  };
  for (int st = 0; st < n_stages; st += 2) {
    stage(va, st);
    if (st + 1 < n_stages) stage(vb, st + 1);
  }
  if (ti < NB) {
    // acc64[tj][r] = C[16 ti + 4 quad + r][16 tj + l16] (this chunk's part), tj >= ti.
    // Workgroups start at different blocks (by their index), so that the
    // atomic adds of workgroups finishing together spread over addresses.
    double* o = p.out + size_t(h) * D * D;
    for (int k = 0; k < NB; ++k) {
      const int tj = (k + int(blockIdx.x)) % NB;
      if (tj < ti) continue;
      double v[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = t == tj ? acc64[t][r] : v[r];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __hip_atomic_fetch_add(o + size_t(16 * ti + 4 * quad + r) * D + 16 * tj + l16, v[r] * p.scale,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Lower-triangle blocks (16-channel block tj < ti) from their mirror images.
__global__ void mirror_blocks_kernel(double* out, int d) {
  double* o = out + size_t(blockIdx.y) * d * d;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < d * d; e += gridDim.x * blockDim.x) {
    const int a = e / d, b = e % d;
    if ((b >> 4) < (a >> 4)) o[e] = o[size_t(b) * d + a];
  }
}

__global__ void zero_f64_kernel(double* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x) p[i] = 0.0;
}

}  // namespace

namespace oscar_launch {

hipError_t calib_gram(int d, const void* x, int64_t n_rows, int n_x_heads, int n_kv, void* out, hipStream_t stream) {
  const int group = n_x_heads / n_kv;
  const size_t n_out = size_t(n_kv) * d * d;
  hipLaunchKernelGGL(zero_f64_kernel, dim3(unsigned(std::min<size_t>(1024, (n_out + 255) / 256))), dim3(256), 0, stream,
                     static_cast<double*>(out), n_out);
  const int64_t pooled = n_rows * group;
  GramParams p{static_cast<const uint16_t*>(x), n_rows, n_x_heads, group, static_cast<double*>(out),
               1.0 / double(pooled)};
  const dim3 grid(static_cast<unsigned>((pooled + kGramRows - 1) / kGramRows), static_cast<unsigned>(n_kv));
  if (d == 128) hipLaunchKernelGGL(calib_gram_kernel<128>, grid, dim3(kGramThreads), 0, stream, p);
  else hipLaunchKernelGGL(calib_gram_kernel<64>, grid, dim3(kGramThreads), 0, stream, p);
  hipLaunchKernelGGL(mirror_blocks_kernel, dim3(unsigned((d * d + 255) / 256), unsigned(n_kv)), dim3(256), 0, stream,
                     static_cast<double*>(out), d);
  return hipGetLastError();
}

}  // namespace oscar_launch
