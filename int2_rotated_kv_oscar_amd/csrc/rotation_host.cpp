// Offline calibration on the host in float64: oscar_build_rotation.
//
// [TS] 2.1: the key target is the query covariance Q^T Q, the value target is
// V^T S^T S V (S = attention scores).  [TS] 2.2.A: eigendecompose the targets,
// compose R = U . H_Had . P_br, estimate one clip threshold per layer from the
// rotated calibration activations.  Readings (causal calibration scores,
// descending eigen order with a sign rule, linear quantile) are stated in
// include/oscar.h.
//
// The O(N^2 d) causal attention that produces S V for the value target is the
// only heavy loop; it runs blocked over query rows on a pool of std::threads.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

#include "common.h"

namespace {

using std::size_t;

// Symmetric eigendecomposition by cyclic Jacobi rotations.  a (d x d,
// row-major) is destroyed; on return w holds the eigenvalues and v the
// eigenvectors as columns.  Converged when every off-diagonal entry is at most
// 1e-14 * ||A||_F.
bool jacobi_eigen(std::vector<double>& a, int d, int max_sweeps, std::vector<double>& w,
                  std::vector<double>& v) {
  v.assign(size_t(d) * d, 0.0);
  for (int i = 0; i < d; ++i) v[size_t(i) * d + i] = 1.0;
  double frob = 0.0;
  for (double x : a) frob += x * x;
  frob = std::sqrt(frob);
  const double tol = 1e-14 * frob;
  bool converged = (frob == 0.0);
  for (int sweep = 0; sweep < max_sweeps && !converged; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) off = std::max(off, std::fabs(a[size_t(p) * d + q]));
    if (off <= tol) {
      converged = true;
      break;
    }
    for (int p = 0; p < d - 1; ++p) {
      for (int q = p + 1; q < d; ++q) {
        const double apq = a[size_t(p) * d + q];
        if (apq == 0.0) continue;
        const double app = a[size_t(p) * d + p], aqq = a[size_t(q) * d + q];
        // rotation angle that annihilates a_pq: tan(2 phi) = 2 a_pq / (a_qq - a_pp)
        const double theta = (aqq - app) / (2.0 * apq);
        double t = 1.0 / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        if (theta < 0) t = -t;
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < d; ++k) {  // columns p, q
          const double akp = a[size_t(k) * d + p], akq = a[size_t(k) * d + q];
          a[size_t(k) * d + p] = c * akp - s * akq;
          a[size_t(k) * d + q] = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {  // rows p, q
          const double apk = a[size_t(p) * d + k], aqk = a[size_t(q) * d + k];
          a[size_t(p) * d + k] = c * apk - s * aqk;
          a[size_t(q) * d + k] = s * apk + c * aqk;
        }
        a[size_t(p) * d + q] = a[size_t(q) * d + p] = 0.0;
        for (int k = 0; k < d; ++k) {
          const double vkp = v[size_t(k) * d + p], vkq = v[size_t(k) * d + q];
          v[size_t(k) * d + p] = c * vkp - s * vkq;
          v[size_t(k) * d + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  if (!converged) {
    double off = 0.0;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) off = std::max(off, std::fabs(a[size_t(p) * d + q]));
    converged = off <= tol;
  }
  w.resize(d);
  for (int i = 0; i < d; ++i) w[i] = a[size_t(i) * d + i];
  return converged;
}

// Descending order; each column negated so its largest-|.| entry (lowest
// index on ties) is positive.
void sort_and_sign(int d, std::vector<double>& w, std::vector<double>& v) {
  std::vector<int> order(d);
  for (int i = 0; i < d; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
  std::vector<double> w2(d), v2(size_t(d) * d);
  for (int j = 0; j < d; ++j) {
    const int src = order[j];
    w2[j] = w[src];
    int imax = 0;
    double amax = -1.0;
    for (int i = 0; i < d; ++i) {
      const double x = std::fabs(v[size_t(i) * d + src]);
      if (x > amax) { amax = x; imax = i; }
    }
    const double sgn = v[size_t(imax) * d + src] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) v2[size_t(i) * d + j] = sgn * v[size_t(i) * d + src];
  }
  w.swap(w2);
  v.swap(v2);
}

int bitrev(int j, int bits) {
  int r = 0;
  for (int b = 0; b < bits; ++b) { r = (r << 1) | (j & 1); j >>= 1; }
  return r;
}

// R = U . (H / sqrt(d)) . P_br with (M P)[k][c] = M[k][br(c)].
void compose_rotation(int d, const std::vector<double>& u, double* r) {
  int bits = 0;
  while ((1 << bits) < d) ++bits;
  // Sylvester Hadamard entry: H[i][j] = (-1)^{popcount(i & j)}
  std::vector<double> uh(size_t(d) * d, 0.0);
  const double inv = 1.0 / std::sqrt(double(d));
  for (int k = 0; k < d; ++k)
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) {
        const double h = (__builtin_popcount(unsigned(i & j)) & 1) ? -1.0 : 1.0;
        acc += u[size_t(k) * d + i] * h;
      }
      uh[size_t(k) * d + j] = acc * inv;
    }
  for (int k = 0; k < d; ++k)
    for (int c = 0; c < d; ++c) r[size_t(k) * d + c] = uh[size_t(k) * d + bitrev(c, bits)];
}

// Runs fn(task, worker) for task in [0, n_tasks) on up to n_threads workers.
void run_parallel(int n_threads, int n_tasks, const std::function<void(int, int)>& fn) {
  std::atomic<int> next{0};
  auto worker = [&](int wid) {
    for (int t = next++; t < n_tasks; t = next++) fn(t, wid);
  };
  const int nt = std::max(1, std::min(n_threads, n_tasks));
  std::vector<std::thread> pool;
  for (int i = 1; i < nt; ++i) pool.emplace_back(worker, i);
  worker(0);
  for (auto& th : pool) th.join();
}

// O rows [r0, r1) of one query head: causal softmax(q k^T / sqrt(d)) v.
// q: row stride sq, k/v: row stride skv, all float64 copies.
void causal_block(const double* q, size_t sq, const double* k, const double* v, size_t skv, int d,
                  int r0, int r1, double* o, size_t so, std::vector<double>& scratch) {
  const int nk = r1;
  const int nr = r1 - r0;
  scratch.resize(size_t(nr) * nk);
  const double scale = 1.0 / std::sqrt(double(d));
  // scores in 2-row x 4-key blocks, 4 independent partial sums per pair so
  // the channel loop vectorises without reassociating a single sum
  for (int a = 0; a < nr; a += 2) {
    const int na = std::min(2, nr - a);
    const int kmax = std::min(nk, r0 + a + na);  // causal: keys <= last row
    for (int j = 0; j < kmax; j += 4) {
      const int nj = std::min(4, kmax - j);
      double acc[2][4][4] = {};
      const double* qr[2];
      const double* kr[4];
      for (int x = 0; x < 2; ++x) qr[x] = q + size_t(r0 + a + (x < na ? x : 0)) * sq;
      for (int y = 0; y < 4; ++y) kr[y] = k + size_t(j + (y < nj ? y : 0)) * skv;
      for (int c = 0; c < d; c += 4)
        for (int x = 0; x < 2; ++x)
          for (int y = 0; y < 4; ++y)
            for (int l = 0; l < 4; ++l) acc[x][y][l] += qr[x][c + l] * kr[y][c + l];
      for (int x = 0; x < na; ++x)
        for (int y = 0; y < nj; ++y)
          scratch[size_t(a + x) * nk + j + y] =
              ((acc[x][y][0] + acc[x][y][1]) + (acc[x][y][2] + acc[x][y][3])) * scale;
    }
  }
  for (int a = 0; a < nr; ++a) {
    const int r = r0 + a;
    double* s = &scratch[size_t(a) * nk];
    double m = -INFINITY;
    for (int j = 0; j <= r; ++j) m = std::max(m, s[j]);
    double tot = 0.0;
    for (int j = 0; j <= r; ++j) { s[j] = std::exp(s[j] - m); tot += s[j]; }
    double* out = o + size_t(r) * so;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int j = 0; j <= r; ++j) {
      const double p = s[j] / tot;
      const double* vj = v + size_t(j) * skv;
      for (int c = 0; c < d; ++c) out[c] += p * vj[c];
    }
  }
}

double linear_quantile(std::vector<double>& a, double qq) {
  const size_t m = a.size();
  const double rr = qq * double(m - 1);
  size_t lo = size_t(std::floor(rr));
  if (lo >= m) lo = m - 1;
  std::nth_element(a.begin(), a.begin() + lo, a.end());
  const double alo = a[lo];
  double ahi = alo;
  if (lo + 1 < m) ahi = *std::min_element(a.begin() + lo + 1, a.end());
  return alo + (rr - double(lo)) * (ahi - alo);
}

// [TS] 2.2.A steps 2-3 for one target: eigenbasis (descending, canonical
// signs) and R = U . H . P_br; false if the eigensolver did not converge.
bool rotation_from_target(int d, std::vector<double>& c, int max_sweeps, double* r, double* eig, int h) {
  std::vector<double> w, u;
  const bool ok = jacobi_eigen(c, d, max_sweeps, w, u);
  sort_and_sign(d, w, u);
  compose_rotation(d, u, r);
  if (eig) std::memcpy(eig + size_t(h) * d, w.data(), sizeof(double) * d);
  return ok;
}

// Per-layer clip thresholds ([TS] 2.2.A step 4): the quantile of |x R|
// pooled over rows, heads and channels, for K (which 0) and V (which 1).
void clip_thresholds(int d, int n_kv_heads, size_t N, const std::vector<double>& k, const std::vector<double>& v,
                     const double* r_k, const double* r_v, double clip_quantile, int n_threads, double* tau_k,
                     double* tau_v) {
  for (int which = 0; which < 2; ++which) {
    const std::vector<double>& x = which ? v : k;
    const double* r = which ? r_v : r_k;
    std::vector<double> y(N * n_kv_heads * d);
    run_parallel(n_threads, n_kv_heads, [&](int h, int) {
      const double* rh = r + size_t(h) * d * d;
      for (size_t n = 0; n < N; ++n) {
        const double* xr = &x[(n * n_kv_heads + h) * d];
        double* out = &y[(size_t(h) * N + n) * d];
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        for (int kk = 0; kk < d; ++kk) {
          const double xv = xr[kk];
          const double* rrow = rh + size_t(kk) * d;
          for (int c = 0; c < d; ++c) out[c] += xv * rrow[c];
        }
        for (int c = 0; c < d; ++c) out[c] = std::fabs(out[c]);
      }
    });
    (which ? *tau_v : *tau_k) = linear_quantile(y, clip_quantile);
  }
}

}  // namespace

extern "C" oscar_status oscar_build_rotation(int32_t d, int32_t n_kv_heads, int32_t group_q,
                                             int64_t n_rows, const float* q_calib,
                                             const float* k_calib, const float* v_calib,
                                             const float* o_calib, double clip_quantile,
                                             int32_t max_sweeps, int32_t n_threads, double* r_k,
                                             double* r_v, double* tau_k, double* tau_v,
                                             double* eig_k, double* eig_v) {
  using oscar::fail;
  oscar::clear_error();
  if (!q_calib || !k_calib || !v_calib || !r_k || !r_v || !tau_k || !tau_v)
    return fail(OSCAR_ERR_INVALID_ARG, "null required pointer");
  if (n_rows < 2 || n_kv_heads < 1) return fail(OSCAR_ERR_INVALID_ARG, "n_rows < 2 or n_kv_heads < 1");
  if (!(clip_quantile > 0.0 && clip_quantile <= 1.0))
    return fail(OSCAR_ERR_INVALID_ARG, "clip_quantile outside (0, 1]");
  if (d != 64 && d != 128) return fail(OSCAR_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (group_q < 1 || group_q > 16) return fail(OSCAR_ERR_UNSUPPORTED, "group_q outside [1, 16]");
  if (max_sweeps < 0) return fail(OSCAR_ERR_INVALID_ARG, "max_sweeps < 0");
  if (max_sweeps == 0) max_sweeps = 64;
  if (n_threads <= 0) n_threads = int(std::max(1u, std::thread::hardware_concurrency()));
  const int hq = n_kv_heads * group_q;
  const size_t N = size_t(n_rows);
  const size_t nq = N * hq * d, nkv = N * n_kv_heads * d;
  for (size_t i = 0; i < nq; ++i)
    if (!std::isfinite(q_calib[i]) || (o_calib && !std::isfinite(o_calib[i])))
      return fail(OSCAR_ERR_NUMERIC, "non-finite calibration value");
  for (size_t i = 0; i < nkv; ++i)
    if (!std::isfinite(k_calib[i]) || !std::isfinite(v_calib[i]))
      return fail(OSCAR_ERR_NUMERIC, "non-finite calibration value");

  std::vector<double> q(q_calib, q_calib + nq), k(k_calib, k_calib + nkv), v(v_calib, v_calib + nkv);
  std::vector<double> o;
  if (o_calib) {
    o.assign(o_calib, o_calib + nq);
  } else {
    // Causal calibration attention, tasks = (query head, block of 64 rows);
    // later blocks cost more, so hand them out first.
    o.assign(nq, 0.0);
    const int blk = 64;
    const int nblk = int((N + blk - 1) / blk);
    std::vector<std::vector<double>> scratch{static_cast<size_t>(n_threads)};
    run_parallel(n_threads, hq * nblk, [&](int t, int wid) {
      const int i = t % hq;
      const int b = nblk - 1 - t / hq;
      const int h = i / group_q;
      const int r0 = b * blk, r1 = int(std::min(N, size_t(r0 + blk)));
      causal_block(&q[size_t(i) * d], size_t(hq) * d, &k[size_t(h) * d], &v[size_t(h) * d],
                   size_t(n_kv_heads) * d, d, r0, r1, &o[size_t(i) * d], size_t(hq) * d,
                   scratch[size_t(wid)]);
    });
  }

  // Targets, eigenbases and rotations per KV head.
  std::vector<int> ok(n_kv_heads, 1);
  run_parallel(n_threads, 2 * n_kv_heads, [&](int t, int) {
    const int h = t / 2;
    const bool value = t % 2;
    const std::vector<double>& src = value ? o : q;
    std::vector<double> c(size_t(d) * d, 0.0);
    for (int i = h * group_q; i < (h + 1) * group_q; ++i)
      for (size_t n = 0; n < N; ++n) {
        const double* x = &src[(n * hq + i) * d];
        for (int a = 0; a < d; ++a) {
          const double xa = x[a];
          double* row = &c[size_t(a) * d];
          for (int b = 0; b < d; ++b) row[b] += xa * x[b];
        }
      }
    const double norm = 1.0 / (double(N) * group_q);
    for (double& x : c) x *= norm;
    if (!rotation_from_target(d, c, max_sweeps, (value ? r_v : r_k) + size_t(h) * d * d,
                              value ? eig_v : eig_k, h)) ok[h] = 0;
  });
  for (int h = 0; h < n_kv_heads; ++h)
    if (!ok[h]) return fail(OSCAR_ERR_NUMERIC, "Jacobi eigensolver did not converge");

  clip_thresholds(d, n_kv_heads, N, k, v, r_k, r_v, clip_quantile, n_threads, tau_k, tau_v);
  return OSCAR_OK;
}

extern "C" oscar_status oscar_build_fixed_rotation(int32_t variant, int32_t d, int32_t n_kv_heads, int64_t n_rows,
                                                   const float* k_calib, const float* v_calib,
                                                   double clip_quantile, int32_t n_threads, double* r_k,
                                                   double* r_v, double* tau_k, double* tau_v) {
  using oscar::fail;
  oscar::clear_error();
  if (!k_calib || !v_calib || !r_k || !r_v || !tau_k || !tau_v)
    return fail(OSCAR_ERR_INVALID_ARG, "null required pointer");
  if (variant != OSCAR_ROTATION_HADAMARD && variant != OSCAR_ROTATION_IDENTITY)
    return fail(OSCAR_ERR_INVALID_ARG, "unknown rotation variant");
  if (n_rows < 2 || n_kv_heads < 1) return fail(OSCAR_ERR_INVALID_ARG, "n_rows < 2 or n_kv_heads < 1");
  if (!(clip_quantile > 0.0 && clip_quantile <= 1.0))
    return fail(OSCAR_ERR_INVALID_ARG, "clip_quantile outside (0, 1]");
  if (d != 64 && d != 128) return fail(OSCAR_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (n_threads <= 0) n_threads = int(std::max(1u, std::thread::hardware_concurrency()));
  const size_t N = size_t(n_rows);
  const size_t nkv = N * n_kv_heads * d;
  for (size_t i = 0; i < nkv; ++i)
    if (!std::isfinite(k_calib[i]) || !std::isfinite(v_calib[i]))
      return fail(OSCAR_ERR_NUMERIC, "non-finite calibration value");
  // Hadamard-only: the fixed factor H . P_br of the composite rotation (U = I);
  // identity: no rotation
  std::vector<double> eye(size_t(d) * d, 0.0);
  for (int i = 0; i < d; ++i) eye[size_t(i) * d + i] = 1.0;
  std::vector<double> r(size_t(d) * d);
  if (variant == OSCAR_ROTATION_HADAMARD) compose_rotation(d, eye, r.data());
  else r = eye;
  for (int h = 0; h < n_kv_heads; ++h) {
    std::memcpy(r_k + size_t(h) * d * d, r.data(), sizeof(double) * d * d);
    std::memcpy(r_v + size_t(h) * d * d, r.data(), sizeof(double) * d * d);
  }
  std::vector<double> k(k_calib, k_calib + nkv), v(v_calib, v_calib + nkv);
  clip_thresholds(d, n_kv_heads, N, k, v, r_k, r_v, clip_quantile, n_threads, tau_k, tau_v);
  return OSCAR_OK;
}

extern "C" oscar_status oscar_build_rotation_from_targets(int32_t d, int32_t n_kv_heads, const double* c_q,
                                                          const double* c_s, int64_t n_rows, const float* k_calib,
                                                          const float* v_calib, double clip_quantile,
                                                          int32_t max_sweeps, int32_t n_threads, double* r_k,
                                                          double* r_v, double* tau_k, double* tau_v, double* eig_k,
                                                          double* eig_v) {
  using oscar::fail;
  oscar::clear_error();
  if (!c_q || !c_s || !k_calib || !v_calib || !r_k || !r_v || !tau_k || !tau_v)
    return fail(OSCAR_ERR_INVALID_ARG, "null required pointer");
  if (n_rows < 2 || n_kv_heads < 1) return fail(OSCAR_ERR_INVALID_ARG, "n_rows < 2 or n_kv_heads < 1");
  if (!(clip_quantile > 0.0 && clip_quantile <= 1.0))
    return fail(OSCAR_ERR_INVALID_ARG, "clip_quantile outside (0, 1]");
  if (d != 64 && d != 128) return fail(OSCAR_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (max_sweeps < 0) return fail(OSCAR_ERR_INVALID_ARG, "max_sweeps < 0");
  if (max_sweeps == 0) max_sweeps = 64;
  if (n_threads <= 0) n_threads = int(std::max(1u, std::thread::hardware_concurrency()));
  const size_t N = size_t(n_rows), nkv = N * n_kv_heads * d, nc = size_t(n_kv_heads) * d * d;
  for (size_t i = 0; i < nc; ++i)
    if (!std::isfinite(c_q[i]) || !std::isfinite(c_s[i])) return fail(OSCAR_ERR_NUMERIC, "non-finite target value");
  for (size_t i = 0; i < nkv; ++i)
    if (!std::isfinite(k_calib[i]) || !std::isfinite(v_calib[i]))
      return fail(OSCAR_ERR_NUMERIC, "non-finite calibration value");
  std::vector<int> ok(n_kv_heads, 1);
  run_parallel(n_threads, 2 * n_kv_heads, [&](int t, int) {
    const int h = t / 2;
    const bool value = t % 2;
    const double* src = (value ? c_s : c_q) + size_t(h) * d * d;
    // symmetric part (targets accumulated on the GPU may differ from
    // symmetry by rounding)
    std::vector<double> c(size_t(d) * d);
    for (int a = 0; a < d; ++a)
      for (int b = 0; b < d; ++b) c[size_t(a) * d + b] = 0.5 * (src[size_t(a) * d + b] + src[size_t(b) * d + a]);
    if (!rotation_from_target(d, c, max_sweeps, (value ? r_v : r_k) + size_t(h) * d * d, value ? eig_v : eig_k, h))
      ok[h] = 0;
  });
  for (int h = 0; h < n_kv_heads; ++h)
    if (!ok[h]) return fail(OSCAR_ERR_NUMERIC, "Jacobi eigensolver did not converge");
  std::vector<double> k(k_calib, k_calib + nkv), v(v_calib, v_calib + nkv);
  clip_thresholds(d, n_kv_heads, N, k, v, r_k, r_v, clip_quantile, n_threads, tau_k, tau_v);
  return OSCAR_OK;
}
