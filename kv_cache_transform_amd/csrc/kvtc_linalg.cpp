// Host dense linear algebra for calibration, fp64: blocked products and a
// symmetric eigensolver (Householder tridiagonalisation followed by the
// implicit symmetric QR iteration with Wilkinson shifts, as in Golub and Van
// Loan, "Matrix Computations", sections 8.3.1-8.3.3). There is no LAPACK on
// the target hosts, so these are written out here.
#include "kvtc_linalg.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace kvtc {

void parallel_for(int n, int threads, const std::function<void(int)>& fn) {
  if (threads <= 1 || n <= 1) {
    for (int i = 0; i < n; ++i) fn(i);
    return;
  }
  threads = std::min(threads, n);
  std::vector<std::thread> pool;
  std::atomic<int> next{0};
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&] {
      for (int i = next++; i < n; i = next++) fn(i);
    });
  for (auto& th : pool) th.join();
}

// C[i][j] (+)= sum_k A(i,k) * B[k][j] for i in [0,m), j in [0,n), k in [0,kk),
// with A(i,k) = A[i*sai + k*sak] and B row-major with leading dimension ldb,
// C row-major with leading dimension ldc. Blocked 4x8 register tiles; the
// (i, j) blocks of 64 x 256 are distributed over threads. When `upper` is set
// only blocks with j-block end > i-block start are computed (symmetric use).
void gemm_f64(int m, int n, int kk, const double* A, long sai, long sak, const double* B,
              long ldb, double* C, long ldc, bool upper, int threads) {
  constexpr int MC = 64, NC = 256, KC = 256;
  const int mb = (m + MC - 1) / MC, nb = (n + NC - 1) / NC;
  std::vector<std::pair<int, int>> blocks;
  for (int bi = 0; bi < mb; ++bi)
    for (int bj = 0; bj < nb; ++bj)
      if (!upper || (bj + 1) * NC > bi * MC) blocks.emplace_back(bi, bj);
  parallel_for((int)blocks.size(), threads, [&](int idx) {
    const int i0 = blocks[idx].first * MC, j0 = blocks[idx].second * NC;
    const int i1 = std::min(m, i0 + MC), j1 = std::min(n, j0 + NC);
    for (int i = i0; i < i1; ++i) std::memset(C + (long)i * ldc + j0, 0, sizeof(double) * (j1 - j0));
    for (int k0 = 0; k0 < kk; k0 += KC) {
      const int k1 = std::min(kk, k0 + KC);
      for (int i = i0; i < i1; i += 4) {
        const int ni = std::min(4, i1 - i);
        for (int j = j0; j < j1; j += 8) {
          const int nj = std::min(8, j1 - j);
          double acc[4][8] = {};
          if (ni == 4 && nj == 8) {
            for (int k = k0; k < k1; ++k) {
              const double* b = B + (long)k * ldb + j;
              const double a0 = A[(long)(i + 0) * sai + (long)k * sak];
              const double a1 = A[(long)(i + 1) * sai + (long)k * sak];
              const double a2 = A[(long)(i + 2) * sai + (long)k * sak];
              const double a3 = A[(long)(i + 3) * sai + (long)k * sak];
              for (int jj = 0; jj < 8; ++jj) {
                const double bv = b[jj];
                acc[0][jj] += a0 * bv;
                acc[1][jj] += a1 * bv;
                acc[2][jj] += a2 * bv;
                acc[3][jj] += a3 * bv;
              }
            }
          } else {
            for (int k = k0; k < k1; ++k)
              for (int ii = 0; ii < ni; ++ii) {
                const double a = A[(long)(i + ii) * sai + (long)k * sak];
                for (int jj = 0; jj < nj; ++jj) acc[ii][jj] += a * B[(long)k * ldb + j + jj];
              }
          }
          for (int ii = 0; ii < ni; ++ii)
            for (int jj = 0; jj < nj; ++jj) C[(long)(i + ii) * ldc + j + jj] += acc[ii][jj];
        }
      }
    }
  });
}

// ---------------------------------------------------------------------------
// Symmetric eigensolver.
//
// Step 1, Householder tridiagonalisation: for k = 0..n-3 a reflector
// H_k = I - beta v v^T with v[0..k] = 0 maps column k below the diagonal onto
// a multiple of e_{k+1}; A <- H_k A H_k is applied as the symmetric rank-2
// update A <- A - v w^T - w v^T with p = beta A v, w = p - (beta p^T v / 2) v.
// Q = H_0 H_1 ... H_{n-3} is accumulated afterwards, so A = Q T Q^T.
//
// Step 2, implicit symmetric QR with a Wilkinson shift on the tridiagonal T:
// each step chases a bulge down an unreduced block with plane rotations
// R = [[c, s], [-s, c]] acting on rows/columns (k, k+1); T <- R T R^T, and the
// eigenvector matrix Z <- Z R^T. Off-diagonals below eps * (|d_i| + |d_i+1|)
// are set to zero (deflation).
//
// Z is kept transposed (zt[j] is eigenvector j, contiguous) so that each
// rotation is a pass over two contiguous rows.
// ---------------------------------------------------------------------------
int sym_eigen(int n, std::vector<double>& a, std::vector<double>& evals,
              std::vector<double>& zt) {
  // a: n x n symmetric row-major, destroyed.
  std::vector<double> d(n), e(std::max(n - 1, 1), 0.0);
  std::vector<double> betas(n, 0.0);
  std::vector<double> vs((size_t)n * n, 0.0);  // reflector k stored in row k
  std::vector<double> p(n), w(n);
  for (int k = 0; k + 2 < n; ++k) {
    const int m = k + 1;
    double sigma = 0.0;
    for (int i = m + 1; i < n; ++i) sigma += a[(size_t)i * n + k] * a[(size_t)i * n + k];
    const double x0 = a[(size_t)m * n + k];
    double* v = vs.data() + (size_t)k * n;
    if (sigma == 0.0) {
      e[k] = x0;
      betas[k] = 0.0;
      continue;
    }
    const double mu = std::sqrt(x0 * x0 + sigma);
    // v = x - alpha e1 with alpha = -sign(x0) * mu (no cancellation).
    const double alpha = x0 >= 0 ? -mu : mu;
    v[m] = x0 - alpha;
    for (int i = m + 1; i < n; ++i) v[i] = a[(size_t)i * n + k];
    double vtv = v[m] * v[m] + sigma;
    const double beta = 2.0 / vtv;
    betas[k] = beta;
    e[k] = alpha;
    // p = beta * A[m:, m:] v
    for (int i = m; i < n; ++i) {
      const double* ai = a.data() + (size_t)i * n;
      double s = 0.0;
      for (int j = m; j < n; ++j) s += ai[j] * v[j];
      p[i] = beta * s;
    }
    double ptv = 0.0;
    for (int i = m; i < n; ++i) ptv += p[i] * v[i];
    const double half = 0.5 * beta * ptv;
    for (int i = m; i < n; ++i) w[i] = p[i] - half * v[i];
    for (int i = m; i < n; ++i) {
      double* ai = a.data() + (size_t)i * n;
      const double vi = v[i], wi = w[i];
      for (int j = m; j < n; ++j) ai[j] -= vi * w[j] + wi * v[j];
    }
  }
  for (int i = 0; i < n; ++i) d[i] = a[(size_t)i * n + i];
  if (n >= 2) e[n - 2] = a[(size_t)(n - 1) * n + (n - 2)];
  // Q = H_0 (H_1 (... (H_{n-3} I))): apply the reflectors from the left in
  // reverse order, then store the columns of Q as the rows of zt.
  std::vector<double> q((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) q[(size_t)i * n + i] = 1.0;
  for (int k = n - 3; k >= 0; --k) {
    const double beta = betas[k];
    if (beta == 0.0) continue;
    const double* v = vs.data() + (size_t)k * n;
    const int m = k + 1;
    // Q <- H_k Q touches rows m.. of Q; column j: q[:, j] -= beta v (v^T q[:, j])
    std::vector<double> t(n, 0.0);
    for (int i = m; i < n; ++i) {
      const double vi = v[i];
      const double* qi = q.data() + (size_t)i * n;
      for (int j = 0; j < n; ++j) t[j] += vi * qi[j];
    }
    for (int i = m; i < n; ++i) {
      const double f = beta * v[i];
      double* qi = q.data() + (size_t)i * n;
      for (int j = 0; j < n; ++j) qi[j] -= f * t[j];
    }
  }
  zt.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) zt[(size_t)j * n + i] = q[(size_t)i * n + j];

  // Implicit symmetric QR on (d, e).
  const double eps = std::numeric_limits<double>::epsilon();
  double anorm = 0.0;
  for (int i = 0; i < n; ++i)
    anorm = std::max(anorm, std::fabs(d[i]) + (i + 1 < n ? std::fabs(e[i]) : 0.0) +
                                (i > 0 ? std::fabs(e[i - 1]) : 0.0));
  // An off-diagonal is negligible relative to its neighbours, or below the
  // backward error the tridiagonalisation already made (eps * ||A||).
  auto small = [&](int i) {
    const double ae = std::fabs(e[i]);
    return ae <= eps * (std::fabs(d[i]) + std::fabs(d[i + 1])) || ae <= eps * anorm * 1e-3;
  };
  long iters = 0;
  const long max_iters = 60L * n + 100;
  int hi = n - 1;
  while (hi > 0) {
    if (small(hi - 1)) {
      e[hi - 1] = 0.0;
      --hi;
      continue;
    }
    int lo = hi - 1;
    while (lo > 0 && !small(lo - 1)) --lo;
    if (++iters > max_iters) return -1;
    // Wilkinson shift from the trailing 2x2 block.
    const double delta = 0.5 * (d[hi - 1] - d[hi]);
    const double b = e[hi - 1];
    const double den = delta + std::copysign(std::hypot(delta, b), delta == 0.0 ? 1.0 : delta);
    const double mu = d[hi] - b * b / den;
    double x = d[lo] - mu, z = e[lo];
    for (int k = lo; k < hi; ++k) {
      const double r = std::hypot(x, z);
      double c = 1.0, s = 0.0;
      if (r != 0.0) {
        c = x / r;
        s = z / r;
      }
      if (k > lo) e[k - 1] = r;
      const double dk = d[k], dk1 = d[k + 1], ek = e[k];
      d[k] = c * c * dk + 2.0 * c * s * ek + s * s * dk1;
      d[k + 1] = s * s * dk - 2.0 * c * s * ek + c * c * dk1;
      e[k] = (c * c - s * s) * ek + c * s * (dk1 - dk);
      if (k + 1 < hi) {
        z = s * e[k + 1];
        e[k + 1] = c * e[k + 1];
        x = e[k];
      }
      double* zk = zt.data() + (size_t)k * n;
      double* zk1 = zt.data() + (size_t)(k + 1) * n;
      for (int j = 0; j < n; ++j) {
        const double u = zk[j], v = zk1[j];
        zk[j] = c * u + s * v;
        zk1[j] = -s * u + c * v;
      }
    }
  }
  evals = d;
  return 0;
}

}  // namespace kvtc
