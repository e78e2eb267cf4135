// Host dense linear algebra used by calibration (fp64).
#pragma once

#include <atomic>
#include <functional>
#include <limits>
#include <vector>

namespace kvtc {

// Run fn(0..n-1) over up to `threads` std::threads (dynamic assignment).
void parallel_for(int n, int threads, const std::function<void(int)>& fn);

// C = A * B with A(i,k) = A[i*sai + k*sak]; see kvtc_linalg.cpp.
void gemm_f64(int m, int n, int kk, const double* A, long sai, long sak, const double* B,
              long ldb, double* C, long ldc, bool upper, int threads);

// Eigen-decomposition of a symmetric n x n matrix `a` (row-major, destroyed):
// evals[j] and eigenvector zt[j*n .. j*n+n) (unsorted). Returns 0 on success,
// -1 if the QR iteration did not converge.
int sym_eigen(int n, std::vector<double>& a, std::vector<double>& evals, std::vector<double>& zt);

}  // namespace kvtc
