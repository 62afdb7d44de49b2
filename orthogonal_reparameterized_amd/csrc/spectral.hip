// Spectral diagnostics of a weight (the hyperspherical energy of its neurons and the entropy of its singular
// values), the metrics the POET pages monitor next to the spectrum-preservation claim (Experimental setup, Metrics).
//
// Both start from a Gram matrix formed in float64 from the float32 weight, so that nothing downstream is limited by
// the squaring of the spectrum a Gram matrix implies (a float32 Gram would lose the small singular values):
//   hyperspherical energy   C = W W^T (m x m); cos_ij = C_ij / sqrt(C_ii C_jj); per neuron
//                           E_i = sum_{j != i} (2 - 2 cos_ij)^(-s/2)   (||w^_i - w^_j||^2 = 2 - 2 cos_ij);
//   singular-value entropy  C = W^T W or W W^T, whichever is smaller (r = min(m, n)); C = Q T Q^T with T
//                           tridiagonal by r - 2 Householder reflections; the eigenvalues of T by Sturm-count
//                           bisection; sigma = sqrt(lambda); p = sigma / sum sigma; H = -sum p log p.
// Everything after the Gram runs in float64 on the vector units. The Gram kernel is a tiled float64 product over
// the upper-triangular tile pairs (C is symmetric, the lower tile is written as the transpose). The reductions are
// fixed-order trees, so results are deterministic.
#include <algorithm>
#include <cmath>

#include "../../include/poet.h"
#include "internal.h"

namespace poet {
namespace {

#define HIP_RET_LAST()                                \
  do {                                                \
    const hipError_t e_ = hipGetLastError();          \
    if (e_ != hipSuccess) return e_;                  \
  } while (0)

constexpr int GT = 64;   // Gram tile (GT x GT outputs per workgroup, 4 x 4 per thread)
constexpr int GK = 16;   // K chunk staged in LDS
constexpr int kThreads = 256;

// C[i][j] = sum_k A(i, k) A(j, k), with A(i, k) = W[i][k] (TRANS = false: C = W W^T, r = rows, K = cols) or
// W[k][i] (TRANS = true: C = W^T W, r = cols, K = rows). blockIdx.x enumerates tile pairs (ti <= tj).
template <bool TRANS>
__global__ __launch_bounds__(kThreads) void k_gram_f64(const float* __restrict__ W, int64_t ldw, int r, int K,
                                                       double* __restrict__ C, int64_t ldc) {
  __shared__ double As[GK][GT + 1];
  __shared__ double Bs[GK][GT + 1];
  const int nt = (r + GT - 1) / GT;
  int ti = 0, rem = blockIdx.x;
  while (rem >= nt - ti) { rem -= nt - ti; ++ti; }
  const int tj = ti + rem;
  const int i0 = ti * GT, j0 = tj * GT;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += GK) {
    for (int e = threadIdx.x; e < GK * GT; e += kThreads) {
      int kk, ii;
      if (TRANS) { kk = e / GT; ii = e % GT; } else { ii = e / GK; kk = e % GK; }
      const int k = k0 + kk, ia = i0 + ii, ib = j0 + ii;
      double a = 0.0, b = 0.0;
      if (k < K) {
        if (ia < r) a = TRANS ? W[(int64_t)k * ldw + ia] : W[(int64_t)ia * ldw + k];
        if (ib < r) b = TRANS ? W[(int64_t)k * ldw + ib] : W[(int64_t)ib * ldw + k];
      }
      As[kk][ii] = a;
      Bs[kk][ii] = b;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < GK; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { a[u] = As[kk][ty * 4 + u]; b[u] = Bs[kk][tx * 4 + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + ty * 4 + u, j = j0 + tx * 4 + v;
      if (i < r && j < r) {
        C[(int64_t)i * ldc + j] = acc[u][v];
        C[(int64_t)j * ldc + i] = acc[u][v];
      }
    }
}

// fixed-order tree sum of one value per thread over the workgroup; the result is returned to every thread
__device__ double block_sum(double x, double* red) {
  red[threadIdx.x] = x;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double s = red[0];
  __syncthreads();
  return s;
}

// E_i = sum_{j != i} (2 - 2 C_ij / sqrt(C_ii C_jj))^(-s/2), one workgroup per row
__global__ __launch_bounds__(kThreads) void k_he_rows(const double* __restrict__ C, int64_t ldc, int r, double s,
                                                      double* __restrict__ E) {
  __shared__ double red[kThreads];
  const int i = blockIdx.x;
  const double cii = C[(int64_t)i * ldc + i];
  double part = 0.0;
  for (int j = threadIdx.x; j < r; j += kThreads) {
    if (j == i) continue;
    const double cs = C[(int64_t)i * ldc + j] / sqrt(cii * C[(int64_t)j * ldc + j]);
    const double d2 = fmax(2.0 - 2.0 * cs, 0.0);
    part += pow(d2, -0.5 * s);
  }
  const double tot = block_sum(part, red);
  if (threadIdx.x == 0) E[i] = tot;
}

// out[0] = sum of x[0..n) (one workgroup, fixed order)
__global__ __launch_bounds__(kThreads) void k_sum_f64(const double* __restrict__ x, int n, double* __restrict__ out) {
  __shared__ double red[kThreads];
  double part = 0.0;
  for (int i = threadIdx.x; i < n; i += kThreads) part += x[i];
  const double tot = block_sum(part, red);
  if (threadIdx.x == 0) out[0] = tot;
}

// ---- Householder tridiagonalization of the symmetric r x r C, step k (0 <= k <= r - 3) -----------------------
// The reflector H = I - 2 u u^T (||u|| = 1) maps x = C[k][k+1..r) to (alpha, 0, ..., 0), alpha = -sign(x0) ||x||,
// with u = (x - alpha e_1) / ||x - alpha e_1||. Every workgroup of the step recomputes u from row k (which equals
// column k below the diagonal); workgroup 0 also stores u, d_k = C[k][k] and e_k = alpha.
__device__ void reflector(const double* __restrict__ C, int64_t ldc, int r, int k, double* red, double* x0,
                          double* alpha, double* vnorm) {
  const int L = r - k - 1;
  const double* row = C + (int64_t)k * ldc + k + 1;
  double part = 0.0;
  for (int j = threadIdx.x; j < L; j += kThreads) part += row[j] * row[j];
  const double sig2 = block_sum(part, red);
  *x0 = row[0];
  const double sig = sqrt(sig2);
  *alpha = *x0 >= 0.0 ? -sig : sig;
  // ||x - alpha e_1||^2 = sig^2 - 2 alpha x0 + alpha^2 = 2 sig^2 + 2 sig |x0|
  *vnorm = sqrt(2.0 * sig2 + 2.0 * sig * fabs(*x0));
}

__device__ __forceinline__ double u_at(const double* row, int j, double x0, double alpha, double vnorm) {
  return vnorm > 0.0 ? (j == 0 ? x0 - alpha : row[j]) / vnorm : 0.0;
}

constexpr int kTriRows = 16;  // trailing rows per workgroup

// p_i = sum_{j > k} C[i][j] u_j for the rows i in (k, r) of this workgroup; workgroup 0 writes u, d_k, e_k
__global__ __launch_bounds__(kThreads) void k_tri_matvec(const double* __restrict__ C, int64_t ldc, int r, int k,
                                                         double* __restrict__ u, double* __restrict__ p,
                                                         double* __restrict__ d, double* __restrict__ e) {
  __shared__ double red[kThreads];
  double x0, alpha, vnorm;
  reflector(C, ldc, r, k, red, &x0, &alpha, &vnorm);
  const int L = r - k - 1;
  const double* rowk = C + (int64_t)k * ldc + k + 1;
  if (blockIdx.x == 0) {
    for (int j = threadIdx.x; j < L; j += kThreads) u[j] = u_at(rowk, j, x0, alpha, vnorm);
    if (threadIdx.x == 0) {
      d[k] = C[(int64_t)k * ldc + k];
      e[k] = vnorm > 0.0 ? alpha : x0;  // x = 0: no reflection, the off-diagonal stays x0 (= 0)
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int q = wave; q < kTriRows; q += kThreads / 64) {
    const int i = blockIdx.x * kTriRows + q;  // trailing row index (row k + 1 + i)
    if (i >= L) break;
    const double* ri = C + (int64_t)(k + 1 + i) * ldc + k + 1;
    double s = 0.0;
    for (int j = lane; j < L; j += 64) s += ri[j] * u_at(rowk, j, x0, alpha, vnorm);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_down(s, off, 64);
    if (lane == 0) p[i] = s;
  }
}

// C[i][j] -= 2 (u_i w_j + w_i u_j) on the trailing block, w = p - (u^T p) u; row and column k are left as they are
// (later steps never read them again)
__global__ __launch_bounds__(kThreads) void k_tri_update(double* __restrict__ C, int64_t ldc, int r, int k,
                                                         const double* __restrict__ u, const double* __restrict__ p) {
  __shared__ double red[kThreads];
  const int L = r - k - 1;
  double part = 0.0;
  for (int j = threadIdx.x; j < L; j += kThreads) part += u[j] * p[j];
  const double K = block_sum(part, red);
  const int i0 = blockIdx.x * kTriRows;
  for (int q = 0; q < kTriRows; ++q) {
    const int i = i0 + q;
    if (i >= L) break;
    const double ui = u[i], wi = p[i] - K * ui;
    double* ri = C + (int64_t)(k + 1 + i) * ldc + k + 1;
    for (int j = threadIdx.x; j < L; j += kThreads) {
      const double uj = u[j], wj = p[j] - K * uj;
      ri[j] -= 2.0 * (ui * wj + wi * uj);
    }
  }
}

// the last diagonal and off-diagonal entries of T
__global__ void k_tri_last(const double* __restrict__ C, int64_t ldc, int r, double* __restrict__ d,
                           double* __restrict__ e) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  if (r >= 2) {
    d[r - 2] = C[(int64_t)(r - 2) * ldc + r - 2];
    e[r - 2] = C[(int64_t)(r - 2) * ldc + r - 1];
  }
  d[r - 1] = C[(int64_t)(r - 1) * ldc + r - 1];
}

// number of eigenvalues of the tridiagonal (d, e) below x (Sturm sequence of the LDL^T pivots)
__device__ int sturm_count(const double* __restrict__ d, const double* __restrict__ e, int r, double x, double tiny) {
  int cnt = 0;
  double q = d[0] - x;
  for (int j = 0;; ++j) {
    if (fabs(q) < tiny) q = -tiny;
    cnt += q < 0.0;
    if (j + 1 >= r) break;
    q = d[j + 1] - x - e[j] * e[j] / q;
  }
  return cnt;
}

// lam[t] = the t-th smallest eigenvalue of the tridiagonal (d, e), by bisection inside the Gershgorin interval
__global__ __launch_bounds__(kThreads) void k_bisect(const double* __restrict__ d, const double* __restrict__ e, int r,
                                                     double* __restrict__ lam) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= r) return;
  double lo = INFINITY, hi = -INFINITY, norm = 0.0;
  for (int j = 0; j < r; ++j) {
    const double rad = (j > 0 ? fabs(e[j - 1]) : 0.0) + (j + 1 < r ? fabs(e[j]) : 0.0);
    lo = fmin(lo, d[j] - rad);
    hi = fmax(hi, d[j] + rad);
  }
  norm = fmax(fabs(lo), fabs(hi));
  const double tiny = 1e-300 + 1e-30 * norm;
  lo -= 1e-12 * norm + 1e-300;
  hi += 1e-12 * norm + 1e-300;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;  // the interval is down to adjacent doubles
    if (sturm_count(d, e, r, mid, tiny) > t) hi = mid;
    else lo = mid;
  }
  lam[t] = 0.5 * (lo + hi);
}

// sigma = sqrt(max(lambda, 0)), p = sigma / sum sigma, out[0] = -sum p log p (one workgroup)
__global__ __launch_bounds__(kThreads) void k_sv_entropy(const double* __restrict__ lam, int r,
                                                         double* __restrict__ sigma, double* __restrict__ out) {
  __shared__ double red[kThreads];
  double part = 0.0;
  for (int t = threadIdx.x; t < r; t += kThreads) {
    const double sg = sqrt(fmax(lam[t], 0.0));
    if (sigma) sigma[r - 1 - t] = sg;  // descending, as an SVD lists them
    part += sg;
  }
  const double S = block_sum(part, red);
  part = 0.0;
  for (int t = threadIdx.x; t < r; t += kThreads) {
    const double pr = sqrt(fmax(lam[t], 0.0)) / S;
    if (pr > 0.0) part -= pr * log(pr);
  }
  const double H = block_sum(part, red);
  if (threadIdx.x == 0) out[0] = S > 0.0 ? H : 0.0;
}

int ntile_pairs(int r) {
  const int nt = (r + GT - 1) / GT;
  return nt * (nt + 1) / 2;
}

}  // namespace

hipError_t launch_gram_f64(const float* W, int64_t ldw, int rows, int cols, bool trans, double* C, int64_t ldc,
                           hipStream_t st) {
  const int r = trans ? cols : rows, K = trans ? rows : cols;
  if (r <= 0) return hipSuccess;
  ProfScope prof(POET_K_DIAG, st, 2.0 * r * r * K, 4.0 * rows * cols + 8.0 * r * r);
  if (trans) hipLaunchKernelGGL((k_gram_f64<true>), dim3(ntile_pairs(r)), dim3(kThreads), 0, st, W, ldw, r, K, C, ldc);
  else hipLaunchKernelGGL((k_gram_f64<false>), dim3(ntile_pairs(r)), dim3(kThreads), 0, st, W, ldw, r, K, C, ldc);
  return hipGetLastError();
}

hipError_t launch_he_rows(const double* C, int64_t ldc, int r, double s, double* E, double* total, hipStream_t st) {
  if (r <= 0) return hipSuccess;
  ProfScope prof(POET_K_DIAG, st, 0, 8.0 * r * r);
  hipLaunchKernelGGL(k_he_rows, dim3(r), dim3(kThreads), 0, st, C, ldc, r, s, E);
  HIP_RET_LAST();
  hipLaunchKernelGGL(k_sum_f64, dim3(1), dim3(kThreads), 0, st, E, r, total);
  return hipGetLastError();
}

hipError_t launch_sym_eig_entropy(double* C, int64_t ldc, int r, double* u, double* p, double* d, double* e,
                                  double* lam, double* sigma, double* entropy, hipStream_t st) {
  if (r <= 0) return hipSuccess;
  ProfScope prof(POET_K_DIAG, st, 0, 16.0 * r * (double)r * r / 3.0);
  for (int k = 0; k + 2 < r; ++k) {
    const int L = r - k - 1;
    const dim3 grid((L + kTriRows - 1) / kTriRows);
    hipLaunchKernelGGL(k_tri_matvec, grid, dim3(kThreads), 0, st, C, ldc, r, k, u, p, d, e);
    HIP_RET_LAST();
    hipLaunchKernelGGL(k_tri_update, grid, dim3(kThreads), 0, st, C, ldc, r, k, u, p);
    HIP_RET_LAST();
  }
  hipLaunchKernelGGL(k_tri_last, dim3(1), dim3(64), 0, st, C, ldc, r, d, e);
  HIP_RET_LAST();
  hipLaunchKernelGGL(k_bisect, dim3((r + kThreads - 1) / kThreads), dim3(kThreads), 0, st, d, e, r, lam);
  HIP_RET_LAST();
  hipLaunchKernelGGL(k_sv_entropy, dim3(1), dim3(kThreads), 0, st, lam, r, sigma, entropy);
  return hipGetLastError();
}

}  // namespace poet
