// Exact Cayley primitives R = (I + Q)(I - Q)^{-1}, the map the truncated Cayley-Neumann series approximates
// ("Builds on ... Cayley parameterization", Experimental setup of the POET pages): an accuracy reference for the
// built primitives. With A = I - Q, (I + Q) A^{-1} = (2I - A) A^{-1} = 2 A^{-1} - I, so one inverse per primitive
// suffices. A's symmetric part is the identity (Q is skew), so Gauss-Jordan elimination needs no pivoting: every
// pivot is at least 1 in magnitude, and the growth is bounded for such matrices.
//
// One workgroup of 1024 threads per primitive (bp <= 256): thread (j, g) owns column j and the 64 rows
// 64 g .. 64 g + 63 of A (float32), the first 32 in registers and the other 32 in LDS (the thread's own slots,
// 128 KB for the workgroup; all 64 in registers would exceed the 128 VGPRs a 1024-thread workgroup leaves a
// wave). Step p of the in-place Gauss-Jordan inversion publishes the old row p and column p through LDS; then every
// owned element is updated from them:
//   A[p][p] <- 1/a,  A[p][j] <- A[p][j]/a,  A[i][p] <- -A[i][p]/a,  A[i][j] <- A[i][j] - A[i][p] A[p][j]/a,
// with a = A[p][p]. After bp steps the thread's elements hold A^{-1}; R = 2 A^{-1} - I is written row-major
// (coalesced over j). Padding rows and columns (a short last block) hold the identity throughout and come out as
// the identity.
#include "../../include/poet.h"
#include "internal.h"

namespace poet {
namespace {

constexpr int kCols = 256, kRowsPerThread = 64, kRegRows = 32, kThreads = 1024;

__device__ __forceinline__ float gj_update(float x, int i, int j, int piv, float cip, float inv, float rj) {
  if (i == piv) return j == piv ? inv : rj;
  if (j == piv) return -cip * inv;
  return x - cip * rj;
}

__global__ __launch_bounds__(kThreads) void k_cayley_exact(const float* __restrict__ theta, int mode, int d, int bp,
                                                           float* __restrict__ prim) {
  __shared__ float rowbuf[kCols];
  __shared__ float colbuf[kCols];
  __shared__ float spill[(kRowsPerThread - kRegRows) * kThreads];  // slot (v - kRegRows) * kThreads + thread
  const int p = blockIdx.x;
  const int c = prim_size(mode, d, bp, p);
  const int64_t toff = theta_off(bp, p);
  const int t = threadIdx.x, j = t & (kCols - 1), g = t / kCols;
  const int i0 = g * kRowsPerThread;
  float a[kRegRows];
  for (int v = 0; v < kRowsPerThread; ++v) {  // A = I - Q, Q_ij = theta(i, j) above the diagonal, -theta(j, i) below
    const int i = i0 + v;
    float q = 0.f;
    if (i < c && j < c && i != j) q = i < j ? theta[toff + tri_pos(i, j, c)] : -theta[toff + tri_pos(j, i, c)];
    const float x = (i == j ? 1.f : 0.f) - q;
    if (v < kRegRows) {
#pragma unroll
      for (int u = 0; u < kRegRows; ++u) a[u] = u == v ? x : a[u];
    } else {
      spill[(v - kRegRows) * kThreads + t] = x;
    }
  }
  for (int piv = 0; piv < bp; ++piv) {
    if (j == piv) {
#pragma unroll
      for (int v = 0; v < kRegRows; ++v) colbuf[i0 + v] = a[v];
      for (int v = kRegRows; v < kRowsPerThread; ++v) colbuf[i0 + v] = spill[(v - kRegRows) * kThreads + t];
    }
    if (g == piv / kRowsPerThread) {
      const int vp = piv % kRowsPerThread;
      float x = 0.f;
      if (vp < kRegRows) {
#pragma unroll
        for (int v = 0; v < kRegRows; ++v) x = v == vp ? a[v] : x;
      } else {
        x = spill[(vp - kRegRows) * kThreads + t];
      }
      rowbuf[j] = x;
    }
    __syncthreads();
    const float inv = 1.f / colbuf[piv];
    const float rj = rowbuf[j] * inv;  // the new row piv, off its pivot
#pragma unroll
    for (int v = 0; v < kRegRows; ++v) a[v] = gj_update(a[v], i0 + v, j, piv, colbuf[i0 + v], inv, rj);
    for (int v = kRegRows; v < kRowsPerThread; ++v) {
      float& x = spill[(v - kRegRows) * kThreads + t];
      x = gj_update(x, i0 + v, j, piv, colbuf[i0 + v], inv, rj);
    }
    __syncthreads();
  }
  if (j < bp) {
    float* out = prim + (int64_t)p * bp * bp;
#pragma unroll
    for (int v = 0; v < kRegRows; ++v) {
      const int i = i0 + v;
      if (i < bp) out[(int64_t)i * bp + j] = 2.f * a[v] - (i == j ? 1.f : 0.f);
    }
    for (int v = kRegRows; v < kRowsPerThread; ++v) {
      const int i = i0 + v;
      if (i < bp) out[(int64_t)i * bp + j] = 2.f * spill[(v - kRegRows) * kThreads + t] - (i == j ? 1.f : 0.f);
    }
  }
}

}  // namespace

hipError_t launch_cayley_exact(const float* theta, int mode, int d, int bp, int nprim, float* prim, hipStream_t st) {
  if (nprim <= 0) return hipSuccess;
  if (bp > kCols) return hipErrorInvalidValue;
  ProfScope prof(POET_K_CHAIN, st, 2.0 * bp * bp * (double)bp * nprim, (double)nprim * bp * bp * 6.0);
  hipLaunchKernelGGL(k_cayley_exact, dim3(nprim), dim3(kThreads), 0, st, theta, mode, d, bp, prim);
  return hipGetLastError();
}

}  // namespace poet
