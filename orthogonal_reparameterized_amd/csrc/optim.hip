// Optimizer step on the packed skew parameters: AdamW (Loshchilov and Hutter, "Decoupled Weight Decay
// Regularization", ICLR 2019), elementwise over every parameter of up to MAXG sides in one launch, and the reset of
// its moments at merge-then-reinitialize. Purely HBM-bound: a parameter reads theta, its gradient and both moments
// (16 bytes) and writes theta and the moments back (12 bytes); each thread moves four adjacent parameters with
// 16-byte accesses where the side's buffers allow it.
#include <algorithm>

#include "../../include/poet.h"
#include "internal.h"

namespace poet {
namespace {

constexpr int kThreads = 256;

struct AdamArgs {
  int n = 0;
  OptSide s[MAXG];
  float lr = 0.f, b1 = 0.f, b2 = 0.f, eps = 0.f, wd = 0.f;
  float inv_bc1 = 1.f, inv_bc2 = 1.f;  // 1 / (1 - beta^t) of the bias corrections
  int vec[MAXG];                       // 1: the side's four buffers are 16-byte aligned
};

__device__ __forceinline__ void adam_one(float& th, float g, float& m, float& v, const AdamArgs& a) {
  m = a.b1 * m + (1.f - a.b1) * g;
  v = a.b2 * v + (1.f - a.b2) * g * g;
  const float mhat = m * a.inv_bc1, vhat = v * a.inv_bc2;
  th = th - a.lr * (mhat / (sqrtf(vhat) + a.eps) + a.wd * th);
}

// blockIdx.y = side; a grid-stride loop over groups of four parameters
__global__ __launch_bounds__(kThreads) void k_adamw(const AdamArgs a) {
  const OptSide& s = a.s[blockIdx.y];
  float* __restrict__ th = s.theta;
  const float* __restrict__ gr = s.grad;
  float* __restrict__ mm = s.m;
  float* __restrict__ vv = s.v;
  const int64_t n = s.n;
  const int64_t n4 = a.vec[blockIdx.y] ? n / 4 : 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += stride) {
    float4 t = reinterpret_cast<float4*>(th)[q];
    const float4 g = reinterpret_cast<const float4*>(gr)[q];
    float4 m = reinterpret_cast<float4*>(mm)[q];
    float4 v = reinterpret_cast<float4*>(vv)[q];
    adam_one(t.x, g.x, m.x, v.x, a);
    adam_one(t.y, g.y, m.y, v.y, a);
    adam_one(t.z, g.z, m.z, v.z, a);
    adam_one(t.w, g.w, m.w, v.w, a);
    reinterpret_cast<float4*>(th)[q] = t;
    reinterpret_cast<float4*>(mm)[q] = m;
    reinterpret_cast<float4*>(vv)[q] = v;
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float t = th[i], m = mm[i], v = vv[i];
    adam_one(t, gr[i], m, v, a);
    th[i] = t;
    mm[i] = m;
    vv[i] = v;
  }
}

// m, v <- 0 for every side (blockIdx.y = side)
__global__ __launch_bounds__(kThreads) void k_zero2(const AdamArgs a) {
  const OptSide& s = a.s[blockIdx.y];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < s.n; i += stride) {
    s.m[i] = 0.f;
    s.v[i] = 0.f;
  }
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

dim3 opt_grid(const OptGroup& g) {
  int64_t most = 0;
  for (int i = 0; i < g.n; ++i) most = std::max<int64_t>(most, g.s[i].n);
  const int64_t want = (most / 4 + kThreads - 1) / kThreads;
  return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 1024)), g.n);
}

}  // namespace

hipError_t launch_adamw_group(const OptGroup& g, float lr, float b1, float b2, float eps, float wd, double inv_bc1,
                              double inv_bc2, hipStream_t st) {
  if (g.n <= 0) return hipSuccess;
  if (g.n > MAXG) return hipErrorInvalidValue;
  AdamArgs a;
  a.n = g.n;
  double bytes = 0;
  for (int i = 0; i < g.n; ++i) {
    a.s[i] = g.s[i];
    a.vec[i] = al16(g.s[i].theta) && al16(g.s[i].grad) && al16(g.s[i].m) && al16(g.s[i].v);
    bytes += 28.0 * g.s[i].n;
  }
  a.lr = lr; a.b1 = b1; a.b2 = b2; a.eps = eps; a.wd = wd;
  a.inv_bc1 = (float)inv_bc1; a.inv_bc2 = (float)inv_bc2;
  ProfScope prof(POET_K_OPTIM, st, 0, bytes);
  hipLaunchKernelGGL(k_adamw, opt_grid(g), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_moments_reset_group(const OptGroup& g, hipStream_t st) {
  if (g.n <= 0) return hipSuccess;
  if (g.n > MAXG) return hipErrorInvalidValue;
  AdamArgs a;
  a.n = g.n;
  double bytes = 0;
  for (int i = 0; i < g.n; ++i) {
    a.s[i] = g.s[i];
    bytes += 8.0 * g.s[i].n;
  }
  ProfScope prof(POET_K_OPTIM, st, 0, bytes);
  hipLaunchKernelGGL(k_zero2, opt_grid(g), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace poet
