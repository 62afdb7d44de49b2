// Sustained bf16 matrix-core rate of the device: every wave issues chains of v_mfma_f32_32x32x16_bf16 on register
// operands and nothing else (no memory traffic inside the loop), eight waves per workgroup (two per SIMD, as the
// token GEMM runs). Timed over a grid that fills every CU several times, it gives the rate the matrix cores sustain
// at the clock they hold under that load, the ceiling a GEMM can approach; in a counter run its
// SQ_VALU_MFMA_BUSY_CYCLES reads what "busy every cycle" looks like. A measurement aid, not part of the method.
#include "../../include/poet.h"
#include "internal.h"
#include "strip_mma.h"

namespace poet {
namespace {

using namespace strip;

constexpr int kWaves = 8;
constexpr int kChains = 4;  // independent accumulators per wave: enough to hide the issue-to-issue dependency

__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mfma_probe(int64_t iters,
                                                                                                    float* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16x8 a, b;
#pragma unroll
  for (int v = 0; v < 8; ++v) {  // small lane-dependent operands: the sums stay far from overflow
    a[v] = (__bf16)(1e-3f * (float)((lane + v) & 15));
    b[v] = (__bf16)(1e-3f * (float)((lane * 3 + v) & 7) - 4e-3f);
  }
  f32x16 c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = 0.f;
  for (int64_t t = 0; t < iters; ++t) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  if (lane == 0) out[(int64_t)blockIdx.x * kWaves + wave] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int64_t iters, int workgroups, float* out, hipStream_t st) {
  // one 32 x 32 x 16 product is 2 * 32 * 32 * 16 = 32768 flops
  const double flops = 32768.0 * kChains * (double)iters * kWaves * workgroups;
  ProfScope prof(POET_K_MISC, st, flops, 4.0 * kWaves * workgroups);
  hipLaunchKernelGGL(k_mfma_probe, dim3(workgroups), dim3(64 * kWaves), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace poet
