// Generic batched MFMA GEMM for gfx950, used for every dense contraction of the POET layer that is not a
// token GEMM: the Cayley-Neumann power chain, its adjoint, applying block-diagonal or gathered factors to W0,
// and the primitive-gradient contractions. Operands may be float32 or bf16 in global memory in either
// orientation; they are converted to the MFMA operand type while staged into LDS (K-contiguous per row), so
// each lane reads its MFMA fragment as one vector.
//
// Wave layout: 4 waves per workgroup in a 2 x 2 grid, each wave owns a (BM/2) x (BN/2) sub-tile made of
// 32 x 32 MFMA tiles. Output fragment of a 32 x 32 MFMA: accumulator r of lane l holds
// C[(r/4)*8 + (l/32)*4 + r%4][l%32].
#include "internal.h"

namespace poet {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float ld_elem(const void* p, int dt, int64_t i) {
  return dt == BF16 ? (float)(reinterpret_cast<const __bf16*>(p)[i]) : reinterpret_cast<const float*>(p)[i];
}

template <bool MMA_BF16>
struct Cfg;
template <>
struct Cfg<true> {
  using T = __bf16;
  static constexpr int BK = 32, PAD = 8, KSTEP = 16;
};
template <>
struct Cfg<false> {
  using T = float;
  static constexpr int BK = 16, PAD = 1, KSTEP = 2;
};

template <int BM, int BN, bool MMA_BF16, bool AK, bool BKM>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const GemmDesc g) {
  using C = Cfg<MMA_BF16>;
  using TL = typename C::T;
  constexpr int BK = C::BK, LDK = C::BK + C::PAD;
  constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 tiles per wave in M and N
  __shared__ __attribute__((aligned(16))) TL As[BM * LDK];
  __shared__ __attribute__((aligned(16))) TL Bs[BN * LDK];

  const int z = blockIdx.z;
  int M = g.M, N = g.N, K = g.K;
  if (g.Mtot > 0) M = min(M, g.Mtot - z * g.M);
  if (g.Ntot > 0) N = min(N, g.Ntot - z * g.N);
  if (g.Ktot > 0) K = min(K, g.Ktot - z * g.K);
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  if (m0 >= M || n0 >= N) return;  // uniform per workgroup

  const size_t asz = dtype_size(g.a_dt), bsz = dtype_size(g.b_dt);
  const char* Ab = reinterpret_cast<const char*>(g.A) + (size_t)(z * g.sA) * asz;
  const char* Bb = reinterpret_cast<const char*>(g.B) + (size_t)(z * g.sB) * bsz;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    // stage A tile (BM x BK) as As[i][k]
    for (int e = tid; e < BM * BK; e += 256) {
      int i, kk;
      if (AK) { i = e / BK; kk = e % BK; } else { kk = e / BM; i = e % BM; }
      const int gi = m0 + i, gk = k0 + kk;
      float v = 0.f;
      if (gi < M && gk < K) {
        v = ld_elem(Ab, g.a_dt, AK ? (int64_t)gi * g.lda + gk : (int64_t)gk * g.lda + gi);
        if (g.a_sub_eye && gi == gk) v -= 1.f;
      }
      As[i * LDK + kk] = (TL)v;
    }
    // stage B tile (BK x BN) as Bs[j][k]
    for (int e = tid; e < BN * BK; e += 256) {
      int j, kk;
      if (BKM) { j = e / BK; kk = e % BK; } else { kk = e / BN; j = e % BN; }
      const int gj = n0 + j, gk = k0 + kk;
      float v = 0.f;
      if (gj < N && gk < K) {
        v = ld_elem(Bb, g.b_dt, BKM ? (int64_t)gj * g.ldb + gk : (int64_t)gk * g.ldb + gj);
        if (g.b_sub_eye && gj == gk) v -= 1.f;
      }
      Bs[j * LDK + kk] = (TL)v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += C::KSTEP) {
      if constexpr (MMA_BF16) {
        bf16x8 af[TM], bfr[TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
          af[a] = *reinterpret_cast<const bf16x8*>(&As[(wm + a * 32 + (lane & 31)) * LDK + ks + (lane >> 5) * 8]);
#pragma unroll
        for (int b = 0; b < TN; ++b)
          bfr[b] = *reinterpret_cast<const bf16x8*>(&Bs[(wn + b * 32 + (lane & 31)) * LDK + ks + (lane >> 5) * 8]);
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
      } else {
        float af[TM], bfr[TN];
#pragma unroll
        for (int a = 0; a < TM; ++a) af[a] = As[(wm + a * 32 + (lane & 31)) * LDK + ks + (lane >> 5)];
#pragma unroll
        for (int b = 0; b < TN; ++b) bfr[b] = Bs[(wn + b * 32 + (lane & 31)) * LDK + ks + (lane >> 5)];
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], bfr[b], acc[a][b], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue
  const int64_t zc = (int64_t)z * g.sC, zd = (int64_t)z * g.sD, za = (int64_t)z * g.sAcc;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int j = n0 + wn + b * 32 + (lane & 31);
        if (i < M && j < N) {
          float out = g.alpha * acc[a][b][r];
          if (g.D) out += g.beta * g.D[zd + (int64_t)i * g.ldd + j];
          if (g.E) out += (float)reinterpret_cast<const __bf16*>(g.E)[(int64_t)z * g.sE + (int64_t)i * g.lde + j];
          if (g.C) {
            const int64_t ci = zc + (int64_t)i * g.ldc + j;
            if (g.c_dt == BF16) reinterpret_cast<__bf16*>(g.C)[ci] = (__bf16)out;
            else reinterpret_cast<float*>(g.C)[ci] = out;
          }
          if (g.C2) {
            const int64_t ci = (int64_t)z * g.sC2 + (int64_t)i * g.ldc2 + j;
            if (g.c2_dt == BF16) reinterpret_cast<__bf16*>(g.C2)[ci] = (__bf16)out;
            else reinterpret_cast<float*>(g.C2)[ci] = out;
          }
          if (g.Acc) g.Acc[za + (int64_t)i * g.ldacc + j] += g.gamma * out;
        }
      }
}

template <int BM, int BN, bool MMA_BF16>
hipError_t launch_t(const GemmDesc& g, hipStream_t st) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch);
  dim3 block(256);
  if (g.a_kmajor && g.b_kmajor) hipLaunchKernelGGL((gemm_generic_kernel<BM, BN, MMA_BF16, true, true>), grid, block, 0, st, g);
  else if (g.a_kmajor) hipLaunchKernelGGL((gemm_generic_kernel<BM, BN, MMA_BF16, true, false>), grid, block, 0, st, g);
  else if (g.b_kmajor) hipLaunchKernelGGL((gemm_generic_kernel<BM, BN, MMA_BF16, false, true>), grid, block, 0, st, g);
  else hipLaunchKernelGGL((gemm_generic_kernel<BM, BN, MMA_BF16, false, false>), grid, block, 0, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmDesc& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (fast_gemm_eligible(g)) return launch_fast_gemm(g, st);
  return launch_generic_gemm(g, st);
}

hipError_t launch_generic_gemm(const GemmDesc& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  const double mn = (double)g.M * g.N, bt = g.batch;
  const double bytes = bt * ((double)g.M * g.K * dtype_size(g.a_dt) + (double)g.K * g.N * dtype_size(g.b_dt) +
                             (g.C ? mn * dtype_size(g.c_dt) : 0.0) + (g.C2 ? mn * dtype_size(g.c2_dt) : 0.0) + (g.D ? mn * 4.0 : 0.0) + (g.E ? mn * 2.0 : 0.0) + (g.Acc ? mn * 8.0 : 0.0));
  ProfScope prof(g.kclass, st, 2.0 * mn * g.K * bt, bytes);
  const bool small = g.M <= 64 || g.N <= 64;
  if (g.compute == BF16) return small ? launch_t<64, 64, true>(g, st) : launch_t<128, 128, true>(g, st);
  return small ? launch_t<64, 64, false>(g, st) : launch_t<128, 128, false>(g, st);
}

}  // namespace poet
