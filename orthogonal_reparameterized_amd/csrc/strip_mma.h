// Device helpers shared by the kernels that keep one square block (up to 256 x 256 bf16) resident in LDS and
// multiply it into a 64-column strip held transposed in LDS, four waves of 64 rows each
// (power_chain.hip, bs_apply.hip).
//
// LDS layout: rows of 512 B (256 bf16); the 16-byte chunk index of element k is XOR-ed with (row & 15), so the 16
// rows (or strip columns) that a 16-lane group reads at one logical chunk fall in 16 distinct bank groups.
// MFMA: v_mfma_f32_32x32x16_bf16. Operand A of lane l holds A[l % 32][8 (l / 32) + v], v = 0..7; operand B holds
// B[8 (l / 32) + v][l % 32]; accumulator register r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
#pragma once
#include "internal.h"

namespace poet {
namespace strip {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int MAXB = 256;        // largest block
constexpr int SW = 64;           // strip width
constexpr int ROWB = MAXB * 2;   // LDS row bytes
constexpr int NT = 256;          // threads per workgroup
constexpr int A_BYTES = MAXB * ROWB, X_BYTES = SW * ROWB;

__device__ __forceinline__ int loff(int row, int k) {  // byte offset of element k of LDS row `row`
  return row * ROWB + (((k >> 3) ^ (row & 15)) << 4) + (k & 7) * 2;
}
__device__ __forceinline__ void sts(char* base, int row, int k, __bf16 v) {
  *reinterpret_cast<__bf16*>(base + loff(row, k)) = v;
}
__device__ __forceinline__ __bf16 lds(const char* base, int row, int k) {
  return *reinterpret_cast<const __bf16*>(base + loff(row, k));
}

// K extent of the products for a block of size b: a multiple of 32 (LDS columns [b, kpad) must hold zeros)
__host__ __device__ inline int kpad_of(int b) { return (b + 31) / 32 * 32; }

__device__ __forceinline__ void zero(f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
}

// acc[a][b] += A[wr + 32a + (0..31)][0:kpad] . X[0:kpad][32b + (0..31)], with A row-major in Aq and X stored
// transposed in Xs (Xs row n = column n of X). Fragments of step ks+1 are read while step ks multiplies.
__device__ __forceinline__ void mma_strip(const char* Aq, const char* Xs, int wr, int kpad, int lane,
                                          f32x16 (&acc)[2][2]) {
  const int ra = wr + (lane & 31), rb = lane & 31, kh = (lane >> 5) * 8;
  const int ksteps = kpad / 16;  // even
  bf16x8 a0[2], b0[2], a1[2], b1[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    a0[t] = *reinterpret_cast<const bf16x8*>(Aq + loff(ra + 32 * t, kh));
    b0[t] = *reinterpret_cast<const bf16x8*>(Xs + loff(rb + 32 * t, kh));
  }
  for (int ks = 0; ks < ksteps; ks += 2) {
    const int k1 = (ks + 1) * 16 + kh;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      a1[t] = *reinterpret_cast<const bf16x8*>(Aq + loff(ra + 32 * t, k1));
      b1[t] = *reinterpret_cast<const bf16x8*>(Xs + loff(rb + 32 * t, k1));
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[a], b0[b], acc[a][b], 0, 0, 0);
    if (ks + 2 < ksteps) {
      const int k2 = (ks + 2) * 16 + kh;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a0[t] = *reinterpret_cast<const bf16x8*>(Aq + loff(ra + 32 * t, k2));
        b0[t] = *reinterpret_cast<const bf16x8*>(Xs + loff(rb + 32 * t, k2));
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[a], b1[b], acc[a][b], 0, 0, 0);
  }
}

// acc[a][b] += A[wr + 32a + (0..31)][0:kpad] . X[0:kpad][c0 + 32b + (0..31)] for NB column tiles (b < NB); the
// same pipelining as mma_strip.
template <int NB>
__device__ __forceinline__ void mma_strip_n(const char* Aq, const char* Xs, int wr, int c0, int kpad, int lane,
                                            f32x16 (&acc)[2][NB]) {
  const int ra = wr + (lane & 31), rb = c0 + (lane & 31), kh = (lane >> 5) * 8;
  const int ksteps = kpad / 16;  // even
  bf16x8 a0[2], b0[NB], a1[2], b1[NB];
#pragma unroll
  for (int t = 0; t < 2; ++t) a0[t] = *reinterpret_cast<const bf16x8*>(Aq + loff(ra + 32 * t, kh));
#pragma unroll
  for (int t = 0; t < NB; ++t) b0[t] = *reinterpret_cast<const bf16x8*>(Xs + loff(rb + 32 * t, kh));
  for (int ks = 0; ks < ksteps; ks += 2) {
    const int k1 = (ks + 1) * 16 + kh;
#pragma unroll
    for (int t = 0; t < 2; ++t) a1[t] = *reinterpret_cast<const bf16x8*>(Aq + loff(ra + 32 * t, k1));
#pragma unroll
    for (int t = 0; t < NB; ++t) b1[t] = *reinterpret_cast<const bf16x8*>(Xs + loff(rb + 32 * t, k1));
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[a], b0[b], acc[a][b], 0, 0, 0);
    if (ks + 2 < ksteps) {
      const int k2 = (ks + 2) * 16 + kh;
#pragma unroll
      for (int t = 0; t < 2; ++t) a0[t] = *reinterpret_cast<const bf16x8*>(Aq + loff(ra + 32 * t, k2));
#pragma unroll
      for (int t = 0; t < NB; ++t) b0[t] = *reinterpret_cast<const bf16x8*>(Xs + loff(rb + 32 * t, k2));
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[a], b1[b], acc[a][b], 0, 0, 0);
  }
}

// row / column (within the wave's 64 x 64 tile origin (wr, 0)) of accumulator register r of tile (a, b)
__device__ __forceinline__ int acc_row(int wr, int a, int r, int lane) { return wr + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }
__device__ __forceinline__ int acc_col(int b, int lane) { return b * 32 + (lane & 31); }

}  // namespace strip
}  // namespace poet
