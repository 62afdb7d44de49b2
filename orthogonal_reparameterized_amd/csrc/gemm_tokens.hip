// Token GEMMs of the POET layer on gfx950 bf16 MFMA (float32 accumulation):
//   forward           Y  = X  W^T   (A = X  K-major, B = W  K-major)
//   input gradient    dX = dY W     (A = dY K-major, B = W  N-major)
//   weight gradient   G  = dY^T X   (A = dY M-major, B = X  N-major; K = tokens)
//
// Workgroup tile 256 x 256 x 64, 4 waves in a 2 x 2 grid, each wave 128 x 128 as 4 x 4 v_mfma_f32_32x32x16_bf16.
// Operands go straight from global memory into LDS (global_load_lds_dwordx4: lane l of a wave writes the 16
// bytes at the wave's LDS base + 16 l, from any global address it chooses), in a two-stage ring: the DMA of
// K-tile t+1 runs while the MFMAs consume tile t, one barrier per tile. Both stage layouts are 32 KB:
//   K-major operand: 256 rows x 128 B; the 16-byte chunk index is XOR-ed with f(row mod 32) =
//     (row & 7) ^ ((row >> 3) & 3): 16 consecutive rows read at one logical chunk hit 16 distinct 16-byte bank
//     groups, so the ds_read_b128 fragments are conflict-free;
//   M/N-major operand: 64 k-rows x 512 B; the 64-byte block index is XOR-ed with (k-row & 3), so the 4 k-rows a
//     16-lane group reads with ds_read_b64_tr_b16 fall in 4 different 64-byte bank windows (in each 16-lane
//     group, lane j supplies the address of 4 consecutive elements of k-row j/4; lane i receives the elements
//     of column i of those 4 k-rows: an MFMA fragment of the transposed operand).
// Rows or columns past M / N are fetched from a clamped (valid) address: they only reach outputs that are
// never stored. The K tail of the last tile is zeroed in LDS after its DMA lands.
// Tiles are assigned XCD-aware: workgroup id w runs on XCD w % 8, so each XCD takes a contiguous range of the
// row-major tile order and neighbouring tiles on one XCD share their A rows in that XCD's L2.
#include "internal.h"

namespace poet {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = 256 * BK * 2;  // bytes of one operand's stage (both layouts)

__device__ __forceinline__ int swz(int r32) { return (r32 & 7) ^ ((r32 >> 3) & 3); }

// Direct global->LDS DMA of one 256 x 64 operand tile. Per-thread source offsets are fixed for the K loop.
template <bool KMAJ>
struct Operand {
  const char* base;  // operand base (bytes)
  uint32_t ld2;      // leading dimension in bytes
  int R, K;
  uint32_t off[8];   // byte offset of this lane's source for DMA instruction j: row base (K-major) / column
  int chk;           // K-major: logical 16-byte chunk this lane fetches

  __device__ __forceinline__ void init(const __bf16* b, int64_t ld, int r0, int R_, int K_, int wave, int lane) {
    base = reinterpret_cast<const char*>(b);
    ld2 = (uint32_t)(ld * 2);
    R = R_; K = K_;
    if constexpr (KMAJ) {
      // instruction j of wave w fills rows 8 (4 j + w) + lane / 8, physical chunk lane % 8, whose logical
      // chunk (k offset / 8 inside the tile) is chk
      const int r32 = 8 * wave + (lane >> 3);
      chk = (lane & 7) ^ swz(r32);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = min(r0 + 32 * j + r32, R - 1);
        off[j] = (uint32_t)row * ld2;
      }
    } else {
      // instruction j of wave w fills k-rows 2 (4 j + w) + lane / 32, physical 16-byte chunk lane % 32
      const int pc = lane & 31;
      const int kr4 = (2 * wave + (lane >> 5)) & 3;
      const int lch = (((pc >> 2) ^ kr4) << 2) | (pc & 3);
      const int rmax = ((R + 7) / 8) * 8 - 8;
      const int col = min(r0 + lch * 8, rmax);
      chk = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) off[j] = (uint32_t)col * 2;  // k-row added per tile
    }
  }

  __device__ __forceinline__ void dma(char* __restrict__ st, int k0, int wave, int lane) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      char* dst = st + (4 * j + wave) * 1024;
      uint32_t o;
      if constexpr (KMAJ) {
        const int kmax = ((K + 7) / 8) * 8 - 8;  // keep the 16-byte read inside the row's first ceil8(K) elements
        o = off[j] + (uint32_t)min(k0 + 8 * chk, kmax) * 2;
      } else {
        const int kr = min(k0 + 2 * (4 * j + wave) + (lane >> 5), K - 1);
        o = off[j] + (uint32_t)kr * ld2;
      }
      __builtin_amdgcn_global_load_lds((gbl_void*)(base + o), (lds_void*)dst, 16, 0, 0);
    }
  }

  // zero the part of a staged tile that lies at k >= K (kv = K - k0 valid k values, 0 < kv < 64)
  __device__ __forceinline__ void zero_tail(char* __restrict__ st, int kv, int tid) const {
    if constexpr (KMAJ) {
      const int row = tid, s = swz(row & 31);
      for (int k = kv; k < BK; ++k)
        *reinterpret_cast<short*>(st + row * 128 + (((k >> 3) ^ s) << 4) + (k & 7) * 2) = 0;
    } else {
      for (int e = kv * 32 + tid; e < BK * 32; e += 256)
        *reinterpret_cast<u32x4*>(st + e * 16) = u32x4{0, 0, 0, 0};
    }
  }
};

// MFMA operand fragment for rows [rb, rb + 32) (rb a multiple of 32) and k-step ks of a staged tile.
template <bool KMAJ>
__device__ __forceinline__ bf16x8 frag(const char* __restrict__ st, int rb, int ks, int lane) {
  if constexpr (KMAJ) {
    const int r32 = lane & 31;
    const int ch = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(st + (rb + r32) * 128 + ((ch ^ swz(r32)) << 4));
  } else {
    const int j = lane & 15;
    const int kr = ks * 16 + (lane >> 5) * 8 + (j >> 2);
    const int within = ((lane >> 4) & 1) * 32 + (j & 3) * 8;
    const int blk = (rb >> 5) ^ (j >> 2);
    const char* p = st + kr * 512 + blk * 64 + within;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 512));
    const i16x8 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, c);
  }
}

template <bool AK, bool BK_>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_tok_kernel(const TokGemm p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * STAGE];

  const int ntn = (p.N + BN - 1) / BN, ntm = (p.M + BM - 1) / BM, ntiles = ntm * ntn;
  const int per = (ntiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= ntiles) return;
  const int m0 = (t / ntn) * BM, n0 = (t % ntn) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;

  Operand<AK> oa;
  Operand<BK_> ob;
  oa.init(p.A, p.lda, m0, p.M, p.K, wave, lane);
  ob.init(p.B, p.ldb, n0, p.N, p.K, wave, lane);

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = (p.K + BK - 1) / BK;
  if (nk > 0) {
    oa.dma(smem, 0, wave, lane);
    ob.dma(smem + STAGE, 0, wave, lane);
  }
  for (int kt = 0; kt < nk; ++kt) {
    char* sa = smem + (kt & 1) * 2 * STAGE;
    char* sb = sa + STAGE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int kv = p.K - kt * BK;
    if (kv < BK) {  // last, partial K tile
      oa.zero_tail(sa, kv, tid);
      ob.zero_tail(sb, kv, tid);
      __syncthreads();
    }
    if (kt + 1 < nk) {
      char* na = smem + ((kt + 1) & 1) * 2 * STAGE;
      oa.dma(na, (kt + 1) * BK, wave, lane);
      ob.dma(na + STAGE, (kt + 1) * BK, wave, lane);
    }
    // fragments of k-step ks + 1 are read from LDS while the 16 MFMAs of k-step ks run
    bf16x8 fa[2][4], fb[2][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) fa[0][a] = frag<AK>(sa, wr + a * 32, 0, lane);
#pragma unroll
    for (int b = 0; b < 4; ++b) fb[0][b] = frag<BK_>(sb, wc + b * 32, 0, lane);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int a = 0; a < 4; ++a) fa[c ^ 1][a] = frag<AK>(sa, wr + a * 32, ks + 1, lane);
#pragma unroll
        for (int b = 0; b < 4; ++b) fb[c ^ 1][b] = frag<BK_>(sb, wc + b * 32, ks + 1, lane);
      }
      // the next k-step's LDS reads stay ahead of this k-step's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][a], fb[c][b], acc[a][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: accumulator r of lane l in a 32x32 tile is C[(r/4)*8 + (l/32)*4 + r%4][l%32]
  const int row0 = m0 + wr + (lane >> 5) * 4, col0 = n0 + wc + (lane & 31);
  const int rlim = p.M - row0, clim = p.N - col0;
  const int64_t ldc = p.ldc;
  if (p.c_f32) {
    float* cb = reinterpret_cast<float*>(p.C) + (int64_t)row0 * ldc + col0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = a * 32 + (r >> 2) * 8 + (r & 3);
        if (dr < rlim) {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (b * 32 < clim) cb[dr * ldc + b * 32] = acc[a][b][r];
        }
      }
  } else {
    __bf16* cb = reinterpret_cast<__bf16*>(p.C) + (int64_t)row0 * ldc + col0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = a * 32 + (r >> 2) * 8 + (r & 3);
        if (dr < rlim) {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (b * 32 < clim) cb[dr * ldc + b * 32] = (__bf16)acc[a][b][r];
        }
      }
  }
}

}  // namespace

bool tok_gemm_supported(const TokGemm& p) {
  auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  // 32-bit byte offsets: every operand must span fewer than 2^31 bytes
  const double ea = 2.0 * (p.a_kmajor ? p.M : p.K) * p.lda, eb = 2.0 * (p.b_kmajor ? p.N : p.K) * p.ldb;
  return p.lda % 8 == 0 && p.ldb % 8 == 0 && al(p.A) && al(p.B) && ea < 2.0e9 && eb < 2.0e9;
}

hipError_t launch_tok_gemm(const TokGemm& p, int kclass, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const double flops = 2.0 * p.M * p.N * (double)p.K;
  const double bytes = 2.0 * ((double)p.M * p.K + (double)p.K * p.N) + (double)p.M * p.N * (p.c_f32 ? 4 : 2);
  ProfScope prof(kclass, st, flops, bytes);
  const int ntiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const dim3 grid(((ntiles + 7) / 8) * 8), block(256);
  if (p.a_kmajor && p.b_kmajor) hipLaunchKernelGGL((gemm_tok_kernel<true, true>), grid, block, 0, st, p);
  else if (p.a_kmajor) hipLaunchKernelGGL((gemm_tok_kernel<true, false>), grid, block, 0, st, p);
  else if (p.b_kmajor) hipLaunchKernelGGL((gemm_tok_kernel<false, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((gemm_tok_kernel<false, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace poet
