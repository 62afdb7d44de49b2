// bf16 x bf16 -> float32 GEMM on gfx950 MFMA, used for every bf16 contraction of the POET layer:
//   token GEMMs        Y = X W^T, dX = dY W, G = dY^T X (K = tokens)
//   weight side        factors applied to W0, primitive-gradient contractions, Cayley-Neumann power chain
//                      and its adjoint (batched over the primitives of a side)
//
// Workgroup tile 256 x 256 x 64, 8 waves in a 2 x 4 grid (two per SIMD), each wave 128 x 64 as 4 x 2
// v_mfma_f32_32x32x16_bf16.
// Operands go straight from global memory into LDS (global_load_lds_dwordx4: lane l of a wave writes the 16
// bytes at the wave's LDS base + 16 l, from any global address it chooses), in a two-stage ring: the DMA of
// K-tile t+1 runs while the MFMAs consume tile t, one barrier per tile, placed before the last k-step so that the
// next DMA and the next tile's first fragment reads overlap that k-step's MFMAs (one DMA instruction after each of
// its MFMAs, and the next tile's first fragment reads from the second MFMA on). A k-step's fragment reads for the
// next k-step are issued between its MFMAs (one MFMA, two reads), which measured ~3% faster than one burst.
// Both stage layouts are 32 KB:
//   K-major operand: 256 rows x 128 B; the 16-byte chunk index is XOR-ed with f(row mod 32) =
//     (row & 7) ^ ((row >> 3) & 3): 16 consecutive rows read at one logical chunk hit 16 distinct 16-byte bank
//     groups, so the ds_read_b128 fragments are conflict-free;
//   M/N-major operand: 64 k-rows x 512 B; the 64-byte block index is XOR-ed with (k-row & 3), so the 4 k-rows a
//     16-lane group reads with ds_read_b64_tr_b16 fall in 4 different 64-byte bank windows (in each 16-lane
//     group, lane j supplies the address of 4 consecutive elements of k-row j/4; lane i receives the elements
//     of column i of those 4 k-rows: an MFMA fragment of the transposed operand).
// Rows or columns past M / N are fetched from a clamped (valid) address: they only reach outputs that are
// never stored. The K tail of the last tile is zeroed in LDS after its DMA lands. A wave's finished 128 x 64
// tile leaves through LDS as row-contiguous vector stores.
//
// Work decomposition: (batch, split, tile) triples in one 1-D grid. Workgroup id w runs on XCD w % 8, so each
// XCD takes a contiguous range of that order: neighbouring tiles on one XCD share A rows in its L2. With
// split-K each split writes its float32 partial tile; a second kernel sums the partials in split order (so
// results do not depend on timing) and applies the epilogue.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "internal.h"

namespace poet {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = 256 * BK * 2;  // bytes of one operand's stage (both layouts)

constexpr int MAXGP = 16;
struct GroupEntry {
  int64_t offA = 0, offB = 0, offC = 0, offE = 0, lda = 0, ldb = 0;
  int b0 = 0, Mtot = 0, Ntot = 0, pad = 0;
};

// Kernel arguments, passed by value. NP is the capacity of the problem table: MAXGP for grouped launches, 1 for
// the others (a single-problem launch carries no 1 KB table: the runtime stages every launch's arguments, and a
// stream of many small launches with large arguments stalls the host's enqueue until that stream drains).
template <int NP>
struct FastArgsT {
  GemmDesc g;
  int ntm, ntn, splits, kchunk;
  int use_part;  // write float32 partial tiles; a second kernel reduces them and applies the epilogue
  // nprob > 0: the launch holds nprob problems of g's shape (M, N, K, strides, output type); problem p owns batch
  // entries [prob[p].b0, prob[p + 1].b0) and reads / writes its operands at byte offsets from g's, with its own
  // leading dimensions and extents
  int nprob = 0;
  GroupEntry prob[NP];
};

// an epilogue the main kernel stores directly: out = acc into C (no addend, scale, second copy or accumulate)
inline bool plain_epilogue(const GemmDesc& g) { return !g.D && !g.C2 && !g.Acc && g.alpha == 1.f && g.C; }

__device__ __forceinline__ int swz(int r32) { return (r32 & 7) ^ ((r32 >> 3) & 3); }

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8), issued through the
// builtin so that the compiler's own wait insertion accounts for them
constexpr int WAIT_LGKM0 = 0xC07F;  // lgkmcnt(0)
constexpr int WAIT_VM0 = 0x0F70;    // vmcnt(0)

// Direct global->LDS DMA of one 256 x 64 operand tile. Per-thread source offsets are fixed for the K loop.
template <bool KMAJ, int NW>
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
      // instruction j of wave w fills rows 8 (NW j + w) + lane / 8, physical chunk lane % 8, whose logical
      // chunk (k offset / 8 inside the tile) is chk
      const int r32 = (8 * wave + (lane >> 3)) & 31;
      chk = (lane & 7) ^ swz(r32);
#pragma unroll
      for (int j = 0; j < 32 / NW; ++j) {
        const int row = min(r0 + 8 * (NW * j + wave) + (lane >> 3), R - 1);
        off[j] = (uint32_t)row * ld2;
      }
    } else {
      // instruction j of wave w fills k-rows 2 (NW j + w) + lane / 32, physical 16-byte chunk lane % 32
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

  // DMA instruction j (of 8) of the tile at k0 into stage st
  __device__ __forceinline__ void dma_one(char* __restrict__ st, int k0, int j, int wave, int lane) const {
    char* dst = st + (NW * j + wave) * 1024;
    uint32_t o;
    if constexpr (KMAJ) {
      const int kmax = ((K + 7) / 8) * 8 - 8;  // keep the 16-byte read inside the row's first ceil8(K) elements
      o = off[j] + (uint32_t)min(k0 + 8 * chk, kmax) * 2;
    } else {
      const int kr = min(k0 + 2 * (NW * j + wave) + (lane >> 5), K - 1);
      o = off[j] + (uint32_t)kr * ld2;
    }
    __builtin_amdgcn_global_load_lds((gbl_void*)(base + o), (lds_void*)dst, 16, 0, 0);
  }
  __device__ __forceinline__ void dma(char* __restrict__ st, int k0, int wave, int lane) const {
#pragma unroll
    for (int j = 0; j < 32 / NW; ++j) dma_one(st, k0, j, wave, lane);
  }

  // zero the part of a staged tile that lies at k >= kend (kv = kend - k0 valid k values, 0 < kv < 64)
  __device__ __forceinline__ void zero_tail(char* __restrict__ st, int kv, int tid) const {
    if constexpr (KMAJ) {
      if (tid >= 256) return;
      const int row = tid, s = swz(row & 31);
      for (int k = kv; k < BK; ++k)
        *reinterpret_cast<short*>(st + row * 128 + (((k >> 3) ^ s) << 4) + (k & 7) * 2) = 0;
    } else {
      for (int e = kv * 32 + tid; e < BK * 32; e += 64 * NW)
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

__device__ __forceinline__ void store_out(void* C, int dt, int64_t i, float v) {
  if (dt == BF16) reinterpret_cast<__bf16*>(C)[i] = (__bf16)v;
  else reinterpret_cast<float*>(C)[i] = v;
}

// out = alpha * acc + beta * D ; C <- out ; C2 <- out ; Acc += gamma * out
__device__ __forceinline__ void epilogue_one(const GemmDesc& g, int z, int row, int col, float acc) {
  float out = g.alpha * acc;
  if (g.D) out += g.beta * g.D[(int64_t)z * g.sD + (int64_t)row * g.ldd + col];
  if (g.E) out += (float)reinterpret_cast<const __bf16*>(g.E)[(int64_t)z * g.sE + (int64_t)row * g.lde + col];
  if (g.C) store_out(g.C, g.c_dt, (int64_t)z * g.sC + (int64_t)row * g.ldc + col, out);
  if (g.C2) store_out(g.C2, g.c2_dt, (int64_t)z * g.sC2 + (int64_t)row * g.ldc2 + col, out);
  if (g.Acc) g.Acc[(int64_t)z * g.sAcc + (int64_t)row * g.ldacc + col] += g.gamma * out;
}

// Store a wave's (32 WM) x (32 WN) accumulator tile at out (row pitch ld elements, dtype dt; rlim x clim of it valid)
// through the wave's Ep<WN>::BYTES of LDS, one 32-row band at a time: the band is written in accumulator order
// (row pitch EP floats, so the two half-waves land in disjoint banks) and read back as row-contiguous float4
// chunks, which go out as 16-byte (float32) or 8-byte (bf16) stores when the row is aligned for them. The region
// is the wave's own and one wave's LDS accesses complete in order, so the bands need no barrier: the global
// stores of one band stay in flight while the next is staged (a workgroup barrier would wait for all of them).
// e (nullable): a bf16 addend at the output's coordinates (row pitch lde), added before the output is rounded; its
// loads for a band are issued before the band's trip through LDS, which covers their latency.
template <int WN>
struct Ep {
  static constexpr int EP = 32 * WN + 8, BYTES = 32 * EP * 4;
};
template <int WM, int WN>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[WM][WN], char* lds, void* out, int dt, int64_t ld,
                                               int rlim, int clim, int lane, const __bf16* e = nullptr,
                                               int64_t lde = 0) {
  constexpr int EP = Ep<WN>::EP, NV = 4 * WN, PR = 8 * WN;  // float4 per lane per band, float4 per row
  float* ep = reinterpret_cast<float*>(lds);
  const bool vec = ld % 4 == 0 && (reinterpret_cast<uintptr_t>(out) % (dt == BF16 ? 8 : 16)) == 0;
  const bool evec = lde % 4 == 0 && (reinterpret_cast<uintptr_t>(e) & 7) == 0;
  // one 32-row band of the accumulators through the wave's LDS region: written in accumulator order, read back as
  // row-contiguous float4 chunks (chunk u of the lane: row c / PR, columns 4 (c % PR) .. + 3, c = lane + 64 u)
  auto stage = [&](int a, f32x4 (&vv)[NV]) {
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * EP + b * 32 + (lane & 31)] = acc[a][b][r];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int c = lane + 64 * u;
      vv[u] = *reinterpret_cast<const f32x4*>(ep + (c / PR) * EP + (c % PR) * 4);
    }
  };
  // a whole, aligned tile without an addend (every token GEMM but the edges): straight-line code, no per-element
  // checks (the checked version below costs a few percent of a token GEMM in instruction issue)
  if (__builtin_expect(!e && vec && rlim >= 32 * WM && clim >= 32 * WN, 1)) {
    if (dt == BF16) {
#pragma unroll
      for (int a = 0; a < WM; ++a) {
        f32x4 vv[NV];
        stage(a, vv);
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int c = lane + 64 * u, row = a * 32 + c / PR, c4 = (c % PR) * 4;
          bf16x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = (__bf16)vv[u][t];
          *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(out) + (int64_t)row * ld + c4) = w;
        }
      }
    } else {
#pragma unroll
      for (int a = 0; a < WM; ++a) {
        f32x4 vv[NV];
        stage(a, vv);
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int c = lane + 64 * u, row = a * 32 + c / PR, c4 = (c % PR) * 4;
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (int64_t)row * ld + c4) = vv[u];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int a = 0; a < WM; ++a) {
    bf16x4 ex[NV];
    if (e) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int c = lane + 64 * u, c4 = (c % PR) * 4, row = a * 32 + c / PR;
        ex[u] = bf16x4{};
        if (evec && row < rlim && c4 + 4 <= clim) ex[u] = *reinterpret_cast<const bf16x4*>(e + (int64_t)row * lde + c4);
      }
    }
    f32x4 vv[NV];
    stage(a, vv);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int c = lane + 64 * u, rr = c / PR, c4 = (c % PR) * 4, row = a * 32 + rr;
      if (row >= rlim || c4 >= clim) continue;
      f32x4 v = vv[u];
      if (e) {
        const __bf16* q = e + (int64_t)row * lde + c4;
        if (evec && c4 + 4 <= clim) {
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] += (float)ex[u][t];
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (c4 + t < clim) v[t] += (float)q[t];
        }
      }
      const int64_t o = (int64_t)row * ld + c4;
      if (dt == BF16) {
        __bf16* q = reinterpret_cast<__bf16*>(out) + o;
        if (vec && c4 + 4 <= clim) {
          bf16x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = (__bf16)v[t];
          *reinterpret_cast<bf16x4*>(q) = w;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (c4 + t < clim) q[t] = (__bf16)v[t];
        }
      } else {
        float* q = reinterpret_cast<float*>(out) + o;
        if (vec && c4 + 4 <= clim) {
          *reinterpret_cast<f32x4*>(q) = v;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (c4 + t < clim) q[t] = v[t];
        }
      }
    }
  }
}

// A symmetric / skew-symmetric product (GemmDesc::tri) computes only the tiles on and above the diagonal; an
// off-diagonal tile also goes out transposed, times the sign, into its mirror tile below the diagonal, straight from
// the accumulators: a lane's four consecutive rows of one column are four consecutive columns of one row of the
// mirror tile (8-byte bf16 stores, 16 contiguous bytes per row per instruction).
template <int WM, int WN>
__device__ __forceinline__ void store_mirror(const f32x16 (&acc)[WM][WN], char* cz, int dt, int64_t ld, int row0,
                                             int col0, int n, float sign, int lane) {
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int drow = col0 + b * 32 + (lane & 31), dcol = row0 + a * 32 + q * 8 + (lane >> 5) * 4;
        if (drow >= n || dcol >= n) continue;
        const int64_t o = (int64_t)drow * ld + dcol;
        if (dt == BF16) {
          __bf16* p = reinterpret_cast<__bf16*>(cz) + o;
          if (dcol + 4 <= n && (o & 3) == 0) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(sign * acc[a][b][4 * q + e]);
            *reinterpret_cast<bf16x4*>(p) = w;
          } else {
            for (int e = 0; e < 4 && dcol + e < n; ++e) p[e] = (__bf16)(sign * acc[a][b][4 * q + e]);
          }
        } else {
          float* p = reinterpret_cast<float*>(cz) + o;
          for (int e = 0; e < 4 && dcol + e < n; ++e) p[e] = sign * acc[a][b][4 * q + e];
        }
      }
}

// TAG only separates kernel symbols for profiling: 1, 2, 3 = the token GEMMs Y, dX, G; 0 = everything else.
// GROUP: the launch holds several problems of one shape (nprob and prob of the arguments).
// Waves per workgroup and their grid over the 256 x 256 tile. Eight waves (two per SIMD, wave tile 128 x 64) measured
// 7-12% faster than four (one per SIMD, 128 x 128) on every token-GEMM shape, bit-identical: with one wave per SIMD
// each barrier and copy wait stalls the matrix core, while a second wave keeps issuing MFMAs (sixteen waves, 64 x 64,
// ran the same as eight). The extra fragment reads (LDS active ~13% of the cycles with four waves) do not bind.
constexpr int KNW = 8;
template <int NW> struct WaveGrid;
template <> struct WaveGrid<4> { static constexpr int GR = 2, GC = 2; };   // wave tile 128 x 128
template <> struct WaveGrid<8> { static constexpr int GR = 2, GC = 4; };   // 128 x 64
constexpr int smem_bytes(int nw) {
  return 4 * STAGE > nw * Ep<8 / WaveGrid<KNW>::GC>::BYTES ? 4 * STAGE : nw * Ep<8 / WaveGrid<KNW>::GC>::BYTES;
}

template <bool AK, bool BK_, int TAG, bool GROUP = false, int NW = KNW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void gemm_bf16_kernel(const FastArgsT<GROUP ? MAXGP : 1> fa_) {
  constexpr int WM = 8 / WaveGrid<NW>::GR, WN = 8 / WaveGrid<NW>::GC;  // 32 x 32 blocks per wave
  constexpr int NDMA = 32 / NW;        // DMA instructions per operand per wave and tile
  __shared__ __attribute__((aligned(1024))) char smem[smem_bytes(NW)];
  const GemmDesc& g = fa_.g;
  const int ntm = fa_.ntm, ntn = fa_.ntn, splits = fa_.splits;
  // tiles of one (batch, split): all of them, or for a symmetric / skew-symmetric product (tri) only those on and
  // above the diagonal, row after row (each off-diagonal one also fills its mirror tile below, store_mirror)
  const int per_entry = g.tri ? ntm * (ntm + 1) / 2 : ntm * ntn;
  const int ntiles = g.batch * splits * per_entry;
  const int per = (ntiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= ntiles) return;
  // tile order inside one (batch, split): patches of GM row bands x GN column tiles, patch after patch along N,
  // then the next GM row bands. An XCD's workgroups run a contiguous range of this order together, so they share
  // the K-slices of a few A row bands and a few B column tiles in its L2 (column-fastest order over a wide N
  // would stream all of B once per row band)
  const int zs = t / per_entry, tl = t % per_entry;
  int tm, tn;
  if (g.tri) {
    tm = 0;
    int rest = tl;
    while (rest >= ntm - tm) rest -= ntm - tm++;
    tn = tm + rest;
  } else {
    constexpr int GM = 4, GN = 8;
    const int sr = tl / (GM * ntn), rem = tl % (GM * ntn);
    const int rows = min(GM, ntm - GM * sr);
    const int ngn = (ntn + GN - 1) / GN;
    const int gi = min(rem / (rows * GN), ngn - 1);
    const int r2 = rem - rows * GN * gi;
    const int w = min(GN, ntn - gi * GN);
    tm = GM * sr + r2 / w;
    tn = gi * GN + r2 % w;
  }
  // zg: batch entry over both problems (indexes the partials). With one tile per batch entry (the token-axis
  // contractions, one bp x bp block each) the entries of one K range are adjacent, so the workgroups an XCD runs
  // together read whole rows of the token-major operands rather than one block's columns of many rows
  const bool zfast = ntm * ntn == 1;
  const int s = zfast ? zs / g.batch : zs % splits, zg = zfast ? zs % g.batch : zs / splits;
  int z = zg;
  const char* Ab = reinterpret_cast<const char*>(g.A);
  const char* Bb = reinterpret_cast<const char*>(g.B);
  char* Cb = reinterpret_cast<char*>(g.C);
  const char* Eb = reinterpret_cast<const char*>(g.E);
  int64_t lda = g.lda, ldb = g.ldb;
  int Mtot = g.Mtot, Ntot = g.Ntot;
  if constexpr (GROUP) {
    int p = 0;
    for (int q = 1; q < fa_.nprob; ++q)
      if (zg >= fa_.prob[q].b0) p = q;
    const GroupEntry& e = fa_.prob[p];
    z = zg - keep_s(e.b0);
    Ab += keep_s(e.offA); Bb += keep_s(e.offB); Cb += keep_s(e.offC);
    if (Eb) Eb += keep_s(e.offE);
    lda = keep_s(e.lda); ldb = keep_s(e.ldb); Mtot = keep_s(e.Mtot); Ntot = keep_s(e.Ntot);
  }
  int M = g.M, N = g.N, K = g.K;
  if (Mtot > 0) M = min(M, Mtot - z * g.M);
  if (Ntot > 0) N = min(N, Ntot - z * g.N);
  if (g.Ktot > 0) K = min(K, g.Ktot - z * g.K);
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= M || n0 >= N) return;
  const int kb = s * fa_.kchunk, ke = min(K, kb + fa_.kchunk);

  // the wave index is uniform: as a scalar, the LDS addresses derived from it (DMA destinations in M0) need no
  // per-instruction readfirstlane
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = (wave / WaveGrid<NW>::GC) * 32 * WM, wc = (wave % WaveGrid<NW>::GC) * 32 * WN;

  Operand<AK, NW> oa;
  Operand<BK_, NW> ob;
  oa.init(reinterpret_cast<const __bf16*>(Ab) + (int64_t)z * g.sA, lda, m0, M, ke, wave, lane);
  ob.init(reinterpret_cast<const __bf16*>(Bb) + (int64_t)z * g.sB, ldb, n0, N, ke, wave, lane);

  f32x16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = kb < ke ? (ke - kb + BK - 1) / BK : 0;
  // Two-stage ring: the DMA of tile t+1 is in flight while tile t is multiplied. The barrier that retires tile
  // t's stage (and confirms tile t+1) sits before the MFMAs of tile t's last k-step, so the DMA of tile t+2 and
  // the LDS reads of tile t+1's first fragments are issued while those MFMAs run.
  bf16x8 fa[2][WM], fb[2][WN];
  if (nk > 0) {
    oa.dma(smem, kb, wave, lane);
    ob.dma(smem + STAGE, kb, wave, lane);
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    __syncthreads();
    const int kv = ke - kb;
    if (kv < BK) {  // the first tile is partial (and the only one)
      oa.zero_tail(smem, kv, tid);
      ob.zero_tail(smem + STAGE, kv, tid);
      __syncthreads();
    }
    if (nk > 1) {
      oa.dma(smem + 2 * STAGE, kb + BK, wave, lane);
      ob.dma(smem + 3 * STAGE, kb + BK, wave, lane);
    }
#pragma unroll
    for (int a = 0; a < WM; ++a) fa[0][a] = frag<AK>(smem, wr + a * 32, 0, lane);
#pragma unroll
    for (int b = 0; b < WN; ++b) fb[0][b] = frag<BK_>(smem + STAGE, wc + b * 32, 0, lane);
  }
  for (int kt = 0; kt < nk; ++kt) {
    char* sa = smem + (kt & 1) * 2 * STAGE;
    char* sb = sa + STAGE;
    // k-steps 0..2: fragments of k-step ks + 1 are read from LDS while the 16 MFMAs of k-step ks run
#pragma unroll
    for (int ks = 0; ks < BK / 16 - 1; ++ks) {
      const int c = ks & 1;
      // k-step ks's fragments were issued a k-step ago: retire them here, so that the MFMAs below need no wait on
      // the (up to 16) reads issued next, which a 4-bit LDS counter could not express
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < WM; ++a) fa[c ^ 1][a] = frag<AK>(sa, wr + a * 32, ks + 1, lane);
#pragma unroll
      for (int b = 0; b < WN; ++b) fb[c ^ 1][b] = frag<BK_>(sb, wc + b * 32, ks + 1, lane);
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][a], fb[c][b], acc[a][b], 0, 0, 0);
      // the fragment reads go out between the MFMAs (one MFMA, two reads), not as one burst ahead of them
#pragma unroll
      for (int q = 0; q < (WM + WN) / 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      }
      __builtin_amdgcn_sched_group_barrier(0x008, WM * WN - (WM + WN) / 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    char* na = smem + ((kt + 1) & 1) * 2 * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      // tile kt+1 has landed (its DMA is the only one in flight) and every wave has read tile kt
      __builtin_amdgcn_s_waitcnt(WAIT_VM0);
      __syncthreads();
      const int kv = ke - (kb + (kt + 1) * BK);
      if (kv < BK) {  // tile kt+1 is the last one and partial
        oa.zero_tail(na, kv, tid);
        ob.zero_tail(na + STAGE, kv, tid);
        __syncthreads();
      }
    } else {
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // last k-step: its MFMAs each followed by one DMA instruction of tile kt+2 (into the stage tile kt held, which
    // no wave reads any more) and, from MFMA Q0 on, by the fragment reads of tile kt+1's first k-step, so the matrix
    // core keeps running while they issue (with eight waves the other wave of the SIMD covers the shorter gap
    // between the last reads and their use). They run without
    // conditions: past the end the copies read clamped (valid) addresses, and in the last tile (no barrier above,
    // other waves may still read its stage) they go to the other stage, which nothing reads again; the epilogue's
    // first barrier waits for them. The fragments read past the end are never used.
    char* da = more ? sa : na;
    const int k2 = kb + (kt + 2) * BK;
    constexpr int Q0 = NW == 4 ? 4 : (NW == 8 ? 1 : 0);  // first MFMA followed by a fragment read of the next tile
    constexpr int NR = WM + WN, PER = NR > WM * WN ? 2 : 1;   // next-tile fragment reads, per MFMA
#pragma unroll
    for (int q = 0; q < WM * WN; ++q) {
      const int a = q / WN, b = q % WN;
      acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][a], fb[1][b], acc[a][b], 0, 0, 0);
      if (q < NDMA) oa.dma_one(da, k2, q, wave, lane);
      else if (q < 2 * NDMA) ob.dma_one(da + STAGE, k2, q - NDMA, wave, lane);
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int r = (q - Q0) * PER + t;
        if (q >= Q0 && r < NR) {
          if (r < WM) fa[0][r] = frag<AK>(na, wr + r * 32, 0, lane);
          else fb[0][r - WM] = frag<BK_>(na + STAGE, wc + (r - WM) * 32, 0, lane);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the wave's tile goes out through LDS (every wave is past its last fragment read first)
  __syncthreads();
  const int wrow0 = m0 + wr, wcol0 = n0 + wc;
  if (fa_.use_part) {  // raw partial tile; the reduction kernel sums the splits and applies the epilogue
    float* pb = g.part + ((int64_t)(s * g.batch + zg) * g.M + wrow0) * g.N + wcol0;
    store_tile_lds<WM, WN>(acc, smem + wave * Ep<WN>::BYTES, pb, F32, g.N, M - wrow0, N - wcol0, lane);
    return;
  }
  if (!g.C) return;
  char* cb = Cb + ((int64_t)z * g.sC + (int64_t)wrow0 * g.ldc + wcol0) * dtype_size(g.c_dt);
  // the bf16 addend serves only the non-token products (TAG 0): the token GEMMs' epilogue keeps no code for it
  const __bf16* eb = TAG == 0 && Eb ? reinterpret_cast<const __bf16*>(Eb) + (int64_t)z * g.sE + (int64_t)wrow0 * g.lde + wcol0
                                    : nullptr;
  store_tile_lds<WM, WN>(acc, smem + wave * Ep<WN>::BYTES, cb, g.c_dt, g.ldc, M - wrow0, N - wcol0, lane, eb, g.lde);
  if constexpr (TAG == 0) {  // the token GEMMs (TAG 1-3) keep no code for it
    if (g.tri && tm != tn)
      store_mirror<WM, WN>(acc, Cb + (int64_t)z * g.sC * dtype_size(g.c_dt), g.c_dt, g.ldc, wrow0, wcol0, M,
                           (float)g.tri, lane);
  }
}

// Sum the split-K partials of every output element in split order, then apply the epilogue.
// Work item: four adjacent columns of one partial row (one column where N is not a multiple of 4), read from every
// split as one 16-byte load; 32-bit indices (the partials of one launch are far below 2^31 elements).
template <int NP>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const FastArgsT<NP> fa_) {
  const GemmDesc& g = fa_.g;
  const int64_t mn = (int64_t)g.M * g.N;
  const bool v4 = (g.N & 3) == 0;
  const int nq = v4 ? g.N >> 2 : g.N, rows = g.batch * g.M, items = rows * nq;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < items; e += gridDim.x * blockDim.x) {
    const int r = e / nq, q = e - r * nq;
    const int zg = r / g.M, row = r - zg * g.M, col = v4 ? 4 * q : q;
    int p = 0;  // problem of a grouped launch (plain epilogue)
    for (int u = 1; u < fa_.nprob; ++u)
      if (zg >= fa_.prob[u].b0) p = u;
    const int z = fa_.nprob > 0 ? zg - fa_.prob[p].b0 : zg;
    int M = g.M, N = g.N;
    const int Mtot = fa_.nprob > 0 ? fa_.prob[p].Mtot : g.Mtot, Ntot = fa_.nprob > 0 ? fa_.prob[p].Ntot : g.Ntot;
    if (Mtot > 0) M = min(M, Mtot - z * g.M);
    if (Ntot > 0) N = min(N, Ntot - z * g.N);
    if (row >= M || col >= N) continue;
    const int64_t rc = (int64_t)row * g.N + col;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    if (v4) {
      for (int sp = 0; sp < fa_.splits; ++sp)
        sum += *reinterpret_cast<const f32x4*>(g.part + (int64_t)(sp * g.batch + zg) * mn + rc);
    } else {
      for (int sp = 0; sp < fa_.splits; ++sp) sum[0] += g.part[(int64_t)(sp * g.batch + zg) * mn + rc];
    }
    const int nc = v4 ? min(4, N - col) : 1;
    for (int t = 0; t < nc; ++t) {
      if (fa_.nprob > 0) {
        char* cb = reinterpret_cast<char*>(g.C) + fa_.prob[p].offC;
        float o = sum[t];
        if (g.E)
          o += (float)reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(g.E) + fa_.prob[p].offE)
                   [(int64_t)z * g.sE + (int64_t)row * g.lde + col + t];
        store_out(cb, g.c_dt, (int64_t)z * g.sC + (int64_t)row * g.ldc + col + t, o);
      } else {
        epilogue_one(g, z, row, col + t, sum[t]);
      }
    }
  }
}

}  // namespace

bool fast_gemm_eligible(const GemmDesc& g) {
  auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (g.compute != BF16 || g.a_dt != BF16 || g.b_dt != BF16 || g.a_sub_eye || g.b_sub_eye) return false;
  if (g.M < 128 || g.N < 128 || g.batch < 1) return false;
  if (g.tri && (g.M != g.N || !plain_epilogue(g) || g.defer_reduce || g.kclass <= 2)) return false;
  if ((!plain_epilogue(g) || g.defer_reduce) && (!g.part || g.part_elems < (size_t)g.batch * g.M * g.N)) return false;
  if (g.lda % 8 || g.ldb % 8 || g.sA % 8 || g.sB % 8 || !al(g.A) || !al(g.B)) return false;
  // 32-bit byte offsets inside one batch's operands
  const double ea = 2.0 * (g.a_kmajor ? g.M : g.K) * (double)g.lda, eb = 2.0 * (g.b_kmajor ? g.N : g.K) * (double)g.ldb;
  return ea < 2.0e9 && eb < 2.0e9;
}

int fast_gemm_splits(const GemmDesc& g) {
  // Split K only where it shortens the launch. A work item (one output tile, nk / S K-tiles) holds one CU (256 CUs,
  // one workgroup each), so the items take ceil(tiles S / 256) rounds of about nk / S + 1.5 K-tile times (the 1.5
  // is the pipeline fill and the epilogue). S > 1 adds float32 partials, written by the items and read back by the
  // reduction: about 8 S + 4 bytes per output element, counted at one K-tile time per 5 MB. Candidates keep at
  // least two K-tiles per split and fit the scratch the caller provided; a larger S must win by 3% or more.
  if (g.tri) return 1;  // the tiles on and above the diagonal store their mirror tiles themselves: no partials
  const int tiles = g.batch * ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const int nk = (g.K + BK - 1) / BK;
  const double outs = (double)g.batch * g.M * g.N;
  int best_s = 1;
  double best = 0.0;
  for (int S = 1; S <= 16; S *= 2) {
    if (S > 1 && (!g.part || nk < 2 * S || (size_t)S * (size_t)outs > g.part_elems)) break;
    const double rounds = std::ceil((double)tiles * S / 256.0);
    double cost = rounds * ((double)nk / S + 1.5);
    if (S > 1) cost += (8.0 * S + 4.0) * outs / 5.0e6;
    if (S == 1 || cost < 0.97 * best) { best = cost; best_s = S; }
  }
  return best_s;
}

hipError_t launch_fast_gemm(const GemmDesc& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  FastArgsT<1> fa;
  fa.g = g;
  fa.ntm = (g.M + BM - 1) / BM;
  fa.ntn = (g.N + BN - 1) / BN;
  const int tiles = g.batch * (g.tri ? fa.ntm * (fa.ntm + 1) / 2 : fa.ntm * fa.ntn);
  const int nk = (g.K + BK - 1) / BK;
  const int S = fast_gemm_splits(g);
  fa.splits = S;
  fa.kchunk = ((nk + S - 1) / S) * BK;
  fa.use_part = (S > 1 || !plain_epilogue(g) || g.defer_reduce) ? 1 : 0;
  const double flops = 2.0 * g.M * g.N * (double)g.K * g.batch;
  const double bytes = g.batch * (2.0 * ((double)g.M * g.K + (double)g.K * g.N) +
                                  (double)g.M * g.N * ((g.C ? dtype_size(g.c_dt) : 0) + (g.D ? 4 : 0) + (g.E ? 2 : 0) +
                                                       (g.C2 ? dtype_size(g.c2_dt) : 0) + (g.Acc ? 8 : 0)));
  ProfScope prof(g.kclass, st, flops, bytes);
  const dim3 grid(((tiles * S + 7) / 8) * 8), block(64 * KNW);
  if (g.kclass == 0 && !g.E && g.a_kmajor && g.b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, 1>), grid, block, 0, st, fa);
  else if (g.kclass == 1 && !g.E && g.a_kmajor && !g.b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, 2>), grid, block, 0, st, fa);
  else if (g.kclass == 2 && !g.E && !g.a_kmajor && !g.b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, 3>), grid, block, 0, st, fa);
  else if (g.a_kmajor && g.b_kmajor) hipLaunchKernelGGL((gemm_bf16_kernel<true, true, 0>), grid, block, 0, st, fa);
  else if (g.a_kmajor) hipLaunchKernelGGL((gemm_bf16_kernel<true, false, 0>), grid, block, 0, st, fa);
  else if (g.b_kmajor) hipLaunchKernelGGL((gemm_bf16_kernel<false, true, 0>), grid, block, 0, st, fa);
  else hipLaunchKernelGGL((gemm_bf16_kernel<false, false, 0>), grid, block, 0, st, fa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !fa.use_part || g.defer_reduce) return e;
  const int64_t total = (int64_t)g.batch * g.M * (g.N % 4 == 0 ? g.N / 4 : g.N);
  const int rg = (int)std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3(rg), dim3(256), 0, st, fa);
  return hipGetLastError();
}

bool fast_gemm_group_eligible(const GemmDesc* pr, int n) {
  if (n < 1 || n > MAXGP) return false;
  const GemmDesc& a = pr[0];
  size_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    const GemmDesc& b = pr[i];
    if (!fast_gemm_eligible(b) || !plain_epilogue(b) || b.defer_reduce) return false;
    if (b.a_kmajor != a.a_kmajor || b.b_kmajor != a.b_kmajor || b.M != a.M || b.N != a.N || b.K != a.K ||
        b.Ktot != a.Ktot || b.sA != a.sA || b.sB != a.sB || b.ldc != a.ldc || b.sC != a.sC || b.c_dt != a.c_dt ||
        !b.E != !a.E || b.lde != a.lde || b.sE != a.sE || b.tri != a.tri)
      return false;
    blocks += (size_t)b.batch;
  }
  // the split-K partials of every problem (at least 2 splits) in the first one's scratch; no scratch: no split
  return !a.part || a.part_elems >= 2 * blocks * a.M * a.N;
}

bool fast_gemm_pair_eligible(const GemmDesc& a, const GemmDesc& b) {
  const GemmDesc pr[2] = {a, b};
  return fast_gemm_group_eligible(pr, 2);
}

hipError_t launch_fast_gemm_group(const GemmDesc* pr, int n, hipStream_t st) {
  GemmDesc g = pr[0];
  g.batch = 0;
  FastArgsT<MAXGP> fa;
  fa.nprob = n;
  for (int i = 0; i < n; ++i) {
    GroupEntry& e = fa.prob[i];
    e.b0 = g.batch;
    e.offA = reinterpret_cast<const char*>(pr[i].A) - reinterpret_cast<const char*>(pr[0].A);
    e.offB = reinterpret_cast<const char*>(pr[i].B) - reinterpret_cast<const char*>(pr[0].B);
    e.offC = reinterpret_cast<const char*>(pr[i].C) - reinterpret_cast<const char*>(pr[0].C);
    e.offE = pr[0].E ? reinterpret_cast<const char*>(pr[i].E) - reinterpret_cast<const char*>(pr[0].E) : 0;
    e.lda = pr[i].lda; e.ldb = pr[i].ldb; e.Mtot = pr[i].Mtot; e.Ntot = pr[i].Ntot;
    g.batch += pr[i].batch;
  }
  if (g.batch <= 0 || g.M <= 0 || g.N <= 0) return hipSuccess;
  fa.g = g;
  fa.ntm = (g.M + BM - 1) / BM;
  fa.ntn = (g.N + BN - 1) / BN;
  const int tiles = g.batch * (g.tri ? fa.ntm * (fa.ntm + 1) / 2 : fa.ntm * fa.ntn);
  const int nk = (g.K + BK - 1) / BK;
  const int S = fast_gemm_splits(g);
  fa.splits = S;
  fa.kchunk = ((nk + S - 1) / S) * BK;
  fa.use_part = S > 1 ? 1 : 0;
  const double flops = 2.0 * g.M * g.N * (double)g.K * g.batch;
  const double bytes = g.batch * (2.0 * ((double)g.M * g.K + (double)g.K * g.N) +
                                  (double)g.M * g.N * (dtype_size(g.c_dt) + (g.E ? 2 : 0)));
  ProfScope prof(g.kclass, st, flops, bytes);
  const dim3 grid(((tiles * S + 7) / 8) * 8), block(64 * KNW);
  if (g.a_kmajor && g.b_kmajor) hipLaunchKernelGGL((gemm_bf16_kernel<true, true, 0, true>), grid, block, 0, st, fa);
  else if (g.a_kmajor) hipLaunchKernelGGL((gemm_bf16_kernel<true, false, 0, true>), grid, block, 0, st, fa);
  else if (g.b_kmajor) hipLaunchKernelGGL((gemm_bf16_kernel<false, true, 0, true>), grid, block, 0, st, fa);
  else hipLaunchKernelGGL((gemm_bf16_kernel<false, false, 0, true>), grid, block, 0, st, fa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !fa.use_part) return e;
  const int64_t total = (int64_t)g.batch * g.M * (g.N % 4 == 0 ? g.N / 4 : g.N);
  const int rg = (int)std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(splitk_reduce_kernel<MAXGP>, dim3(rg), dim3(256), 0, st, fa);
  return hipGetLastError();
}

hipError_t launch_fast_gemm_pair(const GemmDesc& a, const GemmDesc& b, hipStream_t st) {
  const GemmDesc pr[2] = {a, b};
  return launch_fast_gemm_group(pr, 2, st);
}

}  // namespace poet
