// Block-diagonal factor applied to bf16 activations (POET reparameterization W = R W0 P with the factors moved
// onto the activations: X P^T, Z R^T, dY R, dX' P):
//   out[t, block] = in[t, block] F_block^T   (trans)   or   in[t, block] F_block,
// for every block of the factor (size c = min(bp, d - b bp), bp <= 256) and every token t, with F taken as identity
// + delta: the MFMA operand is the delta F - I rounded to bf16 (k_act_operand writes it as bf16 rows), the float32
// accumulators start from the input element itself (the identity part, exact), and only the output is rounded to
// bf16. Rounding the whole factor instead would cost a rounding of its diagonal 1 + O(|Q|^2)
// at the bf16 step of 2^-8 near 1, an error as large as the output's own rounding.
//
// Weight-stationary: a workgroup owns one block and a run of 32-token tiles. Its 4 waves each hold 64 output
// columns of the block's operand (all of K, 16 k-steps x 2 column tiles of bf16x8 fragments: 128 registers),
// loaded and rounded once. The 32 x 256 activation tiles stream through a four-stage LDS ring by DMA
// (global_load_lds), three tiles' copies in flight while the current one is multiplied
// (v_mfma_f32_32x32x16_bf16, 32 tokens x 64 columns per wave per tile); the finished tile goes through an LDS
// buffer of its own and leaves as coalesced 16-byte row chunks. Rows past the last token are read from the
// last token (finite values, never stored); the columns of a partial last chunk past the block (row padding,
// any bits, NaN included) are cleared in LDS by the lanes that copied them. The operand comes in fragment order
// where the block is a multiple of 32 (one wave's load of a fragment reads 1 KB contiguous), else in row order.
#include <algorithm>

#include "poet.h"
#include "strip_mma.h"

namespace poet {
namespace {

using namespace strip;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int AT = 256;             // threads (4 waves)
constexpr int TM = 32;              // tokens per tile
constexpr int TILE_BYTES = TM * ROWB;  // 16 KB
constexpr int NST = 4;                 // ring stages: copies run up to NST - 1 tiles ahead
constexpr int WAIT_VM0 = 0x0F70;
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 raw buffer descriptor word 3
constexpr uint32_t OOB = 0x80000000u;    // an offset past the end of the output buffer (under 2 GB)
// s_waitcnt immediate for vmcnt(n), lgkmcnt and expcnt left free (gfx9 encoding: vmcnt bits 3:0 and 15:14)
constexpr int vm_wait(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

struct ActArgs {
  const __bf16* in; int64_t ldi;
  __bf16* out; int64_t ldo;
  const __bf16* Bt; // nblk bp x bp blocks of bf16 operand rows: Bt[j][k] = B(k, j)
  int T, d, bp, nblk;
  int tiles_per_wg; // token tiles per workgroup
  int ngrp;         // token groups: ceil(ceil(T / TM) / tiles_per_wg)
};

// Operand rows for the kernel below: Bt[b][j][k] = bf16(B(k, j)) with B the delta F_b - I, B(k, j) = F_b[j][k] - [j = k]
// (trans) or F_b[k][j] - [j = k], for j, k < c (the block's size) and zero elsewhere in the bp x bp block, in fragment order where
// act_frag_layout(bp), else in row order. Row order: consecutive threads take consecutive k (trans: coalesced
// reads) or consecutive j (no trans: the strided side is the read of F, coalesced in j). Fragment order:
// consecutive threads write consecutive elements.
__global__ void k_act_operand(const float* __restrict__ F, int bp, int d, int nblk, int trans, __bf16* __restrict__ Bt) {
  const int64_t per = (int64_t)bp * bp, total = per * nblk;
  const bool frag = act_frag_layout(bp);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(e / per);
    const int rem = (int)(e % per);
    const int c = min(bp, d - b * bp);
    int j, k;
    if (frag) {  // rem = ((g (bp / 16) + s) 64 + l) 8 + v
      const int v = rem & 7, l = (rem >> 3) & 63, gs = rem >> 9, s = gs % (bp >> 4), g = gs / (bp >> 4);
      j = 32 * g + (l & 31);
      k = 16 * s + 8 * (l >> 5) + v;
    } else if (trans) {
      j = rem / bp; k = rem % bp;
    } else {
      k = rem / bp; j = rem % bp;
    }
    const bool in = j < c && k < c;
    const float f = F[(int64_t)b * per + (in ? (trans ? (int64_t)j * bp + k : (int64_t)k * bp + j) : 0)];
    Bt[(int64_t)b * per + (frag ? rem : (int64_t)j * bp + k)] = (__bf16)(in ? f - (j == k ? 1.f : 0.f) : 0.f);
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its global ones (a
// __syncthreads() also drains every copy and store in flight, which would serialize the next tile's DMA with the
// current tile's MFMAs). The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// NK: k-steps of 16 covering the block size (4, 8 or 16); every loop over them is unrolled without conditions.
// FRAG: the operand is in fragment order.
template <int NK, bool FRAG>
__global__ __launch_bounds__(AT, 2) void act_apply_kernel(const ActArgs a) {
  __shared__ __attribute__((aligned(16))) char ring[NST * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char obuf[TILE_BYTES];  // the finished tile, on its way out
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = a.nblk * a.ngrp;
  // XCD-aware order: hardware workgroup b runs on XCD b % 8 and takes logical id (b % 8) per + b / 8
  const int per = (nb + 7) / 8;
  const int L = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (L >= nb) return;
  // logical id = (token group, block) with the block fastest: the workgroups running together on an XCD cover
  // whole rows of the same tokens (DRAM pages are read whole), and all blocks' operands fit in its L2
  const int blk = L % a.nblk, grp = L / a.nblk;
  const int b0 = blk * a.bp, c = min(a.bp, a.d - b0);
  const int ntile = (a.T + TM - 1) / TM;
  const int tile0 = grp * a.tiles_per_wg, tile1 = min(ntile, tile0 + a.tiles_per_wg);
  const int kh = (lane >> 5) * 8, j32 = lane & 31;

  // ---- DMA of token tile `tile` into ring stage `st`: instruction q (of 4) of wave w fills LDS bytes (4q + w) KB
  // + 16 lane, i.e. row 8q + h (h = 2w + lane / 32), physical chunk lane % 32, logical chunk (lane % 32) ^ (row % 16)
  const int h = wave * 2 + (lane >> 5);
  // chunks past the block's columns read its last whole chunk instead (finite activations, which meet a zero
  // operand); a partial last chunk is read as it is and its tail cleared in LDS
  const int last_chunk = (c - 1) >> 3, fill_chunk = max((c >> 3) - 1, 0);
  int lch[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int lc = j32 ^ (8 * e + h);
    lch[e] = lc <= last_chunk ? lc : fill_chunk;
  }
  const char* inb = reinterpret_cast<const char*>(a.in) + (int64_t)b0 * 2;  // uniform base; 32-bit offsets below
  auto dma = [&](int tile, int st) {
#pragma unroll
    for (int q = 0; q < TM / 8; ++q) {
      const uint32_t row = (uint32_t)min(tile * TM + 8 * q + h, a.T - 1);
      const uint32_t off = row * (uint32_t)a.ldi * 2u + 16u * (uint32_t)lch[q & 1];
      __builtin_amdgcn_global_load_lds((gbl_void*)(inb + off), (lds_void*)(ring + st * TILE_BYTES + (q * 4 + wave) * 1024),
                                       16, 0, 0);
    }
  };
  // A partial last chunk holds row padding past column c (any bits, NaN included). Every lane that copied it
  // (for a block narrower than one chunk, also into the positions of the chunks past it) clears its elements from
  // c % 8 on in its own 16 bytes of the stage, once its copies have landed and before the barrier that publishes
  // the tile: no extra barrier.
  // Elements [nv, 8) of the chunk (nv = c % 8 valid) are cleared by at most three aligned writes: one 2-byte write
  // when nv is odd, one 4-byte write when the next even element is 2 or 6, one 8-byte write of elements 4..7 when
  // the remainder starts there (the choices are uniform, only the copying lanes write).
  const bool ragged = (c & 7) != 0;
  const int nv = c & 7, e1 = nv + (nv & 1), e2 = e1 + (e1 & 2);
  const bool mine0 = lch[0] == (c >> 3), mine1 = lch[1] == (c >> 3);
  auto clear_pad = [&](int st) {
#pragma unroll
    for (int q = 0; q < TM / 8; ++q) {
      if (!(q & 1 ? mine1 : mine0)) continue;
      char* dst = ring + st * TILE_BYTES + (q * 4 + wave) * 1024 + 16 * lane;
      if (nv & 1) *reinterpret_cast<unsigned short*>(dst + 2 * nv) = 0;
      if (e1 & 2) *reinterpret_cast<uint32_t*>(dst + 2 * e1) = 0u;
      if (e2 == 4) *reinterpret_cast<uint64_t*>(dst + 8) = 0ull;
    }
  };

  // the first NST - 1 tiles' copies run while the operand is loaded
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (tile0 + i < tile1) dma(tile0 + i, i);

  // ---- resident operand: B(k, j) for this wave's columns j = 64 wave + 32 u + j32 and k = 16 ks + kh + v, from the
  // bf16 rows Bt[j][k] = B(k, j) (one 16-byte load per fragment: in fragment order the wave's 64 loads of one
  // fragment are 1 KB contiguous). Bt is zero outside the block's c x c corner and the fragments are zero for
  // k >= bp, so B vanishes for every k >= c.
  const __bf16* Bt = a.Bt + (int64_t)blk * a.bp * a.bp;
  bf16x8 bfr[2][NK];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = min(wave * 64 + u * 32 + j32, a.bp - 1);  // columns past bp: never stored, any finite value
    const int g = min(wave * 2 + u, a.bp / 32 - 1);          // (fragment order) their column group
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      // k past bp: zero (the staged activations there hold copies of a real chunk, not zeros)
      const int k = ks * 16 + kh;
      bf16x8 f;
      if constexpr (FRAG)
        f = *reinterpret_cast<const bf16x8*>(Bt + ((int64_t)(g * (a.bp >> 4) + min(ks, (a.bp >> 4) - 1)) * 64 + lane) * 8);
      else
        f = *reinterpret_cast<const bf16x8*>(Bt + (int64_t)j * a.bp + min(k, a.bp - 8));
      bfr[u][ks] = k < a.bp ? f : bf16x8{};
    }
  }

  // output through a raw buffer resource: every thread issues the same number of stores per tile (positions
  // outside the matrix go to an offset past the buffer's end, which the hardware drops), so the wait at the top of
  // the next tile can leave exactly those stores in flight and wait only for the copy issued before them
  const __amdgpu_buffer_rsrc_t Ob =
      __builtin_amdgcn_make_buffer_rsrc(a.out, (short)0, (int)((uint32_t)a.T * (uint32_t)a.ldo * 2u), RSRC_WORD3);
  const bool whole = (c & 7) == 0;  // every 16-byte chunk of the block is whole: one 16-byte store per chunk
  // Each thread issues, per tile, its copy of tile + NST - 1 (TM/8 instructions) and then its stores of the tile
  // (SQ per tile: one 16-byte store per row chunk, plus three (8-, 4- and 2-byte) stores for a partial last chunk).
  // The copy of tile t was issued three iterations earlier (or before the loop, then complete at the first wait),
  // followed by the stores of t-3, t-2, t-1 and the copies of t+1, t+2 where those exist: waiting until at most
  // that many are outstanding retires exactly the copy of t.
  constexpr int SQ = TM / 8, SQP = 4 * (TM / 8), CP = TM / 8;
  static_assert(3 * SQP + 2 * CP <= 63, "the outstanding count must fit the counter");
  for (int tile = tile0; tile < tile1; ++tile) {
    const int st = (tile - tile0) % NST;
    const int later = (tile + 1 < tile1) + (tile + 2 < tile1);  // copies issued after this tile's
    if (tile == tile0) {
      __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    } else if (whole) {
      if (later == 2) __builtin_amdgcn_s_waitcnt(vm_wait(3 * SQ + 2 * CP));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(vm_wait(3 * SQ + CP));
      else __builtin_amdgcn_s_waitcnt(vm_wait(3 * SQ));
    } else {
      if (later == 2) __builtin_amdgcn_s_waitcnt(vm_wait(3 * SQP + 2 * CP));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(vm_wait(3 * SQP + CP));
      else __builtin_amdgcn_s_waitcnt(vm_wait(3 * SQP));
    }
    if (ragged) clear_pad(st);
    lds_barrier();  // the tile's copy has landed everywhere; every wave is done with the previous tile's stage
    if (tile + NST - 1 < tile1) dma(tile + NST - 1, (st + NST - 1) % NST);
    const char* A = ring + st * TILE_BYTES;
    // fragment address of k-step ks: row (r * 32 + j32), chunk (2 ks + lane / 32) ^ (j32 & 15); the swizzle key passes
    // through an empty asm statement so that the 16 per-step addresses are recomputed (one XOR each), not kept live
    uint32_t xkey = (uint32_t)(j32 & 15);
    asm volatile("" : "+v"(xkey));
    const uint32_t hb = (uint32_t)(lane >> 5);
    auto frag_at = [&](int r, int ks) {
      const uint32_t o = (uint32_t)(r * 32 + j32) * ROWB + ((((uint32_t)(2 * ks) | hb) ^ xkey) << 4);
      return *reinterpret_cast<const bf16x8*>(A + o);
    };
    bf16x4 outv[2][4];  // [u][q]: four consecutive columns of one token, rounded to bf16
    {
      // the identity part: the accumulators start from the input element of the same token and column, read from the
      // staged tile (row j32, logical chunk 8 wave + 4 u + q, elements 4 (lane / 32) .. 4 (lane / 32) + 3: one 8-byte
      // read, in flight together with the first fragment reads); the products of the delta add to it in float32
      bf16x4 xid[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t ch = (uint32_t)(8 * wave + 4 * u + q);
          xid[u][q] = *reinterpret_cast<const bf16x4*>(A + (uint32_t)j32 * ROWB + (((ch ^ xkey) << 4) | (hb << 3)));
        }
      f32x16 acc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][q * 4 + e] = (float)xid[u][q][e];
      // k-steps pipelined by hand: the fragment of step ks + 2 is read while step ks multiplies, and a scheduling
      // barrier per step keeps the compiler from hoisting every read (and its registers) to the top. The product is
      // taken transposed, out^T = B^T in^T (the operand fragments as the left factor, the token fragments as the
      // right), so that a lane's accumulators hold four consecutive columns of one token.
      bf16x8 af[3];
      af[0] = frag_at(0, 0);
      af[1] = frag_at(0, 1);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        if (ks + 2 < NK) af[(ks + 2) % 3] = frag_at(0, ks + 2);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[u][ks], af[ks % 3], acc[u], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) outv[u][q][e] = (__bf16)acc[u][q * 4 + e];
    }
    // the output tile leaves through its own LDS buffer (every wave finished reading it for the previous tile before
    // this tile's first barrier), as rows of 512 B in the swizzled layout: one 8-byte write per four columns, read
    // back as 16-byte row chunks and stored coalesced
    char* O = obuf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)  // token j32, columns 64 wave + 32 u + 8 q + 4 (lane / 32) + (0..3)
        *reinterpret_cast<bf16x4*>(O + loff(j32, wave * 64 + u * 32 + 8 * q + 4 * (lane >> 5))) = outv[u][q];
    lds_barrier();
    {
#pragma unroll
      for (int q = 0; q < TM / 8; ++q) {  // chunk lane % 32 of row 8 q + h
        const int row = 8 * q + h, t = tile * TM + row;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(O + row * ROWB + ((j32 ^ (row & 15)) << 4));
        const int col = 8 * j32;  // first column of the chunk (logical chunk j32)
        const uint32_t o = ((uint32_t)t * (uint32_t)a.ldo + (uint32_t)(b0 + col)) * 2u;
        // whole chunks: one 16-byte store; a partial last chunk (nv = c % 8 elements): its first nv & 4 elements,
        // then nv & 2, then nv & 1, in one 8-, 4- and 2-byte store (each aligned: the chunk starts 16-byte aligned)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), Ob, t < a.T && col + 8 <= c ? o : OOB, 0, 0);
        if (!whole) {
          const int nv = c & 7;
          const bool part = t < a.T && col < c && col + 8 > c;
          const u32x4 w = __builtin_bit_cast(u32x4, v);
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, Ob, part && (nv & 4) ? o : OOB, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(w[(nv & 4) >> 1], Ob, part && (nv & 2) ? o + 2u * (nv & 4) : OOB, 0, 0);
          // element nv & 6 is even: the low half of its 32-bit word (taken with a shift and mask, not an element
          // extraction from the bf16 vector, which fed a 16-bit store wrongly)
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(w[(nv & 6) >> 1] & 0xFFFFu), Ob,
                                                part && (nv & 1) ? o + 2u * (nv & 6) : OOB, 0, 0);
        }
      }
    }
  }
}

}  // namespace

bool act_apply_eligible(int bp, const void* in, int64_t ldi, const void* out, int64_t ldo, int T) {
  auto al = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  return bp >= 8 && bp <= MAXB && bp % 8 == 0 && ldi % 8 == 0 && ldo % 8 == 0 && al(in) && al(out) &&
         (double)T * ldi * 2 < 4294967296.0 &&  // 32-bit byte offsets into the input
         (double)T * ldo * 2 < 2147483648.0;    // the output buffer under 2 GB
}

hipError_t launch_act_operand(const float* F, int bp, int d, int nblk, bool trans, __bf16* Bt, hipStream_t st) {
  const int64_t total = (int64_t)nblk * bp * bp;
  if (total == 0) return hipSuccess;
  ProfScope prof(POET_K_MISC, st, 0.0, 6.0 * total);
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 2048);
  hipLaunchKernelGGL(k_act_operand, dim3(grid), dim3(256), 0, st, F, bp, d, nblk, trans ? 1 : 0, Bt);
  return hipGetLastError();
}

hipError_t launch_act_apply(const __bf16* in, int64_t ldi, __bf16* out, int64_t ldo, const __bf16* Bt, int T, int d,
                            int bp, int nblk, hipStream_t st) {
  if (T <= 0 || nblk <= 0) return hipSuccess;
  ActArgs a;
  a.in = in; a.ldi = ldi; a.out = out; a.ldo = ldo; a.Bt = Bt; a.T = T; a.d = d; a.bp = bp; a.nblk = nblk;
  // token tiles per workgroup: about two workgroups per CU over the whole launch, at least two tiles each (so that
  // the operand load is shared by some tiles)
  const int ntile = (T + TM - 1) / TM;
  const int want = std::max(1, 512 / nblk);
  a.tiles_per_wg = std::max(2, (ntile + want - 1) / want);
  a.ngrp = (ntile + a.tiles_per_wg - 1) / a.tiles_per_wg;
  const int64_t nb = (int64_t)nblk * a.ngrp;
  ProfScope prof(POET_K_APPLY, st, 2.0 * T * (double)bp * d, 4.0 * T * (double)d);
  const unsigned grid = (unsigned)((nb + 7) / 8 * 8);
  if (act_frag_layout(bp)) {
    if (bp <= 64) hipLaunchKernelGGL((act_apply_kernel<4, true>), dim3(grid), dim3(AT), 0, st, a);
    else if (bp <= 128) hipLaunchKernelGGL((act_apply_kernel<8, true>), dim3(grid), dim3(AT), 0, st, a);
    else hipLaunchKernelGGL((act_apply_kernel<16, true>), dim3(grid), dim3(AT), 0, st, a);
  } else {
    if (bp <= 64) hipLaunchKernelGGL((act_apply_kernel<4, false>), dim3(grid), dim3(AT), 0, st, a);
    else if (bp <= 128) hipLaunchKernelGGL((act_apply_kernel<8, false>), dim3(grid), dim3(AT), 0, st, a);
    else hipLaunchKernelGGL((act_apply_kernel<16, false>), dim3(grid), dim3(AT), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace poet
