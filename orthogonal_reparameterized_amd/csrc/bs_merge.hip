// In-place merge of block-diagonal orthogonal factors into the fixed weight, W0 <- R W0 P (POET, the
// merge-then-reinitialize step), for blocks of up to 256, to float32 accuracy on bf16 MFMA.
//
// Two passes over W0, each in place:
//   P pass   W0[i, J] <- W0[i, J] + W0[i, J] dP_J          (every row i, every block J of P)
//   R pass   W0[I, j] <- W0[I, j] + dR_I W0[I, j]          (every block I of R, every column j)
// with dF = F - I. A workgroup owns a panel of 128 rows (P pass) or 128 columns (R pass) across one whole block,
// so it reads exactly the elements it writes and no other workgroup touches them: the pass is race-free in place.
//
// float32 accuracy from bf16 products: each float32 operand x is split as x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi) (together 16 significant bits), and the delta product is taken as
//   a b ~ hi(a) hi(b) + hi(a) lo(b) + lo(a) hi(b)
// on v_mfma_f32_32x32x16_bf16 with float32 accumulation; the dropped lo(a) lo(b) term and the rounding of the lo
// parts are below 2^-16 of |a||b| per product. The identity part (the W0 element itself) is exact: it is the
// accumulator's starting value. The result differs from a float32 product by about 2^-17 |dF| |W0| per element.
//
// Data flow of one workgroup (4 waves, 32 panel lines each):
//   resident operand  the W0 panel over the block, loaded once into registers and split into hi/lo MFMA
//                     fragments (16 k-steps x 2 x 8 bf16 per lane);
//   streamed operand  the factor delta in 64-line strips, pre-split into hi/lo bf16 by a small kernel and copied
//                     into LDS by DMA (global_load_lds), one strip (64 KB) at a time; two workgroups share a CU.
// The R pass also writes the bf16 (or float32) shadow copy of the merged weight.
#include <type_traits>
#include <vector>

#include "poet.h"
#include "strip_mma.h"

namespace poet {
namespace {

using namespace strip;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int MT = 256;              // 4 waves
constexpr int PANEL = 128;           // panel lines per workgroup (32 per wave)
constexpr int STRIP_BYTES = 65536;   // 64 lines x 512 B of hi, then the same of lo
constexpr int NKS = MAXB / 16;       // k-steps of a 256 block
constexpr int WAIT_VM0 = 0x0F70;     // s_waitcnt vmcnt(0)

struct MergeArgs {
  float* W; int64_t ld; int m, n;
  int bp, nblk;        // block size and block count of the factor
  const char* split;   // pre-split deltas: strip s of block b at split + (b * nstr + s) * STRIP_BYTES
  int nstr;            // strips per block in that buffer: ceil(bp / 64)
  void* shadow; int sh_dt; int64_t ld_sh;  // R pass: copy of the merged weight (nullable)
  int vec;             // P pass: rows 16-byte aligned and whole 8-column groups in every block (float4 loads)
  int first;           // first logical workgroup of this entry in its launch
};
// The passes of up to MAXG weights (same pass, same k-step class) in one launch: entry e owns logical workgroups
// [a[e].first, a[e + 1].first), and total is the sum over the entries.
struct MergeGroup {
  int n = 0, total = 0;
  MergeArgs a[MAXG];
};

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& h, bf16x8& l) {
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    h[v] = (__bf16)x[v];
    l[v] = (__bf16)(x[v] - (float)h[v]);
  }
}

// Pre-split factor deltas. For block b (size c = min(bp, d - b bp)) and strip line r, 16-byte chunk q:
//   value(r, k) = F_b[k][r] - [k == r] (transpose: the P pass streams columns of dP) or F_b[r][k] - [r == k],
// zero outside r, k < c; hi at line r of the strip's first 32 KB, lo at the same place in its second 32 KB.
// Grouped over up to 2 MAXG factors: workgroups [a[e].wg0, a[e + 1].wg0) take factor e.
struct SplitEntry {
  const float* prim; char* out;
  int bp, d, nblk, nstr, transpose, wg0;
};
struct SplitGroup {
  int n = 0;
  SplitEntry a[2 * MAXG];
};
__global__ void k_merge_split(const SplitGroup G) {
  int e = 0;
  for (int q = 1; q < G.n; ++q)
    if ((int)blockIdx.x >= G.a[q].wg0) e = q;
  const SplitEntry& ge = G.a[e];
  const float* prim = keep_s(ge.prim);
  char* out = keep_s(ge.out);
  const int bp = keep_s(ge.bp), d = keep_s(ge.d), nblk = keep_s(ge.nblk), nstr = keep_s(ge.nstr);
  const int transpose = keep_s(ge.transpose), wg0 = keep_s(ge.wg0);
  const int nwg = (e + 1 < G.n ? G.a[e + 1].wg0 : (int)gridDim.x) - wg0;
  const int lines = nstr * 64;
  const int64_t total = (int64_t)nblk * lines * 32;
  for (int64_t t = (int64_t)(blockIdx.x - wg0) * blockDim.x + threadIdx.x; t < total; t += (int64_t)nwg * blockDim.x) {
    // transpose: consecutive threads take consecutive lines (coalesced column reads); else consecutive chunks
    int r, q, b;
    if (transpose) { r = (int)(t % lines); q = (int)((t / lines) % 32); b = (int)(t / ((int64_t)lines * 32)); }
    else { q = (int)(t % 32); r = (int)((t / 32) % lines); b = (int)(t / ((int64_t)lines * 32)); }
    const int c = min(bp, d - b * bp);
    const float* F = prim + (int64_t)b * bp * bp;
    float x[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int k = q * 8 + v;
      const bool in = r < c && k < c;
      const float f = F[in ? (transpose ? (int64_t)k * bp + r : (int64_t)r * bp + k) : 0];
      x[v] = in ? f - (k == r ? 1.f : 0.f) : 0.f;
    }
    bf16x8 h, l;
    split8(x, h, l);
    char* o = out + ((int64_t)b * nstr + r / 64) * STRIP_BYTES + (r % 64) * ROWB + q * 16;
    *reinterpret_cast<bf16x8*>(o) = h;
    *reinterpret_cast<bf16x8*>(o + STRIP_BYTES / 2) = l;
  }
}

// W0 (and the shadow) are addressed through raw buffer resources (base, size in bytes): a load past the end returns
// 0 and a store past the end is dropped, so edge tiles need no clamped addresses. Offsets are 32-bit byte offsets
// (each matrix under 2 GB).
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 buffer descriptor word 3 (raw buffer, 32-bit data)
constexpr uint32_t OOB = 0x80000000u;    // an offset past the end of any buffer here (each is under 2 GB)

// the buffer builtins move raw 32-bit words: reinterpret, never convert
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void bstore(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}

// NK: k-steps of 16 covering the block size (4, 8 or 16); loops over them are fully unrolled with no branches, so
// every load is issued up front (values outside the block are replaced by zeros)
template <bool RS, int NK>
__global__ __launch_bounds__(MT, 2) void merge_pass_kernel(const MergeGroup G) {
  __shared__ __attribute__((aligned(16))) char buf[STRIP_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD-aware order: hardware workgroup b runs on XCD b % 8; consecutive logical ids (the panels of one block,
  // which stream the same strips) go to one XCD
  const int per = (G.total + 7) / 8;
  const int L = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (L >= G.total) return;
  int e = 0;
  for (int q = 1; q < G.n; ++q)
    if (L >= G.a[q].first) e = q;
  MergeArgs a;
  {
    const MergeArgs& ga = G.a[e];
    a.W = keep_s(ga.W); a.ld = keep_s(ga.ld); a.m = keep_s(ga.m); a.n = keep_s(ga.n);
    a.bp = keep_s(ga.bp); a.nblk = keep_s(ga.nblk); a.split = keep_s(ga.split); a.nstr = keep_s(ga.nstr);
    a.shadow = keep_s(ga.shadow); a.sh_dt = keep_s(ga.sh_dt); a.ld_sh = keep_s(ga.ld_sh);
    a.vec = keep_s(ga.vec); a.first = keep_s(ga.first);
  }
  const int pdim = RS ? a.n : a.m;    // panel dimension: W columns (R pass) or rows (P pass)
  const int bdim = RS ? a.m : a.n;    // block dimension
  const int npan = (pdim + PANEL - 1) / PANEL;
  const int blk = (L - a.first) / npan, pan = (L - a.first) % npan;
  const int b0 = blk * a.bp, c = min(a.bp, bdim - b0);
  const int nstr = (c + 63) / 64;
  const int line0 = pan * PANEL + wave * 32;            // this wave's first panel line
  const int p = line0 + (lane & 31);                    // this lane's panel line (resident operand)
  const bool pin = p < pdim;
  const int kh = (lane >> 5) * 8;
  const uint32_t ld4 = (uint32_t)a.ld * 4;              // row pitch in bytes
  const __amdgpu_buffer_rsrc_t W =
      __builtin_amdgcn_make_buffer_rsrc(a.W, (short)0, (int)((uint32_t)a.m * ld4), RSRC_WORD3);

  // ---- resident operand: W0 over the block at this lane's line, split into hi/lo fragments
  //   P pass: A fragment, row p, k = block columns;  R pass: B fragment, column p, k = block rows
  // Loaded and split four k-steps at a time (a scheduling barrier keeps the loads of later groups from being
  // hoisted, which would hold every raw float32 value and its split at once).
  bf16x8 rh[NK], rl[NK];
#pragma unroll
  for (int g = 0; g < NK; g += 4) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = (g + u) * 16 + kh;  // first of this lane's 8 block indices
      if constexpr (RS) {   // column p of rows b0 + k + v (rows past the matrix read as 0)
        const uint32_t o = (uint32_t)(b0 + k) * ld4 + (uint32_t)p * 4;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float f = bload(W, o + v * ld4);
          x[u][v] = pin && k + v < c ? f : 0.f;
        }
      } else if (a.vec) {  // 16-byte aligned rows, c % 8 == 0: two float4 loads
        const uint32_t o = (uint32_t)p * ld4 + (uint32_t)(b0 + k) * 4;
        const f32x4 u0 = bload4(W, o);
        const f32x4 u1 = bload4(W, o + 16);
        const bool in = k < c;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[u][v] = in ? u0[v] : 0.f;
          x[u][v + 4] = in ? u1[v] : 0.f;
        }
      } else {
        const uint32_t o = (uint32_t)p * ld4 + (uint32_t)(b0 + k) * 4;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float f = bload(W, o + v * 4);
          x[u][v] = k + v < c ? f : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) split8(x[u], rh[g + u], rl[g + u]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // accumulator register r of tile t of strip s covers
  //   P pass: W0 row line0 + ti, block column s*64 + t*32 + tj;   R pass: block row s*64 + t*32 + ti, W0 column line0 + tj
  // with ti = 8 (r / 4) + 4 (lane / 32) + r % 4 and tj = lane % 32
  const int ti0 = (lane >> 5) * 4, tj = lane & 31;
  // byte offset of this lane's element of register 0, tile 0, strip 0; register r adds cr(r) rows, tile t and
  // strip s add 32 t + 64 s block lines
  const uint32_t base = RS ? (uint32_t)(b0 + ti0) * ld4 + (uint32_t)(line0 + tj) * 4
                           : (uint32_t)(line0 + ti0) * ld4 + (uint32_t)(b0 + tj) * 4;
  const uint32_t bstep = RS ? 32 * ld4 : 32 * 4;  // one tile (32 block lines)
  // R pass: the shadow copy, addressed the same way (element size esz, row pitch ld_sh)
  const uint32_t esz = a.sh_dt == BF16 ? 2 : 4, lds4 = (uint32_t)a.ld_sh * esz;
  const __amdgpu_buffer_rsrc_t SH = __builtin_amdgcn_make_buffer_rsrc(
      a.shadow ? a.shadow : a.W, (short)0, a.shadow ? (int)((uint32_t)a.m * lds4) : 0, RSRC_WORD3);
  const uint32_t sbase = (uint32_t)(b0 + ti0) * lds4 + (uint32_t)(line0 + tj) * esz;
  const char* strips = a.split + (int64_t)blk * a.nstr * STRIP_BYTES;
  uint32_t dma_off[2];
  {
    const int h = wave * 2 + (lane >> 5);
#pragma unroll
    for (int e = 0; e < 2; ++e) dma_off[e] = h * ROWB + (((lane & 31) ^ (8 * e + h)) << 4);
  }
  for (int s = 0; s < nstr; ++s) {
    // accumulators start at the W0 elements they update (the identity part, exact). The tile base offsets pass
    // through an empty asm statement so that the compiler recomputes the per-register offsets in each strip
    // instead of keeping 32 of them live across the loop.
    uint32_t tb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      tb[t] = base + (uint32_t)(2 * s + t) * bstep;
      asm volatile("" : "+v"(tb[t]));
    }
    f32x16 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = bload(W, tb[t] + (uint32_t)((r >> 2) * 8 + (r & 3)) * ld4);
    // strip s of the block's deltas -> LDS. DMA instruction q of wave w fills LDS bytes [(4q + w) KB, +1 KB), lane l
    // the 16 bytes at +16 l: strip line 8q + h (h = 2w + l / 32; lines 64.. are the lo half), physical chunk l % 32,
    // whose logical chunk is (l % 32) ^ (line % 16) = (l % 32) ^ (8 (q % 2) + h). The source offset is therefore
    // q * 4 KB (uniform) + h * 512 + 16 * that chunk (one of two per-lane values).
    {
      const char* src = strips + (int64_t)s * STRIP_BYTES;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        __builtin_amdgcn_global_load_lds((gbl_void*)(src + q * 4096 + dma_off[q & 1]),
                                         (lds_void*)(buf + (q * 4 + wave) * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    __syncthreads();

    // k-step loop, software-pipelined by hand: the fragments of step ks + 1 are read while step ks multiplies;
    // a scheduling barrier per step stops the compiler from hoisting every read (and its registers) to the top
    bf16x8 sh[2][2], sl[2][2];  // [pipeline slot][tile]
    auto read_frags = [&](int ks, int slot) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int off = loff(t * 32 + tj, ks * 16 + kh);
        sh[slot][t] = *reinterpret_cast<const bf16x8*>(buf + off);
        sl[slot][t] = *reinterpret_cast<const bf16x8*>(buf + STRIP_BYTES / 2 + off);
      }
    };
    read_frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < NK) read_frags(ks + 1, cur ^ 1);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (RS) {  // rows: strip lines (delta rows); columns: resident W0 columns
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh[cur][t], rh[ks], acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl[cur][t], rh[ks], acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh[cur][t], rl[ks], acc[t], 0, 0, 0);
        } else {             // rows: resident W0 rows; columns: strip lines (delta columns)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rh[ks], sh[cur][t], acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rh[ks], sl[cur][t], acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rl[ks], sh[cur][t], acc[t], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // every wave is done reading the strip before the next one is copied in

    // stores, without branches: a position outside the block or the matrix gets an offset past the end of the
    // buffer (OOB), which the hardware drops; rows past the matrix are past its end already
    // (three copies of the store loop under uniform branches: W0 only, W0 + bf16 shadow, W0 + float32 shadow)
    auto store_tiles = [&](auto shadow_kind) {
      constexpr int SK = decltype(shadow_kind)::value;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int bl = s * 64 + t * 32;  // first block line of the tile
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = (r >> 2) * 8 + (r & 3);
          const bool in = RS ? (bl + ti0 + cr < c && line0 + tj < a.n) : (bl + tj < c);
          bstore(acc[t][r], W, in ? tb[t] + (uint32_t)cr * ld4 : OOB);
          if constexpr (SK != 0) {
            const uint32_t so = in ? sbase + (uint32_t)(bl + cr) * lds4 : OOB;
            if constexpr (SK == 1)
              __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)acc[t][r]), SH, so, 0, 0);
            else
              bstore(acc[t][r], SH, so);
          }
        }
      }
    };
    if (!RS || !a.shadow) store_tiles(std::integral_constant<int, 0>());
    else if (esz == 2) store_tiles(std::integral_constant<int, 1>());
    else store_tiles(std::integral_constant<int, 2>());
  }
}

template <int NK>
void launch_pass(bool rside, const MergeGroup& g, hipStream_t st) {
  const unsigned grid = (unsigned)((g.total + 7) / 8 * 8);
  if (rside) hipLaunchKernelGGL((merge_pass_kernel<true, NK>), dim3(grid), dim3(MT), 0, st, g);
  else hipLaunchKernelGGL((merge_pass_kernel<false, NK>), dim3(grid), dim3(MT), 0, st, g);
}

int nk_class(int bp) { return bp <= 64 ? 0 : bp <= 128 ? 1 : 2; }

// one pass (rside) of every item whose factor falls in k-step class cls, MAXG items per launch
hipError_t launch_pass_class(const MergeItem* it, int n, const std::vector<char*>& split, bool rside, int cls,
                             hipStream_t st) {
  MergeGroup g;
  auto flush = [&]() -> hipError_t {
    if (g.n == 0) return hipSuccess;
    if (cls == 0) launch_pass<4>(rside, g, st);
    else if (cls == 1) launch_pass<8>(rside, g, st);
    else launch_pass<16>(rside, g, st);
    g = MergeGroup();
    return hipGetLastError();
  };
  for (int i = 0; i < n; ++i) {
    const MergeItem& x = it[i];
    const int bp = rside ? x.bpR : x.bpP, nblk = rside ? x.nR : x.nP;
    if (x.m <= 0 || x.n <= 0 || nblk <= 0 || nk_class(bp) != cls) continue;
    MergeArgs& a = g.a[g.n++];
    a.W = x.W; a.ld = x.ld; a.m = x.m; a.n = x.n; a.bp = bp; a.nblk = nblk; a.split = split[2 * i + (rside ? 1 : 0)];
    a.nstr = (bp + 63) / 64;
    a.shadow = rside ? x.shadow : nullptr; a.sh_dt = x.sh_dt; a.ld_sh = x.ld_sh;
    // float4 loads of the P pass need 16-byte aligned rows and whole 8-column groups in every block
    a.vec = x.ld % 4 == 0 && reinterpret_cast<uintptr_t>(x.W) % 16 == 0 && bp % 8 == 0 && x.n % 8 == 0;
    a.first = g.total;
    g.total += ((rside ? x.n : x.m) + PANEL - 1) / PANEL * nblk;
    if (g.n == MAXG) {
      const hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
  }
  return flush();
}

}  // namespace

bool bs_merge_eligible(int bp, int m, int64_t ld) { return bp >= 1 && bp <= MAXB && (double)m * ld * 4 < 2147483648.0; }

size_t bs_merge_split_bytes(int bp, int nblk) { return (size_t)nblk * ((bp + 63) / 64) * STRIP_BYTES; }

size_t bs_merge_group_bytes(const MergeItem* it, int n) {
  size_t b = 0;
  for (int i = 0; i < n; ++i) b += bs_merge_split_bytes(it[i].bpP, it[i].nP) + bs_merge_split_bytes(it[i].bpR, it[i].nR);
  return b;
}

hipError_t launch_bs_merge_group(const MergeItem* it, int n, char* split, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  double flops = 0, bytes = 0;
  for (int i = 0; i < n; ++i) {
    const double mn = (double)it[i].m * it[i].n;
    flops += 6.0 * mn * (it[i].bpR + it[i].bpP);
    bytes += mn * (16.0 + (it[i].shadow ? dtype_size(it[i].sh_dt) : 0));
  }
  ProfScope prof(POET_K_MERGE, st, flops, bytes);
  // every factor's deltas pre-split into its own region of the scratch: P of item i at split[2 i], R at split[2 i + 1]
  std::vector<char*> sp(2 * (size_t)n);
  SplitGroup sg;
  int wg = 0;
  for (int i = 0; i < n; ++i) {
    for (int r = 0; r < 2; ++r) {
      const int bp = r ? it[i].bpR : it[i].bpP, nblk = r ? it[i].nR : it[i].nP;
      sp[2 * i + r] = split;
      split += bs_merge_split_bytes(bp, nblk);
      if (it[i].m <= 0 || it[i].n <= 0 || nblk <= 0) continue;
      SplitEntry& e = sg.a[sg.n++];
      e.prim = r ? it[i].primR : it[i].primP; e.out = sp[2 * i + r];
      e.bp = bp; e.d = r ? it[i].m : it[i].n; e.nblk = nblk; e.nstr = (bp + 63) / 64; e.transpose = r ? 0 : 1;
      e.wg0 = wg;
      const int64_t items = (int64_t)nblk * e.nstr * 64 * 32;
      wg += (int)std::min<int64_t>((items + 255) / 256, 1024);
      if (sg.n == 2 * MAXG) {
        hipLaunchKernelGGL(k_merge_split, dim3(wg), dim3(256), 0, st, sg);
        const hipError_t er = hipGetLastError();
        if (er != hipSuccess) return er;
        sg = SplitGroup();
        wg = 0;
      }
    }
  }
  if (sg.n > 0) {
    hipLaunchKernelGGL(k_merge_split, dim3(wg), dim3(256), 0, st, sg);
    const hipError_t er = hipGetLastError();
    if (er != hipSuccess) return er;
  }
  for (int rside = 0; rside < 2; ++rside)  // every P pass, then every R pass
    for (int cls = 0; cls < 3; ++cls) {
      const hipError_t er = launch_pass_class(it, n, sp, rside != 0, cls, st);
      if (er != hipSuccess) return er;
    }
  return hipSuccess;
}

}  // namespace poet
