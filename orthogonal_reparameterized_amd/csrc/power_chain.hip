// Power chain X_{j+1} = Q X_j (j = 0 .. steps-1) of every primitive of a side, in one launch, for primitives of
// size bp <= 256 (POET-BS blocks). It serves two steps of the layer:
//   the Cayley-Neumann build   X_0 = Q, so X_j = Q^{j+1}. The kernel writes the saved powers Q^2 .. Q^k (bf16)
//     and completes the factor R_k = I + 2 Q + 2 (Q^2 + .. + Q^k) + Q^{k+1} in float32 on top of I + 2 Q, which
//     the caller has written with the linear term exact from theta.
//   the Neumann adjoint        X_0 = dR, so X_j = Q^j dR = H_j, written (bf16) side by side for j = 0..steps.
// Q comes from the saved bf16 power Q (the caller's first saved power).
// Several sides can share one launch (a table of up to MAXG sides, side = blockIdx.y), so that the blocks of all
// the linears of a transformer block fill the machine together.
// Column strips are independent (X_{j+1}[:, S] = Q X_j[:, S]), so one workgroup owns one 64-column strip of one
// primitive through all steps: Q stays resident in LDS (bp x bp bf16, up to 128 KB), the strip lives transposed
// in LDS (64 x bp bf16, 32 KB) and is overwritten by each new power after a barrier. Products run on
// v_mfma_f32_32x32x16_bf16 with float32 accumulation; each power is rounded to bf16 before it feeds the next
// product (as a bf16 operand would be).
#include <algorithm>

#include "strip_mma.h"

namespace poet {
namespace {

using namespace strip;

// barrier for LDS hazards only: the global stores of the powers are left in flight (nothing here reads them back)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool BUILD>
__global__ __launch_bounds__(NT) void power_chain_kernel(const ChainGroup G) {
  __shared__ __attribute__((aligned(16))) char smem[A_BYTES + X_BYTES];  // 160 KB
  char* Aq = smem;            // Q[i][k]
  char* Xs = smem + A_BYTES;  // X[k][n] stored as Xs[n][k]
  ChainArgs c;
  {
    const ChainArgs& t = G.a[blockIdx.y];
    c.bp = keep_s(t.bp); c.nprim = keep_s(t.nprim); c.steps = keep_s(t.steps); c.build = BUILD;
    c.prim = keep_s(t.prim); c.A = keep_s(t.A); c.sA = keep_s(t.sA);
    c.X0 = keep_s(t.X0); c.ldx0 = keep_s(t.ldx0); c.sx0 = keep_s(t.sx0);
    c.Y = keep_s(t.Y); c.ldy = keep_s(t.ldy); c.sy = keep_s(t.sy); c.jstep = keep_s(t.jstep);
    c.write_x0 = keep_s(t.write_x0);
    c.ops = keep_s(t.ops); c.d = keep_s(t.d); c.mode = keep_s(t.mode);
  }
  const int bp = c.bp, nstrips = (bp + SW - 1) / SW;
  if ((int)blockIdx.x >= c.nprim * nstrips) return;
  const int p = blockIdx.x / nstrips, n0 = (blockIdx.x % nstrips) * SW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rowsA = min(MAXB, (bp + 63) / 64 * 64);  // rows the waves read
  const int kpad = kpad_of(bp);                      // K extent of the products (zero beyond bp)

  // Q -> LDS from the bf16 blocks: thread = (16-byte chunk tid % 32, first row tid / 32), 8 rows apart; loads
  // are unconditional at a valid address and issued in groups of 8 before their LDS stores
  {
    const __bf16* Ab = c.A + (int64_t)p * c.sA;
    const int ch = tid & 31;
    const bool chin = ch * 8 < bp;
    for (int i0 = tid >> 5; i0 < rowsA; i0 += 64) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 8;
        const bool in = chin && i < bp;
        v[u] = *reinterpret_cast<const u32x4*>(Ab + (in ? (int64_t)i * bp + ch * 8 : 0));
        if (!in) v[u] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 8;
        if (ch * 8 < kpad) *reinterpret_cast<u32x4*>(Aq + i * ROWB + ((ch ^ (i & 15)) << 4)) = v[u];
      }
    }
  }
  if constexpr (BUILD) {
    __syncthreads();
    // X_0 = Q strip, transposed from the staged Q: thread = (column n = tid % 64, rows tid / 64 + 4t)
    const int n = tid & 63;
    for (int k = tid >> 6; k < kpad; k += 4) sts(Xs, n, k, n0 + n < bp ? lds(Aq, k, n0 + n) : (__bf16)0.f);
  } else {
    // X_0 strip -> LDS (transposed) in float32 chunks of 4 columns: thread = (chunk tid % 16, rows tid / 16 + 16t);
    // H_0 = bf16(X_0) to the output when asked
    const float* X0 = c.X0 + (int64_t)p * c.sx0;
    const int n = (tid & 15) * 4, gn = n0 + n;
    for (int k0 = tid >> 4; k0 < kpad; k0 += 64) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * 16;
        const bool in = k < bp && gn < bp;
        v[u] = *reinterpret_cast<const f32x4*>(X0 + (in ? (int64_t)k * c.ldx0 + gn : 0));
        if (!in) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * 16;
        if (k >= kpad) continue;
        bf16x4 b;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          b[t] = (__bf16)v[u][t];
          sts(Xs, n + t, k, b[t]);
        }
        if (c.write_x0 && k < bp && gn < bp)
          *reinterpret_cast<bf16x4*>(c.Y + (int64_t)p * c.sy + (int64_t)k * c.ldy + gn) = b;
      }
    }
  }
  __syncthreads();

  const int wr = wave * 64;  // this wave's 64 rows of the strip
  // BUILD: S = I + 2Q (the caller's prim) + 2 (Q^2 + .. + Q^k) with the bf16 powers, at this lane's outputs (plain
  // registers, updated without branches); the 64 loads are unconditional (index 0 stands in outside the block)
  float S[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S[a][b][r] = 0.f;
        if constexpr (BUILD) {
          const int i = acc_row(wr, a, r, lane), gn = n0 + acc_col(b, lane);
          const bool in = i < bp && gn < bp;
          S[a][b][r] = c.prim[in ? (int64_t)p * bp * bp + (int64_t)i * bp + gn : 0];
        }
      }
  for (int j = 1; j <= c.steps; ++j) {
    f32x16 acc[2][2];
    zero(acc);
    if (wr < bp) mma_strip(Aq, Xs, wr, kpad, lane, acc);
    lds_barrier();  // every wave is done reading the strip of X_{j-1}
    const bool last = j == c.steps;
    if (BUILD && last) {  // R_k = S + Q^{k+1}
      // The finished strip leaves through LDS (both regions are free: every wave is past its last product):
      // float32 rows [i][n] (pitch RP floats: the two half-waves of a write land in different banks) in the Q
      // region, and, for the operand copies, the bf16 strip transposed in the strip buffer. Then every store to
      // global memory is a coalesced 16-byte chunk.
      constexpr int RP = 72;
      float* Rs = reinterpret_cast<float*>(Aq);
      const int cb = c.mode == 1 ? bp : min(bp, c.d - p * bp);  // the block's size (zero outside it in ops)
      const bool ops = c.ops != nullptr;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = acc_row(wr, a, r, lane), n = acc_col(b, lane);
            const float v = S[a][b][r] + acc[a][b][r];
            Rs[i * RP + n] = v;
            if (ops && i < bp) sts(Xs, n, i, (__bf16)(i < cb && n0 + n < cb ? v - (i == n0 + n ? 1.f : 0.f) : 0.f));
          }
      lds_barrier();
      const int nv = min(SW, bp - n0);  // columns of this strip inside the block
      float* prim = c.prim + (int64_t)p * bp * bp;
      __bf16* opsF = ops ? c.ops + (int64_t)p * bp * bp : nullptr;
      const bool frag = act_frag_layout(bp);  // operand copies in fragment order (else in row order)
      for (int e = tid; e < bp * (SW / 4); e += NT) {  // rows i, 4-column chunks
        const int i = e / (SW / 4), n4 = (e % (SW / 4)) * 4;
        if (n4 >= nv) continue;
        const f32x4 v = *reinterpret_cast<const f32x4*>(Rs + i * RP + n4);
        *reinterpret_cast<f32x4*>(prim + (int64_t)i * bp + n0 + n4) = v;
        if (ops) {  // the third copy: the delta F - I of the whole block (padding included), in row order
          bf16x4 r;
#pragma unroll
          for (int t = 0; t < 4; ++t) r[t] = (__bf16)(v[t] - (i == n0 + n4 + t ? 1.f : 0.f));
          *reinterpret_cast<bf16x4*>(c.ops + 2 * (int64_t)c.nprim * bp * bp + (int64_t)p * bp * bp + (int64_t)i * bp +
                                     n0 + n4) = r;
        }
        if (ops && !frag) {
          bf16x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            w[t] = (__bf16)(i < cb && n0 + n4 + t < cb ? v[t] - (i == n0 + n4 + t ? 1.f : 0.f) : 0.f);
          *reinterpret_cast<bf16x4*>(opsF + (int64_t)i * bp + n0 + n4) = w;
        }
      }
      if (ops && frag) {  // F's rows (operand row j = i, k = column n) in fragment order: 8 columns per 16 bytes
        const int nks = nv / 16;  // k-steps this strip covers (nv is a multiple of 32 here)
        for (int e = tid; e < (bp / 32) * nks * 64; e += NT) {
          const int l = e & 63, s = (e >> 6) % nks, g = (e >> 6) / nks;
          const int i = 32 * g + (l & 31), n = 16 * s + 8 * (l >> 5);
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(Rs + i * RP + n);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(Rs + i * RP + n + 4);
          bf16x8 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            w[t] = (__bf16)(i < cb && n0 + n + t < cb ? v0[t] - (i == n0 + n + t ? 1.f : 0.f) : 0.f);
            w[t + 4] = (__bf16)(i < cb && n0 + n + t + 4 < cb ? v1[t] - (i == n0 + n + t + 4 ? 1.f : 0.f) : 0.f);
          }
          *reinterpret_cast<bf16x8*>(opsF + act_frag_index(bp, i, n0 + n)) = w;
        }
      }
      if (ops) {  // the transpose: operand row j = n0 + n, k = i (F's column n0 + n), from the strip buffer
        __bf16* opsT = c.ops + (int64_t)c.nprim * bp * bp + (int64_t)p * bp * bp;
        const int nch = bp / 8;
        for (int e = tid; e < SW * nch; e += NT) {
          // fragment order: consecutive threads take consecutive lanes of one fragment (16-byte chunks of one
          // column group and k-step); row order: consecutive chunks of one row
          int n, ch;
          if (frag) {
            const int l = e & 63, gs = e >> 6, s = gs % (bp / 16), gl = gs / (bp / 16);
            n = 32 * gl + (l & 31);
            ch = 2 * s + (l >> 5);
          } else {
            n = e / nch;
            ch = e - n * nch;
          }
          if (n < nv) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(Xs + n * ROWB + ((ch ^ (n & 15)) << 4));
            const int64_t o = frag ? act_frag_index(bp, n0 + n, ch * 8) : (int64_t)(n0 + n) * bp + ch * 8;
            *reinterpret_cast<u32x4*>(opsT + o) = v;
          }
        }
      }
      break;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int n = acc_col(b, lane), gn = n0 + n;
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // 4 consecutive rows per group of accumulators
          const int i0 = acc_row(wr, a, q * 4, lane);
          bf16x4 v4;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v4[t] = (__bf16)acc[a][b][q * 4 + t];
            if (BUILD) S[a][b][q * 4 + t] += 2.f * (float)v4[t];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (i0 + t < bp && gn < bp) c.Y[(int64_t)p * c.sy + (int64_t)j * c.jstep + (int64_t)(i0 + t) * c.ldy + gn] = v4[t];
          if (!last) *reinterpret_cast<bf16x4*>(Xs + loff(n, i0)) = v4;  // next operand (rows >= bp stay zero)
        }
      }
    lds_barrier();
  }
}

}  // namespace

bool power_chain_eligible(int bp, int dt, const void* A) {
  return dt == BF16 && bp > 0 && bp <= MAXB && bp % 8 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0;
}

hipError_t launch_power_chain_group(const ChainGroup& g, int kclass, hipStream_t st) {
  if (g.n <= 0 || g.n > MAXG) return g.n == 0 ? hipSuccess : hipErrorInvalidValue;
  int gx = 0, build = -1;
  double flops = 0, bytes = 0;
  for (int i = 0; i < g.n; ++i) {
    const ChainArgs& c = g.a[i];
    if (c.bp <= 0 || c.bp > MAXB) return hipErrorInvalidValue;
    if (build >= 0 && build != c.build) return hipErrorInvalidValue;
    build = c.build;
    if (c.nprim <= 0 || c.steps <= 0) continue;
    gx = std::max(gx, c.nprim * ((c.bp + SW - 1) / SW));
    flops += 2.0 * c.bp * (double)c.bp * c.bp * c.steps * c.nprim;
    bytes += (double)c.nprim * c.bp * c.bp * 2.0 * (c.steps + 2);
  }
  if (gx == 0) return hipSuccess;
  ProfScope prof(kclass, st, flops, bytes);
  // sides with fewer workgroups than the widest one leave the excess of their row of the grid at once
  const dim3 grid(gx, g.n);
  if (build) hipLaunchKernelGGL(power_chain_kernel<true>, grid, dim3(NT), 0, st, g);
  else hipLaunchKernelGGL(power_chain_kernel<false>, grid, dim3(NT), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_power_chain(const ChainArgs& c, int kclass, hipStream_t st) {
  ChainGroup g;
  g.n = 1;
  g.a[0] = c;
  return launch_power_chain_group(g, kclass, st);
}

}  // namespace poet
