// Fused application of two block-diagonal orthogonal factors (POET-BS on both sides) to the fixed weight:
//   T = W0 P,   W = R T = R W0 P,   RW0 = R W0,
// for blocks of up to 256 (POET reparameterization W = R W0 P with block-diagonal R and P; the bf16 activation
// path). Each factor is applied as identity + delta: the delta (primitive minus I) and the other operand are
// rounded to bf16 for v_mfma_f32_32x32x16_bf16, the identity part is added in float32:
//   T   = W0 + bf16(W0) bf16(dP)        (float32; written as bf16 when asked)
//   W   = T + bf16(dR) bf16(T)          (written in the activation dtype)
//   RW0 = W0 + bf16(dR) bf16(W0)        (written as bf16)
// One workgroup owns 64 columns of one P block within one R block: all rows of the R block (up to 256) by the
// strip. Phase 1 stages the W0 tile of the (R block, P block) pair and the dP strip, phase 2 restages dR and
// keeps T of the strip transposed in LDS as the second product's operand, phase 3 swaps in the W0 strip for R W0.
// Every operand is read from its float32 source and converted while staged, so no bf16 copies are made.
#include "poet.h"
#include "strip_mma.h"

namespace poet {
namespace {

using namespace strip;

struct Frag {  // 64 float32 values at this lane's accumulator positions
  f32x16 v[2][2];
};

__global__ __launch_bounds__(NT) void bs_apply_kernel(const ApplyArgs c) {
  __shared__ __attribute__((aligned(16))) char smem[A_BYTES + X_BYTES];  // 160 KB
  char* Aq = smem;
  char* Xs = smem + A_BYTES;
  const int nsP = (c.bpP + SW - 1) / SW, nb = c.nR * c.nP * nsP;
  // XCD-aware order: hardware workgroup b runs on XCD b % 8; consecutive logical ids (the strips of one W0 tile,
  // then the P blocks of one R block) go to one XCD so that its L2 serves the shared tiles
  const int per = (nb + 7) / 8;
  const int L = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (L >= nb) return;
  const int s = L % nsP, cblk = (L / nsP) % c.nP, r = L / (nsP * c.nP);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wr = wave * 64;
  const int bpR = c.bpR, bpP = c.bpP;
  const int i_base = r * bpR, mr = min(bpR, c.m - i_base);
  const int j_base = cblk * bpP, nc = min(bpP, c.n - j_base);
  const int n0 = s * SW;                          // strip origin within the P block
  const int rowsA = min(MAXB, (bpR + 63) / 64 * 64);
  const int kR = kpad_of(bpR), kP = kpad_of(bpP);
  const float* W0 = c.W0 + (int64_t)i_base * c.ldw + j_base;
  const bool needT = c.Tb != nullptr || c.W != nullptr;

  // float32 W0 at this lane's output positions (the identity parts of T and of R W0)
  Frag w0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = acc_row(wr, a, q, lane), j = n0 + acc_col(b, lane);
        const bool in = i < mr && j < nc;
        w0.v[a][b][q] = W0[in ? (int64_t)i * c.ldw + j : 0];
        if (!in) w0.v[a][b][q] = 0.f;
      }

  f32x16 acc[2][2];
  if (needT) {
    // ---- phase 1: Aq = bf16 W0 tile (rows < mr, columns < nc, zero to rowsA x kP); Xs = bf16 dP strip, transposed
    {
      const int q4 = tid & 63;  // float4 chunk of a row: columns 4 q4 .. 4 q4 + 3
      for (int i0 = tid >> 6; i0 < rowsA; i0 += 32) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * 4;
          const bool in = i < mr && 4 * q4 < nc;  // row padding up to a multiple of 4 columns is readable
          v[u] = *reinterpret_cast<const f32x4*>(W0 + (in ? (int64_t)i * c.ldw + 4 * q4 : 0));
          if (!in) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * 4;
          if (4 * q4 >= kP) continue;
          bf16x4 b;
#pragma unroll
          for (int t = 0; t < 4; ++t) b[t] = (__bf16)(4 * q4 + t < nc ? v[u][t] : 0.f);
          *reinterpret_cast<bf16x4*>(Aq + loff(i, 4 * q4)) = b;
        }
      }
      // dP strip: Xs[n][k] = P[k][n0 + n] - (k == n0 + n), k < kP (zero at k >= nc or n0 + n >= nc)
      const float* Pb = c.primP + (int64_t)cblk * bpP * bpP;
      const int n = (tid & 15) * 4, gn = n0 + n;
      for (int k0 = tid >> 4; k0 < kP; k0 += 64) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = k0 + u * 16;
          const bool in = k < nc && gn < bpP;
          v[u] = *reinterpret_cast<const f32x4*>(Pb + (in ? (int64_t)k * bpP + gn : 0));
          if (!in) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = k0 + u * 16;
          if (k >= kP) continue;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float d = gn + t < nc ? v[u][t] - (k == gn + t ? 1.f : 0.f) : 0.f;
            sts(Xs, n + t, k, (__bf16)d);
          }
        }
      }
    }
    __syncthreads();
    zero(acc);
    if (wr < bpR) mma_strip(Aq, Xs, wr, kP, lane, acc);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] += w0.v[a][b];  // T (float32)
    if (c.Tb) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int i = acc_row(wr, a, q, lane), j = n0 + acc_col(b, lane);
            if (i < mr && j < nc) c.Tb[(int64_t)(i_base + i) * c.ldw + j_base + j] = (__bf16)acc[a][b][q];
          }
    }
    __syncthreads();  // phase 1 operands are dead
  }
  if (c.W == nullptr && c.RW0b == nullptr) return;

  // ---- phase 2: Aq = bf16 dR block; Xs = bf16 T strip (transposed, from the accumulators)
  {
    const float* Rb = c.primR + (int64_t)r * bpR * bpR;
    const int q4 = tid & 63;
    for (int i0 = tid >> 6; i0 < rowsA; i0 += 32) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 4;
        const bool in = i < mr && 4 * q4 < bpR;
        v[u] = *reinterpret_cast<const f32x4*>(Rb + (in ? (int64_t)i * bpR + 4 * q4 : 0));
        if (!in) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 4;
        if (4 * q4 >= kR) continue;
        bf16x4 b;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int k = 4 * q4 + t;
          b[t] = (__bf16)(k < mr ? v[u][t] - (i == k ? 1.f : 0.f) : 0.f);
        }
        *reinterpret_cast<bf16x4*>(Aq + loff(i, 4 * q4)) = b;
      }
    }
  }
  if (c.W) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 v4;
#pragma unroll
          for (int t = 0; t < 4; ++t) v4[t] = (__bf16)acc[a][b][q * 4 + t];  // rows >= mr hold zeros
          *reinterpret_cast<bf16x4*>(Xs + loff(acc_col(b, lane), acc_row(wr, a, q * 4, lane))) = v4;
        }
    __syncthreads();
    if (wr < bpR) mma_strip(Aq, Xs, wr, kR, lane, acc);  // acc = T + dR T
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int i = acc_row(wr, a, q, lane), j = n0 + acc_col(b, lane);
          if (i >= mr || j >= nc) continue;
          const int64_t o = (int64_t)(i_base + i) * c.ldw + j_base + j;
          if (c.w_dt == BF16) reinterpret_cast<__bf16*>(c.W)[o] = (__bf16)acc[a][b][q];
          else reinterpret_cast<float*>(c.W)[o] = acc[a][b][q];
        }
    if (c.RW0b == nullptr) return;
    __syncthreads();  // the T strip is dead
  }

  // ---- phase 3: Xs = bf16 W0 strip (transposed): Xs[n][k] = W0[k][n0 + n], k < mr
  {
    const int n = (tid & 15) * 4, gn = n0 + n;
    for (int k0 = tid >> 4; k0 < kR; k0 += 64) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * 16;
        const bool in = k < mr && gn < nc;
        v[u] = *reinterpret_cast<const f32x4*>(W0 + (in ? (int64_t)k * c.ldw + gn : 0));
        if (!in) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * 16;
        if (k >= kR) continue;
#pragma unroll
        for (int t = 0; t < 4; ++t) sts(Xs, n + t, k, (__bf16)(gn + t < nc ? v[u][t] : 0.f));
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = w0.v[a][b];
  if (wr < bpR) mma_strip(Aq, Xs, wr, kR, lane, acc);  // acc = W0 + dR W0
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = acc_row(wr, a, q, lane), j = n0 + acc_col(b, lane);
        if (i < mr && j < nc) c.RW0b[(int64_t)(i_base + i) * c.ldw + j_base + j] = (__bf16)acc[a][b][q];
      }
}

}  // namespace

bool bs_apply_eligible(int bpR, int bpP, const float* W0, int64_t ldw, const float* primR, const float* primP) {
  auto al = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  return bpR > 0 && bpP > 0 && bpR <= MAXB && bpP <= MAXB && bpR % 8 == 0 && bpP % 8 == 0 && ldw % 4 == 0 &&
         al(W0) && al(primR) && al(primP);
}

hipError_t launch_bs_apply(const ApplyArgs& c, hipStream_t st) {
  const int nsP = (c.bpP + SW - 1) / SW;
  const int64_t nb = (int64_t)c.nR * c.nP * nsP;
  if (nb == 0) return hipSuccess;
  if (nb > (int64_t)1 << 30) return hipErrorInvalidValue;
  const double mn = (double)c.m * c.n;
  const bool T = c.Tb || c.W;
  const double flops = 2.0 * mn * ((T ? c.bpP : 0) + (c.W ? c.bpR : 0) + (c.RW0b ? c.bpR : 0));
  const double bytes = mn * (4.0 + (c.Tb ? 2 : 0) + (c.W ? dtype_size(c.w_dt) : 0) + (c.RW0b ? 2 : 0));
  ProfScope prof(POET_K_APPLY, st, flops, bytes);
  const int64_t grid = (nb + 7) / 8 * 8;
  hipLaunchKernelGGL(bs_apply_kernel, dim3((unsigned)grid), dim3(NT), 0, st, c);
  return hipGetLastError();
}

}  // namespace poet
