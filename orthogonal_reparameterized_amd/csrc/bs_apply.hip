// Fused application of two block-diagonal orthogonal factors (POET-BS on both sides) to the fixed weight:
//   T = W0 P,   W = R T = R W0 P,   RW0 = R W0,
// for blocks of up to 256 (POET reparameterization W = R W0 P with block-diagonal R and P; the bf16 activation
// path). Each factor is applied as identity + delta: the delta (primitive minus I) and the other operand are
// rounded to bf16 for v_mfma_f32_32x32x16_bf16, the identity part is added in float32:
//   T   = W0 + bf16(W0) bf16(dP)        (float32; written as bf16 when asked)
//   W   = T + bf16(dR) bf16(T)          (written in the activation dtype)
//   RW0 = W0 + bf16(dR) bf16(W0)        (written as bf16)
// One workgroup (8 waves, 64 rows x 32 columns each) owns 64 columns of one P block within one R block: all rows
// of the R block (up to 256) by the strip. Phase 1 stages the W0 tile of the (R block, P block) pair and the dP strip, phase 2 restages dR and
// keeps T of the strip transposed in LDS as the second product's operand, phase 3 swaps in the W0 strip for R W0.
// Every operand is read from its float32 source and converted while staged, so no bf16 copies are made.
#include "poet.h"
#include "strip_mma.h"

namespace poet {
namespace {

using namespace strip;

constexpr int NTA = 512;  // 8 waves: two per SIMD, so that one wave's MFMAs run while the other waits on memory

// float32 values at this lane's accumulator positions: rows wr + (0..63), columns n0 + wc + (0..31)
struct Frag {
  f32x16 v[2][1];
};

// Stage rows [0, rowsA) x chunks [0, kpad/4) of a float32 block (row pitch ld, rows < rlim and columns < clim
// valid, the rest zero) as bf16 into LDS rows, subtracting the identity when sub_eye. Each thread owns one
// float4 chunk column and walks rows 8 apart, issuing 8 loads before their LDS stores.
__device__ __forceinline__ void stage_block(char* Aq, const float* src, int64_t ld, int rowsA, int kpad, int rlim,
                                            int clim, bool sub_eye, int tid) {
  const int q4 = tid & 63;
  for (int i0 = tid >> 6; i0 < rowsA; i0 += 64) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 8;
      const bool in = i < rlim && 4 * q4 < clim;  // row padding up to a multiple of 4 columns is readable
      v[u] = *reinterpret_cast<const f32x4*>(src + (in ? (int64_t)i * ld + 4 * q4 : 0));
      if (!in) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 8;
      if (i >= rowsA || 4 * q4 >= kpad) continue;
      bf16x4 b;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = 4 * q4 + t;
        b[t] = (__bf16)(k < clim ? v[u][t] - (sub_eye && i == k ? 1.f : 0.f) : 0.f);
      }
      *reinterpret_cast<bf16x4*>(Aq + loff(i, 4 * q4)) = b;
    }
  }
}

// Stage a 64-column strip transposed: Xs[n][k] = src[k][n0 + n] (row pitch ld) for k < kpad, as bf16, zero at
// k >= rlim or n0 + n >= clim, minus the identity (k == n0 + n) when sub_eye.
__device__ __forceinline__ void stage_strip(char* Xs, const float* src, int64_t ld, int n0, int kpad, int rlim,
                                            int clim, bool sub_eye, int tid) {
  const int n = (tid & 15) * 4, gn = n0 + n;
  for (int k0 = tid >> 4; k0 < kpad; k0 += 128) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * 32;
      const bool in = k < rlim && gn < clim;
      v[u] = *reinterpret_cast<const f32x4*>(src + (in ? (int64_t)k * ld + gn : 0));
      if (!in) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * 32;
      if (k >= kpad) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float d = gn + t < clim ? v[u][t] - (sub_eye && k == gn + t ? 1.f : 0.f) : 0.f;
        sts(Xs, n + t, k, (__bf16)d);
      }
    }
  }
}

__global__ __launch_bounds__(NTA) void bs_apply_kernel(const ApplyArgs c) {
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = (wave & 3) * 64, wc = (wave >> 2) * 32;  // this wave: rows wr.., strip columns wc..wc+31
  const int bpR = c.bpR, bpP = c.bpP;
  const int i_base = r * bpR, mr = min(bpR, c.m - i_base);
  const int j_base = cblk * bpP, nc = min(bpP, c.n - j_base);
  const int n0 = s * SW;                          // strip origin within the P block
  const int rowsA = min(MAXB, (bpR + 63) / 64 * 64);
  const int kR = kpad_of(bpR), kP = kpad_of(bpP);
  const float* W0 = c.W0 + (int64_t)i_base * c.ldw + j_base;
  const bool needT = c.Tb != nullptr || c.W != nullptr;
  auto rowof = [&](int a, int q) { return acc_row(wr, a, q, lane); };
  const int jcol = n0 + wc + (lane & 31);  // this lane's column within the P block

  // float32 W0 at this lane's output positions (the identity parts of T and of R W0)
  Frag w0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = rowof(a, q);
      const bool in = i < mr && jcol < nc;
      w0.v[a][0][q] = W0[in ? (int64_t)i * c.ldw + jcol : 0];
      if (!in) w0.v[a][0][q] = 0.f;
    }

  f32x16 acc[2][1];
  if (needT) {
    // ---- phase 1: Aq = bf16 W0 tile (rows < mr, columns < nc); Xs = bf16 dP strip, transposed
    stage_block(Aq, W0, c.ldw, rowsA, kP, mr, nc, false, tid);
    stage_strip(Xs, c.primP + (int64_t)cblk * bpP * bpP, bpP, n0, kP, nc, nc, true, tid);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 2; ++a) acc[a][0] = w0.v[a][0];
    if (wr < bpR) mma_strip_n<1>(Aq, Xs, wr, wc, kP, lane, acc);  // T = W0 + W0 dP (float32)
    if (c.Tb) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int i = rowof(a, q);
          if (i < mr && jcol < nc) c.Tb[(int64_t)(i_base + i) * c.ldw + j_base + jcol] = (__bf16)acc[a][0][q];
        }
    }
    __syncthreads();  // phase 1 operands are dead
  }
  if (c.W == nullptr && c.RW0b == nullptr) return;

  // ---- phase 2: Aq = bf16 dR block; Xs = bf16 T strip (transposed, from the accumulators)
  stage_block(Aq, c.primR + (int64_t)r * bpR * bpR, bpR, rowsA, kR, mr, mr, true, tid);
  if (c.W) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v4;
#pragma unroll
        for (int t = 0; t < 4; ++t) v4[t] = (__bf16)acc[a][0][q * 4 + t];  // rows >= mr hold zeros
        *reinterpret_cast<bf16x4*>(Xs + loff(wc + (lane & 31), rowof(a, q * 4))) = v4;
      }
    __syncthreads();
    if (wr < bpR) mma_strip_n<1>(Aq, Xs, wr, wc, kR, lane, acc);  // acc = T + dR T
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = rowof(a, q);
        if (i >= mr || jcol >= nc) continue;
        const int64_t o = (int64_t)(i_base + i) * c.ldw + j_base + jcol;
        if (c.w_dt == BF16) reinterpret_cast<__bf16*>(c.W)[o] = (__bf16)acc[a][0][q];
        else reinterpret_cast<float*>(c.W)[o] = acc[a][0][q];
      }
    if (c.RW0b == nullptr) return;
    __syncthreads();  // the T strip is dead
  }

  // ---- phase 3: Xs = bf16 W0 strip (transposed): Xs[n][k] = W0[k][n0 + n], k < mr
  stage_strip(Xs, W0, c.ldw, n0, kR, mr, nc, false, tid);
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 2; ++a) acc[a][0] = w0.v[a][0];
  if (wr < bpR) mma_strip_n<1>(Aq, Xs, wr, wc, kR, lane, acc);  // acc = W0 + dR W0
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = rowof(a, q);
      if (i < mr && jcol < nc) c.RW0b[(int64_t)(i_base + i) * c.ldw + j_base + jcol] = (__bf16)acc[a][0][q];
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
  hipLaunchKernelGGL(bs_apply_kernel, dim3((unsigned)grid), dim3(NTA), 0, st, c);
  return hipGetLastError();
}

}  // namespace poet
