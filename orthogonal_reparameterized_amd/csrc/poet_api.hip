// C ABI of the POET layer: host-side validation, workspace planning and the launch sequence of each call.
// Nothing here computes on the host; every step of the method runs in the kernels of this library.
#include <cmath>
#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/poet.h"
#include "internal.h"

using namespace poet;

namespace {

thread_local std::string g_err;
thread_local poet_status g_last = POET_OK;

poet_status fail(poet_status st, const char* fmt, ...) {
  g_last = st;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

// hipError_t helpers: return the first failing call's error
#define HIP_RET(expr)                 \
  do {                                \
    const hipError_t r_ = (expr);     \
    if (r_ != hipSuccess) return r_;  \
  } while (0)

#define HIP_TRY(expr)                                                                        \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess) return fail(POET_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

struct SideInfo {
  int mode = 0, d = 0, bp = 0, nprim = 0, k = 0, dtype = 0;
  int ldp = 0;      // row pitch of the saved powers and the adjoint's work blocks (bf16: bp rounded up to 8)
  size_t plen = 0;  // elements of one saved power over all primitives: nprim * bp * ldp
  size_t theta_len = 0, prim_len = 0, powers_len = 0;
};

bool side_info(const poet_side* s, SideInfo* o, const char* name) {
  if (!s) return fail(POET_E_ARG, "%s: null side", name), false;
  if (s->mode != POET_BS && s->mode != POET_FS) return fail(POET_E_ARG, "%s: bad mode %d", name, s->mode), false;
  if (s->dtype != POET_F32 && s->dtype != POET_BF16) return fail(POET_E_DTYPE, "%s: bad dtype %d", name, s->dtype), false;
  if (s->d < 1) return fail(POET_E_SHAPE, "%s: d = %d must be >= 1", name, s->d), false;
  if (s->b < 1 || s->b > s->d) return fail(POET_E_SHAPE, "%s: b = %d must be in [1, d = %d]", name, s->b, s->d), false;
  if (s->b > POET_MAX_PRIM) return fail(POET_E_UNSUPPORTED, "%s: primitive size %d > %d", name, s->b, POET_MAX_PRIM), false;
  if (s->k < 0 || s->k > POET_MAX_K) return fail(POET_E_SHAPE, "%s: k = %d must be in [0, %d]", name, s->k, POET_MAX_K), false;
  o->mode = s->mode; o->d = s->d; o->bp = s->b; o->k = s->k; o->dtype = s->dtype;
  o->nprim = s->mode == POET_FS ? 1 : (s->d + s->b - 1) / s->b;
  size_t th = 0;
  for (int p = 0; p < o->nprim; ++p) {
    const size_t c = s->mode == POET_FS ? (size_t)s->b : (size_t)std::min(s->b, s->d - p * s->b);
    th += c * (c - 1) / 2;
  }
  o->theta_len = th;
  o->prim_len = (size_t)o->nprim * o->bp * o->bp;
  o->ldp = o->dtype == POET_BF16 ? (o->bp + 7) / 8 * 8 : o->bp;
  o->plen = (size_t)o->nprim * o->bp * o->ldp;
  o->powers_len = (size_t)o->k * o->plen;
  return true;
}

bool layer_info(const poet_layer* L, SideInfo* R, SideInfo* P) {
  if (!L) return fail(POET_E_ARG, "null layer"), false;
  if (L->m < 1 || L->n < 1) return fail(POET_E_SHAPE, "m = %d and n = %d must be >= 1", L->m, L->n), false;
  if (L->T < 0) return fail(POET_E_SHAPE, "T = %d must be >= 0", L->T), false;
  if (L->ldw < L->n || L->ldx < L->n || L->ldy < L->m)
    return fail(POET_E_SHAPE, "leading dims ldw=%d ldx=%d ldy=%d too small for m=%d n=%d", L->ldw, L->ldx, L->ldy, L->m,
                L->n), false;
  if (L->act_dtype != POET_F32 && L->act_dtype != POET_BF16)
    return fail(POET_E_DTYPE, "bad act_dtype %d", L->act_dtype), false;
  if (L->m > 65535 * 64 || L->n > 65535 * 64 || L->T > 65535 * 64)
    return fail(POET_E_UNSUPPORTED, "dimension beyond the kernels' grid limits"), false;
  if (!side_info(&L->R, R, "R") || !side_info(&L->P, P, "P")) return false;
  if (R->d != L->m) return fail(POET_E_SHAPE, "R.d = %d must equal m = %d", R->d, L->m), false;
  if (P->d != L->n) return fail(POET_E_SHAPE, "P.d = %d must equal n = %d", P->d, L->n), false;
  return true;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bump allocator over the caller's workspace; with base == nullptr it only measures.
struct Arena {
  char* base;
  size_t off = 0;
  explicit Arena(void* b) : base(reinterpret_cast<char*>(b)) {
    if (base) {  // align the first block
      const uintptr_t u = reinterpret_cast<uintptr_t>(base);
      off = align_up(u, 256) - u;
    }
  }
  template <class T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  void* take_bytes(size_t bytes) { return take<char>(bytes); }
  size_t used() const { return off + 256; }  // slack for the initial alignment
};

// ------------------------------------------------------------------------------------------------------------
// Applying a factor. apply_P: T = W0 P (float32 out). apply_R: out = R src (src float32, out dtype out_dt).
// BS: one batched GEMM over the blocks, identity + delta (the delta is the primitive minus I, the identity part
// is the float32 addend). FS: gather the sampled columns/rows, GEMM with the primitive's delta, scatter back.
// ------------------------------------------------------------------------------------------------------------
struct FsBufs {
  float *Ac = nullptr, *C1 = nullptr;  // m x sP
  float *Br = nullptr, *C2 = nullptr;  // sR x n
  // bf16 operands of the fast kernel (rows padded to multiples of 8) and the scratch of its addend epilogue
  __bf16 *Acb = nullptr, *dPb = nullptr;  // m x ldpP, sP x ldpP
  __bf16 *Brb = nullptr, *dRb = nullptr;  // sR x ldn, sR x ldpR
  float* part = nullptr;
  size_t part_elems = 0;
};

inline int pad8(int x) { return (x + 7) / 8 * 8; }

// bf16 FS factor application on the fast kernel: bf16 activations and a bf16 side
bool fs_bf16(const poet_layer& L, const SideInfo& S) { return S.mode == POET_FS && L.act_dtype == BF16 && S.dtype == BF16; }

void plan_fs(Arena& a, const poet_layer& L, const SideInfo& R, const SideInfo& P, FsBufs* f) {
  if (P.mode == POET_FS) { f->Ac = a.take<float>((size_t)L.m * P.bp); f->C1 = a.take<float>((size_t)L.m * P.bp); }
  if (R.mode == POET_FS) { f->Br = a.take<float>((size_t)R.bp * L.n); f->C2 = a.take<float>((size_t)R.bp * L.n); }
  if (fs_bf16(L, P)) { f->Acb = a.take<__bf16>((size_t)L.m * P.ldp); f->dPb = a.take<__bf16>((size_t)P.bp * P.ldp); }
  if (fs_bf16(L, R)) { f->Brb = a.take<__bf16>((size_t)R.bp * pad8(L.n)); f->dRb = a.take<__bf16>((size_t)R.bp * R.ldp); }
  if (fs_bf16(L, P) || fs_bf16(L, R)) {
    f->part_elems = std::max(fs_bf16(L, P) ? (size_t)L.m * P.bp : 0, fs_bf16(L, R) ? (size_t)R.bp * L.n : 0);
    f->part = a.take<float>(f->part_elems);
  }
}

hipError_t apply_P(const poet_layer& L, const SideInfo& P, const float* W0, const float* prim, const int32_t* idx,
                   float* T, int compute, const FsBufs& f, hipStream_t st) {
  const int m = L.m, n = L.n;
  GemmDesc g;
  g.compute = compute;
  g.kclass = POET_K_APPLY;
  if (P.mode == POET_BS) {
    g.M = m; g.N = P.bp; g.K = P.bp; g.Ntot = n; g.Ktot = n; g.batch = P.nprim;
    g.A = W0; g.lda = L.ldw; g.sA = P.bp; g.a_dt = F32; g.a_kmajor = 1;
    g.B = prim; g.ldb = P.bp; g.sB = (int64_t)P.bp * P.bp; g.b_dt = F32; g.b_kmajor = 0; g.b_sub_eye = 1;
    g.D = W0; g.ldd = L.ldw; g.sD = P.bp; g.beta = 1.f;
    g.C = T; g.ldc = L.ldw; g.sC = P.bp; g.c_dt = F32;
    return launch_gemm(g, st);
  }
  const int s = P.bp;
  const bool fast = f.Acb && compute == BF16;  // W0[:, I] in float32 (addend) and, for the fast kernel, in bf16
  hipError_t e = launch_gather_cols_to(W0, L.ldw, m, idx, s, n, f.Ac, F32, s, st, fast ? f.Acb : nullptr, P.ldp);
  if (e != hipSuccess) return e;
  g.M = m; g.N = s; g.K = s;
  g.D = f.Ac; g.ldd = s; g.beta = 1.f;
  g.C = f.C1; g.ldc = s; g.c_dt = F32;
  if (fast) {  // C1 = W0[:, I] + bf16(W0[:, I]) bf16(G_P - I) on the fast kernel
    if ((e = launch_delta_bf16(prim, 1, s, P.ldp, f.dPb, st)) != hipSuccess) return e;
    g.A = f.Acb; g.lda = P.ldp; g.a_dt = BF16; g.a_kmajor = 1;
    g.B = f.dPb; g.ldb = P.ldp; g.b_dt = BF16; g.b_kmajor = 0;
    g.part = f.part; g.part_elems = f.part_elems;
  } else {
    g.A = f.Ac; g.lda = s; g.a_dt = F32; g.a_kmajor = 1;
    g.B = prim; g.ldb = s; g.b_dt = F32; g.b_kmajor = 0; g.b_sub_eye = 1;
  }
  if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  if ((e = launch_convert(W0, L.ldw, T, L.ldw, F32, m, n, st)) != hipSuccess) return e;
  return launch_scatter_cols(f.C1, s, m, idx, s, n, T, L.ldw, st);
}

hipError_t apply_R(const poet_layer& L, const SideInfo& R, const float* src, const float* prim, const int32_t* idx,
                   void* out, int out_dt, int64_t ldo, int compute, const FsBufs& f, hipStream_t st) {
  const int m = L.m, n = L.n;
  GemmDesc g;
  g.compute = compute;
  g.kclass = POET_K_APPLY;
  if (R.mode == POET_BS) {
    g.M = R.bp; g.N = n; g.K = R.bp; g.Mtot = m; g.Ktot = m; g.batch = R.nprim;
    g.A = prim; g.lda = R.bp; g.sA = (int64_t)R.bp * R.bp; g.a_dt = F32; g.a_kmajor = 1; g.a_sub_eye = 1;
    g.B = src; g.ldb = L.ldw; g.sB = (int64_t)R.bp * L.ldw; g.b_dt = F32; g.b_kmajor = 0;
    g.D = src; g.ldd = L.ldw; g.sD = (int64_t)R.bp * L.ldw; g.beta = 1.f;
    g.C = out; g.ldc = ldo; g.sC = (int64_t)R.bp * ldo; g.c_dt = out_dt;
    return launch_gemm(g, st);
  }
  const int s = R.bp;
  const bool fast = f.Brb && compute == BF16;  // src[I, :] in float32 (addend) and, for the fast kernel, in bf16
  hipError_t e = launch_gather_rows_to(src, F32, L.ldw, idx, s, m, n, f.Br, F32, n, st, fast ? f.Brb : nullptr, pad8(n));
  if (e != hipSuccess) return e;
  g.M = s; g.N = n; g.K = s;
  g.D = f.Br; g.ldd = n; g.beta = 1.f;
  g.C = f.C2; g.ldc = n; g.c_dt = F32;
  if (fast) {  // C2 = src[I, :] + bf16(G_R - I) bf16(src[I, :]) on the fast kernel
    if ((e = launch_delta_bf16(prim, 1, s, R.ldp, f.dRb, st)) != hipSuccess) return e;
    g.A = f.dRb; g.lda = R.ldp; g.a_dt = BF16; g.a_kmajor = 1;
    g.B = f.Brb; g.ldb = pad8(n); g.b_dt = BF16; g.b_kmajor = 0;
    g.part = f.part; g.part_elems = f.part_elems;
  } else {
    g.A = prim; g.lda = s; g.a_dt = F32; g.a_kmajor = 1; g.a_sub_eye = 1;
    g.B = f.Br; g.ldb = n; g.b_dt = F32; g.b_kmajor = 0;
  }
  if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  if ((e = launch_convert(src, L.ldw, out, ldo, out_dt, m, n, st)) != hipSuccess) return e;
  return launch_scatter_rows(f.C2, n, idx, s, m, n, out, out_dt, ldo, st);
}

// Both sides POET-FS with bf16 operands and activations: W = R W0 P straight into bf16, with no float32 copy of
// W0 P. Off the sampled rows I_R, W is W0 P, which differs from W0 only in the columns I_P (C1 = (W0 P)[:, I_P],
// float32 block plus one bf16 product as in apply_P); the rows I_R are apply_R's product on the rows I_R of W0 P,
// whose float32 (Br) and bf16 (Brb) copies are the rows of W0 patched with C1[I_R, :]. The same products and
// roundings as apply_P followed by apply_R.
hipError_t fs_weight_bf16(const poet_layer& L, const SideInfo& R, const SideInfo& P, const float* W0,
                          const float* primR, const float* primP, const int32_t* idxR, const int32_t* idxP, void* W,
                          const FsBufs& f, hipStream_t st) {
  const int m = L.m, n = L.n, sR = R.bp, sP = P.bp, ldn = pad8(n);
  hipError_t e;
  if ((e = launch_gather_cols_to(W0, L.ldw, m, idxP, sP, n, f.Ac, F32, sP, st, f.Acb, P.ldp)) != hipSuccess) return e;
  if ((e = launch_delta_bf16(primP, 1, sP, P.ldp, f.dPb, st)) != hipSuccess) return e;
  GemmDesc g;
  g.compute = BF16;
  g.kclass = POET_K_APPLY;
  g.part = f.part; g.part_elems = f.part_elems;
  g.beta = 1.f; g.c_dt = F32;
  g.M = m; g.N = sP; g.K = sP;  // C1 = W0[:, I_P] + bf16(W0[:, I_P]) bf16(G_P - I)
  g.A = f.Acb; g.lda = P.ldp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = f.dPb; g.ldb = P.ldp; g.b_dt = BF16; g.b_kmajor = 0;
  g.D = f.Ac; g.ldd = sP; g.C = f.C1; g.ldc = sP;
  if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  if ((e = launch_convert(W0, L.ldw, W, L.ldw, BF16, m, n, st)) != hipSuccess) return e;
  if ((e = launch_scatter_cols_to(f.C1, sP, m, idxP, sP, n, W, BF16, L.ldw, st)) != hipSuccess) return e;
  if ((e = launch_gather_rows_to(W0, F32, L.ldw, idxR, sR, m, n, f.Br, F32, n, st, f.Brb, ldn)) != hipSuccess) return e;
  if ((e = launch_patch_block(f.C1, sP, idxR, m, idxP, n, sR, sP, f.Br, n, f.Brb, ldn, st)) != hipSuccess) return e;
  if ((e = launch_delta_bf16(primR, 1, sR, R.ldp, f.dRb, st)) != hipSuccess) return e;
  g.M = sR; g.N = n; g.K = sR;  // C2 = Br + bf16(G_R - I) Brb
  g.A = f.dRb; g.lda = R.ldp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = f.Brb; g.ldb = ldn; g.b_dt = BF16; g.b_kmajor = 0;
  g.D = f.Br; g.ldd = n; g.C = f.C2; g.ldc = n;
  if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  return launch_scatter_rows(f.C2, n, idxR, sR, m, n, W, BF16, L.ldw, st);
}

// Both sides POET-FS with bf16 operands: the gradient's two operands, Z[I_R, :] (Z = W0 P) and (R W0)[:, I_P],
// formed from W0 directly instead of from the whole of W0 P and R W0. Off the sampled rows (columns) both are W0; on
// the sampled block W0[I_R, I_P] they are W0[I_R, I_P] G_P and G_R W0[I_R, I_P], each as the float32 block plus one
// bf16 product of its delta (the same form as apply_P / apply_R):
//   Zr  (sR x ldn,  bf16) = W0[I_R, :] with columns I_P replaced by W0[I_R, I_P] + bf16(W0[I_R, I_P]) bf16(G_P - I)
//   Acp (m x ldpP, bf16)  = W0[:, I_P] with rows I_R replaced by W0[I_R, I_P] + bf16(G_R - I) bf16(W0[I_R, I_P])
hipError_t fs_grad_operands(const poet_layer& L, const SideInfo& R, const SideInfo& P, const float* W0,
                            const float* primR, const float* primP, const int32_t* idxR, const int32_t* idxP,
                            __bf16* Zr, __bf16* Acp, const FsBufs& f, hipStream_t st) {
  const int m = L.m, n = L.n, sR = R.bp, sP = P.bp, ldn = pad8(n);
  hipError_t e;
  // W0[I_R, :] in float32 (Br) and bf16 (Zr); the block W0[I_R, I_P] in float32 (Ac, pitch sP) and bf16 (Acb)
  if ((e = launch_gather_rows_to(W0, F32, L.ldw, idxR, sR, m, n, f.Br, F32, n, st, Zr, ldn)) != hipSuccess) return e;
  if ((e = launch_gather_cols_to(f.Br, n, sR, idxP, sP, n, f.Ac, F32, sP, st, f.Acb, P.ldp)) != hipSuccess) return e;
  if ((e = launch_gather_cols_to(W0, L.ldw, m, idxP, sP, n, Acp, BF16, P.ldp, st)) != hipSuccess) return e;
  if ((e = launch_delta_bf16(primP, 1, sP, P.ldp, f.dPb, st)) != hipSuccess) return e;
  if ((e = launch_delta_bf16(primR, 1, sR, R.ldp, f.dRb, st)) != hipSuccess) return e;
  GemmDesc g;
  g.compute = BF16;
  g.kclass = POET_K_APPLY;
  g.part = f.part; g.part_elems = f.part_elems;
  g.D = f.Ac; g.ldd = sP; g.beta = 1.f;
  g.c_dt = F32; g.ldc = sP;
  // C1 = W0[I_R, I_P] G_P
  g.M = sR; g.N = sP; g.K = sP;
  g.A = f.Acb; g.lda = P.ldp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = f.dPb; g.ldb = P.ldp; g.b_dt = BF16; g.b_kmajor = 0;
  g.C = f.C1;
  if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  if ((e = launch_scatter_cols_to(f.C1, sP, sR, idxP, sP, n, Zr, BF16, ldn, st)) != hipSuccess) return e;
  // C2 = G_R W0[I_R, I_P]
  g.M = sR; g.N = sP; g.K = sR;
  g.A = f.dRb; g.lda = R.ldp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = f.Acb; g.ldb = P.ldp; g.b_dt = BF16; g.b_kmajor = 0;
  g.C = f.C2;
  if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  return launch_scatter_rows(f.C2, sP, idxR, sR, m, sP, Acp, BF16, P.ldp, st);
}

// ------------------------------------------------------------------------------------------------------------
// bf16 application of block-diagonal factors (both sides POET-BS, bf16 activations). The factor deltas and a
// bf16 copy of W0 are MFMA operands; the identity parts are added in float32 through the epilogue addend.
//   apply_P_b: T = W0 + W0 dP  -> Tb (bf16) and, when Tf != null, Tf (float32)
//   apply_R_b: out = src + dR src, with src given as a bf16 operand (srcb) and in float32 (srcf)
// ------------------------------------------------------------------------------------------------------------
struct Part {  // float32 scratch through which the bf16 kernel applies addend epilogues and split-K
  float* p = nullptr;
  size_t n = 0;
};

// part elements the bf16 factor applications need: one float32 product per output element (block-padded)
size_t apply_part_elems(const poet_layer& L, const SideInfo& R, const SideInfo& P) {
  return std::max((size_t)P.nprim * P.bp * L.m, (size_t)R.nprim * R.bp * L.n);
}

hipError_t apply_P_b(const poet_layer& L, const SideInfo& P, const float* W0, const __bf16* W0b, const __bf16* dPb,
                     __bf16* Tb, float* Tf, const Part& part, hipStream_t st) {
  GemmDesc g;
  g.part = part.p; g.part_elems = part.n;
  g.kclass = POET_K_APPLY;
  g.compute = BF16;
  g.M = L.m; g.N = P.bp; g.K = P.bp; g.Ntot = L.n; g.Ktot = L.n; g.batch = P.nprim;
  g.A = W0b; g.lda = L.ldw; g.sA = P.bp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = dPb; g.ldb = P.bp; g.sB = (int64_t)P.bp * P.bp; g.b_dt = BF16; g.b_kmajor = 0;
  g.D = W0; g.ldd = L.ldw; g.sD = P.bp; g.beta = 1.f;
  g.C = Tb; g.ldc = L.ldw; g.sC = P.bp; g.c_dt = BF16;
  if (Tf) { g.C2 = Tf; g.ldc2 = L.ldw; g.sC2 = P.bp; g.c2_dt = F32; }
  return launch_gemm(g, st);
}

hipError_t apply_R_b(const poet_layer& L, const SideInfo& R, const __bf16* srcb, const float* srcf, const __bf16* dRb,
                     void* out, int out_dt, const Part& part, hipStream_t st) {
  GemmDesc g;
  g.part = part.p; g.part_elems = part.n;
  g.kclass = POET_K_APPLY;
  g.compute = BF16;
  g.M = R.bp; g.N = L.n; g.K = R.bp; g.Mtot = L.m; g.Ktot = L.m; g.batch = R.nprim;
  g.A = dRb; g.lda = R.bp; g.sA = (int64_t)R.bp * R.bp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = srcb; g.ldb = L.ldw; g.sB = (int64_t)R.bp * L.ldw; g.b_dt = BF16; g.b_kmajor = 0;
  g.D = srcf; g.ldd = L.ldw; g.sD = (int64_t)R.bp * L.ldw; g.beta = 1.f;
  g.C = out; g.ldc = L.ldw; g.sC = (int64_t)R.bp * L.ldw; g.c_dt = out_dt;
  return launch_gemm(g, st);
}

// ------------------------------------------------------------------------------------------------------------
// Backward through the truncated Cayley-Neumann series of one side, then the skew projection.
// R_k = I + sum_{i=1}^{k+1} a_i Q^i with a_i = 2 (i <= k), a_{k+1} = 1. The gradient of <dR, R_k> is
//   dQ = sum_i a_i sum_{j<i} (Q^T)^j dR (Q^T)^{i-1-j} = sum_{j=0}^{k} H_j C_j,
//   H_j = Q^j dR,   C_j = sum_{t=0}^{k-j} a_{t+j+1} (-1)^{t+j} Q^t     (using Q^T = -Q).
// Phase 1 builds H_1..H_k by k products with Q (H_0 = dR); phase 2 is one product with K = (k+1) b against the
// stacked C_j (polynomials in Q formed elementwise from the saved powers). The identity term a_1 dR of H_0 C_0
// is added in float32 through the epilogue addend, so only the higher-order corrections carry operand rounding.
// ------------------------------------------------------------------------------------------------------------
struct AdjBufs {
  float* dQ = nullptr;
  void* H = nullptr;   // nprim x bp x (k+1) ldp, side dtype
  void* Cs = nullptr;  // nprim x (k+1) ldp x ldp, side dtype
  float* part = nullptr;
  size_t part_elems = 0;
};

size_t adj_h_elems(const SideInfo& S) { return (size_t)S.nprim * S.bp * S.ldp * (S.k + 1); }
size_t adj_c_elems(const SideInfo& S) { return (size_t)S.nprim * S.ldp * S.ldp * (S.k + 1); }

hipError_t launch_grouped(const std::vector<GemmDesc>& all, hipStream_t st);

// H_j = Q^j H_0 (j = 1..k) of the nprim blocks of one side, from its saved powers Q^1 = Q .. Q^k (power t - 1 at
// element (t - 1) plen, block stride bp ldp): k products that do not depend on one another, so they share grouped
// launches instead of running as a chain of k launches. H rows have pitch ldh = (k+1) ldp, H_j at column j ldp.
void h_products(const SideInfo& S, const void* powers, char* H, std::vector<GemmDesc>* out) {
  const int bp = S.bp, k = S.k, ldp = S.ldp, ldh = (k + 1) * ldp;
  const size_t esz = dtype_size(S.dtype);
  for (int j = 1; j <= k; ++j) {
    GemmDesc g;
    g.kclass = POET_K_ADJOINT;
    g.compute = S.dtype; g.M = g.N = g.K = bp; g.batch = S.nprim;
    g.A = reinterpret_cast<const char*>(powers) + (size_t)(j - 1) * S.plen * esz; g.lda = ldp;
    g.sA = (int64_t)bp * ldp; g.a_dt = S.dtype; g.a_kmajor = 1;
    g.B = H; g.ldb = ldh; g.sB = (int64_t)bp * ldh; g.b_dt = S.dtype; g.b_kmajor = 0;
    g.C = H + (size_t)j * ldp * esz; g.ldc = ldh; g.sC = (int64_t)bp * ldh; g.c_dt = S.dtype;
    out->push_back(g);  // no split-K scratch: the launch holds k times the tiles of one product
  }
}

// H_j sits at column j ldp of the H rows (16-byte aligned operands for the bf16 kernel); with ldp > bp the gap
// columns are zeroed, and the matching rows of the coefficient stack are zero, so the phase-2 product can run
// over K = (k+1) ldp.
hipError_t neumann_adjoint(const SideInfo& S, const float* dRg, const void* powers, float* dtheta, const AdjBufs& b,
                           hipStream_t st) {
  if (S.theta_len == 0) return hipSuccess;
  const int64_t pp = (int64_t)S.bp * S.bp;
  if (S.k == 0) return launch_skew_project(dRg, nullptr, S.mode, S.d, S.bp, S.nprim, dtheta, st);
  const int bp = S.bp, k = S.k, ldp = S.ldp, ldh = (k + 1) * ldp;
  const int64_t hs = (int64_t)bp * ldh;
  char* H = reinterpret_cast<char*>(b.H);
  hipError_t e = hipSuccess;
  const bool chain = ldp == bp && power_chain_eligible(bp, S.dtype, powers);
  if (chain) {  // H_0 = dR and H_{j+1} = Q H_j in one launch
    ChainArgs c;
    c.bp = bp; c.nprim = S.nprim; c.steps = k;
    c.A = reinterpret_cast<const __bf16*>(powers); c.sA = pp;
    c.X0 = dRg; c.ldx0 = bp; c.sx0 = pp;
    c.Y = reinterpret_cast<__bf16*>(H); c.ldy = ldh; c.sy = hs; c.jstep = bp; c.write_x0 = 1;
    e = launch_power_chain(c, POET_K_ADJOINT, st);
  } else {
    if (ldp > bp && S.dtype == BF16) {  // zero the gap columns (the products below write only the first bp of each
      // block, and the workspace holds other data between calls)
      if ((e = launch_zero_gaps(reinterpret_cast<__bf16*>(H), (int64_t)S.nprim * bp, ldh, ldp, bp, k + 1, st)) !=
          hipSuccess)
        return e;
    }
    e = launch_convert(dRg, bp, H, ldh, S.dtype, S.nprim * bp, bp, st);  // H_0 = dR
    if (e == hipSuccess) {  // H_j = Q^j H_0 from the saved powers
      std::vector<GemmDesc> pr;
      h_products(S, powers, H, &pr);
      e = launch_grouped(pr, st);
    }
  }
  if (e != hipSuccess) return e;
  if ((e = launch_adjoint_coefs(powers, S.dtype, S.nprim, bp, ldp, k, b.Cs, st)) != hipSuccess) return e;
  GemmDesc g;  // dQ = a_1 dR + [H_0 .. H_k] [C_0; ..; C_k]
  g.kclass = POET_K_ADJOINT;
  g.compute = S.dtype; g.M = g.N = bp; g.K = (k + 1) * ldp; g.batch = S.nprim;
  g.A = H; g.lda = ldh; g.sA = hs; g.a_dt = S.dtype; g.a_kmajor = 1;
  g.B = b.Cs; g.ldb = ldp; g.sB = (int64_t)(k + 1) * ldp * ldp; g.b_dt = S.dtype; g.b_kmajor = 0;
  g.C = b.dQ; g.ldc = bp; g.sC = pp; g.c_dt = F32;
  g.part = b.part; g.part_elems = b.part_elems;
  g.defer_reduce = 1;
  if (fast_gemm_eligible(g)) {  // the split-K partials go straight into the skew projection with a_1 dR = 2 dR
    const int ns = fast_gemm_splits(g);
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
    return launch_reduce_skew(b.part, ns, S.nprim * pp, dRg, 2.f, S.mode, S.d, S.bp, S.nprim, dtheta, st);
  }
  g.defer_reduce = 0;
  g.D = dRg; g.ldd = bp; g.sD = pp; g.beta = 2.f;  // a_1 = 2 for k >= 1
  if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  return launch_skew_project(b.dQ, nullptr, S.mode, S.d, S.bp, S.nprim, dtheta, st);
}

ApplyArgs apply_args(const poet_layer& L, const SideInfo& R, const SideInfo& P, const float* W0, const float* primR,
                     const float* primP, __bf16* Tb, void* W, int w_dt, __bf16* RW0b) {
  ApplyArgs a;
  a.m = L.m; a.n = L.n; a.bpR = R.bp; a.nR = R.nprim; a.bpP = P.bp; a.nP = P.nprim;
  a.W0 = W0; a.ldw = L.ldw; a.primR = primR; a.primP = primP;
  a.Tb = Tb; a.W = W; a.w_dt = w_dt; a.RW0b = RW0b;
  return a;
}

// The primitive-gradient contraction g (output dR blocks, reduced over its K splits across the whole machine), then
// the adjoint. A ragged last block writes only its true extent, so dR is zero-filled first.
// a ragged last block of a BS side is written only over its extent: zero the rest of its bp x bp block first
hipError_t clear_ragged(const SideInfo& S, float* dR, hipStream_t st) {
  if (S.mode != POET_BS || S.d % S.bp == 0) return hipSuccess;
  const size_t pp = (size_t)S.bp * S.bp;
  return launch_fill(dR + (S.nprim - 1) * pp, pp, 0.f, st);
}
hipError_t contract_only(const SideInfo& S, const GemmDesc& g, float* dR, hipStream_t st) {
  hipError_t e;
  if ((e = clear_ragged(S, dR, st)) != hipSuccess) return e;
  return launch_gemm(g, st);
}
hipError_t contract_and_adjoint(const SideInfo& S, const GemmDesc& g, float* dR, const void* powers, float* dtheta,
                                const AdjBufs& b, hipStream_t st) {
  hipError_t e;
  if ((e = contract_only(S, g, dR, st)) != hipSuccess) return e;
  return neumann_adjoint(S, dR, powers, dtheta, b, st);
}

// ------------------------------------------------------------------------------------------------------------
// Workspace plans (the same code sizes and carves the workspace)
// ------------------------------------------------------------------------------------------------------------
// bf16 block-diagonal path: both sides POET-BS and bf16 activations
bool bs_bf16(const poet_layer& L, const SideInfo& R, const SideInfo& P) {
  return L.act_dtype == BF16 && R.mode == POET_BS && P.mode == POET_BS;
}

struct FwdPlan {
  void* W = nullptr;
  float* T = nullptr;                    // W0 P, float32
  __bf16 *W0b = nullptr, *Tb = nullptr;  // bf16 path: W0 and W0 P as bf16 operands
  __bf16 *dRb = nullptr, *dPb = nullptr; // bf16 path: factor deltas
  Part part;                             // bf16 path: epilogue scratch of the factor applications
  FsBufs fs;
};
size_t plan_fwd(const poet_layer& L, const SideInfo& R, const SideInfo& P, void* ws, bool need_W, FwdPlan* p) {
  Arena a(ws);
  const size_t mn = (size_t)L.m * L.ldw;
  if (need_W) p->W = a.take_bytes(mn * dtype_size(L.act_dtype));
  p->T = a.take<float>(mn);
  if (bs_bf16(L, R, P)) {
    p->W0b = a.take<__bf16>(mn);
    p->Tb = a.take<__bf16>(mn);
    p->dRb = a.take<__bf16>(R.prim_len);
    p->dPb = a.take<__bf16>(P.prim_len);
    p->part.n = apply_part_elems(L, R, P);
    p->part.p = a.take<float>(p->part.n);
  }
  plan_fs(a, L, R, P, &p->fs);
  return a.used();
}

struct BwdPlan {
  void* W = nullptr;
  float *T = nullptr, *RW0 = nullptr, *G = nullptr, *dRg = nullptr, *dPg = nullptr;
  __bf16 *W0b = nullptr, *Tb = nullptr, *RW0b = nullptr, *Gb = nullptr, *dRb = nullptr, *dPb = nullptr;
  AdjBufs adj;
  FsBufs fs;
  float *Gr = nullptr, *Zr = nullptr, *Acp = nullptr, *Gc = nullptr;
};
size_t plan_bwd(const poet_layer& L, const SideInfo& R, const SideInfo& P, void* ws, bool need_W, BwdPlan* p) {
  Arena a(ws);
  const size_t mn = (size_t)L.m * L.ldw;
  if (need_W) p->W = a.take_bytes(mn * dtype_size(L.act_dtype));
  const bool fast = bs_bf16(L, R, P);
  if (fast) {
    if (need_W) p->T = a.take<float>(mn);
    p->W0b = a.take<__bf16>(mn);
    p->Tb = a.take<__bf16>(mn);
    p->RW0b = a.take<__bf16>(mn);
    p->Gb = a.take<__bf16>(mn);
    p->dRb = a.take<__bf16>(R.prim_len);
    p->dPb = a.take<__bf16>(P.prim_len);
  } else {
    p->T = a.take<float>(mn);
    p->RW0 = a.take<float>(mn);
    p->G = a.take<float>(mn);
  }
  p->dRg = a.take<float>(R.prim_len);
  p->dPg = a.take<float>(P.prim_len);
  p->adj.dQ = a.take<float>(std::max(R.prim_len, P.prim_len));
  p->adj.H = a.take_bytes(std::max(adj_h_elems(R) * dtype_size(R.dtype), adj_h_elems(P) * dtype_size(P.dtype)));
  p->adj.Cs = a.take_bytes(std::max(adj_c_elems(R) * dtype_size(R.dtype), adj_c_elems(P) * dtype_size(P.dtype)));
  // split-K partial sums: the weight gradient with up to 4 splits, or the primitive products with up to 16
  p->adj.part_elems = std::max({4 * mn, 16 * std::max(R.prim_len, P.prim_len), apply_part_elems(L, R, P)});
  p->adj.part = a.take<float>(p->adj.part_elems);
  plan_fs(a, L, R, P, &p->fs);
  // FS gathers: float32, or bf16 with padded rows in the same room
  const size_t gr = std::max((size_t)R.bp * L.n, ((size_t)R.bp * pad8(L.n) + 1) / 2);
  const size_t gc = std::max((size_t)L.m * P.bp, ((size_t)L.m * P.ldp + 1) / 2);
  if (R.mode == POET_FS) { p->Gr = a.take<float>(gr); p->Zr = a.take<float>(gr); }
  if (P.mode == POET_FS) { p->Acp = a.take<float>(gc); p->Gc = a.take<float>(gc); }
  return a.used();
}

// ------------------------------------------------------------------------------------------------------------
// Activation-side application (both sides POET-BS, bf16 activations). The factors act on the activations around
// the W0 GEMM and W is never formed:
//   forward   X' = X P^T,  Z = X' W0^T,  Y = Z R^T
//   backward  dZ = dY R,  dX' = dZ W0,  dX = dX' P;  dL/dR = blocks of dY^T Z,  dL/dP = blocks of dX'^T X
// With at least as many tokens as W0 has rows (columns), P (R) is folded into the bf16 copy of W0 instead:
// Z = X (W0 P)^T and dX' = dY (R W0), so X' and dZ are never formed.
// (the same products as the weight-side path, associated the other way: G W0P^T = dY^T X P^T W0^T = dY^T Z).
// Every product is a bf16 GEMM with float32 accumulation; the factors enter as bf16 copies of the primitives.
// ------------------------------------------------------------------------------------------------------------
bool act_path_ok(const poet_layer& L, const SideInfo& R, const SideInfo& P) {
  return L.act_dtype == BF16 && R.mode == POET_BS && P.mode == POET_BS;
}

// A factor is folded into the weight (W0 P for the forward's token GEMM, R W0 for the backward's) instead of being
// applied to the tokens (X P^T, dY R) when there are at least as many tokens as the weight has rows (P) or columns
// (R): the fold touches m x n elements, the application T x n (or T x m).
// Blocks below 128 are not folded: the product would run on the generic kernel.
bool fold_P(const poet_layer& L, const SideInfo& P) { return L.T >= L.m && P.bp >= 128; }
bool fold_R(const poet_layer& L, const SideInfo& R) { return L.T >= L.n && R.bp >= 128; }

struct ActFwdPlan {
  __bf16 *Xp = nullptr, *W0P = nullptr, *Rb = nullptr, *Pb = nullptr;
};
size_t plan_fwd_act(const poet_layer& L, const SideInfo& R, const SideInfo& P, void* ws, ActFwdPlan* p) {
  Arena a(ws);
  if (fold_P(L, P)) p->W0P = a.take<__bf16>((size_t)L.m * L.ldw);
  else p->Xp = a.take<__bf16>((size_t)L.T * L.ldx);
  p->Rb = a.take<__bf16>(R.prim_len);
  p->Pb = a.take<__bf16>(P.prim_len);
  return a.used();
}

// Blocks below 128 (the bf16 kernel's smallest tile) are contracted g = floor(256 / bp) at a time: the product of a
// super-block of g adjacent blocks (size g bp, 129..256) runs on the fast kernel and its g diagonal sub-blocks are
// kept (the off-diagonal products are extra MFMA work in a pass bound by reading the two token-major operands).
int super_group(const SideInfo& S) { return S.bp < 128 ? 256 / S.bp : 1; }
size_t super_elems(const SideInfo& S) {
  const int g = super_group(S);
  if (g == 1) return 0;
  const size_t sb = (size_t)g * S.bp, nsb = (S.nprim + g - 1) / g;
  return nsb * sb * sb;
}

struct ActBwdPlan {
  __bf16 *dZ = nullptr, *RW0 = nullptr, *dXp = nullptr, *Rb = nullptr, *Pb = nullptr;
  float *dRg = nullptr, *dPg = nullptr;
  float* sup = nullptr;  // super-block products of small blocks
  size_t sup_elems = 0;
  AdjBufs adj;
};
size_t plan_bwd_act(const poet_layer& L, const SideInfo& R, const SideInfo& P, void* ws, ActBwdPlan* p) {
  Arena a(ws);
  if (fold_R(L, R)) p->RW0 = a.take<__bf16>((size_t)L.m * L.ldw);
  else p->dZ = a.take<__bf16>((size_t)L.T * L.ldy);
  p->dXp = a.take<__bf16>((size_t)L.T * L.ldx);
  p->Rb = a.take<__bf16>(R.prim_len);
  p->Pb = a.take<__bf16>(P.prim_len);
  p->dRg = a.take<float>(R.prim_len);
  p->dPg = a.take<float>(P.prim_len);
  p->sup_elems = std::max(super_elems(R), super_elems(P));
  p->sup = p->sup_elems ? a.take<float>(p->sup_elems) : nullptr;
  p->adj.dQ = a.take<float>(std::max(R.prim_len, P.prim_len));
  p->adj.H = a.take_bytes(std::max(adj_h_elems(R) * dtype_size(R.dtype), adj_h_elems(P) * dtype_size(P.dtype)));
  p->adj.Cs = a.take_bytes(std::max(adj_c_elems(R) * dtype_size(R.dtype), adj_c_elems(P) * dtype_size(P.dtype)));
  // split-K partial sums of the token-axis contractions (up to 16 splits of both sides' blocks, which can share
  // one launch) and of the adjoint products
  p->adj.part_elems = 16 * std::max({R.prim_len + P.prim_len, p->sup_elems});
  p->adj.part = a.take<float>(p->adj.part_elems);
  return a.used();
}

// out[:, block] = in[:, block] F_block^T (trans) or in[:, block] F_block, over the blocks of side S (T rows), with F
// as identity + delta: Db holds the bf16 deltas F - I in row order and the identity part adds in itself
GemmDesc act_apply(const SideInfo& S, int T, const void* in, int64_t ldi, const __bf16* Db, bool trans, void* out,
                   int64_t ldo) {
  GemmDesc g;
  g.kclass = POET_K_APPLY;
  g.compute = BF16;
  g.M = T; g.N = S.bp; g.K = S.bp; g.Ntot = g.Ktot = S.d; g.batch = S.nprim;
  g.A = in; g.lda = ldi; g.sA = S.bp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = Db; g.ldb = S.bp; g.sB = (int64_t)S.bp * S.bp; g.b_dt = BF16; g.b_kmajor = trans ? 1 : 0;
  g.C = out; g.ldc = ldo; g.sC = S.bp; g.c_dt = BF16;
  g.E = in; g.lde = ldi; g.sE = S.bp;
  return g;
}

// diagonal blocks of A^T B over the T tokens: dF_block = A[:, block]^T B[:, block], float32 bp x bp blocks
GemmDesc act_contract(const SideInfo& S, int T, const void* A, int64_t lda, const void* B, int64_t ldb, float* dF,
                      const AdjBufs& adj) {
  GemmDesc g;
  g.kclass = POET_K_CONTRACT;
  g.compute = BF16;
  g.M = g.N = S.bp; g.K = T; g.Mtot = g.Ntot = S.d; g.batch = S.nprim;
  g.A = A; g.lda = lda; g.sA = S.bp; g.a_dt = BF16; g.a_kmajor = 0;
  g.B = B; g.ldb = ldb; g.sB = S.bp; g.b_dt = BF16; g.b_kmajor = 0;
  g.C = dF; g.ldc = S.bp; g.sC = (int64_t)S.bp * S.bp; g.c_dt = F32;
  g.part = adj.part; g.part_elems = adj.part_elems;
  return g;
}

// dF = blocks of A^T B over the tokens (small blocks through super-block products), then the adjoint unless dtheta
// is null (the caller finishes the primitive gradient dF itself, e.g. with poet_adjoint_group)
hipError_t act_contract_adjoint(const SideInfo& S, int T, const void* A, int64_t lda, const void* B, int64_t ldb,
                                float* dF, const void* powers, float* dtheta, const ActBwdPlan& p, hipStream_t st) {
  const int g = super_group(S);
  hipError_t e;
  if (g == 1) {
    if ((e = contract_only(S, act_contract(S, T, A, lda, B, ldb, dF, p.adj), dF, st)) != hipSuccess) return e;
  } else {
    SideInfo U = S;  // the super-block view: blocks of g bp
    U.bp = g * S.bp;
    U.nprim = (S.nprim + g - 1) / g;
    GemmDesc gd = act_contract(U, T, A, lda, B, ldb, p.sup, p.adj);
    if ((e = launch_gemm(gd, st)) != hipSuccess) return e;
    if ((e = launch_extract_diag(p.sup, U.bp, g, S.bp, S.d, S.nprim, dF, st)) != hipSuccess) return e;
  }
  return dtheta ? neumann_adjoint(S, dF, powers, dtheta, p.adj, st) : hipSuccess;
}

// bf16 deltas F - I of a side's primitives, row-major bp x bp blocks (zero in the identity padding of ragged blocks)
hipError_t deltas_bf16(const SideInfo& S, const float* prim, __bf16* out, hipStream_t st) {
  return launch_delta_bf16(prim, S.nprim, S.bp, S.bp, out, st);
}

// out = in F^T (trans) or in F over the blocks of side S: the weight-stationary kernel where it applies, else a
// batched GEMM. Both apply F as identity + delta: the bf16 operand is the delta F - I, from ops (the caller's copies
// of the deltas of F and F^T, zero outside each block's corner) or written to the scratch Fb first, and the identity
// part adds the input in float32 before the output is rounded.
hipError_t act_factor(const SideInfo& S, int T, const void* in, int64_t ldi, const float* prim, const void* ops,
                      __bf16* Fb, bool trans, void* out, int64_t ldo, hipStream_t st) {
  hipError_t e;
  const __bf16* opsF = reinterpret_cast<const __bf16*>(ops);
  if (act_apply_eligible(S.bp, in, ldi, out, ldo, T)) {
    const __bf16* Bt = opsF ? opsF + (trans ? 0 : S.prim_len) : Fb;  // rows Bt[j][k] = B(k, j)
    if (!opsF && (e = launch_act_operand(prim, S.bp, S.d, S.nprim, trans, Fb, st)) != hipSuccess) return e;
    return launch_act_apply(reinterpret_cast<const __bf16*>(in), ldi, reinterpret_cast<__bf16*>(out), ldo, Bt, T,
                            S.d, S.bp, S.nprim, st);
  }
  // the batched GEMM takes the deltas in row order: the third part of the caller's copies
  if (!opsF && (e = deltas_bf16(S, prim, Fb, st)) != hipSuccess) return e;
  return launch_gemm(act_apply(S, T, in, ldi, opsF ? opsF + 2 * S.prim_len : Fb, trans, out, ldo), st);
}

// A factor folded into the bf16 copy of W0 (row pitch ldw): P side out = W0b P (P's blocks along the columns), R side
// out = R W0b (R's blocks along the rows), with the factor as identity + delta: one batched bf16 GEMM over the
// factor's blocks with the deltas F - I as bf16 operands in row order (the third part of the caller's operand
// copies, else made in Db), W0b itself added in float32 before the one rounding of the output; ragged last blocks
// through the extents.
GemmDesc fold_desc(const poet_layer& L, const SideInfo& S, bool rside, const void* W0b, const __bf16* Db, __bf16* out) {
  GemmDesc g;
  g.kclass = POET_K_APPLY;
  g.compute = BF16;
  g.batch = S.nprim;
  g.K = S.bp;
  g.a_dt = g.b_dt = BF16;
  g.c_dt = BF16;
  g.C = out; g.ldc = L.ldw;
  g.E = W0b; g.lde = L.ldw;  // the identity part: W0b at the output's position
  if (!rside) {  // out[:, J] = W0b[:, J] P_J
    g.M = L.m; g.N = S.bp; g.Ntot = g.Ktot = L.n;
    g.A = W0b; g.lda = L.ldw; g.sA = S.bp; g.a_kmajor = 1;
    g.B = Db; g.ldb = S.bp; g.sB = (int64_t)S.bp * S.bp; g.b_kmajor = 0;  // B(k, j) = P_J[k][j] - I
    g.sC = g.sE = S.bp;
  } else {  // out[I, :] = R_I W0b[I, :]
    g.M = S.bp; g.N = L.n; g.Mtot = g.Ktot = L.m;
    g.A = Db; g.lda = S.bp; g.sA = (int64_t)S.bp * S.bp; g.a_kmajor = 1;  // A(i, k) = R_I[i][k] - I
    g.B = W0b; g.ldb = L.ldw; g.sB = (int64_t)S.bp * L.ldw; g.b_kmajor = 0;
    g.sC = g.sE = (int64_t)S.bp * L.ldw;
  }
  return g;
}
hipError_t fold_factor(const poet_layer& L, const SideInfo& S, bool rside, const void* W0b, const float* prim,
                       const void* ops, __bf16* Fb, __bf16* out, hipStream_t st) {
  if (ops) {
    Fb = const_cast<__bf16*>(reinterpret_cast<const __bf16*>(ops)) + 2 * S.prim_len;
  } else {
    const hipError_t e = deltas_bf16(S, prim, Fb, st);
    if (e != hipSuccess) return e;
  }
  return launch_gemm(fold_desc(L, S, rside, W0b, Fb, out), st);
}

// products of one shape (sizes, orientations, strides, output pitch and type) share a grouped launch, 16 at most
bool same_shape(const GemmDesc& a, const GemmDesc& b) {
  return a.M == b.M && a.N == b.N && a.K == b.K && a.Mtot == b.Mtot && a.Ntot == b.Ntot && a.Ktot == b.Ktot &&
         a.batch == b.batch && a.a_kmajor == b.a_kmajor && a.b_kmajor == b.b_kmajor && a.lda == b.lda &&
         a.ldb == b.ldb && a.sA == b.sA && a.sB == b.sB && a.ldc == b.ldc && a.sC == b.sC && a.c_dt == b.c_dt;
}
hipError_t launch_grouped(const std::vector<GemmDesc>& all, hipStream_t st) {
  std::vector<bool> done(all.size(), false);
  for (size_t i = 0; i < all.size(); ++i) {
    if (done[i]) continue;
    GemmDesc pr[MAXG];
    int n = 0;
    for (size_t j = i; j < all.size() && n < MAXG; ++j)
      if (!done[j] && same_shape(all[i], all[j])) { pr[n++] = all[j]; done[j] = true; }
    if (n > 1 && fast_gemm_group_eligible(pr, n)) {
      HIP_RET(launch_fast_gemm_group(pr, n, st));
    } else {
      for (int u = 0; u < n; ++u) HIP_RET(launch_gemm(pr[u], st));
    }
  }
  return hipSuccess;
}

// Buffers of the float32-accurate FS merge of one side (reused by the other): the gathered columns (P) or rows (R)
// of W0 in float32 (Dg) and as three bf16 parts (Xcat), the factor delta's three parts (Fcat), the product (C) and
// its split-K scratch.
struct Fs3Bufs {
  float* Dg = nullptr;
  __bf16 *Xcat = nullptr, *Fcat = nullptr;
  float *C = nullptr, *part = nullptr;
  size_t part_elems = 0;
};

// float32 scratch the fast kernel's split-K and addend epilogue take for one M x N x K product
size_t fs3_part_elems(int M, int N, int K) {
  GemmDesc g;
  g.M = M; g.N = N; g.K = K;
  g.part = reinterpret_cast<float*>(256);  // split count with unlimited scratch (nothing is dereferenced)
  g.part_elems = ~(size_t)0;
  return (size_t)fast_gemm_splits(g) * M * N;
}

struct MergePlan {
  bool inplace = false;   // both sides block-diagonal with blocks <= 256: two in-place passes over W0
  char* split = nullptr;  // their pre-split factor deltas
  bool fs3 = false;       // both sides FS: gather, float32-accurate bf16 product, scatter, in place per side
  Fs3Bufs f3;
  float *T = nullptr, *Wn = nullptr;
  int32_t* flags = nullptr;
  FsBufs fs;
};
size_t plan_merge(const poet_layer& L, const SideInfo& R, const SideInfo& P, void* ws, MergePlan* p) {
  Arena a(ws);
  p->inplace = R.mode == POET_BS && P.mode == POET_BS && bs_merge_eligible(R.bp, L.m, L.ldw) &&
                bs_merge_eligible(P.bp, L.m, L.ldw);
  if (p->inplace) {
    p->split = reinterpret_cast<char*>(
        a.take_bytes(bs_merge_split_bytes(R.bp, R.nprim) + bs_merge_split_bytes(P.bp, P.nprim)));
    return a.used();
  }
  p->fs3 = R.mode == POET_FS && P.mode == POET_FS;
  if (p->fs3) {
    const size_t m = L.m, n = L.n, sP = P.bp, sR = R.bp, spP = pad8(P.bp), spR = pad8(R.bp);
    p->f3.Dg = a.take<float>(std::max(m * sP, sR * n));
    p->f3.C = a.take<float>(std::max(m * sP, sR * n));
    p->f3.Xcat = a.take<__bf16>(std::max(m * 3 * spP, 3 * spR * pad8(L.n)));
    p->f3.Fcat = a.take<__bf16>(std::max(3 * spP * spP, sR * 3 * spR));
    p->f3.part_elems = std::max(fs3_part_elems(L.m, P.bp, 3 * (int)spP), fs3_part_elems(R.bp, L.n, 3 * (int)spR));
    p->f3.part = a.take<float>(p->f3.part_elems);
    p->flags = a.take<int32_t>((size_t)std::max(L.m, L.n));
    return a.used();
  }
  const size_t mn = (size_t)L.m * L.ldw;
  p->T = a.take<float>(mn);
  p->Wn = a.take<float>(mn);
  plan_fs(a, L, R, P, &p->fs);
  if (R.mode == POET_FS || P.mode == POET_FS) p->flags = a.take<int32_t>((size_t)std::max(L.m, L.n));
  return a.used();
}

bool check_ws(void* ws, size_t have, size_t need) {
  if (have < need) return fail(POET_E_WORKSPACE, "workspace of %zu bytes < %zu needed", have, need), false;
  if (!ws && need > 0) return fail(POET_E_ARG, "null workspace"), false;
  return true;
}

// ---- grouped calls: the per-block kernels of many sides (e.g. every linear of a transformer block) in shared
// launches of up to MAXG sides each ----
bool group_sides(int32_t count, const poet_side* sides, std::vector<SideInfo>* out) {
  if (count < 0) return fail(POET_E_ARG, "count = %d must be >= 0", count), false;
  if (count > 0 && !sides) return fail(POET_E_ARG, "null sides"), false;
  out->resize(count);
  char name[32];
  for (int i = 0; i < count; ++i) {
    snprintf(name, sizeof name, "sides[%d]", i);
    if (!side_info(&sides[i], &(*out)[i], name)) return false;
  }
  return true;
}

// the fused chain kernel takes the side (BS or FS, bf16, primitive <= 256 and a multiple of 8, unpadded powers)
bool chain_side(const SideInfo& S, const void* powers) {
  return S.k > 0 && S.ldp == S.bp && power_chain_eligible(S.bp, S.dtype, powers);
}

// build chunks: sides whose chain runs as GEMMs (k >= 1, bf16, not on the fused chain, primitives of at least 128
// so the fast kernel takes the products) sharing (bp, ldp, k), at most MAXG per chunk; each power step of a chunk
// is one grouped GEMM. Sizing passes powers = nullptr (aligned buffers assumed).
struct BuildChunk {
  int bp = 0, ldp = 0, k = 0;
  size_t prim_elems = 0;
  std::vector<int> idx;
};
bool gemm_chain_side(const SideInfo& S, const void* powers) {
  const bool al = !powers || (reinterpret_cast<uintptr_t>(powers) & 15) == 0;
  return S.k > 0 && S.dtype == BF16 && S.bp >= 128 && al && !chain_side(S, powers ? powers : (const void*)256);
}
std::vector<BuildChunk> build_chunks(const std::vector<SideInfo>& S, void* const* powers) {
  std::vector<BuildChunk> ch;
  for (int i = 0; i < (int)S.size(); ++i) {
    if (!gemm_chain_side(S[i], powers ? powers[i] : nullptr)) continue;
    BuildChunk* c = nullptr;
    for (auto& x : ch)
      if (x.bp == S[i].bp && x.ldp == S[i].ldp && x.k == S[i].k && (int)x.idx.size() < MAXG) c = &x;
    if (!c) { ch.emplace_back(); c = &ch.back(); c->bp = S[i].bp; c->ldp = S[i].ldp; c->k = S[i].k; }
    c->idx.push_back(i);
    c->prim_elems += S[i].prim_len;
  }
  return ch;
}
// split-K scratch of a chunk's power products: up to 4 splits of every block
size_t build_chunk_part_elems(const BuildChunk& c) { return 8 * c.prim_elems; }

// split-K scratch of the build's power-chain GEMMs: bf16 sides the fused chain kernel does not take (FS, or BS
// blocks above 256 or not a multiple of 8); room for up to 8 splits of one power
size_t build_part_elems(const SideInfo& i) {
  const bool gemm_chain = i.dtype == BF16 && i.k > 0 && !(i.ldp == i.bp && i.bp <= 256 && i.bp % 8 == 0);
  return gemm_chain ? 8 * i.prim_len : 0;
}

// Accurate square term of a bf16 chain that runs as separate products. The bf16 chain rounds Q to bf16 as a product
// operand and keeps Q^2 in bf16: two relative errors of 2^-9 on the series' largest term beyond the linear one, which
// the float32 merge then folds into W0 (about 7e-6 relative on a merged LLaMA-1.3B weight at s = 1024 and 2e-5 at
// s = 2730). So (2Q)^2 is formed to float32 accuracy from three bf16 parts of 2Q = prim - I (exact in float32 after
// theta_prep): hi = bf16(x), lo = bf16(x - hi), stacked along K as [hi | hi | lo] times [hi ; lo ; hi], one bf16
// product with K = 3 ldp giving hi*hi + hi*lo + lo*hi. The chain finalize takes it in place of the saved P_2;
// the bf16 powers still serve the higher terms and the adjoint.
bool sq_side(const SideInfo& S) { return build_part_elems(S) > 0; }
struct SqBufs {
  __bf16* A3 = nullptr;  // per primitive bp x 3 ldp (K-major left operand)
  __bf16* B3 = nullptr;  // per primitive 3 ldp x ldp (rows of the right operand)
  float* q2 = nullptr;   // per primitive bp x bp
};
void plan_sq(Arena& a, const SideInfo& S, SqBufs* b) {
  const size_t np = S.nprim, bp = S.bp, lp = S.ldp;
  b->A3 = a.take<__bf16>(np * bp * 3 * lp);
  b->B3 = a.take<__bf16>(np * 3 * lp * lp);
  b->q2 = a.take<float>(np * bp * bp);
}
size_t sq_bytes(const SideInfo& S) {
  Arena a(nullptr);
  SqBufs b;
  plan_sq(a, S, &b);
  return a.used();
}
// the three-part operands of 2Q = prim - I, block by block (the identity is subtracted on each block's diagonal)
hipError_t sq_split(const SideInfo& S, const float* prim, const SqBufs& b, hipStream_t st) {
  const int bp = S.bp, lp = S.ldp;
  for (int p = 0; p < S.nprim; ++p) {
    const float* src = prim + (int64_t)p * bp * bp;
    HIP_RET(launch_split3(src, bp, nullptr, nullptr, bp, bp, 1, bp, bp, bp, lp, b.A3 + (int64_t)p * bp * 3 * lp,
                          3 * lp, lp, 0b100, nullptr, 0, st));
    HIP_RET(launch_split3(src, bp, nullptr, nullptr, bp, bp, 1, bp, bp, lp, lp, b.B3 + (int64_t)p * 3 * lp * lp, lp,
                          (int64_t)lp * lp, 0b010, nullptr, 0, st));
  }
  return hipSuccess;
}
GemmDesc sq_gemm(const SideInfo& S, const SqBufs& b, float* part, size_t part_elems) {
  GemmDesc g;
  g.kclass = POET_K_CHAIN;
  g.compute = BF16; g.M = g.N = S.bp; g.K = 3 * S.ldp; g.batch = S.nprim;
  g.A = b.A3; g.lda = 3 * S.ldp; g.sA = (int64_t)S.bp * 3 * S.ldp; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = b.B3; g.ldb = S.ldp; g.sB = (int64_t)3 * S.ldp * S.ldp; g.b_dt = BF16; g.b_kmajor = 0;
  g.C = b.q2; g.c_dt = F32; g.ldc = S.bp; g.sC = (int64_t)S.bp * S.bp;
  g.part = part; g.part_elems = part_elems;
  return g;
}

// adjoint chunks: sides sharing (bp, k) whose adjoint runs on the fused chain, at most MAXG per chunk
// fused: the H chain runs on the fused chain kernel (blocks <= 256, ldp = bp); otherwise as grouped GEMMs (ldp >= bp)
struct AdjChunk {
  int bp = 0, ldp = 0, k = 0, nb = 0;
  bool fused = true;
  std::vector<int> idx;
};
std::vector<AdjChunk> adjoint_chunks(const std::vector<SideInfo>& S, const void* const* powers, std::vector<int>* solo) {
  std::vector<AdjChunk> ch;
  for (int i = 0; i < (int)S.size(); ++i) {
    if (S[i].theta_len == 0) continue;
    const void* pw = powers ? powers[i] : reinterpret_cast<const void*>(256);  // sizing: assume aligned powers
    const bool fused = chain_side(S[i], pw);
    if (!fused && !gemm_chain_side(S[i], powers ? powers[i] : nullptr)) { solo->push_back(i); continue; }
    AdjChunk* c = nullptr;
    for (auto& x : ch)
      if (x.fused == fused && x.bp == S[i].bp && x.ldp == S[i].ldp && x.k == S[i].k && (int)x.idx.size() < MAXG) c = &x;
    if (!c) {
      ch.emplace_back(); c = &ch.back();
      c->bp = S[i].bp; c->ldp = S[i].ldp; c->k = S[i].k; c->fused = fused;
    }
    c->idx.push_back(i);
    c->nb += S[i].nprim;
  }
  return ch;
}

// scratch of one chunk: H_0..H_k and the coefficient stack of every block (bf16), the adjoint product's split-K
// partials (up to 4 splits; at least one float32 block per primitive, which also serves the unsplit generic path)
struct AdjChunkBufs {
  __bf16 *H = nullptr, *Cs = nullptr;
  float* part = nullptr;
  size_t part_elems = 0;
};
size_t plan_adj_chunk(const AdjChunk& c, void* ws, AdjChunkBufs* b) {
  Arena a(ws);
  const size_t pp = (size_t)c.bp * c.bp, nb = (size_t)c.nb;
  b->H = a.take<__bf16>(nb * c.bp * (size_t)c.ldp * (c.k + 1));
  b->Cs = a.take<__bf16>(nb * (size_t)c.ldp * c.ldp * (c.k + 1));
  b->part_elems = 4 * nb * pp;
  b->part = a.take<float>(b->part_elems);
  return a.used();
}

// scratch of one side's own adjoint (sides the chunks do not take)
size_t plan_adj_solo(const SideInfo& S, void* ws, AdjBufs* b) {
  Arena a(ws);
  b->dQ = a.take<float>(S.prim_len);
  b->H = a.take_bytes(adj_h_elems(S) * dtype_size(S.dtype));
  b->Cs = a.take_bytes(adj_c_elems(S) * dtype_size(S.dtype));
  b->part_elems = 4 * S.prim_len;
  b->part = a.take<float>(b->part_elems);
  return a.used();
}

size_t adjoint_group_bytes(const std::vector<SideInfo>& S, const void* const* powers) {
  std::vector<int> solo;
  const auto ch = adjoint_chunks(S, powers, &solo);
  size_t need = 0;
  AdjChunkBufs cb;
  for (const auto& c : ch) need = std::max(need, plan_adj_chunk(c, nullptr, &cb));
  AdjBufs sb;
  for (size_t i = 0; i < S.size(); ++i)  // any side may end up on its own (misaligned powers)
    if (S[i].theta_len > 0 && S[i].k > 0) need = std::max(need, plan_adj_solo(S[i], nullptr, &sb));
  return need;
}

// the Neumann adjoint and skew projection of one chunk (see neumann_adjoint for the algebra): H_j of every block
// side by side (row pitch (k+1) ldp), the coefficient stacks, one product over all blocks, one projection
hipError_t adjoint_chunk(const AdjChunk& c, const std::vector<SideInfo>& S, const float* const* dprim,
                         const void* const* powers, float* const* dtheta, const AdjChunkBufs& b, hipStream_t st) {
  const int bp = c.bp, k = c.k, ldp = c.ldp, ldh = (k + 1) * ldp;
  const int64_t pp = (int64_t)bp * bp, hs = (int64_t)bp * ldh;
  hipError_t e;
  if (c.fused) {  // H_0 = dR and H_{j+1} = Q H_j for every block of the chunk in one launch
    ChainGroup g;
    int boff = 0;
    for (int i : c.idx) {
      ChainArgs& a = g.a[g.n++];
      a.bp = bp; a.nprim = S[i].nprim; a.steps = k;
      a.A = reinterpret_cast<const __bf16*>(powers[i]); a.sA = pp;
      a.X0 = dprim[i]; a.ldx0 = bp; a.sx0 = pp;
      a.Y = b.H + (size_t)boff * hs; a.ldy = ldh; a.sy = hs; a.jstep = bp; a.write_x0 = 1;
      boff += S[i].nprim;
    }
    if ((e = launch_power_chain_group(g, POET_K_ADJOINT, st)) != hipSuccess) return e;
  } else {  // H_0 = bf16(dR), then H_j = Q^j H_0 from each side's saved powers, k products per side in grouped
    // launches
    if (ldp > bp && (e = launch_zero_gaps(b.H, (int64_t)c.nb * bp, ldh, ldp, bp, k + 1, st)) != hipSuccess)
      return e;  // the gap columns past bp stay zero
    int boff = 0;
    std::vector<GemmDesc> pr;
    for (int i : c.idx) {
      __bf16* Hi = b.H + (size_t)boff * hs;
      if ((e = launch_convert(dprim[i], bp, Hi, ldh, BF16, S[i].nprim * bp, bp, st)) != hipSuccess) return e;
      h_products(S[i], powers[i], reinterpret_cast<char*>(Hi), &pr);
      boff += S[i].nprim;
    }
    if ((e = launch_grouped(pr, st)) != hipSuccess) return e;
  }
  {  // the coefficient stacks C_0..C_k from the saved powers
    CoefGroup g;
    g.bp = bp; g.ldp = ldp; g.k = k;
    int boff = 0;
    for (int i : c.idx) {
      CoefSide& a = g.s[g.n++];
      a.powers = powers[i]; a.out = b.Cs + (size_t)boff * (k + 1) * ldp * ldp; a.nprim = S[i].nprim;
      boff += S[i].nprim;
    }
    if ((e = launch_adjoint_coefs_group(g, BF16, st)) != hipSuccess) return e;
  }
  GemmDesc g;  // [H_0 .. H_k] [C_0; ..; C_k] for all blocks of the chunk as one batch
  g.kclass = POET_K_ADJOINT;
  g.compute = BF16; g.M = g.N = bp; g.K = ldh; g.batch = c.nb;
  g.A = b.H; g.lda = ldh; g.sA = hs; g.a_dt = BF16; g.a_kmajor = 1;
  g.B = b.Cs; g.ldb = ldp; g.sB = (int64_t)(k + 1) * ldp * ldp; g.b_dt = BF16; g.b_kmajor = 0;
  g.C = b.part; g.ldc = bp; g.sC = pp; g.c_dt = F32;
  g.part = b.part; g.part_elems = b.part_elems;
  int ns = 1;
  g.defer_reduce = 1;
  if (fast_gemm_eligible(g)) {  // split-K partials, reduced with a_1 dR = 2 dR inside the skew projection
    ns = fast_gemm_splits(g);
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  } else {  // the product itself lands in the partial buffer (one split)
    g.defer_reduce = 0;
    g.part = nullptr; g.part_elems = 0;
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
  }
  SkewGroup sg;
  sg.bp = bp; sg.part = b.part; sg.split_stride = (int64_t)c.nb * pp; sg.beta = 2.f;  // a_1 = 2 for k >= 1
  int boff = 0;
  for (int i : c.idx) {
    SkewSide& a = sg.s[sg.n++];
    a.D = dprim[i]; a.dtheta = dtheta[i]; a.mode = S[i].mode; a.d = S[i].d; a.nprim = S[i].nprim; a.boff = boff;
    boff += S[i].nprim;
  }
  return launch_reduce_skew_group(sg, ns, st);
}

bool check_idx(const SideInfo& S, const void* idx, const char* name) {
  if (S.mode == POET_FS && !idx) return fail(POET_E_ARG, "%s: FS side needs an index set", name), false;
  if (S.mode == POET_BS && idx) return fail(POET_E_ARG, "%s: BS side takes no index set", name), false;
  return true;
}

}  // namespace

// ---- allocation-free sampler ----------------------------------------------------------------------------
// The sampler's per-index flags live in a file-scope device array instead of a caller workspace. Each device holds
// its own copy of the array at its own address, looked up once per device with the device current and kept; kernels
// only ever see that address (the array's name is a host-side stand-in in host code).
static __device__ __align__(256) int32_t scratch[POET_NOALLOC_MAX_D];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device id; nullptr until looked up

hipError_t scratch_address(int32_t** out) {
  int dev = 0;
  HIP_RET(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_RET(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = reinterpret_cast<int32_t*>(g_scratch_ptr[dev]);
  return hipSuccess;
}
}  // namespace

// ============================================================================================================
extern "C" {

size_t poet_theta_len(const poet_side* s) {
  SideInfo i;
  return side_info(s, &i, "side") ? i.theta_len : 0;
}
size_t poet_num_prims(const poet_side* s) {
  SideInfo i;
  return side_info(s, &i, "side") ? (size_t)i.nprim : 0;
}
size_t poet_prim_len(const poet_side* s) {
  SideInfo i;
  return side_info(s, &i, "side") ? i.prim_len : 0;
}
size_t poet_powers_len(const poet_side* s) {
  SideInfo i;
  return side_info(s, &i, "side") ? i.powers_len : 0;
}
size_t poet_build_workspace_bytes(const poet_side* s, int with_powers) {
  SideInfo i;
  if (!side_info(s, &i, "side")) return 0;
  if (i.k == 0) return 0;
  const size_t pw = with_powers ? 0 : align_up(i.powers_len * dtype_size(i.dtype), 256);
  const size_t part = build_part_elems(i) * sizeof(float);
  const size_t sq = sq_side(i) ? sq_bytes(i) : 0;
  return pw + part == 0 ? 0 : pw + part + sq + 512;
}
size_t poet_sample_workspace_bytes(int32_t d) { return d > 0 ? align_up((size_t)d * 4, 256) + 256 : 0; }

size_t poet_workspace_bytes(const poet_layer* L, int op) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return 0;
  switch (op) {
    case POET_OP_BUILD: return 0;
    case POET_OP_FWD: { FwdPlan p; return plan_fwd(*L, R, P, nullptr, true, &p); }
    case POET_OP_BWD: { BwdPlan p; return plan_bwd(*L, R, P, nullptr, true, &p); }
    case POET_OP_MERGE: { MergePlan p; return plan_merge(*L, R, P, nullptr, &p); }
    case POET_OP_FWD_ACT: { ActFwdPlan p; return plan_fwd_act(*L, R, P, nullptr, &p); }
    case POET_OP_BWD_ACT: { ActBwdPlan p; return plan_bwd_act(*L, R, P, nullptr, &p); }
    default: fail(POET_E_ARG, "bad op %d", op); return 0;
  }
}

poet_status poet_build_orthogonal(const poet_side* s, const float* theta, float* prim, void* powers, float* qnorm,
                                  int32_t flags, void* ws, size_t ws_bytes, void* stream) {
  SideInfo S;
  if (!side_info(s, &S, "side")) return g_last;
  if (flags != POET_BUILD_STEP && flags != POET_BUILD_MERGE) return fail(POET_E_ARG, "bad build flags %d", flags);
  if (!prim) return fail(POET_E_ARG, "null prim");
  if (!theta && S.theta_len > 0) return fail(POET_E_ARG, "null theta");
  const size_t need = poet_build_workspace_bytes(s, powers != nullptr);
  if (!check_ws(ws, ws_bytes, need)) return g_last;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t esz = dtype_size(S.dtype);
  // powers P_1 = Q, ..., P_k (the caller's buffer, or the workspace when the caller keeps none), then the split-K
  // scratch of the GEMM chain
  char* pw = reinterpret_cast<char*>(powers);
  Arena a(ws);
  if (!powers && S.k > 0) pw = reinterpret_cast<char*>(a.take_bytes(S.powers_len * esz));
  const size_t part_elems = build_part_elems(S);
  float* part = part_elems ? a.take<float>(part_elems) : nullptr;
  SqBufs sq;
  if (sq_side(S) && flags == POET_BUILD_MERGE) plan_sq(a, S, &sq);
  if (qnorm) HIP_TRY(launch_qnorm(theta, S.mode, S.d, S.bp, S.nprim, qnorm, st));
  // prim = I + coef Q (coef 2 for k >= 1) with Q exact from theta, and the first saved power Q
  HIP_TRY(launch_theta_prep(theta, S.mode, S.d, S.bp, S.nprim, S.k, prim, S.k > 0 ? (void*)pw : nullptr, S.dtype,
                            S.ldp, st));
  if (S.k > 0 && S.ldp == S.bp && power_chain_eligible(S.bp, S.dtype, pw)) {
    // the k products and the rest of the series in one launch, Q resident in LDS
    ChainArgs c;
    c.bp = S.bp; c.nprim = S.nprim; c.steps = S.k; c.build = 1; c.prim = prim;
    c.A = reinterpret_cast<const __bf16*>(pw); c.sA = (int64_t)S.bp * S.bp;
    c.Y = reinterpret_cast<__bf16*>(pw); c.ldy = S.bp; c.sy = (int64_t)S.bp * S.bp; c.jstep = (int64_t)S.plen;
    HIP_TRY(launch_power_chain(c, POET_K_CHAIN, st));
    return POET_OK;
  }
  if (S.k == 0) return POET_OK;  // R_0 = I + Q
  const int64_t pp = (int64_t)S.bp * S.bp;
  const int64_t ps = (int64_t)S.bp * S.ldp;
  if (sq.q2) {  // (2Q)^2 to float32 accuracy while prim still holds I + 2Q
    HIP_TRY(sq_split(S, prim, sq, st));
    HIP_TRY(launch_gemm(sq_gemm(S, sq, part, part_elems), st));
  }
  // P_{i+1} = Q P_i; the last power goes straight into prim (float32). With the accurate square and k == 1 the series
  // ends at Q^2 and no chain product is needed.
  for (int i = 1; i <= S.k && !(sq.q2 && S.k == 1); ++i) {
    GemmDesc g;
    g.kclass = POET_K_CHAIN;
    g.compute = S.dtype; g.M = g.N = g.K = S.bp; g.batch = S.nprim;
    g.A = pw; g.lda = S.ldp; g.sA = ps; g.a_dt = S.dtype; g.a_kmajor = 1;
    g.B = pw + (size_t)(i - 1) * S.plen * esz; g.ldb = S.ldp; g.sB = ps; g.b_dt = S.dtype; g.b_kmajor = 0;
    if (i < S.k) { g.C = pw + (size_t)i * S.plen * esz; g.c_dt = S.dtype; g.ldc = S.ldp; g.sC = ps; }
    else { g.C = prim; g.c_dt = F32; g.ldc = S.bp; g.sC = pp; }
    g.part = part; g.part_elems = part_elems;
    g.tri = (i + 1) % 2 == 0 ? 1 : -1;  // Q^(i+1): symmetric or skew-symmetric, as in the grouped build
    HIP_TRY(launch_gemm(g, st));
  }
  // prim = I + 2Q + 2(P_2 + ... + P_k) + P_{k+1}, the linear term exact from theta (P_2 from q2 when formed)
  HIP_TRY(launch_chain_finalize(theta, S.mode, S.d, S.bp, S.nprim, S.k, pw, S.dtype, S.ldp, prim, st, sq.q2));
  return POET_OK;
}

poet_status poet_build_orthogonal_exact(const poet_side* s, const float* theta, float* prim, void* stream) {
  SideInfo S;
  if (!side_info(s, &S, "side")) return g_last;
  if (!prim) return fail(POET_E_ARG, "null prim");
  if (!theta && S.theta_len > 0) return fail(POET_E_ARG, "null theta");
  if (S.bp > 256)
    return fail(POET_E_UNSUPPORTED, "exact Cayley primitives of size %d: this build takes primitives up to 256", S.bp);
  if (S.nprim > 65535) return fail(POET_E_UNSUPPORTED, "%d primitives exceed one launch", S.nprim);
  HIP_TRY(launch_cayley_exact(theta, S.mode, S.d, S.bp, S.nprim, prim, reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

poet_status poet_sample_indices(int32_t d, int32_t s, uint64_t seed, uint32_t linear_id, uint32_t side,
                                uint32_t epoch, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (d < 1 || s < 0 || s > d) return fail(POET_E_SHAPE, "need d >= 1 and 0 <= s <= d (d=%d s=%d)", d, s);
  if (!idx && s > 0) return fail(POET_E_ARG, "null idx");
  if (!check_ws(ws, ws_bytes, poet_sample_workspace_bytes(d))) return g_last;
  Arena a(ws);
  int32_t* flags = a.take<int32_t>((size_t)d);
  HIP_TRY(launch_sample(d, s, sampler_hash(seed, linear_id, side, epoch), flags, idx,
                        reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

poet_status poet_sample_indices_noalloc(int32_t d, int32_t s, uint64_t seed, uint32_t linear_id, uint32_t side,
                                        uint32_t epoch, int32_t* idx, void* stream) {
  if (d < 1 || s < 0 || s > d) return fail(POET_E_SHAPE, "need d >= 1 and 0 <= s <= d (d=%d s=%d)", d, s);
  if (d > POET_NOALLOC_MAX_D)
    return fail(POET_E_SHAPE, "d = %d exceeds the allocation-free sampler's maximum %d (use poet_sample_indices)", d,
                POET_NOALLOC_MAX_D);
  if (!idx && s > 0) return fail(POET_E_ARG, "null idx");
  int32_t* flags = nullptr;
  HIP_TRY(scratch_address(&flags));
  // every flag of [0, d) is written by the ranking kernel before the compaction reads it: nothing to clear
  HIP_TRY(launch_sample(d, s, sampler_hash(seed, linear_id, side, epoch), flags, idx,
                        reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

poet_status poet_sample_permutation(int32_t d, uint64_t seed, uint32_t linear_id, uint32_t side, uint32_t epoch,
                                    int32_t* perm, int32_t* inv, void* stream) {
  if (d < 1) return fail(POET_E_SHAPE, "need d >= 1 (d=%d)", d);
  if (!perm) return fail(POET_E_ARG, "null perm");
  HIP_TRY(launch_sample_permutation(d, sampler_hash(seed, linear_id, side, epoch), perm, inv,
                                    reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

poet_status poet_gather2d(int32_t rows, int32_t cols, int32_t elem_bytes, const void* in, int64_t ldi, int32_t in_rows,
                          int32_t in_cols, const int32_t* row_idx, const int32_t* col_idx, void* out, int64_t ldo,
                          void* stream) {
  if (rows < 0 || cols < 0 || in_rows < 1 || in_cols < 1)
    return fail(POET_E_SHAPE, "need rows, cols >= 0 and in_rows, in_cols >= 1");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(POET_E_ARG, "elem_bytes = %d must be 2 or 4", elem_bytes);
  if (ldi < in_cols || ldo < cols) return fail(POET_E_SHAPE, "leading dimensions below the row lengths");
  if (!row_idx && rows > in_rows) return fail(POET_E_SHAPE, "rows > in_rows without a row index");
  if (!col_idx && cols > in_cols) return fail(POET_E_SHAPE, "cols > in_cols without a column index");
  if (rows == 0 || cols == 0) return POET_OK;
  if (!in || !out) return fail(POET_E_ARG, "null in or out");
  HIP_TRY(launch_gather2d(rows, cols, elem_bytes, in, ldi, in_rows, in_cols, row_idx, col_idx, out, ldo,
                          reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

poet_status poet_linear_fwd(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                            const int32_t* idxR, const int32_t* idxP, const void* X, void* Y, void* W_out, void* ws,
                            size_t ws_bytes, void* stream) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  if (!W0 || !primR || !primP) return fail(POET_E_ARG, "null W0 or primitive");
  if (L->T > 0 && (!X || !Y)) return fail(POET_E_ARG, "null X or Y");
  if (!check_idx(R, idxR, "R") || !check_idx(P, idxP, "P")) return g_last;
  FwdPlan p;
  const size_t need = plan_fwd(*L, R, P, nullptr, W_out == nullptr, &p);
  if (!check_ws(ws, ws_bytes, need)) return g_last;
  plan_fwd(*L, R, P, ws, W_out == nullptr, &p);
  void* W = W_out ? W_out : p.W;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int act = L->act_dtype;
  if (bs_bf16(*L, R, P) && bs_apply_eligible(R.bp, P.bp, W0, L->ldw, primR, primP)) {
    HIP_TRY(launch_bs_apply(apply_args(*L, R, P, W0, primR, primP, nullptr, W, act, nullptr), st));
  } else if (bs_bf16(*L, R, P)) {
    HIP_TRY(launch_convert(W0, L->ldw, p.W0b, L->ldw, BF16, L->m, L->n, st));
    HIP_TRY(launch_delta_bf16(primR, R.nprim, R.bp, R.bp, p.dRb, st));
    HIP_TRY(launch_delta_bf16(primP, P.nprim, P.bp, P.bp, p.dPb, st));
    HIP_TRY(apply_P_b(*L, P, W0, p.W0b, p.dPb, p.Tb, p.T, p.part, st));
    HIP_TRY(apply_R_b(*L, R, p.Tb, p.T, p.dRb, W, act, p.part, st));
  } else if (act == BF16 && fs_bf16(*L, R) && fs_bf16(*L, P) && p.fs.Acb && p.fs.Brb) {
    HIP_TRY(fs_weight_bf16(*L, R, P, W0, primR, primP, idxR, idxP, W, p.fs, st));
  } else {
    HIP_TRY(apply_P(*L, P, W0, primP, idxP, p.T, act, p.fs, st));
    HIP_TRY(apply_R(*L, R, p.T, primR, idxR, W, act, L->ldw, act, p.fs, st));
  }
  if (L->T > 0) {  // Y = X W^T
    GemmDesc g;
    g.kclass = POET_K_TOKEN_FWD;
    g.compute = act; g.M = L->T; g.N = L->m; g.K = L->n;
    g.A = X; g.lda = L->ldx; g.a_dt = act; g.a_kmajor = 1;
    g.B = W; g.ldb = L->ldw; g.b_dt = act; g.b_kmajor = 1;
    g.C = Y; g.ldc = L->ldy; g.c_dt = act;
    HIP_TRY(launch_gemm(g, st));
  }
  return POET_OK;
}

}  // extern "C"

namespace {
// the weight-side backward; with dprimR/dprimP given it stops at the primitive gradients
// ZrIn / AcpIn (both or neither): the FS gradient operands formed beforehand by poet_fs_form (with Win its W); then
// W0 and the primitives are not read
poet_status bwd_weight(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                       const void* powersR, const void* powersP, const int32_t* idxR, const int32_t* idxP,
                       const void* Win, const void* X, const void* dY, void* dX, float* dthetaR, float* dthetaP,
                       float* dprimR, float* dprimP, void* ws, size_t ws_bytes, void* stream,
                       const void* ZrIn = nullptr, const void* AcpIn = nullptr) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  const bool formed = ZrIn && AcpIn;
  if (!formed && (!W0 || !primR || !primP)) return fail(POET_E_ARG, "null W0 or primitive");
  if (L->T > 0 && (!X || !dY)) return fail(POET_E_ARG, "null X or dY");
  const bool prims_only = dprimR || dprimP;
  if (prims_only) {
    if (!dprimR || !dprimP) return fail(POET_E_ARG, "null dprim");
  } else {
    if ((R.theta_len > 0 && !dthetaR) || (P.theta_len > 0 && !dthetaP)) return fail(POET_E_ARG, "null dtheta");
    if ((R.k > 0 && R.theta_len > 0 && !powersR) || (P.k > 0 && P.theta_len > 0 && !powersP))
      return fail(POET_E_ARG, "saved powers are required when k >= 1");
  }
  if (!check_idx(R, idxR, "R") || !check_idx(P, idxP, "P")) return g_last;
  BwdPlan p;
  const size_t need = plan_bwd(*L, R, P, nullptr, Win == nullptr, &p);
  if (!check_ws(ws, ws_bytes, need)) return g_last;
  plan_bwd(*L, R, P, ws, Win == nullptr, &p);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int act = L->act_dtype, m = L->m, n = L->n;
  const int64_t ldw = L->ldw;
  const bool fast = bs_bf16(*L, R, P);
  const void* W = Win;
  // both sides FS in bf16 with W given: the gradient's operands come from W0 and the sampled blocks alone
  const bool fs_pair = W && fs_bf16(*L, R) && fs_bf16(*L, P) && p.fs.Acb && p.fs.Brb;
  if (formed && !fs_pair) return fail(POET_E_UNSUPPORTED, "formed operands need both sides POET-FS in bf16 and W");
  if (formed) {  // the gradient's operands as formed beforehand (the same values fs_grad_operands writes)
    p.Zr = reinterpret_cast<float*>(const_cast<void*>(ZrIn));
    p.Acp = reinterpret_cast<float*>(const_cast<void*>(AcpIn));
  }
  if (fast && bs_apply_eligible(R.bp, P.bp, W0, ldw, primR, primP)) {
    // bf16 operands of the gradient: Z = W0 P (R side), R W0 (P side), and W when it is not given
    void* Wout = W ? nullptr : p.W;
    HIP_TRY(launch_bs_apply(apply_args(*L, R, P, W0, primR, primP, p.Tb, Wout, act, p.RW0b), st));
    if (!W) W = p.W;
  } else if (fast) {
    // bf16 operands: W0, the factor deltas, Z = W0 P (R-side gradient), R W0 (P-side gradient), G
    HIP_TRY(launch_convert(W0, ldw, p.W0b, ldw, BF16, m, n, st));
    HIP_TRY(launch_delta_bf16(primR, R.nprim, R.bp, R.bp, p.dRb, st));
    HIP_TRY(launch_delta_bf16(primP, P.nprim, P.bp, P.bp, p.dPb, st));
    HIP_TRY(apply_P_b(*L, P, W0, p.W0b, p.dPb, p.Tb, W ? nullptr : p.T, Part{p.adj.part, p.adj.part_elems}, st));
    if (!W) {
      HIP_TRY(apply_R_b(*L, R, p.Tb, p.T, p.dRb, p.W, act, Part{p.adj.part, p.adj.part_elems}, st));
      W = p.W;
    }
    HIP_TRY(apply_R_b(*L, R, p.W0b, W0, p.dRb, p.RW0b, BF16, Part{p.adj.part, p.adj.part_elems}, st));
  } else if (fs_pair && formed) {
    // nothing to form: Zr and Acp were given
  } else if (fs_pair) {
    // Z[I_R, :] and (R W0)[:, I_P], the only parts of Z = W0 P and R W0 the gradient reads
    HIP_TRY(fs_grad_operands(*L, R, P, W0, primR, primP, idxR, idxP, reinterpret_cast<__bf16*>(p.Zr),
                             reinterpret_cast<__bf16*>(p.Acp), p.fs, st));
  } else {
    // Z = W0 P (needed by the R-side gradient) and, when not given, W = R Z
    HIP_TRY(apply_P(*L, P, W0, primP, idxP, p.T, act, p.fs, st));
    if (!W) {
      HIP_TRY(apply_R(*L, R, p.T, primR, idxR, p.W, act, ldw, act, p.fs, st));
      W = p.W;
    }
    // R W0 (needed by the P-side gradient)
    HIP_TRY(apply_R(*L, R, W0, primR, idxR, p.RW0, F32, ldw, act, p.fs, st));
  }
  if (dX && L->T > 0) {  // dX = dY W
    GemmDesc g;
    g.kclass = POET_K_TOKEN_DX;
    g.compute = act; g.M = L->T; g.N = n; g.K = m;
    g.A = dY; g.lda = L->ldy; g.a_dt = act; g.a_kmajor = 1;
    g.B = W; g.ldb = ldw; g.b_dt = act; g.b_kmajor = 0;
    g.C = dX; g.ldc = L->ldx; g.c_dt = act;
    HIP_TRY(launch_gemm(g, st));
  }
  {  // G = dY^T X  (K = T; T == 0 gives G = 0)
    GemmDesc g;
    g.kclass = POET_K_TOKEN_GW;
    g.compute = act; g.M = m; g.N = n; g.K = L->T;
    g.A = dY; g.lda = L->ldy; g.a_dt = act; g.a_kmajor = 0;
    g.B = X; g.ldb = L->ldx; g.b_dt = act; g.b_kmajor = 0;
    if (fast) { g.C = p.Gb; g.c_dt = BF16; } else { g.C = p.G; g.c_dt = F32; }
    g.ldc = ldw;
    g.part = p.adj.part; g.part_elems = p.adj.part_elems;
    HIP_TRY(launch_gemm(g, st));
  }
  // primitive blocks of dL/dR = G Z^T (into the caller's dprimR when the adjoint is left to the caller)
  float* dRg = prims_only ? dprimR : p.dRg;
  float* dPg = prims_only ? dprimP : p.dPg;
  if (R.theta_len > 0 || prims_only) {
    GemmDesc g;
    g.kclass = POET_K_CONTRACT;
    g.compute = act;
    g.part = p.adj.part; g.part_elems = p.adj.part_elems;
    if (R.mode == POET_BS) {
      g.M = g.N = R.bp; g.K = n; g.Mtot = g.Ntot = m; g.batch = R.nprim;
      if (fast) {
        g.A = p.Gb; g.a_dt = BF16; g.B = p.Tb; g.b_dt = BF16;
      } else {
        g.A = p.G; g.a_dt = F32; g.B = p.T; g.b_dt = F32;
      }
      g.lda = ldw; g.sA = (int64_t)R.bp * ldw; g.a_kmajor = 1;
      g.ldb = ldw; g.sB = (int64_t)R.bp * ldw; g.b_kmajor = 1;
      g.C = dRg; g.ldc = R.bp; g.sC = (int64_t)R.bp * R.bp; g.c_dt = F32;
    } else {
      g.M = g.N = R.bp; g.K = n;
      g.C = dRg; g.ldc = R.bp; g.c_dt = F32;
      if (fs_bf16(*L, R)) {  // gathered rows as bf16 operands (row pitch padded to 8) on the fast kernel
        const int ldn = pad8(n);
        HIP_TRY(launch_gather_rows_to(p.G, F32, ldw, idxR, R.bp, m, n, p.Gr, BF16, ldn, st));
        if (!fs_pair) HIP_TRY(launch_gather_rows_to(p.T, F32, ldw, idxR, R.bp, m, n, p.Zr, BF16, ldn, st));
        g.A = p.Gr; g.lda = ldn; g.a_dt = BF16; g.a_kmajor = 1;
        g.B = p.Zr; g.ldb = ldn; g.b_dt = BF16; g.b_kmajor = 1;
      } else {
        HIP_TRY(launch_gather_rows(p.G, F32, ldw, idxR, R.bp, m, n, p.Gr, n, st));
        HIP_TRY(launch_gather_rows(p.T, F32, ldw, idxR, R.bp, m, n, p.Zr, n, st));
        g.A = p.Gr; g.lda = n; g.a_dt = F32; g.a_kmajor = 1;
        g.B = p.Zr; g.ldb = n; g.b_dt = F32; g.b_kmajor = 1;
      }
    }
    if (prims_only) HIP_TRY(contract_only(R, g, dRg, st));
    else HIP_TRY(contract_and_adjoint(R, g, dRg, powersR, dthetaR, p.adj, st));
  }
  // primitive blocks of dL/dP = (R W0)^T G
  if (P.theta_len > 0 || prims_only) {
    GemmDesc g;
    g.kclass = POET_K_CONTRACT;
    g.compute = act;
    g.part = p.adj.part; g.part_elems = p.adj.part_elems;
    if (P.mode == POET_BS) {
      g.M = g.N = P.bp; g.K = m; g.Mtot = g.Ntot = n; g.batch = P.nprim;
      if (fast) {
        g.A = p.RW0b; g.a_dt = BF16; g.B = p.Gb; g.b_dt = BF16;
      } else {
        g.A = p.RW0; g.a_dt = F32; g.B = p.G; g.b_dt = F32;
      }
      g.lda = ldw; g.sA = P.bp; g.a_kmajor = 0;
      g.ldb = ldw; g.sB = P.bp; g.b_kmajor = 0;
      g.C = dPg; g.ldc = P.bp; g.sC = (int64_t)P.bp * P.bp; g.c_dt = F32;
    } else {
      g.M = g.N = P.bp; g.K = m;
      g.C = dPg; g.ldc = P.bp; g.c_dt = F32;
      if (fs_bf16(*L, P)) {  // gathered columns as bf16 operands (row pitch ldp) on the fast kernel
        if (!fs_pair) HIP_TRY(launch_gather_cols_to(p.RW0, ldw, m, idxP, P.bp, n, p.Acp, BF16, P.ldp, st));
        HIP_TRY(launch_gather_cols_to(p.G, ldw, m, idxP, P.bp, n, p.Gc, BF16, P.ldp, st));
        g.A = p.Acp; g.lda = P.ldp; g.a_dt = BF16; g.a_kmajor = 0;
        g.B = p.Gc; g.ldb = P.ldp; g.b_dt = BF16; g.b_kmajor = 0;
      } else {
        HIP_TRY(launch_gather_cols(p.RW0, ldw, m, idxP, P.bp, n, p.Acp, P.bp, st));
        HIP_TRY(launch_gather_cols(p.G, ldw, m, idxP, P.bp, n, p.Gc, P.bp, st));
        g.A = p.Acp; g.lda = P.bp; g.a_dt = F32; g.a_kmajor = 0;
        g.B = p.Gc; g.ldb = P.bp; g.b_dt = F32; g.b_kmajor = 0;
      }
    }
    if (prims_only) HIP_TRY(contract_only(P, g, dPg, st));
    else HIP_TRY(contract_and_adjoint(P, g, dPg, powersP, dthetaP, p.adj, st));
  }
  return POET_OK;
}
}  // namespace

extern "C" {

poet_status poet_linear_bwd(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                            const void* powersR, const void* powersP, const int32_t* idxR, const int32_t* idxP,
                            const void* Win, const void* X, const void* dY, void* dX, float* dthetaR, float* dthetaP,
                            void* ws, size_t ws_bytes, void* stream) {
  return bwd_weight(L, W0, primR, primP, powersR, powersP, idxR, idxP, Win, X, dY, dX, dthetaR, dthetaP, nullptr,
                    nullptr, ws, ws_bytes, stream);
}

poet_status poet_linear_bwd_prims(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                                  const int32_t* idxR, const int32_t* idxP, const void* W, const void* X,
                                  const void* dY, void* dX, float* dprimR, float* dprimP, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!dprimR || !dprimP) return fail(POET_E_ARG, "null dprim");
  return bwd_weight(L, W0, primR, primP, nullptr, nullptr, idxR, idxP, W, X, dY, dX, nullptr, nullptr, dprimR, dprimP,
                    ws, ws_bytes, stream);
}

size_t poet_fs_form_workspace_bytes(const poet_layer* L) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return 0;
  Arena a(nullptr);
  FsBufs f;
  plan_fs(a, *L, R, P, &f);
  return a.used();
}

poet_status poet_fs_form(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                         const int32_t* idxR, const int32_t* idxP, void* W, void* Zr, void* Acp, void* ws,
                         size_t ws_bytes, void* stream) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  if (!(fs_bf16(*L, R) && fs_bf16(*L, P)))
    return fail(POET_E_UNSUPPORTED, "poet_fs_form needs both sides POET-FS with bf16 sides and activations");
  if (!W0 || !primR || !primP || !W || !Zr || !Acp) return fail(POET_E_ARG, "null W0, primitive or output");
  if (!check_idx(R, idxR, "R") || !check_idx(P, idxP, "P")) return g_last;
  if (!check_ws(ws, ws_bytes, poet_fs_form_workspace_bytes(L))) return g_last;
  Arena a(ws);
  FsBufs f;
  plan_fs(a, *L, R, P, &f);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(fs_weight_bf16(*L, R, P, W0, primR, primP, idxR, idxP, W, f, st));
  HIP_TRY(fs_grad_operands(*L, R, P, W0, primR, primP, idxR, idxP, reinterpret_cast<__bf16*>(Zr),
                           reinterpret_cast<__bf16*>(Acp), f, st));
  return POET_OK;
}

poet_status poet_linear_fwd_formed(const poet_layer* L, const void* W, const void* X, void* Y, void* stream) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  if (!W) return fail(POET_E_ARG, "null W");
  if (L->T > 0 && (!X || !Y)) return fail(POET_E_ARG, "null X or Y");
  if (L->T == 0) return POET_OK;
  GemmDesc g;  // Y = X W^T
  g.kclass = POET_K_TOKEN_FWD;
  g.compute = L->act_dtype; g.M = L->T; g.N = L->m; g.K = L->n;
  g.A = X; g.lda = L->ldx; g.a_dt = L->act_dtype; g.a_kmajor = 1;
  g.B = W; g.ldb = L->ldw; g.b_dt = L->act_dtype; g.b_kmajor = 1;
  g.C = Y; g.ldc = L->ldy; g.c_dt = L->act_dtype;
  HIP_TRY(launch_gemm(g, reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

poet_status poet_linear_bwd_formed_prims(const poet_layer* L, const void* W, const void* Zr, const void* Acp,
                                         const int32_t* idxR, const int32_t* idxP, const void* X, const void* dY,
                                         void* dX, float* dprimR, float* dprimP, void* ws, size_t ws_bytes,
                                         void* stream) {
  if (!dprimR || !dprimP) return fail(POET_E_ARG, "null dprim");
  if (!W || !Zr || !Acp) return fail(POET_E_ARG, "null W, Zr or Acp");
  return bwd_weight(L, nullptr, nullptr, nullptr, nullptr, nullptr, idxR, idxP, W, X, dY, dX, nullptr, nullptr, dprimR,
                    dprimP, ws, ws_bytes, stream, Zr, Acp);
}

int poet_act_path_supported(const poet_layer* L) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return 0;
  return act_path_ok(*L, R, P) ? 1 : 0;
}

poet_status poet_weight_shadow(const poet_layer* L, const float* W0, void* W0_shadow, void* stream) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  if (!W0 || !W0_shadow) return fail(POET_E_ARG, "null W0 or shadow");
  HIP_TRY(launch_convert(W0, L->ldw, W0_shadow, L->ldw, L->act_dtype, L->m, L->n,
                         reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

}  // extern "C"

namespace {
// the activation-side forward; W0P (nullable) is W0 P made beforehand (poet_fold_weights_group), else P is folded
// here or applied to the tokens
poet_status fwd_act(const poet_layer* L, const void* W0b, const void* W0P, const float* primR, const float* primP,
                    const void* opsR, const void* opsP, const void* X, void* Y, void* Z, void* ws, size_t ws_bytes,
                    void* stream) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  if (!act_path_ok(*L, R, P)) return fail(POET_E_UNSUPPORTED, "the activation-side path needs POET-BS sides and bf16 activations");
  if (!primR || (!W0P && (!W0b || !primP))) return fail(POET_E_ARG, "null W0 shadow or primitive");
  if (L->T > 0 && (!X || !Y || !Z)) return fail(POET_E_ARG, "null X, Y or Z");
  ActFwdPlan p;
  if (!check_ws(ws, ws_bytes, plan_fwd_act(*L, R, P, nullptr, &p))) return g_last;
  plan_fwd_act(*L, R, P, ws, &p);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (L->T == 0) return POET_OK;
  const int T = L->T;
  const bool fold = W0P || fold_P(*L, P);
  if (!W0P) {
    if (fold) HIP_TRY(fold_factor(*L, P, false, W0b, primP, opsP, p.Pb, p.W0P, st));  // W0P = W0 P
    else HIP_TRY(act_factor(P, T, X, L->ldx, primP, opsP, p.Pb, true, p.Xp, L->ldx, st));  // X' = X P^T
  }
  {  // Z = X (W0 P)^T = X' W0^T
    GemmDesc g;
    g.kclass = POET_K_TOKEN_FWD;
    g.compute = BF16; g.M = T; g.N = L->m; g.K = L->n;
    g.A = fold ? X : p.Xp; g.lda = L->ldx; g.a_dt = BF16; g.a_kmajor = 1;
    g.B = W0P ? W0P : fold ? p.W0P : W0b; g.ldb = L->ldw; g.b_dt = BF16; g.b_kmajor = 1;
    g.C = Z; g.ldc = L->ldy; g.c_dt = BF16;
    HIP_TRY(launch_gemm(g, st));
  }
  HIP_TRY(act_factor(R, T, Z, L->ldy, primR, opsR, p.Rb, true, Y, L->ldy, st));  // Y = Z R^T
  return POET_OK;
}
}  // namespace

extern "C" {

poet_status poet_linear_fwd_act(const poet_layer* L, const void* W0b, const float* primR, const float* primP,
                                const void* opsR, const void* opsP, const void* X, void* Y, void* Z, void* ws,
                                size_t ws_bytes, void* stream) {
  return fwd_act(L, W0b, nullptr, primR, primP, opsR, opsP, X, Y, Z, ws, ws_bytes, stream);
}

poet_status poet_linear_fwd_folded(const poet_layer* L, const void* W0P, const float* primR, const void* opsR,
                                   const void* X, void* Y, void* Z, void* ws, size_t ws_bytes, void* stream) {
  if (!W0P) return fail(POET_E_ARG, "null folded weight");
  return fwd_act(L, nullptr, W0P, primR, nullptr, opsR, nullptr, X, Y, Z, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {
// the activation-side backward; with dprimR/dprimP given it stops at the primitive gradients
poet_status bwd_act(const poet_layer* L, const void* W0b, const void* RW0, const float* primR, const float* primP,
                    const void* opsR, const void* opsP, const void* powersR,
                    const void* powersP, const void* X, const void* Z, const void* dY, void* dX, float* dthetaR,
                    float* dthetaP, float* dprimR, float* dprimP, void* ws, size_t ws_bytes, void* stream) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  if (!act_path_ok(*L, R, P)) return fail(POET_E_UNSUPPORTED, "the activation-side path needs POET-BS sides and bf16 activations");
  if (!primP || (!RW0 && (!W0b || !primR))) return fail(POET_E_ARG, "null W0 shadow or primitive");
  if (L->T > 0 && (!X || !Z || !dY)) return fail(POET_E_ARG, "null X, Z or dY");
  const bool prims_only = dprimR || dprimP;
  if (prims_only) {
    if (!dprimR || !dprimP) return fail(POET_E_ARG, "null dprim");
  } else {
    if ((R.theta_len > 0 && !dthetaR) || (P.theta_len > 0 && !dthetaP)) return fail(POET_E_ARG, "null dtheta");
    if ((R.k > 0 && R.theta_len > 0 && !powersR) || (P.k > 0 && P.theta_len > 0 && !powersP))
      return fail(POET_E_ARG, "saved powers are required when k >= 1");
  }
  ActBwdPlan p;
  if (!check_ws(ws, ws_bytes, plan_bwd_act(*L, R, P, nullptr, &p))) return g_last;
  plan_bwd_act(*L, R, P, ws, &p);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int T = L->T;
  if (T > 0) {
    const bool fold = RW0 || fold_R(*L, R);
    if (!RW0) {
      if (fold) HIP_TRY(fold_factor(*L, R, true, W0b, primR, opsR, p.Rb, p.RW0, st));  // RW0 = R W0
      else HIP_TRY(act_factor(R, T, dY, L->ldy, primR, opsR, p.Rb, false, p.dZ, L->ldy, st));  // dZ = dY R
    }
    {  // dX' = dY (R W0) = dZ W0
      GemmDesc g;
      g.kclass = POET_K_TOKEN_DX;
      g.compute = BF16; g.M = T; g.N = L->n; g.K = L->m;
      g.A = fold ? dY : p.dZ; g.lda = L->ldy; g.a_dt = BF16; g.a_kmajor = 1;
      g.B = RW0 ? RW0 : fold ? p.RW0 : W0b; g.ldb = L->ldw; g.b_dt = BF16; g.b_kmajor = 0;
      g.C = p.dXp; g.ldc = L->ldx; g.c_dt = BF16;
      HIP_TRY(launch_gemm(g, st));
    }
    if (dX) HIP_TRY(act_factor(P, T, p.dXp, L->ldx, primP, opsP, p.Pb, false, dX, L->ldx, st));  // dX = dX' P
  }
  // primitive blocks of dL/dR = dY^T Z and dL/dP = dX'^T X (zero when T == 0), then the adjoint; the two
  // contractions share one launch when their shapes allow
  float* dR = prims_only ? dprimR : p.dRg;
  float* dP = prims_only ? dprimP : p.dPg;
  if (super_group(R) == 1 && super_group(P) == 1 && R.theta_len > 0 && P.theta_len > 0) {
    const GemmDesc gR = act_contract(R, T, dY, L->ldy, Z, L->ldy, dR, p.adj);
    const GemmDesc gP = act_contract(P, T, p.dXp, L->ldx, X, L->ldx, dP, p.adj);
    if (fast_gemm_pair_eligible(gR, gP)) {
      HIP_TRY(clear_ragged(R, dR, st));
      HIP_TRY(clear_ragged(P, dP, st));
      HIP_TRY(launch_fast_gemm_pair(gR, gP, st));
      if (prims_only) return POET_OK;
      HIP_TRY(neumann_adjoint(R, dR, powersR, dthetaR, p.adj, st));
      HIP_TRY(neumann_adjoint(P, dP, powersP, dthetaP, p.adj, st));
      return POET_OK;
    }
  }
  if (prims_only) {
    HIP_TRY(act_contract_adjoint(R, T, dY, L->ldy, Z, L->ldy, dprimR, nullptr, nullptr, p, st));
    HIP_TRY(act_contract_adjoint(P, T, p.dXp, L->ldx, X, L->ldx, dprimP, nullptr, nullptr, p, st));
    return POET_OK;
  }
  if (R.theta_len > 0) HIP_TRY(act_contract_adjoint(R, T, dY, L->ldy, Z, L->ldy, p.dRg, powersR, dthetaR, p, st));
  if (P.theta_len > 0) HIP_TRY(act_contract_adjoint(P, T, p.dXp, L->ldx, X, L->ldx, p.dPg, powersP, dthetaP, p, st));
  return POET_OK;
}
}  // namespace

// the in-place block-diagonal merge of one weight, as an item of launch_bs_merge_group
MergeItem merge_item(const poet_layer& L, const SideInfo& R, const SideInfo& P, float* W0, void* shadow,
                     const float* primR, const float* primP) {
  MergeItem it;
  it.W = W0; it.ld = L.ldw; it.m = L.m; it.n = L.n;
  it.bpR = R.bp; it.nR = R.nprim; it.primR = primR;
  it.bpP = P.bp; it.nP = P.nprim; it.primP = primP;
  it.shadow = shadow; it.sh_dt = L.act_dtype; it.ld_sh = L.ldw;
  return it;
}

// In-place FS merge of one side to float32 accuracy on bf16 MFMA. With X the gathered float32 block of W0 (P: the
// columns I, m x s; R: the rows I, s x n) and dF = F - I the factor's delta, the block becomes X + X dF (P) or
// X + dF X (R): the identity part is the float32 addend, and the delta product is hi*hi + hi*lo + lo*hi of the
// two operands' bf16 parts, one product with K = 3 s' (s' = s rounded up to 8, zero padded), the parts stacked
// along K as [hi | hi | lo] on the left operand and [hi ; lo ; hi] on the right. The result is scattered back.
hipError_t fs3_merge_side(const poet_layer& L, const SideInfo& S, bool rside, float* W0, const float* prim,
                          const int32_t* idx, const Fs3Bufs& f, hipStream_t st) {
  const int m = L.m, n = L.n, s = S.bp, sp = pad8(S.bp);
  GemmDesc g;
  g.compute = BF16;
  g.kclass = POET_K_MERGE;
  g.part = f.part; g.part_elems = f.part_elems;
  g.a_dt = g.b_dt = BF16;
  g.K = 3 * sp;
  g.beta = 1.f;
  g.c_dt = F32;
  if (!rside) {  // columns I: Xcat m x 3s' (K-major left operand), Fcat 3s' x s' (rows of the right operand)
    HIP_RET(launch_split3(W0, L.ldw, nullptr, idx, m, n, 0, m, s, m, sp, f.Xcat, 3 * sp, sp, 0b100, f.Dg, s, st));
    HIP_RET(launch_split3(prim, s, nullptr, nullptr, s, s, 1, s, s, sp, sp, f.Fcat, sp, (int64_t)sp * sp, 0b010,
                          nullptr, 0, st));
    g.M = m; g.N = s;
    g.A = f.Xcat; g.lda = 3 * sp; g.a_kmajor = 1;
    g.B = f.Fcat; g.ldb = sp; g.b_kmajor = 0;
    g.D = f.Dg; g.ldd = s;
    g.C = f.C; g.ldc = s;
    HIP_RET(launch_gemm(g, st));
    return launch_scatter_cols(f.C, s, m, idx, s, n, W0, L.ldw, st);
  }
  // rows I: Fcat s x 3s' (K-major left operand), Xcat 3s' x n' (rows of the right operand, n' = n rounded up to 8)
  const int np = pad8(n);
  HIP_RET(launch_split3(W0, L.ldw, idx, nullptr, m, n, 0, s, n, sp, np, f.Xcat, np, (int64_t)sp * np, 0b010, f.Dg, n,
                        st));
  HIP_RET(launch_split3(prim, s, nullptr, nullptr, s, s, 1, s, s, s, sp, f.Fcat, 3 * sp, sp, 0b100, nullptr, 0, st));
  g.M = s; g.N = n;
  g.A = f.Fcat; g.lda = 3 * sp; g.a_kmajor = 1;
  g.B = f.Xcat; g.ldb = np; g.b_kmajor = 0;
  g.D = f.Dg; g.ldd = n;
  g.C = f.C; g.ldc = n;
  HIP_RET(launch_gemm(g, st));
  return launch_scatter_rows(f.C, n, idx, s, m, n, W0, F32, L.ldw, st);
}

// W0 <- R W0 P of a weight outside the in-place path (FS sides, blocks above 256), through its MergePlan buffers
hipError_t merge_general(const poet_layer& L, const SideInfo& R, const SideInfo& P, float* W0, void* W0_shadow,
                         const float* primR, const float* primP, const int32_t* idxR, const int32_t* idxP,
                         const MergePlan& p, hipStream_t st) {
  if (p.fs3) {  // W0 <- W0 P on the columns I_P, then W0 <- R W0 on the rows I_R, in place; then the shadow
    HIP_RET(fs3_merge_side(L, P, false, W0, primP, idxP, p.f3, st));
    HIP_RET(fs3_merge_side(L, R, true, W0, primR, idxR, p.f3, st));
    if (W0_shadow) HIP_RET(launch_convert(W0, L.ldw, W0_shadow, L.ldw, L.act_dtype, L.m, L.n, st));
    return hipSuccess;
  }
  HIP_RET(apply_P(L, P, W0, primP, idxP, p.T, F32, p.fs, st));
  HIP_RET(apply_R(L, R, p.T, primR, idxR, p.Wn, F32, L.ldw, F32, p.fs, st));
  HIP_RET(launch_convert(p.Wn, L.ldw, W0, L.ldw, F32, L.m, L.n, st));
  if (W0_shadow) HIP_RET(launch_convert(p.Wn, L.ldw, W0_shadow, L.ldw, L.act_dtype, L.m, L.n, st));
  return hipSuccess;
}

// fresh index sets of a weight's FS sides for epoch epoch_next
hipError_t merge_resample(const SideInfo& R, const SideInfo& P, int32_t* idxR, int32_t* idxP, int32_t* flags,
                          uint64_t seed, uint32_t linear_id, uint32_t epoch_next, hipStream_t st) {
  if (R.mode == POET_FS)
    HIP_RET(launch_sample(R.d, R.bp, sampler_hash(seed, linear_id, POET_SIDE_R, epoch_next), flags, idxR, st));
  if (P.mode == POET_FS)
    HIP_RET(launch_sample(P.d, P.bp, sampler_hash(seed, linear_id, POET_SIDE_P, epoch_next), flags, idxP, st));
  return hipSuccess;
}

// Workspace of a grouped merge: the pre-split deltas of every in-place weight at once, or the largest single-weight
// plan of the others (which run one after another, after the in-place ones), whichever is larger.
size_t merge_group_bytes(int32_t count, const poet_layer* layers) {
  std::vector<MergeItem> items;
  size_t solo = 0;
  for (int i = 0; i < count; ++i) {
    SideInfo R, P;
    if (!layer_info(&layers[i], &R, &P)) return 0;
    MergePlan p;
    const size_t one = plan_merge(layers[i], R, P, nullptr, &p);
    if (p.inplace) items.push_back(merge_item(layers[i], R, P, nullptr, nullptr, nullptr, nullptr));
    else solo = std::max(solo, one);
  }
  return std::max(solo, items.empty() ? (size_t)0 : bs_merge_group_bytes(items.data(), (int)items.size()) + 256);
}

extern "C" {

poet_status poet_linear_bwd_act(const poet_layer* L, const void* W0b, const float* primR, const float* primP,
                                const void* opsR, const void* opsP, const void* powersR, const void* powersP,
                                const void* X, const void* Z, const void* dY, void* dX, float* dthetaR,
                                float* dthetaP, void* ws, size_t ws_bytes, void* stream) {
  return bwd_act(L, W0b, nullptr, primR, primP, opsR, opsP, powersR, powersP, X, Z, dY, dX, dthetaR, dthetaP, nullptr,
                 nullptr, ws, ws_bytes, stream);
}

poet_status poet_linear_bwd_act_prims(const poet_layer* L, const void* W0b, const float* primR, const float* primP,
                                      const void* opsR, const void* opsP, const void* X, const void* Z,
                                      const void* dY, void* dX, float* dprimR, float* dprimP, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (!dprimR || !dprimP) return fail(POET_E_ARG, "null dprim");
  return bwd_act(L, W0b, nullptr, primR, primP, opsR, opsP, nullptr, nullptr, X, Z, dY, dX, nullptr, nullptr, dprimR,
                 dprimP, ws, ws_bytes, stream);
}

poet_status poet_linear_bwd_folded_prims(const poet_layer* L, const void* RW0, const float* primP, const void* opsP,
                                         const void* X, const void* Z, const void* dY, void* dX, float* dprimR,
                                         float* dprimP, void* ws, size_t ws_bytes, void* stream) {
  if (!RW0) return fail(POET_E_ARG, "null folded weight");
  if (!dprimR || !dprimP) return fail(POET_E_ARG, "null dprim");
  return bwd_act(L, nullptr, RW0, nullptr, primP, nullptr, opsP, nullptr, nullptr, X, Z, dY, dX, nullptr, nullptr,
                 dprimR, dprimP, ws, ws_bytes, stream);
}

// Workspace of a grouped fold: bf16 row-order copies of every primitive (used where no operand copies are given).
size_t poet_fold_group_workspace_bytes(int32_t count, const poet_layer* layers) {
  if (count <= 0 || !layers) return 0;
  Arena a(nullptr);
  for (int i = 0; i < count; ++i) {
    SideInfo R, P;
    if (!layer_info(&layers[i], &R, &P)) return 0;
    a.take<__bf16>(R.prim_len);
    a.take<__bf16>(P.prim_len);
  }
  return a.used();
}

poet_status poet_fold_weights_group(int32_t count, const poet_layer* layers, const void* const* W0b,
                                    const float* const* primR, const float* const* primP, const void* const* opsR,
                                    const void* const* opsP, void* const* W0P, void* const* RW0, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (count < 0) return fail(POET_E_ARG, "count = %d must be >= 0", count);
  if (count == 0) return POET_OK;
  if (!layers || !W0b) return fail(POET_E_ARG, "null layers or W0 shadow table");
  if (!W0P && !RW0) return POET_OK;
  std::vector<SideInfo> R(count), P(count);
  for (int i = 0; i < count; ++i) {
    if (!layer_info(&layers[i], &R[i], &P[i])) return g_last;
    if (!act_path_ok(layers[i], R[i], P[i]))
      return fail(POET_E_UNSUPPORTED, "layers[%d]: folding needs POET-BS sides and bf16 activations", i);
    if (!W0b[i]) return fail(POET_E_ARG, "null W0b[%d]", i);
    if (W0P && W0P[i] && !(primP && primP[i])) return fail(POET_E_ARG, "null primP[%d]", i);
    if (RW0 && RW0[i] && !(primR && primR[i])) return fail(POET_E_ARG, "null primR[%d]", i);
  }
  if (!check_ws(ws, ws_bytes, poet_fold_group_workspace_bytes(count, layers))) return g_last;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Arena a(ws);
  std::vector<GemmDesc> gP, gR;
  for (int i = 0; i < count; ++i) {
    const poet_layer& L = layers[i];
    __bf16* fR = a.take<__bf16>(R[i].prim_len);
    __bf16* fP = a.take<__bf16>(P[i].prim_len);
    if (W0P && W0P[i]) {  // row-order deltas of P: the third part of the operand copies, or converted here
      const __bf16* Fb = opsP && opsP[i] ? reinterpret_cast<const __bf16*>(opsP[i]) + 2 * P[i].prim_len : fP;
      if (Fb == fP) HIP_TRY(deltas_bf16(P[i], primP[i], fP, st));
      gP.push_back(fold_desc(L, P[i], false, W0b[i], Fb, reinterpret_cast<__bf16*>(W0P[i])));
    }
    if (RW0 && RW0[i]) {
      const __bf16* Fb = opsR && opsR[i] ? reinterpret_cast<const __bf16*>(opsR[i]) + 2 * R[i].prim_len : fR;
      if (Fb == fR) HIP_TRY(deltas_bf16(R[i], primR[i], fR, st));
      gR.push_back(fold_desc(L, R[i], true, W0b[i], Fb, reinterpret_cast<__bf16*>(RW0[i])));
    }
  }
  HIP_TRY(launch_grouped(gP, st));
  HIP_TRY(launch_grouped(gR, st));
  return POET_OK;
}

size_t poet_build_group_workspace_bytes(int32_t count, const poet_side* sides) {
  std::vector<SideInfo> S;
  if (!group_sides(count, sides, &S)) return 0;
  size_t need = 0;
  for (int i = 0; i < count; ++i) need = std::max(need, poet_build_workspace_bytes(&sides[i], 1));
  for (const auto& c : build_chunks(S, nullptr)) {
    size_t sq = 0;
    for (int i : c.idx) sq += sq_bytes(S[i]);
    need = std::max(need, build_chunk_part_elems(c) * sizeof(float) + sq + 512);
  }
  return need;
}

poet_status poet_build_orthogonal_group(int32_t count, const poet_side* sides, const float* const* theta,
                                        float* const* prim, void* const* powers, void* const* ops, int32_t flags,
                                        void* ws, size_t ws_bytes, void* stream) {
  std::vector<SideInfo> S;
  if (!group_sides(count, sides, &S)) return g_last;
  if (flags != POET_BUILD_STEP && flags != POET_BUILD_MERGE) return fail(POET_E_ARG, "bad build flags %d", flags);
  if (count == 0) return POET_OK;
  if (!theta || !prim || !powers) return fail(POET_E_ARG, "null pointer table");
  for (int i = 0; i < count; ++i) {
    if (!prim[i]) return fail(POET_E_ARG, "null prim[%d]", i);
    if (!theta[i] && S[i].theta_len > 0) return fail(POET_E_ARG, "null theta[%d]", i);
    if (!powers[i] && S[i].k > 0) return fail(POET_E_ARG, "null powers[%d] (required when k >= 1)", i);
    if (ops && ops[i] && S[i].mode != POET_BS) return fail(POET_E_ARG, "ops[%d] given for an FS side", i);
  }
  if (!check_ws(ws, ws_bytes, poet_build_group_workspace_bytes(count, sides))) return g_last;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // sides on the fused chain, k = 0 sides (which need only I + Q) and sides whose chain runs as grouped GEMMs share
  // the theta launches; the rest build one by one
  const std::vector<BuildChunk> chunks = build_chunks(S, powers);
  std::vector<char> in_chunk(count, 0);
  for (const auto& c : chunks)
    for (int i : c.idx) in_chunk[i] = 1;
  std::vector<int> grouped;
  auto side_ops = [&](int i) -> __bf16* { return ops ? reinterpret_cast<__bf16*>(ops[i]) : nullptr; };
  for (int i = 0; i < count; ++i) {
    if (S[i].k == 0 || chain_side(S[i], powers[i]) || in_chunk[i]) grouped.push_back(i);
    else if (poet_build_orthogonal(&sides[i], theta[i], prim[i], powers[i], nullptr, flags, ws, ws_bytes, stream) !=
             POET_OK)
      return g_last;
  }
  for (size_t c0 = 0; c0 < grouped.size(); c0 += MAXG) {
    const size_t c1 = std::min(grouped.size(), c0 + MAXG);
    PrepGroup pg;
    ChainGroup cg;
    for (size_t u = c0; u < c1; ++u) {
      const int i = grouped[u];
      const SideInfo& T = S[i];
      PrepSide& a = pg.s[pg.n++];
      a.theta = theta[i]; a.prim = prim[i]; a.q = T.k > 0 ? powers[i] : nullptr; a.q_dt = T.dtype; a.ldq = T.ldp;
      a.mode = T.mode; a.d = T.d; a.bp = T.bp; a.nprim = T.nprim; a.coef = T.k == 0 ? 1.f : 2.f;
      if (T.k == 0 || in_chunk[i]) continue;
      ChainArgs& c = cg.a[cg.n++];
      c.bp = T.bp; c.nprim = T.nprim; c.steps = T.k; c.build = 1; c.prim = prim[i];
      c.A = reinterpret_cast<const __bf16*>(powers[i]); c.sA = (int64_t)T.bp * T.bp;
      c.Y = reinterpret_cast<__bf16*>(powers[i]); c.ldy = T.bp; c.sy = (int64_t)T.bp * T.bp; c.jstep = (int64_t)T.plen;
      c.ops = side_ops(i); c.d = T.d; c.mode = T.mode;
    }
    HIP_TRY(launch_theta_prep_group(pg, st));
    HIP_TRY(launch_power_chain_group(cg, POET_K_CHAIN, st));
  }
  // GEMM chains: P_{i+1} = Q P_i for every side of a chunk in one launch per step (the last power straight into
  // prim in float32), then the rest of the series for all of them
  for (const auto& c : chunks) {
    Arena a(ws);
    const size_t part_elems = build_chunk_part_elems(c);
    float* part = a.take<float>(part_elems);
    const int n = (int)c.idx.size();
    // for a merge: (2Q)^2 of every side to float32 accuracy (prim holds I + 2Q after the theta launch), one grouped
    // product
    const bool accurate_sq = flags == POET_BUILD_MERGE;
    std::vector<SqBufs> sq(n);
    if (accurate_sq) {
      GemmDesc pr[MAXG];
      for (int u = 0; u < n; ++u) {
        plan_sq(a, S[c.idx[u]], &sq[u]);
        HIP_TRY(sq_split(S[c.idx[u]], prim[c.idx[u]], sq[u], st));
        pr[u] = sq_gemm(S[c.idx[u]], sq[u], part, part_elems);
      }
      if (fast_gemm_group_eligible(pr, n)) {
        HIP_TRY(launch_fast_gemm_group(pr, n, st));
      } else {
        for (int u = 0; u < n; ++u) HIP_TRY(launch_gemm(pr[u], st));
      }
    }
    for (int step = 1; step <= c.k && !(accurate_sq && c.k == 1); ++step) {  // k == 1: ends at the accurate Q^2
      GemmDesc pr[MAXG];
      for (int u = 0; u < n; ++u) {
        const int i = c.idx[u];
        const SideInfo& T = S[i];
        const size_t esz = dtype_size(T.dtype);
        char* pw = reinterpret_cast<char*>(powers[i]);
        const int64_t ps = (int64_t)T.bp * T.ldp;
        GemmDesc& g = pr[u];
        g.kclass = POET_K_CHAIN;
        g.compute = BF16; g.M = g.N = g.K = T.bp; g.batch = T.nprim;
        g.A = pw; g.lda = T.ldp; g.sA = ps; g.a_dt = BF16; g.a_kmajor = 1;
        g.B = pw + (size_t)(step - 1) * T.plen * esz; g.ldb = T.ldp; g.sB = ps; g.b_dt = BF16; g.b_kmajor = 0;
        if (step < c.k) { g.C = pw + (size_t)step * T.plen * esz; g.c_dt = BF16; g.ldc = T.ldp; g.sC = ps; }
        else { g.C = prim[i]; g.c_dt = F32; g.ldc = T.bp; g.sC = (int64_t)T.bp * T.bp; }
        g.part = part; g.part_elems = part_elems;
        // Q^(step+1) of a skew-symmetric Q is symmetric (even power) or skew-symmetric (odd): the tiles on and
        // above the diagonal, each off-diagonal one also written transposed below it
        g.tri = (step + 1) % 2 == 0 ? 1 : -1;
      }
      if (fast_gemm_group_eligible(pr, n)) {
        HIP_TRY(launch_fast_gemm_group(pr, n, st));
      } else {
        for (int u = 0; u < n; ++u) HIP_TRY(launch_gemm(pr[u], st));
      }
    }
    FinGroup fg;
    for (int u = 0; u < n; ++u) {
      const int i = c.idx[u];
      FinSide& f = fg.s[fg.n++];
      f.q2 = sq[u].q2;
      f.theta = theta[i]; f.powers = powers[i]; f.prim = prim[i]; f.mode = S[i].mode; f.d = S[i].d; f.bp = S[i].bp;
      f.nprim = S[i].nprim; f.k = S[i].k; f.dt = S[i].dtype; f.ldp = S[i].ldp;
    }
    HIP_TRY(launch_chain_finalize_group(fg, st));
  }
  // the operand copies of sides the chain did not finish (k = 0, or built one by one)
  for (int i = 0; i < count; ++i) {
    __bf16* o = side_ops(i);
    if (!o || chain_side(S[i], powers[i])) continue;
    HIP_TRY(launch_act_operand(prim[i], S[i].bp, S[i].d, S[i].nprim, true, o, st));
    HIP_TRY(launch_act_operand(prim[i], S[i].bp, S[i].d, S[i].nprim, false, o + S[i].prim_len, st));
    HIP_TRY(deltas_bf16(S[i], prim[i], o + 2 * S[i].prim_len, st));
  }
  return POET_OK;
}

poet_status poet_adamw_group(int32_t count, const poet_side* sides, float* const* theta, const float* const* dtheta,
                             float* const* m, float* const* v, const poet_adamw* hp, int32_t step, void* stream) {
  std::vector<SideInfo> S;
  if (!group_sides(count, sides, &S)) return g_last;
  if (!hp) return fail(POET_E_ARG, "null hyperparameters");
  const auto finite = [](float x) { return x == x && x - x == 0.f; };
  if (!finite(hp->lr) || hp->lr < 0.f) return fail(POET_E_ARG, "lr = %g must be finite and >= 0", hp->lr);
  if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f) || !(hp->beta2 >= 0.f && hp->beta2 < 1.f))
    return fail(POET_E_ARG, "betas (%g, %g) must be in [0, 1)", hp->beta1, hp->beta2);
  if (!finite(hp->eps) || !(hp->eps > 0.f)) return fail(POET_E_ARG, "eps = %g must be finite and > 0", hp->eps);
  if (!finite(hp->weight_decay) || hp->weight_decay < 0.f)
    return fail(POET_E_ARG, "weight_decay = %g must be finite and >= 0", hp->weight_decay);
  if (step < 1) return fail(POET_E_ARG, "step = %d must be >= 1 (steps since the last reset)", step);
  if (count == 0) return POET_OK;
  if (!theta || !dtheta || !m || !v) return fail(POET_E_ARG, "null pointer table");
  for (int i = 0; i < count; ++i)
    if (S[i].theta_len > 0 && (!theta[i] || !dtheta[i] || !m[i] || !v[i]))
      return fail(POET_E_ARG, "null theta, dtheta, m or v for side %d", i);
  // the bias corrections 1 / (1 - beta^t) in double
  const double inv_bc1 = 1.0 / (1.0 - std::pow((double)hp->beta1, (double)step));
  const double inv_bc2 = 1.0 / (1.0 - std::pow((double)hp->beta2, (double)step));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  OptGroup g;
  for (int i = 0; i <= count; ++i) {
    if (g.n == MAXG || (i == count && g.n > 0)) {
      HIP_TRY(launch_adamw_group(g, hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, inv_bc1, inv_bc2, st));
      g.n = 0;
    }
    if (i == count || S[i].theta_len == 0) continue;
    OptSide& o = g.s[g.n++];
    o.theta = theta[i]; o.grad = dtheta[i]; o.m = m[i]; o.v = v[i]; o.n = (int64_t)S[i].theta_len;
  }
  return POET_OK;
}

poet_status poet_optimizer_reset_group(int32_t count, const poet_side* sides, float* const* m, float* const* v,
                                       void* stream) {
  std::vector<SideInfo> S;
  if (!group_sides(count, sides, &S)) return g_last;
  if (count == 0) return POET_OK;
  if (!m || !v) return fail(POET_E_ARG, "null pointer table");
  for (int i = 0; i < count; ++i)
    if (S[i].theta_len > 0 && (!m[i] || !v[i])) return fail(POET_E_ARG, "null m or v for side %d", i);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  OptGroup g;
  for (int i = 0; i <= count; ++i) {
    if (g.n == MAXG || (i == count && g.n > 0)) {
      HIP_TRY(launch_moments_reset_group(g, st));
      g.n = 0;
    }
    if (i == count || S[i].theta_len == 0) continue;
    OptSide& o = g.s[g.n++];
    o.m = m[i]; o.v = v[i]; o.n = (int64_t)S[i].theta_len;
  }
  return POET_OK;
}

size_t poet_spectral_workspace_bytes(int32_t m, int32_t n) {
  if (m < 1 || n < 1) return fail(POET_E_SHAPE, "m = %d and n = %d must be >= 1", m, n), 0;
  const size_t r = (size_t)std::min(m, n);
  const size_t he = align_up((size_t)m * m * 8, 256) + align_up((size_t)m * 8, 256);
  const size_t sv = align_up(r * r * 8, 256) + 5 * align_up(r * 8, 256);
  return std::max(he, sv) + 256;
}

poet_status poet_hyperspherical_energy(int32_t m, int32_t n, const float* W, int64_t ldw, float s,
                                       double* energy_rows, double* energy, void* ws, size_t ws_bytes,
                                       void* stream) {
  if (m < 1 || n < 1 || ldw < n) return fail(POET_E_SHAPE, "need m, n >= 1 and ldw >= n (m=%d n=%d ldw=%lld)", m, n,
                                             (long long)ldw);
  if (!(s > 0.f) || !(s < 1e30f)) return fail(POET_E_ARG, "s = %g must be finite and > 0", s);
  if (!W || !energy) return fail(POET_E_ARG, "null W or energy");
  if ((int64_t)m * m > ((int64_t)1 << 40)) return fail(POET_E_UNSUPPORTED, "m = %d too large", m);
  if (!check_ws(ws, ws_bytes, poet_spectral_workspace_bytes(m, n))) return g_last;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Arena a(ws);
  double* C = a.take<double>((size_t)m * m);
  double* E = a.take<double>((size_t)m);
  HIP_TRY(launch_gram_f64(W, ldw, m, n, false, C, m, st));
  HIP_TRY(launch_he_rows(C, m, m, (double)s, energy_rows ? energy_rows : E, energy, st));
  return POET_OK;
}

poet_status poet_singular_value_entropy(int32_t m, int32_t n, const float* W, int64_t ldw, double* sigma,
                                        double* entropy, void* ws, size_t ws_bytes, void* stream) {
  if (m < 1 || n < 1 || ldw < n) return fail(POET_E_SHAPE, "need m, n >= 1 and ldw >= n (m=%d n=%d ldw=%lld)", m, n,
                                             (long long)ldw);
  if (!W || !entropy) return fail(POET_E_ARG, "null W or entropy");
  if (!check_ws(ws, ws_bytes, poet_spectral_workspace_bytes(m, n))) return g_last;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int r = std::min(m, n);
  Arena a(ws);
  double* C = a.take<double>((size_t)r * r);
  double* u = a.take<double>(r);
  double* p = a.take<double>(r);
  double* d = a.take<double>(r);
  double* e = a.take<double>(r);
  double* lam = a.take<double>(r);
  // the smaller Gram: W^T W (n x n) for a tall W, W W^T (m x m) otherwise
  HIP_TRY(launch_gram_f64(W, ldw, m, n, n <= m, C, r, st));
  HIP_TRY(launch_sym_eig_entropy(C, r, r, u, p, d, e, lam, sigma, entropy, st));
  return POET_OK;
}

size_t poet_adjoint_group_workspace_bytes(int32_t count, const poet_side* sides) {
  std::vector<SideInfo> S;
  if (!group_sides(count, sides, &S)) return 0;
  return adjoint_group_bytes(S, nullptr);
}

poet_status poet_adjoint_group(int32_t count, const poet_side* sides, const float* const* dprim,
                               const void* const* powers, float* const* dtheta, void* ws, size_t ws_bytes,
                               void* stream) {
  std::vector<SideInfo> S;
  if (!group_sides(count, sides, &S)) return g_last;
  if (count == 0) return POET_OK;
  if (!dprim || !powers || !dtheta) return fail(POET_E_ARG, "null pointer table");
  for (int i = 0; i < count; ++i) {
    if (S[i].theta_len == 0) continue;
    if (!dprim[i] || !dtheta[i]) return fail(POET_E_ARG, "null dprim[%d] or dtheta[%d]", i, i);
    if (!powers[i] && S[i].k > 0) return fail(POET_E_ARG, "null powers[%d] (required when k >= 1)", i);
  }
  if (!check_ws(ws, ws_bytes, adjoint_group_bytes(S, nullptr))) return g_last;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  std::vector<int> solo;
  const auto chunks = adjoint_chunks(S, powers, &solo);
  for (const auto& c : chunks) {
    AdjChunkBufs b;
    plan_adj_chunk(c, ws, &b);
    HIP_TRY(adjoint_chunk(c, S, dprim, powers, dtheta, b, st));
  }
  for (int i : solo) {
    AdjBufs b;
    plan_adj_solo(S[i], ws, &b);
    HIP_TRY(neumann_adjoint(S[i], dprim[i], powers[i], dtheta[i], b, st));
  }
  return POET_OK;
}

poet_status poet_merge(const poet_layer* L, float* W0, void* W0_shadow, float* thetaR, float* thetaP,
                       const float* primR, const float* primP, int32_t* idxR, int32_t* idxP, uint64_t seed,
                       uint32_t linear_id, uint32_t epoch_next, void* ws, size_t ws_bytes, void* stream) {
  SideInfo R, P;
  if (!layer_info(L, &R, &P)) return g_last;
  if (!W0 || !primR || !primP) return fail(POET_E_ARG, "null W0 or primitive");
  if ((R.theta_len > 0 && !thetaR) || (P.theta_len > 0 && !thetaP)) return fail(POET_E_ARG, "null theta");
  if (!check_idx(R, idxR, "R") || !check_idx(P, idxP, "P")) return g_last;
  MergePlan p;
  const size_t need = plan_merge(*L, R, P, nullptr, &p);
  if (!check_ws(ws, ws_bytes, need)) return g_last;
  plan_merge(*L, R, P, ws, &p);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.inplace) {  // W0 <- W0 P, then W0 <- R W0 (writing the shadow), in place
    const MergeItem it = merge_item(*L, R, P, W0, W0_shadow, primR, primP);
    HIP_TRY(launch_bs_merge_group(&it, 1, p.split, st));
  } else {
    HIP_TRY(merge_general(*L, R, P, W0, W0_shadow, primR, primP, idxR, idxP, p, st));
  }
  if (R.theta_len > 0) HIP_TRY(launch_fill(thetaR, R.theta_len, 0.f, st));
  if (P.theta_len > 0) HIP_TRY(launch_fill(thetaP, P.theta_len, 0.f, st));
  HIP_TRY(merge_resample(R, P, idxR, idxP, p.flags, seed, linear_id, epoch_next, st));
  return POET_OK;
}

size_t poet_merge_group_workspace_bytes(int32_t count, const poet_layer* layers) {
  if (count <= 0 || !layers) return 0;
  return merge_group_bytes(count, layers);
}

poet_status poet_merge_group(int32_t count, const poet_layer* layers, float* const* W0, void* const* W0_shadow,
                             float* const* thetaR, float* const* thetaP, const float* const* primR,
                             const float* const* primP, int32_t* const* idxR, int32_t* const* idxP, uint64_t seed,
                             const uint32_t* linear_id, uint32_t epoch_next, void* ws, size_t ws_bytes,
                             void* stream) {
  if (count < 0) return fail(POET_E_ARG, "count = %d must be >= 0", count);
  if (count == 0) return POET_OK;
  if (!layers || !W0 || !thetaR || !thetaP || !primR || !primP || !linear_id)
    return fail(POET_E_ARG, "null layers, W0, theta, primitive or linear_id table");
  std::vector<SideInfo> R(count), P(count);
  std::vector<std::pair<uintptr_t, uintptr_t>> spans;  // byte ranges of every W0 and shadow
  for (int i = 0; i < count; ++i) {
    const poet_layer& L = layers[i];
    if (!layer_info(&L, &R[i], &P[i])) return g_last;
    if (!W0[i] || !primR[i] || !primP[i]) return fail(POET_E_ARG, "null W0[%d] or primitive", i);
    if ((R[i].theta_len > 0 && !thetaR[i]) || (P[i].theta_len > 0 && !thetaP[i]))
      return fail(POET_E_ARG, "null thetaR[%d] or thetaP[%d]", i, i);
    if (!check_idx(R[i], idxR ? idxR[i] : nullptr, "R") || !check_idx(P[i], idxP ? idxP[i] : nullptr, "P"))
      return g_last;
    const uintptr_t w = reinterpret_cast<uintptr_t>(W0[i]);
    spans.push_back({w, w + ((size_t)(L.m - 1) * L.ldw + L.n) * 4});
    if (W0_shadow && W0_shadow[i]) {
      const uintptr_t h = reinterpret_cast<uintptr_t>(W0_shadow[i]);
      spans.push_back({h, h + ((size_t)(L.m - 1) * L.ldw + L.n) * dtype_size(L.act_dtype)});
    }
  }
  std::sort(spans.begin(), spans.end());
  for (size_t u = 1; u < spans.size(); ++u)
    if (spans[u].first < spans[u - 1].second) return fail(POET_E_ARG, "the weights or shadows of the group overlap");
  if (!check_ws(ws, ws_bytes, merge_group_bytes(count, layers))) return g_last;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  std::vector<MergeItem> items;
  std::vector<int> general;
  for (int i = 0; i < count; ++i) {
    MergePlan p;
    plan_merge(layers[i], R[i], P[i], nullptr, &p);
    if (p.inplace)
      items.push_back(merge_item(layers[i], R[i], P[i], W0[i], W0_shadow ? W0_shadow[i] : nullptr, primR[i], primP[i]));
    else
      general.push_back(i);
  }
  if (!items.empty()) {
    Arena a(ws);
    char* split = reinterpret_cast<char*>(a.take_bytes(bs_merge_group_bytes(items.data(), (int)items.size())));
    HIP_TRY(launch_bs_merge_group(items.data(), (int)items.size(), split, st));
  }
  for (int i : general) {  // one at a time, each through the whole workspace
    MergePlan p;
    plan_merge(layers[i], R[i], P[i], ws, &p);
    HIP_TRY(merge_general(layers[i], R[i], P[i], W0[i], W0_shadow ? W0_shadow[i] : nullptr, primR[i], primP[i],
                          idxR ? idxR[i] : nullptr, idxP ? idxP[i] : nullptr, p, st));
    HIP_TRY(merge_resample(R[i], P[i], idxR ? idxR[i] : nullptr, idxP ? idxP[i] : nullptr, p.flags, seed,
                           linear_id[i], epoch_next, st));
  }
  FillGroup fg;
  for (int i = 0; i < count; ++i) {
    if (R[i].theta_len > 0) fg.a[fg.n++] = FillEntry{thetaR[i], R[i].theta_len};
    if (P[i].theta_len > 0) fg.a[fg.n++] = FillEntry{thetaP[i], P[i].theta_len};
    if (fg.n + 2 > 2 * MAXG || i + 1 == count) {
      if (fg.n > 0) HIP_TRY(launch_fill_group(fg, 0.f, st));
      fg = FillGroup();
    }
  }
  return POET_OK;
}

poet_status poet_debug_gemm(const poet_gemm_desc* d, int force_generic, int* used_fast, void* stream) {
  if (!d) return fail(POET_E_ARG, "null descriptor");
  if (d->M < 0 || d->N < 0 || d->K < 0 || d->batch < 0) return fail(POET_E_SHAPE, "negative size");
  if (!d->A || !d->B) return fail(POET_E_ARG, "null A or B");
  GemmDesc g;
  g.M = d->M; g.N = d->N; g.K = d->K; g.Mtot = d->Mtot; g.Ntot = d->Ntot; g.Ktot = d->Ktot; g.batch = d->batch;
  g.A = d->A; g.lda = d->lda; g.sA = d->sA; g.a_dt = d->a_dt; g.a_kmajor = d->a_kmajor;
  g.B = d->B; g.ldb = d->ldb; g.sB = d->sB; g.b_dt = d->b_dt; g.b_kmajor = d->b_kmajor;
  g.C = d->C; g.ldc = d->ldc; g.sC = d->sC; g.c_dt = d->c_dt;
  g.C2 = d->C2; g.ldc2 = d->ldc2; g.sC2 = d->sC2; g.c2_dt = d->c2_dt;
  g.D = d->D; g.ldd = d->ldd; g.sD = d->sD;
  g.Acc = d->Acc; g.ldacc = d->ldacc; g.sAcc = d->sAcc;
  g.alpha = d->alpha; g.beta = d->beta; g.gamma = d->gamma;
  g.compute = d->compute;
  g.part = d->part; g.part_elems = d->part_elems;
  const bool fast = !force_generic && fast_gemm_eligible(g);
  if (used_fast) *used_fast = fast ? 1 : 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(fast ? launch_gemm(g, st) : launch_generic_gemm(g, st));
  return POET_OK;
}

poet_status poet_mfma_probe(int64_t iters, int32_t workgroups, float* out, void* stream) {
  if (iters < 1) return fail(POET_E_ARG, "iters = %lld must be >= 1", (long long)iters);
  if (workgroups < 1 || workgroups > 65535) return fail(POET_E_ARG, "workgroups = %d must be in [1, 65535]", workgroups);
  if (!out) return fail(POET_E_ARG, "null out");
  HIP_TRY(launch_mfma_probe(iters, workgroups, out, reinterpret_cast<hipStream_t>(stream)));
  return POET_OK;
}

const char* poet_status_string(int status) {
  switch (status) {
    case POET_OK: return "POET_OK";
    case POET_E_ARG: return "POET_E_ARG: invalid argument";
    case POET_E_SHAPE: return "POET_E_SHAPE: inconsistent or unsupported shape";
    case POET_E_DTYPE: return "POET_E_DTYPE: unsupported dtype";
    case POET_E_WORKSPACE: return "POET_E_WORKSPACE: workspace too small";
    case POET_E_HIP: return "POET_E_HIP: HIP runtime or launch failure";
    case POET_E_UNSUPPORTED: return "POET_E_UNSUPPORTED: not implemented for these arguments";
  }
  return "unknown poet_status";
}

const char* poet_last_error(void) { return g_err.c_str(); }
const char* poet_version(void) { return "poet-mi355x 0.1 (gfx950)"; }

}  // extern "C"
