// Internal declarations shared by the library's translation units (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace poet {

enum DType : int { F32 = 0, BF16 = 1 };

// Packed skew-parameter layout of a side (shared by the kernels that read theta):
// size of primitive p (the last BS block may be short)
__device__ __forceinline__ int prim_size(int mode, int d, int bp, int p) {
  return mode == 1 ? bp : min(bp, d - p * bp);
}
// packed position of (i, j), i < j < c, in row-major strict-upper order
__device__ __forceinline__ int64_t tri_pos(int i, int j, int c) {
  return (int64_t)i * c - (int64_t)i * (i + 1) / 2 + (j - i - 1);
}
// offset of primitive p's parameters (every primitive before p is a full bp x bp block)
__device__ __forceinline__ int64_t theta_off(int bp, int p) { return (int64_t)p * bp * (bp - 1) / 2; }

__host__ __device__ inline size_t dtype_size(int dt) { return dt == BF16 ? 2 : 4; }

// A batched GEMM  out = alpha * op(A) op(B) + beta * D ;  C <- out (if C) ;  Acc += gamma * out (if Acc).
//   A is M x K: a_kmajor -> A(i,k) = A[i*lda + k] (row-major), else A(i,k) = A[k*lda + i].
//   B is K x N: b_kmajor -> B(k,j) = B[j*ldb + k] (stored N x K), else B(k,j) = B[k*ldb + j].
//   a_sub_eye / b_sub_eye subtract the identity from the (square-block) operand on load, so a factor
//   F = I + dF is applied as its delta dF and the identity part is added in float32 through D.
//   Batch z offsets every operand by its stride s*; with *tot > 0 the extent of batch z along that dimension
//   is min(dim, tot - z*dim) (the short last block of a block-diagonal factor).
//   compute selects the MFMA type: F32 -> v_mfma_f32_32x32x2_f32, BF16 -> v_mfma_f32_32x32x16_bf16 (operands
//   rounded to bf16 when staged into LDS, float32 accumulation).
struct GemmDesc {
  int M = 0, N = 0, K = 0;
  int Mtot = 0, Ntot = 0, Ktot = 0;
  int batch = 1;
  const void* A = nullptr; int64_t lda = 0, sA = 0; int a_dt = F32; int a_kmajor = 1; int a_sub_eye = 0;
  const void* B = nullptr; int64_t ldb = 0, sB = 0; int b_dt = F32; int b_kmajor = 1; int b_sub_eye = 0;
  void* C = nullptr; int64_t ldc = 0, sC = 0; int c_dt = F32;
  // optional bf16 addend in the output's coordinates, added to the product before the output is rounded (the
  // identity part of a factor applied as identity + delta): out(i, j) = alpha AB(i, j) + beta D(i, j) + E(i, j)
  const void* E = nullptr; int64_t lde = 0, sE = 0;
  const float* D = nullptr; int64_t ldd = 0, sD = 0;
  float* Acc = nullptr; int64_t ldacc = 0, sAcc = 0;
  float alpha = 1.f, beta = 0.f, gamma = 0.f;
  int compute = F32;
  int kclass = 7;  // profiler kernel class (POET_K_* in poet.h)
  // optional second copy of the output (e.g. a float32 and a bf16 version of the same product)
  void* C2 = nullptr; int64_t ldc2 = 0, sC2 = 0; int c2_dt = F32;
  // optional float32 scratch for split-K partial sums on the bf16 fast path (deterministic reduction)
  float* part = nullptr; size_t part_elems = 0;
  // fast path only: leave the raw split-K partials in part (split s of batch z at part + (s*batch + z)*M*N, rows of
  // N floats; only the valid extent of each batch is written) for the caller to reduce; no epilogue is applied
  int defer_reduce = 0;
  // square batch entries (M == N): the product is known to be symmetric (tri = +1) or skew-symmetric (tri = -1),
  // e.g. a power of a skew-symmetric matrix. The fast path computes only the 256 x 256 output tiles on and above
  // the diagonal (no split-K) and writes each off-diagonal one a second time, transposed and times tri, below it;
  // the generic path computes every tile.
  int tri = 0;
};

// Fast path for bf16 x bf16 products (gemm_bf16.hip): 256x256x64 tiles, batched, split-K. Returns false (and
// launches nothing) when the descriptor does not qualify; launch_gemm then uses the generic kernel.
bool fast_gemm_eligible(const GemmDesc& g);
int fast_gemm_splits(const GemmDesc& g);  // split-K count the fast path uses for g
hipError_t launch_fast_gemm(const GemmDesc& g, hipStream_t st);
// Up to 16 problems of one shape (M, N, K, operand orientations, batch strides, output pitch and type) in one
// launch, each with its own operands, leading dimensions, extents and batch count (e.g. the R- and P-side
// token-axis contractions of a linear, or one power-chain step of many FS sides); plain epilogue; the split-K
// partials of all go to the first problem's scratch (none: no split-K).
bool fast_gemm_group_eligible(const GemmDesc* probs, int n);
hipError_t launch_fast_gemm_group(const GemmDesc* probs, int n, hipStream_t st);
bool fast_gemm_pair_eligible(const GemmDesc& a, const GemmDesc& b);
hipError_t launch_fast_gemm_pair(const GemmDesc& a, const GemmDesc& b, hipStream_t st);

// Power chain X_{j+1} = Q X_j, j = 0..steps-1, of nprim primitives of size bp <= 256 (power_chain.hip), with Q
// the bf16 blocks A (row pitch bp, stride sA).
//   build:   X_0 = Q; Q^{j+1} (bf16) is written at Y + j*jstep for j = 1..steps-1 (row pitch ldy, stride sy), and
//            prim (float32 bp x bp blocks, holding I + 2Q on entry) becomes I + 2Q + 2(Q^2 + .. + Q^steps) + Q^{steps+1}.
//   adjoint: X_0 from the float32 blocks X0 (row pitch ldx0, stride sx0); X_j (bf16) is written at Y + j*jstep for
//            j = 1..steps, and for j = 0 when write_x0.
struct ChainArgs {
  int bp = 0, nprim = 0, steps = 0;
  int build = 0;
  float* prim = nullptr;
  const __bf16* A = nullptr; int64_t sA = 0;
  const float* X0 = nullptr; int64_t ldx0 = 0, sx0 = 0;
  __bf16* Y = nullptr; int64_t ldy = 0, sy = 0, jstep = 0;
  int write_x0 = 0;
  // build only, nullable: bf16 copies of the deltas R_p - I of the finished primitives for the activation-side
  // products: the delta and its transpose as operand rows (zero outside each block's c x c corner, c = min(bp, d - p
  // bp) for BS, bp for FS; in fragment order where act_frag_layout(bp)), then at offset 2 nprim bp^2 the deltas of
  // the whole padded blocks, row-major
  __bf16* ops = nullptr;
  int d = 0, mode = 0;
};
bool power_chain_eligible(int bp, int dt, const void* A);  // A: the power/Q buffer (16-byte aligned)
hipError_t launch_power_chain(const ChainArgs& c, int kclass, hipStream_t st);
// A kernel reads its side's entry of a table at a dynamic index; without this the compiler reloads each field from
// the kernel arguments at every use. Copied once through keep_s, the fields stay in scalar registers.
template <class T>
__device__ __forceinline__ T keep_s(T v) {
  if constexpr (sizeof(T) == 8) {
    uint64_t u = __builtin_bit_cast(uint64_t, v);
    asm volatile("" : "+s"(u));
    return __builtin_bit_cast(T, u);
  } else {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    asm volatile("" : "+s"(u));
    return __builtin_bit_cast(T, u);
  }
}

// Up to MAXG sides in one launch (all with the same build flag; each side keeps its own sizes and buffers).
constexpr int MAXG = 16;
struct ChainGroup {
  int n = 0;
  ChainArgs a[MAXG];
};
hipError_t launch_power_chain_group(const ChainGroup& g, int kclass, hipStream_t st);

// ---- side tables: one launch over up to MAXG sides (the per-block kernels of several linears together) ----
struct PrepSide {
  const float* theta = nullptr; float* prim = nullptr; void* q = nullptr;
  int q_dt = BF16, ldq = 0, mode = 0, d = 0, bp = 0, nprim = 0;
  float coef = 2.f;
};
struct PrepGroup { int n = 0; PrepSide s[MAXG]; };
hipError_t launch_theta_prep_group(const PrepGroup& g, hipStream_t st);

struct CoefSide { const void* powers = nullptr; void* out = nullptr; int nprim = 0; };
struct CoefGroup { int n = 0, bp = 0, ldp = 0, k = 0; CoefSide s[MAXG]; };  // one (bp, ldp, k) for all sides
hipError_t launch_adjoint_coefs_group(const CoefGroup& g, int dt, hipStream_t st);

// dtheta of each side from split-K partials part[s * split_stride + (boff + p) bp^2 + ...] plus beta D
struct SkewSide { const float* D = nullptr; float* dtheta = nullptr; int mode = 0, d = 0, nprim = 0, boff = 0; };
struct SkewGroup { int n = 0, bp = 0; const float* part = nullptr; int64_t split_stride = 0; float beta = 0.f; SkewSide s[MAXG]; };
hipError_t launch_reduce_skew_group(const SkewGroup& g, int nsplit, hipStream_t st);

// prim += I + 2 Q + 2 (P_2 + .. + P_k) for the sides of a GEMM-built chain (prim holds P_{k+1} on entry)
struct FinSide {
  const float* theta = nullptr; const void* powers = nullptr; float* prim = nullptr;
  // q2 (nullable, float32, bp x bp per primitive): (2Q)^2 formed to float32 accuracy; when given it replaces the
  // saved bf16 power Q^2 in the series, and for k == 1 prim holds no chain product to add
  const float* q2 = nullptr;
  int mode = 0, d = 0, bp = 0, nprim = 0, k = 0, dt = BF16, ldp = 0;
};
struct FinGroup { int n = 0; FinSide s[MAXG]; };
hipError_t launch_chain_finalize_group(const FinGroup& g, hipStream_t st);

// AdamW on the packed skew parameters of up to MAXG sides in one launch (optim.hip): theta, m, v updated in place
// from grad; inv_bc1 / inv_bc2 are the bias-correction factors 1 / (1 - beta^t) of the step
struct OptSide { float* theta = nullptr; const float* grad = nullptr; float* m = nullptr; float* v = nullptr; int64_t n = 0; };
struct OptGroup { int n = 0; OptSide s[MAXG]; };
hipError_t launch_adamw_group(const OptGroup& g, float lr, float b1, float b2, float eps, float wd, double inv_bc1,
                              double inv_bc2, hipStream_t st);
// m, v <- 0 for every side of the group (the optimizer state after merge-then-reinitialize)
hipError_t launch_moments_reset_group(const OptGroup& g, hipStream_t st);

// prim = (I + Q)(I - Q)^{-1} of every primitive of a side (bp <= 256), float32, padded with the identity (cayley.hip)
hipError_t launch_cayley_exact(const float* theta, int mode, int d, int bp, int nprim, float* prim, hipStream_t st);

// Spectral diagnostics (spectral.hip). C (r x r float64, row pitch ldc) = W W^T (trans false, r = rows) or W^T W
// (trans true, r = cols) of the float32 rows x cols W (row pitch ldw).
hipError_t launch_gram_f64(const float* W, int64_t ldw, int rows, int cols, bool trans, double* C, int64_t ldc,
                           hipStream_t st);
// E[i] = sum_{j != i} (2 - 2 C_ij / sqrt(C_ii C_jj))^(-s/2) and total[0] = sum_i E[i]
hipError_t launch_he_rows(const double* C, int64_t ldc, int r, double s, double* E, double* total, hipStream_t st);
// Eigenvalues of the symmetric C (overwritten) by Householder tridiagonalization and bisection; sigma (nullable,
// r, descending) = sqrt of them, entropy[0] = -sum p log p of p = sigma / sum sigma. u, p, d, e, lam: r doubles each.
hipError_t launch_sym_eig_entropy(double* C, int64_t ldc, int r, double* u, double* p, double* d, double* e,
                                  double* lam, double* sigma, double* entropy, hipStream_t st);


// Fused application of block-diagonal factors on both sides (bs_apply.hip), blocks bpR, bpP <= 256, W0 float32
// m x n with row pitch ldw (rows readable up to a multiple of 4 columns), primitives float32 bp x bp blocks:
// Tb = bf16(W0 P), W = R W0 P (dtype w_dt), RW0b = bf16(R W0), each written (row pitch ldw) when non-null.
struct ApplyArgs {
  int m = 0, n = 0, bpR = 0, nR = 0, bpP = 0, nP = 0;
  const float* W0 = nullptr; int64_t ldw = 0;
  const float* primR = nullptr;
  const float* primP = nullptr;
  __bf16* Tb = nullptr;
  void* W = nullptr; int w_dt = BF16;
  __bf16* RW0b = nullptr;
};
bool bs_apply_eligible(int bpR, int bpP, const float* W0, int64_t ldw, const float* primR, const float* primP);
hipError_t launch_bs_apply(const ApplyArgs& c, hipStream_t st);

// In-place merge of block-diagonal factors into W0 (bs_merge.hip), blocks bp <= 256, float32 accuracy, for
// several weights at once: every item's factor deltas are pre-split in one launch, then
//   P pass:  W[:, J] <- W[:, J] F_J for every block J of the columns (F = P, blocks along n), all items together
//   R pass:  W[I, :] <- F_I W[I, :] for every block I of the rows (F = R, blocks along m), all items together;
//            also writes shadow (dtype sh_dt, row pitch ld_sh) when non-null
// primR / primP: nR / nP float32 bpR x bpR / bpP x bpP blocks. The items' W (and shadows) must not overlap.
struct MergeItem {
  float* W = nullptr; int64_t ld = 0; int m = 0, n = 0;
  int bpR = 0, nR = 0; const float* primR = nullptr;
  int bpP = 0, nP = 0; const float* primP = nullptr;
  void* shadow = nullptr; int sh_dt = BF16; int64_t ld_sh = 0;
};
bool bs_merge_eligible(int bp, int m, int64_t ld);  // W0 (m x ld floats) under 2 GB
size_t bs_merge_split_bytes(int bp, int nblk);
size_t bs_merge_group_bytes(const MergeItem* it, int n);  // scratch of launch_bs_merge_group
hipError_t launch_bs_merge_group(const MergeItem* it, int n, char* split, hipStream_t st);

// Block-diagonal factor applied to bf16 activations (act_apply.hip) as identity + delta: out[t, block] =
// in[t, block] + in[t, block] B_block for T tokens of dimension d, blocks bp <= 256 (a multiple of 8), with the
// operand B = (F - I)^T (trans) or F - I given as bf16 rows Bt[j][k] = B(k, j) (fragment order where
// act_frag_layout(bp), else row order) by launch_act_operand from the nblk float32 bp x bp primitives F. Row
// pitches ldi, ldo multiples of 8, in and out 16-byte aligned, the input under 4 GB.
// Layout of the bf16 operand rows Bt[j][k] = B(k, j) of one bp x bp block:
//   row order       element (j, k) at j bp + k;
//   fragment order  (bp a multiple of 32) the MFMA fragments in the order the kernel loads them: column group
//                   g = j / 32, k-step s = k / 16, lane l = 32 ((k / 8) % 2) + j % 32, element v = k % 8 at
//                   ((g (bp / 16) + s) 64 + l) 8 + v, so that one fragment load of a wave reads 1 KB contiguous.
__host__ __device__ inline bool act_frag_layout(int bp) { return bp % 32 == 0; }
__host__ __device__ inline int64_t act_frag_index(int bp, int j, int k) {
  return ((int64_t)((j >> 5) * (bp >> 4) + (k >> 4)) * 64 + ((k >> 3) & 1) * 32 + (j & 31)) * 8 + (k & 7);
}
bool act_apply_eligible(int bp, const void* in, int64_t ldi, const void* out, int64_t ldo, int T);
hipError_t launch_act_operand(const float* F, int bp, int d, int nblk, bool trans, __bf16* Bt, hipStream_t st);
hipError_t launch_act_apply(const __bf16* in, int64_t ldi, __bf16* out, int64_t ldo, const __bf16* Bt, int T, int d,
                            int bp, int nblk, hipStream_t st);

// launch profiler (profiler.hip): no-ops unless poet_profile_enable(1) was called
int prof_begin(int kclass, hipStream_t st, double flops, double bytes);
void prof_end(int rec, hipStream_t st);
struct ProfScope {
  int rec;
  hipStream_t st;
  ProfScope(int c, hipStream_t s, double f, double b) : rec(prof_begin(c, s, f, b)), st(s) {}
  ~ProfScope() { prof_end(rec, st); }
};

hipError_t launch_gemm(const GemmDesc& g, hipStream_t st);
hipError_t launch_generic_gemm(const GemmDesc& g, hipStream_t st);  // never the fast path



// ---- elementwise / data-movement kernels (kernels_misc.hip) ------------------------------------------
// theta -> prim = I + coef*Q (coef 1 for k = 0, else 2) and, when q_out != null, Q in dtype q_dt.
hipError_t launch_theta_prep(const float* theta, int mode, int d, int bp, int nprim, int k, float* prim,
                             void* q_out, int q_dt, int ldq, hipStream_t st);  // q_out: bp x ldq blocks
hipError_t launch_qnorm(const float* theta, int mode, int d, int bp, int nprim, float* qnorm, hipStream_t st);
// dtheta_p = X_ij - X_ji with X = dQ + G1 (G1 nullable) for i < j < c of every primitive.
hipError_t launch_skew_project(const float* dQ, const float* G1, int mode, int d, int bp, int nprim,
                               float* dtheta, hipStream_t st);
// dtheta_p = X_ij - X_ji, X = (sum over nsplit float32 partials in split order) + beta D, for i < j < c of every
// primitive; split s of primitive p at part + s*split_stride + p*bp*bp (row pitch bp), D float32 bp x bp blocks
// (nullable: no addend).
hipError_t launch_reduce_skew(const float* part, int nsplit, int64_t split_stride, const float* D, float beta, int mode,
                              int d, int bp, int nprim, float* dtheta, hipStream_t st);
hipError_t launch_fill(float* p, size_t n, float v, hipStream_t st);
// zeros the gap columns [bp, ldp) of nblk side-by-side blocks (block j at column j ldp) in each of rows rows of a
// bf16 matrix with row pitch ld
hipError_t launch_zero_gaps(__bf16* H, int64_t rows, int64_t ld, int ldp, int bp, int nblk, hipStream_t st);
struct FillEntry { float* p = nullptr; size_t n = 0; };
struct FillGroup { int n = 0; FillEntry a[2 * MAXG]; };  // n >= 1 entries filled in one launch
hipError_t launch_fill_group(const FillGroup& g, float v, hipStream_t st);
// prim[p] (bp x bp) = diagonal sub-block p % g of super-block p / g (g bp x g bp, row pitch sb = g bp) of sup, zero
// past a ragged last block (dimension d)
hipError_t launch_extract_diag(const float* sup, int sb, int g, int bp, int d, int nprim, float* prim, hipStream_t st);
// dst (rows x cols, ld_dst, dtype dst_dt) <- src (float32, ld_src)
hipError_t launch_convert(const float* src, int64_t ld_src, void* dst, int64_t ld_dst, int dst_dt, int rows,
                          int cols, hipStream_t st);
// dst[r][j] = src[r][idx[j]]  (rows x s), src float32 with ld_src
hipError_t launch_gather_cols(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim,
                              float* dst, int64_t ld_dst, hipStream_t st);
// dst[r][idx[j]] = src[r][j]
hipError_t launch_scatter_cols(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim,
                               float* dst, int64_t ld_dst, hipStream_t st);
// dst[i][c] = src[idx[i]][c]  (s x cols)
hipError_t launch_gather_rows(const void* src, int src_dt, int64_t ld_src, const int32_t* idx, int s, int dlim,
                              int cols, float* dst, int64_t ld_dst, hipStream_t st);
// dst[idx[i]][c] = src[i][c], dst of dtype dst_dt
hipError_t launch_scatter_rows(const float* src, int64_t ld_src, const int32_t* idx, int s, int dlim, int cols,
                               void* dst, int dst_dt, int64_t ld_dst, hipStream_t st);
hipError_t launch_sample(int d, int s, uint64_t h, int32_t* flags, int32_t* idx, hipStream_t st);
// perm[r] = the index of rank r of the same keys (inv[i] = rank of i, nullable): permuted POET-BS
hipError_t launch_sample_permutation(int d, uint64_t h, int32_t* perm, int32_t* inv, hipStream_t st);
// out[i][j] = in[row_idx[i]][col_idx[j]] (null index arrays: identity), elements of 2 or 4 bytes, indices clamped
hipError_t launch_gather2d(int rows, int cols, int elem_bytes, const void* in, int64_t ldi, int in_rows, int in_cols,
                           const int32_t* row_idx, const int32_t* col_idx, void* out, int64_t ldo, hipStream_t st);
// Three bf16 parts of X (rows x cols, float32) for products to float32 accuracy on bf16 MFMA:
// X(i, j) = src[r(i) * ld_src + c(j)] - [sub_eye && i == j], r(i) = ridx ? ridx[i] : i, c(j) = cidx ? cidx[j] : j
// (indices clamped to rlim / clim). Part t = 0, 1, 2 is hi(X) = bf16(X), or lo(X) = bf16(X - hi(X)) where bit t of
// lo_mask is set, written at dst + t tstride with element (i, j) at i ld_dst + j over prows x pcols (zero outside
// rows x cols). D (nullable, row pitch ld_d) receives X in float32.
hipError_t launch_split3(const float* src, int64_t ld_src, const int32_t* ridx, const int32_t* cidx, int rlim, int clim,
                         int sub_eye, int rows, int cols, int prows, int pcols, __bf16* dst, int64_t ld_dst,
                         int64_t tstride, int lo_mask, float* D, int64_t ld_d, hipStream_t st);
// prim = I + 2 Q + 2 (P_2 + ... + P_k) + P_{k+1} with prim holding P_{k+1} on entry (k >= 1), Q from theta;
// powers[t-1] = P_t as bp x ldp blocks. With q2 ((2Q)^2 in float32, bp x bp per primitive) the Q^2 term is q2 / 4
// instead of P_2, and for k == 1 prim's entry value is not used (the series ends at Q^2).
hipError_t launch_chain_finalize(const float* theta, int mode, int d, int bp, int nprim, int k, const void* powers,
                                 int dt, int ldp, float* prim, hipStream_t st, const float* q2 = nullptr);
// out = bf16(prim - I) for nprim bp x bp primitives (the delta of a factor as an MFMA operand), written as bp x ldo
// blocks with zero columns past bp
hipError_t launch_delta_bf16(const float* prim, int nprim, int bp, int ldo, __bf16* out, hipStream_t st);

// Matrix-core rate probe (mfma_probe.hip): workgroups x 8 waves, each issuing 4 x iters bf16 MFMAs of 32 x 32 x 16 on
// registers; out receives one float per wave (workgroups x 8).
hipError_t launch_mfma_probe(int64_t iters, int workgroups, float* out, hipStream_t st);
// Coefficient polynomials of the two-phase Neumann adjoint, stacked per primitive as (k+1) ldp x ldp blocks (rows
// and columns past bp zero): block j = sum_{t} a_{t+j+1} (-1)^{t+j} Q^t over t = 0..k-j (t >= 1 for j = 0),
// Q^0 = I, Q^t = powers[t-1] (bp x ldp blocks), with a_i = 2 for i <= k and a_{k+1} = 1. Dtype dt (the powers').
hipError_t launch_adjoint_coefs(const void* powers, int dt, int nprim, int bp, int ldp, int k, void* out, hipStream_t st);
// gathers into a typed destination (dst_dt) and, when dst2 is given, also into a bf16 copy (same read)
hipError_t launch_gather_cols_to(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim,
                                 void* dst, int dst_dt, int64_t ld_dst, hipStream_t st, __bf16* dst2 = nullptr,
                                 int64_t ld_dst2 = 0);
hipError_t launch_gather_rows_to(const void* src, int src_dt, int64_t ld_src, const int32_t* idx, int s, int dlim,
                                 int cols, void* dst, int dst_dt, int64_t ld_dst, hipStream_t st, __bf16* dst2 = nullptr,
                                 int64_t ld_dst2 = 0);
// dst[i][cidx[j]] = C[ridx[i]][j] for i < sr, j < sc, and its bf16 copy dst2[i][cidx[j]]
hipError_t launch_patch_block(const float* C, int64_t ldc, const int32_t* ridx, int rlim, const int32_t* cidx, int clim,
                              int sr, int sc, float* dst, int64_t ld_dst, __bf16* dst2, int64_t ld_dst2, hipStream_t st);
// dst[r][idx[j]] = src[r][j] into a typed destination (dst_dt)
hipError_t launch_scatter_cols_to(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim,
                                  void* dst, int dst_dt, int64_t ld_dst, hipStream_t st);
uint64_t sampler_hash(uint64_t seed, uint32_t linear_id, uint32_t side, uint32_t epoch);

}  // namespace poet
