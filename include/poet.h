/*
 * poet.h -- C ABI of the MI355X (gfx950) POET reparameterized linear layer.
 *
 * The layer (POET pages: "Reparameterized LLM Training via Orthogonal Equivalence Transformation", the
 * one-line method summary and the Approach section) keeps each weight as W = R * W0 * P, with W0 a fixed
 * random m x n matrix (m = out features, n = in features) and R (m x m), P (n x n) learnable orthogonal
 * factors. R and P are built from skew-symmetric generators Q by the truncated Cayley-Neumann series
 *     R_k = (I + Q)(I + Q + Q^2 + ... + Q^k)
 * ("Cayley-Neumann parameterization", Approach section; k = 0 keeps no term beyond the identity, the
 * setting the "Measured effects" table reports as not converging). Each factor is made of primitives
 * ("stochastic primitive optimization", Approach section):
 *   POET-BS  block-diagonal primitives of size b (Key results: POET-BS with b = 256); when b does not
 *            divide d the last block has size d mod b;
 *   POET-FS  one dense s x s primitive acting on a sampled index set of s of the d indices, the identity
 *            elsewhere (Key results: POET-FS with b = 1/2, i.e. s = d/2).
 * The merge-then-reinitialize step (Approach section; the "Measured effects" table finds a period of 400
 * steps best) folds R and P into W0, resets the generators to zero and, for POET-FS, samples fresh indices.
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library never allocates device
 *    memory. Scratch space comes from the caller's workspace `ws` of at least poet_workspace_bytes() bytes
 *    (any alignment is accepted; the library aligns internally).
 *  - Matrices are row-major. W0, W, the bf16 shadow and the weight-gradient use leading dimension ldw >= n;
 *    X and dX use ldx >= n; Y and dY use ldy >= m (all in elements). A buffer holds whole rows: rows * ld
 *    elements (kernels may read, never write, the padding of a row). bf16 operands whose leading dimension is
 *    a multiple of 8 elements and whose base is 16-byte aligned take the fast token-GEMM path.
 *  - Skew parameters theta (and gradients dtheta) are float32, packed per primitive as the strict upper
 *    triangle in row-major order (0,1),(0,2),...,(c-2,c-1); Q_ij = theta_p, Q_ji = -theta_p. A side's
 *    primitives are concatenated in order (BS: block 0 first).
 *  - Primitives `prim` are float32, each stored as a bp x bp matrix (bp = b, or s for FS) padded with the
 *    identity outside the leading c x c block of a short last BS block.
 *  - Index sets are int32, strictly ascending, within [0, d). Invalid index sets (not ascending, out of
 *    range, repeated) give unspecified numbers; gathers clamp every index into [0, d) so no access leaves
 *    the caller's buffers.
 *  - Every call is asynchronous on the caller's HIP stream (`stream` is a hipStream_t; NULL = default
 *    stream) and never synchronizes. Arguments are validated on the host BEFORE anything is launched: on a
 *    non-OK status nothing was enqueued and no output was touched. POET_E_HIP means a launch failed; the
 *    stream's pending work is then undefined.
 *  - Calls are reentrant; the only global state is a thread-local last-error message.
 *  - Precision: act_dtype POET_F32 computes everything in float32 on fp32 MFMA. POET_BF16 feeds bf16
 *    activations and a bf16 materialized W to bf16 MFMA with float32 accumulation; the factors are applied
 *    as identity + delta so the identity part is added in float32. A side's dtype selects the operand type
 *    of its power chain (the linear term 2Q is always added in float32). The merge is float32.
 */
#ifndef POET_H
#define POET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POET_OK = 0,
  POET_E_ARG = 1,         /* null pointer where one is required, or an out-of-range enum value */
  POET_E_SHAPE = 2,       /* inconsistent or unsupported sizes / leading dimensions */
  POET_E_DTYPE = 3,       /* unsupported dtype combination */
  POET_E_WORKSPACE = 4,   /* ws_bytes smaller than poet_workspace_bytes() */
  POET_E_HIP = 5,         /* a HIP launch or runtime call failed */
  POET_E_UNSUPPORTED = 6  /* valid request this build does not implement */
} poet_status;

enum { POET_BS = 0, POET_FS = 1 };                 /* side modes */
enum { POET_F32 = 0, POET_BF16 = 1 };              /* dtypes */
enum { POET_SIDE_R = 0, POET_SIDE_P = 1 };         /* side ids used by the FS index sampler */
enum { POET_OP_BUILD = 0, POET_OP_FWD = 1, POET_OP_BWD = 2, POET_OP_MERGE = 3, POET_OP_FWD_ACT = 4, POET_OP_BWD_ACT = 5 };

/* Maximum supported Neumann terms and primitive size (a primitive must fit the kernels' tiling). */
#define POET_MAX_K 16
#define POET_MAX_PRIM 8192
#define POET_NOALLOC_MAX_D 65536

/* One orthogonal factor. mode: POET_BS or POET_FS. d: its dimension (m for R, n for P).
 * b: BS block size (1 <= b <= d) or FS sample count s (1 <= s <= d). k: Neumann terms, 0 <= k <= POET_MAX_K.
 * dtype: operand type of the power chain and of the saved powers (POET_F32 or POET_BF16). */
typedef struct poet_side {
  int32_t mode, d, b, k, dtype;
} poet_side;

/* One linear: W0 is m x n (out x in), X is T x n, Y is T x m. */
typedef struct poet_layer {
  int32_t m, n, T;
  int32_t ldw, ldx, ldy;
  int32_t act_dtype; /* POET_F32 or POET_BF16: type of X, Y, dY, dX, W and the W0 shadow */
  poet_side R, P;    /* R.d must equal m and P.d must equal n */
} poet_layer;

/* ---- sizes (pure host functions; return 0 for an invalid side/layer) --------------------------------- */

/* Number of packed skew parameters of a side: sum over primitives of c(c-1)/2. */
size_t poet_theta_len(const poet_side* s);
/* Number of primitives of a side: ceil(d/b) for BS, 1 for FS. */
size_t poet_num_prims(const poet_side* s);
/* Float32 elements of a side's primitive buffer: num_prims * bp * bp. */
size_t poet_prim_len(const poet_side* s);
/* Elements (of the side's dtype) of the saved powers Q^1..Q^k: k * num_prims * bp * ldp, where the row pitch ldp
 * is bp for float32 sides and bp rounded up to a multiple of 8 for bf16 sides (0 when k == 0). */
size_t poet_powers_len(const poet_side* s);
/* Workspace bytes a layer op needs (POET_OP_FWD, _BWD, _MERGE, _FWD_ACT or _BWD_ACT; POET_OP_BUILD gives 0, see
 * poet_build_workspace_bytes). For POET_OP_FWD the figure assumes W_out == NULL, and for POET_OP_BWD that
 * W == NULL (upper bounds). */
size_t poet_workspace_bytes(const poet_layer* L, int op);
/* Workspace bytes poet_sample_indices needs for dimension d. */
size_t poet_sample_workspace_bytes(int32_t d);
/* Workspace bytes poet_build_orthogonal needs: 0 when k == 0; otherwise room for the power chain
 * (poet_powers_len elements of the side's dtype) when it is given no powers buffer, plus, for bf16 sides whose
 * chain runs as separate products (FS, or BS blocks above 256 or not a multiple of 8), split-K scratch of
 * 8 * poet_prim_len floats. */
size_t poet_build_workspace_bytes(const poet_side* s, int with_powers);

/* ---- the hot path ---------------------------------------------------------------------------------- */

/* Build all primitives of one side from its skew parameters (truncated Cayley-Neumann series; Approach
 * section of the POET pages).
 *   theta  [poet_theta_len]  float32 in.
 *   prim   [poet_prim_len]   float32 out: R_k = I + 2(Q + ... + Q^k) + Q^{k+1} per primitive, padded.
 *   powers [poet_powers_len] out, side dtype, nullable: Q^1..Q^k of every primitive (power i of primitive
 *          p at offset ((i-1)*num_prims + p)*bp*ldp, row pitch ldp, see poet_powers_len; the pad columns
 *          are unspecified), needed by poet_linear_bwd when k >= 1.
 *   qnorm  [num_prims]       float32 out, nullable: Frobenius norm of each primitive's Q. The series
 *          converges for ||Q||_2 < 1; the pages warn it can diverge without enough terms (Limitations).
 *   flags  POET_BUILD_STEP or POET_BUILD_MERGE (below).
 *   ws     at least poet_build_workspace_bytes(s, powers != NULL) bytes (may be NULL when that is 0). */
poet_status poet_build_orthogonal(const poet_side* s, const float* theta, float* prim, void* powers,
                                  float* qnorm, int32_t flags, void* ws, size_t ws_bytes, void* stream);

/* Build precision. A bf16 chain that runs as separate products (FS sides, BS blocks above 256 or not a multiple
 * of 8; poet_build_workspace_bytes(s, 1) > 0 exactly for those) keeps Q^2 in bf16 for the training step, whose
 * products round their operands to bf16 anyway (POET_BUILD_STEP). A merge folds the primitives into the float32
 * W0, so a build that precedes one forms the square term to float32 accuracy from three bf16 parts of 2Q
 * (POET_BUILD_MERGE): two more products and the splits per side. Other sides build the same either way. Any
 * other flag value gives POET_E_ARG. */
#define POET_BUILD_STEP 0
#define POET_BUILD_MERGE 1

/* The exact Cayley primitives R = (I + Q)(I - Q)^{-1} of one side (the map the truncated series approximates;
 * "Builds on ... Cayley parameterization", Experimental setup), an accuracy reference for poet_build_orthogonal:
 * prim [poet_prim_len] float32 out, padded with the identity like the built primitives. Primitives up to 256
 * (POET_E_UNSUPPORTED above). Float32 Gauss-Jordan inversion of I - Q without pivoting (its symmetric part is the
 * identity), one workgroup per primitive; no workspace. */
poet_status poet_build_orthogonal_exact(const poet_side* s, const float* theta, float* prim, void* stream);

/* Sample the FS index set of one side (the sampled sub-block of stochastic primitive optimization,
 * Approach section; POET-FS with b = 1/2 in Key results). Counter-based: with SM one SplitMix64 output
 * step (Steele, Lea and Flood, OOPSLA 2014), h = SM(SM(SM(SM(seed) ^ linear_id) ^ side) ^ epoch),
 * key_i = SM(h ^ i); the s indices with the smallest (key_i, i) are written to idx [s] in ascending order.
 * Bit-exact and deterministic. ws: at least poet_sample_workspace_bytes(d) bytes. */
poet_status poet_sample_indices(int32_t d, int32_t s, uint64_t seed, uint32_t linear_id, uint32_t side,
                                uint32_t epoch, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* poet_sample_indices for callers that cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight loops, harnesses that forbid allocation): the same index set, bit for bit, with the per-index
 * scratch taken from a device array inside the library (d * 4 bytes of POET_NOALLOC_MAX_D * 4; each GPU the
 * library runs on holds its own copy until the process ends). d > POET_NOALLOC_MAX_D gives POET_E_SHAPE before any
 * launch. Calls on one GPU share that scratch: calls that overlap in time on one GPU (different streams, other
 * threads) race and give unspecified index sets; calls ordered on one stream are safe. Allocates nothing and
 * launches only kernels. */
poet_status poet_sample_indices_noalloc(int32_t d, int32_t s, uint64_t seed, uint32_t linear_id, uint32_t side,
                                        uint32_t epoch, int32_t* idx, void* stream);

/* Permuted POET-BS (a reading of the sampled sub-block primitives of stochastic primitive optimization, Approach
 * section of the method summary): the blocks of a side sit on consecutive runs of b ranks of a random permutation
 * of [0, d), fresh at each merge. The permutation comes from the same keys as poet_sample_indices: perm[r] = the
 * index of rank r in the order of (key_i, i), so the s lowest ranks are that call's index set; inv[i] = the rank of
 * index i (nullable). perm, inv: [d] int32 device, caller-owned. Bit-exact; one launch, no workspace. d >= 1 and
 * non-null perm, else POET_E_SHAPE / POET_E_ARG. */
poet_status poet_sample_permutation(int32_t d, uint64_t seed, uint32_t linear_id, uint32_t side, uint32_t epoch,
                                    int32_t* perm, int32_t* inv, void* stream);

/* Row and column gather, the relabeling that carries permuted POET-BS (a block-diagonal layer on the permuted
 * coordinates Pi_R W0 Pi_P^T, with the activations gathered into and out of them):
 *   out[i][j] = in[row_idx[i]][col_idx[j]]  for i < rows, j < cols,
 * a NULL index array meaning the identity. Elements of elem_bytes = 2 or 4 are moved bit for bit (bf16 activations,
 * float32 weights, int32 index arrays). in [in_rows x ldi], out [rows x ldo] device, caller-owned, not overlapping;
 * indices are clamped into [0, in_rows) / [0, in_cols). Bad sizes give POET_E_SHAPE, null pointers POET_E_ARG. */
poet_status poet_gather2d(int32_t rows, int32_t cols, int32_t elem_bytes, const void* in, int64_t ldi, int32_t in_rows,
                          int32_t in_cols, const int32_t* row_idx, const int32_t* col_idx, void* out, int64_t ldo,
                          void* stream);

/* Forward of one POET linear (one-line method summary: W = R W0 P): materializes W (act dtype) and
 * computes Y = X W^T.
 *   W0     [m x ldw] float32 in.    primR/primP: built primitives of R and P (float32 in).
 *   idxR/idxP: FS index sets [s] (int32 in); must be NULL for a BS side.
 *   X      [T x ldx] act dtype in.  Y [T x ldy] act dtype out.
 *   W_out  [m x ldw] act dtype out, nullable: keeps the materialized W (can be passed to the backward).
 * T == 0 is allowed (only W is produced). */
poet_status poet_linear_fwd(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                            const int32_t* idxR, const int32_t* idxP, const void* X, void* Y, void* W_out,
                            void* ws, size_t ws_bytes, void* stream);

/* Backward of one POET linear to its input and to the skew parameters: dX = dY W, the weight-space
 * gradient G = dY^T X, the primitive blocks of dL/dR = G (W0 P)^T and dL/dP = (R W0)^T G, the Neumann
 * adjoint and the skew projection d theta_p = dQ_ij - dQ_ji.
 *   powersR/powersP: saved powers from poet_build_orthogonal (may be NULL when that side's k == 0).
 *   W      [m x ldw] act dtype in, nullable: the W_out of the matching forward; recomputed when NULL.
 *   X [T x ldx], dY [T x ldy] act dtype in.  dX [T x ldx] act dtype out, nullable (then not computed).
 *   dthetaR [poet_theta_len(R)], dthetaP [poet_theta_len(P)] float32 out (overwritten, not accumulated). */
poet_status poet_linear_bwd(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                            const void* powersR, const void* powersP, const int32_t* idxR,
                            const int32_t* idxP, const void* W, const void* X, const void* dY, void* dX,
                            float* dthetaR, float* dthetaP, void* ws, size_t ws_bytes, void* stream);

/* As poet_linear_bwd, but it stops at the primitive gradients and leaves the Neumann adjoint to
 * poet_adjoint_group: dprimR [poet_prim_len(R)], dprimP [poet_prim_len(P)] float32 out, the primitive blocks of
 * dL/dR and dL/dP (BS: entries outside a ragged last block's extent are zero; FS: the s x s block on the index
 * set). Workspace: POET_OP_BWD. */
poet_status poet_linear_bwd_prims(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                                  const int32_t* idxR, const int32_t* idxP, const void* W, const void* X,
                                  const void* dY, void* dX, float* dprimR, float* dprimP, void* ws, size_t ws_bytes,
                                  void* stream);

/* The POET-FS weight side with its operands formed ahead of the token products (both sides POET-FS, bf16 sides and
 * activations). W = R W0 P depends only on W0, the primitives and the index sets, so a step can form every linear's W
 * (and the two gradient operands) right after the build, before any activation exists, and several linears' forms
 * can run at once on separate streams:
 *   poet_fs_form:  W [m x ldw] bf16 out (the W poet_linear_fwd materializes, bit for bit), Zr [R.b x pad8(n)] bf16
 *                  out = (W0 P)[I_R, :], Acp [m x pad8(P.b)] bf16 out = (R W0)[:, I_P] (the operands
 *                  poet_linear_bwd forms, bit for bit); ws: poet_fs_form_workspace_bytes(L) bytes.
 *   poet_linear_fwd_formed:  Y = X W^T with that W (no workspace).
 *   poet_linear_bwd_formed_prims:  as poet_linear_bwd_prims with that W, Zr and Acp (W0 and the primitives are not
 *                  read); ws: poet_workspace_bytes(L, POET_OP_BWD) bytes.
 * Layers that are not both-FS bf16 give POET_E_UNSUPPORTED. */
size_t poet_fs_form_workspace_bytes(const poet_layer* L);
poet_status poet_fs_form(const poet_layer* L, const float* W0, const float* primR, const float* primP,
                         const int32_t* idxR, const int32_t* idxP, void* W, void* Zr, void* Acp, void* ws,
                         size_t ws_bytes, void* stream);
poet_status poet_linear_fwd_formed(const poet_layer* L, const void* W, const void* X, void* Y, void* stream);
poet_status poet_linear_bwd_formed_prims(const poet_layer* L, const void* W, const void* Zr, const void* Acp,
                                         const int32_t* idxR, const int32_t* idxP, const void* X, const void* dY,
                                         void* dX, float* dprimR, float* dprimP, void* ws, size_t ws_bytes,
                                         void* stream);

/* ---- activation-side application ---------------------------------------------------------------------
 * The same layer with the factors applied to the activations around the W0 GEMM (W is never formed); the
 * products of the weight-side calls above, associated the other way (W = R W0 P from the method summary):
 *   forward   X' = X P^T,  Z = X' W0^T,  Y = Z R^T
 *   backward  dZ = dY R,  dX' = dZ W0,  dX = dX' P,  dL/dR = blocks of dY^T Z,  dL/dP = blocks of dX'^T X,
 *             then the Neumann adjoint and skew projection as in poet_linear_bwd.
 * With T >= m the forward folds P into W0 instead (Z = X (W0 P)^T), with T >= n the backward folds R
 * (dX' = dY (R W0)): the same products associated the other way, each with one bf16 rounding of the folded
 * weight in place of the rounding of X' or dZ.
 * Both sides POET-BS and bf16 activations (poet_act_path_supported); every product is a bf16 GEMM with float32
 * accumulation, and every factor is applied as identity + delta: the bf16 copy of the delta F - I is the MFMA
 * operand and the identity part adds the factor's input (X, Z, dY, dX' or W0b) in float32 before the output's one
 * rounding. W0b is W0 in bf16 (row pitch ldw), made once by
 * poet_weight_shadow and kept current by passing it as poet_merge's W0_shadow. Workspaces: POET_OP_FWD_ACT and
 * POET_OP_BWD_ACT of poet_workspace_bytes. */
int poet_act_path_supported(const poet_layer* L);  /* 1 when the calls below apply to L, else 0 */

/* W0_shadow [m x ldw] act dtype out: W0 rounded to the act dtype (round to nearest even). */
poet_status poet_weight_shadow(const poet_layer* L, const float* W0, void* W0_shadow, void* stream);

/* opsR/opsP (nullable, bf16 in): operand copies of the deltas D = F - I of the primitives F, 3 * poet_prim_len(side)
 * elements: block p of D at offset p*bp*bp and its transpose at num_prims*bp*bp + p*bp*bp, both zero outside the
 * block's c x c corner, then at 2*num_prims*bp*bp + p*bp*bp block p of D over the whole padded block (row-major,
 * bf16 of F - I; zero in the identity padding); poet_build_orthogonal_group writes them. Each bp x bp block M (M = F or F^T) of the first two parts is
 * stored row-major (M(i, j) at i*bp + j) unless bp is a multiple of 32; then it is stored in the order the MFMA
 * fragments of the application kernel are loaded: M(i, j) at ((i/32 * bp/16 + j/16) * 64 + (j/8 % 2) * 32 +
 * i % 32) * 8 + j % 8. NULL: the call makes what it needs in its workspace from primR/primP. */

/* X [T x ldx] in, Y [T x ldy] out, Z [T x ldy] out: X P^T W0^T, kept for the backward (all bf16). */
poet_status poet_linear_fwd_act(const poet_layer* L, const void* W0b, const float* primR, const float* primP,
                                const void* opsR, const void* opsP, const void* X, void* Y, void* Z, void* ws,
                                size_t ws_bytes, void* stream);

/* X [T x ldx], Z [T x ldy] (from the forward), dY [T x ldy] in; dX [T x ldx] out, nullable; dthetaR, dthetaP
 * float32 out (overwritten). powersR/powersP as in poet_linear_bwd. */
poet_status poet_linear_bwd_act(const poet_layer* L, const void* W0b, const float* primR, const float* primP,
                                const void* opsR, const void* opsP, const void* powersR, const void* powersP,
                                const void* X, const void* Z, const void* dY, void* dX, float* dthetaR,
                                float* dthetaP, void* ws, size_t ws_bytes, void* stream);

/* As poet_linear_bwd_act, but it stops at the primitive gradients and leaves the Neumann adjoint to
 * poet_adjoint_group, so that the adjoints of many linears run together:
 *   dprimR [poet_prim_len(R)], dprimP [poet_prim_len(P)] float32 out: the bp x bp blocks of dL/dR (blocks of
 *   dY^T Z) and dL/dP (blocks of dX'^T X); entries outside a ragged last block's extent are zero.
 * Workspace: POET_OP_BWD_ACT. */
poet_status poet_linear_bwd_act_prims(const poet_layer* L, const void* W0b, const float* primR, const float* primP,
                                      const void* opsR, const void* opsP, const void* X, const void* Z,
                                      const void* dY, void* dX, float* dprimR, float* dprimP, void* ws,
                                      size_t ws_bytes, void* stream);

/* The same forward and backward with the factors folded into the weight beforehand (poet_fold_weights_group):
 * W0P [m x ldw] bf16 = W0 P, RW0 [m x ldw] bf16 = R W0, each one bf16 rounding of the exact product of the bf16
 * copies. Forward: Z = X W0P^T, Y = Z R^T (Y, Z as in poet_linear_fwd_act). Backward: dX' = dY RW0, dX = dX' P
 * (dX nullable), dprimR / dprimP as in poet_linear_bwd_act_prims. Workspaces: POET_OP_FWD_ACT, POET_OP_BWD_ACT. */
poet_status poet_linear_fwd_folded(const poet_layer* L, const void* W0P, const float* primR, const void* opsR,
                                   const void* X, void* Y, void* Z, void* ws, size_t ws_bytes, void* stream);
poet_status poet_linear_bwd_folded_prims(const poet_layer* L, const void* RW0, const float* primP, const void* opsP,
                                         const void* X, const void* Z, const void* dY, void* dX, float* dprimR,
                                         float* dprimP, void* ws, size_t ws_bytes, void* stream);

/* ---- grouped calls ------------------------------------------------------------------------------------
 * The per-block steps of many sides (for instance both sides of every linear of a transformer block) in shared
 * launches, so that their blocks fill the GPU together instead of one small grid per side. Each side keeps its
 * own buffers; the tables are host arrays of count device pointers, entry i belonging to sides[i]. Results are
 * those of the one-side calls (the adjoint's split-K summation order may differ). */

/* poet_build_orthogonal for count sides (no qnorm; flags as there). powers[i] is required for every side with
 * k >= 1.
 * ops: nullable table; where ops[i] is non-NULL (BS sides only) it receives the bf16 operand copies of side i's
 * primitives that the activation-side calls take (layout above poet_linear_fwd_act).
 * ws: at least poet_build_group_workspace_bytes(count, sides) bytes (may be NULL when that is 0). */
size_t poet_build_group_workspace_bytes(int32_t count, const poet_side* sides);
poet_status poet_build_orthogonal_group(int32_t count, const poet_side* sides, const float* const* theta,
                                        float* const* prim, void* const* powers, void* const* ops, int32_t flags,
                                        void* ws, size_t ws_bytes, void* stream);

/* The Neumann adjoint and skew projection of count sides (the last step of the backward to the skew
 * parameters, Approach section): dprim[i] float32 in (poet_linear_bwd_act_prims), powers[i] the saved powers
 * of sides[i] (required when k >= 1), dtheta[i] [poet_theta_len] float32 out (overwritten). Sides with
 * theta_len 0 are skipped (their pointers may be NULL).
 * ws: at least poet_adjoint_group_workspace_bytes(count, sides) bytes. */
size_t poet_adjoint_group_workspace_bytes(int32_t count, const poet_side* sides);
poet_status poet_adjoint_group(int32_t count, const poet_side* sides, const float* const* dprim,
                               const void* const* powers, float* const* dtheta, void* ws, size_t ws_bytes,
                               void* stream);

/* The factors of count linears folded into their bf16 weights (the weights the folded activation-side calls
 * take): W0P[i] = W0b[i] P_i and RW0[i] = R_i W0b[i] (bf16, m x ldw, row pitch ldw), one batched product per factor
 * over its blocks, products of one shape in shared launches; the factor enters as identity + delta (W0b plus the
 * product with the bf16 delta, one rounding). The tables W0P and RW0 are nullable, and so is each
 * entry (nothing written for it); opsR / opsP (nullable tables and entries) are the operand copies of
 * poet_build_orthogonal_group, whose row-order part is used; without them the primitives are converted in the
 * workspace. Both sides POET-BS, bf16 activations. ws: poet_fold_group_workspace_bytes(count, layers) bytes. */
size_t poet_fold_group_workspace_bytes(int32_t count, const poet_layer* layers);
poet_status poet_fold_weights_group(int32_t count, const poet_layer* layers, const void* const* W0b,
                                    const float* const* primR, const float* const* primP, const void* const* opsR,
                                    const void* const* opsP, void* const* W0P, void* const* RW0, void* ws,
                                    size_t ws_bytes, void* stream);

/* Merge-then-reinitialize (Approach section; period 400 in the "Measured effects" table):
 *   W0 <- R W0 P in float32 (in place), using the same truncated primitives the forward pass uses;
 *   W0_shadow [m x ldw] act dtype out, nullable: a copy of the merged W0 in the act dtype;
 *   thetaR, thetaP <- 0 (so R = P = I afterwards);
 *   FS sides: idxR/idxP are read for the merge, then overwritten with the index set sampled for
 *   (seed, linear_id, side, epoch_next). BS sides pass NULL index pointers. */
poet_status poet_merge(const poet_layer* L, float* W0, void* W0_shadow, float* thetaR, float* thetaP,
                       const float* primR, const float* primP, int32_t* idxR, int32_t* idxP, uint64_t seed,
                       uint32_t linear_id, uint32_t epoch_next, void* ws, size_t ws_bytes, void* stream);

/* poet_merge for count weights (for instance the linears of a transformer block), with the in-place
 * block-diagonal merges of all of them in shared launches (one split of every factor's deltas, one P pass, one R
 * pass, one theta reset) and the others (FS sides, blocks above 256) one after another. Entry i of each table
 * belongs to layers[i], with poet_merge's meaning; W0_shadow, idxR and idxP are nullable tables (NULL: no
 * shadows, no index sets), and linear_id[i] is linear i's sampler id. The weights and shadows of the group must
 * not overlap (checked: POET_E_ARG). Results are those of poet_merge on each weight.
 * ws: at least poet_merge_group_workspace_bytes(count, layers) bytes. */
size_t poet_merge_group_workspace_bytes(int32_t count, const poet_layer* layers);
poet_status poet_merge_group(int32_t count, const poet_layer* layers, float* const* W0, void* const* W0_shadow,
                             float* const* thetaR, float* const* thetaP, const float* const* primR,
                             const float* const* primP, int32_t* const* idxR, int32_t* const* idxP, uint64_t seed,
                             const uint32_t* linear_id, uint32_t epoch_next, void* ws, size_t ws_bytes,
                             void* stream);

/* ---- optimizer step on the skew parameters -------------------------------------------------------------
 * The pages train R and P through their skew generators (Approach section) and name AdamW only as the baseline
 * optimizer of dense training (Key results); the generators' optimizer is not stated. This library provides AdamW
 * (Loshchilov and Hutter, ICLR 2019) on the packed parameters, elementwise:
 *     m <- b1 m + (1 - b1) g ;  v <- b2 v + (1 - b2) g^2 ;
 *     theta <- theta - lr ( (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) + weight_decay theta ),
 * and reinitializes the moments with the parameters at each merge (poet_optimizer_reset_group; the step count t
 * then restarts at 1): after a merge a parameter describes a rotation about the new W0 and, for POET-FS, a newly
 * sampled index pair, so old moments no longer refer to it. */
typedef struct poet_adamw {
  float lr, beta1, beta2, eps, weight_decay;  /* lr >= 0, 0 <= beta < 1, eps > 0, weight_decay >= 0 */
} poet_adamw;

/* One AdamW step on count sides in shared launches: theta[i], m[i], v[i] [poet_theta_len(sides[i])] float32 in/out
 * (updated in place), dtheta[i] float32 in (the gradient from poet_adjoint_group or poet_linear_bwd*). step >= 1 is
 * t, the number of steps since the last reset. Sides with no parameters are skipped (their pointers may be NULL).
 * Bad hyperparameters or step < 1: POET_E_ARG before any launch. */
poet_status poet_adamw_group(int32_t count, const poet_side* sides, float* const* theta, const float* const* dtheta,
                             float* const* m, float* const* v, const poet_adamw* hp, int32_t step, void* stream);

/* The moments m[i], v[i] of count sides set to zero (the optimizer state after merge-then-reinitialize). */
poet_status poet_optimizer_reset_group(int32_t count, const poet_side* sides, float* const* m, float* const* v,
                                       void* stream);

/* ---- spectral diagnostics of a weight ---------------------------------------------------------------------
 * The metrics the POET pages report next to the spectrum claim (Experimental setup, Metrics: hyperspherical energy
 * and singular-value entropy), computed on the GPU from a float32 m x n weight W (row pitch ldw >= n), for instance
 * W0 before and after a merge or a materialized W = R W0 P. Both form a Gram matrix in float64 and work in float64
 * from there; outputs are float64 device buffers. Rows of W must be nonzero for the energy.
 *   hyperspherical energy (Liu et al., NeurIPS 2018) of the neurons (rows): with w^_i = w_i / ||w_i||,
 *     E_i = sum over j != i of ||w^_i - w^_j||^(-s),  energy = sum_i E_i  (s > 0; the pages' parameters are not
 *     given, s = 1 is the usual choice);
 *   singular-value entropy (the effective-rank entropy of Roy and Vetterli, 2007): with sigma the r = min(m, n)
 *     singular values and p = sigma / sum sigma, entropy = -sum p log p; sigma (nullable) receives them, descending.
 * ws: at least poet_spectral_workspace_bytes(m, n) bytes (either call). */
size_t poet_spectral_workspace_bytes(int32_t m, int32_t n);
poet_status poet_hyperspherical_energy(int32_t m, int32_t n, const float* W, int64_t ldw, float s,
                                       double* energy_rows /* [m], nullable */, double* energy /* [1] */, void* ws,
                                       size_t ws_bytes, void* stream);
poet_status poet_singular_value_entropy(int32_t m, int32_t n, const float* W, int64_t ldw,
                                        double* sigma /* [min(m, n)], nullable */, double* entropy /* [1] */,
                                        void* ws, size_t ws_bytes, void* stream);

/* ---- diagnostics ------------------------------------------------------------------------------------ */

/* One internal GEMM of the library, exposed for kernel-level testing (not part of the layer's hot path):
 *   out = alpha * op(A) op(B) + beta * D ;  C <- out ;  C2 <- out ;  Acc += gamma * out
 * A is M x K: a_kmajor != 0 -> A(i,k) = A[i*lda + k], else A[k*lda + i]. B is K x N: b_kmajor != 0 ->
 * B(k,j) = B[j*ldb + k], else B[k*ldb + j]. Batch z offsets each operand by z times its stride s*; with
 * Mtot/Ntot/Ktot > 0 the extent of batch z is min(M, Mtot - z*M) (same for N, K). C, C2, D, Acc may be NULL.
 * a_dt, b_dt, c_dt, c2_dt: POET_F32 or POET_BF16; compute: the MFMA operand type. part / part_elems: float32
 * scratch that allows split-K on the bf16 path (NULL disables it). All pointers are device pointers.
 * force_generic != 0 runs the generic kernel even where the bf16 fast kernel applies; *used_fast (nullable)
 * reports which kernel ran. Validation is minimal (sizes >= 0, non-null A and B): this entry is for tests. */
typedef struct poet_gemm_desc {
  int32_t M, N, K, Mtot, Ntot, Ktot, batch;
  const void* A; int64_t lda, sA; int32_t a_dt, a_kmajor;
  const void* B; int64_t ldb, sB; int32_t b_dt, b_kmajor;
  void* C; int64_t ldc, sC; int32_t c_dt;
  void* C2; int64_t ldc2, sC2; int32_t c2_dt;
  const float* D; int64_t ldd, sD;
  float* Acc; int64_t ldacc, sAcc;
  float alpha, beta, gamma;
  int32_t compute;
  float* part; size_t part_elems;
} poet_gemm_desc;
poet_status poet_debug_gemm(const poet_gemm_desc* d, int force_generic, int* used_fast, void* stream);

/* Measurement aid, not an operation of the method: the sustained rate of the bf16 matrix cores. Launches
 * `workgroups` workgroups of 8 waves (two per SIMD); each wave issues 4 * iters v_mfma_f32_32x32x16_bf16 on register
 * operands (32768 flops each) with no memory traffic, then writes one float of its sums to out (device, float32,
 * workgroups * 8 elements, caller-owned). The caller times it (events on `stream`): flops / time is the ceiling
 * that the clock held under full matrix load allows a GEMM; a counter run over it shows what a fully busy matrix
 * core reads. iters >= 1, 1 <= workgroups <= 65535, out non-null, else POET_E_ARG. */
poet_status poet_mfma_probe(int64_t iters, int32_t workgroups, float* out, void* stream);

/* Kernel classes timed by the optional launch profiler. */
enum {
  POET_K_TOKEN_FWD = 0,  /* Y = X W^T */
  POET_K_TOKEN_DX = 1,   /* dX = dY W */
  POET_K_TOKEN_GW = 2,   /* G = dY^T X (the weight-space gradient) */
  POET_K_CHAIN = 3,      /* Cayley-Neumann power chain */
  POET_K_ADJOINT = 4,    /* Neumann adjoint */
  POET_K_APPLY = 5,      /* applying R and P to W0 (materialize, merge) */
  POET_K_CONTRACT = 6,   /* primitive-gradient contractions */
  POET_K_MISC = 7,       /* packing, projection, conversion, sampling */
  POET_K_MERGE = 8,      /* merge passes W0 <- R W0 P */
  POET_K_GATHER = 9,     /* FS gathers and scatters of sampled rows / columns (and the sampled-block patch) */
  POET_K_OPTIM = 10,     /* optimizer step on the skew parameters and its moment reset */
  POET_K_DIAG = 11,      /* spectral diagnostics (hyperspherical energy, singular-value entropy) */
  POET_K_NCLASS = 12
};
/* Start (on != 0: clears previous records) or stop recording a HIP event pair around every kernel launch the
 * library issues, on the launch's own stream. Process-wide; intended for benchmarking, adds one event pair
 * per launch while on. */
void poet_profile_enable(int on);
/* Sum over the recorded launches of class kclass: launch count, total duration in ms (waits for the recorded
 * events) and the algorithmic floating-point operations of those launches (2*M*N*K per GEMM; 0 for
 * data-movement classes) and algorithmic bytes (operands read once, results written once).
 * Returns POET_E_ARG for a bad class, POET_E_HIP if an event query fails. */
poet_status poet_profile_query(int kclass, int64_t* launches, double* total_ms, double* flops, double* bytes);
/* Text of a status code; any other int gives an "unknown status" text (an int, so that a code from outside the
 * enum's range is a valid argument). */
const char* poet_status_string(int status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* poet_last_error(void);
const char* poet_version(void);

#ifdef __cplusplus
}
#endif
#endif /* POET_H */
