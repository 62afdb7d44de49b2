"""Plain float64 CPU oracle of the POET reparameterized linear layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may
import this module. The product path (the HIP library and its Python binding) never calls it, and it shares no
code with that path: the only thing both sides use is the seeded input generator module, which holds none of
the method's arithmetic.

Sources. The method is described on the pages about POET ("Reparameterized LLM Training via Orthogonal
Equivalence Transformation", arXiv 2506.08001):
  * the one-line method summary and the Approach section: each weight is W = R W0 P with a fixed random W0 and
    learnable orthogonal R, P; spectrum preserved exactly; scaled by stochastic primitive optimization (sampled
    sub-block orthogonal primitives merged periodically) and a truncated Neumann-series Cayley
    parameterization;
  * the Key results: POET-FS with b = 1/2 (fully stochastic, a sampled half of each dimension) and POET-BS with
    b = 256 (block size);
  * the "Measured effects" table: merge-then-reinitialize every 400 steps is the best period; keeping no
    Neumann term (k = 0) does not converge;
  * the Limitations: the Neumann approximation needs periodic reinitialization and diverges with too few
    terms;
  * the Experimental setup ("Builds on ... Cayley parameterization").
The pages give no formulas. Where they leave a step open this oracle takes the plainest reading consistent with
them; every such reading is listed where it is used ("Reading:").

Everything is float64 NumPy. Matrix products use ``@`` (a library GEMM) as plain steps; no blocking, fusion or
reordering is done beyond what the definitions state.

Parity status: every function here is pinned by tests against closed forms, textbook routines, finite
differences, an independent library implementation (AdamW) or values printed on the pages, except the FS index
sampler's specific draws (the pages name no random generator; see ``sample_indices``) and the permutation drawn
from the same keys (``sample_permutation``), the block-size remainder reading (see ``block_sizes``) and the
optimizer state across a merge (see ``optimizer_state_after_merge``), which are "parity unpinned" beyond their
structural invariants.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

MODE_BS, MODE_FS, MODE_BSP = 0, 1, 2
SIDE_R, SIDE_P = 0, 1

_MASK64 = (1 << 64) - 1
# SplitMix64 constants as published by Steele, Lea and Flood, "Fast splittable pseudorandom number generators"
# (OOPSLA 2014): the golden-ratio increment and the two multipliers of the 64-bit finalizer.
_SM_GAMMA = 0x9E3779B97F4A7C15
_SM_M1 = 0xBF58476D1CE4E5B9
_SM_M2 = 0x94D049BB133111EB


# ----------------------------------------------------------------------------------------------------------
# Index sampling for POET-FS (stochastic primitive optimization picks a random sub-block of indices)
# ----------------------------------------------------------------------------------------------------------

def splitmix64(x):
    """One output step of SplitMix64 from 64-bit state ``x``: advance by the golden gamma, then finalize.

    Works on Python ints and on numpy uint64 arrays (wrapping arithmetic modulo 2**64).
    """
    if isinstance(x, np.ndarray):
        with np.errstate(over="ignore"):
            z = x.astype(np.uint64) + np.uint64(_SM_GAMMA)
            z = (z ^ (z >> np.uint64(30))) * np.uint64(_SM_M1)
            z = (z ^ (z >> np.uint64(27))) * np.uint64(_SM_M2)
            return z ^ (z >> np.uint64(31))
    z = (int(x) + _SM_GAMMA) & _MASK64
    z = ((z ^ (z >> 30)) * _SM_M1) & _MASK64
    z = ((z ^ (z >> 27)) * _SM_M2) & _MASK64
    return z ^ (z >> 31)


def sample_indices(d: int, s: int, seed: int, linear_id: int, side: int, epoch: int) -> np.ndarray:
    """Draw the s of d indices one POET-FS primitive acts on (ascending int32).

    The pages say only that the primitives are sampled sub-blocks (Approach section) and that POET-FS with
    b = 1/2 samples half of the dimension (Key results). Reading: a uniformly random s-subset, fresh at each
    merge, drawn with a counter-based generator so that it depends only on (seed, linear_id, side, epoch):
      h     = SM(SM(SM(SM(seed) ^ linear_id) ^ side) ^ epoch)
      key_i = SM(h ^ i)                     for i in [0, d)
    and the subset is the s indices with the smallest (key_i, i), listed in ascending order of i.
    Parity unpinned beyond its invariants: the pages fix no generator.
    """
    if not (0 <= s <= d):
        raise ValueError("need 0 <= s <= d")
    h = splitmix64(seed & _MASK64)
    h = splitmix64(h ^ (linear_id & 0xFFFFFFFF))
    h = splitmix64(h ^ (side & 0xFFFFFFFF))
    h = splitmix64(h ^ (epoch & 0xFFFFFFFF))
    i = np.arange(d, dtype=np.uint64)
    keys = splitmix64(np.uint64(h) ^ i)
    order = np.lexsort((i, keys))  # primary key: keys, ties by index
    return np.sort(order[:s]).astype(np.int32)


def sample_permutation(d: int, seed: int, linear_id: int, side: int, epoch: int) -> np.ndarray:
    """The random permutation of permuted POET-BS: perm[r] = the index of rank r among the keys of
    ``sample_indices`` (the same (seed, linear_id, side, epoch) hash and SplitMix64 keys, ordered by (key_i, i)).

    Reading: the pages call the primitives sampled sub-blocks and leave open whether POET-BS blocks are contiguous;
    the permuted variant draws a uniformly random partition into blocks, fresh at each merge, as a random
    permutation of [0, d) cut into consecutive runs of b ranks. Drawn from the FS keys, so that the s lowest ranks
    are exactly the FS index set of the same draw. Parity unpinned beyond its invariants (no generator is given).
    """
    h = splitmix64(seed & _MASK64)
    h = splitmix64(h ^ (linear_id & 0xFFFFFFFF))
    h = splitmix64(h ^ (side & 0xFFFFFFFF))
    h = splitmix64(h ^ (epoch & 0xFFFFFFFF))
    i = np.arange(d, dtype=np.uint64)
    keys = splitmix64(np.uint64(h) ^ i)
    return np.lexsort((i, keys)).astype(np.int32)


# ----------------------------------------------------------------------------------------------------------
# Primitive layout of one side
# ----------------------------------------------------------------------------------------------------------

def block_sizes(mode: int, d: int, b: int) -> List[int]:
    """Sizes of the primitives of one side.

    POET-BS: consecutive diagonal blocks of size b. Reading: when b does not divide d the last block has size
    d mod b (plain chunking of a block-diagonal matrix). Permuted POET-BS: the same sizes, taken over the ranks of
    a permutation. POET-FS: one primitive of size s = b.
    """
    if mode == MODE_FS:
        return [b]
    sizes, off = [], 0
    while off < d:
        c = min(b, d - off)
        sizes.append(c)
        off += c
    return sizes


def theta_len(mode: int, d: int, b: int) -> int:
    """Packed skew parameters of one side: c(c-1)/2 per primitive of size c."""
    return sum(c * (c - 1) // 2 for c in block_sizes(mode, d, b))


def skew_from_theta(theta: np.ndarray, c: int) -> np.ndarray:
    """Skew-symmetric c x c Q from its packed strict upper triangle (row-major order (0,1),(0,2),...).

    Reading: the parameters are the entries of Q themselves, Q_ij = theta_p and Q_ji = -theta_p for i < j.
    """
    Q = np.zeros((c, c), dtype=np.float64)
    iu = np.triu_indices(c, 1)
    Q[iu] = np.asarray(theta, dtype=np.float64)
    return Q - Q.T


def skew_project(dQ: np.ndarray) -> np.ndarray:
    """Gradient of the packed parameters from the gradient of Q: d theta_p = dQ_ij - dQ_ji (i < j)."""
    iu = np.triu_indices(dQ.shape[0], 1)
    return dQ[iu] - dQ.T[iu]


# ----------------------------------------------------------------------------------------------------------
# Cayley and truncated Cayley-Neumann maps
# ----------------------------------------------------------------------------------------------------------

def cayley_exact(Q: np.ndarray) -> np.ndarray:
    """Exact Cayley map (I + Q)(I - Q)^{-1} of a skew-symmetric Q (LAPACK solve)."""
    I = np.eye(Q.shape[0])
    return (I + Q) @ np.linalg.solve(I - Q, I)


def cayley_neumann(Q: np.ndarray, k: int) -> np.ndarray:
    """Truncated Cayley-Neumann map R_k = (I + Q) (I + Q + ... + Q^k).

    The inverse (I - Q)^{-1} of the Cayley map is replaced by its Neumann series cut after the Q^k term.
    k = 0 keeps no term beyond the identity, so R_0 = I + Q (the configuration the pages report as not
    converging).
    """
    c = Q.shape[0]
    S = np.eye(c)
    Qi = np.eye(c)
    for _ in range(k):
        Qi = Qi @ Q
        S = S + Qi
    return (np.eye(c) + Q) @ S


def neumann_adjoint(Q: np.ndarray, dR: np.ndarray, k: int) -> np.ndarray:
    """Gradient with respect to Q of <dR, R_k(Q)> for R_k = I + 2(Q + ... + Q^k) + Q^{k+1}.

    Expanding (I + Q)(I + ... + Q^k) gives coefficients a_i = 2 for 1 <= i <= k and a_{k+1} = 1. The derivative
    of Q^i in direction E is sum_{j=0}^{i-1} Q^j E Q^{i-1-j}; its adjoint applied to dR is
    sum_j (Q^T)^j dR (Q^T)^{i-1-j}. This function writes that double sum out literally.
    """
    QT = Q.T
    pw = [np.eye(Q.shape[0])]
    for _ in range(k + 1):
        pw.append(pw[-1] @ QT)
    dQ = np.zeros_like(dR, dtype=np.float64)
    for i in range(1, k + 2):
        a = 2.0 if i <= k else 1.0
        for j in range(i):
            dQ = dQ + a * (pw[j] @ dR @ pw[i - 1 - j])
    return dQ


# ----------------------------------------------------------------------------------------------------------
# One side: primitives from parameters, and the full d x d factor
# ----------------------------------------------------------------------------------------------------------

def build_orthogonal(mode: int, d: int, b: int, k: int, theta: np.ndarray) -> List[np.ndarray]:
    """All primitives R_c of one side, each the truncated Cayley-Neumann map of its skew generator."""
    theta = np.asarray(theta, dtype=np.float64)
    out, off = [], 0
    for c in block_sizes(mode, d, b):
        nt = c * (c - 1) // 2
        out.append(cayley_neumann(skew_from_theta(theta[off:off + nt], c), k))
        off += nt
    return out


def assemble(mode: int, d: int, prims: Sequence[np.ndarray], idx: Optional[np.ndarray] = None) -> np.ndarray:
    """The full d x d orthogonal factor.

    POET-BS: block-diagonal of the primitives. POET-FS: identity with the primitive placed on the sampled
    index set, F[idx, idx] = G (the other rows and columns are left untouched). Permuted POET-BS (idx = the
    permutation perm): primitive p sits on the index set I_p = perm[p b : p b + c], F[I_p, I_p] = G_p, i.e.
    F = Pi^T blockdiag(G) Pi with (Pi x)_r = x_perm[r]; the blocks cover every index.
    """
    F = np.eye(d)
    if mode == MODE_FS:
        idx = np.asarray(idx, dtype=np.int64)
        F[np.ix_(idx, idx)] = prims[0]
        return F
    if mode == MODE_BSP:
        for I, G in zip(prim_blocks(mode, d, prims_b(prims), idx), prims):
            F[np.ix_(I, I)] = G
        return F
    off = 0
    for G in prims:
        c = G.shape[0]
        F[off:off + c, off:off + c] = G
        off += c
    return F


def prims_b(prims: Sequence[np.ndarray]) -> int:
    """The block size b of a list of BS primitives (all b x b but a smaller last one)."""
    return max(G.shape[0] for G in prims)


def prim_blocks(mode: int, d: int, b: int, idx: Optional[np.ndarray] = None) -> List[np.ndarray]:
    """Index set of each primitive: consecutive ranges (BS), consecutive runs of the permutation idx (permuted
    BS), or the sampled indices (FS)."""
    if mode == MODE_FS:
        return [np.asarray(idx, dtype=np.int64)]
    out, off = [], 0
    for c in block_sizes(mode, d, b):
        r = np.arange(off, off + c)
        out.append(np.asarray(idx, dtype=np.int64)[r] if mode == MODE_BSP else r)
        off += c
    return out


def pack_prims(mode: int, d: int, b: int, prims: Sequence[np.ndarray]) -> np.ndarray:
    """Primitives in the library's storage layout: each padded to b x b with the identity."""
    out = np.zeros((len(prims), b, b))
    for p, G in enumerate(prims):
        out[p] = np.eye(b)
        c = G.shape[0]
        out[p, :c, :c] = G
    return out


# ----------------------------------------------------------------------------------------------------------
# The layer: forward, backward to the skew parameters, merge-then-reinitialize
# ----------------------------------------------------------------------------------------------------------

class Side:
    """Oracle-side description of one factor (mode, dimension d, block size or sample count b, terms k)."""

    def __init__(self, mode: int, d: int, b: int, k: int):
        self.mode, self.d, self.b, self.k = int(mode), int(d), int(b), int(k)

    @classmethod
    def of(cls, spec) -> "Side":
        return cls(spec.mode, spec.d, spec.b, spec.k)


def factor(side: Side, theta: np.ndarray, idx: Optional[np.ndarray] = None) -> np.ndarray:
    return assemble(side.mode, side.d, build_orthogonal(side.mode, side.d, side.b, side.k, theta), idx)


def linear_fwd(sR: Side, sP: Side, W0, thetaR, thetaP, idxR, idxP, X):
    """Forward of one POET linear: W = R W0 P (the reparameterization) and Y = X W^T (out x in weight)."""
    R = factor(sR, thetaR, idxR)
    P = factor(sP, thetaP, idxP)
    W = R @ np.asarray(W0, dtype=np.float64) @ P
    Y = np.asarray(X, dtype=np.float64) @ W.T
    return {"Y": Y, "W": W, "R": R, "P": P}


def linear_bwd(sR: Side, sP: Side, W0, thetaR, thetaP, idxR, idxP, X, dY):
    """Backward of one POET linear for upstream gradient dY = dL/dY.

    dX = dY W and the weight-space gradient G = dY^T X. With W = R W0 P, dL/dR = G (W0 P)^T and
    dL/dP = (R W0)^T G; only the entries that belong to a primitive are parameters, so each primitive receives
    the block of those products on its own index set (a diagonal block for BS, [idx, idx] for FS). Each block
    goes through the Neumann adjoint and the skew projection.
    """
    W0 = np.asarray(W0, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    primsR = build_orthogonal(sR.mode, sR.d, sR.b, sR.k, thetaR)
    primsP = build_orthogonal(sP.mode, sP.d, sP.b, sP.k, thetaP)
    R = assemble(sR.mode, sR.d, primsR, idxR)
    P = assemble(sP.mode, sP.d, primsP, idxP)
    W = R @ W0 @ P
    dX = dY @ W
    G = dY.T @ X
    W0P = W0 @ P
    RW0 = R @ W0
    dthR = _side_grad(sR, thetaR, idxR, lambda I: G[I, :] @ W0P[I, :].T)
    dthP = _side_grad(sP, thetaP, idxP, lambda J: RW0[:, J].T @ G[:, J])
    return {"dX": dX, "dthetaR": dthR, "dthetaP": dthP, "G": G}


def _side_grad(side: Side, theta, idx, block_grad):
    theta = np.asarray(theta, dtype=np.float64)
    out, off = [], 0
    for I in prim_blocks(side.mode, side.d, side.b, idx):
        c = len(I)
        nt = c * (c - 1) // 2
        Q = skew_from_theta(theta[off:off + nt], c)
        dQ = neumann_adjoint(Q, block_grad(I), side.k)
        out.append(skew_project(dQ))
        off += nt
    return np.concatenate(out) if out else np.zeros(0)


def merge(sR: Side, sP: Side, W0, thetaR, thetaP, idxR, idxP, seed: int, linear_id: int, epoch_next: int):
    """Merge-then-reinitialize: fold the current R and P into the fixed weight, W0 <- R W0 P, reset the skew
    parameters to zero (so R = P = I afterwards) and, for POET-FS, draw fresh index sets for the next epoch.

    Reading: the merge folds the same truncated R_k, P_k the forward pass uses, so the layer's function is
    unchanged by the merge itself. Permuted POET-BS draws a fresh permutation for the next epoch as FS draws a
    fresh index set.
    """
    R = factor(sR, thetaR, idxR)
    P = factor(sP, thetaP, idxP)
    W0n = R @ np.asarray(W0, dtype=np.float64) @ P
    out = {"W0": W0n, "thetaR": np.zeros(len(thetaR)), "thetaP": np.zeros(len(thetaP)),
           "idxR": None, "idxP": None}
    if sR.mode == MODE_FS:
        out["idxR"] = sample_indices(sR.d, sR.b, seed, linear_id, SIDE_R, epoch_next)
    if sP.mode == MODE_FS:
        out["idxP"] = sample_indices(sP.d, sP.b, seed, linear_id, SIDE_P, epoch_next)
    if sR.mode == MODE_BSP:
        out["idxR"] = sample_permutation(sR.d, seed, linear_id, SIDE_R, epoch_next)
    if sP.mode == MODE_BSP:
        out["idxP"] = sample_permutation(sP.d, seed, linear_id, SIDE_P, epoch_next)
    return out


# ----------------------------------------------------------------------------------------------------------
# Optimizer step on the skew parameters, and its state across a merge
# ----------------------------------------------------------------------------------------------------------

def adamw_step(theta, grad, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float):
    """One AdamW update of packed skew parameters (Loshchilov and Hutter, "Decoupled Weight Decay
    Regularization", ICLR 2019), written out from its definition:

        m_t = beta1 m_{t-1} + (1 - beta1) g            first moment
        v_t = beta2 v_{t-1} + (1 - beta2) g^2          second moment
        m^  = m_t / (1 - beta1^t),  v^ = v_t / (1 - beta2^t)
        theta_t = theta_{t-1} - lr (m^ / (sqrt(v^) + eps) + weight_decay theta_{t-1})

    with t = step >= 1 counted from the last reset. The pages train R and P through their skew generators
    (Approach section) and compare against AdamW (Key results) but do not name the optimizer of the generators.
    Reading: AdamW, elementwise on the packed parameters. Returns (theta_t, m_t, v_t) in float64.
    """
    if step < 1:
        raise ValueError("step counts from 1")
    theta = np.asarray(theta, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    theta = theta - lr * (mhat / (np.sqrt(vhat) + eps) + weight_decay * theta)
    return theta, m, v


def optimizer_state_after_merge(m, v):
    """Moments and step count of the skew parameters after merge-then-reinitialize.

    The pages reset the generators at each merge and, for POET-FS, resample which index pairs they act on
    (Approach section); they say nothing of the optimizer state. Reading: the moments are reinitialized with the
    parameters (zero, and the bias-correction count restarts at 0), since after the merge a parameter describes a
    rotation about a new reference W0 and, for POET-FS, a different index pair."""
    return np.zeros(len(m)), np.zeros(len(v)), 0


# ----------------------------------------------------------------------------------------------------------
# Exact Cayley primitives (the map the truncated series approximates)
# ----------------------------------------------------------------------------------------------------------

def build_orthogonal_exact(mode: int, d: int, b: int, theta: np.ndarray) -> List[np.ndarray]:
    """All primitives of one side through the exact Cayley map (I + Q)(I - Q)^{-1} of their skew generators: the
    limit k -> infinity of the truncated series, used as an accuracy reference ("Builds on ... Cayley
    parameterization", Experimental setup)."""
    theta = np.asarray(theta, dtype=np.float64)
    out, off = [], 0
    for c in block_sizes(mode, d, b):
        nt = c * (c - 1) // 2
        out.append(cayley_exact(skew_from_theta(theta[off:off + nt], c)))
        off += nt
    return out


# ----------------------------------------------------------------------------------------------------------
# Spectral diagnostics of a weight (Experimental setup, Metrics: hyperspherical energy, singular-value entropy)
# ----------------------------------------------------------------------------------------------------------

def hyperspherical_energy(W, s: float = 1.0) -> float:
    """Hyperspherical energy of the neurons of W (Liu et al., "Learning towards Minimum Hyperspherical Energy",
    NeurIPS 2018): with w^_i the rows of W scaled to unit norm (one row per output neuron),

        E_s = sum over ordered pairs i != j of ||w^_i - w^_j||^(-s)      (s > 0).

    The pages name the metric without its parameters. Reading: s = 1, rows as neurons, the plain sum over ordered
    pairs (no normalization)."""
    return float(np.sum(hyperspherical_energy_rows(W, s)))


def hyperspherical_energy_rows(W, s: float = 1.0, rows=None) -> np.ndarray:
    """Per-neuron terms of the hyperspherical energy: E_i = sum over j != i of ||w^_i - w^_j||^(-s), for the
    neurons i in `rows` (all by default); E_s is their sum over all i."""
    W = np.asarray(W, dtype=np.float64)
    Wn = W / np.linalg.norm(W, axis=1, keepdims=True)
    rows = range(Wn.shape[0]) if rows is None else rows
    out = []
    for i in rows:
        dist = np.linalg.norm(Wn[i][None, :] - Wn, axis=1)
        dist[i] = np.inf  # the pair (i, i) is excluded
        out.append(float(np.sum(dist ** (-s))))
    return np.asarray(out)


def singular_value_entropy(W) -> float:
    """Shannon entropy of the normalized singular values of W (Roy and Vetterli, "The effective rank", EUSIPCO
    2007): p_i = sigma_i / sum_j sigma_j, H = -sum_i p_i log p_i (natural log, 0 log 0 = 0). The singular values
    come from LAPACK's SVD. Reading: the pages name the metric only; the effective-rank normalization by the sum
    of the singular values is taken."""
    sig = np.linalg.svd(np.asarray(W, dtype=np.float64), compute_uv=False)
    p = sig / sig.sum()
    p = p[p > 0]
    return float(-np.sum(p * np.log(p)))
