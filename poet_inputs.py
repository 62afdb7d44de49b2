"""Seeded synthetic inputs for the POET layer, shared by the oracle-side tests and the GPU-side callers.

This module holds no arithmetic of the method itself: it only names the workload shapes and draws the random
tensors a caller feeds in (fixed weight W0, skew parameters, activations, upstream gradients). Both the CPU
oracle's tests and the GPU binding's tests/bench import it, so that both sides see bit-identical inputs.

Workloads follow the LLaMA-shaped layers the POET pages evaluate on ("Reparameterized LLM Training via
Orthogonal Equivalence Transformation", Key results and Experimental setup: LLaMA-60M to LLaMA-3B pretraining
on C4). C4 activations are not available and not needed for the hot path; they are replaced by seeded
Gaussian tensors with the same shapes. The fixed weight uses the normalized Gaussian initialization the same
page's ablation table prefers (each neuron's weight vector has unit norm).

Recipe: every tensor is drawn by ``numpy.random.default_rng(SeedSequence([cfg_id, layer, linear_idx, kind]))``
(PCG64). W0 and the skew parameters are drawn in float64 and cast to float32; X and dY are drawn directly as
float32 standard normals. Tensors that a bf16 workload feeds as bf16 are additionally rounded to bf16
(round-to-nearest-even) on the host, and both sides consume those rounded values.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# kind ids for the seed sequence
KIND_W0, KIND_THETA_R, KIND_THETA_P, KIND_X, KIND_DY = 0, 1, 2, 3, 4

# linear order inside a LLaMA block; the linear id of linear j in layer l is 7*l + j
LINEAR_NAMES = ("q", "k", "v", "o", "gate", "up", "down")

MODE_BS, MODE_FS = 0, 1
DT_F32, DT_BF16 = 0, 1


@dataclasses.dataclass(frozen=True)
class SideSpec:
    """One orthogonal factor: R (output side, d = m) or P (input side, d = n).

    mode: MODE_BS (block-diagonal, b = block size) or MODE_FS (one sampled primitive, b = sample count s).
    k: number of Neumann terms beyond the identity. dtype: operand type of the power chain.
    """
    mode: int
    d: int
    b: int
    k: int
    dtype: int


@dataclasses.dataclass(frozen=True)
class LinearSpec:
    name: str
    m: int  # out features (rows of W0)
    n: int  # in features (cols of W0)
    T: int  # tokens
    act_dtype: int
    R: SideSpec
    P: SideSpec
    linear_id: int


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    hidden: int
    ffn: int
    T: int
    mode: int
    b: Optional[int]       # BS block size (None for FS)
    frac: Optional[float]  # FS sampled fraction (None for BS)
    k: int
    dtype: int
    layers: int
    single: Optional[Tuple[int, int]] = None  # (m, n) for a single-linear workload
    seed: int = 0                             # FS sampler seed

    def linears(self, layer: int = 0) -> List[LinearSpec]:
        if self.single is not None:
            shapes = [("w", self.single[0], self.single[1])]
        else:
            h, f = self.hidden, self.ffn
            shapes = [("q", h, h), ("k", h, h), ("v", h, h), ("o", h, h),
                      ("gate", f, h), ("up", f, h), ("down", h, f)]
        out = []
        for j, (nm, m, n) in enumerate(shapes):
            out.append(LinearSpec(nm, m, n, self.T, self.dtype,
                                  self._side(m), self._side(n), 7 * layer + j))
        return out

    def _side(self, d: int) -> SideSpec:
        if self.mode == MODE_BS:
            return SideSpec(MODE_BS, d, min(self.b, d), self.k, self.dtype)
        return SideSpec(MODE_FS, d, int(d * self.frac), self.k, self.dtype)


WORKLOADS = {
    1: Workload(1, "poet_bs32_single_256x256_fp32", 256, 256, 64, MODE_BS, 32, None, 3, DT_F32, 1,
                single=(256, 256), seed=1000),
    2: Workload(2, "llama60m_block_bs64_bf16_T8192", 512, 1376, 8192, MODE_BS, 64, None, 4, DT_BF16, 1, seed=2000),
    3: Workload(3, "llama1.3b_block_bs256_bf16_T16384", 2048, 5461, 16384, MODE_BS, 256, None, 5, DT_BF16, 1,
                seed=3000),
    4: Workload(4, "llama1.3b_block_fs_half_bf16_T16384", 2048, 5461, 16384, MODE_FS, None, 0.5, 5, DT_BF16, 1,
                seed=4000),
    5: Workload(5, "llama3b_24layer_fs_half_bf16_T32768", 2560, 6848, 32768, MODE_FS, None, 0.5, 5, DT_BF16, 24,
                seed=5000),
}

THETA_STD = 1e-3  # "Q params ~N(0,1e-3)" read as standard deviation 1e-3


def rng_for(cfg_id: int, layer: int, linear_idx: int, kind: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, layer, linear_idx, kind]))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) >> 16) << 16
    r = r.astype(np.uint32)
    out = r.view(np.float32).copy()
    out[nan] = np.float32(np.nan)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values already rounded to bf16 (a uint16 array)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def row_normalized_gaussian(rng: np.random.Generator, m: int, n: int) -> np.ndarray:
    """Standard normal m x n matrix with each row scaled to unit L2 norm, as float32."""
    w = rng.standard_normal((m, n))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    return w.astype(np.float32)


def n_theta(side: SideSpec) -> int:
    """Count of packed skew parameters of one side (strict upper triangle of each primitive)."""
    if side.mode == MODE_FS:
        return side.b * (side.b - 1) // 2
    total, off = 0, 0
    while off < side.d:
        c = min(side.b, side.d - off)
        total += c * (c - 1) // 2
        off += c
    return total


def gen_linear(cfg_id: int, layer: int, lin: LinearSpec, theta_std: float = THETA_STD,
               T: Optional[int] = None):
    """Inputs of one linear: W0 (m x n, float32), thetaR, thetaP (float32), X (T x n), dY (T x m).

    X and dY are float32 holding bf16-rounded values when the linear's activations are bf16.
    """
    j = lin.linear_id % 7
    T = lin.T if T is None else T
    W0 = row_normalized_gaussian(rng_for(cfg_id, layer, j, KIND_W0), lin.m, lin.n)
    tR = (rng_for(cfg_id, layer, j, KIND_THETA_R).standard_normal(n_theta(lin.R)) * theta_std).astype(np.float32)
    tP = (rng_for(cfg_id, layer, j, KIND_THETA_P).standard_normal(n_theta(lin.P)) * theta_std).astype(np.float32)
    X = rng_for(cfg_id, layer, j, KIND_X).standard_normal((T, lin.n), dtype=np.float32)
    dY = rng_for(cfg_id, layer, j, KIND_DY).standard_normal((T, lin.m), dtype=np.float32)
    if lin.act_dtype == DT_BF16:
        X, dY = round_bf16(X), round_bf16(dY)
    return W0, tR, tP, X, dY


def gen_weights(cfg_id: int, layer: int, lin: LinearSpec, theta_std: float = THETA_STD):
    """W0, thetaR, thetaP of one linear (the same draws gen_linear makes), without the activations."""
    j = lin.linear_id % 7
    W0 = row_normalized_gaussian(rng_for(cfg_id, layer, j, KIND_W0), lin.m, lin.n)
    tR = (rng_for(cfg_id, layer, j, KIND_THETA_R).standard_normal(n_theta(lin.R)) * theta_std).astype(np.float32)
    tP = (rng_for(cfg_id, layer, j, KIND_THETA_P).standard_normal(n_theta(lin.P)) * theta_std).astype(np.float32)
    return W0, tR, tP


def pad_ld(n: int, mult: int = 64) -> int:
    return (n + mult - 1) // mult * mult
