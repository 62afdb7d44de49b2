"""Helpers for the GPU parity tests: run one POET linear through the C ABI and through the oracle on the same
seeded inputs, and compare with the relative Frobenius error

    rel(gpu, ref) = ||gpu - ref||_F / ||ref||_F

against 1e-5 for float32 paths and 2e-2 for bf16 activations with float32 accumulation."""
import sys

import numpy as np

import oracle as O
import poet_inputs as PI

TOL = {PI.DT_F32: 1e-5, PI.DT_BF16: 2e-2}


def announce(msg: str):
    """Name the case on the real stderr before a GPU step (survives output capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def rel(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(gpu - ref)
    return float(num / den) if den > 0 else float(num)


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def make_linear(name, m, n, T, mode, bR, bP, k, dt, linear_id=0, side_dt=None):
    sd = dt if side_dt is None else side_dt
    return PI.LinearSpec(name, m, n, T, dt, PI.SideSpec(mode, m, bR, k, sd), PI.SideSpec(mode, n, bP, k, sd),
                         linear_id)


def oracle_indices(lin, seed, epoch=0):
    iR = O.sample_indices(lin.m, lin.R.b, seed, lin.linear_id, O.SIDE_R, epoch) if lin.R.mode == PI.MODE_FS else None
    iP = O.sample_indices(lin.n, lin.P.b, seed, lin.linear_id, O.SIDE_P, epoch) if lin.P.mode == PI.MODE_FS else None
    return iR, iP


def gpu_linear(lin, W0, tR, tP, iR, iP, seed=0, pad=0, stream=None):
    """A PoetLinear for the spec with leading dims padded by `pad` elements."""
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    return PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                      seed=seed, linear_id=lin.linear_id, ldw=lin.n + pad, ldx=lin.n + pad, ldy=lin.m + pad,
                      idxR=iR, idxP=iP)


def put_act(pl, A, ld):
    import torch
    t = torch.zeros((A.shape[0], ld), dtype=pl.act, device=pl.dev)
    if A.shape[0]:
        t[:, :A.shape[1]] = torch.from_numpy(np.ascontiguousarray(A, dtype=np.float32)).to(pl.dev).to(pl.act)
    return t
