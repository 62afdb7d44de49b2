"""Helpers for the GPU parity tests: run one POET linear through the C ABI and through the oracle on the same
seeded inputs, and compare with the relative Frobenius error

    rel(gpu, ref) = ||gpu - ref||_F / ||ref||_F

against 1e-5 for float32 paths and 2e-2 for bf16 activations with float32 accumulation, and element by element
with a local bound at the same bar: per row of a matrix output (a token row of Y or dX, a row of W or W0) and per
primitive of a skew-parameter gradient,

    max |gpu - ref| over the group  <=  tol * max |ref| over the group,

so that one wrong row, one wrong column band or one wrong primitive block cannot hide inside a norm taken over
the whole tensor."""
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


def row_err(gpu, ref) -> float:
    """Worst per-row ratio max_j |gpu_ij - ref_ij| / max_j |ref_ij| of two 2-D arrays (rows whose reference is all
    zero are held to an absolute zero error)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    num = np.abs(gpu - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    ratio = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(ratio.max())


def theta_groups(mode: int, d: int, b: int):
    """Packed-parameter lengths c(c-1)/2 of the primitives of one side, in storage order."""
    return [c * (c - 1) // 2 for c in O.block_sizes(mode, d, b)]


def block_err(gpu, ref, groups) -> float:
    """Worst per-primitive ratio max |gpu - ref| / max |ref| over consecutive groups of a packed 1-D vector."""
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert gpu.shape == ref.shape and sum(groups) == ref.size, (gpu.shape, ref.shape, sum(groups))
    worst, off = 0.0, 0
    for g in groups:
        if g:
            num = np.abs(gpu[off:off + g] - ref[off:off + g]).max()
            den = np.abs(ref[off:off + g]).max()
            worst = max(worst, float(num / den) if den > 0 else (0.0 if num == 0 else np.inf))
        off += g
    return worst


def check(errs: dict, name: str, gpu, ref, tol: float, groups=None):
    """Record and assert both bars for one output: the relative Frobenius error and the local element bound
    (per row for 2-D outputs, per primitive for a packed gradient with `groups`)."""
    errs[name] = rel(gpu, ref)
    errs[name + "_el"] = block_err(gpu, ref, groups) if groups is not None else row_err(gpu, ref)
    assert errs[name] <= tol, (name, errs[name], tol)
    assert errs[name + "_el"] <= tol, (name + "_el", errs[name + "_el"], tol)


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
