"""GPU parity of single linears at their full sizes (LLaMA-1.3B BS and FS, LLaMA-3B FS), bf16, row pitch padded
to 64 elements, at the full token counts (16384, 32768).

Each linear runs on its own (``PoetLinear.build``, then the one-linear forward and backward calls); the grouped
and folded launch sequence the benchmark times is checked separately, on whole blocks, in
``test_gpu_bench_path.py``. The oracle computes the materialized weight in full and the token outputs on a seeded
sample of 256 token rows (tokens are independent rows of Y = X W^T and dX = dY W, so the sample is exact, not an
approximation). The skew-parameter gradients need the full weight-space gradient dY^T X and are compared in full.
Bars: relative Frobenius error <= 2e-2 (bf16 activations, float32 accumulation), and the same bar element by
element per row (W, Y, dX) and per primitive (d theta).
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import TOL, announce, check, oracle_indices, put_act, rel, theta_groups, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(cfg_id, name, path="weight", merge=False):
    wl = PI.WORKLOADS[cfg_id]
    lin = [l for l in wl.linears() if l.name == name][0]
    announce(f"fullsize cfg={wl.name} linear={name} m={lin.m} n={lin.n} T={lin.T}")
    W0, tR, tP, X, dY = PI.gen_linear(cfg_id, 0, lin)
    iR, iP = oracle_indices(lin, wl.seed)
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                    seed=wl.seed, linear_id=lin.linear_id, ldw=PI.pad_ld(lin.n), ldx=PI.pad_ld(lin.n),
                    ldy=PI.pad_ld(lin.m), idxR=iR, idxP=iP, path=path)
    pl.build()
    Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
    Y, dX = pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx)
    W = None
    if path == "act":
        Z = pl.alloc_act(lin.T, pl.L.ldy)
        pl.forward_act(Xd, Y, Z)
        pl.backward_act(Xd, Z, dYd, dX)
    else:
        W = pl.alloc_W()
        pl.forward(Xd, Y, W_out=W)
        pl.backward(Xd, dYd, dX, W=W)
    torch.cuda.synchronize()

    sR, sP = O.Side.of(lin.R), O.Side.of(lin.P)
    rows = np.sort(np.random.default_rng(1234).choice(lin.T, 256, replace=False))
    f = O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, X[rows])
    Wref = f["W"]
    g = O.linear_bwd(sR, sP, W0, tR, tP, iR, iP, X, dY)
    errs = {}
    tol = TOL[lin.act_dtype]
    try:
        if W is not None:
            check(errs, "W", to_np(W)[:, :lin.n], Wref, tol)
        check(errs, "Y_rows", to_np(Y)[rows, :lin.m], f["Y"], tol)
        check(errs, "dX_rows", to_np(dX)[rows, :lin.n], g["dX"][rows], tol)
        check(errs, "dthetaR", to_np(pl.dthetaR)[:len(tR)], g["dthetaR"], tol, theta_groups(lin.R.mode, lin.R.d, lin.R.b))
        check(errs, "dthetaP", to_np(pl.dthetaP)[:len(tP)], g["dthetaP"], tol, theta_groups(lin.P.mode, lin.P.d, lin.P.b))
        if merge:
            pl.merge()
            torch.cuda.synchronize()
            mg = O.merge(sR, sP, W0, tR, tP, iR, iP, wl.seed, lin.linear_id, 1)
            check(errs, "merge", to_np(pl.W0)[:, :lin.n], mg["W0"], 1e-5)
            for got, want in ((pl.idxR, mg["idxR"]), (pl.idxP, mg["idxP"])):
                if want is not None:
                    np.testing.assert_array_equal(got.cpu().numpy(), want)
    finally:
        announce(f"fullsize errors {errs}")


@pytest.mark.parametrize("name", ["gate", "down", "q"])
def test_llama1p3b_bs256_fullsize(name):
    _run(3, name)


@pytest.mark.parametrize("name", ["gate", "down"])
def test_llama1p3b_bs256_fullsize_act_path(name):
    """The activation-side path on one linear (the one-linear build, so no grouped launches and no folds; the
    grouped, folded sequence is in test_gpu_bench_path.py), on the same sampled references."""
    _run(3, name, path="act")


@pytest.mark.parametrize("name", ["up", "o", "down"])
def test_llama1p3b_fs_half_fullsize(name):
    """LLaMA-1.3B POET-FS b = 1/2 linears: up (R side s = 2730 of 5461 rows), o (s = 1024 both sides) and down
    (P side s = 2730 over 5461 columns), each followed by its merge and the index resampling."""
    _run(4, name, merge=True)


def test_llama3b_fs_half_fullsize_q():
    """LLaMA-3B q (2560 x 2560, POET-FS b = 1/2, s = 1280 per side, k = 5, bf16) at 32768 tokens."""
    _run(5, "q")


@pytest.mark.parametrize("name", ["gate", "down"])
def test_llama3b_fs_half_fullsize_wide(name):
    """The 6848-wide LLaMA-3B linears at 32768 tokens: gate (6848 x 2560, R side s = 3424) and down (2560 x 6848,
    P side s = 3424), the largest FS primitives of the configurations, with their merges (three-part products on
    the 3424-wide gathered blocks) and the index resampling."""
    _run(5, name, merge=True)


def test_llama60m_block_grouped_act_path():
    """The LLaMA-60M block (7 linears, BS b = 64, k = 4, bf16, 8192 tokens) as the benchmark runs it: activation
    side, grouped build and adjoint over all 14 sides; every output checked in full against the oracle."""
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    wl = PI.WORKLOADS[2]
    announce(f"grouped act-path block cfg={wl.name}")
    lins, data = [], []
    for lin in wl.linears(0):
        W0, tR, tP, X, dY = PI.gen_linear(2, 0, lin)
        pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                        seed=wl.seed, linear_id=lin.linear_id, ldw=PI.pad_ld(lin.n), ldx=PI.pad_ld(lin.n),
                        ldy=PI.pad_ld(lin.m), path="act")
        assert pl.act_path
        Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
        bufs = (Xd, dYd, pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx))
        lins.append(pl)
        data.append((lin, W0, tR, tP, X, dY, bufs))
    group = PoetGroup(lins)
    group.build()
    for pl, (lin, W0, tR, tP, X, dY, (Xd, dYd, Y, Z, dX)) in zip(lins, data):
        pl.forward_act(Xd, Y, Z)
        pl.backward_act_prims(Xd, Z, dYd, dX)
    group.finish_backward()
    torch.cuda.synchronize()
    for pl, (lin, W0, tR, tP, X, dY, (Xd, dYd, Y, Z, dX)) in zip(lins, data):
        sR, sP = O.Side.of(lin.R), O.Side.of(lin.P)
        f = O.linear_fwd(sR, sP, W0, tR, tP, None, None, X)
        g = O.linear_bwd(sR, sP, W0, tR, tP, None, None, X, dY)
        errs = {}
        tol = TOL[lin.act_dtype]
        try:
            check(errs, "Y", to_np(Y)[:, :lin.m], f["Y"], tol)
            check(errs, "dX", to_np(dX)[:, :lin.n], g["dX"], tol)
            check(errs, "dthetaR", to_np(pl.dthetaR)[:len(tR)], g["dthetaR"], tol,
                  theta_groups(lin.R.mode, lin.R.d, lin.R.b))
            check(errs, "dthetaP", to_np(pl.dthetaP)[:len(tP)], g["dthetaP"], tol,
                  theta_groups(lin.P.mode, lin.P.d, lin.P.b))
        finally:
            announce(f"{lin.name}: {errs}")
