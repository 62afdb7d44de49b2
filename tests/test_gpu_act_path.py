"""GPU parity of the activation-side path (the factors applied to the activations around the W0 GEMM,
poet_linear_fwd_act / poet_linear_bwd_act) against the CPU oracle, through the C ABI.

The oracle defines the layer once (Y = X W^T with W = R W0 P and its gradients); the activation-side path
reaches the same outputs by the other association, so the same references and the same bar apply: relative
Frobenius error <= 2e-2 for bf16 activations with float32 accumulation. The bf16 copy of W0 that the path
reads is made by poet_weight_shadow and refreshed by the merge; a merge followed by a forward checks both.
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import check, theta_groups, TOL, announce, make_linear, put_act, rel, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def act_linear(lin, W0, tR, tP, pad=0):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    return PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                      linear_id=lin.linear_id, ldw=lin.n + pad, ldx=lin.n + pad, ldy=lin.m + pad, path="act")


def run_act(lin, pad=0, theta_std=PI.THETA_STD, tag="", check_merge=False):
    announce(f"act-path {tag} m={lin.m} n={lin.n} T={lin.T} b=({lin.R.b},{lin.P.b}) k={lin.R.k} pad={pad}")
    W0, tR, tP, X, dY = PI.gen_linear(98, 0, lin, theta_std=theta_std)
    sR, sP = O.Side.of(lin.R), O.Side.of(lin.P)
    ref_f = O.linear_fwd(sR, sP, W0, tR, tP, None, None, X)
    ref_b = O.linear_bwd(sR, sP, W0, tR, tP, None, None, X, dY)
    pl = act_linear(lin, W0, tR, tP, pad)
    assert pl.act_path
    pl.build()
    Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
    Y, Z, dX = pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx)
    pl.forward_act(Xd, Y, Z)
    pl.backward_act(Xd, Z, dYd, dX)
    torch.cuda.synchronize()
    tol = TOL[lin.act_dtype]
    out = {}
    try:
        if lin.T:
            check(out, "Y", to_np(Y)[:, :lin.m], ref_f["Y"], tol)
            check(out, "dX", to_np(dX)[:, :lin.n], ref_b["dX"], tol)
        if len(tR):
            check(out, "dthetaR", to_np(pl.dthetaR)[:len(tR)], ref_b["dthetaR"], tol,
                  theta_groups(lin.R.mode, lin.R.d, lin.R.b))
        if len(tP):
            check(out, "dthetaP", to_np(pl.dthetaP)[:len(tP)], ref_b["dthetaP"], tol,
                  theta_groups(lin.P.mode, lin.P.d, lin.P.b))
    finally:
        announce(f"act-path {tag} errors {out}")
    if check_merge:  # merge, rebuild the (now identity) factors, forward again: Y = X W0_merged^T
        pl.merge()
        pl.build()
        pl.forward_act(Xd, Y, Z)
        torch.cuda.synchronize()
        mg = O.merge(sR, sP, W0, tR, tP, None, None, 0, lin.linear_id, 1)
        assert rel(to_np(pl.W0)[:, :lin.n], mg["W0"]) <= 1e-5
        np.testing.assert_array_equal(to_np(pl.W0b)[:, :lin.n], PI.round_bf16(to_np(pl.W0)[:, :lin.n]))
        y2 = X.astype(np.float64) @ mg["W0"].T
        assert rel(to_np(Y)[:, :lin.m], y2) <= tol
    return out, pl


@pytest.mark.parametrize("m,n,bR,bP,T,k,pad", [
    (520, 384, 256, 256, 1000, 5, 0),   # ragged last R block of 8 rows, two P blocks
    (300, 200, 128, 136, 300, 4, 8),    # blocks not powers of two, padded rows
    (256, 192, 64, 48, 130, 3, 0),      # blocks below the fast kernel's 128 (generic kernel)
    (272, 190, 96, 40, 77, 2, 2),       # odd token count, ragged both sides
])
def test_act_path_parity(m, n, bR, bP, T, k, pad):
    lin = make_linear(f"act-{m}-{n}", m, n, T, PI.MODE_BS, bR, bP, k, PI.DT_BF16, linear_id=4)
    run_act(lin, pad=pad, tag=f"{bR}-{bP}")


def test_act_path_zero_tokens():
    lin = make_linear("act-empty", 256, 256, 0, PI.MODE_BS, 128, 128, 3, PI.DT_BF16)
    out, pl = run_act(lin, tag="T=0")
    assert np.all(to_np(pl.dthetaR) == 0) and np.all(to_np(pl.dthetaP) == 0)


def test_act_path_merge_refreshes_w0_copy():
    # float32 sides: at this theta a bf16 power chain's rounding would exceed the merge's float32 bar
    lin = make_linear("act-merge", 384, 256, 256, PI.MODE_BS, 128, 128, 4, PI.DT_BF16, linear_id=6,
                      side_dt=PI.DT_F32)
    run_act(lin, theta_std=0.02, tag="merge", check_merge=True)


def test_act_path_matches_weight_path():
    """Both associations of the same layer agree with each other (not only with the oracle)."""
    lin = make_linear("act-vs-weight", 512, 512, 512, PI.MODE_BS, 256, 256, 5, PI.DT_BF16, linear_id=1)
    W0, tR, tP, X, dY = PI.gen_linear(97, 0, lin)
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    announce("act-vs-weight 512x512 b=256")
    res = {}
    for path in ("weight", "act"):
        pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                        path=path)
        pl.build()
        Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
        Y, dX = pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx)
        if path == "act":
            Z = pl.alloc_act(lin.T, pl.L.ldy)
            pl.forward_act(Xd, Y, Z)
            pl.backward_act(Xd, Z, dYd, dX)
        else:
            pl.forward(Xd, Y)
            pl.backward(Xd, dYd, dX)
        torch.cuda.synchronize()
        res[path] = [to_np(t) for t in (Y, dX, pl.dthetaR, pl.dthetaP)]
    for a, b in zip(res["weight"], res["act"]):
        assert rel(b, a) <= 2e-2
