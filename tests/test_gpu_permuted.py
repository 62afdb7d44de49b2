"""Permuted POET-BS on the GPU against the float64 oracle (MODE_BSP), through the C ABI.

- poet_sample_permutation: bit for bit the oracle's permutation (integer work), and inv its inverse;
- poet_gather2d: bit for bit numpy's fancy indexing, for bf16 activations, float32 weights and int32 index arrays;
- PermutedPoetLinear (a BS layer on the relabeled weight Pi_R W0 Pi_P^T with gathered activations), on the weight
  side and on the activation side: Y, dX against the oracle's permuted layer at the bf16 bar, dtheta per primitive;
  a float32 layer at the float32 bar; then merge-then-reinitialize: the merged W0 in original coordinates at the
  float32 bar, theta zero, the next epoch's permutations equal to the oracle's, and the layer's output after the
  merge against the oracle's merged layer.
Shapes: 600 x 384 with blocks of 256 and 128 (a ragged last R block of 88), 512 tokens, k = 5, theta from the input
recipe (standard deviation 1e-3: the bf16 power chain of the BS build keeps the primitives, and so the merged W0,
at the float32 bar there); and a float32 320 x 200 layer with blocks of 64 and 48.
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import TOL, announce, check, make_linear, put_act, theta_groups, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("d", [1, 7, 64, 300, 2048, 5461])
@pytest.mark.parametrize("seed,epoch", [(0, 0), (12345, 7)])
def test_permutation_sampler_bit_exact(d, seed, epoch):
    from orthogonal_reparameterized_amd import binding as B
    announce(f"permutation sampler d={d} seed={seed} epoch={epoch}")
    perm = torch.full((d,), -1, dtype=torch.int32, device="cuda")
    inv = torch.full((d,), -1, dtype=torch.int32, device="cuda")
    B.poet_sample_permutation(d, seed, 5, B.POET_SIDE_P, epoch, perm, inv)
    torch.cuda.synchronize()
    want = O.sample_permutation(d, seed, 5, O.SIDE_P, epoch)
    np.testing.assert_array_equal(perm.cpu().numpy(), want)
    np.testing.assert_array_equal(inv.cpu().numpy(), np.argsort(want))


def test_gather2d_bit_exact():
    from orthogonal_reparameterized_amd import binding as B
    rng = np.random.default_rng(3)
    announce("gather2d")
    # bf16 activations: columns gathered by a permutation, padded leading dimensions on both sides
    X = torch.randn((1000, 800), device="cuda").to(torch.bfloat16)
    cols = rng.permutation(777).astype(np.int32)
    out = torch.zeros((1000, 784), dtype=torch.bfloat16, device="cuda")
    B.poet_gather2d(X[:, :777], out, col_idx=torch.from_numpy(cols).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out[:, :777].view(torch.int16).cpu().numpy(),
                                  X[:, :777].view(torch.int16).cpu().numpy()[:, cols])
    assert not out[:, 777:].any()
    # the same through the general kernel (an output pitch that is not a multiple of 8 elements)
    out2 = torch.zeros((1000, 781), dtype=torch.bfloat16, device="cuda")
    B.poet_gather2d(X[:, :777], out2, col_idx=torch.from_numpy(cols).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out2[:, :777], out[:, :777])
    # float32 weight: rows and columns, with repeats and a shorter output
    W = torch.randn((300, 200), device="cuda")
    r = rng.integers(0, 300, 250).astype(np.int32)
    c = rng.integers(0, 200, 190).astype(np.int32)
    o = torch.empty((250, 190), device="cuda")
    B.poet_gather2d(W, o, torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o.cpu().numpy(), W.cpu().numpy()[np.ix_(r, c)])
    # int32: composing two permutations
    a, b = rng.permutation(5461).astype(np.int32), rng.permutation(5461).astype(np.int32)
    comp = torch.empty((1, 5461), dtype=torch.int32, device="cuda")
    B.poet_gather2d(torch.from_numpy(a).cuda().view(1, -1), comp, col_idx=torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(comp.cpu().numpy()[0], a[b])


def _case(m, n, T, bR, bP, k, dt, path, seed):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PermutedPoetLinear
    lin = make_linear("perm", m, n, T, PI.MODE_BS, bR, bP, k, dt, linear_id=4)
    W0, tR, tP, X, dY = PI.gen_linear(seed, 0, lin)
    pl = PermutedPoetLinear(m, n, T, B.side_of(lin.R), B.side_of(lin.P), dt, W0, tR, tP, seed=seed, linear_id=4,
                            path=path)
    sR, sP = O.Side(O.MODE_BSP, m, bR, k), O.Side(O.MODE_BSP, n, bP, k)
    iR = O.sample_permutation(m, seed, 4, O.SIDE_R, 0)
    iP = O.sample_permutation(n, seed, 4, O.SIDE_P, 0)
    return lin, pl, (W0, tR, tP, X, dY), (sR, sP, iR, iP)


def _run(pl, X, dY, path):
    L = pl.L
    Xd, dYd = put_act(pl, X, L.ldx), put_act(pl, dY, L.ldy)
    T = X.shape[0]
    Y, dX = pl.alloc_act(T, L.ldy), pl.alloc_act(T, L.ldx)
    pl.build()
    if path == "act":
        Z = pl.alloc_act(T, L.ldy)
        pl.forward_act(Xd, Y, Z)
        pl.backward_act(Xd, Z, dYd, dX)
    else:
        pl.forward(Xd, Y)
        pl.backward(Xd, dYd, dX)
    torch.cuda.synchronize()
    return to_np(Y)[:, :pl.m], to_np(dX)[:, :pl.n]


@pytest.mark.parametrize("dt,path", [(PI.DT_BF16, "weight"), (PI.DT_BF16, "act"), (PI.DT_F32, "weight")])
def test_permuted_layer_matches_oracle_and_merges(dt, path):
    if dt == PI.DT_BF16:
        m, n, T, bR, bP = 600, 384, 512, 256, 128
    else:
        m, n, T, bR, bP = 320, 200, 96, 64, 48
    lin, pl, (W0, tR, tP, X, dY), (sR, sP, iR, iP) = _case(m, n, T, bR, bP, 5, dt, path, 91)
    tol = TOL[dt]
    announce(f"permuted BS {m}x{n} T={T} dt={dt} path={path}")
    np.testing.assert_array_equal(pl.permR.cpu().numpy(), iR)
    np.testing.assert_array_equal(pl.permP.cpu().numpy(), iP)
    Y, dX = _run(pl, X, dY, path)
    fw = O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, X)
    bw = O.linear_bwd(sR, sP, W0, tR, tP, iR, iP, X, dY)
    errs = {}
    try:
        check(errs, "Y", Y, fw["Y"], tol)
        check(errs, "dX", dX, bw["dX"], tol)
        check(errs, "dthetaR", to_np(pl.dthetaR), bw["dthetaR"], tol, theta_groups(PI.MODE_BS, m, bR))
        check(errs, "dthetaP", to_np(pl.dthetaP), bw["dthetaP"], tol, theta_groups(PI.MODE_BS, n, bP))
        # merge-then-reinitialize, then the next epoch's permutations
        pl.merge()
        torch.cuda.synchronize()
        mg = O.merge(sR, sP, W0, tR, tP, iR, iP, seed=91, linear_id=4, epoch_next=1)
        check(errs, "W0", to_np(pl.original_weight()), mg["W0"], 1e-5)
        assert not pl.thetaR.any() and not pl.thetaP.any()
        np.testing.assert_array_equal(pl.permR.cpu().numpy(), mg["idxR"])
        np.testing.assert_array_equal(pl.permP.cpu().numpy(), mg["idxP"])
        Y2, _ = _run(pl, X, dY, path)
        fw2 = O.linear_fwd(sR, sP, mg["W0"], mg["thetaR"], mg["thetaP"], mg["idxR"], mg["idxP"], X)
        check(errs, "Y_after_merge", Y2, fw2["Y"], tol)
    finally:
        announce(f"permuted BS errors {errs}")
