"""GPU parity of exactly the step the benchmark times, on whole LLaMA-1.3B blocks at full size.

The block is made by ``bench.build_block``, grouped by ``bench.block_group`` with the benchmark's default flags
and stepped by ``bench.step``, the same functions the benchmark's timed region calls, so the launch sequence
checked here is the timed one:

- POET-BS b = 256, k = 5 (the default workload): activation-side path, the grouped build of the attention
  linears' 8 sides on the launch stream and of the MLP linears' 6 on the side stream (each writing the bf16 operand
  copies), grouped folds of P into W0 and of R into W0 on each stream, per linear the folded forward and the folded
  backward to the primitive gradients, the grouped Neumann adjoint of each class (152 blocks of 256), the MLP
  class's adjoint and update left on the side stream as in the pipelined benchmark;
- POET-FS b = 1/2, k = 5: weight-side path, grouped build of the 14 FS chains (s = 1024 on the launch stream, 2730
  on the side stream), W and the FS gradient operands formed in the build on the formation streams, per linear the
  forward and the backward to the primitive gradients from them, the grouped adjoint of each class;

each step ending with the grouped AdamW update of every side's skew parameters; then the grouped
merge-then-reinitialize of the whole block (``PoetGroup.merge``), as the benchmark's merge leg runs it (a build, then
the merge), at the recipe's parameters.

Inputs: W0 and the skew parameters come from the seeded host recipe; the activations X and upstream gradients dY
are the ones the benchmark draws on the device, copied back so that the oracle sees exactly the values the GPU
used. The step is run twice from the same parameters and optimizer state and must give bit-identical outputs,
parameters and moments (split-K sums are fixed-order).

Bars: token outputs Y and dX on 256 sampled rows per linear (tokens are independent rows, so the sample is exact),
d theta of every side in full, and the updated parameters and moments of the AdamW step (taken by the oracle from
the oracle's gradient), all against the float64 oracle at the bf16 bar 2e-2 (relative Frobenius, and the same bar
per row / per primitive); the merged W0 of every linear in full at the float32 bar 1e-5; the bf16 copy of
W0 equal to the merged W0 rounded; theta and the moments reset to zero; FS index sets equal to the oracle's for
epoch 1.
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import TOL, announce, check, theta_groups, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(lins):
    """The written part of each linear's outputs (row padding and spare gradient slots are never written)."""
    from orthogonal_reparameterized_amd import binding as B
    out = []
    for e in lins:
        lin, pl = e["spec"], e["pl"]
        out.append((e["Y"][:, :lin.m].clone(), e["dX"][:, :lin.n].clone(),
                    pl.dthetaR[:B.poet_theta_len(pl.L.R)].clone(), pl.dthetaP[:B.poet_theta_len(pl.L.P)].clone()))
    return out


def _state(lins):
    return [tuple(t.clone() for t in (e["pl"].thetaR, e["pl"].thetaP, e["pl"].mR, e["pl"].mP, e["pl"].vR, e["pl"].vP))
            for e in lins]


def _restore(lins, state, opt_steps):
    for e, st in zip(lins, state):
        pl = e["pl"]
        for dst, src in zip((pl.thetaR, pl.thetaP, pl.mR, pl.mP, pl.vR, pl.vP), st):
            dst.copy_(src)
        pl.opt_steps = opt_steps


def _block_as_benched(cfg_id):
    import bench
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    wl = PI.WORKLOADS[cfg_id]
    announce(f"bench path {wl.name}: allocating the block as the benchmark does")
    lins = bench.build_block(wl, torch, B, PI, PoetLinear, "auto")
    args = bench.parser().parse_args([])
    group = bench.block_group(lins, PoetGroup, args)
    assert group._side_idx, "the benchmark's block has a side class"
    pipe = not args.no_pipeline
    before = _state(lins)
    announce(f"bench path {wl.name}: step 1")
    bench.step(lins, group, pipeline=pipe)
    torch.cuda.synchronize()
    first, after = _outputs(lins), _state(lins)
    announce(f"bench path {wl.name}: step 2 from the same state (determinism)")
    _restore(lins, before, 0)
    bench.step(lins, group, pipeline=pipe)
    torch.cuda.synchronize()
    for e, a, b, c in zip(lins, first, _outputs(lins), _state(lins)):
        for x, y, nm in zip(a, b, ("Y", "dX", "dthetaR", "dthetaP")):
            assert torch.equal(x, y), (e["spec"].name, nm, "differs between two runs of the same step")
    for e, a, c in zip(lins, after, _state(lins)):
        for x, y, nm in zip(a, c, ("thetaR", "thetaP", "mR", "mP", "vR", "vP")):
            assert torch.equal(x, y), (e["spec"].name, nm, "differs between two runs of the same step")
    return wl, lins, group


def _check_block(cfg_id, act_path):
    import bench
    wl, lins, group = _block_as_benched(cfg_id)
    assert all(e["pl"].act_path == act_path for e in lins)
    host = []
    for e in lins:  # the values the GPU used, before the update and the merge change theta and W0
        lin, pl = e["spec"], e["pl"]
        W0, tR, tP = PI.gen_weights(wl.cfg_id, 0, lin)
        host.append({"W0": W0, "tR": tR, "tP": tP, "X": to_np(e["X"])[:, :lin.n], "dY": to_np(e["dY"])[:, :lin.m],
                     "iR": None if pl.idxR is None else pl.idxR.cpu().numpy().copy(),
                     "iP": None if pl.idxP is None else pl.idxP.cpu().numpy().copy(),
                     "tR1": to_np(pl.thetaR)[:len(tR)].copy(), "tP1": to_np(pl.thetaP)[:len(tP)].copy(),
                     "mR1": to_np(pl.mR)[:len(tR)].copy(), "mP1": to_np(pl.mP)[:len(tP)].copy(),
                     "vR1": to_np(pl.vR)[:len(tR)].copy(), "vP1": to_np(pl.vP)[:len(tP)].copy()})
        if lin.R.mode == PI.MODE_FS:  # the epoch-0 draw of the benchmark's linears is the oracle's
            iR, iP = (O.sample_indices(d, s.b, wl.seed, lin.linear_id, side, 0)
                      for d, s, side in ((lin.m, lin.R, O.SIDE_R), (lin.n, lin.P, O.SIDE_P)))
            np.testing.assert_array_equal(host[-1]["iR"], iR)
            np.testing.assert_array_equal(host[-1]["iP"], iP)
        assert pl.opt_steps == 1
    # the merge folds the factors of the recipe's parameters theta0 (oracle-side values, put back for it)
    for e, h in zip(lins, host):
        pl = e["pl"]
        pl.thetaR[:len(h["tR"])].copy_(torch.from_numpy(h["tR"]))
        pl.thetaP[:len(h["tP"])].copy_(torch.from_numpy(h["tP"]))
    announce(f"bench path {wl.name}: grouped build and merge at the recipe's theta")
    group.build()
    group.merge()
    torch.cuda.synchronize()
    tol = TOL[PI.DT_BF16]
    hp = {k: float(np.float32(x)) for k, x in bench.OPTIMIZER.items()}  # the float32 values the C ABI receives
    rows = np.sort(np.random.default_rng(31).choice(wl.T, 256, replace=False))
    for e, h in zip(lins, host):
        lin, pl = e["spec"], e["pl"]
        sR, sP = O.Side.of(lin.R), O.Side.of(lin.P)
        gR, gP = theta_groups(lin.R.mode, lin.R.d, lin.R.b), theta_groups(lin.P.mode, lin.P.d, lin.P.b)
        f = O.linear_fwd(sR, sP, h["W0"], h["tR"], h["tP"], h["iR"], h["iP"], h["X"][rows])
        g = O.linear_bwd(sR, sP, h["W0"], h["tR"], h["tP"], h["iR"], h["iP"], h["X"], h["dY"])
        mg = O.merge(sR, sP, h["W0"], h["tR"], h["tP"], h["iR"], h["iP"], wl.seed, lin.linear_id, 1)
        # the AdamW step from zero moments on the oracle's gradient: bf16 bar (it carries the gradient's error)
        oR = O.adamw_step(h["tR"], g["dthetaR"], np.zeros(len(h["tR"])), np.zeros(len(h["tR"])), 1, **hp)
        oP = O.adamw_step(h["tP"], g["dthetaP"], np.zeros(len(h["tP"])), np.zeros(len(h["tP"])), 1, **hp)
        errs = {}
        try:
            check(errs, "Y_rows", to_np(e["Y"])[rows, :lin.m], f["Y"], tol)
            check(errs, "dX_rows", to_np(e["dX"])[rows, :lin.n], g["dX"][rows], tol)
            check(errs, "dthetaR", to_np(pl.dthetaR)[:len(h["tR"])], g["dthetaR"], tol, gR)
            check(errs, "dthetaP", to_np(pl.dthetaP)[:len(h["tP"])], g["dthetaP"], tol, gP)
            for nm, want, gr in (("tR1", oR[0], gR), ("tP1", oP[0], gP), ("mR1", oR[1], gR),
                                 ("mP1", oP[1], gP), ("vR1", oR[2], gR), ("vP1", oP[2], gP)):
                check(errs, nm, h[nm], want, tol, gr)
            check(errs, "merged_W0", to_np(pl.W0)[:, :lin.n], mg["W0"], 1e-5)
        finally:
            announce(f"bench path {wl.name} {lin.name}: {errs}")
        assert float(pl.thetaR.abs().max()) == 0.0 and float(pl.thetaP.abs().max()) == 0.0, lin.name
        # the merge reinitializes the optimizer state with the parameters
        for t in (pl.mR, pl.mP, pl.vR, pl.vP):
            assert float(t.abs().max()) == 0.0, lin.name
        assert pl.epoch == 1 and pl.opt_steps == 0
        if pl.W0b is not None:  # the bf16 copy the activation side reads is the merged W0, rounded
            np.testing.assert_array_equal(to_np(pl.W0b)[:, :lin.n], PI.round_bf16(to_np(pl.W0)[:, :lin.n]))
        for got, want in ((pl.idxR, mg["idxR"]), (pl.idxP, mg["idxP"])):
            if want is not None:
                np.testing.assert_array_equal(got.cpu().numpy(), want)


def test_llama1p3b_bs256_block_as_benched():
    """LLaMA-1.3B block, POET-BS b = 256, k = 5, bf16, 16384 tokens: the benchmark's default step and merge."""
    _check_block(3, act_path=True)


def test_llama1p3b_fs_half_block_as_benched():
    """LLaMA-1.3B block, POET-FS b = 1/2, k = 5, bf16, 16384 tokens: the FS workload's step and merge."""
    _check_block(4, act_path=False)
