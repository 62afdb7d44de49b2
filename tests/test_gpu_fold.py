"""The activation-side path with the factors folded into the weight: W0P = W0 P for the forward's token GEMM and
RW0 = R W0 for the backward's (poet_fold_weights_group, poet_linear_fwd_folded, poet_linear_bwd_folded_prims).

A block of linears whose token count is at least their rows and columns, blocks of 128 and more (ragged last
blocks, blocks not a power of two, padded rows), plus one linear with fewer tokens than rows (not folded), run
through PoetGroup (grouped build, grouped fold, folded forward and backward, grouped adjoint). Checked against:
  - the one-linear calls (poet_linear_fwd_act / poet_linear_bwd_act_prims, which fold inside the call when the
    shape asks for it): bit for bit (the same products on the same kernel);
  - float64 products of the bf16 copies for W0P and RW0 (one bf16 rounding);
  - the oracle for Y, dX and dtheta (bf16 bar).
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import TOL, announce, check, make_linear, put_act, rel, theta_groups, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# name, m, n, bR, bP, T, k, row padding
SPECS = [
    ("q", 512, 512, 256, 256, 1024, 5, 0),
    ("k", 512, 512, 256, 256, 1024, 5, 0),
    ("gate", 600, 384, 256, 128, 1024, 5, 8),   # ragged last R block (88), padded rows
    ("down", 384, 600, 128, 256, 1024, 5, 8),   # ragged last P block
    ("odd", 300, 272, 136, 136, 1024, 4, 4),    # blocks not a power of two
    ("wide", 1100, 512, 256, 256, 1024, 5, 0),  # T < m: P is applied to the tokens, R still folded
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _linear(spec, i):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    name, m, n, bR, bP, T, k, pad = spec
    lin = make_linear(name, m, n, T, PI.MODE_BS, bR, bP, k, PI.DT_BF16, linear_id=i)
    W0, tR, tP, X, dY = PI.gen_linear(31, 0, lin, theta_std=0.01)
    mk = lambda: PoetLinear(m, n, T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP, linear_id=i,
                            ldw=n + pad, ldx=n + pad, ldy=m + pad, path="act")
    return lin, (W0, tR, tP, X, dY), mk(), mk()


def test_folded_group_matches_one_linear_calls_and_oracle():
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup
    cases = [_linear(spec, i) for i, spec in enumerate(SPECS)]
    group = PoetGroup([g for _, _, _, g in cases])
    announce("fold: one-linear calls")
    one_out, acts = [], []
    for lin, (W0, tR, tP, X, dY), one, _ in cases:
        Xd, dYd = put_act(one, X, one.L.ldx), put_act(one, dY, one.L.ldy)
        acts.append((Xd, dYd))
        Y, Z, dX = (one.alloc_act(lin.T, one.L.ldy), one.alloc_act(lin.T, one.L.ldy), one.alloc_act(lin.T, one.L.ldx))
        one.build()
        one.forward_act(Xd, Y, Z)
        one.backward_act_prims(Xd, Z, dYd, dX)
        one_out.append((Y, Z, dX))
    torch.cuda.synchronize()
    announce("fold: grouped build, fold, folded forward and backward")
    group.build()
    grp_out = []
    for (lin, _, _, pl), (Xd, dYd) in zip(cases, acts):
        Y, Z, dX = (pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx))
        pl.forward_act(Xd, Y, Z)
        pl.backward_act_prims(Xd, Z, dYd, dX)
        grp_out.append((Y, Z, dX))
    group.finish_backward()
    torch.cuda.synchronize()
    for (lin, (W0, tR, tP, X, dY), one, pl), o1, o2 in zip(cases, one_out, grp_out):
        foldP, foldR = lin.T >= lin.m, lin.T >= lin.n
        assert (pl.W0P is not None) == foldP and (pl.RW0 is not None) == foldR, lin.name
        for a, b, nm, w in zip(o1, o2, ("Y", "Z", "dX"), (lin.m, lin.m, lin.n)):  # (row padding is never written)
            assert torch.equal(a[:, :w], b[:, :w]), (lin.name, nm)
        assert torch.equal(one.dprimR, pl.dprimR) and torch.equal(one.dprimP, pl.dprimP), lin.name
        # the folded weights: one bf16 rounding of the products of the bf16 copies
        W0b = to_np(pl.W0b)[:, :lin.n].astype(np.float64)
        if foldP:
            Pb = np.zeros((lin.n, lin.n))
            for p, c in enumerate(O.block_sizes(PI.MODE_BS, lin.n, lin.P.b)):
                blk = PI.round_bf16(to_np(pl.primP).reshape(-1, lin.P.b, lin.P.b)[p, :c, :c]).astype(np.float64)
                Pb[p * lin.P.b:p * lin.P.b + c, p * lin.P.b:p * lin.P.b + c] = blk
            e = rel(to_np(pl.W0P)[:, :lin.n], W0b @ Pb)
            assert e <= 2 ** -8, (lin.name, "W0P", e)
        if foldR:
            Rb = np.zeros((lin.m, lin.m))
            for p, c in enumerate(O.block_sizes(PI.MODE_BS, lin.m, lin.R.b)):
                blk = PI.round_bf16(to_np(pl.primR).reshape(-1, lin.R.b, lin.R.b)[p, :c, :c]).astype(np.float64)
                Rb[p * lin.R.b:p * lin.R.b + c, p * lin.R.b:p * lin.R.b + c] = blk
            e = rel(to_np(pl.RW0)[:, :lin.n], Rb @ W0b)
            assert e <= 2 ** -8, (lin.name, "RW0", e)
        # the layer against the oracle
        sR, sP = O.Side.of(lin.R), O.Side.of(lin.P)
        f = O.linear_fwd(sR, sP, W0, tR, tP, None, None, X)
        g = O.linear_bwd(sR, sP, W0, tR, tP, None, None, X, dY)
        errs = {}
        try:
            tol = TOL[PI.DT_BF16]
            check(errs, "Y", to_np(o2[0])[:, :lin.m], f["Y"], tol)
            check(errs, "dX", to_np(o2[2])[:, :lin.n], g["dX"], tol)
            check(errs, "dthetaR", to_np(pl.dthetaR)[:len(tR)], g["dthetaR"], tol,
                  theta_groups(lin.R.mode, lin.R.d, lin.R.b))
            check(errs, "dthetaP", to_np(pl.dthetaP)[:len(tP)], g["dthetaP"], tol,
                  theta_groups(lin.P.mode, lin.P.d, lin.P.b))
        finally:
            announce(f"fold {lin.name} (P folded {foldP}, R folded {foldR}): {errs}")


def test_side_linears_pipelined_steps_match_one_call():
    """PoetGroup(side_linears=...): the named linears build, fold and run their adjoint and AdamW update on the side
    stream (finish_backward(join=False) leaves the last two open into the next step); three training steps end in
    the same theta, moments, Y, Z and dX as three steps of one call per step on the launch stream, bit for bit."""
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("fold: side-stream linears, pipelined steps vs one call per step")
    cases = [_linear(spec, i) for i, spec in enumerate(SPECS)]
    hp = B.adamw(lr=1e-3)
    out = []
    for pick, open_ in ((lambda c: c[2], False), (lambda c: c[3], True)):
        pls = [pick(c) for c in cases]
        g = PoetGroup(pls, side_linears=[2, 3, 5]) if open_ else PoetGroup(pls, side_chains=False)
        assert bool(g._side_idx) == open_
        bufs = []
        for (lin, (W0, tR, tP, X, dY), _, _), pl in zip(cases, pls):
            bufs.append((put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldy),
                         pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx)))
        for _ in range(3):
            g.build()
            for pl, (Xd, dYd, Y, Z, dX) in zip(pls, bufs):
                pl.forward_act(Xd, Y, Z)
                pl.backward_act_prims(Xd, Z, dYd, dX)
            g.finish_backward(join=not open_)
            g.optimizer_step(hp)
        torch.cuda.synchronize()
        out.append([t.clone() for (lin, _, _, _), pl, (_, _, Y, Z, dX) in zip(cases, pls, bufs)
                    for t in (pl.thetaR, pl.thetaP, pl.mR, pl.vP, Y[:, :lin.m], Z[:, :lin.m], dX[:, :lin.n])])
    for i, (a, b) in enumerate(zip(*out)):
        assert torch.equal(a, b), f"state {i} ({SPECS[i // 7][0]}) differs from one call per step"


def test_shared_side_stream_stack_then_merge_matches_one_call():
    """Two groups (layers) sharing one workspace and one side stream with its workspace, as a stack runs them:
    forward through both, backward in reverse with finish_backward(join=False) and the update per layer, two steps,
    then a merge of each group. theta, moments, outputs and the merged W0 equal those of groups that make one call
    per step on the launch stream, bit for bit."""
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("fold: two layers sharing one side stream, pipelined, then merge")
    specs = SPECS[:4]
    layers = [[_linear(spec, 10 * l + i) for i, spec in enumerate(specs)] for l in range(2)]
    hp = B.adamw(lr=1e-3)
    out = []
    for use in (2, 3):  # the same linears twice: tuple slot 2 and slot 3 of each case
        open_ = use == 3
        pls = [[c[use] for c in cs] for cs in layers]
        ws = torch.empty(max(PoetGroup.workspace_bytes(p, open_, [2, 3] if open_ else None) for p in pls),
                         dtype=torch.uint8, device="cuda")
        side = None
        if open_:
            sneed = max(PoetGroup.side_workspace_bytes(p, [2, 3]) for p in pls)
            side = (torch.cuda.Stream(), torch.empty(sneed, dtype=torch.uint8, device="cuda"))
        groups = [PoetGroup(p, ws=ws, side_linears=[2, 3], side=side) if open_ else
                  PoetGroup(p, ws=ws, side_chains=False) for p in pls]
        bufs = [[(put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldy),
                  pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx))
                 for (lin, (W0, tR, tP, X, dY), _, _), pl in zip(cs, p)] for cs, p in zip(layers, pls)]
        for _ in range(2):
            for g, p, b in zip(groups, pls, bufs):
                g.build()
                for pl, (Xd, dYd, Y, Z, dX) in zip(p, b):
                    pl.forward_act(Xd, Y, Z)
            for g, p, b in zip(reversed(groups), reversed(pls), reversed(bufs)):
                for pl, (Xd, dYd, Y, Z, dX) in zip(reversed(p), reversed(b)):
                    pl.backward_act_prims(Xd, Z, dYd, dX)
                g.finish_backward(join=not open_)
                g.optimizer_step(hp)
        state = [t.clone() for p, b in zip(pls, bufs) for pl, (_, _, Y, Z, dX) in zip(p, b)
                 for t in (pl.thetaR, pl.thetaP, pl.mR, pl.vP, Y[:, :pl.m], Z[:, :pl.m], dX[:, :pl.n])]
        for g in groups:
            g.build()
            g.merge()
        torch.cuda.synchronize()
        out.append(state + [pl.W0.clone() for p in pls for pl in p])
    for i, (a, b) in enumerate(zip(*out)):
        assert torch.equal(a, b), f"state {i} differs from one call per step"
