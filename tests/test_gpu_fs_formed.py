"""POET-FS operands formed in the group build (poet_fs_form, poet_linear_fwd_formed, poet_linear_bwd_formed_prims).

For a weight-side linear with both sides POET-FS, W = R W0 P and the gradient operands Zr = (W0 P)[I_R, :] and
Acp = (R W0)[:, I_P] depend on the primitives and W0 alone, so PoetGroup(form_fs=True) forms them right after the
build, on side streams that overlap the formations of different linears. The forward and backward that read them
run the same kernels on the same values as the forward and backward that form them inline, so:

- W, Y, dX and the primitive gradients (hence dtheta after the grouped adjoint) must equal the inline path's bit for
  bit, for linears spread over two formation streams (three FS linears: one each with a ragged m, with row pitches
  padded beyond n, with s = 520 / 300 GEMM chains) next to a POET-BS weight-side linear the group leaves as it is;
- Y and dtheta also meet the bf16 bar against the oracle;
- the formed operands are dropped by a one-linear build and by a merge, and a forward that asks for W_out is refused;
- a formed grouped step captured into a HIP graph (the fork to the side streams and the join captured with it)
  replays bit for bit like the eager step, three times, with eager work in between;
- with the sides in three classes (s = 520 and s = 300 built as products, the rest on the fused chain), the group
  builds and differentiates the s = 520 class on its side stream beside the rest: Y, dX and dtheta equal those of
  the group that makes one call per step (side_chains=False), bit for bit, formed and inline; so do the merged W0
  and the resampled index sets of a merge, whose build at the merge's precision also splits;
- three training steps with finish_backward(join=False), which leaves the side class's adjoint and AdamW update on
  the side stream into the next step's build, end with the same theta, moments, Y and dX as three steps of the
  group that makes one call per step, bit for bit, formed and inline; so do two layers stepped as a stack that
  share one side stream and every workspace.
"""
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import TOL, announce, check, make_linear, oracle_indices, put_act, theta_groups, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SPECS = [("fs0", 600, 1040, 256, PI.MODE_FS, 300, 520, 5, 0),
         ("fs1", 1040, 600, 256, PI.MODE_FS, 520, 300, 5, 8),
         ("fs2", 512, 384, 200, PI.MODE_FS, 256, 192, 4, 0),
         ("bs", 520, 384, 256, PI.MODE_BS, 256, 128, 4, 0)]


def _block(seed=93):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    out = []
    for i, (name, m, n, T, mode, bR, bP, k, pad) in enumerate(SPECS):
        lin = make_linear(name, m, n, T, mode, bR, bP, k, PI.DT_BF16, linear_id=10 + i)
        W0, tR, tP, X, dY = PI.gen_linear(seed, 0, lin, theta_std=0.01)
        iR, iP = oracle_indices(lin, 17)
        pl = PoetLinear(m, n, T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP, seed=17,
                        linear_id=lin.linear_id, ldw=n + pad, ldx=n + pad, ldy=m + pad, idxR=iR, idxP=iP,
                        path="weight")
        Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
        out.append(dict(lin=lin, pl=pl, W0=W0, tR=tR, tP=tP, X=X, dY=dY, iR=iR, iP=iP, Xd=Xd, dYd=dYd,
                        Y=pl.alloc_act(T, pl.L.ldy), dX=pl.alloc_act(T, pl.L.ldx), W=pl.alloc_W()))
    return out


def _step(group, blk, formed):
    group.build()
    for e in blk:
        pl = e["pl"]
        keep = None if (formed and pl.formed is not None) else e["W"]
        pl.forward(e["Xd"], e["Y"], W_out=keep)
        pl.backward_prims(e["Xd"], e["dYd"], e["dX"], W=keep)
    group.finish_backward()


def _outs(blk):
    """The written parts (row pitches can be padded beyond them)."""
    o = []
    for e in blk:
        pl = e["pl"]
        o += [t.clone() for t in (e["Y"][:, :pl.m], e["dX"][:, :pl.n], pl.dprimR, pl.dprimP, pl.dthetaR,
                                  pl.dthetaP)]
    return o


def _formed_parts(pl):
    W, Zr, Acp = pl.formed
    return [W[:, :pl.n].clone(), Zr[:, :pl.n].clone(), Acp[:, :pl.L.P.b].clone()]


def test_formed_matches_inline_and_oracle():
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("FS formed in the build vs formed inline")
    blk = _block()
    lins = [e["pl"] for e in blk]
    inline = PoetGroup(lins)
    formed = PoetGroup(lins, form_fs=True, form_streams=2)
    assert len(formed._formed) == 3 and len(formed._form_streams) == 2
    _step(inline, blk, False)
    torch.cuda.synchronize()
    want = _outs(blk)
    W_inline = [e["W"].clone() for e in blk]
    for e in blk:
        for t in (e["Y"], e["dX"], e["pl"].dthetaR, e["pl"].dthetaP):  # dtheta is formed from the dprims
            t.fill_(float("nan"))
    _step(formed, blk, True)
    torch.cuda.synchronize()
    got = _outs(blk)
    names = ("Y", "dX", "dprimR", "dprimP", "dthetaR", "dthetaP")
    for i, (a, b) in enumerate(zip(want, got)):
        e = blk[i // len(names)]
        assert torch.equal(a, b), f"{e['lin'].name}: {names[i % len(names)]} differs from the inline path"
    for e, Wi in zip(blk, W_inline):
        pl = e["pl"]
        if pl.formed is None:
            assert e["lin"].name == "bs"
            continue
        assert torch.equal(pl.formed[0][:, :pl.n], Wi[:, :pl.n]), f"{e['lin'].name}: formed W"
    for e in blk:
        lin, pl = e["lin"], e["pl"]
        sR, sP = O.Side.of(lin.R), O.Side.of(lin.P)
        fw = O.linear_fwd(sR, sP, e["W0"], e["tR"], e["tP"], e["iR"], e["iP"], e["X"])
        bw = O.linear_bwd(sR, sP, e["W0"], e["tR"], e["tP"], e["iR"], e["iP"], e["X"], e["dY"])
        nR, nP = len(e["tR"]), len(e["tP"])
        errs = {}
        try:
            check(errs, "Y", to_np(e["Y"])[:, :lin.m], fw["Y"], TOL[PI.DT_BF16])
            check(errs, "dX", to_np(e["dX"])[:, :lin.n], bw["dX"], TOL[PI.DT_BF16])
            check(errs, "dthetaR", to_np(pl.dthetaR)[:nR], bw["dthetaR"], TOL[PI.DT_BF16],
                  theta_groups(lin.R.mode, lin.R.d, lin.R.b))
            check(errs, "dthetaP", to_np(pl.dthetaP)[:nP], bw["dthetaP"], TOL[PI.DT_BF16],
                  theta_groups(lin.P.mode, lin.P.d, lin.P.b))
        finally:
            announce(f"{lin.name} vs oracle: {errs}")


def test_formed_operands_are_dropped_when_stale():
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("FS formed operands: state")
    blk = _block(94)[:2]
    lins = [e["pl"] for e in blk]
    g = PoetGroup(lins, form_fs=True)
    g.build()
    assert all(pl.formed is not None for pl in lins)
    with pytest.raises(ValueError):
        lins[0].forward(blk[0]["Xd"], blk[0]["Y"], W_out=blk[0]["W"])
    lins[0].build()  # a one-linear build does not form them
    assert lins[0].formed is None and lins[1].formed is not None
    g.build()
    g.merge()
    torch.cuda.synchronize()
    assert all(pl.formed is None for pl in lins)


def test_formed_graph_replay_matches_eager():
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("FS formed: graph replay")
    blk = _block(95)
    group = PoetGroup([e["pl"] for e in blk], form_fs=True, form_streams=2)

    def outs():
        o = _outs(blk)
        for e in blk:
            if e["pl"].formed is not None:
                o += _formed_parts(e["pl"])
        return o

    _step(group, blk, True)
    torch.cuda.synchronize()
    eager = outs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(group, blk, True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(group, blk, True)
    for rep in range(3):
        for e in blk:  # eager work between replays: clobber the outputs and the formed operands
            for t in (e["Y"], e["dX"], e["pl"].dthetaR, e["pl"].dthetaP):
                t.fill_(float("nan"))
            if e["pl"].formed is not None:
                for t in e["pl"].formed:
                    t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outs())):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step (output {i})"


def test_side_chains_match_one_call():
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("FS side-class stream vs one grouped call")
    blk = _block(96)
    lins = [e["pl"] for e in blk]
    one = PoetGroup(lins, side_chains=False)
    assert not one._side_idx
    _step(one, blk, False)
    torch.cuda.synchronize()
    want = _outs(blk)
    names = ("Y", "dX", "dprimR", "dprimP", "dthetaR", "dthetaP")
    for form in (False, True):
        g = PoetGroup(lins, form_fs=form)
        assert g._side_idx == [1, 2]  # fs0's P and fs1's R: s = 520
        for e in blk:
            for t in (e["Y"], e["dX"], e["pl"].dthetaR, e["pl"].dthetaP):
                t.fill_(float("nan"))
        _step(g, blk, form)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(want, _outs(blk))):
            e = blk[i // len(names)]
            assert torch.equal(a, b), f"form={form} {e['lin'].name}: {names[i % len(names)]} differs from one call"


def test_side_chains_merge_matches_one_call():
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("FS side-class stream: merge vs one grouped call")
    out = []
    for side_chains in (False, True):
        blk = _block(97)  # the same linears twice
        lins = [e["pl"] for e in blk]
        g = PoetGroup(lins, side_chains=side_chains)
        assert bool(g._side_idx) == side_chains
        g.build()
        g.merge()
        torch.cuda.synchronize()
        out.append([t.clone() for pl in lins for t in (pl.W0, pl.idxR, pl.idxP, pl.thetaR, pl.thetaP)
                    if t is not None])
    assert len(out[0]) == len(out[1])
    for i, (a, b) in enumerate(zip(*out)):
        assert torch.equal(a, b), f"merged state {i} differs from one call"


def test_open_finish_backward_matches_joined_steps():
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("FS side-class stream: steps with the adjoint and update left open vs one call per step")
    hp = B.adamw(lr=1e-3)
    out = {}
    for mode in ("one", "open", "open_formed"):
        blk = _block(98)  # the same linears each time
        lins = [e["pl"] for e in blk]
        form = mode == "open_formed"
        g = PoetGroup(lins, side_chains=mode != "one", form_fs=form)
        for _ in range(3):
            g.build()
            for e in blk:
                pl = e["pl"]
                keep = None if (form and pl.formed is not None) else e["W"]
                pl.forward(e["Xd"], e["Y"], W_out=keep)
                pl.backward_prims(e["Xd"], e["dYd"], e["dX"], W=keep)
            g.finish_backward(join=mode == "one")
            assert g._side_open == (mode != "one")
            g.optimizer_step(hp)
        torch.cuda.synchronize()
        out[mode] = [t.clone() for e in blk for t in (e["pl"].thetaR, e["pl"].thetaP, e["pl"].mR, e["pl"].vP,
                                                        e["Y"][:, :e["pl"].m], e["dX"][:, :e["pl"].n])]
    for mode in ("open", "open_formed"):
        for i, (a, b) in enumerate(zip(out["one"], out[mode])):
            assert torch.equal(a, b), f"{mode}: state {i} differs from one call per step"


def test_shared_side_stream_layers_match_one_call():
    """Two layers (groups) of FS linears sharing one workspace, the formation workspaces, and one side stream with
    its workspace, stepped as a stack: forward through both (FS operands formed in each build), backward in reverse
    with finish_backward(join=False) and the update per layer, two steps. theta, moments, Y and dX equal those of
    groups making one call per step with inline formation, bit for bit."""
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup
    announce("FS: two layers sharing one side stream, pipelined")
    hp = B.adamw(lr=1e-3)
    out = []
    for open_ in (False, True):
        layers = [_block(99)[:3], _block(100)[:3]]  # the FS linears of two blocks
        pls = [[e["pl"] for e in blk] for blk in layers]
        ws = torch.empty(max(PoetGroup.workspace_bytes(p, open_) for p in pls), dtype=torch.uint8, device="cuda")
        kw = {}
        if open_:
            fneed = max(PoetGroup.form_workspace_bytes(p) for p in pls)
            sneed = max(PoetGroup.side_workspace_bytes(p) for p in pls)
            kw = dict(form_fs=True, form_ws=[torch.empty(fneed, dtype=torch.uint8, device="cuda") for _ in range(2)],
                      side=(torch.cuda.Stream(), torch.empty(sneed, dtype=torch.uint8, device="cuda")))
        groups = [PoetGroup(p, ws=ws, side_chains=open_, **kw) for p in pls]
        assert all(bool(g._side_idx) == open_ for g in groups)
        for _ in range(2):
            for g, blk in zip(groups, layers):
                g.build()
                for e in blk:
                    pl = e["pl"]
                    pl.forward(e["Xd"], e["Y"], W_out=None if pl.formed is not None else e["W"])
            for g, blk in zip(reversed(groups), reversed(layers)):
                for e in reversed(blk):
                    pl = e["pl"]
                    pl.backward_prims(e["Xd"], e["dYd"], e["dX"], W=None if pl.formed is not None else e["W"])
                g.finish_backward(join=not open_)
                g.optimizer_step(hp)
        torch.cuda.synchronize()
        out.append([t.clone() for blk in layers for e in blk
                    for t in (e["pl"].thetaR, e["pl"].thetaP, e["pl"].mR, e["pl"].vP, e["Y"][:, :e["pl"].m],
                              e["dX"][:, :e["pl"].n])])
    for i, (a, b) in enumerate(zip(*out)):
        assert torch.equal(a, b), f"state {i} differs from one call per step"
