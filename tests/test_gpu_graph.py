"""HIP graph capture of one POET step: a step (build, forward, backward of a linear on either path) captured on a
side stream with torch's CUDAGraph, replayed several times with eager work and synchronization between the
replays; every replay must reproduce the eager step bit for bit (the library issues only kernel launches, so the
graph holds no memset or copy nodes)."""
import pytest

import poet_inputs as PI
from tests.gpu_util import announce, make_linear, put_act

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("path", ["act", "weight"])
def test_graph_replay_matches_eager(path):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    lin = make_linear(f"graph-{path}", 520, 384, 700, PI.MODE_BS, 256, 128, 4, PI.DT_BF16, linear_id=3)
    announce(f"graph replay path={path}")
    W0, tR, tP, X, dY = PI.gen_linear(96, 0, lin)
    pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP, path=path)
    Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
    Y, dX = pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx)
    keep = pl.alloc_act(lin.T, pl.L.ldy) if path == "act" else pl.alloc_W()

    def step():
        pl.build()
        if path == "act":
            pl.forward_act(Xd, Y, keep)
            pl.backward_act(Xd, keep, dYd, dX)
        else:
            pl.forward(Xd, Y, W_out=keep)
            pl.backward(Xd, dYd, dX, W=keep)

    outs = lambda: [t.clone() for t in (pl.primR, pl.primP, Y, dX, pl.dthetaR, pl.dthetaP)]  # noqa: E731
    step()
    torch.cuda.synchronize()
    eager = outs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (Y, dX, pl.dthetaR, pl.dthetaP):  # eager work between replays: clobber the outputs
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs()):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"


def test_graph_replay_grouped_block_matches_eager():
    """The grouped step (one build and one adjoint over the sides of two linears, with the operand copies the build
    writes) captured and replayed the same way."""
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    announce("graph replay grouped block")
    specs = [make_linear("graph-g0", 520, 384, 700, PI.MODE_BS, 256, 128, 4, PI.DT_BF16, linear_id=1),
             make_linear("graph-g1", 384, 520, 700, PI.MODE_BS, 128, 256, 4, PI.DT_BF16, linear_id=5)]
    lins, bufs = [], []
    for lin in specs:
        W0, tR, tP, X, dY = PI.gen_linear(95, 0, lin)
        pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                        linear_id=lin.linear_id, path="act")
        lins.append(pl)
        bufs.append((put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldy),
                     pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldx)))
    group = PoetGroup(lins)

    def step():
        group.build()
        for pl, (Xd, dYd, Y, Z, dX) in zip(lins, bufs):
            pl.forward_act(Xd, Y, Z)
            pl.backward_act_prims(Xd, Z, dYd, dX)
        group.finish_backward()

    def outs():
        o = []
        for pl, (Xd, dYd, Y, Z, dX) in zip(lins, bufs):
            o += [t.clone() for t in (pl.primR, pl.primP, pl.opsR, pl.opsP, Y, dX, pl.dthetaR, pl.dthetaP)]
        return o

    step()
    torch.cuda.synchronize()
    eager = outs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for pl, (Xd, dYd, Y, Z, dX) in zip(lins, bufs):
            for t in (Y, dX, pl.dthetaR, pl.dthetaP, pl.opsR, pl.opsP):
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outs())):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step (output {i})"
