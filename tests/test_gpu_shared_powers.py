"""Two layers sharing one set of saved-power buffers, as a stack that recomputes the powers in the backward runs
them (bench.py --recompute powers): the forward builds layer 0 then layer 1 (layer 1's build overwrites the shared
powers), and the backward rebuilds each layer with PoetGroup.build(again=True) before its backward, which forms the
powers again and keeps the folds and formed FS operands of the forward's build. dtheta must equal that of the same
two layers with powers of their own, bit for bit, on the activation side (folded BS) and on the weight side (FS pairs
formed in the build)."""
import pytest

import poet_inputs as PI
from tests.gpu_util import announce, make_linear, oracle_indices, put_act

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _layers(mode, share):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    if mode == PI.MODE_BS:
        spec, path, T = (520, 384, 256, 128, 5), "act", 600
    else:
        spec, path, T = (600, 520, 300, 260, 5), "weight", 256
    m, n, bR, bP, k = spec
    layers = []
    for layer in range(2):
        lin = make_linear(f"l{layer}", m, n, T, mode, bR, bP, k, PI.DT_BF16, linear_id=30 + layer)
        W0, tR, tP, X, dY = PI.gen_linear(70 + layer, 0, lin, theta_std=0.01)
        iR, iP = oracle_indices(lin, 5)
        pl = PoetLinear(m, n, T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP, seed=5,
                        linear_id=lin.linear_id, idxR=iR, idxP=iP, path=path)
        if share and layer == 1:
            pl.powersR, pl.powersP = layers[0]["pl"].powersR, layers[0]["pl"].powersP
        g = PoetGroup([pl], form_fs=mode == PI.MODE_FS)
        keep = pl.alloc_act(T, pl.L.ldy) if path == "act" else None
        layers.append(dict(pl=pl, g=g, X=put_act(pl, X, pl.L.ldx), dY=put_act(pl, dY, pl.L.ldy),
                           Y=pl.alloc_act(T, pl.L.ldy), dX=pl.alloc_act(T, pl.L.ldx), keep=keep))
    return layers


def _step(layers, share):
    for e in layers:
        e["g"].build()
        if e["pl"].act_path:
            e["pl"].forward_act(e["X"], e["Y"], e["keep"])
        else:
            e["pl"].forward(e["X"], e["Y"])
    for e in reversed(layers):
        if share:
            e["g"].build(again=True)
        if e["pl"].act_path:
            e["pl"].backward_act_prims(e["X"], e["keep"], e["dY"], e["dX"])
        else:
            e["pl"].backward_prims(e["X"], e["dY"], e["dX"])
        e["g"].finish_backward()
    torch.cuda.synchronize()
    return [t.clone() for e in layers for t in (e["dX"], e["pl"].dthetaR, e["pl"].dthetaP)]


@pytest.mark.parametrize("mode", [PI.MODE_BS, PI.MODE_FS])
def test_shared_powers_rebuilt_in_the_backward(mode):
    announce(f"shared saved powers, rebuilt in the backward: mode={mode}")
    own = _step(_layers(mode, False), False)
    shared = _step(_layers(mode, True), True)
    for i, (a, b) in enumerate(zip(own, shared)):
        assert torch.equal(a, b), f"output {i} differs with shared, rebuilt powers"
