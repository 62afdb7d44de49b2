"""poet_merge_group: merge-then-reinitialize of several weights in shared launches.

The group holds block-diagonal weights of all three k-step classes of the in-place passes (blocks up to 64, 128 and
256), ragged last blocks, blocks that are not a multiple of 8 (no float4 loads), padded rows, bf16 and float32
shadows and no shadow, plus two weights outside the in-place path (FS sides, and a block above 256). Each is
checked against poet_merge on an identical copy (bitwise: per element the grouped launches do the same
arithmetic) and against the oracle's W0 <- R W0 P (float32 bar) and fresh index sets (exact).
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import announce, check, make_linear, rel, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SEED = 11

# name, m, n, mode, bR, bP, k, act dtype, side dtype, row padding, path, theta std
SPECS = [
    ("q", 520, 384, PI.MODE_BS, 256, 128, 3, PI.DT_BF16, PI.DT_F32, 0, "act", 0.02),
    ("gate", 700, 520, PI.MODE_BS, 256, 256, 3, PI.DT_BF16, PI.DT_F32, 6, "act", 0.02),
    ("small", 257, 129, PI.MODE_BS, 64, 36, 3, PI.DT_F32, PI.DT_F32, 3, "weight", 0.02),
    ("fs", 300, 260, PI.MODE_FS, 150, 130, 3, PI.DT_BF16, PI.DT_BF16, 0, "weight", PI.THETA_STD),
    ("big", 600, 320, PI.MODE_BS, 300, 64, 2, PI.DT_F32, PI.DT_F32, 0, "weight", 0.01),
    ("down", 384, 700, PI.MODE_BS, 128, 256, 3, PI.DT_BF16, PI.DT_F32, 4, "act", 0.02),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _copies(spec, linear_id):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetLinear
    name, m, n, mode, bR, bP, k, dt, sdt, pad, path, std = spec
    lin = make_linear(name, m, n, 16, mode, bR, bP, k, dt, linear_id=linear_id, side_dt=sdt)
    W0, tR, tP, _, _ = PI.gen_linear(0, 0, lin, theta_std=std)

    def mk():
        return PoetLinear(m, n, 16, B.side_of(lin.R), B.side_of(lin.P), dt, W0, tR, tP, seed=SEED,
                          linear_id=linear_id, ldw=n + pad, ldx=n + pad, ldy=m + pad, path=path)
    return lin, mk(), mk(), (W0, tR, tP)


def test_merge_group_matches_per_weight_merges_and_oracle():
    from orthogonal_reparameterized_amd.layer import PoetGroup
    cases = [_copies(spec, i) for i, spec in enumerate(SPECS)]
    for lin, one, grp, _ in cases:
        one.build()
        grp.build()
    torch.cuda.synchronize()
    before = [(None if one.idxR is None else one.idxR.cpu().numpy().copy(),
               None if one.idxP is None else one.idxP.cpu().numpy().copy()) for _, one, _, _ in cases]
    announce("merge group: per-weight merges")
    for _, one, _, _ in cases:
        one.merge()
    torch.cuda.synchronize()
    announce("merge group: grouped merge of " + ", ".join(lin.name for lin, _, _, _ in cases))
    PoetGroup([grp for _, _, grp, _ in cases]).merge()
    torch.cuda.synchronize()
    for (lin, one, grp, (W0, tR, tP)), (iR, iP) in zip(cases, before):
        assert torch.equal(grp.W0, one.W0), lin.name
        if one.W0b is not None:  # (the shadow's padding columns are never written)
            assert torch.equal(grp.W0b[:, :lin.n], one.W0b[:, :lin.n]), lin.name
        for a, b in ((grp.idxR, one.idxR), (grp.idxP, one.idxP)):
            assert (a is None) == (b is None) and (a is None or torch.equal(a, b)), lin.name
        assert float(grp.thetaR.abs().max()) == 0.0 and float(grp.thetaP.abs().max()) == 0.0, lin.name
        assert grp.epoch == one.epoch == 1
        mg = O.merge(O.Side.of(lin.R), O.Side.of(lin.P), W0, tR, tP, iR, iP, SEED, lin.linear_id, 1)
        errs = {}
        try:
            check(errs, "W0", to_np(grp.W0)[:, :lin.n], mg["W0"], 1e-5)
        finally:
            announce(f"merge group {lin.name}: {errs}")
        if grp.W0b is not None:  # the shadow is the merged W0 in the act dtype
            ref = torch.from_numpy(to_np(grp.W0)).to(grp.W0b.dtype)
            assert torch.equal(grp.W0b.cpu()[:, :lin.n], ref[:, :lin.n]), lin.name
        for got, want in ((grp.idxR, mg["idxR"]), (grp.idxP, mg["idxP"])):
            if want is not None:
                assert np.array_equal(got.cpu().numpy(), want), lin.name


def test_merge_group_of_one_equals_merge():
    """A group of one block-diagonal weight takes the same launches as poet_merge."""
    from orthogonal_reparameterized_amd.layer import PoetGroup
    lin, one, grp, _ = _copies(SPECS[1], 4)
    one.build()
    grp.build()
    one.merge()
    PoetGroup([grp]).merge()
    torch.cuda.synchronize()
    assert torch.equal(grp.W0, one.W0) and torch.equal(grp.W0b[:, :lin.n], one.W0b[:, :lin.n])
