"""GPU checks of the grouped calls through the C ABI: poet_build_orthogonal_group, poet_linear_bwd_act_prims and
poet_adjoint_group.

The grouped build runs the same per-block arithmetic as the one-side build, so its primitives and saved powers
must equal those of poet_build_orthogonal bit for bit, for every kind of side (fused-chain sides that share the
launches, and sides the group hands to the one-side path). The grouped adjoint is checked against the oracle's
Neumann adjoint and skew projection on the same primitive gradients (bar: 1e-5 relative for float32 sides,
2e-2 for bf16 sides), and a block of linears run with backward_act_prims + finish_backward must reproduce the
per-linear backward (the adjoint's split-K summation order may differ, hence a 1e-5 relative bar rather than
equality).
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import TOL, announce, check, make_linear, put_act, rel, theta_groups, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (mode, d, b, k, dtype): fused-chain sides of several block sizes (one ragged), an FS side; sides whose chain runs as
# grouped GEMMs (FS primitives of 1050 and 300, padded row pitch; BS blocks of 512, ragged); and sides the group
# leaves to the one-side path (float32, a block of 100) or that need no chain (k = 0)
SIDES = [
    (PI.MODE_BS, 520, 256, 5, PI.DT_BF16),
    (PI.MODE_BS, 384, 128, 4, PI.DT_BF16),
    (PI.MODE_BS, 200, 64, 3, PI.DT_BF16),
    (PI.MODE_FS, 300, 128, 5, PI.DT_BF16),
    (PI.MODE_FS, 2100, 1050, 5, PI.DT_BF16),
    (PI.MODE_FS, 4000, 1050, 5, PI.DT_BF16),
    (PI.MODE_FS, 700, 300, 5, PI.DT_BF16),
    (PI.MODE_BS, 1100, 512, 2, PI.DT_BF16),
    (PI.MODE_BS, 200, 64, 3, PI.DT_F32),
    (PI.MODE_BS, 300, 100, 2, PI.DT_BF16),
    (PI.MODE_BS, 256, 64, 0, PI.DT_BF16),
]
# sides whose chain runs as GEMMs: the grouped launches may split K differently from a one-side build, so those
# results agree to the float32 summation order, not bit for bit
GEMM_CHAIN = {i for i, (mode, d, b, k, dt) in enumerate(SIDES) if dt == PI.DT_BF16 and k > 0 and b >= 128 and
              (b > 256 or b % 8)}


def _sides():
    from orthogonal_reparameterized_amd import binding as B
    return [B.side(*s) for s in SIDES]


def _thetas(std, seed=5):
    """Skew parameters of every side at standard deviation std, capped at 0.25 / sqrt(b) so that ||Q||_2 (about
    2 std sqrt(b)) stays near 0.5: the truncated series converges, and summation-order differences between launch
    shapes are not amplified by a diverging chain."""
    rng = np.random.default_rng(seed)
    out = []
    for mode, d, b, k, dt in SIDES:
        n = PI.n_theta(PI.SideSpec(mode, d, b, k, dt))
        out.append((rng.standard_normal(n) * min(std, 0.25 / np.sqrt(b))).astype(np.float32))
    return out


def B_prim_len(s):
    from orthogonal_reparameterized_amd import binding as B
    return B.poet_prim_len(s)


def _alloc(s):
    from orthogonal_reparameterized_amd import binding as B
    dt = torch.bfloat16 if s.dtype == B.POET_BF16 else torch.float32
    prim = torch.zeros(B.poet_prim_len(s), dtype=torch.float32, device="cuda")
    powers = torch.zeros(max(B.poet_powers_len(s), 1), dtype=dt, device="cuda") if s.k > 0 else None
    return prim, powers


def _build_all(sides, thetas_d, grouped, ops=None):
    from orthogonal_reparameterized_amd import binding as B
    bufs = [_alloc(s) for s in sides]
    if grouped:
        B.poet_build_orthogonal_group(sides, thetas_d, [b[0] for b in bufs], [b[1] for b in bufs], ops=ops)
    else:
        for s, th, (prim, pw) in zip(sides, thetas_d, bufs):
            B.poet_build_orthogonal(s, th, prim, pw)
    torch.cuda.synchronize()
    return bufs


def _operand_order(M):
    """Blocks M[p] (b x b) flattened as the library stores its operand copies: row-major, or, for b a multiple of
    32, M(i, j) at ((i // 32 * b // 16 + j // 16) * 64 + (j // 8 % 2) * 32 + i % 32) * 8 + j % 8."""
    nb, b, _ = M.shape
    if b % 32:
        return M.reshape(nb, b * b)
    i, j = np.meshgrid(np.arange(b), np.arange(b), indexing="ij")
    pos = ((i // 32 * (b // 16) + j // 16) * 64 + (j // 8 % 2) * 32 + i % 32) * 8 + j % 8
    out = np.empty((nb, b * b), dtype=M.dtype)
    out[:, pos.ravel()] = M.reshape(nb, b * b)
    return out


def test_build_group_equals_one_side_builds():
    announce("group build vs one-side builds")
    sides = _sides()
    thetas_d = [torch.from_numpy(t).cuda() for t in _thetas(0.02)]
    single = _build_all(sides, thetas_d, grouped=False)
    # operand copies for the BS sides (written by the chain kernel, or by the conversion for the other sides)
    ops = [torch.full((3 * B_prim_len(s),), float("nan"), dtype=torch.bfloat16, device="cuda") if spec[0] == PI.MODE_BS
           else None for spec, s in zip(SIDES, sides)]
    group = _build_all(sides, thetas_d, grouped=True, ops=ops)
    for i, ((pa, wa), (pb, wb)) in enumerate(zip(single, group)):
        if i in GEMM_CHAIN:
            eye = np.eye(SIDES[i][2]).ravel()
            d = (to_np(pa).reshape(-1, eye.size) - eye).ravel()
            assert rel(to_np(pb).reshape(-1, eye.size) - eye, d.reshape(-1, eye.size)) <= 1e-4, f"prim of side {i}"
            assert rel(to_np(wb), to_np(wa)) <= 1e-2, f"powers of side {i}"
        else:
            assert torch.equal(pa, pb), f"prim of side {i} {SIDES[i]}"
            if wa is not None:
                assert torch.equal(wa, wb), f"powers of side {i} {SIDES[i]}"
        if ops[i] is None:
            continue
        # ops = bf16(F - I) and bf16((F - I)^T) per block, zero outside the block's c x c corner, bit for bit (the
        # float32 subtraction of 1 from a diagonal entry near 1 is exact)
        mode, d, b, k, dt = SIDES[i]
        F = to_np(pa).reshape(-1, b, b)
        D = F - np.eye(b, dtype=np.float32)
        want = np.zeros_like(F)
        for p, c in enumerate(O.block_sizes(mode, d, b)):
            want[p, :c, :c] = PI.round_bf16(D[p, :c, :c])
        got = to_np(ops[i]).reshape(3, -1, b * b)
        np.testing.assert_array_equal(got[0], _operand_order(want), err_msg=f"ops of side {i} {SIDES[i]}")
        np.testing.assert_array_equal(got[1], _operand_order(want.transpose(0, 2, 1)),
                                      err_msg=f"transposed ops of side {i}")
        # the third part: the delta of the whole padded block (zero in the identity padding), row-major
        np.testing.assert_array_equal(got[2], PI.round_bf16(D).reshape(-1, b * b), err_msg=f"row ops of side {i}")


def _oracle_dtheta(side_spec, theta, dprim):
    mode, d, b, k, dt = side_spec
    out, off = [], 0
    for p, c in enumerate(O.block_sizes(mode, d, b)):
        nt = c * (c - 1) // 2
        Q = O.skew_from_theta(theta[off:off + nt].astype(np.float64), c)
        dR = dprim[p * b * b:(p + 1) * b * b].reshape(b, b)[:c, :c].astype(np.float64)
        out.append(O.skew_project(O.neumann_adjoint(Q, dR, k)))
        off += nt
    return np.concatenate(out) if out else np.zeros(0)


@pytest.mark.parametrize("std", [1e-3, 0.02])
def test_adjoint_group_against_oracle(std):
    from orthogonal_reparameterized_amd import binding as B
    announce(f"group adjoint vs oracle theta std {std}")
    sides = _sides()
    thetas = _thetas(std, seed=7)
    thetas_d = [torch.from_numpy(t).cuda() for t in thetas]
    bufs = _build_all(sides, thetas_d, grouped=True)
    rng = np.random.default_rng(11)
    dprims, dprims_d, dthetas_d = [], [], []
    for spec, s in zip(SIDES, sides):
        g = rng.standard_normal(B.poet_prim_len(s)).astype(np.float32)
        dprims.append(g)
        dprims_d.append(torch.from_numpy(g).cuda())
        dthetas_d.append(torch.full((max(B.poet_theta_len(s), 1),), float("nan"), device="cuda"))
    B.poet_adjoint_group(sides, dprims_d, [b[1] for b in bufs], dthetas_d)
    torch.cuda.synchronize()
    for i, spec in enumerate(SIDES):
        n = B.poet_theta_len(sides[i])
        ref = _oracle_dtheta(spec, thetas[i], dprims[i])
        errs = {}
        try:
            check(errs, "dtheta", to_np(dthetas_d[i])[:n], ref, TOL[spec[4]], theta_groups(spec[0], spec[1], spec[2]))
        finally:
            announce(f"side {spec}: {errs}")


def test_block_backward_grouped_matches_per_linear():
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    announce("grouped block backward vs per-linear backward")
    specs = [make_linear("q", 520, 384, 300, PI.MODE_BS, 256, 128, 5, PI.DT_BF16, linear_id=0),
             make_linear("gate", 600, 520, 300, PI.MODE_BS, 256, 256, 5, PI.DT_BF16, linear_id=4),
             make_linear("small", 256, 192, 300, PI.MODE_BS, 64, 48, 3, PI.DT_BF16, linear_id=2)]
    lins, acts, refs = [], [], []
    for lin in specs:
        W0, tR, tP, X, dY = PI.gen_linear(98, 0, lin, theta_std=0.01)
        pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                        linear_id=lin.linear_id, path="act")
        lins.append(pl)
        Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
        acts.append((Xd, dYd, pl.alloc_act(lin.T, pl.L.ldy), pl.alloc_act(lin.T, pl.L.ldy),
                     pl.alloc_act(lin.T, pl.L.ldx)))
        sR, sP = O.Side.of(lin.R), O.Side.of(lin.P)
        refs.append(O.linear_bwd(sR, sP, W0, tR, tP, None, None, X, dY))
    group = PoetGroup(lins)
    # per-linear build and backward
    for pl, (Xd, dYd, Y, Z, dX) in zip(lins, acts):
        pl.build()
        pl.forward_act(Xd, Y, Z)
        pl.backward_act(Xd, Z, dYd, dX)
    torch.cuda.synchronize()
    per = [(pl.primR.clone(), pl.primP.clone(), pl.dthetaR.clone(), pl.dthetaP.clone(), a[4].clone())
           for pl, a in zip(lins, acts)]
    # grouped build, per-linear backward to the primitive gradients, grouped adjoint
    for pl in lins:
        pl.dthetaR.fill_(float("nan"))
        pl.dthetaP.fill_(float("nan"))
    group.build()
    for pl, (Xd, dYd, Y, Z, dX) in zip(lins, acts):
        pl.forward_act(Xd, Y, Z)
        pl.backward_act_prims(Xd, Z, dYd, dX)
    group.finish_backward()
    torch.cuda.synchronize()
    for pl, lin, a, p, ref in zip(lins, specs, acts, per, refs):
        assert torch.equal(pl.primR, p[0]) and torch.equal(pl.primP, p[1]), lin.name
        assert torch.equal(a[4], p[4]), lin.name  # dX does not depend on the grouping
        nR, nP = B.poet_theta_len(pl.L.R), B.poet_theta_len(pl.L.P)
        eR = rel(to_np(pl.dthetaR)[:nR], to_np(p[2])[:nR])
        eP = rel(to_np(pl.dthetaP)[:nP], to_np(p[3])[:nP])
        announce(f"{lin.name}: grouped vs per-linear {eR:.2e} {eP:.2e}")
        assert eR <= 1e-5 and eP <= 1e-5, (lin.name, eR, eP)
        errs = {}
        try:
            check(errs, "dthetaR", to_np(pl.dthetaR)[:nR], ref["dthetaR"], TOL[PI.DT_BF16],
                  theta_groups(lin.R.mode, lin.R.d, lin.R.b))
            check(errs, "dthetaP", to_np(pl.dthetaP)[:nP], ref["dthetaP"], TOL[PI.DT_BF16],
                  theta_groups(lin.P.mode, lin.P.d, lin.P.b))
        finally:
            announce(f"{lin.name} vs oracle: {errs}")


def test_block_backward_grouped_matches_per_linear_weight_path_fs():
    """Weight-side linears with FS sides (s = 300 and 520 per side, GEMM chains) and one BS linear: grouped build,
    backward to the primitive gradients and grouped adjoint against the per-linear calls and the oracle."""
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    from tests.gpu_util import oracle_indices
    announce("grouped block backward, weight side, FS")
    specs = [make_linear("fs0", 600, 1040, 256, PI.MODE_FS, 300, 520, 5, PI.DT_BF16, linear_id=7),
             make_linear("fs1", 1040, 600, 256, PI.MODE_FS, 520, 300, 5, PI.DT_BF16, linear_id=8),
             make_linear("bs", 520, 384, 256, PI.MODE_BS, 256, 128, 4, PI.DT_BF16, linear_id=9)]
    lins, data = [], []
    for lin in specs:
        W0, tR, tP, X, dY = PI.gen_linear(94, 0, lin, theta_std=0.01)
        iR, iP = oracle_indices(lin, 17)
        pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP, seed=17,
                        linear_id=lin.linear_id, idxR=iR, idxP=iP, path="weight")
        Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
        lins.append(pl)
        data.append((lin, W0, tR, tP, X, dY, iR, iP, Xd, dYd, pl.alloc_act(lin.T, pl.L.ldy),
                     pl.alloc_act(lin.T, pl.L.ldx), pl.alloc_W()))
    group = PoetGroup(lins)
    for pl, (lin, W0, tR, tP, X, dY, iR, iP, Xd, dYd, Y, dX, W) in zip(lins, data):
        pl.build()
        pl.forward(Xd, Y, W_out=W)
        pl.backward(Xd, dYd, dX, W=W)
    torch.cuda.synchronize()
    per = [(pl.dthetaR.clone(), pl.dthetaP.clone(), d[11].clone()) for pl, d in zip(lins, data)]
    for pl in lins:
        pl.dthetaR.fill_(float("nan"))
        pl.dthetaP.fill_(float("nan"))
    group.build()
    for pl, (lin, W0, tR, tP, X, dY, iR, iP, Xd, dYd, Y, dX, W) in zip(lins, data):
        pl.forward(Xd, Y, W_out=W)
        pl.backward_prims(Xd, dYd, dX, W=W)
    group.finish_backward()
    torch.cuda.synchronize()
    for pl, p, (lin, W0, tR, tP, X, dY, iR, iP, Xd, dYd, Y, dX, W) in zip(lins, per, data):
        ref = O.linear_bwd(O.Side.of(lin.R), O.Side.of(lin.P), W0, tR, tP, iR, iP, X, dY)
        nR, nP = B.poet_theta_len(pl.L.R), B.poet_theta_len(pl.L.P)
        eR, eP = rel(to_np(pl.dthetaR)[:nR], to_np(p[0])[:nR]), rel(to_np(pl.dthetaP)[:nP], to_np(p[1])[:nP])
        eX = rel(to_np(dX)[:, :lin.n], to_np(p[2])[:, :lin.n])
        announce(f"{lin.name}: grouped vs per-linear {eR:.2e} {eP:.2e} dX {eX:.2e}")
        assert eR <= 1e-3 and eP <= 1e-3 and eX <= 1e-3, (lin.name, eR, eP, eX)
        errs = {}
        try:
            check(errs, "dthetaR", to_np(pl.dthetaR)[:nR], ref["dthetaR"], TOL[PI.DT_BF16],
                  theta_groups(lin.R.mode, lin.R.d, lin.R.b))
            check(errs, "dthetaP", to_np(pl.dthetaP)[:nP], ref["dthetaP"], TOL[PI.DT_BF16],
                  theta_groups(lin.P.mode, lin.P.d, lin.P.b))
        finally:
            announce(f"{lin.name} vs oracle: {errs}")
