"""Pins of the CPU oracle against facts fixed outside it (closed forms, textbook routines, finite differences,
published generator outputs, and the parameter counts printed on the POET summary page).

Each pin is chosen so that a plausible mistake in the oracle (a dropped Neumann term, a wrong sign, a transposed
operand, a misplaced block) fails at least one of them; ``test_oracle_mutations.py`` plants such mistakes and
checks that they are caught.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_skew(rng, c, norm2):
    A = np.triu(rng.standard_normal((c, c)), 1)
    Q = A - A.T
    return Q * (norm2 / np.linalg.norm(Q, 2)) if c > 1 else Q


def rot(phi):
    return np.array([[np.cos(phi), np.sin(phi)], [-np.sin(phi), np.cos(phi)]])


# ---------------------------------------------------------------- P1: Q = 0 gives the identity, W = W0 bitwise
@pytest.mark.parametrize("k", range(0, 7))
def test_q_zero_identity(k):
    for c in (1, 2, 5, 33):
        assert np.array_equal(O.cayley_neumann(np.zeros((c, c)), k), np.eye(c))


@pytest.mark.parametrize("mode", [O.MODE_BS, O.MODE_FS, O.MODE_BSP])
def test_q_zero_layer_is_w0(mode):
    rng = np.random.default_rng(1)
    m, n, T = 12, 10, 7
    W0 = rng.standard_normal((m, n))
    X = rng.standard_normal((T, n))
    bR, bP = (6, 5) if mode == O.MODE_FS else (5, 4)
    sR, sP = O.Side(mode, m, bR, 3), O.Side(mode, n, bP, 3)
    idxR = idxP = None
    if mode == O.MODE_FS:
        idxR, idxP = O.sample_indices(m, bR, 7, 0, 0, 0), O.sample_indices(n, bP, 7, 0, 1, 0)
    elif mode == O.MODE_BSP:
        idxR, idxP = O.sample_permutation(m, 7, 0, 0, 0), O.sample_permutation(n, 7, 0, 1, 0)
    out = O.linear_fwd(sR, sP, W0, np.zeros(O.theta_len(mode, m, bR)), np.zeros(O.theta_len(mode, n, bP)),
                       idxR, idxP, X)
    assert np.array_equal(out["W"], W0)
    assert np.array_equal(out["Y"], X @ W0.T)


# ---------------------------------------------------------------- P2: 2 x 2 worked example
def test_2x2_golden_values():
    g = json.load(open(os.path.join(GOLD, "cayley_2x2.json")))
    t = g["t"]
    Q = O.skew_from_theta(np.array([t]), 2)
    assert np.array_equal(Q, np.array([[0.0, t], [-t, 0.0]]))
    for k, R in g["R_k"].items():
        np.testing.assert_allclose(O.cayley_neumann(Q, int(k)), np.array(R), rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.cayley_exact(Q), np.array(g["cayley"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("t", [0.1, 0.3, -0.5, 0.9])
@pytest.mark.parametrize("k", range(0, 9))
def test_2x2_distance_to_rotation(t, k):
    # the exact Cayley map of [[0,t],[-t,0]] is the rotation by 2 atan t; the truncated map is off by |t|^(k+1)
    Q = O.skew_from_theta(np.array([t]), 2)
    R = O.cayley_neumann(Q, k)
    err = np.linalg.norm(R - rot(2 * np.arctan(t)), 2)
    assert err == pytest.approx(abs(t) ** (k + 1), rel=1e-12, abs=1e-15)


# ---------------------------------------------------------------- P3: closed forms of the truncation error
@pytest.mark.parametrize("k", range(0, 7))
@pytest.mark.parametrize("c", [3, 16, 31])
def test_truncation_closed_forms(k, c):
    rng = np.random.default_rng(100 + c + k)
    Q = rand_skew(rng, c, 0.6)
    Rk = O.cayley_neumann(Q, k)
    Rc = O.cayley_exact(Q)
    qn = np.linalg.norm(Q, 2)
    assert np.linalg.norm(Rk - Rc, 2) == pytest.approx(qn ** (k + 1), rel=1e-9)
    Qk1 = np.linalg.matrix_power(Q, k + 1)
    Q2k2 = np.linalg.matrix_power(Q, 2 * k + 2)
    expect = -Q2k2 if k % 2 == 0 else (-2 * Qk1 + Q2k2)
    np.testing.assert_allclose(Rk.T @ Rk - np.eye(c), expect, rtol=0, atol=1e-13)
    # singular values of R_k are |1 - (i lambda)^(k+1)| over the eigenvalues i lambda of Q
    ev = np.linalg.eigvals(Q)
    sv_expect = np.sort(np.abs(1 - ev ** (k + 1)))
    np.testing.assert_allclose(np.sort(np.linalg.svd(Rk, compute_uv=False)), sv_expect, rtol=0, atol=1e-13)


def test_orthogonality_error_shrinks_within_parity():
    rng = np.random.default_rng(5)
    Q = rand_skew(rng, 32, 0.3)
    errs = [np.linalg.norm(O.cayley_neumann(Q, k).T @ O.cayley_neumann(Q, k) - np.eye(32)) for k in range(8)]
    for k in range(2, 8):
        assert errs[k] < errs[k - 2]


# ---------------------------------------------------------------- P5: k -> infinity reaches the exact Cayley
@pytest.mark.parametrize("c", [2, 9, 40])
def test_limit_is_exact_cayley(c):
    rng = np.random.default_rng(c)
    Q = rand_skew(rng, c, 0.5)
    np.testing.assert_allclose(O.cayley_neumann(Q, 80), O.cayley_exact(Q), rtol=0, atol=1e-14)
    Rc = O.cayley_exact(Q)
    np.testing.assert_allclose(Rc.T @ Rc, np.eye(c), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P4: spectrum preservation
def _layer_case(mode, m, n, bR, bP, k, seed, scale):
    rng = np.random.default_rng(seed)
    W0 = rng.standard_normal((m, n))
    W0 /= np.linalg.norm(W0, axis=1, keepdims=True)
    sR, sP = O.Side(mode, m, bR, k), O.Side(mode, n, bP, k)
    tR = rng.standard_normal(O.theta_len(mode, m, bR)) * scale
    tP = rng.standard_normal(O.theta_len(mode, n, bP)) * scale
    idxR = idxP = None
    if mode == O.MODE_FS:
        idxR = O.sample_indices(m, bR, seed, 3, O.SIDE_R, 0)
        idxP = O.sample_indices(n, bP, seed, 3, O.SIDE_P, 0)
    elif mode == O.MODE_BSP:
        idxR = O.sample_permutation(m, seed, 3, O.SIDE_R, 0)
        idxP = O.sample_permutation(n, seed, 3, O.SIDE_P, 0)
    return sR, sP, W0, tR, tP, idxR, idxP


@pytest.mark.parametrize("mode,bR,bP", [(O.MODE_BS, 4, 3), (O.MODE_BS, 12, 10), (O.MODE_FS, 6, 5),
                                        (O.MODE_BSP, 4, 3)])
def test_spectrum_preserved_layer(mode, bR, bP):
    m, n = 12, 10
    # with enough terms the factors are orthogonal to roundoff and the spectrum is kept exactly
    sR, sP, W0, tR, tP, iR, iP = _layer_case(mode, m, n, bR, bP, 60, 11, 0.1)
    W = O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, np.zeros((1, n)))["W"]
    np.testing.assert_allclose(np.linalg.svd(W, compute_uv=False), np.linalg.svd(W0, compute_uv=False),
                               rtol=0, atol=1e-13)
    # with few terms the singular values stay inside the product bounds of the factors' extreme values
    for k in (0, 1, 2, 5):
        sR, sP, W0, tR, tP, iR, iP = _layer_case(mode, m, n, bR, bP, k, 12, 0.1)
        o = O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, np.zeros((1, n)))
        sw = np.linalg.svd(o["W"], compute_uv=False)
        s0 = np.linalg.svd(W0, compute_uv=False)
        rs = np.linalg.svd(o["R"], compute_uv=False)
        ps = np.linalg.svd(o["P"], compute_uv=False)
        assert np.all(sw <= s0 * rs.max() * ps.max() * (1 + 1e-13))
        assert np.all(sw >= s0 * rs.min() * ps.min() * (1 - 1e-13))


def test_fs_assembly_is_permuted_block():
    # F = identity with G on [idx, idx] equals Pi^T blockdiag(G, I) Pi for a permutation Pi listing idx first
    rng = np.random.default_rng(3)
    d, s = 11, 5
    idx = np.sort(rng.choice(d, s, replace=False))
    G = rng.standard_normal((s, s))
    rest = np.setdiff1d(np.arange(d), idx)
    perm = np.concatenate([idx, rest])
    Pi = np.eye(d)[perm]
    B = np.eye(d)
    B[:s, :s] = G
    np.testing.assert_array_equal(O.assemble(O.MODE_FS, d, [G], idx), Pi.T @ B @ Pi)


def test_bsp_assembly_is_conjugated_blockdiag():
    # permuted BS: F = Pi^T blockdiag(G) Pi with Pi the permutation matrix whose row r is e_perm[r] (built here from
    # an identity matrix, independently of the oracle's index bookkeeping), blocks of 4, 4, 2 over d = 10
    rng = np.random.default_rng(5)
    G = [rng.standard_normal((c, c)) for c in (4, 4, 2)]
    perm = rng.permutation(10)
    Pi = np.eye(10)[perm]
    from scipy.linalg import block_diag
    np.testing.assert_array_equal(O.assemble(O.MODE_BSP, 10, G, perm), Pi.T @ block_diag(*G) @ Pi)
    # the index sets are the consecutive runs of the permutation and partition [0, d)
    blocks = O.prim_blocks(O.MODE_BSP, 10, 4, perm)
    assert [list(b) for b in blocks] == [list(perm[0:4]), list(perm[4:8]), list(perm[8:10])]
    assert sorted(np.concatenate(blocks)) == list(range(10))


def test_bsp_identity_permutation_is_bs():
    # with the identity permutation the permuted variant is plain POET-BS, bit for bit
    sR, sP, W0, tR, tP, _, _ = _layer_case(O.MODE_BS, 9, 7, 4, 3, 3, 13, 0.2)
    qR, qP = O.Side(O.MODE_BSP, 9, 4, 3), O.Side(O.MODE_BSP, 7, 3, 3)
    rng = np.random.default_rng(14)
    X, dY = rng.standard_normal((5, 7)), rng.standard_normal((5, 9))
    a = O.linear_fwd(sR, sP, W0, tR, tP, None, None, X)
    b = O.linear_fwd(qR, qP, W0, tR, tP, np.arange(9), np.arange(7), X)
    np.testing.assert_array_equal(a["Y"], b["Y"])
    ga = O.linear_bwd(sR, sP, W0, tR, tP, None, None, X, dY)
    gb = O.linear_bwd(qR, qP, W0, tR, tP, np.arange(9), np.arange(7), X, dY)
    for key in ("dX", "dthetaR", "dthetaP"):
        np.testing.assert_array_equal(ga[key], gb[key])


def test_bsp_is_bs_on_relabeled_coordinates():
    # Pi_R W Pi_P^T of the permuted layer equals the plain BS layer on the relabeled weight Pi_R W0 Pi_P^T
    sR, sP, W0, tR, tP, iR, iP = _layer_case(O.MODE_BSP, 9, 7, 4, 3, 3, 15, 0.2)
    W = O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, np.zeros((1, 7)))["W"]
    bR, bP = O.Side(O.MODE_BS, 9, 4, 3), O.Side(O.MODE_BS, 7, 3, 3)
    Wb = O.linear_fwd(bR, bP, W0[np.ix_(iR, iP)], tR, tP, None, None, np.zeros((1, 7)))["W"]
    np.testing.assert_allclose(W[np.ix_(iR, iP)], Wb, rtol=0, atol=1e-14)


def test_bs_assembly_blocks():
    rng = np.random.default_rng(4)
    G = [rng.standard_normal((c, c)) for c in (4, 4, 2)]
    F = O.assemble(O.MODE_BS, 10, G)
    from scipy.linalg import block_diag
    np.testing.assert_array_equal(F, block_diag(*G))


def test_pack_prims_padded_layout_by_hand():
    # storage layout of the primitives: each one in a b x b slot, identity outside its c x c corner. Written out
    # element by element for a side of d = 7 with b = 3 (blocks 3, 3, 1) and checked against the packing.
    g0 = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0], [7.0, 8.0, 9.0]])
    g1 = -g0.T
    g2 = np.array([[0.5]])
    want = np.array([
        [[1, 2, 3], [4, 5, 6], [7, 8, 9]],
        [[-1, -4, -7], [-2, -5, -8], [-3, -6, -9]],
        [[0.5, 0, 0], [0, 1, 0], [0, 0, 1]],
    ], dtype=np.float64)
    np.testing.assert_array_equal(O.pack_prims(O.MODE_BS, 7, 3, [g0, g1, g2]), want)
    # FS: one s x s primitive fills its slot exactly
    np.testing.assert_array_equal(O.pack_prims(O.MODE_FS, 9, 3, [g0]), g0[None])
    # the packed slots of built primitives hold the blocks of the assembled factor
    th = np.random.default_rng(8).standard_normal(O.theta_len(O.MODE_BS, 7, 3)) * 0.1
    prims = O.build_orthogonal(O.MODE_BS, 7, 3, 2, th)
    F = O.assemble(O.MODE_BS, 7, prims)
    packed = O.pack_prims(O.MODE_BS, 7, 3, prims)
    np.testing.assert_array_equal(packed[0], F[0:3, 0:3])
    np.testing.assert_array_equal(packed[1], F[3:6, 3:6])
    assert packed[2, 0, 0] == F[6, 6] and np.array_equal(packed[2, 1:, 1:], np.eye(2))
    assert not packed[2, 0, 1:].any() and not packed[2, 1:, 0].any()


# ---------------------------------------------------------------- P6: gradients
def _loss(sR, sP, W0, tR, tP, iR, iP, X, dY):
    return float(np.sum(dY * O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, X)["Y"]))


FD_CASES = [
    (O.MODE_BS, 6, 5, 2, 3),   # remainders on both sides
    (O.MODE_BS, 7, 8, 4, 4),
    (O.MODE_BS, 4, 4, 4, 4),
    (O.MODE_FS, 7, 6, 3, 4),
    (O.MODE_FS, 5, 8, 2, 3),
    (O.MODE_BSP, 7, 6, 3, 4),  # permuted blocks with remainders
]


@pytest.mark.parametrize("case", FD_CASES)
@pytest.mark.parametrize("k", [0, 1, 2, 3, 5])
def test_finite_difference_theta(case, k):
    mode, m, n, bR, bP = case
    sR, sP, W0, tR, tP, iR, iP = _layer_case(mode, m, n, bR, bP, k, 21 + k, 0.3)
    rng = np.random.default_rng(22)
    X = rng.standard_normal((5, n))
    dY = rng.standard_normal((5, m))
    g = O.linear_bwd(sR, sP, W0, tR, tP, iR, iP, X, dY)
    h = 1e-6
    for which, th, dth in (("R", tR, g["dthetaR"]), ("P", tP, g["dthetaP"])):
        assert dth.shape == th.shape
        for p in range(len(th)):
            tp, tm = th.copy(), th.copy()
            tp[p] += h
            tm[p] -= h
            if which == "R":
                fd = (_loss(sR, sP, W0, tp, tP, iR, iP, X, dY) - _loss(sR, sP, W0, tm, tP, iR, iP, X, dY)) / (2 * h)
            else:
                fd = (_loss(sR, sP, W0, tR, tp, iR, iP, X, dY) - _loss(sR, sP, W0, tR, tm, iR, iP, X, dY)) / (2 * h)
            assert dth[p] == pytest.approx(fd, rel=1e-6, abs=1e-8), (which, p)


def test_finite_difference_x():
    sR, sP, W0, tR, tP, iR, iP = _layer_case(O.MODE_BS, 6, 5, 2, 3, 3, 31, 0.3)
    rng = np.random.default_rng(32)
    X = rng.standard_normal((3, 5))
    dY = rng.standard_normal((3, 6))
    g = O.linear_bwd(sR, sP, W0, tR, tP, iR, iP, X, dY)
    h = 1e-6
    for t in range(3):
        for i in range(5):
            Xp, Xm = X.copy(), X.copy()
            Xp[t, i] += h
            Xm[t, i] -= h
            fd = (_loss(sR, sP, W0, tR, tP, iR, iP, Xp, dY) - _loss(sR, sP, W0, tR, tP, iR, iP, Xm, dY)) / (2 * h)
            assert g["dX"][t, i] == pytest.approx(fd, rel=1e-7, abs=1e-9)


@pytest.mark.parametrize("c", [3, 8, 20])
@pytest.mark.parametrize("k", range(0, 7))
def test_adjoint_frechet_block(c, k):
    # the Frechet derivative of a polynomial f at A in direction E is the upper-right block of
    # f([[A, E], [0, A]]); the adjoint at Q is the derivative at Q^T (Higham, Functions of Matrices, Thm 3.6)
    rng = np.random.default_rng(40 + c + k)
    Q = rand_skew(rng, c, 0.4)
    dR = rng.standard_normal((c, c))
    Mb = np.block([[Q.T, dR], [np.zeros((c, c)), Q.T]])
    coef = [1.0] + [2.0] * k + [1.0]  # f(x) = 1 + 2x + ... + 2x^k + x^(k+1)
    F = sum(a * np.linalg.matrix_power(Mb, i) for i, a in enumerate(coef))
    np.testing.assert_allclose(O.neumann_adjoint(Q, dR, k), F[:c, c:], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P7: BS with one full block equals FS over all
@pytest.mark.parametrize("k", [0, 3])
def test_bs_single_block_equals_fs_full(k):
    rng = np.random.default_rng(50)
    m, n = 6, 5
    W0 = rng.standard_normal((m, n))
    tR = rng.standard_normal(m * (m - 1) // 2) * 0.2
    tP = rng.standard_normal(n * (n - 1) // 2) * 0.2
    X = rng.standard_normal((4, n))
    dY = rng.standard_normal((4, m))
    bs = (O.Side(O.MODE_BS, m, m, k), O.Side(O.MODE_BS, n, n, k))
    fs = (O.Side(O.MODE_FS, m, m, k), O.Side(O.MODE_FS, n, n, k))
    a = O.linear_bwd(*bs, W0, tR, tP, None, None, X, dY)
    b = O.linear_bwd(*fs, W0, tR, tP, np.arange(m), np.arange(n), X, dY)
    for key in ("dX", "dthetaR", "dthetaP"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_array_equal(O.linear_fwd(*bs, W0, tR, tP, None, None, X)["Y"],
                                  O.linear_fwd(*fs, W0, tR, tP, np.arange(m), np.arange(n), X)["Y"])


# ---------------------------------------------------------------- P8: merge continuity
@pytest.mark.parametrize("mode,bR,bP", [(O.MODE_BS, 4, 3), (O.MODE_FS, 6, 5), (O.MODE_BSP, 4, 3)])
def test_merge_continuity(mode, bR, bP):
    m, n = 12, 10
    sR, sP, W0, tR, tP, iR, iP = _layer_case(mode, m, n, bR, bP, 3, 60, 0.05)
    X = np.random.default_rng(61).standard_normal((9, n))
    y0 = O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, X)["Y"]
    mg = O.merge(sR, sP, W0, tR, tP, iR, iP, seed=60, linear_id=3, epoch_next=1)
    assert np.all(mg["thetaR"] == 0) and np.all(mg["thetaP"] == 0)
    # after the merge the factors are exactly the identity, whatever index sets are drawn
    after = O.linear_fwd(sR, sP, mg["W0"], mg["thetaR"], mg["thetaP"], mg["idxR"], mg["idxP"], X)
    np.testing.assert_array_equal(after["W"], mg["W0"])
    np.testing.assert_allclose(after["Y"], y0, rtol=0, atol=1e-13)
    if mode == O.MODE_FS:
        np.testing.assert_array_equal(mg["idxR"], O.sample_indices(m, bR, 60, 3, O.SIDE_R, 1))
        assert not np.array_equal(mg["idxR"], iR) or not np.array_equal(mg["idxP"], iP)
    if mode == O.MODE_BSP:
        np.testing.assert_array_equal(mg["idxP"], O.sample_permutation(n, 60, 3, O.SIDE_P, 1))
        assert not np.array_equal(mg["idxR"], iR) and not np.array_equal(mg["idxP"], iP)


def test_merge_spectrum_exact_factors():
    # with (numerically) exact Cayley factors, merging keeps the singular values of W0
    sR, sP, W0, tR, tP, iR, iP = _layer_case(O.MODE_BS, 12, 10, 4, 5, 60, 70, 0.1)
    mg = O.merge(sR, sP, W0, tR, tP, iR, iP, 70, 0, 1)
    np.testing.assert_allclose(np.linalg.svd(mg["W0"], compute_uv=False), np.linalg.svd(W0, compute_uv=False),
                               rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P9: parameter counts printed on the pages
def test_parameter_counts_llama_1_3b():
    g = json.load(open(os.path.join(GOLD, "param_counts.json")))
    h, f, L, b = (g["shapes"][x] for x in ("hidden", "ffn", "layers", "block"))
    shapes = [(h, h)] * 4 + [(f, h)] * 2 + [(h, f)]
    poet = L * sum(O.theta_len(O.MODE_BS, m, b) + O.theta_len(O.MODE_BS, n, b) for m, n in shapes)
    dense = L * sum(m * n for m, n in shapes)
    # c(c-1)/2 per primitive; a dense b x b count would be about twice as large
    assert abs(poet - g["poet_bs256_llama1.3b_trainable"]) / g["poet_bs256_llama1.3b_trainable"] < 2.5e-3
    assert round(dense / 1e9, 2) == g["adamw_llama1.3b_trainable"] / 1e9
    assert poet == 118_544_400 and dense == 1_207_910_400


# ---------------------------------------------------------------- P10: index sampler
def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(GOLD, "splitmix64_seed1234567.json")))
    state = g["seed"]
    for want in g["outputs"]:
        assert O.splitmix64(state) == int(want)
        state = (state + 0x9E3779B97F4A7C15) % (1 << 64)
    arr = np.array([g["seed"]], dtype=np.uint64)
    assert int(O.splitmix64(arr)[0]) == int(g["outputs"][0])


@pytest.mark.parametrize("d,s", [(1, 1), (5, 0), (5, 5), (64, 32), (5461, 2730), (2048, 1024)])
def test_sampler_structure(d, s):
    idx = O.sample_indices(d, s, 1234, 5, 1, 2)
    assert idx.dtype == np.int32 and len(idx) == s
    assert np.all(np.diff(idx) > 0) if s > 1 else True
    assert (s == 0) or (idx[0] >= 0 and idx[-1] < d)
    np.testing.assert_array_equal(idx, O.sample_indices(d, s, 1234, 5, 1, 2))


@pytest.mark.parametrize("d", [1, 7, 64, 300, 5461])
def test_permutation_sampler_structure_and_fs_tie(d):
    perm = O.sample_permutation(d, 9, 4, O.SIDE_P, 2)
    assert perm.dtype == np.int32 and sorted(perm) == list(range(d))
    # the s lowest ranks are the FS index set of the same draw, for every s
    for s in sorted({0, 1, d // 3, d // 2, d}):
        np.testing.assert_array_equal(np.sort(perm[:s]), O.sample_indices(d, s, 9, 4, O.SIDE_P, 2))
    if d > 1:
        assert not np.array_equal(perm, O.sample_permutation(d, 9, 4, O.SIDE_P, 3))


def test_sampler_inputs_matter():
    base = O.sample_indices(100, 50, 9, 1, 0, 0)
    for args in [(10, 1, 0, 0), (9, 2, 0, 0), (9, 1, 1, 0), (9, 1, 0, 1)]:
        assert not np.array_equal(base, O.sample_indices(100, 50, *args))


def test_sampler_uniform_inclusion():
    d, s, E = 64, 32, 2000
    counts = np.zeros(d)
    for e in range(E):
        counts[O.sample_indices(d, s, 77, 3, 0, e)] += 1
    p = s / d
    chi2 = np.sum((counts - E * p) ** 2 / (E * p * (1 - p)))
    from scipy.stats import chi2 as chi2d
    assert chi2 < chi2d.ppf(0.9999, d - 1)


# ---------------------------------------------------------------- optimizer on the skew parameters
def test_adamw_matches_torch_reference():
    # an independent implementation: torch.optim.AdamW on the CPU in float64, several steps with fresh gradients
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    n = 37
    hp = dict(lr=3e-3, beta1=0.85, beta2=0.98, eps=1e-7, weight_decay=0.05)
    theta = rng.standard_normal(n) * 1e-3
    t = torch.tensor(theta.copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([t], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    m, v = np.zeros(n), np.zeros(n)
    for step in range(1, 7):
        g = rng.standard_normal(n) * (10.0 ** -step)
        t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        theta, m, v = O.adamw_step(theta, g, m, v, step, **hp)
        np.testing.assert_allclose(theta, t.detach().numpy(), rtol=1e-12, atol=1e-15)
        st = opt.state[t]
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=0)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=0)


def test_adamw_first_step_closed_form():
    # from zero moments the bias corrections give m^ = g and v^ = g^2: the first step moves each parameter by
    # lr * g / (|g| + eps) (plus the decoupled decay lr * wd * theta), whatever beta1 and beta2 are
    g = np.array([2.0, -0.5, 1e-3, 0.0])
    th = np.array([0.1, 0.2, -0.3, 0.4])
    for b1, b2 in ((0.9, 0.999), (0.5, 0.7)):
        out, m, v = O.adamw_step(th, g, np.zeros(4), np.zeros(4), 1, 0.01, b1, b2, 1e-8, 0.1)
        want = th - 0.01 * (g / (np.abs(g) + 1e-8) + 0.1 * th)
        np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-17)
        np.testing.assert_allclose(m, (1 - b1) * g)
        np.testing.assert_allclose(v, (1 - b2) * g * g)


def test_optimizer_state_reset_at_merge():
    m, v, step = O.optimizer_state_after_merge(np.ones(5), np.ones(5))
    assert step == 0 and not m.any() and not v.any() and len(m) == len(v) == 5


# ---------------------------------------------------------------- exact Cayley primitives
@pytest.mark.parametrize("t", [0.3, -1.7])
def test_exact_cayley_2x2_is_rotation(t):
    # (I + Q)(I - Q)^{-1} for Q = [[0, t], [-t, 0]] is the rotation by 2 atan(t), in closed form
    prims = O.build_orthogonal_exact(O.MODE_BS, 2, 2, np.array([t]))
    c, s_ = (1 - t * t) / (1 + t * t), 2 * t / (1 + t * t)
    np.testing.assert_allclose(prims[0], [[c, s_], [-s_, c]], rtol=0, atol=1e-15)


def test_exact_cayley_orthogonal_and_limit():
    rng = np.random.default_rng(12)
    th = rng.standard_normal(O.theta_len(O.MODE_BS, 13, 5)) * 0.05
    ex = O.build_orthogonal_exact(O.MODE_BS, 13, 5, th)
    tr = O.build_orthogonal(O.MODE_BS, 13, 5, 40, th)
    for a, b in zip(ex, tr):
        np.testing.assert_allclose(a.T @ a, np.eye(a.shape[0]), atol=1e-14)
        np.testing.assert_allclose(a, b, atol=1e-14)


# ---------------------------------------------------------------- spectral diagnostics
def test_hyperspherical_energy_closed_forms():
    # orthonormal neurons: every pair at distance sqrt 2, so E_1 = N (N - 1) / sqrt 2
    Qm, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((9, 9)))
    assert O.hyperspherical_energy(Qm[:6] * 3.0) == pytest.approx(6 * 5 / np.sqrt(2), rel=1e-13)
    # two antipodal neurons: distance 2 both ways, E_1 = 1/2 + 1/2; E_2 = 1/4 + 1/4
    W = np.array([[1.0, 2.0], [-2.0, -4.0]])
    assert O.hyperspherical_energy(W) == pytest.approx(1.0, rel=1e-14)
    assert O.hyperspherical_energy(W, s=2.0) == pytest.approx(0.5, rel=1e-14)
    # three neurons at 120 degrees in a plane: distances sqrt 3, E_1 = 6 / sqrt 3
    a = 2 * np.pi / 3
    W = np.array([[1, 0, 0], [np.cos(a), np.sin(a), 0], [np.cos(2 * a), np.sin(2 * a), 0]]) * [[1.0], [5.0], [0.2]]
    assert O.hyperspherical_energy(W) == pytest.approx(6 / np.sqrt(3), rel=1e-13)


def test_hyperspherical_energy_invariances():
    # row scaling and an orthogonal factor on the input side (W0 P) leave every neuron's distances unchanged
    rng = np.random.default_rng(5)
    W = rng.standard_normal((12, 7))
    P = O.cayley_exact(O.skew_from_theta(rng.standard_normal(21) * 0.3, 7))
    e = O.hyperspherical_energy_rows(W)
    np.testing.assert_allclose(O.hyperspherical_energy_rows(W @ P), e, rtol=1e-12)
    np.testing.assert_allclose(O.hyperspherical_energy_rows(W * rng.uniform(0.1, 9, (12, 1))), e, rtol=1e-12)
    np.testing.assert_allclose(O.hyperspherical_energy_rows(W, rows=[3, 0]), e[[3, 0]], rtol=0)
    assert O.hyperspherical_energy(W) == pytest.approx(e.sum(), rel=1e-15)


def test_singular_value_entropy_closed_forms():
    n = 8
    Qm, _ = np.linalg.qr(np.random.default_rng(3).standard_normal((n, n)))
    assert O.singular_value_entropy(2.5 * Qm) == pytest.approx(np.log(n), rel=1e-13)  # flat spectrum
    u, v = np.arange(1.0, 6.0), np.arange(2.0, 5.0)
    assert O.singular_value_entropy(np.outer(u, v)) == pytest.approx(0.0, abs=1e-7)  # rank one
    # singular values 1, 2, 3 (a diagonal matrix with signs and a permutation): p = 1/6, 2/6, 3/6
    D = np.zeros((4, 3))
    D[2, 0], D[0, 1], D[1, 2] = -3.0, 1.0, 2.0
    p = np.array([1, 2, 3]) / 6
    assert O.singular_value_entropy(D) == pytest.approx(-np.sum(p * np.log(p)), rel=1e-13)


def test_singular_value_entropy_is_orthogonally_invariant():
    # the spectrum claim: R W0 P with exactly orthogonal factors keeps every singular value, hence the entropy
    rng = np.random.default_rng(6)
    W0 = rng.standard_normal((9, 6))
    R = O.cayley_exact(O.skew_from_theta(rng.standard_normal(36) * 0.4, 9))
    P = O.cayley_exact(O.skew_from_theta(rng.standard_normal(15) * 0.4, 6))
    assert O.singular_value_entropy(R @ W0 @ P) == pytest.approx(O.singular_value_entropy(W0), rel=1e-13)
