"""Plant plausible mistakes in the CPU oracle (on the CPU only) and check that the pins catch every one.

Each mutation replaces one oracle function with a subtly wrong version; the listed pin tests must then fail.
"""
import numpy as np
import pytest

import oracle as O
import oracle.poet_oracle as PO
import tests.test_oracle_pins as pins

_ORIG = {f: getattr(PO, f) for f in ("neumann_adjoint", "linear_bwd", "assemble", "sample_indices", "adamw_step",
                                     "prim_blocks", "sample_permutation")}


def _cn_drop_last(Q, k):
    c = Q.shape[0]
    S, Qi = np.eye(c), np.eye(c)
    for _ in range(max(k - 1, 0)):
        Qi = Qi @ Q
        S = S + Qi
    return (np.eye(c) + Q) @ S


def _cn_wrong_sign(Q, k):
    c = Q.shape[0]
    S, Qi = np.eye(c), np.eye(c)
    for _ in range(k):
        Qi = Qi @ Q
        S = S + Qi
    return (np.eye(c) - Q) @ S


def _skew_flipped(theta, c):
    Q = np.zeros((c, c))
    Q[np.triu_indices(c, 1)] = theta
    return Q.T - Q


def _adjoint_untransposed(Q, dR, k):
    return _ORIG["neumann_adjoint"](Q.T, dR, k)


def _adjoint_missing_coef(Q, dR, k):
    pw = [np.eye(Q.shape[0])]
    for _ in range(k + 1):
        pw.append(pw[-1] @ Q.T)
    dQ = np.zeros_like(dR)
    for i in range(1, k + 2):
        for j in range(i):
            dQ = dQ + pw[j] @ dR @ pw[i - 1 - j]  # every coefficient 1
    return dQ


def _project_wrong(dQ):
    iu = np.triu_indices(dQ.shape[0], 1)
    return dQ[iu]


def _bwd_transposed_rw0(sR, sP, W0, thetaR, thetaP, idxR, idxP, X, dY):
    # dL/dP taken from W0 R instead of R W0 (a transposed factor)
    W0 = np.asarray(W0, float)
    R = O.factor(sR, thetaR, idxR)
    P = O.factor(sP, thetaP, idxP)
    G = np.asarray(dY, float).T @ np.asarray(X, float)
    W0P = W0 @ P
    W0R = R.T @ W0
    out = _ORIG["linear_bwd"](sR, sP, W0, thetaR, thetaP, idxR, idxP, X, dY)
    out["dthetaP"] = PO._side_grad(sP, thetaP, idxP, lambda J: W0R[:, J].T @ G[:, J])
    del W0P
    return out


def _assemble_fs_rows_only(mode, d, prims, idx=None):
    if mode != O.MODE_FS:
        return _ORIG["assemble"](mode, d, prims, idx)
    F = np.eye(d)
    idx = np.asarray(idx)
    F[idx[:, None], np.arange(len(idx))[None, :]] = prims[0]  # wrong columns
    return F


def _bsp_blocks_inverse(mode, d, b, idx=None):
    # permuted BS blocks taken from the inverse permutation (positions instead of indices)
    if mode != O.MODE_BSP:
        return _ORIG["prim_blocks"](mode, d, b, idx)
    return _ORIG["prim_blocks"](mode, d, b, np.argsort(np.asarray(idx)))


def _permutation_reversed(d, seed, linear_id, side, epoch):
    return _ORIG["sample_permutation"](d, seed, linear_id, side, epoch)[::-1].copy()


def _sampler_descending(d, s, seed, linear_id, side, epoch):
    return _ORIG["sample_indices"](d, s, seed, linear_id, side, epoch)[::-1].copy()


def _adamw_no_bias_correction(theta, grad, m, v, step, lr, beta1, beta2, eps, weight_decay):
    theta = np.asarray(theta, float)
    m = beta1 * np.asarray(m, float) + (1 - beta1) * grad
    v = beta2 * np.asarray(v, float) + (1 - beta2) * grad * grad
    return theta - lr * (m / (np.sqrt(v) + eps) + weight_decay * theta), m, v


def _adamw_coupled_decay(theta, grad, m, v, step, lr, beta1, beta2, eps, weight_decay):
    # L2 regularization folded into the gradient (Adam with weight decay) instead of the decoupled decay
    g = np.asarray(grad, float) + weight_decay * np.asarray(theta, float)
    return _ORIG["adamw_step"](theta, g, m, v, step, lr, beta1, beta2, eps, 0.0)


def _cayley_exact_inverted(Q):
    I = np.eye(Q.shape[0])
    return (I - Q) @ np.linalg.solve(I + Q, I)


def _he_rows_columns_normalized(W, s=1.0, rows=None):
    W = np.asarray(W, float)
    Wn = W / np.linalg.norm(W, axis=0, keepdims=True)  # wrong axis
    rows = range(Wn.shape[0]) if rows is None else rows
    out = []
    for i in rows:
        dist = np.linalg.norm(Wn[i][None, :] - Wn, axis=1)
        dist[i] = np.inf
        out.append(float(np.sum(dist ** (-s))))
    return np.asarray(out)


def _sv_entropy_squared(W):
    sig = np.linalg.svd(np.asarray(W, float), compute_uv=False) ** 2  # energy, not the singular values
    p = sig / sig.sum()
    p = p[p > 0]
    return float(-np.sum(p * np.log(p)))


MUTATIONS = {
    "neumann_drops_last_term": ("cayley_neumann", _cn_drop_last,
                                [lambda: pins.test_2x2_distance_to_rotation(0.3, 2),
                                 lambda: pins.test_2x2_golden_values()]),
    "cayley_sign": ("cayley_neumann", _cn_wrong_sign,
                    [lambda: pins.test_2x2_golden_values(),
                     lambda: pins.test_truncation_closed_forms(2, 16)]),
    "skew_sign": ("skew_from_theta", _skew_flipped, [lambda: pins.test_2x2_golden_values()]),
    "adjoint_untransposed": ("neumann_adjoint", _adjoint_untransposed,
                             [lambda: pins.test_adjoint_frechet_block(8, 2),
                              lambda: pins.test_finite_difference_theta(pins.FD_CASES[0], 2)]),
    "adjoint_coefficients": ("neumann_adjoint", _adjoint_missing_coef,
                             [lambda: pins.test_adjoint_frechet_block(8, 3),
                              lambda: pins.test_finite_difference_theta(pins.FD_CASES[1], 3)]),
    "projection_one_sided": ("skew_project", _project_wrong,
                             [lambda: pins.test_finite_difference_theta(pins.FD_CASES[2], 1)]),
    "bwd_transposed_factor": ("linear_bwd", _bwd_transposed_rw0,
                              [lambda: pins.test_finite_difference_theta(pins.FD_CASES[1], 2)]),
    "fs_assembly_columns": ("assemble", _assemble_fs_rows_only,
                            [lambda: pins.test_fs_assembly_is_permuted_block()]),
    "bsp_blocks_inverse_permutation": ("prim_blocks", _bsp_blocks_inverse,
                                       [lambda: pins.test_bsp_assembly_is_conjugated_blockdiag()]),
    "permutation_reversed": ("sample_permutation", _permutation_reversed,
                             [lambda: pins.test_permutation_sampler_structure_and_fs_tie(64)]),
    "sampler_order": ("sample_indices", _sampler_descending,
                      [lambda: pins.test_sampler_structure(64, 32)]),
    "adamw_no_bias_correction": ("adamw_step", _adamw_no_bias_correction,
                                 [lambda: pins.test_adamw_matches_torch_reference(),
                                  lambda: pins.test_adamw_first_step_closed_form()]),
    "adamw_coupled_decay": ("adamw_step", _adamw_coupled_decay,
                            [lambda: pins.test_adamw_matches_torch_reference(),
                             lambda: pins.test_adamw_first_step_closed_form()]),
    "cayley_exact_inverted": ("cayley_exact", _cayley_exact_inverted,
                              [lambda: pins.test_exact_cayley_2x2_is_rotation(0.3)]),
    "he_wrong_normalization": ("hyperspherical_energy_rows", _he_rows_columns_normalized,
                               [lambda: pins.test_hyperspherical_energy_closed_forms()]),
    "sv_entropy_of_energies": ("singular_value_entropy", _sv_entropy_squared,
                               [lambda: pins.test_singular_value_entropy_closed_forms()]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    fname, bad, checks = MUTATIONS[name]
    for mod in (PO, O):
        monkeypatch.setattr(mod, fname, bad)
    for check in checks:
        with pytest.raises(AssertionError):
            check()
