"""The activation-side factor applications and folds take each factor as identity + delta, element by element.

With F = I + D (D = F - I, the delta), an application out = in F^T multiplies the bf16 copy of D and adds the input
itself in float32, so the only roundings are those of D's entries (relative 2^-9 of entries of size |Q|) and the one
rounding of the output. Rounding the whole factor instead would round its diagonal 1 + O(|Q|^2) at the bf16 spacing
near 1 (2^-8 below 1), an error of the size of the output's own rounding. The bound checked for every element:

    |out - exact| <= 1/2 ulp_bf16(exact) + 2^-8 sum_k |in_k| |D_jk| + 2^-16 sum_k |in_k| |F_jk|

(exact = the float64 product of the bf16 input with the GPU's own float32 primitive; the second term covers the
rounding of D, the third the float32 accumulation of at most 256 terms). A whole-factor rounding breaks it wherever
a diagonal entry rounds by more than the slack, which theta of standard deviation 0.01 on blocks of 256 (diagonal
about 0.95) makes common.

Set-up for the applications: a square layer with W0 = I and theta_R = 0, so that R = I and the token GEMM with the
identity is exact; then Y = bf16(X P^T) and dX = bf16(dY P) are single applications of P, and Y must equal Z bit
for bit (R's delta is zero: only the identity part). Fewer tokens than rows, so nothing is folded. Blocks of 256
(fragment-order operands), 136 (row-order operands) and 20 (not a multiple of 8: the batched-GEMM fallback with the
input as the bf16 addend), each with the operands made inside the call (one-linear build) and with the operand
copies of the grouped build. The folds W0P = W0b P and RW0 = R W0b are checked against the same bound with W0b as
the input.
"""
import numpy as np
import pytest

import poet_inputs as PI
from tests.gpu_util import announce, make_linear, put_act, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dense(prim_flat, d, bp):
    """The d x d block-diagonal factor (float64) from the GPU's primitives (bp x bp blocks, identity padded)."""
    nb = (d + bp - 1) // bp
    blocks = prim_flat[: nb * bp * bp].reshape(nb, bp, bp).astype(np.float64)
    F = np.zeros((d, d))
    for p in range(nb):
        c = min(bp, d - p * bp)
        F[p * bp:p * bp + c, p * bp:p * bp + c] = blocks[p, :c, :c]
    return F


def _half_ulp(x):
    _, e = np.frexp(x)  # |x| = f 2^e, f in [0.5, 1): the bf16 spacing there is 2^(e - 8)
    return np.ldexp(1.0, e - 9)


def _check(name, got, inp, F, trans):
    """got = bf16(inp F^T) (trans) or bf16(inp F), every element against the identity + delta bound."""
    Fm = F.T if trans else F  # out = inp @ Fm
    exact = inp @ Fm
    D = Fm - np.eye(F.shape[0])
    bound = _half_ulp(exact) + 2.0 ** -8 * (np.abs(inp) @ np.abs(D)) + 2.0 ** -16 * (np.abs(inp) @ np.abs(Fm))
    err = np.abs(got.astype(np.float64) - exact)
    worst = float(np.max(err / bound))
    announce(f"{name}: worst error / bound = {worst:.3f}")
    assert worst <= 1.0, (name, worst, np.unravel_index(np.argmax(err / bound), err.shape))


@pytest.mark.parametrize("bP", [256, 136, 20])
@pytest.mark.parametrize("grouped", [False, True])
def test_act_application_is_identity_plus_delta(bP, grouped):
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    n = 512
    T = 200  # fewer tokens than rows and columns: no fold
    lin = make_linear("idd", n, n, T, PI.MODE_BS, 256, bP, 5, PI.DT_BF16, linear_id=2)
    _, _, tP, X, dY = PI.gen_linear(61, 0, lin, theta_std=0.01)
    tR = np.zeros(PI.n_theta(lin.R), np.float32)
    announce(f"identity + delta: bP={bP} grouped={grouped}")
    pl = PoetLinear(n, n, T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, np.eye(n, dtype=np.float32), tR, tP,
                    linear_id=2, path="act")
    Xd, dYd = put_act(pl, X, pl.L.ldx), put_act(pl, dY, pl.L.ldy)
    Y, Z, dX = pl.alloc_act(T, pl.L.ldy), pl.alloc_act(T, pl.L.ldy), pl.alloc_act(T, pl.L.ldx)
    if grouped:
        g = PoetGroup([pl])
        g.build()
        assert pl.opsP is not None and pl.W0P is None and pl.RW0 is None
    else:
        pl.build()
    pl.forward_act(Xd, Y, Z)
    pl.backward_act(Xd, Z, dYd, dX)
    torch.cuda.synchronize()
    assert torch.equal(Y[:, :n], Z[:, :n]), "R = I: the application must return its input exactly"
    P = _dense(to_np(pl.primP), n, bP)
    _check(f"Y = X P^T (bP={bP})", to_np(Y)[:, :n], X.astype(np.float64), P, trans=True)
    _check(f"dX = dY P (bP={bP})", to_np(dX)[:, :n], dY.astype(np.float64), P, trans=False)


def test_folds_are_identity_plus_delta():
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear
    m, n, T = 600, 384, 1024  # T >= m, n: both factors folded; ragged last R block (88)
    lin = make_linear("fold", m, n, T, PI.MODE_BS, 256, 128, 5, PI.DT_BF16, linear_id=3)
    W0, tR, tP, _, _ = PI.gen_linear(62, 0, lin, theta_std=0.01)
    announce("identity + delta: folds")
    pl = PoetLinear(m, n, T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP, linear_id=3, path="act")
    PoetGroup([pl]).build()
    torch.cuda.synchronize()
    assert pl.W0P is not None and pl.RW0 is not None
    W0b = to_np(pl.W0b)[:, :n].astype(np.float64)
    P = _dense(to_np(pl.primP), n, 128)
    R = _dense(to_np(pl.primR), m, 256)
    _check("W0P = W0b P", to_np(pl.W0P)[:, :n], W0b, P, trans=False)
    # RW0 = R W0b: as rows, (RW0)^T = W0b^T R^T
    _check("RW0 = R W0b", to_np(pl.RW0)[:, :n].T, W0b.T, R, trans=True)
