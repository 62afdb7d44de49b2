"""GPU parity of the spectral diagnostics (poet_hyperspherical_energy, poet_singular_value_entropy) against the
float64 oracle, through the C ABI, and the spectrum claim checked with them on the GPU.

Shapes: tall, wide and square small weights (several Gram tiles and ragged edges, r = 1 and 2), the LLaMA-60M
gate weight in full (total energy), and the LLaMA-1.3B gate weight (5461 x 2048) at full size: its singular values
and entropy in full, its per-neuron energies on 64 sampled neurons (each one an exact oracle value). The GPU
works in float64 from the float32 weight and the oracle takes the same float32 values, so the bar is derived from
float64 arithmetic on a Gram matrix: 1e-9 relative (per neuron energy, entropy) and 1e-9 of sigma_max (singular
values), far inside the float32 bar.
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _diag(W, pad=0, s=1.0, rows=True):
    from orthogonal_reparameterized_amd import binding as B
    m, n = W.shape
    Wd = torch.zeros((m, n + pad), dtype=torch.float32, device="cuda")
    Wd[:, :n] = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32))
    e = torch.empty(1, dtype=torch.float64, device="cuda")
    er = torch.empty(m, dtype=torch.float64, device="cuda") if rows else None
    h = torch.empty(1, dtype=torch.float64, device="cuda")
    sg = torch.empty(min(m, n), dtype=torch.float64, device="cuda")
    B.poet_hyperspherical_energy(m, n, Wd, n + pad, s, e, energy_rows=er)
    B.poet_singular_value_entropy(m, n, Wd, n + pad, h, sigma=sg)
    torch.cuda.synchronize()
    return (float(e.item()), None if er is None else er.cpu().numpy(), float(h.item()), sg.cpu().numpy())


@pytest.mark.parametrize("m,n,pad", [(60, 23, 0), (40, 40, 3), (17, 150, 1), (130, 65, 0), (1, 5, 0), (5, 1, 0),
                                     (2, 2, 0), (200, 129, 7)])
def test_spectral_small_against_oracle(m, n, pad):
    announce(f"spectral small m={m} n={n} pad={pad}")
    W = np.random.default_rng(m * 1000 + n).standard_normal((m, n)).astype(np.float32)
    e, er, h, sg = _diag(W, pad)
    ref_rows = O.hyperspherical_energy_rows(W)
    ref_sig = np.linalg.svd(W.astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(er, ref_rows, rtol=1e-9, atol=0)
    assert e == pytest.approx(O.hyperspherical_energy(W), rel=1e-9, abs=0)
    np.testing.assert_allclose(sg, ref_sig, rtol=0, atol=1e-9 * ref_sig.max())
    assert h == pytest.approx(O.singular_value_entropy(W), rel=1e-9, abs=1e-12)


def test_spectral_energy_exponent():
    W = np.random.default_rng(3).standard_normal((50, 20)).astype(np.float32)
    for s in (0.5, 2.0):
        e, er, _, _ = _diag(W, s=s)
        np.testing.assert_allclose(er, O.hyperspherical_energy_rows(W, s=s), rtol=1e-9)


def test_spectral_llama60m_gate_full():
    lin = [l for l in PI.WORKLOADS[2].linears() if l.name == "gate"][0]
    W0, _, _ = PI.gen_weights(2, 0, lin)
    announce(f"spectral llama60m gate {W0.shape}")
    e, er, h, sg = _diag(W0, pad=PI.pad_ld(lin.n) - lin.n)
    assert e == pytest.approx(O.hyperspherical_energy(W0), rel=1e-9)
    assert h == pytest.approx(O.singular_value_entropy(W0), rel=1e-9)


def test_spectral_llama1p3b_gate_full_size():
    lin = [l for l in PI.WORKLOADS[3].linears() if l.name == "gate"][0]
    W0, _, _ = PI.gen_weights(3, 0, lin)
    announce(f"spectral llama1.3b gate {W0.shape}")
    e, er, h, sg = _diag(W0, pad=PI.pad_ld(lin.n) - lin.n)
    rows = np.sort(np.random.default_rng(8).choice(lin.m, 64, replace=False))
    np.testing.assert_allclose(er[rows], O.hyperspherical_energy_rows(W0, rows=rows), rtol=1e-9)
    assert e == pytest.approx(float(np.sum(er)), rel=1e-12)  # the total is the sum of the neurons' energies
    ref_sig = np.linalg.svd(W0.astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(sg, ref_sig, rtol=0, atol=1e-9 * ref_sig.max())
    assert h == pytest.approx(O.singular_value_entropy(W0), rel=1e-9)


@pytest.mark.parametrize("mode,b", [(PI.MODE_BS, 64), (PI.MODE_FS, 300)])
def test_spectrum_preserved_by_the_merge_on_gpu(mode, b):
    """The spectrum claim, measured with the GPU diagnostics across a merge: with k = 2 the singular values of R_k
    are |1 - (i lambda)^3| = sqrt(1 + lambda^6) over the eigenvalues i lambda of Q, so every singular value of the
    merged W0 = R_k W0 P_k lies in [sigma_i(W0), sigma_i(W0) sqrt(1 + ||Q_R||^6) sqrt(1 + ||Q_P||^6)], up to the
    float32 rounding of the merge."""
    from orthogonal_reparameterized_amd import binding as B
    from tests.gpu_util import gpu_linear, make_linear, oracle_indices
    lin = make_linear("spectrum", 700, 600, 8, mode, b, b, 2, PI.DT_F32, linear_id=3)
    W0, tR, tP, _, _ = PI.gen_linear(97, 0, lin, theta_std=0.01)
    iR, iP = oracle_indices(lin, 5)
    announce(f"spectrum across a merge mode={mode} b={b}")
    pl = gpu_linear(lin, W0, tR, tP, iR, iP, seed=5)
    f64 = dict(dtype=torch.float64, device="cuda")
    h0, s0, h1, s1 = torch.empty(1, **f64), torch.empty(600, **f64), torch.empty(1, **f64), torch.empty(600, **f64)
    B.poet_singular_value_entropy(700, 600, pl.W0, pl.L.ldw, h0, sigma=s0)
    pl.build()
    pl.merge()
    B.poet_singular_value_entropy(700, 600, pl.W0, pl.L.ldw, h1, sigma=s1)
    torch.cuda.synchronize()
    qR = max(np.linalg.norm(O.skew_from_theta(t, c), 2) for t, c in _blocks(lin.R, tR))
    qP = max(np.linalg.norm(O.skew_from_theta(t, c), 2) for t, c in _blocks(lin.P, tP))
    s0n, s1n = s0.cpu().numpy(), s1.cpu().numpy()
    tol = 1e-5 * s0n.max()
    upper = np.sqrt(1 + qR ** 6) * np.sqrt(1 + qP ** 6)
    assert np.all(s1n >= s0n - tol), float(np.min(s1n - s0n))
    assert np.all(s1n <= s0n * upper + tol), float(np.max(s1n - s0n * upper))
    assert abs(h1.item() - h0.item()) <= 1e-3 * h0.item()


def _blocks(side, theta):
    off = 0
    for c in O.block_sizes(side.mode, side.d, side.b):
        nt = c * (c - 1) // 2
        yield theta[off:off + nt], c
        off += nt
