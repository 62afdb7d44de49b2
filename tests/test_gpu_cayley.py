"""GPU exact Cayley primitives (poet_build_orthogonal_exact) against the float64 oracle, and the truncation closed
form measured between the GPU's built and exact primitives.

Sides: the LLaMA-1.3B BS sides (2048 and 5461 with the ragged 85 block, b = 256), b = 64 and 32 with a ragged
last block, a single 7 x 7 block, an FS primitive of 200, at theta std 1e-3 and 0.02. Bar: float32 (relative
Frobenius 1e-5 and the same bar per primitive); orthogonality |R^T R - I| <= 1e-5. The closed form
||R_k - R_cay||_2 = ||Q||_2^(k+1) is checked with float32 sides at k = 1, 2 (where the truncation error is far
above float32 rounding) to 1e-3 relative.
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import announce, check, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _exact(mode, d, b, theta):
    from orthogonal_reparameterized_amd import binding as B
    s = B.side(mode, d, b, 3, B.POET_F32)
    th = torch.from_numpy(np.ascontiguousarray(theta, dtype=np.float32)).cuda()
    prim = torch.full((B.poet_prim_len(s),), float("nan"), dtype=torch.float32, device="cuda")
    B.poet_build_orthogonal_exact(s, th, prim)
    torch.cuda.synchronize()
    return to_np(prim).reshape(-1, b, b)


@pytest.mark.parametrize("std", [1e-3, 0.02])
@pytest.mark.parametrize("mode,d,b", [(PI.MODE_BS, 2048, 256), (PI.MODE_BS, 5461, 256), (PI.MODE_BS, 1376, 64),
                                      (PI.MODE_BS, 200, 32), (PI.MODE_BS, 7, 7), (PI.MODE_FS, 450, 200)])
def test_exact_cayley_matches_oracle(mode, d, b, std):
    announce(f"exact cayley mode={mode} d={d} b={b} std={std}")
    theta = (np.random.default_rng(d + b).standard_normal(O.theta_len(mode, d, b)) * std).astype(np.float32)
    got = _exact(mode, d, b, theta)
    ref = O.pack_prims(mode, d, b, O.build_orthogonal_exact(mode, d, b, theta))
    errs = {}
    try:
        check(errs, "prim", got.ravel(), ref.ravel(), 1e-5, [b * b] * ref.shape[0])
    finally:
        announce(f"exact cayley errors {errs}")
    for P in got:
        assert np.abs(P.T.astype(np.float64) @ P - np.eye(b)).max() <= 1e-5


@pytest.mark.parametrize("k", [1, 2])
def test_truncation_closed_form_between_gpu_primitives(k):
    from orthogonal_reparameterized_amd import binding as B
    mode, d, b = PI.MODE_BS, 320, 64
    theta = (np.random.default_rng(k).standard_normal(O.theta_len(mode, d, b)) * 0.02).astype(np.float32)
    announce(f"truncation closed form k={k}")
    s = B.side(mode, d, b, k, B.POET_F32)
    th = torch.from_numpy(theta).cuda()
    prim = torch.empty(B.poet_prim_len(s), dtype=torch.float32, device="cuda")
    pw = torch.empty(max(B.poet_powers_len(s), 1), dtype=torch.float32, device="cuda")
    B.poet_build_orthogonal(s, th, prim, pw, None)
    torch.cuda.synchronize()
    built = to_np(prim).reshape(-1, b, b).astype(np.float64)
    exact = _exact(mode, d, b, theta).astype(np.float64)
    off = 0
    for p in range(d // b):
        nt = b * (b - 1) // 2
        q2 = np.linalg.norm(O.skew_from_theta(theta[off:off + nt], b), 2)
        off += nt
        dist = np.linalg.norm(built[p] - exact[p], 2)
        assert dist == pytest.approx(q2 ** (k + 1), rel=1e-3), (p, dist, q2 ** (k + 1))
