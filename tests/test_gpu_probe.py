"""The matrix-core rate probe (poet_mfma_probe) issues the MFMAs it reports: every wave's output is lane 0's sum of
its 4 accumulator tiles after 4 * iters products, a closed form of the probe's fixed operands (bf16-rounded), checked
for every wave of a small grid at float32 accuracy; and its timed rate stays below the published bf16 peak."""
import numpy as np
import pytest

import poet_inputs as PI
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _lane0_sum(iters):
    """Lane 0 holds column 0 of the 32 x 32 product at rows 8 (r // 4) + r % 4, r = 0..15 (v_mfma_f32_32x32x16_bf16:
    lane l, register r -> row 8 (r // 4) + 4 (l // 32) + r % 4, column l % 32). A[i][k] comes from lane i + 32 (k // 8)
    element k % 8, B[k][j] from lane j + 32 (k // 8) element k % 8."""
    lanes, v = np.arange(64)[:, None], np.arange(8)[None, :]
    a = PI.round_bf16((1e-3 * ((lanes + v) & 15)).astype(np.float32)).astype(np.float64)
    b = PI.round_bf16((1e-3 * ((lanes * 3 + v) & 7) - 4e-3).astype(np.float32)).astype(np.float64)
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for k in range(16):
        A[:, k] = a[np.arange(32) + 32 * (k // 8), k % 8]
        Bm[k, :] = b[np.arange(32) + 32 * (k // 8), k % 8]
    C = A @ Bm
    rows = [8 * (r // 4) + r % 4 for r in range(16)]
    return 4 * iters * C[rows, 0].sum()


def test_mfma_probe_closed_form_and_rate():
    from orthogonal_reparameterized_amd import binding as B
    wgs, iters = 64, 100
    out = torch.full((wgs * 8,), float("nan"), dtype=torch.float32, device="cuda")
    announce(f"mfma probe {wgs} workgroups, {iters} iterations")
    B.poet_mfma_probe(iters, wgs, out)
    torch.cuda.synchronize()
    want = _lane0_sum(iters)
    got = out.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-4)
    import bench
    r = bench.mfma_probe(torch, B, workgroups=512, iters=256, warm_launches=10)
    announce(f"mfma probe rate {r}")
    assert 0 < r["achieved"] <= bench.PEAK_BF16_TFLOPS * 1.02
