"""The allocation-free sampler entry point (poet_sample_indices_noalloc) against the workspace one
(poet_sample_indices), through the C ABI: bit-identical index sets on two calls in a row, the second with a smaller
d (the scratch keeps the first call's flags past the second's d, which must not leak into the result), and the
size limit rejected on the host before any launch."""
import numpy as np
import pytest

from tests.gpu_util import announce

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(B, d, s, key):
    ws = torch.empty(B.poet_sample_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    want = torch.full((s,), -1, dtype=torch.int32, device="cuda")
    got = torch.full((s,), -2, dtype=torch.int32, device="cuda")
    B.poet_sample_indices(d, s, *key, want, ws)
    B.poet_sample_indices_noalloc(d, s, *key, got)
    torch.cuda.synchronize()
    return want.cpu().numpy(), got.cpu().numpy()


def test_noalloc_sampler_matches_workspace_sampler():
    from orthogonal_reparameterized_amd import binding as B
    for d, s, key in [(6848, 3424, (5000, 11, 0, 2)), (1376, 688, (5000, 11, 1, 3)),
                      (B.POET_NOALLOC_MAX_D, 3, (7, 1, 0, 0)), (5, 5, (1, 2, 1, 9)), (64, 1, (3, 3, 0, 1))]:
        announce(f"noalloc sampler d={d} s={s}")
        want, got = _pair(B, d, s, key)
        np.testing.assert_array_equal(got, want)
        assert np.all(np.diff(got) > 0) and got.min() >= 0 and got.max() < d


def test_noalloc_sampler_rejects_oversize_on_host():
    from orthogonal_reparameterized_amd import binding as B
    idx = torch.empty(4, dtype=torch.int32, device="cuda")
    with pytest.raises(B.PoetError, match="maximum"):
        B.poet_sample_indices_noalloc(B.POET_NOALLOC_MAX_D + 1, 4, 0, 0, 0, 0, idx)
