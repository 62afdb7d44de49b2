"""GPU parity of the AdamW step on the packed skew parameters (poet_adamw_group) and of its moment reset
(poet_optimizer_reset_group), through the C ABI, against the float64 oracle.

The sides cover the LLaMA-1.3B BS sides (2048 and 5461 with a ragged 85 block), an FS side (s = 2730), a small
ragged side and a side with no parameters; more sides than one launch's table holds (16), buffers at an offset
of one float (the unvectorized path), three steps in a row with fresh gradients. Inputs are float32; the oracle
takes the same values in float64. Bar: float32, relative Frobenius <= 1e-5 and the same bar per primitive.
"""
import numpy as np
import pytest

import oracle as O
import poet_inputs as PI
from tests.gpu_util import announce, check, theta_groups, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SIDES = [(PI.MODE_BS, 2048, 256), (PI.MODE_BS, 5461, 256), (PI.MODE_FS, 5461, 2730), (PI.MODE_BS, 200, 64),
         (PI.MODE_BS, 7, 1)] + [(PI.MODE_BS, 300 + 37 * i, 48) for i in range(13)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(a, offset):
    """a (float32) on the device starting `offset` floats into its buffer (offset 1: not 16-byte aligned)."""
    buf = torch.zeros(len(a) + offset + 1, dtype=torch.float32, device="cuda")
    t = buf[offset:offset + len(a)]
    t.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)))
    return t


@pytest.mark.parametrize("hp", [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),
                                dict(lr=3e-4, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1)])
def test_adamw_group_matches_oracle(hp):
    from orthogonal_reparameterized_amd import binding as B
    rng = np.random.default_rng(40)
    sides = [B.side(mode, d, b, 3, B.POET_BF16) for mode, d, b in SIDES]
    n = [B.poet_theta_len(s) for s in sides]
    th = [(rng.standard_normal(k) * 1e-3).astype(np.float32) for k in n]
    m = [np.zeros(k, np.float32) for k in n]
    v = [np.zeros(k, np.float32) for k in n]
    off = [i % 2 for i in range(len(sides))]  # every other side unaligned
    thd = [_dev(a, o) for a, o in zip(th, off)]
    md = [_dev(a, o) for a, o in zip(m, off)]
    vd = [_dev(a, o) for a, o in zip(v, off)]
    h = B.adamw(**hp)
    # the hyperparameters cross the C ABI as float32: the oracle takes those same values
    hp = {k: float(np.float32(x)) for k, x in hp.items()}
    for step in (1, 2, 3):
        announce(f"adamw step {step} over {len(sides)} sides, {sum(n)} parameters")
        g = [(rng.standard_normal(k) * 10.0 ** rng.integers(-6, 0)).astype(np.float32) for k in n]
        gd = [_dev(a, o) for a, o in zip(g, off)]
        B.poet_adamw_group(sides, thd, gd, md, vd, h, step)
        torch.cuda.synchronize()
        errs = {}
        try:
            for i, (mode, d, b) in enumerate(SIDES):
                if not n[i]:
                    continue
                th[i], m[i], v[i] = O.adamw_step(th[i], g[i], m[i], v[i], step, **hp)
                grp = theta_groups(mode, d, b)
                check(errs, f"theta{i}", to_np(thd[i]), th[i], 1e-5, grp)
                check(errs, f"m{i}", to_np(md[i]), m[i], 1e-5, grp)
                check(errs, f"v{i}", to_np(vd[i]), v[i], 1e-5, grp)
                # the oracle's next step starts from its own results rounded to float32, the state's precision
                th[i], m[i], v[i] = (x.astype(np.float32) for x in (th[i], m[i], v[i]))
        finally:
            announce(f"adamw step {step}: worst {max(errs.values()) if errs else 0:.2e}")


def test_optimizer_reset_group_zeroes_moments():
    from orthogonal_reparameterized_amd import binding as B
    sides = [B.side(mode, d, b, 3, B.POET_BF16) for mode, d, b in SIDES]
    n = [max(B.poet_theta_len(s), 1) for s in sides]
    ms = [torch.full((k,), 3.0, device="cuda") for k in n]
    vs = [torch.full((k,), 5.0, device="cuda") for k in n]
    announce("optimizer reset")
    B.poet_optimizer_reset_group(sides, ms, vs)
    torch.cuda.synchronize()
    for s, a, b in zip(sides, ms, vs):
        k = B.poet_theta_len(s)
        assert float(a[:k].abs().max() if k else 0) == 0.0 and float(b[:k].abs().max() if k else 0) == 0.0
