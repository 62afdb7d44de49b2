"""Host-side state rules of PoetLinear / PoetGroup (no GPU: the checks fire before any library call).

- Forward, backward and merge refuse to run on factors that were never built, and again after a merge: the
  merge resets theta to zero, so the primitives, their bf16 operand copies and the folded weights of the last
  build belong to the parameters before the reset.
- The merge's epoch advances only when the merge call was accepted; a call rejected by the binding leaves it
  where it was, so the next FS resample uses the right epoch.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from orthogonal_reparameterized_amd import binding as B  # noqa: E402
from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear  # noqa: E402


def _cpu_linear():
    R = B.side(B.POET_BS, 64, 32, 2, B.POET_F32)
    P = B.side(B.POET_BS, 48, 16, 2, B.POET_F32)
    W0 = np.random.default_rng(0).standard_normal((64, 48)).astype(np.float32)
    return PoetLinear(64, 48, 8, R, P, B.POET_F32, W0, device="cpu", path="weight")


def test_calls_refuse_unbuilt_factors():
    pl = _cpu_linear()
    X = torch.zeros((8, 48))
    for call in (lambda: pl.forward(X, X), lambda: pl.backward(X, X, X), lambda: pl.backward_prims(X, X, X),
                 lambda: pl.merge(), lambda: PoetGroup([pl]).merge()):
        with pytest.raises(RuntimeError, match="build"):
            call()
    assert pl.epoch == 0


def test_rejected_merge_keeps_the_epoch():
    pl = _cpu_linear()
    pl.built = True  # as after a build; the binding then rejects the CPU tensors before any launch
    with pytest.raises(ValueError, match="GPU tensor"):
        pl.merge()
    assert pl.epoch == 0 and pl.built
    with pytest.raises(ValueError, match="GPU tensor"):
        PoetGroup([pl]).merge()
    assert pl.epoch == 0 and pl.built


def test_merge_marks_the_build_stale():
    pl = _cpu_linear()
    pl.built = True
    pl.W0P = pl.RW0 = pl.opsR = pl.opsP = object()
    pl._merged()
    assert pl.epoch == 1 and not pl.built
    assert pl.W0P is None and pl.RW0 is None and pl.opsR is None and pl.opsP is None
    with pytest.raises(RuntimeError, match="build"):
        pl.forward(torch.zeros((8, 48)), torch.zeros((8, 64)))


def test_optimizer_step_needs_a_fresh_gradient():
    pl = _cpu_linear()
    with pytest.raises(RuntimeError, match="gradient"):
        pl.optimizer_step(B.adamw())
    with pytest.raises(RuntimeError, match="gradient"):
        PoetGroup([pl]).optimizer_step(B.adamw())
    pl.grad_ready = True  # as after a backward; the binding then rejects the CPU tensors before any launch
    with pytest.raises(ValueError, match="GPU tensor"):
        pl.optimizer_step(B.adamw())
    assert pl.opt_steps == 0 and pl.grad_ready
    pl._stepped()
    assert pl.opt_steps == 1 and not pl.grad_ready and not pl.built
    pl._merged()
    assert pl.opt_steps == 0 and pl.epoch == 1


def test_build_again_needs_unchanged_parameters():
    pl = _cpu_linear()
    with pytest.raises(RuntimeError, match="again"):
        PoetGroup([pl]).build(again=True)  # never built
    pl.built = True
    pl._stepped()  # the parameters changed: the folds and formed operands of the last build are stale
    with pytest.raises(RuntimeError, match="again"):
        PoetGroup([pl]).build(again=True)
