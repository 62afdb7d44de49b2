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


def test_side_class_is_the_gemm_chain_class_with_the_most_work():
    """PoetGroup's side stream takes the sides of one class of bf16 primitives above 256 (equal mode, size and k),
    the one with the most product work, and only when other sides remain for the launch stream."""
    def fs(d, k=5, dt=B.POET_BF16):
        return B.side(B.POET_FS, d, d // 2, k, dt)
    # a LLaMA-1.3B block with s = d/2: q, k, v, o (2048 x 2048), gate and up (5461 x 2048), down (2048 x 5461)
    block = [fs(2048), fs(2048)] * 4 + [fs(5461), fs(2048), fs(5461), fs(2048), fs(2048), fs(5461)]
    assert PoetGroup._side_class(block) == [8, 10, 13]
    assert PoetGroup._side_class([B.side(B.POET_BS, 2048, 256, 5, B.POET_BF16)] * 14) == []  # fused chains only
    assert PoetGroup._side_class([fs(5461)] * 3) == []  # a single class
    assert PoetGroup._side_class([B.side(B.POET_BS, 2048, 256, 5, B.POET_BF16), fs(2048)]) == [1]
    # float32 sides and k = 0 sides do not run as bf16 products
    assert PoetGroup._side_class([fs(2048, dt=B.POET_F32), fs(2048)]) == [1]
    assert PoetGroup._side_class([fs(2048, k=0), fs(2048)]) == [1]
    # more work wins: one 1536-primitive (1536^3 x 5) against three of 1024 (3 x 1024^3 x 5), not against four
    assert PoetGroup._side_class([fs(2048)] * 3 + [fs(3072)]) == [3]
    assert PoetGroup._side_class([fs(2048)] * 4 + [fs(3072)]) == [0, 1, 2, 3]
    # a large POET-BS block size is a class of its own
    assert PoetGroup._side_class([B.side(B.POET_BS, 1024, 512, 3, B.POET_BF16)] * 2 + [fs(2048, k=3)]) == [2]


def test_side_linears_must_name_some_not_all():
    lins = [_cpu_linear(), _cpu_linear()]
    for bad in ([], [0, 1], [2], [-1]):
        with pytest.raises(ValueError, match="side_linears"):
            PoetGroup(lins, side_linears=bad)
    # both sides of each named linear; the class rule is not consulted
    assert PoetGroup._side_class([lins[0].L.R, lins[0].L.P, lins[1].L.R, lins[1].L.P], [1]) == [2, 3]
