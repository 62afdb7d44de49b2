"""Kernel-level checks of the library's GEMMs through the diagnostic entry point poet_debug_gemm.

Operands are random bf16 values; the reference is the float64 product of exactly those values, so the only
legitimate differences are float32 accumulation order and the rounding of the stored output. That makes the
bound tight enough to expose any missing or misplaced term (a dropped k-tile, a wrong block, an epilogue that
skips rows): float32 outputs must agree to 2e-6 relative Frobenius and 2e-5 of the output scale elementwise,
bf16 outputs to one bf16 rounding (2^-8 relative) plus that. Every case runs on the bf16 fast kernel (asserted)
and on the generic kernel.
"""
import zlib

import numpy as np
import pytest

from tests.gpu_util import announce

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dt)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _logical(buf, off, ld, rows, cols, kmajor_rows):
    """rows x cols logical matrix from a flat buffer: element (i, j) at off + i*ld + j when kmajor_rows else
    off + j*ld + i."""
    if kmajor_rows:
        return np.stack([buf[off + i * ld: off + i * ld + cols] for i in range(rows)]) if rows else np.zeros((0, cols))
    return np.stack([buf[off + j * ld: off + j * ld + rows] for j in range(cols)]).T if cols else np.zeros((rows, 0))


CASES = [
    # name, M, N, K, batch, (Mtot, Ntot, Ktot), a_kmajor, b_kmajor, out fp32?, epilogue extras, split-K scratch
    ("nt_ragged_plain_bf16", 300, 520, 1000, 1, (0, 0, 0), 1, 1, False, {}, False),
    ("nn_epilogue_all", 1024, 384, 200, 1, (0, 0, 0), 1, 0, True, {"alpha": -1.0, "D": 2.0, "Acc": 1.5, "C2": True}, False),
    ("tn_splitk", 640, 256, 4096, 1, (0, 0, 0), 0, 0, True, {"D": 1.0}, True),
    ("tk_kmajor_b", 256, 384, 500, 1, (0, 0, 0), 0, 1, False, {}, False),
    ("tn_splitk_bf16_out", 384, 300, 3000, 1, (0, 0, 0), 0, 0, False, {}, True),
    ("batched_ragged_blocks", 256, 256, 256, 3, (600, 600, 600), 1, 0, True, {"D": 1.0, "C2": True}, False),
    ("batched_ragged_splitk", 256, 256, 2048, 3, (700, 700, 0), 1, 1, True, {}, True),
    ("k_zero", 256, 256, 0, 1, (0, 0, 0), 0, 0, True, {"D": 1.0}, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("generic", [False, True])
def test_gemm_against_float64(case, generic):
    from orthogonal_reparameterized_amd import binding as B
    name, M, N, K, batch, tots, ak, bk, out32, ex, use_part = case
    announce(f"gemm {name} generic={generic}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    Mt, Nt, Kt = tots
    ext = lambda tot, d, z: min(d, tot - z * d) if tot > 0 else d  # noqa: E731
    blocky = bool(Mt or Nt or Kt)
    # Storage of an operand: (row dimension, column dimension) of its stored matrix. With ragged totals the
    # batches are blocks of one larger matrix, offset by z * dim along every dimension that has a total (a
    # block-diagonal layout, as the factors of one side); otherwise each batch is a separate full matrix.
    a_dims = ((M, Mt), (K, Kt)) if ak else ((K, Kt), (M, Mt))
    b_dims = ((N, Nt), (K, Kt)) if bk else ((K, Kt), (N, Nt))
    grow = lambda dim, tot: dim * batch if (blocky and tot > 0) else dim  # noqa: E731
    Arows, Acols = grow(*a_dims[0]), grow(*a_dims[1])
    Brows, Bcols = grow(*b_dims[0]), grow(*b_dims[1])
    lda = ((Acols + 7) // 8) * 8 + 8
    ldb = ((Bcols + 7) // 8) * 8 + 8
    nA = max(Arows, 1) * lda * (1 if blocky else batch)
    nB = max(Brows, 1) * ldb * (1 if blocky else batch)
    A = (rng.standard_normal(nA) * 0.5).astype(np.float32)
    Bv = (rng.standard_normal(nB) * 0.5).astype(np.float32)
    Ad, Bd = _dev(A, torch.bfloat16), _dev(Bv, torch.bfloat16)
    A64, B64 = _np(Ad), _np(Bd)

    def off(z, dims, rows, ld):
        if not blocky:
            return z * max(rows, 1) * ld
        (dr, tr), (dc, tc) = dims
        return (z * dr if tr > 0 else 0) * ld + (z * dc if tc > 0 else 0)

    def a_off(z):
        return off(z, a_dims, Arows, lda)

    def b_off(z):
        return off(z, b_dims, Brows, ldb)
    sA = a_off(1) if batch > 1 else 0
    sB = b_off(1) if batch > 1 else 0
    ldc = N + 16
    rowsC = M * batch
    Cdt = torch.float32 if out32 else torch.bfloat16
    Cd = torch.full((rowsC * ldc,), float("nan"), dtype=Cdt, device="cuda")
    C2d = torch.full((rowsC * ldc,), float("nan"), dtype=torch.bfloat16, device="cuda") if ex.get("C2") else None
    Dd = _dev((rng.standard_normal(rowsC * ldc)).astype(np.float32), torch.float32) if "D" in ex else None
    Accd = _dev((rng.standard_normal(rowsC * ldc)).astype(np.float32), torch.float32) if "Acc" in ex else None
    Acc0 = _np(Accd) if Accd is not None else None
    # float32 scratch: ample for split-K when the case asks for it; otherwise exactly one float per output when
    # the epilogue needs one (an addend, a second output, an accumulator, a scale), so one split goes through
    # the partial-tile + reduction path; none at all for a plain store
    plain = not ("D" in ex or "C2" in ex or "Acc" in ex or "alpha" in ex)
    n_part = 16 * batch * M * N + 1 if use_part else (0 if plain else batch * M * N)
    part = torch.empty(n_part, dtype=torch.float32, device="cuda") if n_part else None

    d = B.poet_gemm_desc()
    d.M, d.N, d.K, d.Mtot, d.Ntot, d.Ktot, d.batch = M, N, K, Mt, Nt, Kt, batch
    d.A, d.lda, d.sA, d.a_dt, d.a_kmajor = Ad.data_ptr(), lda, sA, 1, ak
    d.B, d.ldb, d.sB, d.b_dt, d.b_kmajor = Bd.data_ptr(), ldb, sB, 1, bk
    d.C, d.ldc, d.sC, d.c_dt = Cd.data_ptr(), ldc, M * ldc, 0 if out32 else 1
    if C2d is not None:
        d.C2, d.ldc2, d.sC2, d.c2_dt = C2d.data_ptr(), ldc, M * ldc, 1
    if Dd is not None:
        d.D, d.ldd, d.sD, d.beta = Dd.data_ptr(), ldc, M * ldc, ex["D"]
    if Accd is not None:
        d.Acc, d.ldacc, d.sAcc, d.gamma = Accd.data_ptr(), ldc, M * ldc, ex["Acc"]
    d.alpha = ex.get("alpha", 1.0)
    d.compute = 1
    if part is not None:
        d.part, d.part_elems = part.data_ptr(), part.numel()
    fast = B.poet_debug_gemm(d, force_generic=generic)
    torch.cuda.synchronize()
    assert fast == (not generic)

    Cg = _np(Cd)
    C2g = _np(C2d) if C2d is not None else None
    Accg = _np(Accd) if Accd is not None else None
    Dn = _np(Dd) if Dd is not None else None
    for z in range(batch):
        Mz, Nz, Kz = ext(Mt, M, z), ext(Nt, N, z), ext(Kt, K, z)
        Az = _logical(A64, a_off(z), lda, Mz, Kz, True) if ak else _logical(A64, a_off(z), lda, Kz, Mz, True).T
        Bz = _logical(B64, b_off(z), ldb, Nz, Kz, True).T if bk else _logical(B64, b_off(z), ldb, Kz, Nz, True)
        ref = d.alpha * (Az @ Bz) if Kz > 0 else np.zeros((Mz, Nz))
        sl = lambda X: X[z * M * ldc:(z * M + Mz) * ldc].reshape(Mz, ldc)[:, :Nz]  # noqa: E731
        if Dn is not None:
            ref = ref + d.beta * sl(Dn)
        scale = max(np.sqrt(max(Kz, 1)) * 0.25, np.abs(ref).max() if ref.size else 1.0)
        got = sl(Cg)
        err = np.abs(got - ref)
        bound = 2e-5 * scale + (0.0 if out32 else 2.0 ** -8 * np.abs(ref))
        assert np.all(err <= bound), (name, z, float(err.max()), float(scale))
        if out32 and ref.size:
            assert np.linalg.norm(got - ref) <= 2e-6 * max(np.linalg.norm(ref), 1e-30) + 1e-6 * scale
        if C2g is not None:
            assert np.all(np.abs(sl(C2g) - ref) <= 2e-5 * scale + 2.0 ** -8 * np.abs(ref))
        if Accg is not None:
            assert np.all(np.abs(sl(Accg) - (sl(Acc0) + d.gamma * ref)) <= 4e-5 * scale)
        # nothing written outside the batch's extent (rows of this batch beyond Mz keep their NaN fill)
        if Mz < M:
            rest = Cg[(z * M + Mz) * ldc:(z + 1) * M * ldc]
            assert np.all(np.isnan(rest))

