"""Thin ctypes binding of the POET C ABI (``include/poet.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of ``libpoet.so``. The functions
carry the C names and take torch tensors that live on the GPU (torch provides device memory and the current
HIP stream). Before each call the binding checks that every tensor is a contiguous device tensor of the
expected dtype holding at least the bytes the call will touch, so that a wrong buffer becomes a Python
exception instead of an out-of-bounds access. A missing library raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpoet.so")

POET_OK, POET_E_ARG, POET_E_SHAPE, POET_E_DTYPE, POET_E_WORKSPACE, POET_E_HIP, POET_E_UNSUPPORTED = range(7)
POET_BS, POET_FS = 0, 1
POET_F32, POET_BF16 = 0, 1
POET_SIDE_R, POET_SIDE_P = 0, 1
POET_OP_BUILD, POET_OP_FWD, POET_OP_BWD, POET_OP_MERGE, POET_OP_FWD_ACT, POET_OP_BWD_ACT = range(6)
POET_MAX_K, POET_MAX_PRIM = 16, 8192
POET_BUILD_STEP, POET_BUILD_MERGE = 0, 1

EXPORTS = ("poet_theta_len", "poet_num_prims", "poet_prim_len", "poet_powers_len", "poet_workspace_bytes",
           "poet_sample_workspace_bytes", "poet_build_workspace_bytes", "poet_build_orthogonal",
           "poet_sample_indices", "poet_linear_fwd", "poet_linear_bwd", "poet_merge", "poet_status_string",
           "poet_last_error", "poet_version", "poet_profile_enable", "poet_profile_query", "poet_debug_gemm",
           "poet_mfma_probe", "poet_sample_permutation", "poet_gather2d", "poet_fs_form_workspace_bytes",
           "poet_fs_form", "poet_linear_fwd_formed", "poet_linear_bwd_formed_prims",
           "poet_act_path_supported", "poet_weight_shadow", "poet_linear_fwd_act", "poet_linear_bwd_act",
           "poet_linear_bwd_act_prims", "poet_build_group_workspace_bytes", "poet_build_orthogonal_group",
           "poet_adjoint_group_workspace_bytes", "poet_adjoint_group", "poet_linear_bwd_prims",
           "poet_merge_group_workspace_bytes", "poet_merge_group", "poet_linear_fwd_folded",
           "poet_linear_bwd_folded_prims", "poet_fold_group_workspace_bytes", "poet_fold_weights_group",
           "poet_sample_indices_noalloc", "poet_adamw_group", "poet_optimizer_reset_group",
           "poet_spectral_workspace_bytes", "poet_hyperspherical_energy", "poet_singular_value_entropy",
           "poet_build_orthogonal_exact")
POET_NOALLOC_MAX_D = 65536  # largest d poet_sample_indices_noalloc accepts (its device scratch holds d int32 flags)
POET_K_TOKEN_FWD, POET_K_TOKEN_DX, POET_K_TOKEN_GW, POET_K_CHAIN, POET_K_ADJOINT, POET_K_APPLY, POET_K_CONTRACT, \
    POET_K_MISC, POET_K_MERGE, POET_K_GATHER, POET_K_OPTIM, POET_K_DIAG = range(12)
KCLASS_NAMES = ("token_fwd", "token_dx", "token_gw", "chain", "adjoint", "apply", "contract", "misc", "merge",
                "gather", "optim", "diag")


class PoetError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class poet_adamw(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float)]


def adamw(lr: float = 1e-5, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
          weight_decay: float = 0.0) -> poet_adamw:
    return poet_adamw(lr, beta1, beta2, eps, weight_decay)


class poet_side(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("d", ctypes.c_int32), ("b", ctypes.c_int32), ("k", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class poet_layer(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("T", ctypes.c_int32), ("ldw", ctypes.c_int32),
                ("ldx", ctypes.c_int32), ("ldy", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("R", poet_side), ("P", poet_side)]


class poet_gemm_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("Mtot", ctypes.c_int32),
                ("Ntot", ctypes.c_int32), ("Ktot", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("sA", ctypes.c_int64), ("a_dt", ctypes.c_int32),
                ("a_kmajor", ctypes.c_int32),
                ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("sB", ctypes.c_int64), ("b_dt", ctypes.c_int32),
                ("b_kmajor", ctypes.c_int32),
                ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("sC", ctypes.c_int64), ("c_dt", ctypes.c_int32),
                ("C2", ctypes.c_void_p), ("ldc2", ctypes.c_int64), ("sC2", ctypes.c_int64), ("c2_dt", ctypes.c_int32),
                ("D", ctypes.c_void_p), ("ldd", ctypes.c_int64), ("sD", ctypes.c_int64),
                ("Acc", ctypes.c_void_p), ("ldacc", ctypes.c_int64), ("sAcc", ctypes.c_int64),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("gamma", ctypes.c_float),
                ("compute", ctypes.c_int32), ("part", ctypes.c_void_p), ("part_elems", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpoet.so (built by ``orthogonal_reparameterized_amd.build``); raise when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"POET HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I32, U32, U64, VP = (ctypes.POINTER, ctypes.c_size_t, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64,
                               ctypes.c_void_p)
    for nm in ("poet_theta_len", "poet_num_prims", "poet_prim_len", "poet_powers_len"):
        getattr(L, nm).argtypes = [P(poet_side)]
        getattr(L, nm).restype = S
    L.poet_workspace_bytes.argtypes = [P(poet_layer), ctypes.c_int]
    L.poet_workspace_bytes.restype = S
    L.poet_sample_workspace_bytes.argtypes = [I32]
    L.poet_sample_workspace_bytes.restype = S
    L.poet_build_workspace_bytes.argtypes = [P(poet_side), ctypes.c_int]
    L.poet_build_workspace_bytes.restype = S
    L.poet_build_orthogonal.argtypes = [P(poet_side), VP, VP, VP, VP, I32, VP, S, VP]
    L.poet_sample_indices.argtypes = [I32, I32, U64, U32, U32, U32, VP, VP, S, VP]
    L.poet_sample_indices_noalloc.argtypes = [I32, I32, U64, U32, U32, U32, VP, VP]
    L.poet_linear_fwd.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_linear_bwd.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_merge.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, U64, U32, U32, VP, S, VP]
    L.poet_act_path_supported.argtypes = [P(poet_layer)]
    L.poet_weight_shadow.argtypes = [P(poet_layer), VP, VP, VP]
    L.poet_linear_fwd_act.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_linear_bwd_act.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_linear_bwd_prims.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_fs_form_workspace_bytes.argtypes = [P(poet_layer)]
    L.poet_fs_form_workspace_bytes.restype = S
    L.poet_fs_form.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_linear_fwd_formed.argtypes = [P(poet_layer), VP, VP, VP, VP]
    L.poet_linear_bwd_formed_prims.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_linear_bwd_act_prims.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_build_group_workspace_bytes.argtypes = [I32, P(poet_side)]
    L.poet_build_group_workspace_bytes.restype = S
    L.poet_build_orthogonal_group.argtypes = [I32, P(poet_side), P(VP), P(VP), P(VP), P(VP), I32, VP, S, VP]
    L.poet_adjoint_group_workspace_bytes.argtypes = [I32, P(poet_side)]
    L.poet_adjoint_group_workspace_bytes.restype = S
    L.poet_adjoint_group.argtypes = [I32, P(poet_side), P(VP), P(VP), P(VP), VP, S, VP]
    L.poet_adamw_group.argtypes = [I32, P(poet_side), P(VP), P(VP), P(VP), P(VP), P(poet_adamw), I32, VP]
    L.poet_build_orthogonal_exact.argtypes = [P(poet_side), VP, VP, VP]
    L.poet_spectral_workspace_bytes.argtypes = [I32, I32]
    L.poet_spectral_workspace_bytes.restype = S
    L.poet_hyperspherical_energy.argtypes = [I32, I32, VP, ctypes.c_int64, ctypes.c_float, VP, VP, VP, S, VP]
    L.poet_singular_value_entropy.argtypes = [I32, I32, VP, ctypes.c_int64, VP, VP, VP, S, VP]
    L.poet_optimizer_reset_group.argtypes = [I32, P(poet_side), P(VP), P(VP), VP]
    L.poet_linear_fwd_folded.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_linear_bwd_folded_prims.argtypes = [P(poet_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, S, VP]
    L.poet_fold_group_workspace_bytes.argtypes = [I32, P(poet_layer)]
    L.poet_fold_group_workspace_bytes.restype = S
    L.poet_fold_weights_group.argtypes = [I32, P(poet_layer), P(VP), P(VP), P(VP), P(VP), P(VP), P(VP), P(VP), VP, S,
                                          VP]
    L.poet_merge_group_workspace_bytes.argtypes = [I32, P(poet_layer)]
    L.poet_merge_group_workspace_bytes.restype = S
    L.poet_merge_group.argtypes = [I32, P(poet_layer), P(VP), P(VP), P(VP), P(VP), P(VP), P(VP), P(VP), P(VP), U64,
                                   P(U32), U32, VP, S, VP]
    for nm in ("poet_build_orthogonal", "poet_sample_indices", "poet_sample_indices_noalloc", "poet_linear_fwd",
               "poet_linear_bwd", "poet_merge", "poet_act_path_supported", "poet_weight_shadow", "poet_linear_fwd_act", "poet_linear_bwd_act"):
        getattr(L, nm).restype = ctypes.c_int
    L.poet_status_string.argtypes = [ctypes.c_int]
    L.poet_status_string.restype = ctypes.c_char_p
    L.poet_last_error.restype = ctypes.c_char_p
    L.poet_version.restype = ctypes.c_char_p
    L.poet_profile_enable.argtypes = [ctypes.c_int]
    L.poet_profile_enable.restype = None
    L.poet_profile_query.argtypes = [ctypes.c_int, P(ctypes.c_int64), P(ctypes.c_double), P(ctypes.c_double),
                                     P(ctypes.c_double)]
    L.poet_profile_query.restype = ctypes.c_int
    L.poet_debug_gemm.argtypes = [P(poet_gemm_desc), ctypes.c_int, P(ctypes.c_int), VP]
    L.poet_debug_gemm.restype = ctypes.c_int
    L.poet_mfma_probe.argtypes = [ctypes.c_int64, ctypes.c_int32, VP, VP]
    L.poet_mfma_probe.restype = ctypes.c_int
    L.poet_sample_permutation.argtypes = [I32, U64, U32, U32, U32, VP, VP, VP]
    L.poet_sample_permutation.restype = ctypes.c_int
    L.poet_gather2d.argtypes = [I32, I32, I32, VP, ctypes.c_int64, I32, I32, VP, VP, VP, ctypes.c_int64, VP]
    L.poet_gather2d.restype = ctypes.c_int
    _lib = L
    return L


# ---- structs -------------------------------------------------------------------------------------------

def side(mode: int, d: int, b: int, k: int, dtype: int) -> poet_side:
    return poet_side(mode, d, b, k, dtype)


def side_of(spec) -> poet_side:
    """poet_side from any object with mode, d, b, k, dtype attributes."""
    return poet_side(spec.mode, spec.d, spec.b, spec.k, spec.dtype)


def layer(m: int, n: int, T: int, R: poet_side, P: poet_side, act_dtype: int, ldw: Optional[int] = None,
          ldx: Optional[int] = None, ldy: Optional[int] = None) -> poet_layer:
    return poet_layer(m, n, T, ldw or n, ldx or n, ldy or m, act_dtype, R, P)


# ---- sizes ---------------------------------------------------------------------------------------------

def poet_theta_len(s: poet_side) -> int:
    return lib().poet_theta_len(ctypes.byref(s))


def poet_num_prims(s: poet_side) -> int:
    return lib().poet_num_prims(ctypes.byref(s))


def poet_prim_len(s: poet_side) -> int:
    return lib().poet_prim_len(ctypes.byref(s))


def poet_powers_len(s: poet_side) -> int:
    return lib().poet_powers_len(ctypes.byref(s))


def poet_workspace_bytes(L: poet_layer, op: int) -> int:
    return lib().poet_workspace_bytes(ctypes.byref(L), op)


def poet_sample_workspace_bytes(d: int) -> int:
    return lib().poet_sample_workspace_bytes(d)


def poet_build_workspace_bytes(s: poet_side, with_powers: bool) -> int:
    return lib().poet_build_workspace_bytes(ctypes.byref(s), int(bool(with_powers)))


def poet_status_string(st: int) -> str:
    return lib().poet_status_string(st).decode()


def poet_last_error() -> str:
    return lib().poet_last_error().decode()


def poet_version() -> str:
    return lib().poet_version().decode()


def poet_profile_enable(on: bool) -> None:
    lib().poet_profile_enable(int(bool(on)))


def poet_debug_gemm(desc: poet_gemm_desc, force_generic: bool = False, stream=None) -> bool:
    """Run one internal GEMM (kernel-level tests). The caller fills the descriptor with device pointers whose
    buffers it has sized for the described extents. Returns whether the bf16 fast kernel ran."""
    used = ctypes.c_int(0)
    _check(lib().poet_debug_gemm(ctypes.byref(desc), int(bool(force_generic)), ctypes.byref(used), _stream(stream)),
           "poet_debug_gemm")
    return bool(used.value)


def poet_sample_permutation(d: int, seed: int, linear_id: int, side: int, epoch: int, perm, inv=None,
                            stream=None) -> None:
    """perm[r] = the index of rank r (int32 device tensor [d]); inv[i] = the rank of index i (nullable)."""
    _check(lib().poet_sample_permutation(int(d), int(seed), int(linear_id), int(side), int(epoch),
                                         _ptr(perm, "perm", 4 * d, "int32"),
                                         _ptr(inv, "inv", 4 * d, "int32", allow_none=True), _stream(stream)),
           "poet_sample_permutation")


def poet_gather2d(inp, out, row_idx=None, col_idx=None, stream=None) -> None:
    """out[i][j] = inp[row_idx[i]][col_idx[j]] for 2-D device tensors of 2- or 4-byte elements (rows written: the
    length of row_idx, else inp's rows; columns: the length of col_idx, else inp's columns)."""
    torch = _torch()
    if inp.dim() != 2 or out.dim() != 2 or inp.element_size() != out.element_size():
        raise ValueError("inp and out must be 2-D tensors of one element size")
    if inp.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("inp and out must have unit column stride")
    if not (inp.is_cuda and out.is_cuda):
        raise ValueError("inp and out must be GPU tensors")
    rows = row_idx.numel() if row_idx is not None else inp.shape[0]
    cols = col_idx.numel() if col_idx is not None else inp.shape[1]
    if out.shape[0] < rows or out.shape[1] < cols:
        raise ValueError(f"out is {tuple(out.shape)}, the gather writes {rows} x {cols}")
    for t, nm in ((row_idx, "row_idx"), (col_idx, "col_idx")):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()):
            raise TypeError(f"{nm} must be a contiguous int32 GPU tensor")
    _check(lib().poet_gather2d(rows, cols, inp.element_size(), ctypes.c_void_p(inp.data_ptr()), inp.stride(0),
                               inp.shape[0], inp.shape[1],
                               None if row_idx is None else ctypes.c_void_p(row_idx.data_ptr()),
                               None if col_idx is None else ctypes.c_void_p(col_idx.data_ptr()),
                               ctypes.c_void_p(out.data_ptr()), out.stride(0), _stream(stream)), "poet_gather2d")


def poet_mfma_probe(iters: int, workgroups: int, out, stream=None) -> float:
    """Launch the matrix-core rate probe (workgroups x 8 waves, 4 * iters 32x32x16 bf16 MFMAs per wave; out: float32
    device tensor of at least workgroups * 8 elements). Returns the flops it issues; the caller times the launch."""
    _check(lib().poet_mfma_probe(int(iters), int(workgroups), _ptr(out, "out", 4 * 8 * int(workgroups), "float32"),
                                 _stream(stream)), "poet_mfma_probe")
    return 32768.0 * 4 * iters * 8 * workgroups


def poet_profile_query(kclass: int) -> dict:
    n, ms, fl, by = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().poet_profile_query(kclass, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(by)),
           "poet_profile_query")
    return {"launches": n.value, "ms": ms.value, "flops": fl.value, "bytes": by.value}


# ---- marshalling -------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dt_name(dt: int) -> str:
    return "bfloat16" if dt == POET_BF16 else "float32"


def _ptr(t, name: str, nbytes: int, dtype: Optional[str] = None, allow_none: bool = False):
    """Device pointer of tensor t after checking device, contiguity, dtype and size."""
    if t is None:
        if allow_none or nbytes == 0:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and str(t.dtype) != "torch." + dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st: int, where: str):
    if st != POET_OK:
        raise PoetError(st, where, f"{poet_status_string(st)}; {poet_last_error()}")


def _esz(dt: int) -> int:
    return 2 if dt == POET_BF16 else 4


def _side_sizes(s: poet_side):
    return poet_theta_len(s), poet_num_prims(s), poet_prim_len(s), poet_powers_len(s)


# ---- calls ----------------------------------------------------------------------------------------------

def poet_build_orthogonal(s: poet_side, theta, prim, powers=None, qnorm=None, ws=None, stream=None,
                          for_merge: bool = False):
    """Build one side's primitives; for_merge forms the square term of a separate-product bf16 chain to float32
    accuracy (POET_BUILD_MERGE), as a build that precedes a merge takes it."""
    nth, npr, npl, npw = _side_sizes(s)
    need_ws = poet_build_workspace_bytes(s, powers is not None)
    if ws is None and need_ws > 0:  # scratch for the caller that passes none (device memory from torch)
        ws = _torch().empty(need_ws, dtype=_torch().uint8, device=prim.device)
    st = lib().poet_build_orthogonal(
        ctypes.byref(s), _ptr(theta, "theta", 4 * nth, "float32"), _ptr(prim, "prim", 4 * npl, "float32"),
        _ptr(powers, "powers", npw * _esz(s.dtype), _dt_name(s.dtype), allow_none=True),
        _ptr(qnorm, "qnorm", 4 * npr, "float32", allow_none=True),
        POET_BUILD_MERGE if for_merge else POET_BUILD_STEP, _ptr(ws, "ws", need_ws, allow_none=True),
        need_ws if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_build_orthogonal")


def poet_sample_indices(d: int, s: int, seed: int, linear_id: int, side_id: int, epoch: int, idx, ws,
                        stream=None):
    need = poet_sample_workspace_bytes(d)
    st = lib().poet_sample_indices(d, s, seed, linear_id, side_id, epoch, _ptr(idx, "idx", 4 * s, "int32"),
                                   _ptr(ws, "ws", need), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_sample_indices")


def poet_sample_indices_noalloc(d: int, s: int, seed: int, linear_id: int, side_id: int, epoch: int, idx,
                                stream=None):
    """poet_sample_indices without a workspace (the library's own device scratch; d <= POET_NOALLOC_MAX_D).
    Calls that overlap on one GPU share that scratch and race."""
    st = lib().poet_sample_indices_noalloc(d, s, seed, linear_id, side_id, epoch, _ptr(idx, "idx", 4 * s, "int32"),
                                           _stream(stream))
    _check(st, "poet_sample_indices_noalloc")


def _layer_bytes(L: poet_layer):
    e = _esz(L.act_dtype)
    # every row-major buffer holds whole rows of its leading dimension (the kernels may read a row's padding)
    rowsz = lambda rows, ld, cols, es: rows * ld * es  # noqa: E731
    return {"W0": rowsz(L.m, L.ldw, L.n, 4), "W": rowsz(L.m, L.ldw, L.n, e), "X": rowsz(L.T, L.ldx, L.n, e),
            "Y": rowsz(L.T, L.ldy, L.m, e)}


def poet_linear_fwd(L: poet_layer, W0, primR, primP, idxR, idxP, X, Y, W_out=None, ws=None, stream=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_FWD)
    st = lib().poet_linear_fwd(
        ctypes.byref(L), _ptr(W0, "W0", b["W0"], "float32"),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(idxR, "idxR", 4 * L.R.b, "int32", allow_none=True), _ptr(idxP, "idxP", 4 * L.P.b, "int32", allow_none=True),
        _ptr(X, "X", b["X"], act, allow_none=L.T == 0), _ptr(Y, "Y", b["Y"], act, allow_none=L.T == 0),
        _ptr(W_out, "W_out", b["W"], act, allow_none=True), _ptr(ws, "ws", need if W_out is None else 0, allow_none=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_fwd")


def poet_linear_bwd(L: poet_layer, W0, primR, primP, powersR, powersP, idxR, idxP, W, X, dY, dX, dthetaR, dthetaP,
                    ws=None, stream=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_BWD)
    st = lib().poet_linear_bwd(
        ctypes.byref(L), _ptr(W0, "W0", b["W0"], "float32"),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(powersR, "powersR", poet_powers_len(L.R) * _esz(L.R.dtype), _dt_name(L.R.dtype), allow_none=True),
        _ptr(powersP, "powersP", poet_powers_len(L.P) * _esz(L.P.dtype), _dt_name(L.P.dtype), allow_none=True),
        _ptr(idxR, "idxR", 4 * L.R.b, "int32", allow_none=True), _ptr(idxP, "idxP", 4 * L.P.b, "int32", allow_none=True),
        _ptr(W, "W", b["W"], act, allow_none=True),
        _ptr(X, "X", b["X"], act, allow_none=L.T == 0), _ptr(dY, "dY", b["Y"], act, allow_none=L.T == 0),
        _ptr(dX, "dX", b["X"], act, allow_none=True),
        _ptr(dthetaR, "dthetaR", 4 * poet_theta_len(L.R), "float32"),
        _ptr(dthetaP, "dthetaP", 4 * poet_theta_len(L.P), "float32"),
        _ptr(ws, "ws", need if W is None else 0, allow_none=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_bwd")


def poet_linear_bwd_prims(L: poet_layer, W0, primR, primP, idxR, idxP, W, X, dY, dX, dprimR, dprimP, ws=None,
                          stream=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_BWD)
    st = lib().poet_linear_bwd_prims(
        ctypes.byref(L), _ptr(W0, "W0", b["W0"], "float32"),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(idxR, "idxR", 4 * L.R.b, "int32", allow_none=True), _ptr(idxP, "idxP", 4 * L.P.b, "int32", allow_none=True),
        _ptr(W, "W", b["W"], act, allow_none=True),
        _ptr(X, "X", b["X"], act, allow_none=L.T == 0), _ptr(dY, "dY", b["Y"], act, allow_none=L.T == 0),
        _ptr(dX, "dX", b["X"], act, allow_none=True),
        _ptr(dprimR, "dprimR", 4 * poet_prim_len(L.R), "float32"),
        _ptr(dprimP, "dprimP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(ws, "ws", need if W is None else 0, allow_none=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_bwd_prims")


def fs_operand_shapes(L: poet_layer) -> dict:
    """Shapes (rows, row pitch) of the bf16 operands poet_fs_form writes besides W: Zr = (W0 P)[I_R, :] and
    Acp = (R W0)[:, I_P]."""
    pad8 = lambda x: (x + 7) // 8 * 8  # noqa: E731
    return {"Zr": (L.R.b, pad8(L.n)), "Acp": (L.m, pad8(L.P.b))}


def poet_fs_form_workspace_bytes(L: poet_layer) -> int:
    return int(lib().poet_fs_form_workspace_bytes(ctypes.byref(L)))


def poet_fs_form(L: poet_layer, W0, primR, primP, idxR, idxP, W, Zr, Acp, ws=None, stream=None):
    """W = R W0 P (bf16) and the FS gradient operands Zr, Acp, formed ahead of the token products."""
    b = _layer_bytes(L)
    sh = fs_operand_shapes(L)
    need = poet_fs_form_workspace_bytes(L)
    st = lib().poet_fs_form(
        ctypes.byref(L), _ptr(W0, "W0", b["W0"], "float32"),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(idxR, "idxR", 4 * L.R.b, "int32"), _ptr(idxP, "idxP", 4 * L.P.b, "int32"),
        _ptr(W, "W", b["W"], "bfloat16"), _ptr(Zr, "Zr", 2 * sh["Zr"][0] * sh["Zr"][1], "bfloat16"),
        _ptr(Acp, "Acp", 2 * sh["Acp"][0] * sh["Acp"][1], "bfloat16"), _ptr(ws, "ws", need, allow_none=need == 0),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_fs_form")


def poet_linear_fwd_formed(L: poet_layer, W, X, Y, stream=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    st = lib().poet_linear_fwd_formed(ctypes.byref(L), _ptr(W, "W", b["W"], act),
                                      _ptr(X, "X", b["X"], act, allow_none=L.T == 0),
                                      _ptr(Y, "Y", b["Y"], act, allow_none=L.T == 0), _stream(stream))
    _check(st, "poet_linear_fwd_formed")


def poet_linear_bwd_formed_prims(L: poet_layer, W, Zr, Acp, idxR, idxP, X, dY, dX, dprimR, dprimP, ws=None,
                                 stream=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    sh = fs_operand_shapes(L)
    need = poet_workspace_bytes(L, POET_OP_BWD)
    st = lib().poet_linear_bwd_formed_prims(
        ctypes.byref(L), _ptr(W, "W", b["W"], act), _ptr(Zr, "Zr", 2 * sh["Zr"][0] * sh["Zr"][1], "bfloat16"),
        _ptr(Acp, "Acp", 2 * sh["Acp"][0] * sh["Acp"][1], "bfloat16"),
        _ptr(idxR, "idxR", 4 * L.R.b, "int32"), _ptr(idxP, "idxP", 4 * L.P.b, "int32"),
        _ptr(X, "X", b["X"], act, allow_none=L.T == 0), _ptr(dY, "dY", b["Y"], act, allow_none=L.T == 0),
        _ptr(dX, "dX", b["X"], act, allow_none=True),
        _ptr(dprimR, "dprimR", 4 * poet_prim_len(L.R), "float32"),
        _ptr(dprimP, "dprimP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(ws, "ws", need, allow_none=True), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_bwd_formed_prims")


def poet_act_path_supported(L: poet_layer) -> bool:
    return bool(lib().poet_act_path_supported(ctypes.byref(L)))


def poet_weight_shadow(L: poet_layer, W0, W0_shadow, stream=None):
    b = _layer_bytes(L)
    st = lib().poet_weight_shadow(ctypes.byref(L), _ptr(W0, "W0", b["W0"], "float32"),
                                  _ptr(W0_shadow, "W0_shadow", b["W"], _dt_name(L.act_dtype)), _stream(stream))
    _check(st, "poet_weight_shadow")


def _ops(t, name, s: poet_side):
    """Operand copies of a side's primitives (3 * prim_len bf16), or None."""
    return _ptr(t, name, 6 * poet_prim_len(s), "bfloat16", allow_none=True)


def poet_linear_fwd_act(L: poet_layer, W0b, primR, primP, X, Y, Z, ws=None, stream=None, opsR=None, opsP=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_FWD_ACT)
    st = lib().poet_linear_fwd_act(
        ctypes.byref(L), _ptr(W0b, "W0b", b["W"], act),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ops(opsR, "opsR", L.R), _ops(opsP, "opsP", L.P),
        _ptr(X, "X", b["X"], act, allow_none=L.T == 0), _ptr(Y, "Y", b["Y"], act, allow_none=L.T == 0),
        _ptr(Z, "Z", b["Y"], act, allow_none=L.T == 0), _ptr(ws, "ws", need, allow_none=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_fwd_act")


def poet_linear_bwd_act(L: poet_layer, W0b, primR, primP, powersR, powersP, X, Z, dY, dX, dthetaR, dthetaP,
                        ws=None, stream=None, opsR=None, opsP=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_BWD_ACT)
    st = lib().poet_linear_bwd_act(
        ctypes.byref(L), _ptr(W0b, "W0b", b["W"], act),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ops(opsR, "opsR", L.R), _ops(opsP, "opsP", L.P),
        _ptr(powersR, "powersR", poet_powers_len(L.R) * _esz(L.R.dtype), _dt_name(L.R.dtype), allow_none=True),
        _ptr(powersP, "powersP", poet_powers_len(L.P) * _esz(L.P.dtype), _dt_name(L.P.dtype), allow_none=True),
        _ptr(X, "X", b["X"], act, allow_none=L.T == 0), _ptr(Z, "Z", b["Y"], act, allow_none=L.T == 0),
        _ptr(dY, "dY", b["Y"], act, allow_none=L.T == 0), _ptr(dX, "dX", b["X"], act, allow_none=True),
        _ptr(dthetaR, "dthetaR", 4 * poet_theta_len(L.R), "float32"),
        _ptr(dthetaP, "dthetaP", 4 * poet_theta_len(L.P), "float32"),
        _ptr(ws, "ws", need, allow_none=True), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_bwd_act")


def poet_linear_fwd_folded(L: poet_layer, W0P, primR, X, Y, Z, ws=None, stream=None, opsR=None):
    """Activation-side forward with P folded into the weight beforehand: Z = X W0P^T, Y = Z R^T."""
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_FWD_ACT)
    st = lib().poet_linear_fwd_folded(
        ctypes.byref(L), _ptr(W0P, "W0P", b["W"], act), _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"),
        _ops(opsR, "opsR", L.R), _ptr(X, "X", b["X"], act, allow_none=L.T == 0),
        _ptr(Y, "Y", b["Y"], act, allow_none=L.T == 0), _ptr(Z, "Z", b["Y"], act, allow_none=L.T == 0),
        _ptr(ws, "ws", need, allow_none=True), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_fwd_folded")


def poet_linear_bwd_folded_prims(L: poet_layer, RW0, primP, X, Z, dY, dX, dprimR, dprimP, ws=None, stream=None,
                                 opsP=None):
    """Activation-side backward with R folded into the weight beforehand (dX' = dY RW0), up to dprimR, dprimP."""
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_BWD_ACT)
    st = lib().poet_linear_bwd_folded_prims(
        ctypes.byref(L), _ptr(RW0, "RW0", b["W"], act), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ops(opsP, "opsP", L.P), _ptr(X, "X", b["X"], act, allow_none=L.T == 0),
        _ptr(Z, "Z", b["Y"], act, allow_none=L.T == 0), _ptr(dY, "dY", b["Y"], act, allow_none=L.T == 0),
        _ptr(dX, "dX", b["X"], act, allow_none=True), _ptr(dprimR, "dprimR", 4 * poet_prim_len(L.R), "float32"),
        _ptr(dprimP, "dprimP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(ws, "ws", need, allow_none=True), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_bwd_folded_prims")


def poet_linear_bwd_act_prims(L: poet_layer, W0b, primR, primP, X, Z, dY, dX, dprimR, dprimP, ws=None, stream=None,
                              opsR=None, opsP=None):
    b = _layer_bytes(L)
    act = _dt_name(L.act_dtype)
    need = poet_workspace_bytes(L, POET_OP_BWD_ACT)
    st = lib().poet_linear_bwd_act_prims(
        ctypes.byref(L), _ptr(W0b, "W0b", b["W"], act),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ops(opsR, "opsR", L.R), _ops(opsP, "opsP", L.P),
        _ptr(X, "X", b["X"], act, allow_none=L.T == 0), _ptr(Z, "Z", b["Y"], act, allow_none=L.T == 0),
        _ptr(dY, "dY", b["Y"], act, allow_none=L.T == 0), _ptr(dX, "dX", b["X"], act, allow_none=True),
        _ptr(dprimR, "dprimR", 4 * poet_prim_len(L.R), "float32"),
        _ptr(dprimP, "dprimP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(ws, "ws", need, allow_none=True), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_linear_bwd_act_prims")


def _side_array(sides):
    arr = (poet_side * max(1, len(sides)))()
    for i, s in enumerate(sides):
        arr[i] = s
    return arr


def _ptr_table(ts, names, sizes, dtypes, allow_none):
    tab = (ctypes.c_void_p * max(1, len(ts)))()
    for i, t in enumerate(ts):
        p = _ptr(t, names[i], sizes[i], dtypes[i], allow_none=allow_none[i])
        tab[i] = None if p is None else p.value
    return tab


def poet_build_group_workspace_bytes(sides) -> int:
    return int(lib().poet_build_group_workspace_bytes(len(sides), _side_array(sides)))


def poet_adjoint_group_workspace_bytes(sides) -> int:
    return int(lib().poet_adjoint_group_workspace_bytes(len(sides), _side_array(sides)))


def poet_build_orthogonal_group(sides, thetas, prims, powers, ws=None, stream=None, ops=None, for_merge=False):
    """poet_build_orthogonal for every side in ``sides`` (lists of equal length; powers required for k >= 1);
    ``ops`` (optional list, entries may be None) receives the bf16 operand copies of the BS sides' primitives;
    for_merge as in poet_build_orthogonal."""
    n = len(sides)
    if not (len(thetas) == len(prims) == len(powers) == n) or (ops is not None and len(ops) != n):
        raise ValueError("sides, thetas, prims, powers (and ops) must have the same length")
    need = poet_build_group_workspace_bytes(sides)
    if ws is None and need > 0:
        ws = _torch().empty(need, dtype=_torch().uint8, device=prims[0].device)
    th = _ptr_table(thetas, [f"thetas[{i}]" for i in range(n)], [4 * poet_theta_len(s) for s in sides],
                    ["float32"] * n, [False] * n)
    pr = _ptr_table(prims, [f"prims[{i}]" for i in range(n)], [4 * poet_prim_len(s) for s in sides],
                    ["float32"] * n, [False] * n)
    pw = _ptr_table(powers, [f"powers[{i}]" for i in range(n)],
                    [poet_powers_len(s) * _esz(s.dtype) for s in sides], [_dt_name(s.dtype) for s in sides],
                    [s.k == 0 for s in sides])
    op = None if ops is None else _ptr_table(ops, [f"ops[{i}]" for i in range(n)],
                                             [6 * poet_prim_len(s) for s in sides], ["bfloat16"] * n, [True] * n)
    st = lib().poet_build_orthogonal_group(n, _side_array(sides), th, pr, pw, op,
                                           POET_BUILD_MERGE if for_merge else POET_BUILD_STEP,
                                           _ptr(ws, "ws", need, allow_none=True),
                                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_build_orthogonal_group")


def poet_adjoint_group(sides, dprims, powers, dthetas, ws=None, stream=None):
    """Neumann adjoint + skew projection of every side in ``sides`` from its primitive gradient."""
    n = len(sides)
    if not (len(dprims) == len(powers) == len(dthetas) == n):
        raise ValueError("sides, dprims, powers and dthetas must have the same length")
    need = poet_adjoint_group_workspace_bytes(sides)
    if ws is None and need > 0:
        ws = _torch().empty(need, dtype=_torch().uint8, device=dprims[0].device)
    skip = [poet_theta_len(s) == 0 for s in sides]
    dp = _ptr_table(dprims, [f"dprims[{i}]" for i in range(n)], [4 * poet_prim_len(s) for s in sides],
                    ["float32"] * n, skip)
    pw = _ptr_table(powers, [f"powers[{i}]" for i in range(n)],
                    [poet_powers_len(s) * _esz(s.dtype) for s in sides], [_dt_name(s.dtype) for s in sides],
                    [sk or s.k == 0 for sk, s in zip(skip, sides)])
    dt = _ptr_table(dthetas, [f"dthetas[{i}]" for i in range(n)], [4 * poet_theta_len(s) for s in sides],
                    ["float32"] * n, skip)
    st = lib().poet_adjoint_group(n, _side_array(sides), dp, pw, dt, _ptr(ws, "ws", need, allow_none=True),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_adjoint_group")


def poet_adamw_group(sides, thetas, dthetas, ms, vs, hp: poet_adamw, step: int, stream=None):
    """One AdamW step on the packed skew parameters of every side (theta, m, v updated in place); ``step`` counts
    the steps since the last reset, from 1."""
    n = len(sides)
    if not (len(thetas) == len(dthetas) == len(ms) == len(vs) == n):
        raise ValueError("sides, thetas, dthetas, ms and vs must have the same length")
    skip = [poet_theta_len(s) == 0 for s in sides]
    sz = [4 * poet_theta_len(s) for s in sides]
    tabs = [_ptr_table(t, [f"{nm}[{i}]" for i in range(n)], sz, ["float32"] * n, skip)
            for t, nm in ((thetas, "thetas"), (dthetas, "dthetas"), (ms, "ms"), (vs, "vs"))]
    st = lib().poet_adamw_group(n, _side_array(sides), *tabs, ctypes.byref(hp), int(step), _stream(stream))
    _check(st, "poet_adamw_group")


def poet_optimizer_reset_group(sides, ms, vs, stream=None):
    """Zero the AdamW moments of every side (the optimizer state after merge-then-reinitialize)."""
    n = len(sides)
    if not (len(ms) == len(vs) == n):
        raise ValueError("sides, ms and vs must have the same length")
    skip = [poet_theta_len(s) == 0 for s in sides]
    sz = [4 * poet_theta_len(s) for s in sides]
    mt = _ptr_table(ms, [f"ms[{i}]" for i in range(n)], sz, ["float32"] * n, skip)
    vt = _ptr_table(vs, [f"vs[{i}]" for i in range(n)], sz, ["float32"] * n, skip)
    _check(lib().poet_optimizer_reset_group(n, _side_array(sides), mt, vt, _stream(stream)), "poet_optimizer_reset_group")


def poet_build_orthogonal_exact(s: poet_side, theta, prim, stream=None):
    """Exact Cayley primitives (I + Q)(I - Q)^{-1} of one side (primitives up to 256), float32, identity-padded."""
    st = lib().poet_build_orthogonal_exact(ctypes.byref(s), _ptr(theta, "theta", 4 * poet_theta_len(s), "float32"),
                                           _ptr(prim, "prim", 4 * poet_prim_len(s), "float32"), _stream(stream))
    _check(st, "poet_build_orthogonal_exact")


def poet_spectral_workspace_bytes(m: int, n: int) -> int:
    return int(lib().poet_spectral_workspace_bytes(m, n))


def poet_hyperspherical_energy(m: int, n: int, W, ldw: int, s: float, energy, energy_rows=None, ws=None, stream=None):
    """Hyperspherical energy of the m neurons (rows) of the float32 weight W (row pitch ldw): energy [1] float64
    out, energy_rows [m] float64 out (optional)."""
    need = poet_spectral_workspace_bytes(m, n)
    if ws is None:
        ws = _torch().empty(need, dtype=_torch().uint8, device=W.device)
    st = lib().poet_hyperspherical_energy(m, n, _ptr(W, "W", 4 * ((m - 1) * ldw + n), "float32"), ldw, s,
                                          _ptr(energy_rows, "energy_rows", 8 * m, "float64", allow_none=True),
                                          _ptr(energy, "energy", 8, "float64"), _ptr(ws, "ws", need),
                                          ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_hyperspherical_energy")


def poet_singular_value_entropy(m: int, n: int, W, ldw: int, entropy, sigma=None, ws=None, stream=None):
    """Entropy of the normalized singular values of the float32 weight W (row pitch ldw): entropy [1] float64 out,
    sigma [min(m, n)] float64 out, descending (optional)."""
    need = poet_spectral_workspace_bytes(m, n)
    if ws is None:
        ws = _torch().empty(need, dtype=_torch().uint8, device=W.device)
    st = lib().poet_singular_value_entropy(m, n, _ptr(W, "W", 4 * ((m - 1) * ldw + n), "float32"), ldw,
                                           _ptr(sigma, "sigma", 8 * min(m, n), "float64", allow_none=True),
                                           _ptr(entropy, "entropy", 8, "float64"), _ptr(ws, "ws", need),
                                           ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_singular_value_entropy")


def poet_merge(L: poet_layer, W0, W0_shadow, thetaR, thetaP, primR, primP, idxR, idxP, seed: int, linear_id: int,
               epoch_next: int, ws=None, stream=None):
    b = _layer_bytes(L)
    need = poet_workspace_bytes(L, POET_OP_MERGE)
    st = lib().poet_merge(
        ctypes.byref(L), _ptr(W0, "W0", b["W0"], "float32"),
        _ptr(W0_shadow, "W0_shadow", b["W"], _dt_name(L.act_dtype), allow_none=True),
        _ptr(thetaR, "thetaR", 4 * poet_theta_len(L.R), "float32"),
        _ptr(thetaP, "thetaP", 4 * poet_theta_len(L.P), "float32"),
        _ptr(primR, "primR", 4 * poet_prim_len(L.R), "float32"), _ptr(primP, "primP", 4 * poet_prim_len(L.P), "float32"),
        _ptr(idxR, "idxR", 4 * L.R.b, "int32", allow_none=True), _ptr(idxP, "idxP", 4 * L.P.b, "int32", allow_none=True),
        seed, linear_id, epoch_next, _ptr(ws, "ws", need, allow_none=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_merge")


def _layer_array(layers):
    arr = (poet_layer * max(1, len(layers)))()
    for i, L in enumerate(layers):
        arr[i] = L
    return arr


def poet_merge_group_workspace_bytes(layers) -> int:
    return int(lib().poet_merge_group_workspace_bytes(len(layers), _layer_array(layers)))


def poet_merge_group(layers, W0s, shadows, thetaRs, thetaPs, primRs, primPs, idxRs, idxPs, seed: int, linear_ids,
                     epoch_next: int, ws=None, stream=None):
    """poet_merge for every layer in ``layers`` (lists of equal length); ``shadows``, ``idxRs`` and ``idxPs`` may
    be None (no shadows, no index sets) or lists with None entries."""
    n = len(layers)
    shadows = [None] * n if shadows is None else shadows
    idxRs = [None] * n if idxRs is None else idxRs
    idxPs = [None] * n if idxPs is None else idxPs
    if not all(len(t) == n for t in (W0s, shadows, thetaRs, thetaPs, primRs, primPs, idxRs, idxPs, linear_ids)):
        raise ValueError("every table must have one entry per layer")
    need = poet_merge_group_workspace_bytes(layers)
    if ws is None and need > 0:
        ws = _torch().empty(need, dtype=_torch().uint8, device=W0s[0].device)
    bs = [_layer_bytes(L) for L in layers]
    idx = lambda i: f"[{i}]"
    w0 = _ptr_table(W0s, ["W0s" + idx(i) for i in range(n)], [b["W0"] for b in bs], ["float32"] * n, [False] * n)
    sh = _ptr_table(shadows, ["shadows" + idx(i) for i in range(n)], [b["W"] for b in bs],
                    [_dt_name(L.act_dtype) for L in layers], [True] * n)
    tR = _ptr_table(thetaRs, ["thetaRs" + idx(i) for i in range(n)], [4 * poet_theta_len(L.R) for L in layers],
                    ["float32"] * n, [poet_theta_len(L.R) == 0 for L in layers])
    tP = _ptr_table(thetaPs, ["thetaPs" + idx(i) for i in range(n)], [4 * poet_theta_len(L.P) for L in layers],
                    ["float32"] * n, [poet_theta_len(L.P) == 0 for L in layers])
    pR = _ptr_table(primRs, ["primRs" + idx(i) for i in range(n)], [4 * poet_prim_len(L.R) for L in layers],
                    ["float32"] * n, [False] * n)
    pP = _ptr_table(primPs, ["primPs" + idx(i) for i in range(n)], [4 * poet_prim_len(L.P) for L in layers],
                    ["float32"] * n, [False] * n)
    iR = _ptr_table(idxRs, ["idxRs" + idx(i) for i in range(n)], [4 * L.R.b for L in layers], ["int32"] * n,
                    [True] * n)
    iP = _ptr_table(idxPs, ["idxPs" + idx(i) for i in range(n)], [4 * L.P.b for L in layers], ["int32"] * n,
                    [True] * n)
    ids = (ctypes.c_uint32 * max(1, n))(*[int(v) for v in linear_ids])
    st = lib().poet_merge_group(n, _layer_array(layers), w0, sh, tR, tP, pR, pP, iR, iP, seed, ids, epoch_next,
                                _ptr(ws, "ws", need, allow_none=True),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_merge_group")


def poet_fold_group_workspace_bytes(layers) -> int:
    return int(lib().poet_fold_group_workspace_bytes(len(layers), _layer_array(layers)))


def poet_fold_weights_group(layers, W0bs, primRs, primPs, W0Ps, RW0s, ws=None, stream=None, opsRs=None, opsPs=None):
    """W0P[i] = W0b[i] P_i and RW0[i] = R_i W0b[i] for every layer (bf16, m x ldw); W0Ps / RW0s (and opsRs / opsPs)
    may be None or lists with None entries."""
    n = len(layers)
    W0Ps = [None] * n if W0Ps is None else W0Ps
    RW0s = [None] * n if RW0s is None else RW0s
    opsRs = [None] * n if opsRs is None else opsRs
    opsPs = [None] * n if opsPs is None else opsPs
    if not all(len(t) == n for t in (W0bs, primRs, primPs, W0Ps, RW0s, opsRs, opsPs)):
        raise ValueError("every table must have one entry per layer")
    need = poet_fold_group_workspace_bytes(layers)
    if ws is None and need > 0:
        ws = _torch().empty(need, dtype=_torch().uint8, device=W0bs[0].device)
    bs = [_layer_bytes(L) for L in layers]
    act = [_dt_name(L.act_dtype) for L in layers]
    nm = lambda t, i: f"{t}[{i}]"
    w0 = _ptr_table(W0bs, [nm("W0bs", i) for i in range(n)], [b["W"] for b in bs], act, [False] * n)
    pR = _ptr_table(primRs, [nm("primRs", i) for i in range(n)], [4 * poet_prim_len(L.R) for L in layers],
                    ["float32"] * n, [w is None for w in RW0s])
    pP = _ptr_table(primPs, [nm("primPs", i) for i in range(n)], [4 * poet_prim_len(L.P) for L in layers],
                    ["float32"] * n, [w is None for w in W0Ps])
    oR = _ptr_table(opsRs, [nm("opsRs", i) for i in range(n)], [6 * poet_prim_len(L.R) for L in layers],
                    ["bfloat16"] * n, [True] * n)
    oP = _ptr_table(opsPs, [nm("opsPs", i) for i in range(n)], [6 * poet_prim_len(L.P) for L in layers],
                    ["bfloat16"] * n, [True] * n)
    fP = _ptr_table(W0Ps, [nm("W0Ps", i) for i in range(n)], [b["W"] for b in bs], act, [True] * n)
    fR = _ptr_table(RW0s, [nm("RW0s", i) for i in range(n)], [b["W"] for b in bs], act, [True] * n)
    st = lib().poet_fold_weights_group(n, _layer_array(layers), w0, pR, pP, oR, oP, fP, fR,
                                       _ptr(ws, "ws", need, allow_none=True),
                                       0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "poet_fold_weights_group")
