"""Device-resident state of one POET linear and the calls of one training step on it.

``PoetLinear`` owns the GPU buffers of one linear (the fixed weight W0, the skew parameters of R and P, the
FS index sets, the built primitives, the saved Neumann powers and one shared workspace) and issues the C-ABI
calls through the binding. It does no arithmetic of its own.
"""
from __future__ import annotations

from typing import Optional

from . import binding as B


def _torch():
    import torch
    return torch


def _tdt(dt: int):
    torch = _torch()
    return torch.bfloat16 if dt == B.POET_BF16 else torch.float32


def _torch_stream(stream, dev):
    """The torch stream object for a stream argument (None: the current stream; an int: a raw HIP stream handle)."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=dev)
    return stream


def _merge_grade_differs(side: B.poet_side) -> bool:
    """True for sides whose chain runs as separate bf16 products: only their build differs between the step's
    precision and the merge's (poet_build_workspace_bytes(side, 1) > 0 exactly for those)."""
    return B.poet_build_workspace_bytes(side, True) > 0


class PoetLinear:
    """One POET linear W = R W0 P on the GPU.

    R, P are ``poet_side`` structs; W0 is an (m, n) float32 host array (numpy or torch). ``ldw`` pads W0's rows
    (a multiple of 64 elements keeps every row 128-byte aligned). Index sets of FS sides are drawn on the GPU
    with ``poet_sample_indices`` for epoch 0 unless given.

    ``ws`` (optional) is a uint8 device tensor shared with other linears whose calls run one after another on
    one stream (``PoetLinear.workspace_bytes`` gives the size one linear needs).

    ``path`` picks how the factors are applied: "weight" materializes W = R W0 P (poet_linear_fwd/_bwd), "act"
    applies them to the activations around the W0 GEMM (poet_linear_fwd_act/_bwd_act, which keep a bf16 copy
    of W0 that the merge refreshes), "auto" takes "act" wherever the library supports it.
    """

    def __init__(self, m: int, n: int, T: int, R: B.poet_side, P: B.poet_side, act_dtype: int, W0,
                 thetaR=None, thetaP=None, seed: int = 0, linear_id: int = 0, ldw: Optional[int] = None,
                 ldx: Optional[int] = None, ldy: Optional[int] = None, idxR=None, idxP=None, device: str = "cuda",
                 path: str = "weight", ws=None):
        torch = _torch()
        self.dev = torch.device(device)
        self.L = B.layer(m, n, T, R, P, act_dtype, ldw, ldx, ldy)
        if path not in ("weight", "act", "auto"):
            raise ValueError(f"path must be 'weight', 'act' or 'auto', not {path!r}")
        supported = B.poet_act_path_supported(self.L)
        if path == "act" and not supported:
            raise ValueError("the activation-side path needs POET-BS sides and bf16 activations")
        self.act_path = path == "act" or (path == "auto" and supported)
        self.m, self.n, self.T = m, n, T
        self.seed, self.linear_id, self.epoch = seed, linear_id, 0
        self.act = _tdt(act_dtype)
        W0 = torch.as_tensor(W0, dtype=torch.float32)
        self.W0 = torch.zeros((m, self.L.ldw), dtype=torch.float32, device=self.dev)
        self.W0[:, :n] = W0.to(self.dev)
        nR, nP = B.poet_theta_len(R), B.poet_theta_len(P)
        self.thetaR = (torch.zeros(nR) if thetaR is None else torch.as_tensor(thetaR, dtype=torch.float32)).to(self.dev)
        self.thetaP = (torch.zeros(nP) if thetaP is None else torch.as_tensor(thetaP, dtype=torch.float32)).to(self.dev)
        self.primR = torch.empty(B.poet_prim_len(R), dtype=torch.float32, device=self.dev)
        self.primP = torch.empty(B.poet_prim_len(P), dtype=torch.float32, device=self.dev)
        self.powersR = torch.empty(max(B.poet_powers_len(R), 1), dtype=_tdt(R.dtype), device=self.dev)
        self.powersP = torch.empty(max(B.poet_powers_len(P), 1), dtype=_tdt(P.dtype), device=self.dev)
        self.qnormR = torch.empty(B.poet_num_prims(R), dtype=torch.float32, device=self.dev)
        self.qnormP = torch.empty(B.poet_num_prims(P), dtype=torch.float32, device=self.dev)
        self.dthetaR = torch.empty(max(nR, 1), dtype=torch.float32, device=self.dev)
        self.dthetaP = torch.empty(max(nP, 1), dtype=torch.float32, device=self.dev)
        # AdamW moments of the skew parameters and the steps taken since the last reset (a merge resets them)
        self.mR = torch.zeros(max(nR, 1), dtype=torch.float32, device=self.dev)
        self.vR = torch.zeros(max(nR, 1), dtype=torch.float32, device=self.dev)
        self.mP = torch.zeros(max(nP, 1), dtype=torch.float32, device=self.dev)
        self.vP = torch.zeros(max(nP, 1), dtype=torch.float32, device=self.dev)
        self.opt_steps = 0
        self.grad_ready = False  # dthetaR / dthetaP hold the gradient of the current parameters
        wsb = PoetLinear.workspace_bytes(m, n, T, R, P, act_dtype, self.L.ldw, self.L.ldx, self.L.ldy,
                                         "act" if self.act_path else "weight")
        if ws is None:
            self.ws = torch.empty(wsb, dtype=torch.uint8, device=self.dev)
        else:  # shared with other linears whose calls run in order on one stream
            if ws.numel() * ws.element_size() < wsb:
                raise ValueError(f"shared workspace holds {ws.numel() * ws.element_size()} bytes, this linear needs {wsb}")
            self.ws = ws
        self.W0b = None
        # bf16 operand copies of the primitives (both orientations), written by PoetGroup.build; None until then
        # (and after a one-linear build, which leaves them stale)
        self.opsR = self.opsP = None
        # the factors folded into the bf16 weight (W0 P, R W0), written by PoetGroup.build for large token counts;
        # None until then (and after a one-linear build, which leaves them stale)
        self.W0P = self.RW0 = None
        # FS pairs on the weight side: (W, Zr, Acp) = R W0 P and the gradient operands (W0 P)[I_R, :], (R W0)[:, I_P]
        # formed by PoetGroup.build (poet_fs_form); None until then (and after a one-linear build)
        self.formed = None
        self._form_event = None  # recorded on the formation stream after this linear's operands were formed
        self._build_event = None  # recorded on a group's side stream after it built some of this linear's sides
        # True between a build and the next merge: the primitives (and folds, operand copies) match theta and W0
        self.built = False
        if self.act_path:  # W0 in the act dtype, the operand of the activation-side GEMMs
            self.W0b = torch.empty((m, self.L.ldw), dtype=self.act, device=self.dev)
            B.poet_weight_shadow(self.L, self.W0, self.W0b)
        self.idxR = self.idxP = None
        if R.mode == B.POET_FS:
            self.idxR = torch.empty(R.b, dtype=torch.int32, device=self.dev)
            if idxR is None:
                B.poet_sample_indices(m, R.b, seed, linear_id, B.POET_SIDE_R, 0, self.idxR, self.ws)
            else:
                self.idxR.copy_(torch.as_tensor(idxR, dtype=torch.int32))
        if P.mode == B.POET_FS:
            self.idxP = torch.empty(P.b, dtype=torch.int32, device=self.dev)
            if idxP is None:
                B.poet_sample_indices(n, P.b, seed, linear_id, B.POET_SIDE_P, 0, self.idxP, self.ws)
            else:
                self.idxP.copy_(torch.as_tensor(idxP, dtype=torch.int32))

    @staticmethod
    def workspace_bytes(m: int, n: int, T: int, R: B.poet_side, P: B.poet_side, act_dtype: int, ldw=None, ldx=None,
                        ldy=None, path: str = "weight") -> int:
        """Bytes of the workspace one linear of this shape needs (what the constructor allocates)."""
        L = B.layer(m, n, T, R, P, act_dtype, ldw, ldx, ldy)
        act = path == "act" or (path == "auto" and B.poet_act_path_supported(L))
        ops = (B.POET_OP_FWD_ACT, B.POET_OP_BWD_ACT) if act else (B.POET_OP_FWD, B.POET_OP_BWD)
        wsb = max(B.poet_workspace_bytes(L, op) for op in ops + (B.POET_OP_MERGE,))
        return max(wsb, B.poet_sample_workspace_bytes(max(m, n)), B.poet_build_workspace_bytes(R, True),
                   B.poet_build_workspace_bytes(P, True))

    def _powers(self, side: str):
        s = self.L.R if side == "R" else self.L.P
        if B.poet_powers_len(s) == 0:
            return None
        return self.powersR if side == "R" else self.powersP

    def build(self, stream=None, qnorm: bool = False):
        self._await_group(stream)  # a formation still reading the primitives, a side build still writing them
        self.opsR = self.opsP = None  # the one-side build does not write them
        self.W0P = self.RW0 = None
        self.formed = None
        self.built = False
        B.poet_build_orthogonal(self.L.R, self.thetaR, self.primR, self._powers("R"), self.qnormR if qnorm else None,
                                self.ws, stream)
        B.poet_build_orthogonal(self.L.P, self.thetaP, self.primP, self._powers("P"), self.qnormP if qnorm else None,
                                self.ws, stream)
        self.built = True

    def _need_build(self, what: str):
        if not self.built:
            raise RuntimeError(f"{what} needs built factors: call build() (or PoetGroup.build()) after construction "
                               "and after every merge")

    def alloc_act(self, rows: int, ld: int):
        return _torch().empty((rows, ld), dtype=self.act, device=self.dev)

    def alloc_W(self):
        return _torch().empty((self.m, self.L.ldw), dtype=self.act, device=self.dev)

    def forward(self, X, Y, W_out=None, stream=None):
        """Weight-side forward Y = X W^T. W_out (optional) receives W = R W0 P for the backward; where the last
        PoetGroup.build formed W (``formed``), the product reads that W and the layer keeps it (W_out must be None)."""
        self._need_build("forward")
        if self.formed is not None:
            if W_out is not None:
                raise ValueError("this linear keeps the W its group build formed: call forward without W_out")
            self._await_group(stream)
            B.poet_linear_fwd_formed(self.L, self.formed[0], X, Y, stream)
            return
        self._await_group(stream)
        B.poet_linear_fwd(self.L, self.W0, self.primR, self.primP, self.idxR, self.idxP, X, Y, W_out, self.ws, stream)

    def backward(self, X, dY, dX, W=None, stream=None):
        self._need_build("backward")
        self._await_group(stream)
        B.poet_linear_bwd(self.L, self.W0, self.primR, self.primP, self._powers("R"), self._powers("P"), self.idxR,
                          self.idxP, W, X, dY, dX, self.dthetaR, self.dthetaP, self.ws, stream)
        self.grad_ready = True

    def _await_form(self, stream):
        """The launch stream waits, once, for this linear's formation only (a group build: its side stream orders
        itself after the work it left there)."""
        if self._form_event is not None:
            _torch_stream(stream, self.dev).wait_event(self._form_event)
            self._form_event = None

    def _await_group(self, stream):
        """The launch stream waits, once, for this linear's work that a PoetGroup left on its other streams: the
        formation of its FS operands and the build of its sides that ran on the group's side stream (and for nothing
        else on those streams); work on other streams is ordered after it through the launch stream, by the caller."""
        for ev in (self._form_event, self._build_event):
            if ev is not None:
                _torch_stream(stream, self.dev).wait_event(ev)
        self._form_event = self._build_event = None

    def forward_act(self, X, Y, Z, stream=None):
        """Activation-side forward: Y = ((X P^T) W0^T) R^T; Z = X P^T W0^T is kept for backward_act. The bf16
        operand copies of the primitives (and W0 P, folded) come from the last PoetGroup.build, when one made them."""
        self._need_build("forward_act")
        self._await_group(stream)
        if self.W0P is not None:
            B.poet_linear_fwd_folded(self.L, self.W0P, self.primR, X, Y, Z, self.ws, stream, opsR=self.opsR)
        else:
            B.poet_linear_fwd_act(self.L, self.W0b, self.primR, self.primP, X, Y, Z, self.ws, stream,
                                  opsR=self.opsR, opsP=self.opsP)

    def backward_act(self, X, Z, dY, dX, stream=None):
        self._need_build("backward_act")
        self._await_group(stream)
        B.poet_linear_bwd_act(self.L, self.W0b, self.primR, self.primP, self._powers("R"), self._powers("P"), X, Z,
                              dY, dX, self.dthetaR, self.dthetaP, self.ws, stream, opsR=self.opsR, opsP=self.opsP)
        self.grad_ready = True

    def _dprims(self):
        if getattr(self, "dprimR", None) is None:
            torch = _torch()
            self.dprimR = torch.empty(B.poet_prim_len(self.L.R), dtype=torch.float32, device=self.dev)
            self.dprimP = torch.empty(B.poet_prim_len(self.L.P), dtype=torch.float32, device=self.dev)

    def backward_prims(self, X, dY, dX, W=None, stream=None):
        """Weight-side backward up to the primitive gradients dprimR, dprimP; PoetGroup.finish_backward turns them
        into dthetaR, dthetaP for many linears at once."""
        self._need_build("backward_prims")
        self._dprims()
        self.grad_ready = False  # dthetaR / dthetaP come from PoetGroup.finish_backward
        self._await_group(stream)
        if self.formed is not None:  # the operands formed by the group build (W is not used)
            B.poet_linear_bwd_formed_prims(self.L, *self.formed, self.idxR, self.idxP, X, dY, dX, self.dprimR,
                                           self.dprimP, self.ws, stream)
            return
        B.poet_linear_bwd_prims(self.L, self.W0, self.primR, self.primP, self.idxR, self.idxP, W, X, dY, dX,
                                self.dprimR, self.dprimP, self.ws, stream)

    def backward_act_prims(self, X, Z, dY, dX, stream=None):
        """Activation-side backward up to the primitive gradients dprimR, dprimP (the blocks of dL/dR and dL/dP);
        PoetGroup.finish_backward turns them into dthetaR, dthetaP for many linears at once."""
        self._need_build("backward_act_prims")
        self._dprims()
        self.grad_ready = False  # dthetaR / dthetaP come from PoetGroup.finish_backward
        self._await_group(stream)
        if self.RW0 is not None:
            B.poet_linear_bwd_folded_prims(self.L, self.RW0, self.primP, X, Z, dY, dX, self.dprimR, self.dprimP,
                                           self.ws, stream, opsP=self.opsP)
        else:
            B.poet_linear_bwd_act_prims(self.L, self.W0b, self.primR, self.primP, X, Z, dY, dX, self.dprimR,
                                        self.dprimP, self.ws, stream, opsR=self.opsR, opsP=self.opsP)

    def optimizer_step(self, hp: B.poet_adamw, stream=None):
        """One AdamW step on thetaR, thetaP from dthetaR, dthetaP (the parameters change: the next step builds)."""
        if not self.grad_ready:
            raise RuntimeError("optimizer_step needs the gradient of the current parameters: run the backward first")
        self._await_group(stream)
        B.poet_adamw_group([self.L.R, self.L.P], [self.thetaR, self.thetaP], [self.dthetaR, self.dthetaP],
                           [self.mR, self.mP], [self.vR, self.vP], hp, self.opt_steps + 1, stream)
        self._stepped()

    def _stepped(self):
        self.opt_steps += 1
        self.grad_ready = False
        self.built = False

    def merge(self, shadow=None, stream=None):
        """Merge-then-reinitialize; refreshes the bf16 copy of W0 of the activation-side path (and `shadow`,
        when given, receives the merged W0 in the act dtype as well). The merge folds the primitives of the last
        build, built again first at the merge's precision where that differs (POET_BUILD_MERGE); afterwards theta is
        zero and the next step must build again."""
        self._need_build("merge")
        self._await_group(stream)
        for side, th, pr, x in ((self.L.R, self.thetaR, self.primR, "R"), (self.L.P, self.thetaP, self.primP, "P")):
            if _merge_grade_differs(side):
                B.poet_build_orthogonal(side, th, pr, self._powers(x), None, self.ws, stream, for_merge=True)
        B.poet_merge(self.L, self.W0, self.W0b if shadow is None else shadow, self.thetaR, self.thetaP, self.primR,
                     self.primP, self.idxR, self.idxP, self.seed, self.linear_id, self.epoch + 1, self.ws, stream)
        B.poet_optimizer_reset_group([self.L.R, self.L.P], [self.mR, self.mP], [self.vR, self.vP], stream)
        self._merged()
        if shadow is not None and self.W0b is not None:
            B.poet_weight_shadow(self.L, self.W0, self.W0b, stream)

    def _merged(self):
        """State after a merge was enqueued: the next epoch, and the primitives, operand copies and folded weights
        of the last build are stale (they belong to the parameters before the reset)."""
        self.epoch += 1
        self.built = False
        self.grad_ready = False
        self.opt_steps = 0
        self.opsR = self.opsP = None
        self.W0P = self.RW0 = None
        self.formed = self._form_event = self._build_event = None  # the merge's stream has joined that work


class PermutedPoetLinear:
    """Permuted POET-BS on the GPU: R = Pi_R^T B_R Pi_R and P = Pi_P^T B_P Pi_P, with B_R, B_P block-diagonal (the
    POET-BS primitives) and Pi_R, Pi_P random permutations of the output and input dimensions, drawn by
    ``poet_sample_permutation`` and fresh at every merge (a reading of the sampled sub-block primitives, Approach
    section of the method summary).

    Realized as a plain POET-BS ``PoetLinear`` (``inner``) on the relabeled weight W0' = Pi_R W0 Pi_P^T: W = R W0 P
    = Pi_R^T (B_R W0' B_P) Pi_P, so with X' = X Pi_P^T (the columns of X gathered by perm_P) the inner layer gives
    Y' = X' (B_R W0' B_P)^T and Y = Y' Pi_R (the columns of Y' gathered by inv_R); the backward gathers dY by perm_R
    and returns dX' gathered by inv_P; the inner layer's dtheta are the permuted layer's. A merge merges W0' on the
    inner layer and relabels it for the next epoch's permutations (rows by inv_R_old[perm_R_new], columns alike).
    Every step runs in the library's kernels (``poet_gather2d`` moves the data); this class holds buffers only.
    The same calls as ``PoetLinear`` (build, forward/backward, forward_act/backward_act, optimizer_step, merge);
    each backward takes the gathered X' of the forward just before it (its X argument must be that forward's).
    """

    def __init__(self, m: int, n: int, T: int, R: B.poet_side, P: B.poet_side, act_dtype: int, W0,
                 thetaR=None, thetaP=None, seed: int = 0, linear_id: int = 0, ldw: Optional[int] = None,
                 ldx: Optional[int] = None, ldy: Optional[int] = None, device: str = "cuda", path: str = "weight"):
        if R.mode != B.POET_BS or P.mode != B.POET_BS:
            raise ValueError("permuted POET-BS needs POET-BS sides")
        torch = _torch()
        dev = torch.device(device)
        self.m, self.n, self.T = m, n, T
        self.seed, self.linear_id, self.epoch = seed, linear_id, 0
        i32 = dict(dtype=torch.int32, device=dev)
        self.permR, self.invR = torch.empty(m, **i32), torch.empty(m, **i32)
        self.permP, self.invP = torch.empty(n, **i32), torch.empty(n, **i32)
        self._sample(self.epoch)
        W0d = torch.as_tensor(W0, dtype=torch.float32).to(dev).contiguous()
        W0p = torch.empty_like(W0d)
        B.poet_gather2d(W0d, W0p, self.permR, self.permP)
        self.inner = PoetLinear(m, n, T, R, P, act_dtype, W0p, thetaR, thetaP, seed=seed, linear_id=linear_id,
                                ldw=ldw, ldx=ldx, ldy=ldy, device=device, path=path)
        del W0d, W0p
        inner = self.inner
        self.L, self.act, self.act_path, self.dev = inner.L, inner.act, inner.act_path, dev
        self.Xp, self.Yp = inner.alloc_act(T, inner.L.ldx), inner.alloc_act(T, inner.L.ldy)
        self.dYp, self.dXp = inner.alloc_act(T, inner.L.ldy), inner.alloc_act(T, inner.L.ldx)
        self._W0alt = torch.zeros_like(inner.W0)  # the other buffer of the relabeling at a merge
        self._xp_ready = False

    def _sample(self, epoch: int, stream=None):
        B.poet_sample_permutation(self.m, self.seed, self.linear_id, B.POET_SIDE_R, epoch, self.permR, self.invR,
                                  stream)
        B.poet_sample_permutation(self.n, self.seed, self.linear_id, B.POET_SIDE_P, epoch, self.permP, self.invP,
                                  stream)

    # the layer's parameters and gradients are the inner layer's
    def __getattr__(self, name):
        if name in ("thetaR", "thetaP", "dthetaR", "dthetaP", "primR", "primP", "mR", "vR", "mP", "vP",
                    "opt_steps", "grad_ready", "built", "W0b"):
            return getattr(self.inner, name)
        raise AttributeError(name)

    def alloc_act(self, rows: int, ld: int):
        return self.inner.alloc_act(rows, ld)

    def alloc_W(self):
        return self.inner.alloc_W()

    def build(self, stream=None):
        self.inner.build(stream)

    def _in(self, X, stream):
        B.poet_gather2d(X, self.Xp, col_idx=self.permP, stream=stream)
        self._xp_ready = True

    def _take_xp(self):
        if not self._xp_ready:
            raise RuntimeError("the backward of a permuted layer needs the forward just before it (its gathered X')")
        self._xp_ready = False

    def forward(self, X, Y, W_out=None, stream=None):
        """Weight side. W_out (optional) receives the inner layer's W' = B_R W0' B_P (relabeled coordinates)."""
        self._in(X, stream)
        self.inner.forward(self.Xp, self.Yp, W_out, stream)
        B.poet_gather2d(self.Yp, Y, col_idx=self.invR, stream=stream)

    def backward(self, X, dY, dX, W=None, stream=None):
        self._take_xp()
        B.poet_gather2d(dY, self.dYp, col_idx=self.permR, stream=stream)
        self.inner.backward(self.Xp, self.dYp, self.dXp, W, stream)
        B.poet_gather2d(self.dXp, dX, col_idx=self.invP, stream=stream)

    def forward_act(self, X, Y, Z, stream=None):
        """Activation side; Z (kept for backward_act) is the inner layer's, in relabeled coordinates."""
        self._in(X, stream)
        self.inner.forward_act(self.Xp, self.Yp, Z, stream)
        B.poet_gather2d(self.Yp, Y, col_idx=self.invR, stream=stream)

    def backward_act(self, X, Z, dY, dX, stream=None):
        self._take_xp()
        B.poet_gather2d(dY, self.dYp, col_idx=self.permR, stream=stream)
        self.inner.backward_act(self.Xp, Z, self.dYp, self.dXp, stream)
        B.poet_gather2d(self.dXp, dX, col_idx=self.invP, stream=stream)

    def optimizer_step(self, hp: B.poet_adamw, stream=None):
        self.inner.optimizer_step(hp, stream)

    def merge(self, stream=None):
        """Merge-then-reinitialize: the inner merge folds B_R, B_P into W0' and resets theta and the moments;
        then the next epoch's permutations are drawn and W0' is relabeled to them (and its bf16 copy refreshed)."""
        self.inner.merge(stream=stream)
        self.relabel(stream)

    def relabel(self, stream=None):
        """Draw the next epoch's permutations and relabel W0' to them (after a merge of the inner layer, e.g. by
        PoetGroup.merge over inner layers)."""
        torch = _torch()
        oldR, oldP = self.invR.clone(), self.invP.clone()
        self.epoch += 1
        self._sample(self.epoch, stream)
        sigR = torch.empty(1, self.m, dtype=torch.int32, device=self.dev)
        sigP = torch.empty(1, self.n, dtype=torch.int32, device=self.dev)
        B.poet_gather2d(oldR.view(1, -1), sigR, col_idx=self.permR, stream=stream)  # inv_R_old[perm_R_new[i]]
        B.poet_gather2d(oldP.view(1, -1), sigP, col_idx=self.permP, stream=stream)
        inner = self.inner
        B.poet_gather2d(inner.W0[:, :self.n], self._W0alt, sigR.view(-1), sigP.view(-1), stream=stream)
        inner.W0, self._W0alt = self._W0alt, inner.W0
        if inner.W0b is not None:
            B.poet_weight_shadow(inner.L, inner.W0, inner.W0b, stream)

    def original_weight(self, stream=None):
        """W0 in the original coordinates (float32 m x n): W0[x][y] = W0'[inv_R[x]][inv_P[y]]."""
        torch = _torch()
        out = torch.empty((self.m, self.n), dtype=torch.float32, device=self.dev)
        B.poet_gather2d(self.inner.W0[:, :self.n], out, self.invR, self.invP, stream=stream)
        return out


class PoetGroup:
    """The per-block steps of several POET linears (e.g. the seven of a transformer block) in shared launches.

    ``build`` runs the Cayley-Neumann build of both sides of every linear (poet_build_orthogonal_group);
    ``finish_backward`` runs the Neumann adjoint and skew projection of every side from the primitive gradients
    that ``PoetLinear.backward_act_prims`` / ``backward_prims`` left (poet_adjoint_group); ``merge`` runs
    merge-then-reinitialize of every linear (poet_merge_group). Results match the per-linear calls up to the
    float32 summation order of split products."""

    def __init__(self, linears, ws=None, form_fs: bool = False, form_streams: int = 1, form_ws=None,
                 side_chains: bool = True, side=None, side_linears=None):
        """``ws`` (optional): a uint8 device tensor shared with other groups whose calls run one after another on one
        stream (``PoetGroup.workspace_bytes`` gives the size this group needs).

        ``form_fs``: the build also forms, for every weight-side linear with two bf16 POET-FS sides, W = R W0 P and
        the FS gradient operands (poet_fs_form), which the linear's forward and backward_prims then read instead of
        forming them there. The formations of different linears are independent: they run on up to
        ``form_streams`` side streams (default priority) that fork from the build's stream and join it again, so
        that their small kernels overlap; each stream has a workspace of its own (``form_ws``, optional: a list of
        uint8 device tensors, e.g. shared with other groups whose builds run one after another, each of at least
        ``PoetGroup.form_workspace_bytes`` bytes).

        ``side_chains``: where the sides fall in more than one class of ``_chain_class`` (e.g. the s = d/2 POET-FS
        primitives of a transformer block: s = 1024 on the attention linears, 2730 on the MLP's wide side), the class
        with the most product work builds, and later runs its adjoint, on a side stream (default priority) beside
        the rest: each class alone leaves CUs idle (its products have a few hundred tiles or fewer), and the
        linears whose sides are all in the other classes can start their forward before that class is built. Each
        linear waits for its sides' build at its next use. ``side`` (optional): a (stream, uint8 device tensor) pair
        shared with other groups whose calls run one after another, the tensor of at least
        ``PoetGroup.side_workspace_bytes`` bytes. The results are those of one grouped call per step, bit for bit.

        ``side_linears`` (optional, with ``side_chains``): indices into ``linears`` whose sides form the side class
        instead, e.g. the MLP linears of a POET-BS block, whose sides are all one size (their folds then run on the
        side stream too). Best taken from the end of the step order: their gradients come last."""
        torch = _torch()
        self.linears = list(linears)
        if not self.linears:
            raise ValueError("PoetGroup needs at least one linear")
        self.sides = [s for pl in self.linears for s in (pl.L.R, pl.L.P)]
        dev = self.linears[0].dev
        # operand copies for the activation-side calls of BS sides (3 * prim_len bf16 per side)
        self._ops = {}
        for pl in self.linears:
            if pl.act_path:
                self._ops[id(pl)] = tuple(torch.empty(3 * B.poet_prim_len(s), dtype=torch.bfloat16, device=dev)
                                          for s in (pl.L.R, pl.L.P))
        # factors folded into the bf16 weights of activation-side linears with at least as many tokens as the
        # weight has rows (P) or columns (R), blocks of 128 or more (smaller blocks would run on the generic kernel)
        self._fold = {}
        for pl in self.linears:
            if pl.act_path:
                fP = pl.T >= pl.m and pl.L.P.b >= 128
                fR = pl.T >= pl.n and pl.L.R.b >= 128
                self._fold[id(pl)] = (torch.empty((pl.m, pl.L.ldw), dtype=pl.act, device=dev) if fP else None,
                                      torch.empty((pl.m, pl.L.ldw), dtype=pl.act, device=dev) if fR else None)
        # W, Zr, Acp of the FS pairs formed by the build
        self._formed = {}
        if form_fs:
            for pl in self.linears:
                if PoetGroup._formable(pl):
                    sh = B.fs_operand_shapes(pl.L)
                    self._formed[id(pl)] = (pl.alloc_W(), torch.empty(sh["Zr"], dtype=torch.bfloat16, device=dev),
                                            torch.empty(sh["Acp"], dtype=torch.bfloat16, device=dev))
        self._form_streams, self._form_ws = [], []
        if self._formed:
            ns = max(1, min(form_streams, len(self._formed)))
            fneed = PoetGroup.form_workspace_bytes(self.linears)
            if form_ws is None:
                form_ws = [torch.empty(max(fneed, 1), dtype=torch.uint8, device=dev) for _ in range(ns)]
            ns = min(ns, len(form_ws))
            if ns == 0 or any(w.numel() * w.element_size() < fneed for w in form_ws[:ns]):
                raise ValueError(f"the formations of this group need workspaces of {fneed} bytes")
            self._form_ws = list(form_ws[:ns])
            self._form_streams = [torch.cuda.Stream(device=dev) for _ in range(ns)]
            self._form_events = {k: torch.cuda.Event() for k in self._formed}
            # the caching allocator reuses these buffers only after the formation streams' work that precedes
            # their release
            for s in self._form_streams:
                for bufs in self._formed.values():
                    for t in bufs:
                        t.record_stream(s)
                for w in self._form_ws:
                    w.record_stream(s)
        # the side class: its sides' indices in self.sides (side 2i is linear i's R, 2i + 1 its P)
        self._side_lin = None
        if side_linears is not None:
            sl = sorted(set(int(i) for i in side_linears))
            if not sl or sl[0] < 0 or sl[-1] >= len(self.linears) or len(sl) == len(self.linears):
                raise ValueError("side_linears must name some, not all, of the group's linears")
            self._side_lin = sl
        self._side_idx = PoetGroup._side_class(self.sides, self._side_lin) if side_chains else []
        off = set(self._side_idx)
        self._main_idx = [i for i in range(len(self.sides)) if i not in off]
        self._side_stream = self._side_ws = self._side_event = None
        self._side_open = False  # a finish_backward(join=False) left the side class's gradient on the side stream
        if self._side_idx:
            sneed = PoetGroup.side_workspace_bytes(self.linears, self._side_lin)
            if side is None:
                side = (torch.cuda.Stream(device=dev), torch.empty(max(sneed, 1), dtype=torch.uint8, device=dev))
            self._side_stream, self._side_ws = side
            if self._side_ws.numel() * self._side_ws.element_size() < sneed:
                raise ValueError(f"the side stream's calls of this group need a workspace of {sneed} bytes")
            self._side_ws.record_stream(self._side_stream)
            self._side_event = torch.cuda.Event()
        need = PoetGroup.workspace_bytes(self.linears, side_chains, self._side_lin)
        if ws is None:
            self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        else:
            if ws.numel() * ws.element_size() < need:
                raise ValueError(f"shared workspace holds {ws.numel() * ws.element_size()} bytes, this group needs {need}")
            self.ws = ws

    @staticmethod
    def _formable(pl) -> bool:
        L = pl.L
        return (not pl.act_path and L.R.mode == B.POET_FS and L.P.mode == B.POET_FS and L.act_dtype == B.POET_BF16
                and L.R.dtype == B.POET_BF16 and L.P.dtype == B.POET_BF16)

    @staticmethod
    def form_workspace_bytes(linears) -> int:
        """Bytes of the workspace one formation stream needs for these linears (the largest poet_fs_form)."""
        return max([B.poet_fs_form_workspace_bytes(pl.L) for pl in linears if PoetGroup._formable(pl)] or [0])

    @staticmethod
    def _chain_class(side):
        """The class of a side whose Cayley-Neumann chain and Neumann adjoint run as products of whole bf16
        primitives above 256 (POET-FS primitives, large POET-BS blocks): (mode, b, k); None for the other sides."""
        if side.dtype == B.POET_BF16 and side.k > 0 and side.b > 256:
            return (side.mode, side.b, side.k)
        return None

    @staticmethod
    def _side_class(sides, side_linears=None):
        """Indices of the sides that build and run their adjoint on the side stream: both sides of the linears in
        side_linears when given; else the class of _chain_class with the most product work (primitives x b^3 x k),
        when some side falls outside it; else none."""
        if side_linears is not None:
            return [2 * i + r for i in side_linears for r in (0, 1)]
        classes = {}
        for i, s in enumerate(sides):
            classes.setdefault(PoetGroup._chain_class(s), []).append(i)
        work = [(sum(B.poet_num_prims(sides[i]) for i in v) * c[1] ** 3 * c[2], c) for c, v in classes.items()
                if c is not None]
        if len(classes) < 2 or not work:
            return []
        return classes[max(work)[1]]

    @staticmethod
    def side_workspace_bytes(linears, side_linears=None) -> int:
        """Bytes of the workspace of the side stream's calls (build, folds and adjoint of the side class); 0 without
        one."""
        sides = [s for pl in linears for s in (pl.L.R, pl.L.P)]
        idx = PoetGroup._side_class(sides, side_linears)
        if not idx:
            return 0
        sub = [sides[i] for i in idx]
        act = [linears[j].L for j in sorted({i // 2 for i in idx}) if linears[j].act_path]
        return max(B.poet_build_group_workspace_bytes(sub), B.poet_adjoint_group_workspace_bytes(sub),
                   B.poet_fold_group_workspace_bytes(act) if act else 0)

    def _of(self, i, r, p):
        """Attribute r (side i is an R side) or p of the linear that side i belongs to."""
        return getattr(self.linears[i // 2], r if i % 2 == 0 else p)

    def _record_side(self, tensors):
        """The caching allocator reuses these tensors' memory only after the side stream's work enqueued so far
        (nothing to do under graph capture, whose memory outlives the graph)."""
        torch = _torch()
        if torch.cuda.is_current_stream_capturing():
            return
        for t in tensors:
            if t is not None:
                t.record_stream(self._side_stream)

    def _build_sides(self, idx, ws, stream, for_merge=False):
        pls = self.linears
        if not idx:
            return
        B.poet_build_orthogonal_group([self.sides[i] for i in idx], [self._of(i, "thetaR", "thetaP") for i in idx],
                                      [self._of(i, "primR", "primP") for i in idx],
                                      [pls[i // 2]._powers("RP"[i % 2]) for i in idx], ws, stream,
                                      ops=None if for_merge else [self._ops.get(id(pls[i // 2]), (None, None))[i % 2]
                                                                  for i in idx], for_merge=for_merge)

    def _build_all(self, stream):
        """The grouped build of every side: one call, or the side class on the side stream (forked from the launch
        stream) beside one call for the rest; each linear with a side in that class waits for it at its next use."""
        if not self._side_idx:
            self._build_sides(range(len(self.sides)), self.ws, stream)
            return
        main = _torch_stream(stream, self.linears[0].dev)
        self._side_stream.wait_stream(main)
        self._build_sides(self._side_idx, self._side_ws, self._side_stream)
        self._side_event.record(self._side_stream)
        self._record_side([self._of(i, a, b) for i in self._side_idx for a, b in (("thetaR", "thetaP"),
                                                                                    ("primR", "primP"))] +
                          [self.linears[i // 2]._powers("RP"[i % 2]) for i in self._side_idx])
        self._build_sides(self._main_idx, self.ws, stream)
        for i in self._side_idx:
            self.linears[i // 2]._build_event = self._side_event

    def join(self, stream=None):
        """The launch stream waits for all work this group left on its other streams (formations, the side class's
        build, an open finish_backward and the update after it)."""
        self._join_forms(stream)
        self._join_side(stream)

    def _join_side(self, stream):
        if self._side_stream is not None:
            _torch_stream(stream, self.linears[0].dev).wait_stream(self._side_stream)
            for pl in self.linears:
                pl._build_event = None
        self._side_open = False

    @staticmethod
    def workspace_bytes(linears, side_chains: bool = True, side_linears=None) -> int:
        """Bytes of the workspace the grouped calls of these linears need on the launch stream (with
        ``side_chains``, the side class builds and runs its adjoint in a workspace of its own)."""
        sides = [s for pl in linears for s in (pl.L.R, pl.L.P)]
        if side_chains:
            off = set(PoetGroup._side_class(sides, side_linears))
            sides = [s for i, s in enumerate(sides) if i not in off]
        act = [pl for pl in linears if pl.act_path]
        return max(B.poet_build_group_workspace_bytes(sides), B.poet_adjoint_group_workspace_bytes(sides),
                   B.poet_merge_group_workspace_bytes([pl.L for pl in linears]),
                   B.poet_fold_group_workspace_bytes([pl.L for pl in act]) if act else 0)

    def build(self, stream=None, again: bool = False):
        """The grouped Cayley-Neumann build of every side (and the operand copies), then the folds and the formed FS
        operands. ``again``: the parameters have not changed since the last build (every linear is still built), and
        the build runs only to form the saved Neumann powers once more (a stack that shares one set of power buffers
        among its layers rebuilds each layer before its backward): the primitives come out the same, so the folds
        and formed operands of that build stay as they are."""
        if again:
            if not all(pl.built for pl in self.linears):
                raise RuntimeError("build(again=True) needs every linear built since its parameters last changed")
            for pl in self.linears:
                pl._await_form(stream)
            self._build_all(stream)
            return
        # formations (of this group or another) still reading the primitives; work this group left on its side
        # stream (an open finish_backward, the optimizer step after it) precedes the side class's build there
        for pl in self.linears:
            pl._await_form(stream)
        self._build_all(stream)
        for pl in self.linears:
            pl.opsR, pl.opsP = self._ops.get(id(pl), (None, None))
            pl.W0P = pl.RW0 = None
            pl.formed = pl._form_event = None
            pl.built = True
        if self._formed:
            self._form(stream)
        act = [pl for pl in self.linears if pl.act_path and any(f is not None for f in self._fold[id(pl)])]
        # the folds read the primitives: those of linears with a side in the side class run on the side stream,
        # after its build and the launch stream's (for the linear's other side)
        on_side = {i // 2 for i in self._side_idx}
        side_act = [pl for j, pl in enumerate(self.linears) if j in on_side and pl in act]
        main_act = [pl for pl in act if not any(pl is q for q in side_act)]
        for pls, st, ws, on in ((main_act, stream, self.ws, False), (side_act, self._side_stream, self._side_ws, True)):
            if not pls:
                continue
            if on:
                st.wait_stream(_torch_stream(stream, self.linears[0].dev))
            B.poet_fold_weights_group([pl.L for pl in pls], [pl.W0b for pl in pls], [pl.primR for pl in pls],
                                      [pl.primP for pl in pls], [self._fold[id(pl)][0] for pl in pls],
                                      [self._fold[id(pl)][1] for pl in pls], ws, st,
                                      opsRs=[pl.opsR for pl in pls], opsPs=[pl.opsP for pl in pls])
            for pl in pls:
                pl.W0P, pl.RW0 = self._fold[id(pl)]
        if side_act:
            self._record_side([t for pl in side_act for t in self._fold[id(pl)] + (pl.W0b, pl.opsR, pl.opsP)])
            self._mark_side()

    def _form(self, stream):
        """Fork the formation streams from the build's stream and form every FS pair, round robin. The launch stream
        waits for a linear's formation in that linear's forward (or backward), so that formations of later linears
        overlap the token products of earlier ones; finish_backward and merge join the formation streams."""
        main = _torch_stream(stream, self.linears[0].dev)
        pls = [pl for pl in self.linears if id(pl) in self._formed]
        for s in self._form_streams:
            s.wait_stream(main)
        for i, pl in enumerate(pls):
            j = i % len(self._form_streams)
            if pl._build_event is not None:  # a side built on the side stream (the formation's event covers it)
                self._form_streams[j].wait_event(pl._build_event)
                pl._build_event = None
            W, Zr, Acp = self._formed[id(pl)]
            B.poet_fs_form(pl.L, pl.W0, pl.primR, pl.primP, pl.idxR, pl.idxP, W, Zr, Acp, self._form_ws[j],
                           self._form_streams[j])
            self._form_events[id(pl)].record(self._form_streams[j])
            pl.formed, pl._form_event = (W, Zr, Acp), self._form_events[id(pl)]

    def _join_forms(self, stream):
        if self._form_streams:
            main = _torch_stream(stream, self.linears[0].dev)
            for s in self._form_streams:
                main.wait_stream(s)

    def finish_backward(self, stream=None, join: bool = True):
        """The Neumann adjoint and skew projection of every side (dthetaR, dthetaP from dprimR, dprimP).

        ``join=False`` (groups with a side class): the side class's adjoint is left running on the side stream, and
        ``optimizer_step`` updates that class there too, so both overlap the launch stream's next work (the next
        layer's backward, the next step's build of the other classes and the linears that need only those). Each
        linear with a side in that class waits for it at its next use (its next group build orders the side
        class's build after it on the side stream); ``merge`` joins it. Until then the side class's dtheta, theta
        and moments are not ready on the launch stream: synchronize (or join) before reading them, keep the call
        out of graph capture, and let groups that share parameter or power buffers share one side stream."""
        for pl in self.linears:
            if getattr(pl, "dprimR", None) is None:
                raise RuntimeError("finish_backward needs backward_prims or backward_act_prims on every linear first")
        self._join_forms(stream)

        def adjoint(idx, ws, st):
            B.poet_adjoint_group([self.sides[i] for i in idx], [self._of(i, "dprimR", "dprimP") for i in idx],
                                 [self.linears[i // 2]._powers("RP"[i % 2]) for i in idx],
                                 [self._of(i, "dthetaR", "dthetaP") for i in idx], ws, st)
        if self._side_idx:  # the side class on the side stream, forked after the last backward, then joined
            self._side_stream.wait_stream(_torch_stream(stream, self.linears[0].dev))
            adjoint(self._side_idx, self._side_ws, self._side_stream)
            self._record_side([self._of(i, a, b) for i in self._side_idx for a, b in (("dprimR", "dprimP"),
                                                                                        ("dthetaR", "dthetaP"))] +
                              [self.linears[i // 2]._powers("RP"[i % 2]) for i in self._side_idx])
            adjoint(self._main_idx, self.ws, stream)
            if join:
                self._join_side(stream)
            else:
                self._side_open = True
                self._mark_side()
        else:
            adjoint(range(len(self.sides)), self.ws, stream)
        for pl in self.linears:
            pl.grad_ready = True

    def _mark_side(self):
        """Each linear with a side in the side class waits, at its next use, for the side stream's work so far."""
        self._side_event.record(self._side_stream)
        for i in self._side_idx:
            self.linears[i // 2]._build_event = self._side_event

    def optimizer_step(self, hp: B.poet_adamw, stream=None):
        """One AdamW step on the skew parameters of every linear in shared launches (their step counts must agree)."""
        pls = self.linears
        if len({pl.opt_steps for pl in pls}) != 1:
            raise ValueError("PoetGroup.optimizer_step needs one step count across its linears")
        for pl in pls:
            if not pl.grad_ready:
                raise RuntimeError("optimizer_step needs the gradient of the current parameters: run the backward first")
        def adamw(idx, st):
            B.poet_adamw_group([self.sides[i] for i in idx], [self._of(i, "thetaR", "thetaP") for i in idx],
                               [self._of(i, "dthetaR", "dthetaP") for i in idx], [self._of(i, "mR", "mP") for i in idx],
                               [self._of(i, "vR", "vP") for i in idx], hp, pls[0].opt_steps + 1, st)
        if self._side_open:  # the side class's gradient is still on the side stream: update it there
            adamw(self._side_idx, self._side_stream)
            self._record_side([self._of(i, a, b) for i in self._side_idx
                               for a, b in (("thetaR", "thetaP"), ("mR", "mP"), ("vR", "vP"))])
            self._mark_side()
            adamw(self._main_idx, stream)
        else:
            adamw(range(len(self.sides)), stream)
        for pl in pls:
            pl._stepped()

    def merge(self, stream=None):
        """Merge-then-reinitialize of every linear (their sampler seeds and epochs must agree); refreshes each
        linear's bf16 copy of W0 where it keeps one."""
        pls = self.linears
        if len({pl.seed for pl in pls}) != 1 or len({pl.epoch for pl in pls}) != 1:
            raise ValueError("PoetGroup.merge needs one sampler seed and one epoch across its linears")
        for pl in pls:
            pl._need_build("PoetGroup.merge")
        self._join_forms(stream)
        self._join_side(stream)
        # the sides whose build differs at the merge's precision are built again at it first (the side class on the
        # side stream, joined before the merge)
        redo = [i for i in range(len(self.sides)) if _merge_grade_differs(self.sides[i])]
        side = set(self._side_idx)
        if any(i in side for i in redo):
            self._side_stream.wait_stream(_torch_stream(stream, self.linears[0].dev))
            self._build_sides([i for i in redo if i in side], self._side_ws, self._side_stream, for_merge=True)
        self._build_sides([i for i in redo if i not in side], self.ws, stream, for_merge=True)
        self._join_side(stream)
        B.poet_merge_group([pl.L for pl in pls], [pl.W0 for pl in pls], [pl.W0b for pl in pls],
                           [pl.thetaR for pl in pls], [pl.thetaP for pl in pls], [pl.primR for pl in pls],
                           [pl.primP for pl in pls], [pl.idxR for pl in pls], [pl.idxP for pl in pls], pls[0].seed,
                           [pl.linear_id for pl in pls], pls[0].epoch + 1, self.ws, stream)
        B.poet_optimizer_reset_group(self.sides, [t for pl in pls for t in (pl.mR, pl.mP)],
                                     [t for pl in pls for t in (pl.vR, pl.vP)], stream)
        for pl in pls:
            pl._merged()
