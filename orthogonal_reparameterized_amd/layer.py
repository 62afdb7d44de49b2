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
        self.opsR = self.opsP = None  # the one-side build does not write them
        self.W0P = self.RW0 = None
        B.poet_build_orthogonal(self.L.R, self.thetaR, self.primR, self._powers("R"), self.qnormR if qnorm else None,
                                self.ws, stream)
        B.poet_build_orthogonal(self.L.P, self.thetaP, self.primP, self._powers("P"), self.qnormP if qnorm else None,
                                self.ws, stream)

    def alloc_act(self, rows: int, ld: int):
        return _torch().empty((rows, ld), dtype=self.act, device=self.dev)

    def alloc_W(self):
        return _torch().empty((self.m, self.L.ldw), dtype=self.act, device=self.dev)

    def forward(self, X, Y, W_out=None, stream=None):
        B.poet_linear_fwd(self.L, self.W0, self.primR, self.primP, self.idxR, self.idxP, X, Y, W_out, self.ws, stream)

    def backward(self, X, dY, dX, W=None, stream=None):
        B.poet_linear_bwd(self.L, self.W0, self.primR, self.primP, self._powers("R"), self._powers("P"), self.idxR,
                          self.idxP, W, X, dY, dX, self.dthetaR, self.dthetaP, self.ws, stream)

    def forward_act(self, X, Y, Z, stream=None):
        """Activation-side forward: Y = ((X P^T) W0^T) R^T; Z = X P^T W0^T is kept for backward_act. The bf16
        operand copies of the primitives (and W0 P, folded) come from the last PoetGroup.build, when one made them."""
        if self.W0P is not None:
            B.poet_linear_fwd_folded(self.L, self.W0P, self.primR, X, Y, Z, self.ws, stream, opsR=self.opsR)
        else:
            B.poet_linear_fwd_act(self.L, self.W0b, self.primR, self.primP, X, Y, Z, self.ws, stream,
                                  opsR=self.opsR, opsP=self.opsP)

    def backward_act(self, X, Z, dY, dX, stream=None):
        B.poet_linear_bwd_act(self.L, self.W0b, self.primR, self.primP, self._powers("R"), self._powers("P"), X, Z,
                              dY, dX, self.dthetaR, self.dthetaP, self.ws, stream, opsR=self.opsR, opsP=self.opsP)

    def _dprims(self):
        if getattr(self, "dprimR", None) is None:
            torch = _torch()
            self.dprimR = torch.empty(B.poet_prim_len(self.L.R), dtype=torch.float32, device=self.dev)
            self.dprimP = torch.empty(B.poet_prim_len(self.L.P), dtype=torch.float32, device=self.dev)

    def backward_prims(self, X, dY, dX, W=None, stream=None):
        """Weight-side backward up to the primitive gradients dprimR, dprimP; PoetGroup.finish_backward turns them
        into dthetaR, dthetaP for many linears at once."""
        self._dprims()
        B.poet_linear_bwd_prims(self.L, self.W0, self.primR, self.primP, self.idxR, self.idxP, W, X, dY, dX,
                                self.dprimR, self.dprimP, self.ws, stream)

    def backward_act_prims(self, X, Z, dY, dX, stream=None):
        """Activation-side backward up to the primitive gradients dprimR, dprimP (the blocks of dL/dR and dL/dP);
        PoetGroup.finish_backward turns them into dthetaR, dthetaP for many linears at once."""
        self._dprims()
        if self.RW0 is not None:
            B.poet_linear_bwd_folded_prims(self.L, self.RW0, self.primP, X, Z, dY, dX, self.dprimR, self.dprimP,
                                           self.ws, stream, opsP=self.opsP)
        else:
            B.poet_linear_bwd_act_prims(self.L, self.W0b, self.primR, self.primP, X, Z, dY, dX, self.dprimR,
                                        self.dprimP, self.ws, stream, opsR=self.opsR, opsP=self.opsP)

    def merge(self, shadow=None, stream=None):
        """Merge-then-reinitialize; refreshes the bf16 copy of W0 of the activation-side path (and `shadow`,
        when given, receives the merged W0 in the act dtype as well)."""
        self.epoch += 1
        B.poet_merge(self.L, self.W0, self.W0b if shadow is None else shadow, self.thetaR, self.thetaP, self.primR,
                     self.primP, self.idxR, self.idxP, self.seed, self.linear_id, self.epoch, self.ws, stream)
        if shadow is not None and self.W0b is not None:
            B.poet_weight_shadow(self.L, self.W0, self.W0b, stream)


class PoetGroup:
    """The per-block steps of several POET linears (e.g. the seven of a transformer block) in shared launches.

    ``build`` runs the Cayley-Neumann build of both sides of every linear (poet_build_orthogonal_group);
    ``finish_backward`` runs the Neumann adjoint and skew projection of every side from the primitive gradients
    that ``PoetLinear.backward_act_prims`` / ``backward_prims`` left (poet_adjoint_group); ``merge`` runs
    merge-then-reinitialize of every linear (poet_merge_group). Results match the per-linear calls up to the
    float32 summation order of split products."""

    def __init__(self, linears):
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
        act = [pl for pl in self.linears if pl.act_path]
        need = max(B.poet_build_group_workspace_bytes(self.sides), B.poet_adjoint_group_workspace_bytes(self.sides),
                   B.poet_merge_group_workspace_bytes([pl.L for pl in self.linears]),
                   B.poet_fold_group_workspace_bytes([pl.L for pl in act]) if act else 0)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def build(self, stream=None):
        thetas = [t for pl in self.linears for t in (pl.thetaR, pl.thetaP)]
        prims = [t for pl in self.linears for t in (pl.primR, pl.primP)]
        powers = [pl._powers(x) for pl in self.linears for x in ("R", "P")]
        ops = [o for pl in self.linears for o in self._ops.get(id(pl), (None, None))]
        B.poet_build_orthogonal_group(self.sides, thetas, prims, powers, self.ws, stream, ops=ops)
        for pl in self.linears:
            pl.opsR, pl.opsP = self._ops.get(id(pl), (None, None))
            pl.W0P = pl.RW0 = None
        act = [pl for pl in self.linears if pl.act_path and any(f is not None for f in self._fold[id(pl)])]
        if act:
            B.poet_fold_weights_group([pl.L for pl in act], [pl.W0b for pl in act], [pl.primR for pl in act],
                                      [pl.primP for pl in act], [self._fold[id(pl)][0] for pl in act],
                                      [self._fold[id(pl)][1] for pl in act], self.ws, stream,
                                      opsRs=[pl.opsR for pl in act], opsPs=[pl.opsP for pl in act])
            for pl in act:
                pl.W0P, pl.RW0 = self._fold[id(pl)]

    def finish_backward(self, stream=None):
        for pl in self.linears:
            if getattr(pl, "dprimR", None) is None:
                raise RuntimeError("finish_backward needs backward_prims or backward_act_prims on every linear first")
        dprims = [t for pl in self.linears for t in (pl.dprimR, pl.dprimP)]
        powers = [pl._powers(x) for pl in self.linears for x in ("R", "P")]
        dthetas = [t for pl in self.linears for t in (pl.dthetaR, pl.dthetaP)]
        B.poet_adjoint_group(self.sides, dprims, powers, dthetas, self.ws, stream)

    def merge(self, stream=None):
        """Merge-then-reinitialize of every linear (their sampler seeds and epochs must agree); refreshes each
        linear's bf16 copy of W0 where it keeps one."""
        pls = self.linears
        if len({pl.seed for pl in pls}) != 1 or len({pl.epoch for pl in pls}) != 1:
            raise ValueError("PoetGroup.merge needs one sampler seed and one epoch across its linears")
        for pl in pls:
            pl.epoch += 1
        B.poet_merge_group([pl.L for pl in pls], [pl.W0 for pl in pls], [pl.W0b for pl in pls],
                           [pl.thetaR for pl in pls], [pl.thetaP for pl in pls], [pl.primR for pl in pls],
                           [pl.primP for pl in pls], [pl.idxR for pl in pls], [pl.idxP for pl in pls], pls[0].seed,
                           [pl.linear_id for pl in pls], pls[0].epoch, self.ws, stream)
