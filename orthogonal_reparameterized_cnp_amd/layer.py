"""Device buffers of one POET-X linear, allocated with torch, driven through the C ABI.

The class only owns memory and sequences the library calls; all arithmetic is
done by libpoetx kernels.
"""

from __future__ import annotations

import contextlib
from typing import Optional

import torch

from . import binding as B

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}


def lead(d: int) -> int:
    return (d + 63) // 64 * 64


def _check(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype):
    """Reject a tensor the kernels would read or write out of bounds: wrong shape, dtype or
    layout.  Raises ValueError before any launch."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_device(device: torch.device, **tensors):
    """Every given tensor must live on `device`, which must be a GPU (the kernels take raw device
    pointers).  Raises ValueError before any launch."""
    for name, t in tensors.items():
        if t is None:
            continue
        ok = device.type == "cuda" and t.device.type == "cuda"
        if not ok or t.device.index != (device.index if device.index is not None else torch.cuda.current_device()):
            raise ValueError(f"{name} is on {t.device}; the layer's kernels run on {device}, which must be a GPU")


class PoetxLinear:
    def __init__(self, m: int, n: int, b: int, act: str = "bf16", w: str = "bf16", device: str = "cuda",
                 mode: str = "xfast"):
        """mode: "xfast" saves H for the backward; "xmem" saves only the gathered input and the
        backward recomputes H (bit-identical results, T x n fewer saved activations); "xout" saves
        only the gathered input and the backward takes H back from the output Y, which it must be
        given (H Diag((I - Q_P^4)^2) in place of H: dq_P differs, dX and dq_R do not)."""
        self.m, self.n, self.b, self.act, self.w, self.mode = m, n, b, act, w, mode
        self.device = torch.device(device)
        self.desc = B.desc(m, n, b, act, w, mode)
        self.nbR, self.nbP = -(-m // b), -(-n // b)
        L = b * (b - 1) // 2
        u8 = dict(dtype=torch.uint8, device=self.device)
        self.Wt = torch.zeros(B.poetx_weight_bytes(self.desc), **u8)
        adt = B.DTYPES[act]
        self.g_R = torch.empty(B.poetx_g_bytes(m, b, adt), **u8)
        self.g_P = torch.empty(B.poetx_g_bytes(n, b, adt), **u8)
        self.q_R = torch.zeros(self.nbR, L, dtype=torch.float32, device=self.device)
        self.q_P = torch.zeros(self.nbP, L, dtype=torch.float32, device=self.device)
        self.perm_R = torch.arange(m, dtype=torch.int32, device=self.device)
        self.perm_P = torch.arange(n, dtype=torch.int32, device=self.device)
        self.ws = torch.empty(0, **u8)
        self.H_save: Optional[torch.Tensor] = None
        self.T = None  # tokens of the last forward (the saved state's)

    # -- buffers ------------------------------------------------------------
    def _ws(self, nbytes: int) -> torch.Tensor:
        if self.ws.numel() < nbytes:
            self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.ws

    def ws_bytes(self, T: int) -> int:
        d = self.desc
        return max(
            B.poetx_workspace_size(d, T, B.POETX_OP_FWD),
            B.poetx_workspace_size(d, T, B.POETX_OP_BWD),
            B.poetx_workspace_size(d, 0, B.POETX_OP_MERGE),
            B.poetx_workspace_size(B.desc(max(self.m, self.n), 1, self.b, self.act, self.w), 0, B.POETX_OP_CNP),
        )

    def reserve(self, T: int):
        self._ws(self.ws_bytes(T))
        if self.H_save is None or self.H_save.numel() < B.poetx_saved_bytes(self.desc, T):
            self.H_save = torch.empty(B.poetx_saved_bytes(self.desc, T), dtype=torch.uint8, device=self.device)

    # -- state --------------------------------------------------------------
    def load(self, W0: torch.Tensor, w_scale: Optional[torch.Tensor], perm_R, perm_P, q_R, q_P, stream=None):
        """Natural-layout W0 [m][n] (+ int8 column scales) and factor state -> pre-merged layout."""
        self.perm_R.copy_(perm_R)
        self.perm_P.copy_(perm_P)
        self.q_R.copy_(q_R)
        self.q_P.copy_(q_P)
        B.poetx_premerge(self.desc, W0, W0.stride(0), w_scale, self.perm_R, self.perm_P, self.Wt, stream)

    def weight_values(self) -> torch.Tensor:
        """View of the pre-merged weight values [m][lead(n)] (padding columns included)."""
        ldw = lead(self.n)
        es = {"f32": 4, "bf16": 2, "i8": 1}[self.w]
        return self.Wt[: self.m * ldw * es].view(_TORCH_DT[self.w]).view(self.m, ldw)

    def weight_t(self) -> torch.Tensor:
        """View of the transposed copy [n][lead(m)] that bf16 weights keep after the values."""
        if self.w != "bf16":
            raise ValueError("only bf16 weights keep a transposed copy")
        off = (self.m * lead(self.n) * 2 + 255) // 256 * 256
        return self.Wt[off : off + self.n * lead(self.m) * 2].view(torch.bfloat16).view(self.n, lead(self.m))

    def weight_scales(self) -> torch.Tensor:
        ldw = lead(self.n)
        off = (self.m * ldw + 255) // 256 * 256
        return self.Wt[off : off + 4 * ldw].view(torch.float32)

    def g_slices(self, side: str):
        d, g = (self.m, self.g_R) if side == "R" else (self.n, self.g_P)
        nb = -(-d // self.b)
        dt = _TORCH_DT[self.act]
        return g.view(dt).view(2, nb, self.b, self.b)

    # -- calls --------------------------------------------------------------
    def build(self, stream=None):
        adt = B.DTYPES[self.act]
        for q, d, g in ((self.q_R, self.m, self.g_R), (self.q_P, self.n, self.g_P)):
            need = B.poetx_workspace_size(B.desc(d, 1, self.b, self.act, self.w), 0, B.POETX_OP_CNP)
            ws = self._ws(need)
            B.poetx_cnp_build(q, d, self.b, adt, g, ws, ws.numel(), stream)

    def _act_dt(self) -> torch.dtype:
        return _TORCH_DT[self.act]

    def _fwd_args(self, X: torch.Tensor, Y: Optional[torch.Tensor]):
        """Checked forward arguments: T, and Y (allocated if None); the workspace is sized for T."""
        if not isinstance(X, torch.Tensor) or X.dim() != 2:
            raise ValueError("X must be a 2-D tensor [T, m]")
        T = X.shape[0]
        _check(X, "X", (T, self.m), self._act_dt())
        if Y is not None:
            _check(Y, "Y", (T, self.n), self._act_dt())
        _check_device(self.device, X=X, Y=Y)
        self.reserve(T)
        if Y is None:
            Y = torch.empty(T, self.n, dtype=X.dtype, device=self.device)
        return T, Y

    def forward(self, X: torch.Tensor, Y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        T, Y = self._fwd_args(X, Y)
        B.poetx_linear_fwd(self.desc, T, X, self.perm_R, self.perm_P, self.Wt, self.g_R, self.g_P, Y, self.H_save,
                           self.ws, self.ws.numel(), stream)
        self.T = T
        return Y

    def _y_arg(self, Y):
        if self.mode == "xout" and Y is None:
            raise ValueError("the xout mode takes H back from the forward's output: pass Y")
        return Y if self.mode == "xout" else None

    def check_backward(self, T: int, dZ: torch.Tensor, Y=None, dX=None, dq_R=None, dq_P=None):
        """Arguments of a backward over T tokens: the saved state must come from a forward of the
        same T tokens, and every tensor must match the layer's shapes, dtype and device."""
        if self.H_save is None or T != self.T:
            raise ValueError(f"backward over {T} tokens, but the saved state is from a forward of {self.T}")
        adt = self._act_dt()
        _check(dZ, "dZ", (T, self.n), adt)
        if self.mode == "xout":
            _check(Y, "Y", (T, self.n), adt)
        if dX is not None:
            _check(dX, "dX", (T, self.m), adt)
        if dq_R is not None:
            _check(dq_R, "dq_R", tuple(self.q_R.shape), torch.float32)
        if dq_P is not None:
            _check(dq_P, "dq_P", tuple(self.q_P.shape), torch.float32)
        _check_device(self.device, dZ=dZ, Y=Y if self.mode == "xout" else None, dX=dX, dq_R=dq_R, dq_P=dq_P)

    def backward(self, X: torch.Tensor, dZ: torch.Tensor, dX=None, dq_R=None, dq_P=None, stream=None, Y=None):
        """X only gives T (the gathered input is in the saved state); Y: the forward's output (xout)."""
        T = X.shape[0]
        self._y_arg(Y)
        self.check_backward(T, dZ, Y, dX, dq_R, dq_P)
        self.reserve(T)
        if dX is None:
            dX = torch.empty(T, self.m, dtype=X.dtype, device=self.device)
        if dq_R is None:
            dq_R = torch.empty_like(self.q_R)
        if dq_P is None:
            dq_P = torch.empty_like(self.q_P)
        B.poetx_linear_bwd(self.desc, T, self._y_arg(Y), dZ, self.perm_R, self.perm_P, self.Wt, self.g_R, self.g_P,
                           self.q_R, self.q_P, self.H_save, dX, dq_R, dq_P, self.ws, self.ws.numel(), stream)
        return dX, dq_R, dq_P

    def merge_reinit(self, seed_R: int, seed_P: int, stream=None):
        ws = self._ws(B.poetx_workspace_size(self.desc, 0, B.POETX_OP_MERGE))
        B.poetx_merge_reinit(self.desc, self.Wt, self.perm_R, self.perm_P, self.g_R, self.g_P, self.q_R, self.q_P,
                             seed_R, seed_P, ws, ws.numel(), stream)

    def merged_f32(self) -> torch.Tensor:
        """fp32 merged weight before rounding, left at the start of the workspace by merge_reinit."""
        ldw = lead(self.n)
        return self.ws[: self.m * ldw * 4].view(torch.float32).view(self.m, ldw)

    def saved_H(self, T: int) -> torch.Tensor:
        if self.mode != "xfast":
            raise ValueError("only the xfast mode saves H")
        dt = _TORCH_DT[self.act]
        return self.H_save.view(dt)[: T * lead(self.n)].view(T, lead(self.n))


class PoetxGroup:
    """Several linears whose CNP work runs batched: one build of every side's G
    (poetx_cnp_build_batch) and one chain rule for every side's dq
    (poetx_cnp_backward_batch) after each linear's poetx_linear_bwd_dx.

    Results are bit-identical to the per-linear calls; the batch only shares
    launches between the sides.

    batch_grads=True also batches the block gradients: backward_dx computes
    only dX (poetx_linear_bwd_dx_sides) and backward_q forms every side's block
    gradients in shared launches (poetx_block_grads_batch) before the chain
    rule.  Their token-split sums then differ from the per-linear calls', so
    dq matches those to fp32 rounding, not bit for bit.  Every linear's
    backward_dx must come before backward_q, with the same T and no other use
    of those linears in between (the operands live in their workspaces and
    saved state).
    """

    def __init__(self, layers, batch_grads: bool = False):
        if not layers:
            raise ValueError("empty group")
        L0 = layers[0]
        if any(l.b != L0.b or l.act != L0.act or l.device != L0.device for l in layers):
            raise ValueError("the linears of a group must share b, act dtype and device")
        self.layers = list(layers)
        self.b, self.act, self.device = L0.b, L0.act, L0.device
        self.adt = B.DTYPES[self.act]
        self.d = [x for l in self.layers for x in (l.m, l.n)]
        self.first, blocks = [], 0
        for l in self.layers:
            self.first.append(blocks)
            blocks += l.nbR + l.nbP
        self.blocks = blocks
        u8 = dict(dtype=torch.uint8, device=self.device)
        self.dg = torch.empty(B.poetx_cnp_grad_bytes(blocks, self.b, self.adt), **u8)
        self.ws = torch.empty(B.poetx_cnp_batch_workspace_size(self.d, self.b, self.adt), **u8)
        self.batch_grads = batch_grads
        self.built = False  # build() ran since the last backward_q: its workspace holds every side's dense Q and S
        self.sides = [None] * len(self.layers)  # batch_grads: block-gradient operands from backward_dx
        self.rows = None
        self.gws = torch.empty(0, **u8)

    def build(self, stream=None):
        """Every side's G in one batch.  The next backward_q reuses the dense Q and S this leaves in the
        group's workspace: the chain rule is then taken at the q these G were built from, as the forward
        used them.  A backward_q without a group build before it forms Q and S from the current q."""
        q = [x for l in self.layers for x in (l.q_R, l.q_P)]
        g = [x for l in self.layers for x in (l.g_R, l.g_P)]
        B.poetx_cnp_build_batch(q, self.d, self.b, self.adt, g, self.ws, self.ws.numel(), stream)
        self.built = True

    def backward_dx(self, i: int, X: torch.Tensor, dZ: torch.Tensor, dX=None, stream=None, Y=None) -> torch.Tensor:
        """dX of linear i; its block gradients go to the group's gradient state, or with batch_grads wait
        for backward_q (Y: as PoetxLinear.backward)."""
        lay = self.layers[i]
        T = X.shape[0]
        lay._y_arg(Y)
        lay.check_backward(T, dZ, Y, dX)
        lay.reserve(T)
        if dX is None:
            dX = torch.empty(T, lay.m, dtype=X.dtype, device=self.device)
        if self.batch_grads:
            if self.rows is not None and self.rows != T:
                raise ValueError(f"batch_grads: every linear's backward_dx needs the same T ({self.rows}), got {T}")
            self.sides[i] = B.poetx_linear_bwd_dx_sides(lay.desc, T, lay._y_arg(Y), dZ, lay.perm_R, lay.perm_P, lay.Wt,
                                                        lay.g_R, lay.g_P, lay.H_save, dX, lay.ws, lay.ws.numel(), stream)
            self.rows = T
            return dX
        B.poetx_linear_bwd_dx(lay.desc, T, lay._y_arg(Y), dZ, lay.perm_R, lay.perm_P, lay.Wt, lay.g_R, lay.g_P,
                              lay.q_R, lay.q_P, lay.H_save, dX, self.dg, self.first[i], self.blocks, lay.ws,
                              lay.ws.numel(), stream)
        return dX

    def _group_idx(self, idx):
        idx = list(idx)
        if not idx or len(idx) > B.POETX_MAX_GROUP:
            raise ValueError(f"a group call takes 1 .. {B.POETX_MAX_GROUP} linears, got {len(idx)}")
        if len(set(idx)) != len(idx) or any(not 0 <= i < len(self.layers) for i in idx):
            raise ValueError(f"linear indices must be distinct and in [0, {len(self.layers)})")
        return idx

    def forward(self, idx, Xs, Ys=None, stream=None):
        """Forwards of the linears `idx` (indices into the group) in shared launches
        (poetx_linear_fwd_group), each output bit-identical to that linear's own forward.  Xs: one input
        per linear, all with the same T (one tensor may serve several linears, as q, k and v share theirs);
        Ys: outputs, or None to allocate them.  Returns the outputs."""
        idx = self._group_idx(idx)
        Ys = [None] * len(idx) if Ys is None else list(Ys)
        if len(Xs) != len(idx) or len(Ys) != len(idx):
            raise ValueError("one input and one output per linear")
        calls, outs, T = [], [], None
        for i, X, Y in zip(idx, Xs, Ys):
            lay = self.layers[i]
            t, Y = lay._fwd_args(X, Y)
            if T is not None and t != T:
                raise ValueError(f"every linear of a group call needs the same T ({T}), got {t}")
            T = t
            calls.append(dict(dsc=lay.desc, X=X, perm_R=lay.perm_R, perm_P=lay.perm_P, Wt=lay.Wt, g_R=lay.g_R,
                              g_P=lay.g_P, Y=Y, H_save=lay.H_save, ws=lay.ws, ws_bytes=lay.ws.numel()))
            outs.append(Y)
        B.poetx_linear_fwd_group(calls, T, stream)
        for i in idx:
            self.layers[i].T = T
        return outs

    def backward_dx_many(self, idx, dZs, dXs=None, stream=None, Ys=None):
        """backward_dx of the linears `idx` in shared launches (poetx_linear_bwd_dx_group; with batch_grads,
        else one backward_dx each): dX of each, bit-identical to its own backward_dx.  dZs: one output
        gradient per linear; dXs: outputs or None; Ys: the forwards' outputs (xout).  Linears given the
        same dX tensor (they read one input) receive the sum of their input gradients, accumulated in
        fp32 and rounded once (with batch_grads).  Returns the dX."""
        idx = self._group_idx(idx)
        n = len(idx)
        dXs = [None] * n if dXs is None else list(dXs)
        Ys = [None] * n if Ys is None else list(Ys)
        if len(dZs) != n or len(dXs) != n or len(Ys) != n:
            raise ValueError("one dZ, dX and Y entry per linear")
        if not self.batch_grads:
            if any(dX is not None and sum(dX is d for d in dXs) > 1 for dX in dXs):
                raise ValueError("a dX shared by several linears (their summed input gradient) needs batch_grads")
            return [self.backward_dx(i, dZ, dZ, dX, stream, Y) for i, dZ, dX, Y in zip(idx, dZs, dXs, Ys)]
        T = dZs[0].shape[0] if isinstance(dZs[0], torch.Tensor) and dZs[0].dim() == 2 else None
        if T is None:
            raise ValueError("dZ must be a 2-D tensor [T, n]")
        if self.rows is not None and self.rows != T:
            raise ValueError(f"batch_grads: every linear's backward_dx needs the same T ({self.rows}), got {T}")
        calls, outs = [], []
        for i, dZ, dX, Y in zip(idx, dZs, dXs, Ys):
            lay = self.layers[i]
            lay._y_arg(Y)
            lay.check_backward(T, dZ, Y, dX)
            lay.reserve(T)
            if dX is None:
                dX = torch.empty(T, lay.m, dtype=dZ.dtype, device=self.device)
            calls.append(dict(dsc=lay.desc, Y=lay._y_arg(Y), dZ=dZ, perm_R=lay.perm_R, perm_P=lay.perm_P, Wt=lay.Wt,
                              g_R=lay.g_R, g_P=lay.g_P, H_save=lay.H_save, dX=dX, ws=lay.ws, ws_bytes=lay.ws.numel()))
            outs.append(dX)
        sides = B.poetx_linear_bwd_dx_group(calls, T, stream)
        for i, sd in zip(idx, sides):
            self.sides[i] = sd
        self.rows = T
        return outs

    def backward_q(self, dqs=None, stream=None):
        """dq of every side from the gradient state; dqs: [(dq_R, dq_P)] per linear (allocated if None)."""
        if self.batch_grads:
            if any(sd is None for sd in self.sides):
                raise ValueError("batch_grads: backward_dx of every linear must come before backward_q")
            need = B.poetx_block_grads_workspace_size(self.d, self.rows, self.b, self.adt)
            if self.gws.numel() < need:
                self.gws = torch.empty(need, dtype=torch.uint8, device=self.device)
            sides = [x for pair in self.sides for x in pair]
            B.poetx_block_grads_batch(sides, self.rows, self.b, self.adt, self.dg, self.dg.numel(), self.gws,
                                      self.gws.numel(), stream)
            self.sides = [None] * len(self.layers)
            self.rows = None
        if dqs is None:
            dqs = [(torch.empty_like(l.q_R), torch.empty_like(l.q_P)) for l in self.layers]
        q = [x for l in self.layers for x in (l.q_R, l.q_P)]
        dq = [x for pair in dqs for x in pair]
        if self.built:
            # the chain rule at the q the forward's G were built from, reading the build's dense Q and S
            B.poetx_cnp_backward_batch_reuse(q, self.d, self.b, self.adt, self.ws, self.ws.numel(), self.dg,
                                             self.dg.numel(), dq, stream)
            self.built = False
        else:
            B.poetx_cnp_backward_batch(q, self.d, self.b, self.adt, self.dg, self.dg.numel(), dq, stream)
        return dqs


class PoetxAdam:
    """Optimiser state for the packed q of several linears, and the training
    cadence around it: each step() moves every side's q by one Adam step with
    decoupled weight decay (one poetx_adam_step_batch call for all sides);
    every `merge_every` steps (0: never) the factors built from the updated q
    are merged into each linear's weight with new permutations
    (poetx_cnp_build, poetx_merge_reinit) and q and both moments restart from
    zero, together with the bias-correction count.

    merge_seeds(step, i) -> (seed_R, seed_P) gives the permutation seeds of
    linear i at the merge after `step` steps.  step() takes a torch.cuda.Stream
    or None (the current stream); the moments are cleared with a torch fill on
    that stream.  The bias correction uses the step count as a launch argument,
    so a captured graph of step() would replay one count.
    """

    def __init__(self, layers, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
                 merge_every: int = 0, merge_seeds=None):
        if not layers:
            raise ValueError("no linears")
        self.layers = list(layers)
        self.lr, self.beta1, self.beta2, self.eps, self.weight_decay = lr, betas[0], betas[1], eps, weight_decay
        self.merge_every = merge_every
        self.merge_seeds = merge_seeds or (lambda step, i: ((step << 16) | (2 * i), (step << 16) | (2 * i + 1)))
        qs = self.params()
        self.m1 = [torch.zeros_like(q) for q in qs]
        self.m2 = [torch.zeros_like(q) for q in qs]
        self.t = 0  # steps since the last restart
        self.steps = 0  # steps taken

    def params(self):
        return [x for l in self.layers for x in (l.q_R, l.q_P)]

    def step(self, dqs, stream=None) -> bool:
        """dqs: [(dq_R, dq_P)] per linear.  Returns True when this step ended with a merge."""
        if stream is not None and not isinstance(stream, torch.cuda.Stream):
            raise TypeError("stream must be a torch.cuda.Stream or None")
        dq = [x for pair in dqs for x in pair]
        if len(dq) != len(self.m1):
            raise ValueError("one (dq_R, dq_P) pair per linear")
        self.t += 1
        self.steps += 1
        B.poetx_adam_step_batch(self.params(), dq, self.m1, self.m2, self.lr, self.beta1, self.beta2, self.eps,
                                self.weight_decay, self.t, stream=stream)
        if not (self.merge_every and self.steps % self.merge_every == 0):
            return False
        for i, lay in enumerate(self.layers):
            lay.build(stream)
            seed_R, seed_P = self.merge_seeds(self.steps, i)
            lay.merge_reinit(seed_R, seed_P, stream)
            lay.build(stream)  # G of the restarted q (the identity), so the layer is usable at once
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            for m in self.m1 + self.m2:
                m.zero_()
        self.t = 0
        return True


class PoetxSpoFactor:
    """One SPO factor applied to token rows, Y = X F (poetx_spo_fwd / poetx_spo_bwd):
    kind "block" permutes all d columns and holds ceil(d/b) CNP blocks; kind
    "full" holds one b x b CNP block on b chosen columns and passes the others
    through.  Owns q, the column indices, G, the saved state and a workspace."""

    def __init__(self, d: int, b: int, kind: str = "block", act: str = "bf16", device: str = "cuda"):
        self.d, self.b, self.kind, self.act = d, b, kind, act
        self.device = torch.device(device)
        self.desc = B.spo_desc(d, b, kind, act)
        self.d_eff = d if kind == "block" else b
        nb = -(-self.d_eff // b)
        self.adt = B.DTYPES[act]
        self.q = torch.zeros(nb, b * (b - 1) // 2, dtype=torch.float32, device=self.device)
        self.idx = torch.arange(self.d_eff, dtype=torch.int32, device=self.device)
        self.g = torch.empty(B.poetx_g_bytes(self.d_eff, b, self.adt), dtype=torch.uint8, device=self.device)
        self.saved = torch.empty(0, dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(0, dtype=torch.uint8, device=self.device)
        self.T = None  # rows of the last forward (the saved state's)

    def load(self, idx, q):
        self.idx.copy_(idx)
        self.q.copy_(q)

    def _ws(self, nbytes: int) -> torch.Tensor:
        if self.ws.numel() < nbytes:
            self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.ws

    def reserve(self, T: int):
        self._ws(max(B.poetx_spo_workspace_size(self.desc, T, B.POETX_OP_FWD),
                     B.poetx_spo_workspace_size(self.desc, T, B.POETX_OP_BWD)))
        need = B.poetx_spo_saved_bytes(self.desc, T)
        if self.saved.numel() < need:
            self.saved = torch.empty(need, dtype=torch.uint8, device=self.device)

    def build(self, stream=None):
        ws = self._ws(B.poetx_workspace_size(B.desc(self.d_eff, 1, self.b, self.act, self.act), 0, B.POETX_OP_CNP))
        B.poetx_cnp_build(self.q, self.d_eff, self.b, self.adt, self.g, ws, ws.numel(), stream)

    def forward(self, X: torch.Tensor, Y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        if not isinstance(X, torch.Tensor) or X.dim() != 2:
            raise ValueError("X must be a 2-D tensor [T, d]")
        T = X.shape[0]
        adt = _TORCH_DT[self.act]
        _check(X, "X", (T, self.d), adt)
        if Y is not None:
            _check(Y, "Y", (T, self.d), adt)
        _check_device(self.device, X=X, Y=Y)
        self.reserve(T)
        if Y is None:
            Y = torch.empty_like(X)
        B.poetx_spo_fwd(self.desc, T, X, self.idx, self.g, Y, self.saved, self.ws, self.ws.numel(), stream)
        self.T = T
        return Y

    def backward(self, dY: torch.Tensor, dX=None, dq=None, stream=None):
        if not isinstance(dY, torch.Tensor) or dY.dim() != 2:
            raise ValueError("dY must be a 2-D tensor [T, d]")
        T = dY.shape[0]
        if T != self.T:
            raise ValueError(f"backward over {T} rows, but the saved state is from a forward of {self.T}")
        adt = _TORCH_DT[self.act]
        _check(dY, "dY", (T, self.d), adt)
        if dX is not None:
            _check(dX, "dX", (T, self.d), adt)
        if dq is not None:
            _check(dq, "dq", tuple(self.q.shape), torch.float32)
        _check_device(self.device, dY=dY, dX=dX, dq=dq)
        self.reserve(T)
        if dX is None:
            dX = torch.empty_like(dY)
        if dq is None:
            dq = torch.empty_like(self.q)
        B.poetx_spo_bwd(self.desc, T, dY, self.idx, self.g, self.q, self.saved, dX, dq, self.ws, self.ws.numel(),
                        stream)
        return dX, dq


class PoetxChain:
    """A linear with c factors per side, Y = X R_1 .. R_c W0 P_1 .. P_c: the
    outer factors R_1 .. R_{c-1} and P_2 .. P_c are PoetxSpoFactor calls around
    the PoetxLinear, which holds the innermost R_c and P_1 (block-stochastic,
    folded next to the weight)."""

    def __init__(self, linear: PoetxLinear, outer_R=(), outer_P=()):
        self.linear, self.outer_R, self.outer_P = linear, list(outer_R), list(outer_P)
        self.Y_lin = None

    def build(self, stream=None):
        for f in self.outer_R + self.outer_P:
            f.build(stream)
        self.linear.build(stream)

    def forward(self, X: torch.Tensor, stream=None) -> torch.Tensor:
        for f in self.outer_R:
            X = f.forward(X, stream=stream)
        Y = self.linear.forward(X, stream=stream)
        self.Y_lin, self.X_lin = Y, X
        for f in self.outer_P:
            Y = f.forward(Y, stream=stream)
        return Y

    def merge_reinit(self, seed_R: int, seed_P: int, outer_seeds=None, stream=None):
        """Merge every factor into the weight and restart them all at the identity.

        The linear's own R_c and P_1 are merged first (poetx_merge_reinit, new permutations from
        seed_R and seed_P); the fp32 merged weight it leaves in its workspace then takes the outer
        factors, P_2 .. P_c and R_{c-1} .. R_1 in that order (poetx_fold_factor), and is stored in
        the layer's weight format (poetx_store_weight).  Every G is rebuilt from the current q
        first.  The outer factors restart with q = 0 and new index arrays drawn from
        outer_seeds(k, side) (k the position in outer_R / outer_P, side "R" or "P"): a permutation
        for a block factor, the first b entries of one for a fully stochastic factor."""
        lin = self.linear
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            self.build(stream)
            lin.merge_reinit(seed_R, seed_P, stream)
            W32 = lin.merged_f32()
            ldw = W32.shape[1]
            need = [B.poetx_store_workspace_size(lin.desc)]
            need += [B.poetx_fold_workspace_size(lin.desc, 1, f.desc) for f in self.outer_P]
            need += [B.poetx_fold_workspace_size(lin.desc, 0, f.desc) for f in self.outer_R]
            ws = torch.empty(max(need + [256]), dtype=torch.uint8, device=lin.device)
            for f in self.outer_P:
                B.poetx_fold_factor(lin.desc, 1, f.desc, f.idx, f.g, lin.perm_P, W32, ldw, ws, ws.numel(), stream)
            for f in reversed(self.outer_R):
                B.poetx_fold_factor(lin.desc, 0, f.desc, f.idx, f.g, lin.perm_R, W32, ldw, ws, ws.numel(), stream)
            B.poetx_store_weight(lin.desc, W32, ldw, lin.Wt, ws, ws.numel(), stream)
            if outer_seeds is None:
                outer_seeds = lambda k, side: ((seed_R if side == "R" else seed_P) + 0x9E3779B97F4A7C15 * (k + 1)) % (1 << 64)
            for side, facs in (("R", self.outer_R), ("P", self.outer_P)):
                for k, f in enumerate(facs):
                    perm = B.poetx_perm_from_seed(outer_seeds(k, side), f.d)[: f.d_eff]
                    f.idx.copy_(torch.from_numpy(perm.copy()))
                    f.q.zero_()
        self.Y_lin = None

    def backward(self, dZ: torch.Tensor, stream=None):
        """Returns dX, [dq of outer_R], (dq_R, dq_P) of the linear, [dq of outer_P]."""
        dq_outer_P = [None] * len(self.outer_P)
        for k in reversed(range(len(self.outer_P))):
            dZ, dq_outer_P[k] = self.outer_P[k].backward(dZ, stream=stream)
        dX, dq_R, dq_P = self.linear.backward(self.X_lin, dZ, stream=stream, Y=self.Y_lin)
        dq_outer_R = [None] * len(self.outer_R)
        for k in reversed(range(len(self.outer_R))):
            dX, dq_outer_R[k] = self.outer_R[k].backward(dX, stream=stream)
        return dX, dq_outer_R, (dq_R, dq_P), dq_outer_P


class PoetxWeightCentric:
    """The weight-centric baseline (poetx_wc_fwd / poetx_wc_bwd) on the state of a
    PoetxLinear: the same pre-merged weight, G blocks, permutations and q, computed
    by applying the factors to the weight first and then one dense contraction per
    direction.  Owns the weight-side state and a workspace."""

    def __init__(self, linear: PoetxLinear):
        if linear.act != linear.w:
            raise ValueError("the weight-centric path takes layers whose weights have the activation dtype")
        self.lin = linear
        u8 = dict(dtype=torch.uint8, device=linear.device)
        self.state = torch.empty(0, **u8)
        self.ws = torch.empty(0, **u8)
        self.T = None

    def reserve(self, T: int):
        d = self.lin.desc
        need = B.poetx_wc_state_bytes(d, T)
        if self.state.numel() < need:
            self.state = torch.empty(max(need, 256), dtype=torch.uint8, device=self.lin.device)
        need = max(B.poetx_wc_workspace_size(d, T, B.POETX_OP_FWD), B.poetx_wc_workspace_size(d, T, B.POETX_OP_BWD))
        if self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.lin.device)

    def forward(self, X: torch.Tensor, Y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        L = self.lin
        if not isinstance(X, torch.Tensor) or X.dim() != 2:
            raise ValueError("X must be a 2-D tensor [T, m]")
        T = X.shape[0]
        _check(X, "X", (T, L.m), L._act_dt())
        if Y is not None:
            _check(Y, "Y", (T, L.n), L._act_dt())
        _check_device(L.device, X=X, Y=Y)
        self.reserve(T)
        if Y is None:
            Y = torch.empty(T, L.n, dtype=X.dtype, device=L.device)
        B.poetx_wc_fwd(L.desc, T, X, L.perm_R, L.perm_P, L.Wt, L.g_R, L.g_P, Y, self.state, self.ws, self.ws.numel(),
                       stream)
        self.T = T
        return Y

    def backward(self, dZ: torch.Tensor, dX=None, dq_R=None, dq_P=None, stream=None):
        L = self.lin
        if not isinstance(dZ, torch.Tensor) or dZ.dim() != 2:
            raise ValueError("dZ must be a 2-D tensor [T, n]")
        T = dZ.shape[0]
        if T != self.T:
            raise ValueError(f"backward over {T} tokens, but the saved state is from a forward of {self.T}")
        adt = L._act_dt()
        _check(dZ, "dZ", (T, L.n), adt)
        if dX is not None:
            _check(dX, "dX", (T, L.m), adt)
        if dq_R is not None:
            _check(dq_R, "dq_R", tuple(L.q_R.shape), torch.float32)
        if dq_P is not None:
            _check(dq_P, "dq_P", tuple(L.q_P.shape), torch.float32)
        _check_device(L.device, dZ=dZ, dX=dX, dq_R=dq_R, dq_P=dq_P)
        if dX is None:
            dX = torch.empty(T, L.m, dtype=dZ.dtype, device=L.device)
        if dq_R is None:
            dq_R = torch.empty_like(L.q_R)
        if dq_P is None:
            dq_P = torch.empty_like(L.q_P)
        B.poetx_wc_bwd(L.desc, T, dZ, L.perm_R, L.perm_P, L.g_R, L.g_P, L.q_R, L.q_P, self.state, dX, dq_R, dq_P,
                       self.ws, self.ws.numel(), stream)
        return dX, dq_R, dq_P
