"""Dobb as a torch optimizer over a set of 2-D weights, driving libdobb.so's grouped entry points.

The cadence follows the Dobb paper (arXiv 2610.39412): second moments are captured on refresh
iterations only (Table 17: from the first micro-batch by default, or from all of them), the basis is
refreshed every T steps (Table 14; T = 9 in the principal runs), the first refresh is an exact
eigendecomposition and later ones warm-started orthogonal iteration with k = 1 (Table 15), the basis
may be stored in bf16 (Table 18's principal setting), and the update scale is tau sqrt(max(m, n)/m)
with tau = 0.2 (Table 9).  Dobb-G (Tables 12-13) takes the basis from the output-gradient second
moment instead, with blocks of rows: side="output" (update scale tau sqrt(max(m, n)/n), Table 9).

``DobbGroup`` keeps the optimizer state (M, A, Q) of a matrix set as device tensors, marshals the
per-matrix pointer tables once and owns its workspace, so a step is a handful of ctypes calls.  The
C ABI takes one dtype per argument of a grouped call, so the set is partitioned by weight dtype, and
activations and gradients of mixed dtypes (or token counts) are passed in one call per kind.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _abi


def default_update_scale(m: int, n: int, tau: float = 0.2) -> float:
    return tau * math.sqrt(max(m, n) / m)


def default_update_scale_g(m: int, n: int, tau: float = 0.2) -> float:
    """Dobb-G (Table 9): RMS tau sqrt(max(m, n)/n) for the sign update."""
    return tau * math.sqrt(max(m, n) / n)


def _arr(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def _split(idx, key):
    """idx partitioned by key(i), in first-seen order."""
    out = {}
    for i in idx:
        out.setdefault(key(i), []).append(i)
    return list(out.values())


class _Part:
    """Pre-marshalled launch arguments and a workspace for a subset of a DobbGroup's weights (all of
    one weight dtype)."""

    def __init__(self, g: "DobbGroup", idx, stream):
        self.idx = list(idx)
        self.count = len(self.idx)
        self.stream = stream
        shapes = [g.shapes[i] for i in self.idx]
        self.shapes = shapes
        self.sh = (_abi.Shape * self.count)(*[_abi.Shape(*s) for s in shapes])
        # the moments and bases live on the captured axis: inputs (n) for Dobb, outputs (m) for Dobb-G
        self.cshapes = [(1, g.cap_dim(i), g.nb[i]) for i in self.idx]
        self.ash = (_abi.Shape * self.count)(*[_abi.Shape(*c) for c in self.cshapes])
        self.w_dtype = _abi._dtype_code(g.W[self.idx[0]])
        self.W = _arr([g.W[i].data_ptr() for i in self.idx])
        self.M = _arr([g.M[i].data_ptr() for i in self.idx])
        self.A = _arr([g.A[i].data_ptr() for i in self.idx])
        self.Q = _arr([g.Q[i].data_ptr() for i in self.idx])
        self.lam = _arr([g.lam[i].data_ptr() for i in self.idx])
        self.info = _arr([g.info[i].data_ptr() for i in self.idx])
        self.ldx = (ctypes.c_int64 * self.count)(*[c[1] for c in self.cshapes])
        self.hp = (_abi.HParams * self.count)(*[g.hp[i] for i in self.idx])
        self.ws = None
        self.device = g.device
        self.ensure(self.need(g, g.n_tokens))

    def need(self, g, n_tokens):
        qv = _abi.DOBB_WS_BF16_BASIS if g.q_dtype == _abi.DOBB_BF16 else 0
        ash = self.cshapes
        return max(_abi.dobb_workspace_size(g.step_op, self.shapes, 0, g.norm | qv),
                   _abi.dobb_workspace_size(_abi.DOBB_OP_REFRESH, ash, 0, qv),
                   _abi.dobb_workspace_size(_abi.DOBB_OP_ACCUMULATE, ash, max(n_tokens, 1)))

    def ensure(self, nbytes):
        """Grow the workspace to at least nbytes.  A replaced workspace is freed in stream order (the
        second stream's one is recorded on it)."""
        nbytes = max(int(nbytes), 256)
        if self.ws is None or nbytes > self.ws.numel():
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            if self.stream is not None:
                self.ws.record_stream(self.stream)

    def refresh_hp(self, g):
        for k, i in enumerate(self.idx):
            self.hp[k] = g.hp[i]


class DobbGroup:
    """Optimizer state and pre-marshalled launch arguments for a list of weights.

    streams=2 splits the set into the weights with blocks of at most 128 columns and the wider ones
    and runs the two on separate streams (each with its own workspace), joined back into the
    caller's stream: the two kernel families then overlap (the wide blocks' refresh is a chain of
    latency-bound panel launches).  basis_dtype=torch.bfloat16 stores every Q_b in bf16.
    side="output" runs Dobb-G: block_sizes divide the output dimensions, the moments are captured from
    output gradients (accumulate takes N x m tensors) and the step is dobb_step_g."""

    def __init__(self, weights, block_sizes, grads=None, n_tokens: int = 0, lr: float = 2.5e-3,
                 weight_decay: float = 0.0, momentum: float = 0.9, tau: float = 0.2, nesterov: bool = False,
                 norm: int = _abi.DOBB_NORM_SIGN, update_scales=None, streams: int = 1,
                 basis_dtype: torch.dtype = torch.float32, side: str = "input"):
        if side not in ("input", "output"):
            raise ValueError('side must be "input" (Dobb) or "output" (Dobb-G)')
        self.side = side
        self.step_op = _abi.DOBB_OP_STEP if side == "input" else _abi.DOBB_OP_STEP_G
        self.W = list(weights)
        self.nb = [int(b) for b in block_sizes]
        if len(self.nb) != len(self.W):
            raise ValueError("one block size per weight")
        dev = self.W[0].device
        self.device = dev
        self.count = len(self.W)
        for w in self.W:
            _abi._dtype_code(w)
            if w.dim() != 2 or not w.is_contiguous() or w.device != dev:
                raise ValueError("weights must be contiguous 2-D tensors on one device")
        self.shapes = [(w.shape[0], w.shape[1], nb) for w, nb in zip(self.W, self.nb)]
        for i, nb in enumerate(self.nb):
            if self.cap_dim(i) % nb:
                raise ValueError(f"block size {nb} does not divide {self.cap_dim(i)}")
        if basis_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("basis_dtype must be torch.float32 or torch.bfloat16")
        self.q_dtype = _abi.DOBB_BF16 if basis_dtype == torch.bfloat16 else _abi.DOBB_F32
        self.M = [torch.zeros(w.shape, dtype=torch.float32, device=dev) for w in self.W]
        nblk = [self.cap_dim(i) // nb for i, nb in enumerate(self.nb)]
        self.A = [torch.zeros(B, nb, nb, dtype=torch.float32, device=dev) for B, nb in zip(nblk, self.nb)]
        # Q = I before the first refresh (the step is then sign(M)); the identity is exact in bf16
        self.Q = [torch.eye(nb, dtype=basis_dtype, device=dev).expand(B, nb, nb).contiguous()
                  for B, nb in zip(nblk, self.nb)]
        self.lam = [torch.zeros(B, nb, dtype=torch.float32, device=dev) for B, nb in zip(nblk, self.nb)]
        self.info = [torch.zeros(B, dtype=torch.int32, device=dev) for B in nblk]
        self.G = list(grads) if grads is not None else None
        scale_fn = default_update_scale if side == "input" else default_update_scale_g
        scales = update_scales or [scale_fn(m, n, tau) for (m, n, _) in self.shapes]
        self.hp = [_abi.make_hparams(lr, weight_decay, momentum, s, nesterov, norm) for s in scales]
        self.norm = norm
        self.n_tokens = n_tokens
        self._parts = []
        self.set_streams(streams)
        self.refreshes = 0

    def cap_dim(self, i: int) -> int:
        """The dimension the moments of weight i are captured on: n (inputs) or m (outputs, Dobb-G)."""
        return self.W[i].shape[1] if self.side == "input" else self.W[i].shape[0]

    def set_streams(self, streams: int) -> None:
        """Partition the weights for `streams` streams (1 or 2), and by weight dtype; the state
        tensors are kept."""
        narrow = [i for i, nb in enumerate(self.nb) if nb <= 128]
        wide = [i for i, nb in enumerate(self.nb) if nb > 128]
        wdt = lambda i: self.W[i].dtype  # noqa: E731
        self._parts = []
        if streams > 1 and narrow and wide:
            side = torch.cuda.Stream(self.device)
            self._parts = [_Part(self, sub, None) for sub in _split(wide, wdt)]
            self._parts += [_Part(self, sub, side) for sub in _split(narrow, wdt)]
        else:
            self._parts = [_Part(self, sub, None) for sub in _split(range(self.count), wdt)]

    def set_hparams(self, idx=None, lr=None, weight_decay=None, momentum=None) -> None:
        """Change lr, weight decay or momentum of the weights idx (default: all) for later steps."""
        for i in range(self.count) if idx is None else idx:
            h = self.hp[i]
            self.hp[i] = _abi.make_hparams(h.lr if lr is None else lr,
                                           h.weight_decay if weight_decay is None else weight_decay,
                                           h.momentum if momentum is None else momentum,
                                           h.update_scale, bool(h.nesterov), h.norm)
        for part in self._parts:
            part.refresh_hp(self)

    def _run(self, stream, fn):
        """fn(part, stream handle) for every part: those without a stream of their own on the caller's
        stream, the others on theirs, forked from and joined back into the caller's stream."""
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        sides = []
        for part in self._parts:
            if part.stream is not None and part.stream not in sides:
                sides.append(part.stream)
        for s in sides:
            s.wait_stream(main)
        for part in self._parts:
            fn(part, _abi._stream(main if part.stream is None else part.stream))
        for s in sides:
            main.wait_stream(s)

    def _grow(self, N: int) -> None:
        if N > self.n_tokens:
            for part in self._parts:
                part.ensure(part.need(self, N))
            self.n_tokens = N

    def _accumulate(self, part, sh, xs, beta):
        """One grouped capture per (activation dtype, token count) among the part's weights."""
        for sub in _split(part.idx, lambda i: (xs[i].dtype, xs[i].shape[0])):
            if len(sub) == part.count:
                ash, A, ldx = part.ash, part.A, part.ldx
            else:
                ash = (_abi.Shape * len(sub))(*[_abi.Shape(1, self.cap_dim(i), self.nb[i]) for i in sub])
                A = _arr([self.A[i].data_ptr() for i in sub])
                ldx = (ctypes.c_int64 * len(sub))(*[self.cap_dim(i) for i in sub])
            for i in sub:
                x = xs[i]
                if x.dim() != 2 or x.shape[1] != self.cap_dim(i) or not x.is_contiguous() or x.device != self.device:
                    raise ValueError(f"capture {i} must be a contiguous (tokens x {self.cap_dim(i)}) tensor")
            N = xs[sub[0]].shape[0]
            part.ensure(_abi.dobb_workspace_size(_abi.DOBB_OP_ACCUMULATE,
                                                 [(1, self.cap_dim(i), self.nb[i]) for i in sub], N))
            _abi._check(_abi.lib().dobb_accumulate_moment_grouped(
                len(sub), ash, _arr([xs[i].data_ptr() for i in sub]), _abi._dtype_code(xs[sub[0]]), N, ldx,
                float(beta), A, part.ws.data_ptr(), part.ws.numel(), sh), "dobb_accumulate_moment_grouped")

    def _refresh(self, part, sh, mode, iters, warm_start, tol, with_lam):
        _abi._check(_abi.lib().dobb_refresh_basis_grouped(
            part.count, part.ash, part.A, part.Q, self.q_dtype, part.lam if with_lam else None, int(mode),
            int(iters), int(bool(warm_start)), float(tol), part.info, part.ws.data_ptr(), part.ws.numel(), sh),
            "dobb_refresh_basis_grouped")

    def _step(self, part, sh, G):
        """One grouped step per gradient dtype among the part's weights."""
        for i in part.idx:
            g = G[i]
            if tuple(g.shape) != tuple(self.W[i].shape) or not g.is_contiguous() or g.device != self.device:
                raise ValueError(f"gradient {i} must be a contiguous tensor of shape {tuple(self.W[i].shape)}")
        for sub in _split(part.idx, lambda i: G[i].dtype):
            if len(sub) == part.count:
                shp, Wp, Mp, Qp, hp = part.sh, part.W, part.M, part.Q, part.hp
            else:
                pos = {i: k for k, i in enumerate(part.idx)}
                shp = (_abi.Shape * len(sub))(*[_abi.Shape(*self.shapes[i]) for i in sub])
                Wp = _arr([self.W[i].data_ptr() for i in sub])
                Mp = _arr([self.M[i].data_ptr() for i in sub])
                Qp = _arr([self.Q[i].data_ptr() for i in sub])
                hp = (_abi.HParams * len(sub))(*[part.hp[pos[i]] for i in sub])
            fn = _abi.lib().dobb_step_grouped if self.side == "input" else _abi.lib().dobb_step_g_grouped
            _abi._check(fn(len(sub), shp, Wp, part.w_dtype, _arr([G[i].data_ptr() for i in sub]),
                           _abi._dtype_code(G[sub[0]]), Mp, Qp, self.q_dtype, hp, None, None, part.ws.data_ptr(),
                           part.ws.numel(), sh), "dobb_step_grouped" if self.side == "input" else "dobb_step_g_grouped")

    def accumulate(self, xs, beta: float, stream=None) -> None:
        """Capture: A_b <- beta A_b + (1-beta)/N X_b^T X_b for every weight (xs[i] is N_i x n_i, or the
        N_i x m_i output gradients for Dobb-G)."""
        self._grow(max(x.shape[0] for x in xs))
        self._run(stream, lambda part, sh: self._accumulate(part, sh, xs, beta))

    def refresh(self, mode: int, iters: int, warm_start: bool = True, tol: float = 0.0, want_lambda: bool = False,
                stream=None) -> None:
        """Refresh every basis; lambda is filled for the exact mode, and for orthogonal iteration only
        when want_lambda (Rayleigh quotients cost an extra product per block)."""
        with_lam = want_lambda or mode == _abi.DOBB_REFRESH_EXACT
        self._run(stream, lambda part, sh: self._refresh(part, sh, mode, iters, warm_start, tol, with_lam))
        self.refreshes += 1

    def step(self, grads=None, stream=None) -> None:
        G = grads if grads is not None else self.G
        self._run(stream, lambda part, sh: self._step(part, sh, G))

    def refresh_step(self, xs, beta: float, mode: int, iters: int, grads=None, warm_start: bool = True,
                     tol: float = 0.0, want_lambda: bool = False, stream=None) -> None:
        """accumulate, refresh and step in one call: each part runs the three phases back to back on
        its own stream, so with streams=2 one part's refresh overlaps the other's capture and step.
        The result is the same as the three calls in turn."""
        self._grow(max(x.shape[0] for x in xs))
        G = grads if grads is not None else self.G
        with_lam = want_lambda or mode == _abi.DOBB_REFRESH_EXACT

        def go(part, sh):
            self._accumulate(part, sh, xs, beta)
            self._refresh(part, sh, mode, iters, warm_start, tol, with_lam)
            self._step(part, sh, G)
        self._run(stream, go)
        self.refreshes += 1

    def capture_refresh_step(self, xs, beta: float, mode: int, iters: int, grads=None,
                             warm_start: bool = True) -> "torch.cuda.CUDAGraph":
        """A HIP graph of refresh_step(xs, beta, mode, iters, grads): replaying it runs the same
        kernels on the same buffers without the per-launch host work and gaps.  xs, the gradients and
        the optimizer state are bound by address, so the caller refills them in place between replays.
        Capturing runs nothing; the workspaces must already have their size, so call refresh_step once
        (or accumulate with the same token counts) first.  Each replay counts as one refresh."""
        N = max(x.shape[0] for x in xs)
        if N > self.n_tokens:
            raise RuntimeError("call refresh_step once before capturing it (the workspaces are sized there)")
        graph = torch.cuda.CUDAGraph()
        refreshes = self.refreshes
        with torch.cuda.graph(graph):
            self.refresh_step(xs, beta, mode, iters, grads=grads, warm_start=warm_start)
        self.refreshes = refreshes
        return graph


class Dobb(torch.optim.Optimizer):
    """torch.optim interface: 2-D parameters only, each with a block size (default: n // blocks).

    lr, weight_decay and momentum are read from each parameter group at every step, so learning-rate
    schedulers and later edits of ``param_groups`` take effect.  Activations are supplied by the
    caller with ``capture(param, x)`` (or the forward hooks from ``attach_capture_hooks``) before
    ``step()`` on refresh iterations; ``wants_capture()`` says whether the coming step refreshes.
    capture="first" keeps a weight's first micro-batch of a refresh iteration (the principal policy
    of Table 17), capture="all" every micro-batch (their tokens are pooled into one capture).
    basis="output_gradient" runs Dobb-G (Tables 12-13): blocks of rows (m // blocks, or block_size),
    bases of the output-gradient second moment, captured by the backward hooks of
    ``attach_capture_hooks`` (or ``capture(param, grad_output)``).
    """

    def __init__(self, params, lr: float = 2.5e-3, weight_decay: float = 0.0, momentum: float = 0.9,
                 blocks: int = 16, block_size: int | None = None, refresh_period: int = 9, orth_iters: int = 1,
                 beta: float = 0.9, tau: float = 0.2, nesterov: bool = False, streams: int = 1,
                 capture: str = "first", basis_dtype: torch.dtype = torch.float32, basis: str = "activation"):
        super().__init__(params, dict(lr=lr, weight_decay=weight_decay, momentum=momentum))
        if capture not in ("first", "all"):
            raise ValueError('capture must be "first" or "all"')
        if basis not in ("activation", "output_gradient"):
            raise ValueError('basis must be "activation" (Dobb) or "output_gradient" (Dobb-G)')
        params = [p for grp in self.param_groups for p in grp["params"]]
        for p in params:
            if p.dim() != 2:
                raise ValueError("Dobb handles 2-D weights; use another optimizer for the rest")
        self.side = "input" if basis == "activation" else "output"
        axis = 1 if self.side == "input" else 0
        nbs = [block_size or p.shape[axis] // blocks for p in params]
        self._params = params
        self._group = DobbGroup([p.data for p in params], nbs, lr=lr, weight_decay=weight_decay,
                                momentum=momentum, tau=tau, nesterov=nesterov, streams=streams,
                                basis_dtype=basis_dtype, side=self.side)
        self._slots = []                      # per param group: the weight indices
        k = 0
        for grp in self.param_groups:
            self._slots.append(list(range(k, k + len(grp["params"]))))
            k += len(grp["params"])
        self._applied = [None] * len(self.param_groups)
        self.capture_policy = capture
        self.T = int(refresh_period)
        self.k = int(orth_iters)
        self.beta = float(beta)
        self.t = 0
        self._captured: dict[int, list] = {}

    def wants_capture(self) -> bool:
        return self.t % self.T == 0

    def capture(self, param, x: torch.Tensor) -> None:
        """Record (tokens x n) input activations of `param` (Dobb), or (tokens x m) output gradients
        (Dobb-G), for the next refresh: the first call per refresh iteration, or every call with
        capture="all"."""
        x = x.detach().reshape(-1, x.shape[-1])
        got = self._captured.setdefault(id(param), [])
        if self.capture_policy == "all" or not got:
            got.append(x.contiguous())

    def attach_capture_hooks(self, modules):
        """Hooks on nn.Linear modules whose weights this optimizer owns: on refresh iterations their
        inputs (forward pre-hooks; Dobb) or output gradients (backward hooks; Dobb-G) are captured,
        from the first micro-batch, or all of them with capture="all"."""
        handles = []
        owned = {id(p) for p in self._params}
        for mod in modules:
            w = getattr(mod, "weight", None)
            if w is None or id(w) not in owned:
                continue
            if self.side == "input":
                def hook(module, inputs, w=w):
                    if self.wants_capture():
                        self.capture(w, inputs[0])
                handles.append(mod.register_forward_pre_hook(hook))
            else:
                def bhook(module, grad_input, grad_output, w=w):
                    if self.wants_capture() and grad_output[0] is not None:
                        self.capture(w, grad_output[0])
                handles.append(mod.register_full_backward_hook(bhook))
        return handles

    def _sync_hparams(self) -> None:
        for gi, grp in enumerate(self.param_groups):
            cur = (float(grp["lr"]), float(grp["weight_decay"]), float(grp["momentum"]))
            if cur != self._applied[gi]:
                self._group.set_hparams(self._slots[gi], lr=cur[0], weight_decay=cur[1], momentum=cur[2])
                self._applied[gi] = cur

    @torch.no_grad()
    def step(self, closure=None):
        loss = closure() if closure is not None else None
        self._sync_hparams()
        g = self._group
        grads = [p.grad if p.grad is not None else torch.zeros_like(p) for p in self._params]
        if self.wants_capture() and len(self._captured) == len(self._params):
            xs = []
            for p in self._params:
                parts = self._captured[id(p)]
                xs.append(parts[0] if len(parts) == 1 else torch.cat(parts, 0))
            if g.refreshes == 0:
                g.refresh_step(xs, 0.0, _abi.DOBB_REFRESH_EXACT, 0, grads, warm_start=False)
            else:
                g.refresh_step(xs, self.beta, _abi.DOBB_REFRESH_ORTH_ITER, self.k, grads)
        else:
            g.step(grads)
        self._captured.clear()
        self.t += 1
        return loss
