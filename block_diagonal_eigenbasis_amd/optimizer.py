"""Dobb as a torch optimizer over a set of 2-D weights, driving libdobb.so's grouped entry points.

The cadence follows the Dobb paper (arXiv 2610.39412): second moments are captured on refresh
iterations only (Table 17: first micro-batch by default, a caller policy), the basis is refreshed
every T steps (Table 14; T = 9 in the principal runs), the first refresh is an exact
eigendecomposition and later ones warm-started orthogonal iteration with k = 1 (Table 15), and the
update scale is tau sqrt(max(m, n)/m) with tau = 0.2 (Table 9).

``DobbGroup`` keeps the optimizer state (M, A, Q) of a matrix set as device tensors, marshals the
per-matrix pointer tables once and owns its workspace, so a step is a handful of ctypes calls.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _abi


def default_update_scale(m: int, n: int, tau: float = 0.2) -> float:
    return tau * math.sqrt(max(m, n) / m)


def _arr(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


class _Part:
    """Pre-marshalled launch arguments and a workspace for a subset of a DobbGroup's weights."""

    def __init__(self, g: "DobbGroup", idx, stream):
        self.idx = list(idx)
        self.count = len(self.idx)
        self.stream = stream
        shapes = [g.shapes[i] for i in self.idx]
        self.shapes = shapes
        self.sh = (_abi.Shape * self.count)(*[_abi.Shape(*s) for s in shapes])
        self.ash = (_abi.Shape * self.count)(*[_abi.Shape(1, n, nb) for (_, n, nb) in shapes])
        self.W = _arr([g.W[i].data_ptr() for i in self.idx])
        self.M = _arr([g.M[i].data_ptr() for i in self.idx])
        self.A = _arr([g.A[i].data_ptr() for i in self.idx])
        self.Q = _arr([g.Q[i].data_ptr() for i in self.idx])
        self.lam = _arr([g.lam[i].data_ptr() for i in self.idx])
        self.info = _arr([g.info[i].data_ptr() for i in self.idx])
        self.ldx = (ctypes.c_int64 * self.count)(*[n for (_, n, _) in shapes])
        self.hp = (_abi.HParams * self.count)(*[g.hp[i] for i in self.idx])
        self.ws = None
        self.size_ws(g, g.n_tokens)

    def need(self, norm, n_tokens):
        return max(_abi.dobb_workspace_size(_abi.DOBB_OP_STEP, self.shapes, 0, norm),
                   _abi.dobb_workspace_size(_abi.DOBB_OP_REFRESH, [(1, n, nb) for (_, n, nb) in self.shapes]),
                   _abi.dobb_workspace_size(_abi.DOBB_OP_ACCUMULATE, [(1, n, nb) for (_, n, nb) in self.shapes],
                                            max(n_tokens, 1)))

    def size_ws(self, g, n_tokens):
        need = max(self.need(g.norm, n_tokens), 256)
        if self.ws is None or need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=g.device)
            if self.stream is not None:           # freed only once this stream's work on it is done
                self.ws.record_stream(self.stream)


class DobbGroup:
    """Optimizer state and pre-marshalled launch arguments for a list of weights.

    streams=2 splits the set into the weights with blocks of at most 128 columns and the wider ones
    and runs the two on separate streams (each with its own workspace), joined back into the
    caller's stream: the two kernel families then overlap (the wide blocks' refresh is a chain of
    latency-bound panel launches)."""

    def __init__(self, weights, block_sizes, grads=None, n_tokens: int = 0, lr: float = 2.5e-3,
                 weight_decay: float = 0.0, momentum: float = 0.9, tau: float = 0.2, nesterov: bool = False,
                 norm: int = _abi.DOBB_NORM_SIGN, update_scales=None, streams: int = 1):
        self.W = list(weights)
        self.nb = [int(b) for b in block_sizes]
        if len(self.nb) != len(self.W):
            raise ValueError("one block size per weight")
        dev = self.W[0].device
        self.device = dev
        self.count = len(self.W)
        self.shapes = [(w.shape[0], w.shape[1], nb) for w, nb in zip(self.W, self.nb)]
        for (m, n, nb) in self.shapes:
            if n % nb:
                raise ValueError(f"block size {nb} does not divide {n}")
        self.M = [torch.zeros(w.shape, dtype=torch.float32, device=dev) for w in self.W]
        self.A = [torch.zeros(n // nb, nb, nb, dtype=torch.float32, device=dev) for (_, n, nb) in self.shapes]
        eye = [torch.eye(nb, dtype=torch.float32, device=dev).expand(n // nb, nb, nb).contiguous()
               for (_, n, nb) in self.shapes]
        self.Q = eye                       # Q = I before the first refresh (the step is then sign(M))
        self.lam = [torch.zeros(n // nb, nb, dtype=torch.float32, device=dev) for (_, n, nb) in self.shapes]
        self.info = [torch.zeros(n // nb, dtype=torch.int32, device=dev) for (_, n, nb) in self.shapes]
        self.G = list(grads) if grads is not None else None
        scales = update_scales or [default_update_scale(m, n, tau) for (m, n, _) in self.shapes]
        self.hp = [_abi.make_hparams(lr, weight_decay, momentum, s, nesterov, norm) for s in scales]
        self.norm = norm
        self._w_dtype = _abi._dtype_code(self.W[0])
        self.n_tokens = n_tokens
        self._parts = []
        self.set_streams(streams)
        self.refreshes = 0

    def set_streams(self, streams: int) -> None:
        """Partition the weights for `streams` streams (1 or 2); the state tensors are kept.  A
        replaced workspace is freed in stream order (the second stream's one is recorded on it)."""
        narrow = [i for i, nb in enumerate(self.nb) if nb <= 128]
        wide = [i for i, nb in enumerate(self.nb) if nb > 128]
        self._parts = []
        if streams > 1 and narrow and wide:
            self._parts = [_Part(self, wide, None), _Part(self, narrow, torch.cuda.Stream(self.device))]
        else:
            self._parts = [_Part(self, range(self.count), None)]

    def _run(self, stream, fn):
        """fn(part, stream handle) for every part: the first on the caller's stream, the others on
        their own streams, forked from and joined back into the caller's stream."""
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        for part in self._parts[1:]:
            part.stream.wait_stream(main)
        for part in self._parts:
            fn(part, _abi._stream(main if part.stream is None else part.stream))
        for part in self._parts[1:]:
            main.wait_stream(part.stream)

    def _grow(self, N: int) -> None:
        if N > self.n_tokens:
            for part in self._parts:
                part.size_ws(self, N)
            self.n_tokens = N

    def _accumulate(self, part, sh, xs, beta):
        xp = _arr([xs[i].data_ptr() for i in part.idx])
        _abi._check(_abi.lib().dobb_accumulate_moment_grouped(
            part.count, part.ash, xp, _abi._dtype_code(xs[part.idx[0]]), xs[part.idx[0]].shape[0], part.ldx,
            float(beta), part.A, part.ws.data_ptr(), part.ws.numel(), sh), "dobb_accumulate_moment_grouped")

    def _refresh(self, part, sh, mode, iters, warm_start, tol, with_lam):
        _abi._check(_abi.lib().dobb_refresh_basis_grouped(
            part.count, part.ash, part.A, part.Q, part.lam if with_lam else None, int(mode), int(iters),
            int(bool(warm_start)), float(tol), part.info, part.ws.data_ptr(), part.ws.numel(), sh),
            "dobb_refresh_basis_grouped")

    def _step(self, part, sh, G):
        gp = _arr([G[i].data_ptr() for i in part.idx])
        _abi._check(_abi.lib().dobb_step_grouped(
            part.count, part.sh, part.W, self._w_dtype, gp, _abi._dtype_code(G[part.idx[0]]), part.M, part.Q,
            part.hp, None, part.ws.data_ptr(), part.ws.numel(), sh), "dobb_step_grouped")

    def accumulate(self, xs, beta: float, stream=None) -> None:
        """Capture: A_b <- beta A_b + (1-beta)/N X_b^T X_b for every weight (xs[i] is N x n_i)."""
        self._grow(xs[0].shape[0])
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
        self._grow(xs[0].shape[0])
        G = grads if grads is not None else self.G
        with_lam = want_lambda or mode == _abi.DOBB_REFRESH_EXACT

        def go(part, sh):
            self._accumulate(part, sh, xs, beta)
            self._refresh(part, sh, mode, iters, warm_start, tol, with_lam)
            self._step(part, sh, G)
        self._run(stream, go)
        self.refreshes += 1


class Dobb(torch.optim.Optimizer):
    """torch.optim interface: 2-D parameters only, each with a block size (default: n // blocks).

    Activations are supplied by the caller with ``capture(param, x)`` (or the forward hooks from
    ``attach_capture_hooks``) before ``step()`` on refresh iterations; ``wants_capture()`` says whether
    the coming step refreshes.
    """

    def __init__(self, params, lr: float = 2.5e-3, weight_decay: float = 0.0, momentum: float = 0.9,
                 blocks: int = 16, block_size: int | None = None, refresh_period: int = 9, orth_iters: int = 1,
                 beta: float = 0.9, tau: float = 0.2, nesterov: bool = False, streams: int = 1):
        params = list(params)
        super().__init__(params, dict(lr=lr, weight_decay=weight_decay, momentum=momentum))
        for p in params:
            if p.dim() != 2:
                raise ValueError("Dobb handles 2-D weights; use another optimizer for the rest")
        nbs = [block_size or p.shape[1] // blocks for p in params]
        self._params = params
        self._group = DobbGroup([p.data for p in params], nbs, lr=lr, weight_decay=weight_decay,
                                momentum=momentum, tau=tau, nesterov=nesterov, streams=streams)
        self.T = int(refresh_period)
        self.k = int(orth_iters)
        self.beta = float(beta)
        self.t = 0
        self._captured: dict[int, torch.Tensor] = {}

    def wants_capture(self) -> bool:
        return self.t % self.T == 0

    def capture(self, param, x: torch.Tensor) -> None:
        """Record the (tokens x n) input activations of `param` for the next refresh."""
        self._captured[id(param)] = x.detach().reshape(-1, x.shape[-1]).contiguous()

    def attach_capture_hooks(self, modules):
        """Forward pre-hooks on nn.Linear modules whose weights this optimizer owns: on refresh
        iterations the first call's input (first micro-batch) is captured."""
        handles = []
        owned = {id(p) for p in self._params}
        for mod in modules:
            w = getattr(mod, "weight", None)
            if w is None or id(w) not in owned:
                continue

            def hook(module, inputs, w=w):
                if self.wants_capture() and id(w) not in self._captured:
                    self.capture(w, inputs[0])
            handles.append(mod.register_forward_pre_hook(hook))
        return handles

    @torch.no_grad()
    def step(self, closure=None):
        loss = closure() if closure is not None else None
        g = self._group
        grads = [p.grad if p.grad is not None else torch.zeros_like(p) for p in self._params]
        if self.wants_capture() and len(self._captured) == len(self._params):
            xs = [self._captured[id(p)] for p in self._params]
            if len({x.shape[0] for x in xs}) == 1:
                if g.refreshes == 0:
                    g.refresh_step(xs, 0.0, _abi.DOBB_REFRESH_EXACT, 0, grads, warm_start=False)
                else:
                    g.refresh_step(xs, self.beta, _abi.DOBB_REFRESH_ORTH_ITER, self.k, grads)
            else:
                for x, A, (_, n, nb) in zip(xs, g.A, g.shapes):
                    _abi.dobb_accumulate_moment(x, A, nb, self.beta if g.refreshes else 0.0)
                if g.refreshes == 0:
                    g.refresh(_abi.DOBB_REFRESH_EXACT, 0, warm_start=False)
                else:
                    g.refresh(_abi.DOBB_REFRESH_ORTH_ITER, self.k)
                g.step(grads)
        else:
            g.step(grads)
        self._captured.clear()
        self.t += 1
        return loss
