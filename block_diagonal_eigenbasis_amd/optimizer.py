"""Dobb as a torch optimizer over a set of 2-D weights, driving libdobb.so's grouped entry points.

The cadence follows the Dobb paper (arXiv 2610.39412): second moments are captured on refresh
iterations only (Table 17: first micro-batch by default, a caller policy), the basis is refreshed
every T steps (Table 14; T = 9 in the principal runs), the first refresh is an exact
eigendecomposition and later ones warm-started orthogonal iteration with k = 1 (Table 15), and the
update scale is tau sqrt(max(m, n)/m) with tau = 0.2 (Table 9).

``DobbGroup`` keeps the optimizer state (M, A, Q) of a matrix set as device tensors, marshals the
per-matrix pointer tables once and owns one workspace, so a step is a handful of ctypes calls.
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


class DobbGroup:
    """Optimizer state and pre-marshalled launch arguments for a list of weights."""

    def __init__(self, weights, block_sizes, grads=None, n_tokens: int = 0, lr: float = 2.5e-3,
                 weight_decay: float = 0.0, momentum: float = 0.9, tau: float = 0.2, nesterov: bool = False,
                 norm: int = _abi.DOBB_NORM_SIGN, update_scales=None):
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
        self.hp = (_abi.HParams * self.count)(*[
            _abi.make_hparams(lr, weight_decay, momentum, s, nesterov, norm) for s in scales])
        self.norm = norm
        self._sh = (_abi.Shape * self.count)(*[_abi.Shape(*s) for s in self.shapes])
        self._ash = (_abi.Shape * self.count)(*[_abi.Shape(1, n, nb) for (_, n, nb) in self.shapes])
        self._W = _arr([w.data_ptr() for w in self.W])
        self._M = _arr([t.data_ptr() for t in self.M])
        self._A = _arr([t.data_ptr() for t in self.A])
        self._Q = _arr([t.data_ptr() for t in self.Q])
        self._lam = _arr([t.data_ptr() for t in self.lam])
        self._info = _arr([t.data_ptr() for t in self.info])
        self._ldx = (ctypes.c_int64 * self.count)(*[n for (_, n, _) in self.shapes])
        self._w_dtype = _abi._dtype_code(self.W[0])
        need = max(_abi.dobb_workspace_size(_abi.DOBB_OP_STEP, self.shapes, 0, norm),
                   _abi.dobb_workspace_size(_abi.DOBB_OP_REFRESH, [(1, n, nb) for (_, n, nb) in self.shapes]),
                   _abi.dobb_workspace_size(_abi.DOBB_OP_ACCUMULATE, [(1, n, nb) for (_, n, nb) in self.shapes],
                                            max(n_tokens, 1)))
        self.n_tokens = n_tokens
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self.refreshes = 0

    def _stream(self, stream):
        return _abi._stream(stream)

    def accumulate(self, xs, beta: float, stream=None) -> None:
        """Capture: A_b <- beta A_b + (1-beta)/N X_b^T X_b for every weight (xs[i] is N x n_i)."""
        N = xs[0].shape[0]
        if N > self.n_tokens and _abi.dobb_workspace_size(
                _abi.DOBB_OP_ACCUMULATE, [(1, n, nb) for (_, n, nb) in self.shapes], N) > self.ws.numel():
            raise ValueError("workspace sized for fewer tokens; pass n_tokens to DobbGroup")
        xp = _arr([x.data_ptr() for x in xs])
        _abi._check(_abi.lib().dobb_accumulate_moment_grouped(
            self.count, self._ash, xp, _abi._dtype_code(xs[0]), N, self._ldx, float(beta), self._A,
            self.ws.data_ptr(), self.ws.numel(), self._stream(stream)), "dobb_accumulate_moment_grouped")

    def refresh(self, mode: int, iters: int, warm_start: bool = True, tol: float = 0.0, want_lambda: bool = False,
                stream=None) -> None:
        """Refresh every basis; lambda is filled for the exact mode, and for orthogonal iteration only
        when want_lambda (Rayleigh quotients cost an extra product per block)."""
        lam = self._lam if (want_lambda or mode == _abi.DOBB_REFRESH_EXACT) else None
        _abi._check(_abi.lib().dobb_refresh_basis_grouped(
            self.count, self._ash, self._A, self._Q, lam, int(mode), int(iters), int(bool(warm_start)),
            float(tol), self._info, self.ws.data_ptr(), self.ws.numel(), self._stream(stream)),
            "dobb_refresh_basis_grouped")
        self.refreshes += 1

    def step(self, grads=None, stream=None) -> None:
        G = grads if grads is not None else self.G
        gp = _arr([g.data_ptr() for g in G])
        _abi._check(_abi.lib().dobb_step_grouped(
            self.count, self._sh, self._W, self._w_dtype, gp, _abi._dtype_code(G[0]), self._M, self._Q, self.hp,
            None, self.ws.data_ptr(), self.ws.numel(), self._stream(stream)), "dobb_step_grouped")


class Dobb(torch.optim.Optimizer):
    """torch.optim interface: 2-D parameters only, each with a block size (default: n // blocks).

    Activations are supplied by the caller with ``capture(param, x)`` (or the forward hooks from
    ``attach_capture_hooks``) before ``step()`` on refresh iterations; ``wants_capture()`` says whether
    the coming step refreshes.
    """

    def __init__(self, params, lr: float = 2.5e-3, weight_decay: float = 0.0, momentum: float = 0.9,
                 blocks: int = 16, block_size: int | None = None, refresh_period: int = 9, orth_iters: int = 1,
                 beta: float = 0.9, tau: float = 0.2, nesterov: bool = False):
        params = list(params)
        super().__init__(params, dict(lr=lr, weight_decay=weight_decay, momentum=momentum))
        for p in params:
            if p.dim() != 2:
                raise ValueError("Dobb handles 2-D weights; use another optimizer for the rest")
        nbs = [block_size or p.shape[1] // blocks for p in params]
        self._params = params
        self._group = DobbGroup([p.data for p in params], nbs, lr=lr, weight_decay=weight_decay,
                                momentum=momentum, tau=tau, nesterov=nesterov)
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
        if self.wants_capture():
            if len(self._captured) == len(self._params):
                xs = [self._captured[id(p)] for p in self._params]
                if len({x.shape[0] for x in xs}) == 1:
                    g.n_tokens = max(g.n_tokens, xs[0].shape[0])
                    need = _abi.dobb_workspace_size(_abi.DOBB_OP_ACCUMULATE,
                                                    [(1, n, nb) for (_, n, nb) in g.shapes], xs[0].shape[0])
                    if need > g.ws.numel():
                        g.ws = torch.empty(need, dtype=torch.uint8, device=g.device)
                    g.accumulate(xs, self.beta if g.refreshes else 0.0)
                else:
                    for x, p, A, (_, n, nb) in zip(xs, self._params, g.A, g.shapes):
                        _abi.dobb_accumulate_moment(x, A, nb, self.beta if g.refreshes else 0.0)
                if g.refreshes == 0:
                    g.refresh(_abi.DOBB_REFRESH_EXACT, 0, warm_start=False)
                else:
                    g.refresh(_abi.DOBB_REFRESH_ORTH_ITER, self.k)
            self._captured.clear()
        grads = [p.grad if p.grad is not None else torch.zeros_like(p) for p in self._params]
        g.step(grads)
        self.t += 1
        return loss
