"""ctypes binding of libdobb.so (include/dobb.h), with the C names.

Argument marshalling only: every computation runs in the HIP kernels of libdobb.so.  Tensors must be
torch tensors on a ROCm device; the binding checks the dtype, device, shape and contiguity of every
tensor (the grouped forms take one dtype per argument, so every tensor of a list must share it),
allocates the workspace as a torch uint8 tensor (the caching allocator returns 256-byte aligned
blocks) and passes torch's current stream.  There is no fallback: if the library is missing, loading
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdobb.so")

DOBB_OK, DOBB_ERR_INVALID_ARG, DOBB_ERR_SHAPE, DOBB_ERR_DTYPE = 0, -1, -2, -3
DOBB_ERR_WORKSPACE, DOBB_ERR_HIP, DOBB_ERR_NOT_CONVERGED = -4, -5, -6
DOBB_F32, DOBB_BF16 = 0, 1
DOBB_REFRESH_EXACT, DOBB_REFRESH_ORTH_ITER, DOBB_REFRESH_ORTH_ITER_CHOLQR = 0, 1, 2
DOBB_NORM_SIGN, DOBB_NORM_IDENTITY, DOBB_NORM_COL_L2 = 0, 1, 2
DOBB_OP_ACCUMULATE, DOBB_OP_REFRESH, DOBB_OP_STEP, DOBB_OP_STEP_G = 0, 1, 2, 3
DOBB_WS_BF16_BASIS = 16
DOBB_NOALLOC_SCRATCH_BYTES = 64 << 20


class DobbError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("nb", ctypes.c_int64)]


class HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("weight_decay", ctypes.c_float), ("momentum", ctypes.c_float),
                ("update_scale", ctypes.c_float), ("nesterov", ctypes.c_int32), ("norm", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdobb.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the Dobb step has no CPU fallback)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        PS = ctypes.POINTER(Shape)
        PP = ctypes.POINTER(ctypes.c_void_p)
        L.dobb_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, PS, i64, i32]
        L.dobb_workspace_size.restype = sz
        L.dobb_accumulate_moment.argtypes = [PS, vp, ctypes.c_int, i64, i64, f32, vp, vp, sz, vp]
        L.dobb_refresh_basis.argtypes = [PS, vp, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, f32,
                                         vp, vp, sz, vp]
        L.dobb_step.argtypes = [PS, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.POINTER(HParams),
                                vp, vp, vp, sz, vp]
        L.dobb_accumulate_moment_grouped.argtypes = [ctypes.c_int, PS, PP, ctypes.c_int, i64,
                                                     ctypes.POINTER(ctypes.c_int64), f32, PP, vp, sz, vp]
        L.dobb_refresh_basis_grouped.argtypes = [ctypes.c_int, PS, PP, PP, ctypes.c_int, PP, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, f32, PP, vp, sz, vp]
        L.dobb_step_grouped.argtypes = [ctypes.c_int, PS, PP, ctypes.c_int, PP, ctypes.c_int, PP, PP, ctypes.c_int,
                                        ctypes.POINTER(HParams), PP, PP, vp, sz, vp]
        L.dobb_step_g.argtypes = list(L.dobb_step.argtypes)
        L.dobb_step_g_grouped.argtypes = list(L.dobb_step_grouped.argtypes)
        L.dobb_step_noalloc.argtypes = [PS, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                        ctypes.POINTER(HParams), vp, vp, vp]
        for name in ("dobb_accumulate_moment", "dobb_refresh_basis", "dobb_step", "dobb_accumulate_moment_grouped",
                     "dobb_refresh_basis_grouped", "dobb_step_grouped", "dobb_step_noalloc", "dobb_step_g",
                     "dobb_step_g_grouped"):
            getattr(L, name).restype = ctypes.c_int
        L.dobb_status_string.argtypes = [ctypes.c_int]
        L.dobb_status_string.restype = ctypes.c_char_p
        L.dobb_abi_version.restype = ctypes.c_int
        L.dobb_profile_enable.argtypes = [ctypes.c_int]
        L.dobb_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        L.dobb_profile_read.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().dobb_status_string(int(status)).decode()


def dobb_abi_version() -> int:
    return int(lib().dobb_abi_version())


def _check(status: int, what: str) -> None:
    if status != DOBB_OK:
        raise DobbError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DOBB_F32
    if t.dtype == torch.bfloat16:
        return DOBB_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _common_dtype(ts, name: str) -> int:
    """The dtype code shared by every tensor of a grouped argument; a mixed list is rejected (the C
    ABI takes one dtype per argument, and a wrong element size would read or write past a buffer)."""
    dts = {t.dtype for t in ts}
    if len(dts) != 1:
        raise TypeError(f"{name}: every tensor of a grouped call needs the same dtype, got {sorted(map(str, dts))}")
    return _dtype_code(ts[0])


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes: int, device, ws: torch.Tensor | None):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    return ws, ws.numel()


def dobb_workspace_size(op: int, shapes, N: int = 0, variant: int = 0) -> int:
    arr = (Shape * len(shapes))(*[Shape(*s) for s in shapes])
    return int(lib().dobb_workspace_size(int(op), len(shapes), arr, int(N), int(variant)))


# ------------------------------------------------------------------------------------------------
def dobb_accumulate_moment(X: torch.Tensor, A: torch.Tensor, nb: int, beta: float = 0.0,
                           ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """A (B x nb x nb fp32) <- beta A + (1 - beta) / N X_b^T X_b for every block; X is N x n."""
    N, n = X.shape
    shape = Shape(1, n, nb)
    xp = _dev(X, "X")
    ap = _dev(A, "A", torch.float32, (n // nb if nb else 0, nb, nb))
    need = dobb_workspace_size(DOBB_OP_ACCUMULATE, [(1, n, nb)], N)
    ws, wsb = _workspace(need, X.device, ws)
    _check(lib().dobb_accumulate_moment(ctypes.byref(shape), xp, _dtype_code(X), N, n, float(beta), ap,
                                        None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
           "dobb_accumulate_moment")
    return A


def dobb_refresh_basis(A: torch.Tensor, Q: torch.Tensor, mode: int = DOBB_REFRESH_EXACT, iters: int = 0,
                       warm_start: bool = False, tol: float = 0.0, lam: torch.Tensor | None = None,
                       info: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """Refresh Q (B x nb x nb, fp32 or bf16 storage, in/out) from A; see include/dobb.h."""
    B, nb, _ = A.shape
    shape = Shape(1, B * nb, nb)
    ap = _dev(A, "A", torch.float32)
    qp = _dev(Q, "Q", None, A.shape)
    qdt = _dtype_code(Q)
    lp = _dev(lam, "lambda", torch.float32, (B, nb)) if lam is not None else None
    ip = _dev(info, "info", torch.int32, (B,)) if info is not None else None
    need = dobb_workspace_size(DOBB_OP_REFRESH, [(1, B * nb, nb)], 0, DOBB_WS_BF16_BASIS if qdt == DOBB_BF16 else 0)
    ws, wsb = _workspace(need, A.device, ws)
    _check(lib().dobb_refresh_basis(ctypes.byref(shape), ap, qp, qdt, lp, int(mode), int(iters), int(bool(warm_start)),
                                    float(tol), ip, None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
           "dobb_refresh_basis")
    return Q


def make_hparams(lr: float, weight_decay: float, momentum: float, update_scale: float,
                 nesterov: bool = False, norm: int = DOBB_NORM_SIGN) -> HParams:
    return HParams(float(lr), float(weight_decay), float(momentum), float(update_scale), int(bool(nesterov)),
                   int(norm))


def _step_variant(norm: int, q_dtype: int) -> int:
    return int(norm) | (DOBB_WS_BF16_BASIS if q_dtype == DOBB_BF16 else 0)


def dobb_step(W: torch.Tensor, G: torch.Tensor, M: torch.Tensor, Q: torch.Tensor, nb: int, hp: HParams,
              U_out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None,
              C_out: torch.Tensor | None = None):
    """One Dobb step on W (m x n, fp32/bf16) in place; M (fp32) in place; Q fp32 or bf16; U_out and
    C_out optional (fp32 m x n: the update before scaling, and the coefficients C_b = P_b Q_b)."""
    m, n = W.shape
    shape = Shape(m, n, nb)
    wp = _dev(W, "W")
    gp = _dev(G, "G", None, (m, n))
    mp = _dev(M, "M", torch.float32, (m, n))
    qp = _dev(Q, "Q", None, (n // nb, nb, nb))
    qdt = _dtype_code(Q)
    up = _dev(U_out, "U_out", torch.float32, (m, n)) if U_out is not None else None
    cp = _dev(C_out, "C_out", torch.float32, (m, n)) if C_out is not None else None
    need = dobb_workspace_size(DOBB_OP_STEP, [(m, n, nb)], 0, _step_variant(hp.norm, qdt))
    ws, wsb = _workspace(need, W.device, ws)
    _check(lib().dobb_step(ctypes.byref(shape), wp, _dtype_code(W), gp, _dtype_code(G), mp, qp, qdt, ctypes.byref(hp),
                           up, cp, None if ws is None else ws.data_ptr(), wsb, _stream(stream)), "dobb_step")
    return W


def dobb_step_g(W: torch.Tensor, G: torch.Tensor, M: torch.Tensor, P: torch.Tensor, nb: int, hp: HParams,
                U_out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None,
                C_out: torch.Tensor | None = None):
    """One Dobb-G step on W (m x n) in place: blocks of nb rows, P (m/nb x nb x nb, fp32 or bf16) the
    bases of the output-gradient second moment; M (fp32) in place; U_out, C_out optional (fp32)."""
    m, n = W.shape
    shape = Shape(m, n, nb)
    wp = _dev(W, "W")
    gp = _dev(G, "G", None, (m, n))
    mp = _dev(M, "M", torch.float32, (m, n))
    pp = _dev(P, "P", None, (m // nb, nb, nb))
    pdt = _dtype_code(P)
    up = _dev(U_out, "U_out", torch.float32, (m, n)) if U_out is not None else None
    cp = _dev(C_out, "C_out", torch.float32, (m, n)) if C_out is not None else None
    need = dobb_workspace_size(DOBB_OP_STEP_G, [(m, n, nb)], 0, _step_variant(hp.norm, pdt))
    ws, wsb = _workspace(need, W.device, ws)
    _check(lib().dobb_step_g(ctypes.byref(shape), wp, _dtype_code(W), gp, _dtype_code(G), mp, pp, pdt,
                             ctypes.byref(hp), up, cp, None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
           "dobb_step_g")
    return W


def dobb_step_noalloc(W: torch.Tensor, G: torch.Tensor, M: torch.Tensor, Q: torch.Tensor, nb: int, hp: HParams,
                      U_out: torch.Tensor | None = None, C_out: torch.Tensor | None = None, stream=None):
    """dobb_step with the library's static per-GPU scratch instead of a workspace: allocates nothing
    (for callers that cannot, e.g. under graph capture).  Shapes whose workspace exceeds
    DOBB_NOALLOC_SCRATCH_BYTES are refused (DOBB_ERR_WORKSPACE)."""
    m, n = W.shape
    shape = Shape(m, n, nb)
    wp = _dev(W, "W")
    gp = _dev(G, "G", None, (m, n))
    mp = _dev(M, "M", torch.float32, (m, n))
    qp = _dev(Q, "Q", None, (n // nb, nb, nb))
    up = _dev(U_out, "U_out", torch.float32, (m, n)) if U_out is not None else None
    cp = _dev(C_out, "C_out", torch.float32, (m, n)) if C_out is not None else None
    _check(lib().dobb_step_noalloc(ctypes.byref(shape), wp, _dtype_code(W), gp, _dtype_code(G), mp, qp, _dtype_code(Q),
                                   ctypes.byref(hp), up, cp, _stream(stream)), "dobb_step_noalloc")
    return W


# ------------------------------------------------------------------------------------------------
def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[None if t is None else t.data_ptr() for t in ts])


def dobb_accumulate_moment_grouped(Xs, As, nbs, beta: float = 0.0, ws: torch.Tensor | None = None, stream=None):
    count = len(Xs)
    shapes = [(1, X.shape[1], nb) for X, nb in zip(Xs, nbs)]
    N = Xs[0].shape[0]
    for X, A, (_, n, nb) in zip(Xs, As, shapes):
        if X.shape[0] != N:
            raise ValueError("all X of a group need the same token count")
        _dev(X, "X")
        _dev(A, "A", torch.float32, (n // nb, nb, nb))
    dt = _common_dtype(Xs, "X")
    sarr = (Shape * count)(*[Shape(*s) for s in shapes])
    ldx = (ctypes.c_int64 * count)(*[X.shape[1] for X in Xs])
    need = dobb_workspace_size(DOBB_OP_ACCUMULATE, shapes, N)
    ws, wsb = _workspace(need, Xs[0].device, ws)
    _check(lib().dobb_accumulate_moment_grouped(count, sarr, _ptrs(Xs), dt, N, ldx, float(beta), _ptrs(As),
                                                None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
           "dobb_accumulate_moment_grouped")


def dobb_refresh_basis_grouped(As, Qs, mode: int, iters: int, warm_start: bool = False, tol: float = 0.0,
                               lams=None, infos=None, ws: torch.Tensor | None = None, stream=None):
    count = len(As)
    shapes = [(1, A.shape[0] * A.shape[1], A.shape[1]) for A in As]
    for A, Q in zip(As, Qs):
        _dev(A, "A", torch.float32)
        _dev(Q, "Q", None, A.shape)
    qdt = _common_dtype(Qs, "Q")
    sarr = (Shape * count)(*[Shape(*s) for s in shapes])
    need = dobb_workspace_size(DOBB_OP_REFRESH, shapes, 0, DOBB_WS_BF16_BASIS if qdt == DOBB_BF16 else 0)
    ws, wsb = _workspace(need, As[0].device, ws)
    _check(lib().dobb_refresh_basis_grouped(count, sarr, _ptrs(As), _ptrs(Qs), qdt,
                                            _ptrs(lams) if lams is not None else None, int(mode), int(iters),
                                            int(bool(warm_start)), float(tol),
                                            _ptrs(infos) if infos is not None else None,
                                            None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
           "dobb_refresh_basis_grouped")


def dobb_step_grouped(Ws, Gs, Ms, Qs, nbs, hps, U_outs=None, ws: torch.Tensor | None = None, stream=None,
                      C_outs=None):
    count = len(Ws)
    shapes = [(W.shape[0], W.shape[1], nb) for W, nb in zip(Ws, nbs)]
    for W, G, M, Q, (m, n, nb) in zip(Ws, Gs, Ms, Qs, shapes):
        _dev(W, "W"); _dev(G, "G", None, (m, n)); _dev(M, "M", torch.float32, (m, n))
        _dev(Q, "Q", None, (n // nb, nb, nb))
    wdt, gdt, qdt = _common_dtype(Ws, "W"), _common_dtype(Gs, "G"), _common_dtype(Qs, "Q")
    for name, outs in (("U_out", U_outs), ("C_out", C_outs)):
        for o, (m, n, _) in zip(outs or [], shapes):
            if o is not None:
                _dev(o, name, torch.float32, (m, n))
    sarr = (Shape * count)(*[Shape(*s) for s in shapes])
    harr = (HParams * count)(*hps)
    need = dobb_workspace_size(DOBB_OP_STEP, shapes, 0, _step_variant(hps[0].norm, qdt))
    ws, wsb = _workspace(need, Ws[0].device, ws)
    _check(lib().dobb_step_grouped(count, sarr, _ptrs(Ws), wdt, _ptrs(Gs), gdt, _ptrs(Ms), _ptrs(Qs), qdt, harr,
                                   _ptrs(U_outs) if U_outs is not None else None,
                                   _ptrs(C_outs) if C_outs is not None else None,
                                   None if ws is None else ws.data_ptr(), wsb, _stream(stream)), "dobb_step_grouped")


def dobb_step_g_grouped(Ws, Gs, Ms, Ps, nbs, hps, U_outs=None, ws: torch.Tensor | None = None, stream=None,
                        C_outs=None):
    count = len(Ws)
    shapes = [(W.shape[0], W.shape[1], nb) for W, nb in zip(Ws, nbs)]
    for W, G, M, P, (m, n, nb) in zip(Ws, Gs, Ms, Ps, shapes):
        _dev(W, "W"); _dev(G, "G", None, (m, n)); _dev(M, "M", torch.float32, (m, n))
        _dev(P, "P", None, (m // nb, nb, nb))
    wdt, gdt, pdt = _common_dtype(Ws, "W"), _common_dtype(Gs, "G"), _common_dtype(Ps, "P")
    for name, outs in (("U_out", U_outs), ("C_out", C_outs)):
        for o, (m, n, _) in zip(outs or [], shapes):
            if o is not None:
                _dev(o, name, torch.float32, (m, n))
    sarr = (Shape * count)(*[Shape(*s) for s in shapes])
    harr = (HParams * count)(*hps)
    need = dobb_workspace_size(DOBB_OP_STEP_G, shapes, 0, _step_variant(hps[0].norm, pdt))
    ws, wsb = _workspace(need, Ws[0].device, ws)
    _check(lib().dobb_step_g_grouped(count, sarr, _ptrs(Ws), wdt, _ptrs(Gs), gdt, _ptrs(Ms), _ptrs(Ps), pdt, harr,
                                     _ptrs(U_outs) if U_outs is not None else None,
                                     _ptrs(C_outs) if C_outs is not None else None,
                                     None if ws is None else ws.data_ptr(), wsb, _stream(stream)), "dobb_step_g_grouped")


# ------------------------------------------------------------------------------------------------
def dobb_profile_enable(on: bool) -> None:
    lib().dobb_profile_enable(int(bool(on)))


def dobb_profile_reset() -> None:
    lib().dobb_profile_reset()


def dobb_profile_read() -> dict:
    """{kernel name: (launches, total ms)} of the kernels timed while profiling was enabled."""
    cap = 64
    names = (ctypes.c_char_p * cap)()
    launches = (ctypes.c_int64 * cap)()
    ms = (ctypes.c_double * cap)()
    n = lib().dobb_profile_read(names, launches, ms, cap)
    return {names[i].decode(): (int(launches[i]), float(ms[i])) for i in range(min(n, cap))}
