"""Dobb CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain fp64 reference of the Dobb optimizer step ("Dobb: Shard-Local Preconditioning in
Block-Diagonal Eigenbases", arXiv 2610.39412).  The arithmetic lives in ``dobb_oracle.c`` (plain C,
double precision, no BLAS/LAPACK); this module only marshals numpy arrays into it and adds the
pages' two measures (``metrics``).  It is independent of the HIP library: it imports nothing from
the package and the package never imports it.  Only tests/, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may use it.

Every entry point widens its inputs to float64 exactly (fp32 and bf16 values are exactly
representable) and returns float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import metrics  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dobb_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

NORM_SIGN, NORM_IDENTITY, NORM_COL_L2 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile dobb_oracle.c with gcc (IEEE double, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(ctypes.c_double)
        L, D, I = ctypes.c_long, ctypes.c_double, ctypes.c_int
        lib.oracle_accumulate.argtypes = [L, L, L, L, P, D, P]
        lib.oracle_accumulate.restype = None
        lib.oracle_jacobi_eig.argtypes = [L, P, P, P, P, I, D]
        lib.oracle_jacobi_eig.restype = I
        lib.oracle_householder_qr.argtypes = [L, P, P]
        lib.oracle_householder_qr.restype = None
        lib.oracle_orth_iter.argtypes = [L, P, P, I, P, P]
        lib.oracle_orth_iter.restype = None
        lib.oracle_step.argtypes = [L, L, L, P, P, P, P, D, D, D, D, I, I, P]
        lib.oracle_step.restype = None
        lib.oracle_step_g.argtypes = [L, L, L, P, P, P, P, D, D, D, D, I, I, P]
        lib.oracle_step_g.restype = None
        lib.oracle_cholesky_qr2.argtypes = [L, P, P]
        lib.oracle_cholesky_qr2.restype = I
        lib.oracle_orth_iter_cholqr2.argtypes = [L, P, P, I, P, P]
        lib.oracle_orth_iter_cholqr2.restype = I
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """Exact widening of fp32/bf16/fp64 data (numpy array or CPU torch tensor) to C-contiguous fp64."""
    if hasattr(a, "detach"):  # a torch tensor: widen in torch (bf16 is not a numpy dtype)
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _pool(cores: int | None):
    return ThreadPoolExecutor(max_workers=max(1, cores or os.cpu_count() or 1))


def accumulate(X, nb: int, A=None, beta: float = 0.0, cores: int | None = 1) -> np.ndarray:
    """A_b <- beta A_b + (1-beta)/N sum_t x_{t,b} x_{t,b}^T for every block b (X is N x n).

    The blocks are independent; with cores > 1 they are shared among threads (each block's sum is
    the same single loop over the tokens)."""
    X = _f64(X)
    N, n = X.shape
    assert n % nb == 0
    B = n // nb
    A = np.zeros((B, nb, nb)) if A is None else _f64(A).copy()
    lib = _load()
    if not cores or cores == 1:
        lib.oracle_accumulate(N, n, nb, n, _ptr(X), float(beta), _ptr(A))
        return A
    dp = ctypes.POINTER(ctypes.c_double)
    base = X.ctypes.data

    def one(b):
        xb = ctypes.cast(base + 8 * b * nb, dp)      # block b's columns, leading dimension n
        ab = np.ascontiguousarray(A[b])
        lib.oracle_accumulate(N, nb, nb, n, xb, float(beta), _ptr(ab))
        A[b] = ab

    with _pool(cores) as ex:
        list(ex.map(one, range(B)))
    return A


def eig(A, V0=None, max_sweeps: int = 60, tol: float = 1e-14, cores: int | None = None):
    """Exact per-block eigendecomposition by cyclic Jacobi.

    A: (B, nb, nb) symmetric.  V0: optional (B, nb, nb) warm-start basis.
    Returns (lam (B, nb) descending, Q (B, nb, nb) eigenvectors in columns, info (B,) sweeps used
    or -1 if not converged)."""
    A = _f64(A)
    B, nb, _ = A.shape
    V0 = None if V0 is None else _f64(V0)
    lam = np.zeros((B, nb))
    Q = np.zeros((B, nb, nb))
    info = np.zeros(B, dtype=np.int64)
    lib = _load()

    def one(b):
        v0 = _ptr(V0[b]) if V0 is not None else None
        lb, qb = np.zeros(nb), np.zeros((nb, nb))
        info[b] = lib.oracle_jacobi_eig(nb, _ptr(np.ascontiguousarray(A[b])), v0, _ptr(lb), _ptr(qb),
                                        int(max_sweeps), float(tol))
        lam[b], Q[b] = lb, qb

    with _pool(cores) as ex:
        list(ex.map(one, range(B)))
    return lam, Q, info


def householder_qr(Z) -> np.ndarray:
    """Orthonormal factor of a square matrix by Householder QR, with diag(R) > 0."""
    Z = _f64(Z)
    n = Z.shape[0]
    Q = np.zeros((n, n))
    _load().oracle_householder_qr(n, _ptr(Z), _ptr(Q))
    return Q


def cholesky_qr2(Z) -> np.ndarray:
    """Orthonormal factor of a square matrix by Cholesky QR, two passes (diag(R) > 0)."""
    Z = _f64(Z)
    n = Z.shape[0]
    Q = np.zeros((n, n))
    if _load().oracle_cholesky_qr2(n, _ptr(Z), _ptr(Q)) != 0:
        raise np.linalg.LinAlgError("Cholesky QR: a pivot was not positive")
    return Q


def orth_iter(A, Qprev, k: int = 1, cores: int | None = None, qr: str = "householder"):
    """k steps of warm-started orthogonal iteration per block: Q <- qr(A_b Q).Q, with the
    Householder QR (Table 16's principal) or qr="cholesky" (Table 16's Cholesky QR, two passes).

    Returns (Q (B, nb, nb), Rayleigh quotients (B, nb))."""
    if qr not in ("householder", "cholesky"):
        raise ValueError(qr)
    A, Qprev = _f64(A), _f64(Qprev)
    B, nb, _ = A.shape
    Q = np.zeros((B, nb, nb))
    lam = np.zeros((B, nb))
    lib = _load()

    def one(b):
        qb, lb = np.zeros((nb, nb)), np.zeros(nb)
        a, qp = _ptr(np.ascontiguousarray(A[b])), _ptr(np.ascontiguousarray(Qprev[b]))
        if qr == "householder":
            lib.oracle_orth_iter(nb, a, qp, int(k), _ptr(qb), _ptr(lb))
        elif lib.oracle_orth_iter_cholqr2(nb, a, qp, int(k), _ptr(qb), _ptr(lb)) != 0:
            raise np.linalg.LinAlgError(f"Cholesky QR failed in block {b}")
        Q[b], lam[b] = qb, lb

    with _pool(cores) as ex:
        list(ex.map(one, range(B)))
    return Q, lam


def step(W, G, M, Q, nb: int, lr: float, weight_decay: float, momentum: float, update_scale: float,
         nesterov: bool = False, norm: int = NORM_SIGN, cores: int | None = 1):
    """One Dobb step on an m x n weight.  Returns (W_new, M_new, U), all float64 (m, n).

    With the sign and identity norms every row is independent, so with cores > 1 row chunks are
    shared among threads; column-l2 couples the rows and runs whole."""
    W, G, M, Q = _f64(W).copy(), _f64(G), _f64(M).copy(), _f64(Q)
    m, n = W.shape
    assert n % nb == 0 and Q.shape == (n // nb, nb, nb)
    U = np.zeros((m, n))
    lib = _load()
    args = (float(lr), float(weight_decay), float(momentum), float(update_scale), int(bool(nesterov)), int(norm))
    if not cores or cores == 1 or norm == NORM_COL_L2 or m < 2:
        lib.oracle_step(m, n, nb, _ptr(W), _ptr(G), _ptr(M), _ptr(Q), *args, _ptr(U))
        return W, M, U
    nchunk = min(m, 4 * cores)
    bounds = np.linspace(0, m, nchunk + 1).astype(int)

    def one(c):
        r0, r1 = bounds[c], bounds[c + 1]
        if r1 > r0:
            w, mm, u = W[r0:r1], M[r0:r1], U[r0:r1]          # contiguous row slices, written in place
            g = np.ascontiguousarray(G[r0:r1])
            lib.oracle_step(r1 - r0, n, nb, _ptr(w), _ptr(g), _ptr(mm), _ptr(Q), *args, _ptr(u))

    with _pool(cores) as ex:
        list(ex.map(one, range(nchunk)))
    return W, M, U


def step_g(W, G, M, P, nb: int, lr: float, weight_decay: float, momentum: float, update_scale: float,
           nesterov: bool = False, norm: int = NORM_SIGN, cores: int | None = 1):
    """One Dobb-G step on an m x n weight: blocks of nb rows, bases P (m/nb, nb, nb) of the
    output-gradient second moment.  Returns (W_new, M_new, U), all float64 (m, n).

    With the sign and identity norms every column is independent within a block, but a block spans
    all columns, so with cores > 1 whole blocks of rows are shared among threads; Dobb-G-l2 (norm 2)
    normalises within a block too, so blocks stay independent for every norm."""
    W, G, M, P = _f64(W).copy(), _f64(G), _f64(M).copy(), _f64(P)
    m, n = W.shape
    assert m % nb == 0 and P.shape == (m // nb, nb, nb)
    U = np.zeros((m, n))
    lib = _load()
    args = (float(lr), float(weight_decay), float(momentum), float(update_scale), int(bool(nesterov)), int(norm))
    B = m // nb
    if not cores or cores == 1 or B == 1:
        lib.oracle_step_g(m, n, nb, _ptr(W), _ptr(G), _ptr(M), _ptr(P), *args, _ptr(U))
        return W, M, U

    def one(b):
        r = slice(b * nb, (b + 1) * nb)
        w, mm, u = W[r], M[r], U[r]                        # contiguous row blocks, written in place
        g, p = np.ascontiguousarray(G[r]), np.ascontiguousarray(P[b:b + 1])
        lib.oracle_step_g(nb, n, nb, _ptr(w), _ptr(g), _ptr(mm), _ptr(p), *args, _ptr(u))

    with _pool(cores) as ex:
        list(ex.map(one, range(B)))
    return W, M, U


def default_update_scale_g(m: int, n: int, tau: float = 0.2) -> float:
    """Applied scale of the Dobb-G sign update: Table 9's Dobb-G row gives ||O||_F^2 = m and
    RMS tau sqrt(max(m,n)/n), i.e. tau sqrt(max(m,n)/n) on U (whose ||U||_F^2 = m n)."""
    return tau * float(np.sqrt(max(m, n) / n))


def default_update_scale(m: int, n: int, tau: float = 0.2) -> float:
    """Applied scale of the sign update: s = tau sqrt(max(m,n)) on the raw update O = U/sqrt(m),
    whose ||O||_F^2 = n (Table 9, Dobb row), i.e. tau sqrt(max(m,n)/m) on U."""
    return tau * float(np.sqrt(max(m, n) / m))


def refresh(A, Q, mode: str, iters: int, warm_start: bool, cores: int | None = None):
    """The refresh call's semantics: 'exact' -> Jacobi (cold from I, or warm from Q);
    'orth_iter' -> k = iters steps of orthogonal iteration from Q.  Returns (Q_new, lam, info)."""
    if mode == "exact":
        lam, Qn, info = eig(A, V0=Q if warm_start else None, cores=cores)
        return Qn, lam, info
    Qn, lam = orth_iter(A, Q, k=iters, cores=cores)
    return Qn, lam, np.full(A.shape[0], iters, dtype=np.int64)
