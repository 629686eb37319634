"""GPU parity on the Table 1(b) style gradients, and the pages' orthogonality measure of the updates.

Setting (Table 1 caption of the Dobb listing): a 768 x 768 weight whose gradient is D X^T / N, where the
output-gradient second moment has entropy effective rank 80, 50, 20 or 5 % and the activation second
moment is fixed at 15 %.  Here D and X are N x 768 token-major (N = 4096), so the gradient is D^T X / N
in torch layout.  The basis is the exact eigenbasis of the blocks of the activation second moment for
B = 1, 4 and 16 blocks (nb = 768, 192, 48): one accumulate (fp32 activations), one exact refresh and
one step with mu = 0 (so the projected momentum is the gradient).  The pages' own Table 1(b) values
are missing from the listing, so the orthogonality figures are compared GPU against oracle only.

Bars: the end-to-end bar (<= 0.1 % of U's entries differ by more than 1e-3 RMS(U)) for sign and
1e-5 relative Frobenius for column-l2, against the oracle fed A correctly rounded to fp32 (the
precision in which the library stores A; its capture of fp32 activations sums exact products in
fp64, so its A is that same rounding but for near ties), and the orthogonality of the GPU's update
within 1e-3 of the oracle's.  At B = 1 the 768 eigenvalues of this spectrum include pairs
1.6e-7 max(lambda) apart, and the fp32 rounding of A moves those eigenvectors by itself: the oracle's
update from its A rounded to fp32 differs from its update from the fp64 A in 0.13-0.64 % of the
entries.  That floor is printed for every case; it is a property of fp32 storage, not of the kernels.

The oracle's Jacobi eigensolver at nb = 768 is warm-started from LAPACK's eigenvectors (a library
routine used as the starting basis only, to keep the case within seconds): the oracle checks that
basis against its own convergence test (off-diagonal of V^T A V below 1e-14 ||A||_F) and sweeps
until it passes (usually none are needed), then sorts and sign-normalises it.  A warm start reaches
the same eigenbasis as a cold one (pinned on the CPU).
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from oracle import metrics

pytestmark = pytest.mark.gpu
dobb = pytest.importorskip("block_diagonal_eigenbasis_amd")
DEV = "cuda"
N, DIM = 4096, 768
RANKS = [0.80, 0.50, 0.20, 0.05]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


_cache = {}


def _activations():
    if "X" not in _cache:
        rng = np.random.default_rng(2000)
        _cache["X"] = np.float32(workload.activations(N, DIM, 0.15, rng))
    return _cache["X"]


def _gradient(rank):
    key = ("G", rank)
    if key not in _cache:
        rng = np.random.default_rng(2000 + int(round(rank * 100)))
        D = workload.activations(N, DIM, rank, rng)
        _cache[key] = np.float32(D.T @ np.float64(_activations()) / N)
    return _cache[key]


def _oracle_basis(nb, fp32_A=False):
    """The oracle's eigenbasis of its own A blocks, or of those blocks correctly rounded to fp32."""
    key = ("Q", nb, fp32_A)
    if key not in _cache:
        A = oracle.accumulate(_activations(), nb)
        if fp32_A:
            A = np.float64(np.float32(A))
        V0 = np.stack([np.linalg.eigh(a)[1] for a in A]) if nb > 256 else None
        lam, Q, info = oracle.eig(A, V0=V0)
        assert np.all(info >= 0)
        _cache[key] = Q
    return _cache[key]


@pytest.mark.parametrize("B", [1, 4, 16])
@pytest.mark.parametrize("rank", RANKS)
def test_table1b_gradients(rank, B):
    nb = DIM // B
    print(f"table1b rank={rank} B={B}", flush=True)
    X = torch.from_numpy(_activations()).to(DEV)
    Gh = _gradient(rank)
    G = torch.from_numpy(Gh).to(DEV)
    A = torch.empty(B, nb, nb, device=DEV)
    dobb.dobb_accumulate_moment(X, A, nb)
    Q = torch.empty_like(A)
    info = torch.empty(B, dtype=torch.int32, device=DEV)
    dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_EXACT, info=info)
    assert bool((info > 0).all()), "eigensolver did not converge"
    Q_ref, Q_ref32 = _oracle_basis(nb), _oracle_basis(nb, fp32_A=True)
    zeros = np.zeros((DIM, DIM))
    out = {}
    for name, norm, onorm in [("sign", dobb.DOBB_NORM_SIGN, oracle.NORM_SIGN),
                              ("col_l2", dobb.DOBB_NORM_COL_L2, oracle.NORM_COL_L2)]:
        W = torch.zeros(DIM, DIM, device=DEV)
        M = torch.zeros(DIM, DIM, device=DEV)
        U = torch.empty(DIM, DIM, device=DEV)
        dobb.dobb_step(W, G, M, Q, nb, dobb.make_hparams(0.0, 0.0, 0.0, 1.0, norm=norm), U_out=U)
        _, _, U_ref = oracle.step(zeros, Gh, zeros, Q_ref, nb, 0.0, 0.0, 0.0, 1.0, norm=onorm)
        _, _, U_ref32 = oracle.step(zeros, Gh, zeros, Q_ref32, nb, 0.0, 0.0, 0.0, 1.0, norm=onorm)
        Ug = host(U)
        if name == "sign":
            rms = np.sqrt(np.mean(U_ref32 ** 2))
            floor = np.mean(np.abs(U_ref32 - U_ref) > 1e-3 * rms)
            frac64 = np.mean(np.abs(Ug - U_ref) > 1e-3 * rms)
            frac = np.mean(np.abs(Ug - U_ref32) > 1e-3 * rms)
            print(f"  sign: {frac:.2e} of U's entries differ from the oracle on fp32 A "
                  f"({frac64:.2e} from the oracle on fp64 A; fp32-storage floor {floor:.2e})", flush=True)
            assert frac <= 1e-3, f"{frac:.2e} of U's entries differ"
        else:
            floor = np.linalg.norm(U_ref32 - U_ref) / np.linalg.norm(U_ref)
            err64 = np.linalg.norm(Ug - U_ref) / np.linalg.norm(U_ref)
            err = np.linalg.norm(Ug - U_ref32) / np.linalg.norm(U_ref32)
            print(f"  column-l2: relative error {err:.2e} against the oracle on fp32 A "
                  f"({err64:.2e} on fp64 A; fp32-storage floor {floor:.2e})", flush=True)
            assert err <= 1e-5
        o_gpu, o_ref = metrics.orthogonality(Ug), metrics.orthogonality(U_ref32)
        assert abs(o_gpu - o_ref) <= 1e-3
        out[name] = (o_gpu, o_ref)
    print(f"  rank {rank:.0%} B={B}: orthogonality of G {metrics.orthogonality(Gh):.3f}; "
          f"sign {out['sign'][0]:.4f} (oracle {out['sign'][1]:.4f}); "
          f"column-l2 {out['col_l2'][0]:.4f} (oracle {out['col_l2'][1]:.4f})", flush=True)
