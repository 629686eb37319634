"""GPU parity of the orthogonal-iteration refresh with the Cholesky QR routine (Table 16 of the Dobb
listing: "Cholesky" next to the principal Householder) against the oracle's Cholesky QR (two
passes), which is pinned to the unique QR factor with diag(R) > 0 on the CPU (MI355X only).

Bars: orthonormality max|Q^T Q - I| <= 1e-5; each entry of Q within 4 u cond(Z) + 1e-6 of the
oracle's (Z = A_b Q_prev formed in fp32, as for the Householder routine); info = k; Rayleigh
quotients to 1e-5 max|lambda|.  Inputs: random orthonormal bases (the refresh from an unrelated
basis) and warm bases (the exact eigenbasis of a nearby moment, the refresh's steady state).
"""
import numpy as np
import pytest
import torch

import oracle
import workload

pytestmark = pytest.mark.gpu
dobb = pytest.importorskip("block_diagonal_eigenbasis_amd")
DEV = "cuda"
RNG = np.random.default_rng


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def t32(x):
    return torch.as_tensor(np.ascontiguousarray(x), dtype=torch.float32, device=DEV)


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("n,nb,k,start", [(768, 192, 1, "random"), (200, 100, 2, "random"), (75, 25, 1, "random"),
                                          (400, 400, 1, "random"), (260, 130, 1, "random"), (384, 128, 1, "random"),
                                          (10, 5, 3, "random"), (800, 400, 1, "warm"), (1600, 100, 1, "warm"),
                                          (768, 768, 1, "warm"), (96, 48, 2, "warm")])
def test_refresh_cholqr_matches_oracle(n, nb, k, start):
    print(f"refresh cholqr n={n} nb={nb} k={k} {start}", flush=True)
    rng = RNG(17 * n + nb + k)
    A32 = np.float64(np.float32(oracle.accumulate(workload.activations(4096, n, 0.15, rng), nb, cores=8)))
    B = n // nb
    if start == "random":
        Qp = np.stack([workload.haar(nb, rng) for _ in range(B)])
    else:   # the eigenbasis of a nearby moment (another capture of the same spectrum)
        A2 = oracle.accumulate(workload.activations(4096, n, 0.15, RNG(5)), nb, cores=8)
        Qp = np.stack([np.linalg.eigh(a)[1][:, ::-1] for a in 0.9 * A32 + 0.1 * A2])
    Qp = np.float64(np.float32(Qp))
    A, Q = t32(A32), t32(Qp)
    lam = torch.empty(B, nb, device=DEV)
    info = torch.empty(B, dtype=torch.int32, device=DEV)
    dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_ORTH_ITER_CHOLQR, iters=k, lam=lam, info=info)
    Q_ref, lam_ref = oracle.orth_iter(A32, Qp, k=k, qr="cholesky", cores=8)
    got = host(Q)
    assert np.all(info.cpu().numpy() == k)
    worst = 0.0
    for b in range(B):
        assert np.max(np.abs(got[b].T @ got[b] - np.eye(nb))) <= 1e-5
        Z = A32[b] @ Qp[b]
        for _ in range(k - 1):
            Z = A32[b] @ np.linalg.qr(Z)[0]
        cond = np.linalg.cond(Z)
        err = np.max(np.abs(got[b] - Q_ref[b]))
        worst = max(worst, err / (4 * 6e-8 * cond + 1e-6))
        assert err <= 4 * 6e-8 * cond + 1e-6, f"block {b}: {err:.2e} (cond {cond:.1e})"
        np.testing.assert_allclose(host(lam)[b], lam_ref[b], rtol=0, atol=1e-5 * np.max(np.abs(lam_ref[b])))
    print(f"  worst error / bound {worst:.3f}", flush=True)


def test_refresh_cholqr_bf16_basis_and_householder_agree():
    """With a bf16 basis (Table 18's principal storage) the Cholesky routine reads and rounds the basis
    like the Householder one; the two routines give the same basis to the fp32 bound before
    rounding, so at most one bf16 ulp apart."""
    rng = RNG(23)
    n, nb = 800, 400
    A = t32(oracle.accumulate(workload.activations(4096, n, 0.15, rng), nb, cores=8))
    Q0 = torch.empty(n // nb, nb, nb, device=DEV)
    dobb.dobb_refresh_basis(A, Q0, dobb.DOBB_REFRESH_EXACT)
    Qh, Qc = Q0.to(torch.bfloat16), Q0.to(torch.bfloat16)
    dobb.dobb_refresh_basis(A, Qh, dobb.DOBB_REFRESH_ORTH_ITER, iters=1)
    dobb.dobb_refresh_basis(A, Qc, dobb.DOBB_REFRESH_ORTH_ITER_CHOLQR, iters=1)
    a, c = host(Qh), host(Qc)
    assert np.all(np.abs(a - c) <= 2.0 ** -7 * np.abs(a) + 1e-6)


def test_refresh_cholqr_reports_a_rank_deficient_block():
    """A zero moment makes Z = 0: the Gram matrix has no positive pivot, and info says so (-1)."""
    nb = 64
    A = torch.zeros(2, nb, nb, device=DEV)
    A[1] = torch.eye(nb, device=DEV)
    Q = torch.eye(nb, device=DEV).expand(2, nb, nb).contiguous()
    info = torch.empty(2, dtype=torch.int32, device=DEV)
    dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_ORTH_ITER_CHOLQR, iters=1, info=info)
    assert info.cpu().tolist() == [-1, 1]
    np.testing.assert_allclose(host(Q)[1], np.eye(nb), atol=1e-6)
