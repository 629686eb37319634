"""GPU parity at the benchmark matrix shapes, on outputs the oracle can compute one by one.

The step is row-independent, so the oracle runs on sampled rows of a full-size matrix; the
accumulate and refresh are block-independent, so it runs on sampled blocks.  Inputs follow the
workloads: GPT-2 Small (qkv 2304x768, nb = 48), GPT-2 XL (qkv 4800x1600 with nb = 100, fc-proj
1600x6400 with nb = 400, bf16 activations of 16384 tokens) and Llama-7B-style shapes (bf16 weights
and gradients, nb = 128; the stack has no token count, so its captures use 8192 bf16 tokens).
Tolerances as in test_gpu_parity.py; the projection's coefficients are read back through C_out, so
the 1e-5 relative Frobenius bar on C applies to the launch the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from test_gpu_parity import check_w

pytestmark = pytest.mark.gpu
dobb = pytest.importorskip("block_diagonal_eigenbasis_amd")
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def f32(v):
    return float(np.float32(v))


@pytest.mark.parametrize("m,n,nb,dt", [
    (2304, 768, 48, torch.float32), (4800, 1600, 100, torch.float32), (1600, 6400, 400, torch.float32),
    (11008, 4096, 128, torch.bfloat16), (4096, 11008, 128, torch.bfloat16)])
def test_step_fullsize_sampled_rows(m, n, nb, dt):
    print(f"fullsize step {m}x{n} nb={nb} {dt}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(m + n + nb)
    B = n // nb
    Q = torch.linalg.qr(torch.randn(B, nb, nb, device=DEV, generator=g, dtype=torch.float64))[0].float().contiguous()
    W = (0.02 * torch.randn(m, n, device=DEV, generator=g)).to(dt)
    G = torch.randn(m, n, device=DEV, generator=g).to(dt)
    M = torch.randn(m, n, device=DEV, generator=g)
    hp = dict(lr=f32(2.5e-3), weight_decay=f32(0.1), momentum=f32(0.9),
              update_scale=f32(oracle.default_update_scale(m, n)))
    rows = torch.linspace(0, m - 1, 48).long().to(DEV)
    W0, G0, M0 = W[rows].cpu(), G[rows].cpu(), M[rows].cpu()
    U = torch.empty(m, n, device=DEV)
    C = torch.empty(m, n, device=DEV)
    dobb.dobb_step(W, G, M, Q, nb, dobb.make_hparams(**hp), U_out=U, C_out=C)
    Qh = host(Q)
    W_r, M_r, U_r = oracle.step(W0, G0, M0, Qh, nb, hp["lr"], hp["weight_decay"], hp["momentum"], hp["update_scale"])
    Ug, Cg = host(U[rows]), host(C[rows])
    assert np.all(np.abs(host(M[rows]) - M_r) <= 6e-8 * np.abs(M_r) + 1e-30)
    for b in range(B):
        sl = slice(b * nb, (b + 1) * nb)
        C_ref = M_r[:, sl] @ Qh[b]
        assert np.linalg.norm(Cg[:, sl] - C_ref) <= 1e-5 * np.linalg.norm(C_ref), "projection C"
        S = np.rint(Ug[:, sl] @ Qh[b])
        live = np.abs(C_ref) > 1e-5 * np.max(np.abs(C_ref))
        assert np.all(S[live] == np.sign(C_ref[live]))
        R = S @ Qh[b].T
        assert np.linalg.norm(Ug[:, sl] - R) <= 1e-5 * np.linalg.norm(R)
    assert np.mean(np.abs(Ug - U_r) > 1e-3) <= 1e-3
    check_w(host(W[rows]), W0.double().numpy(), Ug, hp, bf16=dt == torch.bfloat16)


@pytest.mark.parametrize("N,n,nb", [(16384, 6400, 400), (16384, 1600, 100), (8192, 3072, 192), (8192, 4096, 128),
                                    (8192, 11008, 128)])
def test_accumulate_and_refresh_fullsize_sampled_blocks(N, n, nb):
    print(f"fullsize accumulate/refresh N={N} n={n} nb={nb}", flush=True)
    X, _ = workload.activations_torch(N, n, 0.15, seed=N + n, device=DEV, dtype=torch.bfloat16)
    B = n // nb
    A = torch.empty(B, nb, nb, device=DEV)
    dobb.dobb_accumulate_moment(X, A, nb)
    blocks = [0, B - 1]
    Ah = host(A)
    for b in blocks:
        ref = oracle.accumulate(X[:, b * nb:(b + 1) * nb].cpu(), nb)[0]
        assert np.max(np.abs(Ah[b] - ref)) <= 4e-7 * np.max(np.abs(ref))
    # exact refresh of the whole set; check the sampled blocks
    Q = torch.empty_like(A)
    lam = torch.empty(B, nb, device=DEV)
    info = torch.empty(B, dtype=torch.int32, device=DEV)
    dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_EXACT, lam=lam, info=info)
    assert np.all(info.cpu().numpy() > 0)
    lam_ref, Q_ref, _ = oracle.eig(Ah[blocks])
    Qh, lh = host(Q), host(lam)
    for i, b in enumerate(blocks):
        nA = np.linalg.norm(Ah[b])
        assert np.max(np.abs(lh[b] - lam_ref[i])) <= 1e-5 * np.max(np.abs(lam_ref[i]))
        assert np.linalg.norm(Ah[b] @ Qh[b] - Qh[b] * lh[b]) <= 1e-5 * nA
        assert np.max(np.abs(Qh[b].T @ Qh[b] - np.eye(nb))) <= 1e-5
    # one warm-started orthogonal-iteration step from that basis on a new capture (EMA 0.9)
    X2, _ = workload.activations_torch(N, n, 0.15, seed=N + n + 1, device=DEV, dtype=torch.bfloat16)
    dobb.dobb_accumulate_moment(X2, A, nb, beta=0.9)
    Qp = host(Q)
    dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_ORTH_ITER, iters=1)
    Ah2 = host(A)
    Q_ref2, _ = oracle.orth_iter(Ah2[blocks], Qp[blocks], k=1)
    Qh2 = host(Q)
    for i, b in enumerate(blocks):
        cond = np.linalg.cond(Ah2[b] @ Qp[b])
        assert np.max(np.abs(Qh2[b].T @ Qh2[b] - np.eye(nb))) <= 1e-5
        assert np.max(np.abs(Qh2[b] - Q_ref2[i])) <= 4 * 6e-8 * cond + 1e-6
