"""GPU edge cases of the Dobb step against the oracle: one-column blocks, single rows, tiny token
counts, the widest blocks of orthogonal iteration and a zero second moment.

* nb = 1: every block basis is [+-1], so the step is sign descent, U = sign(mu M + G) exactly
  (the oracle pins the same reduction on the CPU).
* m = 1: a single row through the narrow and the wide step kernels.
* N = 1 and N = 7 tokens: captures shorter than one staged token chunk.
* nb = 768: orthogonal iteration on blocks wider than the panel kernels' 512 rows.
* A = 0: the exact refresh returns the identity with zero eigenvalues, orthogonal iteration maps
  any basis to the identity (no reflector for a zero column), and the step is then sign descent.
Tolerances as in test_gpu_parity.py.
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


def f32(v):
    return float(np.float32(v))


def _hp(m, n):
    return dict(lr=f32(2.5e-3), weight_decay=f32(0.1), momentum=f32(0.9),
                update_scale=f32(oracle.default_update_scale(m, n)))


def test_step_nb1_is_sign_descent():
    m, n = 37, 64
    rng = RNG(81)
    W, G, M = (t32(0.02 * rng.standard_normal((m, n))), t32(rng.standard_normal((m, n))),
               t32(rng.standard_normal((m, n))))
    Q = t32(rng.choice([-1.0, 1.0], size=(n, 1, 1)))
    hp = _hp(m, n)
    W1, M1, U = W.clone(), M.clone(), torch.empty(m, n, device=DEV)
    dobb.dobb_step(W1, G, M1, Q, 1, dobb.make_hparams(**hp), U_out=U)
    P = host(M1)
    np.testing.assert_array_equal(host(U), np.sign(P))
    W_r, M_r, U_r = oracle.step(W.cpu(), G.cpu(), M.cpu(), host(Q), 1, hp["lr"], hp["weight_decay"], hp["momentum"],
                                hp["update_scale"])
    np.testing.assert_array_equal(host(U), U_r)
    check_w(host(W1), host(W), host(U), hp)


@pytest.mark.parametrize("n,nb", [(800, 100), (800, 400), (96, 48)])
def test_step_single_row(n, nb):
    m = 1
    rng = RNG(83 + nb)
    Q64 = np.stack([workload.haar(nb, rng) for _ in range(n // nb)])
    Q = t32(Q64)
    Qh = host(Q)
    W, G, M = (t32(0.02 * rng.standard_normal((m, n))), t32(rng.standard_normal((m, n))),
               t32(rng.standard_normal((m, n))))
    hp = _hp(m, n)
    W1, M1, U = W.clone(), M.clone(), torch.empty(m, n, device=DEV)
    dobb.dobb_step(W1, G, M1, Q, nb, dobb.make_hparams(**hp), U_out=U)
    W_r, M_r, U_r = oracle.step(W.cpu(), G.cpu(), M.cpu(), Qh, nb, hp["lr"], hp["weight_decay"], hp["momentum"],
                                hp["update_scale"])
    Ug = host(U)
    for b in range(n // nb):
        sl = slice(b * nb, (b + 1) * nb)
        C_ref = M_r[:, sl] @ Qh[b]
        S = np.rint(Ug[:, sl] @ Qh[b])
        live = np.abs(C_ref) > 1e-5 * np.max(np.abs(C_ref))
        assert np.all(S[live] == np.sign(C_ref[live]))
        R = S @ Qh[b].T
        assert np.linalg.norm(Ug[:, sl] - R) <= 1e-5 * np.linalg.norm(R)
    check_w(host(W1), host(W), Ug, hp)


@pytest.mark.parametrize("N,n,nb,dtype", [(1, 400, 100, torch.bfloat16), (7, 800, 400, torch.bfloat16),
                                          (1, 96, 48, torch.float32), (7, 192, 192, torch.float32)])
def test_accumulate_tiny_token_counts(N, n, nb, dtype):
    rng = RNG(N + n)
    X = torch.as_tensor(workload.activations(N, n, 0.15, rng), dtype=torch.float32).to(dtype).to(DEV)
    A = torch.empty(n // nb, nb, nb, device=DEV)
    dobb.dobb_accumulate_moment(X, A, nb)
    A_ref = oracle.accumulate(X.cpu(), nb)
    got = host(A)
    for b in range(n // nb):
        assert np.max(np.abs(got[b] - A_ref[b])) <= 4e-7 * np.max(np.abs(A_ref[b]))
    np.testing.assert_array_equal(got, np.transpose(got, (0, 2, 1)))


def test_refresh_orth_iter_beyond_panel_rows():
    """nb = 768: wider than the 512 rows the panel kernels hold, so the general panel path runs."""
    n = nb = 768
    rng = RNG(87)
    X = workload.activations(2048, n, 0.15, rng)
    A32 = np.float64(np.float32(oracle.accumulate(X, nb)))
    Qp = np.float32(workload.haar(nb, rng))[None]
    A, Q = t32(A32), t32(Qp)
    info = torch.empty(1, dtype=torch.int32, device=DEV)
    dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_ORTH_ITER, iters=1, info=info)
    Q_ref, _ = oracle.orth_iter(A32, Qp.astype(np.float64), k=1)
    got = host(Q)[0]
    assert int(info.cpu()[0]) == 1
    assert np.max(np.abs(got.T @ got - np.eye(nb))) <= 1e-5
    cond = np.linalg.cond(A32[0] @ Qp[0].astype(np.float64))
    assert np.max(np.abs(got - Q_ref[0])) <= 4 * 6e-8 * cond + 1e-6


@pytest.mark.parametrize("nb", [48, 400])
def test_zero_second_moment(nb):
    n, m = 2 * nb, 64
    A = torch.zeros(n // nb, nb, nb, device=DEV)
    Q = torch.empty_like(A)
    lam = torch.empty(n // nb, nb, device=DEV)
    info = torch.empty(n // nb, dtype=torch.int32, device=DEV)
    dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_EXACT, lam=lam, info=info)
    lam_r, Q_r, _ = oracle.eig(np.zeros((n // nb, nb, nb)))
    np.testing.assert_array_equal(host(Q), Q_r)
    np.testing.assert_array_equal(host(lam), lam_r)
    assert bool((info >= 0).all())
    rng = RNG(89)
    Qp = t32(np.stack([workload.haar(nb, rng) for _ in range(n // nb)]))
    dobb.dobb_refresh_basis(A, Qp, dobb.DOBB_REFRESH_ORTH_ITER, iters=1)
    Q_oi, _ = oracle.orth_iter(np.zeros((n // nb, nb, nb)), host(Qp), k=1)
    np.testing.assert_array_equal(host(Qp), Q_oi)
    W, G, M = (t32(0.02 * rng.standard_normal((m, n))), t32(rng.standard_normal((m, n))),
               t32(rng.standard_normal((m, n))))
    hp = _hp(m, n)
    M1, U = M.clone(), torch.empty(m, n, device=DEV)
    dobb.dobb_step(W.clone(), G, M1, Q, nb, dobb.make_hparams(**hp), U_out=U)
    np.testing.assert_array_equal(host(U), np.sign(host(M1)))
