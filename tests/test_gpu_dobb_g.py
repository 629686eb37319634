"""GPU parity of the Dobb-G step (output-gradient basis, blocks of rows; Tables 12-13 of the Dobb
listing) against the fp64 oracle (MI355X only).

Bars as for the activation-side step (test_gpu_parity.py), transposed: the coefficients
C_b = P_b^T M_b (read back through C_out) to 1e-5 relative Frobenius per block; no sign mismatch where
|C_ref| > 1e-5 max|C_ref|; U_b = P_b sign(C_b) to 1e-5; W within one fp32 update; identity and
Dobb-G-l2 updates to 1e-5 relative Frobenius.  The step is independent across columns within a
block, so at full size the oracle runs on sampled columns.  End to end: the output-gradient moment
captured from N x m output gradients, an exact refresh, and one step: <= 0.1 % of U's entries differ.
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


def _case(m, n, nb, seed, w_dtype=torch.float32, g_dtype=torch.float32, p_dtype=torch.float32, mu=0.9, wd=0.1,
          nesterov=False):
    rng = RNG(seed)
    P = t32(np.stack([workload.haar(nb, rng) for _ in range(m // nb)])).to(p_dtype)
    W = t32(0.02 * rng.standard_normal((m, n))).to(w_dtype)
    G = t32(rng.standard_normal((m, n))).to(g_dtype)
    M = t32(rng.standard_normal((m, n)))
    hp = dict(lr=f32(2.5e-3), weight_decay=f32(wd), momentum=f32(mu),
              update_scale=f32(oracle.default_update_scale_g(m, n)), nesterov=nesterov)
    return P, W, G, M, hp


def _run(W, G, M, P, nb, hp, norm):
    W, M = W.clone(), M.clone()
    U = torch.empty(W.shape, device=DEV)
    C = torch.full(W.shape, float("nan"), device=DEV)
    dobb.dobb_step_g(W, G, M, P, nb, dobb.make_hparams(norm=norm, **hp), U_out=U, C_out=C)
    return W, M, U, C


def _check_sign_blocks(Ph, M_eff, Ug, Cg, nb, live_rows=None):
    for b in range(Ph.shape[0]):
        r = slice(b * nb, (b + 1) * nb)
        C_ref = Ph[b].T @ M_eff[r]
        assert np.linalg.norm(Cg[r] - C_ref) <= 1e-5 * np.linalg.norm(C_ref), f"projection C, block {b}"
        S = np.rint(np.linalg.solve(Ph[b], Ug[r]))          # U_b = P_b S_b
        live = np.abs(C_ref) > 1e-5 * np.max(np.abs(C_ref))
        assert np.all(S[live] == np.sign(C_ref[live])), f"sign mismatch outside the dead zone, block {b}"
        R = Ph[b] @ S
        assert np.linalg.norm(Ug[r] - R) <= 1e-5 * np.linalg.norm(R), f"reconstruction, block {b}"


@pytest.mark.parametrize("m,n,nb", [(768, 768, 192), (300, 70, 100), (96, 130, 48), (75, 64, 25), (800, 200, 400),
                                    (128, 96, 128)])
def test_step_g_matches_oracle(m, n, nb):
    print(f"dobb-g step m={m} n={n} nb={nb}", flush=True)
    P, W, G, M, hp = _case(m, n, nb, seed=m + n + nb)
    Ph = host(P)
    W_s, M_s, U_s, C_s = _run(W, G, M, P, nb, hp, dobb.DOBB_NORM_SIGN)
    W_r, M_r, U_r = oracle.step_g(W.cpu(), G.cpu(), M.cpu(), Ph, nb, hp["lr"], hp["weight_decay"], hp["momentum"],
                                  hp["update_scale"])
    assert np.all(np.abs(host(M_s) - M_r) <= 6e-8 * np.abs(M_r) + 1e-30)
    Ug = host(U_s)
    _check_sign_blocks(Ph, M_r, Ug, host(C_s), nb)
    assert np.mean(np.abs(Ug - U_r) > 1e-3) <= 1e-3
    check_w(host(W_s), host(W), Ug, hp)


@pytest.mark.parametrize("m,n,nb", [(192, 100, 64), (300, 52, 100)])
def test_step_g_identity_l2_and_nesterov(m, n, nb):
    """Identity (U = M), Dobb-G-l2 (each coefficient row normalised over the n columns) and Nesterov."""
    print(f"dobb-g identity/l2/nesterov m={m} n={n} nb={nb}", flush=True)
    P, W, G, M, hp = _case(m, n, nb, seed=7 * m + nb, mu=1.0)
    _, _, U_id, _ = _run(W, torch.zeros_like(G), M, P, nb, hp, dobb.DOBB_NORM_IDENTITY)
    np.testing.assert_allclose(host(U_id), host(M), atol=2e-6 * float(M.abs().max()))
    P, W, G, M, hp = _case(m, n, nb, seed=7 * m + nb + 1, nesterov=True)
    Ph = host(P)
    for norm, onorm in [(dobb.DOBB_NORM_COL_L2, oracle.NORM_COL_L2), (dobb.DOBB_NORM_IDENTITY, oracle.NORM_IDENTITY),
                        (dobb.DOBB_NORM_SIGN, oracle.NORM_SIGN)]:
        hp2 = dict(hp, update_scale=f32(0.2 * np.sqrt(max(m, n)) if norm == dobb.DOBB_NORM_COL_L2 else hp["update_scale"]))
        W_g, M_g, U_g, _ = _run(W, G, M, P, nb, hp2, norm)
        W_r, M_r, U_r = oracle.step_g(W.cpu(), G.cpu(), M.cpu(), Ph, nb, hp2["lr"], hp2["weight_decay"],
                                      hp2["momentum"], hp2["update_scale"], nesterov=True, norm=onorm)
        if norm == dobb.DOBB_NORM_SIGN:
            assert np.mean(np.abs(host(U_g) - U_r) > 1e-3) <= 1e-3
        else:
            assert np.linalg.norm(host(U_g) - U_r) <= 1e-5 * np.linalg.norm(U_r), f"norm {norm}"
        check_w(host(W_g), host(W), host(U_g), hp2)


@pytest.mark.parametrize("m,n,nb", [(256, 200, 128), (300, 96, 100)])
def test_step_g_bf16_weights_gradients_and_basis(m, n, nb):
    print(f"dobb-g bf16 m={m} n={n} nb={nb}", flush=True)
    P, W, G, M, hp = _case(m, n, nb, seed=11 + nb, w_dtype=torch.bfloat16, g_dtype=torch.bfloat16,
                           p_dtype=torch.bfloat16)
    Ph = host(P)                       # the bf16 basis values both sides use
    W_s, M_s, U_s, C_s = _run(W, G, M, P, nb, hp, dobb.DOBB_NORM_SIGN)
    W_r, M_r, U_r = oracle.step_g(W.cpu(), G.cpu(), M.cpu(), Ph, nb, hp["lr"], hp["weight_decay"], hp["momentum"],
                                  hp["update_scale"])
    assert np.all(np.abs(host(M_s) - M_r) <= 6e-8 * np.abs(M_r) + 1e-30)
    Ug = host(U_s)
    _check_sign_blocks(Ph, M_r, Ug, host(C_s), nb)
    assert np.mean(np.abs(Ug - U_r) > 1e-3) <= 1e-3
    check_w(host(W_s), host(W), Ug, hp, bf16=True)


@pytest.mark.parametrize("m,n,nb", [(4800, 1600, 300), (1600, 6400, 100), (6400, 1600, 400)])
def test_step_g_fullsize_sampled_columns(m, n, nb):
    """GPT-2 XL shapes with B = 16 blocks on the output axis; the oracle on 40 sampled columns."""
    print(f"dobb-g fullsize {m}x{n} nb={nb}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(m + 3 * n + nb)
    B = m // nb
    P = torch.linalg.qr(torch.randn(B, nb, nb, device=DEV, generator=g, dtype=torch.float64))[0].float().contiguous()
    W = 0.02 * torch.randn(m, n, device=DEV, generator=g)
    G = torch.randn(m, n, device=DEV, generator=g)
    M = torch.randn(m, n, device=DEV, generator=g)
    hp = dict(lr=f32(2.5e-3), weight_decay=f32(0.1), momentum=f32(0.9),
              update_scale=f32(oracle.default_update_scale_g(m, n)))
    cols = torch.linspace(0, n - 1, 40).long().to(DEV)
    W0, G0, M0 = W[:, cols].cpu(), G[:, cols].cpu(), M[:, cols].cpu()
    U = torch.empty(m, n, device=DEV)
    C = torch.empty(m, n, device=DEV)
    dobb.dobb_step_g(W, G, M, P, nb, dobb.make_hparams(**hp), U_out=U, C_out=C)
    Ph = host(P)
    W_r, M_r, U_r = oracle.step_g(W0, G0, M0, Ph, nb, hp["lr"], hp["weight_decay"], hp["momentum"],
                                  hp["update_scale"], cores=8)
    Ug, Cg = host(U[:, cols]), host(C[:, cols])
    assert np.all(np.abs(host(M[:, cols]) - M_r) <= 6e-8 * np.abs(M_r) + 1e-30)
    _check_sign_blocks(Ph, M_r, Ug, Cg, nb)
    assert np.mean(np.abs(Ug - U_r) > 1e-3) <= 1e-3
    check_w(host(W[:, cols]), W0.double().numpy(), Ug, hp)


def test_step_g_grouped_equals_single_calls():
    rng = RNG(61)
    shapes = [(96, 64, 48)] * 5 + [(128, 40, 64)] * 2
    Ws, Gs, Ms, Ps, nbs, hps = [], [], [], [], [], []
    for m, n, nb in shapes:
        Ws.append(t32(0.02 * rng.standard_normal((m, n))))
        Gs.append(t32(rng.standard_normal((m, n))))
        Ms.append(t32(rng.standard_normal((m, n))))
        Ps.append(t32(np.stack([workload.haar(nb, rng) for _ in range(m // nb)])))
        nbs.append(nb)
        hps.append(dobb.make_hparams(2.5e-3, 0.1, 0.9, oracle.default_update_scale_g(m, n)))
    Ws1, Ms1 = [w.clone() for w in Ws], [x.clone() for x in Ms]
    for W, G, M, P, nb, hp in zip(Ws1, Gs, Ms1, Ps, nbs, hps):
        dobb.dobb_step_g(W, G, M, P, nb, hp)
    dobb.dobb_step_g_grouped(Ws, Gs, Ms, Ps, nbs, hps)
    for a, b in zip(Ws + Ms, Ws1 + Ms1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("seed", [0, 1])
def test_dobb_g_end_to_end_768_B4(seed):
    """Output gradients dY (N = 4096 tokens x 768 outputs, a 15 % effective-rank power-law moment, fp32):
    capture with dobb_accumulate_moment on dY, exact refresh, one Dobb-G step with mu = 0 (M = G)."""
    print(f"dobb-g end-to-end seed={seed}", flush=True)
    rng = RNG(300 + seed)
    N, m, n, nb = 4096, 768, 768, 192
    dY = t32(workload.activations(N, m, 0.15, rng))
    G = t32(rng.standard_normal((m, n)))
    W = t32(0.02 * rng.standard_normal((m, n)))
    hp = dict(lr=f32(2.5e-3), weight_decay=f32(0.1), momentum=0.0,
              update_scale=f32(oracle.default_update_scale_g(m, n)))
    A = torch.empty(m // nb, nb, nb, device=DEV)
    dobb.dobb_accumulate_moment(dY, A, nb)
    P = torch.empty_like(A)
    info = torch.empty(m // nb, dtype=torch.int32, device=DEV)
    dobb.dobb_refresh_basis(A, P, dobb.DOBB_REFRESH_EXACT, info=info)
    assert bool((info > 0).all())
    M = torch.zeros(m, n, device=DEV)
    W1, U = W.clone(), torch.empty(m, n, device=DEV)
    dobb.dobb_step_g(W1, G, M, P, nb, dobb.make_hparams(**hp), U_out=U)
    A_ref = oracle.accumulate(dY.cpu(), nb, cores=4)
    _, P_ref, _ = oracle.eig(A_ref)
    W_ref, _, U_ref = oracle.step_g(W.cpu(), G.cpu(), np.zeros((m, n)), P_ref, nb, hp["lr"], hp["weight_decay"],
                                    0.0, hp["update_scale"])
    Ug = host(U)
    rms = np.sqrt(np.mean(U_ref ** 2))
    frac = np.mean(np.abs(Ug - U_ref) > 1e-3 * rms)
    print(f"  differing U entries {frac:.2e}", flush=True)
    assert frac <= 1e-3
