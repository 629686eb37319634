"""Pins of the CPU oracle against what the Dobb pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: values the pages print (Table 1(a),
Table 9 -- fixtures under tests/golden/), LAPACK routines called as independent references
(eigh, qr, svd), closed forms, invariants and brute force on tiny inputs.  The cases are chosen so a
plausible slip in the oracle (a dropped term, a wrong sign or index, a transposed operand) fails one.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
import workload
from oracle import metrics

RNG = np.random.default_rng


def _golden(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return np.array(rows)


def _spd(n, rng, spread=1e3):
    """Symmetric positive definite matrix with distinct log-spaced eigenvalues."""
    lam = np.geomspace(1.0, 1.0 / spread, n)
    V = workload.haar(n, rng)
    return (V * lam) @ V.T, lam


# ------------------------------------------------------------------------------------------------
# the pages' measures (orthogonality, effective rank)

def test_table1a_orthogonality_of_Y_and_signY(golden_dir):
    """Table 1(a): ortho(Y) is fixed by the spectrum; ortho(sign(Y)) within seed noise."""
    rows = _golden(golden_dir, "table1a.txt")
    for frac, ortho_y, ortho_sign in rows:
        Y = workload.table1_matrix(768, frac, RNG(0))
        s = np.linalg.svd(Y, compute_uv=False)
        assert metrics.effective_rank(s) == pytest.approx(frac, abs=1e-6)
        assert metrics.orthogonality(Y) == pytest.approx(ortho_y, abs=5e-4)
        assert metrics.orthogonality(np.sign(Y)) == pytest.approx(ortho_sign, abs=1.2e-2)


def test_orthogonality_closed_forms():
    rng = RNG(1)
    assert metrics.orthogonality(workload.haar(40, rng)) == pytest.approx(1.0, abs=1e-12)
    # m x n with orthonormal columns scaled: all singular values equal -> 1
    q = workload.haar(50, rng)[:, :20] * 3.0
    assert metrics.orthogonality(q) == pytest.approx(1.0, abs=1e-12)
    # rank one -> 1 / sqrt(min(m, n))
    r1 = np.outer(rng.standard_normal(30), rng.standard_normal(12))
    assert metrics.orthogonality(r1) == pytest.approx(1.0 / np.sqrt(12), abs=1e-12)
    # two singular values 3 and 4 in a 2 x 2: (3+4)/(sqrt2 * 5)
    assert metrics.orthogonality(np.diag([3.0, 4.0])) == pytest.approx(7 / (np.sqrt(2) * 5), abs=1e-15)


def test_effective_rank_closed_forms():
    assert metrics.effective_rank(np.r_[np.ones(30), np.zeros(70)]) == pytest.approx(0.30, abs=1e-15)
    assert metrics.effective_rank(np.ones(17)) == pytest.approx(1.0, abs=1e-15)
    assert metrics.effective_rank(np.r_[1.0, np.zeros(9)]) == pytest.approx(0.1, abs=1e-15)


# ------------------------------------------------------------------------------------------------
# accumulate

def test_accumulate_quadratic_form_and_trace():
    """v^T A_b v = ||X_b v||^2 / N and tr A_b = ||X_b||_F^2 / N for every block."""
    rng = RNG(2)
    N, n, nb = 300, 24, 8
    X = rng.standard_normal((N, n))
    A = oracle.accumulate(X, nb)
    for b in range(n // nb):
        Xb = X[:, b * nb:(b + 1) * nb]
        for _ in range(5):
            v = rng.standard_normal(nb)
            assert v @ A[b] @ v == pytest.approx(np.sum((Xb @ v) ** 2) / N, rel=1e-12)
        assert np.trace(A[b]) == pytest.approx(np.sum(Xb ** 2) / N, rel=1e-12)
        np.testing.assert_array_equal(A[b], A[b].T)


def test_accumulate_blocks_are_diagonal_blocks_of_full_moment():
    rng = RNG(3)
    X = rng.standard_normal((97, 30))
    full = oracle.accumulate(X, 30)[0]
    blocks = oracle.accumulate(X, 10)
    for b in range(3):
        np.testing.assert_allclose(blocks[b], full[b * 10:(b + 1) * 10, b * 10:(b + 1) * 10], rtol=1e-13)


def test_accumulate_disjoint_support_gives_diagonal():
    """Tokens that are scaled one-hot vectors give a diagonal second moment of mean squares."""
    N, n = 64, 16
    X = np.zeros((N, n))
    idx = np.arange(N) % n
    X[np.arange(N), idx] = np.arange(1, N + 1)
    A = oracle.accumulate(X, 4)
    for b in range(4):
        want = np.zeros(4)
        for t in range(N):
            if idx[t] // 4 == b:
                want[idx[t] % 4] += (t + 1) ** 2
        np.testing.assert_array_equal(A[b], np.diag(want / N))


def test_accumulate_ema_closed_form():
    """Two captures: A = beta (1-beta) S1/N1 + (1-beta) S2/N2 from a zero start."""
    rng = RNG(4)
    X1, X2 = rng.standard_normal((50, 12)), rng.standard_normal((70, 12))
    beta = 0.9
    A = oracle.accumulate(X1, 6, beta=beta)
    A = oracle.accumulate(X2, 6, A=A, beta=beta)
    for b in range(2):
        s1 = X1[:, b * 6:(b + 1) * 6]
        s2 = X2[:, b * 6:(b + 1) * 6]
        want = beta * (1 - beta) * (s1.T @ s1) / 50 + (1 - beta) * (s2.T @ s2) / 70
        np.testing.assert_allclose(A[b], want, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------------------------------------
# exact refresh (Jacobi)

@pytest.mark.parametrize("n", [2, 5, 16, 48])
def test_jacobi_matches_lapack_eigh(n):
    rng = RNG(10 + n)
    A, _ = _spd(n, rng)
    lam, Q, info = oracle.eig(A[None])
    assert info[0] > 0
    w, V = np.linalg.eigh(A)
    w, V = w[::-1], V[:, ::-1]
    np.testing.assert_allclose(lam[0], w, rtol=1e-11, atol=1e-14)
    # eigenvectors agree up to sign
    s = np.sign(np.sum(Q[0] * V, axis=0))
    np.testing.assert_allclose(Q[0], V * s, atol=1e-9)
    # residual and orthonormality
    assert np.linalg.norm(A @ Q[0] - Q[0] * lam[0]) <= 1e-13 * np.linalg.norm(A)
    assert np.max(np.abs(Q[0].T @ Q[0] - np.eye(n))) <= 1e-13


def _numpy_sign_rule(V):
    """An independent statement of the eigenvector sign convention: each column is flipped so that
    its largest-magnitude entry is positive, ties going to the lowest row index (np.argmax returns
    the first maximum)."""
    V = V.copy()
    for j in range(V.shape[1]):
        i = int(np.argmax(np.abs(V[:, j])))
        if V[i, j] < 0:
            V[:, j] = -V[:, j]
    return V


def test_jacobi_full_matrix_B1_vs_eigh_768():
    """B = 1 versus the full-matrix eigenbasis at the Table 1 size (one 768-wide block, cold start):
    eigenvalues against LAPACK, and eigenvectors compared directly (the sign convention fixes them)
    within the first-order bound of an fp64 solver, c u ||A|| / gap_j."""
    rng = RNG(7)
    X = workload.activations(2048, 768, 0.15, rng)
    A = oracle.accumulate(X, 768)
    lam, Q, info = oracle.eig(A)
    w, V = np.linalg.eigh(A[0])
    w, V = w[::-1], _numpy_sign_rule(V[:, ::-1])
    assert info[0] > 0
    assert np.max(np.abs(lam[0] - w)) <= 1e-12 * w[0]
    gap = np.full(768, np.inf)
    gap[:-1] = np.minimum(gap[:-1], w[:-1] - w[1:])
    gap[1:] = np.minimum(gap[1:], w[:-1] - w[1:])
    err = np.linalg.norm(Q[0] - V, axis=0)
    bound = 1e-12 * np.linalg.norm(A[0]) / gap + 1e-9
    assert np.all(err <= bound), np.max(err / bound)


@pytest.mark.parametrize("n,seed", [(8, 1), (64, 2), (200, 3)])
def test_eigenvector_sign_rule_on_dense_matrices(n, seed):
    """Dense eigenvectors: the largest entry of every column of Q is positive, and Q equals LAPACK's
    eigenvectors with the rule applied by numpy (a first-entry or last-entry rule fails here)."""
    A, _ = _spd(n, RNG(500 + seed))
    lam, Q, info = oracle.eig(A[None])
    w, V = np.linalg.eigh(A)
    V = _numpy_sign_rule(V[:, ::-1])
    np.testing.assert_allclose(Q[0], V, atol=1e-9)
    first = np.sign(Q[0][0, :])
    assert np.any(first < 0), "the test matrix should have columns whose first entry is negative"


def test_eigenvector_sign_rule_ties_go_to_lowest_index():
    """[[2, 1], [1, 2]] has eigenvectors (1, 1)/sqrt(2) (lambda = 3) and (1, -1)/sqrt(2) (lambda = 1):
    both entries of the second tie in magnitude, so the first one is the positive one."""
    lam, Q, _ = oracle.eig(np.array([[[2.0, 1.0], [1.0, 2.0]]]))
    np.testing.assert_allclose(lam[0], [3.0, 1.0], rtol=1e-15)
    r = np.sqrt(0.5)
    np.testing.assert_allclose(Q[0], [[r, r], [r, -r]], rtol=0, atol=1e-15)
    # a tie between entries 1 and 2 of a 3-vector: (0, 1, -1)/sqrt(2) keeps entry 1 positive
    A = np.array([[5.0, 0.0, 0.0], [0.0, 2.0, 1.0], [0.0, 1.0, 2.0]])
    lam, Q, _ = oracle.eig(A[None])
    np.testing.assert_allclose(lam[0], [5.0, 3.0, 1.0], rtol=1e-15)
    np.testing.assert_allclose(Q[0][:, 2], [0.0, r, -r], atol=1e-15)


def test_jacobi_2x2_closed_form():
    a, b, d = 3.0, 1.5, -2.0
    lam, Q, _ = oracle.eig(np.array([[[a, b], [b, d]]]))
    r = np.hypot((a - d) / 2, b)
    np.testing.assert_allclose(lam[0], [(a + d) / 2 + r, (a + d) / 2 - r], rtol=1e-15)
    theta = 0.5 * np.arctan2(2 * b, a - d)
    v = np.array([np.cos(theta), np.sin(theta)])  # eigenvector of the larger eigenvalue
    assert abs(abs(Q[0][:, 0] @ v) - 1.0) < 1e-15


def test_jacobi_diagonal_is_signed_permutation():
    d = np.array([0.3, 2.0, -1.0, 5.0, 0.7])
    lam, Q, info = oracle.eig(np.diag(d)[None])
    np.testing.assert_array_equal(lam[0], np.sort(d)[::-1])
    P = np.zeros((5, 5))
    for j, i in enumerate(np.argsort(-d)):
        P[i, j] = 1.0
    np.testing.assert_array_equal(Q[0], P)   # largest entry made positive
    assert info[0] == 0


def _count_below(A, x):
    """Number of eigenvalues of A below x: negative pivots of A - xI (Sylvester's law of inertia)."""
    M = A - x * np.eye(len(A))
    neg = 0
    for k in range(len(A)):
        p = M[k, k]
        if p < 0:
            neg += 1
        if p == 0:
            p = 1e-300
        M[k + 1:, k + 1:] -= np.outer(M[k + 1:, k], M[k, k + 1:]) / p
    return neg


def test_jacobi_8x8_against_inertia_bisection():
    rng = RNG(8)
    A = rng.standard_normal((8, 8))
    A = A + A.T
    lam, _, _ = oracle.eig(A[None])
    lo, hi = -np.abs(A).sum(), np.abs(A).sum()
    for j in range(8):     # the j-th largest eigenvalue has 8-1-j eigenvalues below it
        a, b = lo, hi
        for _ in range(200):
            mid = 0.5 * (a + b)
            if _count_below(A, mid) <= 7 - j:
                a = mid
            else:
                b = mid
        assert lam[0][j] == pytest.approx(0.5 * (a + b), abs=1e-12)


def test_jacobi_warm_start_same_result():
    rng = RNG(9)
    A, _ = _spd(20, rng)
    lam_c, Q_c, _ = oracle.eig(A[None])
    V0 = workload.haar(20, rng)
    lam_w, Q_w, info = oracle.eig(A[None], V0=V0[None])
    np.testing.assert_allclose(lam_w, lam_c, rtol=1e-12)
    np.testing.assert_allclose(Q_w, Q_c, atol=1e-10)
    # warm start from the exact basis: already diagonal up to rounding -> at most one sweep
    _, _, info2 = oracle.eig(A[None], V0=Q_c)
    assert 0 <= info2[0] <= 1


def test_jacobi_reports_non_convergence():
    rng = RNG(11)
    A, _ = _spd(30, rng)
    _, _, info = oracle.eig(A[None], max_sweeps=1)
    assert info[0] == -1


# ------------------------------------------------------------------------------------------------
# Householder QR and orthogonal iteration

@pytest.mark.parametrize("n", [1, 3, 17, 64])
def test_householder_qr_unique_factor(n):
    rng = RNG(20 + n)
    Z = rng.standard_normal((n, n))
    Q = oracle.householder_qr(Z)
    q, r = np.linalg.qr(Z)
    np.testing.assert_allclose(Q, q * np.sign(np.diag(r)), atol=1e-12)
    R = Q.T @ Z
    assert np.max(np.abs(np.tril(R, -1))) <= 1e-12
    assert np.all(np.diag(R) > 0)


def test_householder_qr_matches_gram_schmidt():
    """QR with diag(R) > 0 is unique: modified Gram-Schmidt on a well-conditioned matrix agrees."""
    rng = RNG(30)
    Z = rng.standard_normal((12, 12)) + 6 * np.eye(12)
    Q = oracle.householder_qr(Z)
    G = Z.copy()
    for j in range(12):
        for i in range(j):
            G[:, j] -= (G[:, i] @ G[:, j]) * G[:, i]
        G[:, j] /= np.linalg.norm(G[:, j])
    np.testing.assert_allclose(Q, G, atol=1e-12)


def test_orth_iter_fixed_point_and_convergence():
    rng = RNG(31)
    A, lam = _spd(16, rng, spread=50)
    w, V = np.linalg.eigh(A)
    V = V[:, ::-1] * np.sign(V[:, ::-1][0])
    # the exact eigenbasis (positive eigenvalues) is a fixed point: A V = V diag(lam), R = diag(lam)
    Q1, rq = oracle.orth_iter(A[None], V[None], k=1)
    np.testing.assert_allclose(Q1[0], V, atol=1e-12)
    np.testing.assert_allclose(rq[0], w[::-1], rtol=1e-12)
    # from a random start, many steps converge to the descending eigenbasis (up to sign)
    Qk, _ = oracle.orth_iter(A[None], workload.haar(16, rng)[None], k=3000)
    np.testing.assert_allclose(np.abs(Qk[0]), np.abs(V), atol=1e-6)


# ------------------------------------------------------------------------------------------------
# the step: projection, sign, reconstruction, update

def _random_basis(B, nb, rng):
    return np.stack([workload.haar(nb, rng) for _ in range(B)])


def test_identity_norm_round_trip():
    rng = RNG(40)
    m, n, nb = 20, 24, 6
    M = rng.standard_normal((m, n))
    Q = _random_basis(n // nb, nb, rng)
    _, _, U = oracle.step(np.zeros((m, n)), np.zeros((m, n)), M, Q, nb, 0.0, 0.0, 1.0, 1.0,
                          norm=oracle.NORM_IDENTITY)
    np.testing.assert_allclose(U, M, atol=1e-13)


def test_sign_update_structure():
    """U_b Q_b has entries +-1, every row of U_b has norm sqrt(nb), ||U||_F^2 = m n (Table 9)."""
    rng = RNG(41)
    m, n, nb = 30, 32, 8
    M = rng.standard_normal((m, n))
    Q = _random_basis(n // nb, nb, rng)
    _, _, U = oracle.step(np.zeros((m, n)), np.zeros((m, n)), M, Q, nb, 0.0, 0.0, 1.0, 1.0)
    for b in range(n // nb):
        S = U[:, b * nb:(b + 1) * nb] @ Q[b]
        np.testing.assert_allclose(np.abs(S), 1.0, atol=1e-13)
        np.testing.assert_allclose(np.linalg.norm(U[:, b * nb:(b + 1) * nb], axis=1), np.sqrt(nb), rtol=1e-13)
    assert np.sum(U * U) == pytest.approx(m * n, rel=1e-13)


def test_projection_uses_Q_not_Q_transpose():
    """Build M from prescribed coefficients: M_b = C0 Q_b^T, so C_b = C0 and U_b = sign(C0) Q_b^T.
    A transposed basis (M Q^T) or reconstruction (S Q) would scramble the sign pattern."""
    rng = RNG(42)
    m, nb = 9, 7
    Q = _random_basis(1, nb, rng)
    C0 = rng.choice([-1.0, 1.0], size=(m, nb)) * rng.uniform(0.1, 1.0, size=(m, nb))
    M = C0 @ Q[0].T
    _, _, U = oracle.step(np.zeros((m, nb)), np.zeros((m, nb)), M, Q, nb, 0.0, 0.0, 1.0, 1.0)
    np.testing.assert_allclose(U @ Q[0], np.sign(C0), atol=1e-13)


def test_brute_force_steepest_direction_8x8():
    """Each row of U_b maximises <m_r, v Q_b^T> over all 2^8 sign vectors v (the l_inf-steepest
    direction in the eigenbasis that Table 13 labels Dobb)."""
    rng = RNG(43)
    nb = 8
    Q = _random_basis(1, nb, rng)
    M = rng.standard_normal((8, nb))
    _, _, U = oracle.step(np.zeros((8, nb)), np.zeros((8, nb)), M, Q, nb, 0.0, 0.0, 1.0, 1.0)
    cands = np.array(list(itertools.product([-1.0, 1.0], repeat=nb))) @ Q[0].T   # 256 x nb
    for r in range(8):
        scores = cands @ M[r]
        best = cands[np.argmax(scores)]
        np.testing.assert_allclose(U[r], best, atol=1e-13)
        assert M[r] @ U[r] == pytest.approx(scores.max(), rel=1e-13)


def test_sign_flip_invariance_bitwise_and_permutation_invariance():
    rng = RNG(44)
    m, n, nb = 16, 20, 5
    M = rng.standard_normal((m, n))
    Q = _random_basis(n // nb, nb, rng)
    z = np.zeros((m, n))
    _, _, U = oracle.step(z, z, M, Q, nb, 0.0, 0.0, 1.0, 1.0)
    flips = rng.choice([-1.0, 1.0], size=(n // nb, 1, nb))
    _, _, U2 = oracle.step(z, z, M, Q * flips, nb, 0.0, 0.0, 1.0, 1.0)
    np.testing.assert_array_equal(U, U2)
    perm = rng.permutation(nb)
    _, _, U3 = oracle.step(z, z, M, Q[:, :, perm], nb, 0.0, 0.0, 1.0, 1.0)
    np.testing.assert_allclose(U, U3, atol=1e-13)


def test_block_size_one_is_sign_descent():
    rng = RNG(45)
    M = rng.standard_normal((9, 11))
    M[0, 0] = 0.0
    Q = np.ones((11, 1, 1))
    _, _, U = oracle.step(np.zeros_like(M), np.zeros_like(M), M, Q, 1, 0.0, 0.0, 1.0, 1.0)
    np.testing.assert_array_equal(U, np.sign(M))


def test_update_rule_and_table9_scale(golden_dir):
    rng = RNG(46)
    for m, n, rms in _golden(golden_dir, "table9_gpt2_rms.txt"):
        m, n = int(m), int(n)
        assert oracle.default_update_scale(m, n) == pytest.approx(rms, rel=1e-12)
    m, n, nb = 24, 48, 12
    W, G, M0 = rng.standard_normal((3, m, n))
    Q = _random_basis(n // nb, nb, rng)
    lr, wd, mu = 0.01, 0.1, 0.9
    s = oracle.default_update_scale(m, n)
    W1, M1, U = oracle.step(W, G, M0, Q, nb, lr, wd, mu, s)
    np.testing.assert_allclose(M1, mu * M0 + G, rtol=1e-15)
    np.testing.assert_allclose(W1, W - lr * (s * U + wd * W), rtol=1e-14, atol=1e-15)
    # RMS of the applied update s*U equals tau sqrt(max(m,n)/m) with nonzero coefficients
    assert np.sqrt(np.mean((s * U) ** 2)) == pytest.approx(0.2 * np.sqrt(max(m, n) / m), rel=1e-12)
    # no gradient, no momentum: only decoupled weight decay acts
    W2, _, U0 = oracle.step(W, np.zeros_like(G), np.zeros_like(M0), Q, nb, lr, wd, mu, s)
    np.testing.assert_array_equal(U0, 0.0)
    np.testing.assert_allclose(W2, (1 - lr * wd) * W, rtol=1e-15)


def test_nesterov_and_nan_propagation():
    rng = RNG(47)
    m, n, nb = 6, 8, 4
    G, M0 = rng.standard_normal((2, m, n))
    Q = _random_basis(2, nb, rng)
    z = np.zeros((m, n))
    _, _, U_n = oracle.step(z, G, M0, Q, nb, 0.0, 0.0, 0.5, 1.0, nesterov=True, norm=oracle.NORM_IDENTITY)
    np.testing.assert_allclose(U_n, G + 0.5 * (0.5 * M0 + G), atol=1e-13)
    Mn = M0.copy()
    Mn[2, 5] = np.nan
    _, _, U = oracle.step(z, z, Mn, Q, nb, 0.0, 0.0, 1.0, 1.0)
    assert np.all(np.isnan(U[2, 4:8])) and np.all(np.isfinite(U[2, :4])) and np.all(np.isfinite(np.delete(U, 2, 0)))


def test_column_l2_variant_norm():
    """Dobb-l2: unit-norm columns of C, so ||U||_F^2 = n (Table 9: raw ||O||_F^2 = n)."""
    rng = RNG(48)
    m, n, nb = 40, 24, 8
    M = rng.standard_normal((m, n))
    Q = _random_basis(3, nb, rng)
    z = np.zeros((m, n))
    _, _, U = oracle.step(z, z, M, Q, nb, 0.0, 0.0, 1.0, 1.0, norm=oracle.NORM_COL_L2)
    assert np.sum(U * U) == pytest.approx(n, rel=1e-12)
    for b in range(3):
        C = U[:, b * nb:(b + 1) * nb] @ Q[b]
        np.testing.assert_allclose(np.linalg.norm(C, axis=0), 1.0, rtol=1e-12)


def test_diagonal_moment_gives_sign_of_momentum():
    """A diagonal second moment has a signed-permutation eigenbasis, so U = sign(M)."""
    rng = RNG(49)
    m, n, nb = 10, 12, 4
    X = np.zeros((40, n))
    X[np.arange(40), np.arange(40) % n] = rng.uniform(1, 2, 40)
    A = oracle.accumulate(X, nb)
    _, Q, _ = oracle.eig(A)
    M = rng.standard_normal((m, n))
    _, _, U = oracle.step(np.zeros((m, n)), np.zeros((m, n)), M, Q, nb, 0.0, 0.0, 1.0, 1.0)
    np.testing.assert_array_equal(U, np.sign(M))


def test_threaded_oracle_equals_single_thread_bitwise():
    """The baseline timing shares independent rows (step) and blocks (capture) among threads: each
    unit is the same loop as in one thread, so the results are bitwise the same."""
    rng = RNG(77)
    m, n, nb = 130, 192, 48
    W, G, M = (rng.standard_normal((m, n)) for _ in range(3))
    Q = np.stack([workload.haar(nb, rng) for _ in range(n // nb)])
    a = oracle.step(W, G, M, Q, nb, 2.5e-3, 0.1, 0.9, 0.2)
    b = oracle.step(W, G, M, Q, nb, 2.5e-3, 0.1, 0.9, 0.2, cores=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    X = rng.standard_normal((333, n))
    A0 = oracle.accumulate(X, nb)
    np.testing.assert_array_equal(A0, oracle.accumulate(X, nb, cores=3))
    np.testing.assert_array_equal(oracle.accumulate(X, nb, A=A0, beta=0.9),
                                  oracle.accumulate(X, nb, A=A0, beta=0.9, cores=4))


# ------------------------------------------------------------------------------------------------
# Dobb-G: the basis of the output-gradient second moment, blocks on the output axis (Tables 12-13)

def test_dobb_g_is_dobb_on_the_transposed_weight():
    """Dobb-G on W (blocks of rows, C_b = P_b^T M_b, U_b = P_b S_b) is Dobb on W^T (blocks of columns,
    C = M^T P, U^T = S^T P^T): the two oracle functions agree on every norm and with Nesterov."""
    rng = RNG(201)
    m, n, nb = 24, 10, 6
    W, G, M = rng.standard_normal((3, m, n))
    P = _random_basis(m // nb, nb, rng)
    for norm in (oracle.NORM_SIGN, oracle.NORM_IDENTITY, oracle.NORM_COL_L2):
        for nest in (False, True):
            Wg, Mg, Ug = oracle.step_g(W, G, M, P, nb, 0.01, 0.1, 0.9, 0.3, nesterov=nest, norm=norm)
            Wt, Mt, Ut = oracle.step(W.T, G.T, M.T, P, nb, 0.01, 0.1, 0.9, 0.3, nesterov=nest, norm=norm)
            np.testing.assert_allclose(Ug, Ut.T, rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(Wg, Wt.T, rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(Mg, Mt.T, rtol=1e-15)


def test_dobb_g_sign_structure_and_table9_scale(golden_dir):
    for m, n, rms in _golden(golden_dir, "table9_dobb_g_rms.txt"):
        assert oracle.default_update_scale_g(int(m), int(n)) == pytest.approx(rms, rel=1e-12)
    rng = RNG(202)
    m, n, nb = 36, 20, 12
    W, G, M = rng.standard_normal((3, m, n))
    P = _random_basis(m // nb, nb, rng)
    s = oracle.default_update_scale_g(m, n)
    W1, M1, U = oracle.step_g(W, G, M, P, nb, 0.01, 0.1, 0.9, s)
    for b in range(m // nb):
        r = slice(b * nb, (b + 1) * nb)
        S = P[b].T @ U[r]                                   # the sign matrix: entries +-1
        np.testing.assert_allclose(np.abs(S), 1.0, atol=1e-13)
        np.testing.assert_allclose(np.linalg.norm(U[r], axis=0), np.sqrt(nb), rtol=1e-13)
    assert np.sum(U * U) == pytest.approx(m * n, rel=1e-12)
    # RMS of the applied update: tau sqrt(max(m, n) / n)
    assert np.sqrt(np.mean((s * U) ** 2)) == pytest.approx(0.2 * np.sqrt(max(m, n) / n), rel=1e-12)
    np.testing.assert_allclose(W1, W - 0.01 * (s * U + 0.1 * W), rtol=1e-14, atol=1e-15)


def test_dobb_g_brute_force_steepest_direction_8x8():
    """Each column of U_b maximises <m_c, P_b v> over all 2^8 sign vectors v: the l_inf-steepest
    direction in the output-side eigenbasis."""
    rng = RNG(203)
    nb = 8
    P = _random_basis(1, nb, rng)
    M = rng.standard_normal((nb, 8))
    _, _, U = oracle.step_g(np.zeros((nb, 8)), np.zeros((nb, 8)), M, P, nb, 0.0, 0.0, 1.0, 1.0)
    cands = P[0] @ np.array(list(itertools.product([-1.0, 1.0], repeat=nb))).T   # nb x 256
    for c in range(8):
        scores = M[:, c] @ cands
        np.testing.assert_allclose(U[:, c], cands[:, np.argmax(scores)], atol=1e-13)


def test_dobb_g_round_trip_block_one_and_sign_flips():
    rng = RNG(204)
    m, n, nb = 20, 7, 5
    W, G, M = rng.standard_normal((3, m, n))
    P = _random_basis(m // nb, nb, rng)
    # identity normalisation: U = P P^T M = M
    _, _, U = oracle.step_g(W, np.zeros_like(G), M, P, nb, 0.0, 0.0, 1.0, 1.0, norm=oracle.NORM_IDENTITY)
    np.testing.assert_allclose(U, M, atol=1e-14)
    # one-row blocks: every basis is [+-1], the step is sign descent
    P1 = rng.choice([-1.0, 1.0], size=(m, 1, 1))
    _, _, U1 = oracle.step_g(W, G, M, P1, 1, 0.0, 0.0, 0.9, 1.0)
    np.testing.assert_array_equal(U1, np.sign(0.9 * M + G))
    # flipping basis vectors leaves U bitwise unchanged
    flips = rng.choice([-1.0, 1.0], size=(m // nb, 1, nb))
    _, _, Ua = oracle.step_g(W, G, M, P, nb, 0.0, 0.0, 0.9, 1.0)
    _, _, Ub = oracle.step_g(W, G, M, P * flips, nb, 0.0, 0.0, 0.9, 1.0)
    np.testing.assert_array_equal(Ua, Ub)


def test_dobb_g_l2_rows_have_unit_norm():
    """Dobb-G-l2: each row of the coefficient block (over the n columns) is normalised, so
    P_b^T U_b has unit rows and ||U||_F^2 = m, Table 9's ||O||_F^2 for Dobb-G-l2 with O = U."""
    rng = RNG(205)
    m, n, nb = 18, 11, 6
    W, G, M = rng.standard_normal((3, m, n))
    P = _random_basis(m // nb, nb, rng)
    _, _, U = oracle.step_g(W, G, M, P, nb, 0.0, 0.0, 0.9, 1.0, norm=oracle.NORM_COL_L2)
    for b in range(m // nb):
        r = slice(b * nb, (b + 1) * nb)
        Ct = P[b].T @ U[r]
        np.testing.assert_allclose(np.linalg.norm(Ct, axis=1), 1.0, rtol=1e-13)
        C = P[b].T @ (0.9 * M[r] + G[r])
        np.testing.assert_allclose(Ct * np.linalg.norm(C, axis=1, keepdims=True), C, rtol=1e-12, atol=1e-13)
    assert np.sum(U * U) == pytest.approx(m, rel=1e-12)
    # threaded over blocks: bitwise the same
    for norm in (oracle.NORM_SIGN, oracle.NORM_COL_L2):
        a = oracle.step_g(W, G, M, P, nb, 0.01, 0.1, 0.9, 0.5, norm=norm)
        b_ = oracle.step_g(W, G, M, P, nb, 0.01, 0.1, 0.9, 0.5, norm=norm, cores=3)
        for x, y in zip(a, b_):
            np.testing.assert_array_equal(x, y)


# ------------------------------------------------------------------------------------------------
# Cholesky QR (Table 16's faster QR routine of the refresh)

@pytest.mark.parametrize("n,cond", [(8, 10.0), (40, 1e3), (100, 1e6)])
def test_cholesky_qr2_is_the_unique_qr_factor(n, cond):
    """QR with diag(R) > 0 is unique: Cholesky QR equals LAPACK's sign-fixed Householder factor and
    the oracle's own Householder QR to cond * 1e-13, is orthonormal to 1e-14 even at cond 1e6 (one
    pass alone loses about cond^2 u = 1e-4 there), and Q^T Z is upper triangular with a positive
    diagonal."""
    rng = RNG(600 + n)
    U, _ = np.linalg.qr(rng.standard_normal((n, n)))
    V, _ = np.linalg.qr(rng.standard_normal((n, n)))
    Z = (U * np.geomspace(1.0, 1.0 / cond, n)) @ V.T
    Q = oracle.cholesky_qr2(Z)
    q, r = np.linalg.qr(Z)
    ref = q * np.sign(np.diag(r))
    np.testing.assert_allclose(Q, ref, atol=1e-13 * cond)
    np.testing.assert_allclose(Q, oracle.householder_qr(Z), atol=1e-13 * cond)
    assert np.max(np.abs(Q.T @ Q - np.eye(n))) <= 1e-14 * n
    R = Q.T @ Z
    assert np.max(np.abs(np.tril(R, -1))) <= 1e-12 * np.linalg.norm(Z)
    assert np.all(np.diag(R) > 0)


def test_cholesky_qr2_reports_rank_deficiency():
    Z = np.ones((5, 5))
    with pytest.raises(np.linalg.LinAlgError):
        oracle.cholesky_qr2(Z)


def test_orth_iter_with_cholesky_qr_equals_householder():
    """Both QR routines give the same refresh (Table 16 compares them as interchangeable routines);
    the exact eigenbasis is a fixed point of either."""
    rng = RNG(610)
    A = np.stack([_spd(24, rng, spread=300)[0] for _ in range(3)])
    Qp = _random_basis(3, 24, rng)
    for k in (1, 2):
        Qh, lh = oracle.orth_iter(A, Qp, k=k)
        Qc, lc = oracle.orth_iter(A, Qp, k=k, qr="cholesky")
        np.testing.assert_allclose(Qc, Qh, atol=1e-11)
        np.testing.assert_allclose(lc, lh, rtol=1e-12, atol=1e-14)
    w, V = np.linalg.eigh(A[0])
    V = V[:, ::-1] * np.sign(V[:, ::-1][0])
    Q1, _ = oracle.orth_iter(A[:1], V[None], k=1, qr="cholesky")
    np.testing.assert_allclose(Q1[0], V, atol=1e-12)
