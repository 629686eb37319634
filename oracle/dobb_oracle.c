/*
 * Dobb CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 implementation of what the Dobb optimizer step computes, written from the
 * pages on "Dobb: Shard-Local Preconditioning in Block-Diagonal Eigenbases" (arXiv 2610.39412):
 * the abstract (paperdot.bitmofang.com and thelatestinai.com listings) and the tables of the
 * thelatestinai.com listing.  Only tests/, the package smoke check and bench.py's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the HIP library, and the HIP
 * library never calls it.
 *
 * Conventions (torch layout): a weight W is m x n row-major (y = W x, m = outputs, n = inputs).
 * Activations X are N x n row-major with leading dimension ldx (token t is row t).  The input axis
 * is cut into B = n / nb contiguous blocks; block b owns columns [b*nb, (b+1)*nb).  Every per-block
 * matrix (A_b, Q_b) is nb x nb row-major, stored block after block.  Q_b holds eigenvectors as
 * COLUMNS: Q_b[p*nb + j] is component p of eigenvector j.
 *
 * All arithmetic is double precision.  Inputs given in fp32/bf16 are widened exactly by the caller.
 * No blocking, fusion or reordering beyond what each definition states.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------------
 * Block-diagonal second moment with EMA.
 * Abstract: Dobb approximates the input-activation second moment with diagonal blocks.  Figure 2
 * caption: second moments are averaged over accumulated mini-batches, so each capture contributes
 * the mean (1/N) sum_t x_t x_t^T.  EMA across captures:  A_b <- beta*A_b + (1-beta) * S_b / N,
 * S_b = sum_t x_{t,b} x_{t,b}^T  (x_{t,b} = the nb entries of token t inside block b).
 * ---------------------------------------------------------------------------------------------- */
void oracle_accumulate(long N, long n, long nb, long ldx, const double *X, double beta, double *A)
{
    long B = n / nb;
    double *S = (double *)malloc(sizeof(double) * nb * nb);
    for (long b = 0; b < B; ++b) {
        memset(S, 0, sizeof(double) * nb * nb);
        for (long t = 0; t < N; ++t) {
            const double *x = X + t * ldx + b * nb;
            for (long p = 0; p < nb; ++p)
                for (long q = 0; q < nb; ++q)
                    S[p * nb + q] += x[p] * x[q];
        }
        double *Ab = A + b * nb * nb;
        for (long i = 0; i < nb * nb; ++i)
            Ab[i] = beta * Ab[i] + (1.0 - beta) * (S[i] / (double)N);
    }
    free(S);
}

/* Sort eigenpairs by descending eigenvalue (ties keep the lower original index first), then give
 * every eigenvector the sign that makes its largest-magnitude entry positive (ties in magnitude go
 * to the lowest row index).  Neither choice changes the Dobb update (a signed permutation of the
 * basis permutes and flips C's columns consistently), it only makes Q and lambda comparable. */
static void sort_and_normalise(long n, double *lam, double *V /* n x n, columns */)
{
    long *order = (long *)malloc(sizeof(long) * n);
    for (long i = 0; i < n; ++i) order[i] = i;
    /* insertion sort: stable, O(n^2), plain */
    for (long i = 1; i < n; ++i) {
        long k = order[i];
        long j = i - 1;
        while (j >= 0 && lam[order[j]] < lam[k]) { order[j + 1] = order[j]; --j; }
        order[j + 1] = k;
    }
    double *lam2 = (double *)malloc(sizeof(double) * n);
    double *V2 = (double *)malloc(sizeof(double) * n * n);
    for (long j = 0; j < n; ++j) {
        long src = order[j];
        lam2[j] = lam[src];
        long arg = 0;
        double best = -1.0;
        for (long p = 0; p < n; ++p) {
            double a = fabs(V[p * n + src]);
            if (a > best) { best = a; arg = p; }
        }
        double sgn = (V[arg * n + src] < 0.0) ? -1.0 : 1.0;
        for (long p = 0; p < n; ++p) V2[p * n + j] = sgn * V[p * n + src];
    }
    memcpy(lam, lam2, sizeof(double) * n);
    memcpy(V, V2, sizeof(double) * n * n);
    free(order); free(lam2); free(V2);
}

/* ------------------------------------------------------------------------------------------------
 * Exact eigendecomposition of one symmetric block (the "Exact eigendecomposition" refresh row of
 * Table 15).  Cyclic Jacobi, row-by-row ordering, with the symmetric 2x2 Schur rotation of the
 * textbook (Golub & Van Loan, symmetric Jacobi):
 *     theta = (a_qq - a_pp) / (2 a_pq),  t = sgn(theta) / (|theta| + sqrt(1 + theta^2)),
 *     c = 1/sqrt(1+t^2),  s = t c,   A <- J^T A J,  V <- V J,
 * with J the identity except J_pp = J_qq = c, J_pq = s, J_qp = -s.
 * Warm start (used by the refresh when a previous basis exists): pass V0 = Q_prev; the rotations
 * are then applied to  Q_prev^T A Q_prev  and accumulated onto Q_prev.
 * Stops when off(A) <= tol * ||A||_F.  Returns the number of sweeps used, or -1 if max_sweeps was
 * reached first.  On return lam is sorted descending and V's columns are sign-normalised.
 * ---------------------------------------------------------------------------------------------- */
int oracle_jacobi_eig(long n, const double *Ain, const double *V0, double *lam, double *V,
                      int max_sweeps, double tol)
{
    double *A = (double *)malloc(sizeof(double) * n * n);
    if (V0) {
        /* A := V0^T Ain V0 */
        double *T = (double *)calloc(n * n, sizeof(double));
        for (long i = 0; i < n; ++i)
            for (long k = 0; k < n; ++k)
                for (long j = 0; j < n; ++j)
                    T[i * n + j] += Ain[i * n + k] * V0[k * n + j];
        memset(A, 0, sizeof(double) * n * n);
        for (long i = 0; i < n; ++i)
            for (long k = 0; k < n; ++k)
                for (long j = 0; j < n; ++j)
                    A[i * n + j] += V0[k * n + i] * T[k * n + j];
        free(T);
        memcpy(V, V0, sizeof(double) * n * n);
    } else {
        memcpy(A, Ain, sizeof(double) * n * n);
        memset(V, 0, sizeof(double) * n * n);
        for (long i = 0; i < n; ++i) V[i * n + i] = 1.0;
    }
    double fro2 = 0.0;
    for (long i = 0; i < n * n; ++i) fro2 += A[i] * A[i];
    double fro = sqrt(fro2);

    int used = -1;
    for (int sweep = 0; sweep <= max_sweeps; ++sweep) {
        double off2 = 0.0;
        for (long p = 0; p < n; ++p)
            for (long q = 0; q < n; ++q)
                if (p != q) off2 += A[p * n + q] * A[p * n + q];
        if (sqrt(off2) <= tol * fro) { used = sweep; break; }
        if (sweep == max_sweeps) break;
        for (long p = 0; p < n - 1; ++p) {
            for (long q = p + 1; q < n; ++q) {
                double apq = A[p * n + q];
                if (apq == 0.0) continue;
                double app = A[p * n + p], aqq = A[q * n + q];
                double theta = (aqq - app) / (2.0 * apq);
                double t;
                if (fabs(theta) > 1e150) t = 0.5 / theta;
                else t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(1.0 + theta * theta));
                double c = 1.0 / sqrt(1.0 + t * t);
                double s = t * c;
                /* columns p, q of A (A J) */
                for (long k = 0; k < n; ++k) {
                    double akp = A[k * n + p], akq = A[k * n + q];
                    A[k * n + p] = c * akp - s * akq;
                    A[k * n + q] = s * akp + c * akq;
                }
                /* rows p, q (J^T (A J)) */
                for (long k = 0; k < n; ++k) {
                    double apk = A[p * n + k], aqk = A[q * n + k];
                    A[p * n + k] = c * apk - s * aqk;
                    A[q * n + k] = s * apk + c * aqk;
                }
                /* the textbook's accurate diagonal and the exact zero */
                A[p * n + p] = app - t * apq;
                A[q * n + q] = aqq + t * apq;
                A[p * n + q] = 0.0;
                A[q * n + p] = 0.0;
                for (long k = 0; k < n; ++k) {
                    double vkp = V[k * n + p], vkq = V[k * n + q];
                    V[k * n + p] = c * vkp - s * vkq;
                    V[k * n + q] = s * vkp + c * vkq;
                }
            }
        }
    }
    for (long i = 0; i < n; ++i) lam[i] = A[i * n + i];
    free(A);
    sort_and_normalise(n, lam, V);
    return used;
}

/* ------------------------------------------------------------------------------------------------
 * Householder QR of a square n x n matrix Z (Table 16: Householder is the principal QR routine).
 * Returns the orthonormal factor Q with the unique sign convention diag(R) > 0.
 * Reflector j: v = x + sgn(x_0) ||x|| e_0 (sgn(0) = +1),  H_j = I - (2 / v^T v) v v^T, applied to the
 * trailing rows; Q = H_0 H_1 ... H_{n-1}, formed by applying the reflectors to I from the last to
 * the first.  Columns of Q are then flipped where R_jj < 0.
 * ---------------------------------------------------------------------------------------------- */
void oracle_householder_qr(long n, const double *Z, double *Q)
{
    double *R = (double *)malloc(sizeof(double) * n * n);
    double *Vh = (double *)calloc(n * n, sizeof(double)); /* reflector j stored in column j */
    double *beta = (double *)calloc(n, sizeof(double));
    double *rdiag = (double *)malloc(sizeof(double) * n);
    double *w = (double *)malloc(sizeof(double) * n);
    memcpy(R, Z, sizeof(double) * n * n);
    for (long j = 0; j < n; ++j) {
        double norm2 = 0.0;
        for (long i = j; i < n; ++i) norm2 += R[i * n + j] * R[i * n + j];
        double alpha = sqrt(norm2);
        if (alpha == 0.0) { beta[j] = 0.0; rdiag[j] = 0.0; continue; }
        double x0 = R[j * n + j];
        double sg = (x0 >= 0.0) ? 1.0 : -1.0;
        for (long i = j; i < n; ++i) Vh[i * n + j] = R[i * n + j];
        Vh[j * n + j] += sg * alpha;
        double vtv = 0.0;
        for (long i = j; i < n; ++i) vtv += Vh[i * n + j] * Vh[i * n + j];
        beta[j] = 2.0 / vtv;
        /* R[j:, j:] -= beta v (v^T R[j:, j:]) */
        for (long k = j; k < n; ++k) {
            double s = 0.0;
            for (long i = j; i < n; ++i) s += Vh[i * n + j] * R[i * n + k];
            w[k] = s;
        }
        for (long i = j; i < n; ++i)
            for (long k = j; k < n; ++k)
                R[i * n + k] -= beta[j] * Vh[i * n + j] * w[k];
        rdiag[j] = -sg * alpha;
    }
    /* Q = H_0 ... H_{n-1} I */
    memset(Q, 0, sizeof(double) * n * n);
    for (long i = 0; i < n; ++i) Q[i * n + i] = 1.0;
    for (long j = n - 1; j >= 0; --j) {
        if (beta[j] == 0.0) continue;
        for (long k = 0; k < n; ++k) {
            double s = 0.0;
            for (long i = j; i < n; ++i) s += Vh[i * n + j] * Q[i * n + k];
            w[k] = s;
        }
        for (long i = j; i < n; ++i)
            for (long k = 0; k < n; ++k)
                Q[i * n + k] -= beta[j] * Vh[i * n + j] * w[k];
    }
    for (long j = 0; j < n; ++j)
        if (rdiag[j] < 0.0)
            for (long i = 0; i < n; ++i) Q[i * n + j] = -Q[i * n + j];
    free(R); free(Vh); free(beta); free(rdiag); free(w);
}

/* ------------------------------------------------------------------------------------------------
 * Orthogonal-iteration refresh of one block (Table 15, "k=1 (principal)", k = 2, 3): starting from
 * the previous basis, k times:  Z = A_b Q ;  Q <- qr(Z).Q  (Householder, diag(R) > 0).
 * No Rayleigh-Ritz rotation: column order is inherited from the previous basis.  lam_out, if given,
 * receives the Rayleigh quotients q_j^T A_b q_j of the new basis (reporting only).
 * ---------------------------------------------------------------------------------------------- */
void oracle_orth_iter(long n, const double *A, const double *Qprev, int k, double *Q, double *lam_out)
{
    double *Z = (double *)malloc(sizeof(double) * n * n);
    memcpy(Q, Qprev, sizeof(double) * n * n);
    for (int it = 0; it < k; ++it) {
        memset(Z, 0, sizeof(double) * n * n);
        for (long i = 0; i < n; ++i)
            for (long l = 0; l < n; ++l)
                for (long j = 0; j < n; ++j)
                    Z[i * n + j] += A[i * n + l] * Q[l * n + j];
        oracle_householder_qr(n, Z, Q);
    }
    if (lam_out) {
        for (long j = 0; j < n; ++j) {
            double s = 0.0;
            for (long p = 0; p < n; ++p) {
                double aq = 0.0;
                for (long q = 0; q < n; ++q) aq += A[p * n + q] * Q[q * n + j];
                s += Q[p * n + j] * aq;
            }
            lam_out[j] = s;
        }
    }
    free(Z);
}

/* ------------------------------------------------------------------------------------------------
 * The Dobb step on one m x n weight (abstract; Table 9; Table 19; Table 21 note on decoupled weight
 * decay):
 *   M <- mu M + G                                   (heavy-ball momentum)
 *   M_eff = M, or G + mu M with Nesterov             (Table 19 ablation; off in the principal run)
 *   for each block b:  C_b = M_eff[:, block b] Q_b   (project into the block eigenbasis)
 *                      S_b = sign(C_b)               (norm 0: sign, sign(0) = 0, NaN stays NaN)
 *                          = C_b                     (norm 1: identity -- a test mode, U = M Q Q^T)
 *                          = C_b diag(1/||c_j||)     (norm 2: column l2, the Dobb-l2 ablation)
 *                      U_b = S_b Q_b^T               (reconstruct)
 *   W <- W - lr (s_eff U + wd W)                     (decoupled weight decay, both terms on old W)
 * s_eff is the applied scale: Table 9 gives raw ||O||_F^2 = n for Dobb (O = U / sqrt(m) for sign)
 * and s = tau sqrt(max(m,n)), so s_eff = tau sqrt(max(m,n)/m) for sign; the caller passes it.
 * U (m x n) receives the reconstruction if non-NULL.
 * ---------------------------------------------------------------------------------------------- */
void oracle_step(long m, long n, long nb, double *W, const double *G, double *M, const double *Q,
                 double lr, double wd, double mu, double s_eff, int nesterov, int norm, double *U)
{
    long B = n / nb;
    double *Meff = (double *)malloc(sizeof(double) * m * n);
    double *Uall = (double *)malloc(sizeof(double) * m * n);
    double *C = (double *)malloc(sizeof(double) * m * nb);
    for (long i = 0; i < m * n; ++i) {
        M[i] = mu * M[i] + G[i];
        Meff[i] = nesterov ? G[i] + mu * M[i] : M[i];
    }
    for (long b = 0; b < B; ++b) {
        const double *Qb = Q + b * nb * nb;
        for (long r = 0; r < m; ++r)
            for (long j = 0; j < nb; ++j) {
                double s = 0.0;
                for (long k = 0; k < nb; ++k) s += Meff[r * n + b * nb + k] * Qb[k * nb + j];
                C[r * nb + j] = s;
            }
        if (norm == 0) {
            for (long i = 0; i < m * nb; ++i) {
                double c = C[i];
                C[i] = (c > 0.0) ? 1.0 : (c < 0.0) ? -1.0 : (c == 0.0) ? 0.0 : c; /* NaN stays */
            }
        } else if (norm == 2) {
            for (long j = 0; j < nb; ++j) {
                double s = 0.0;
                for (long r = 0; r < m; ++r) s += C[r * nb + j] * C[r * nb + j];
                double inv = (s > 0.0) ? 1.0 / sqrt(s) : 0.0;
                for (long r = 0; r < m; ++r) C[r * nb + j] *= inv;
            }
        }
        for (long r = 0; r < m; ++r)
            for (long p = 0; p < nb; ++p) {
                double s = 0.0;
                for (long j = 0; j < nb; ++j) s += C[r * nb + j] * Qb[p * nb + j];
                Uall[r * n + b * nb + p] = s;
            }
    }
    for (long i = 0; i < m * n; ++i)
        W[i] = W[i] - lr * (s_eff * Uall[i] + wd * W[i]);
    if (U) memcpy(U, Uall, sizeof(double) * m * n);
    free(Meff); free(Uall); free(C);
}

/* ------------------------------------------------------------------------------------------------
 * The Dobb-G step (Tables 12-13: the basis comes from the output-gradient second moment instead of
 * the input-activation one; Figure 2 caption: that moment is m x m; Table 7: with each block inside
 * one shard, Dobb-G needs no cross-shard payload, and Dobb-G-l2's normalisation reduces along the
 * input axis, O(m) scalars when that axis is sharded).  Blocks are nb consecutive ROWS of the weight
 * (output units); P holds B = m / nb consecutive nb x nb bases, eigenvectors as columns.
 *   M <- mu M + G;  M_eff = M, or G + mu M with Nesterov (as in oracle_step)
 *   for each block b (rows [b nb, (b+1) nb)):
 *       C_b = P_b^T M_eff[rows of b, :]             (nb x n: coefficients of every column)
 *       S_b = sign(C_b)                              (norm 0; sign(0) = 0, NaN stays NaN)
 *           = C_b                                    (norm 1: identity -- U = P P^T M = M)
 *           = diag(1/||c_i||) C_b                    (norm 2: each row of C_b over the n columns,
 *                                                     Dobb-G-l2)
 *       U[rows of b, :] = P_b S_b                    (reconstruct)
 *   W <- W - lr (s_eff U + wd W)
 * Table 9's Dobb-G row: raw ||O||_F^2 = m and RMS(s O) = tau sqrt(max(m,n)/n), so for sign (whose
 * ||U||_F^2 = m n) O = U / sqrt(n) and s_eff = tau sqrt(max(m,n)/n); the caller passes s_eff.
 * ---------------------------------------------------------------------------------------------- */
void oracle_step_g(long m, long n, long nb, double *W, const double *G, double *M, const double *P,
                   double lr, double wd, double mu, double s_eff, int nesterov, int norm, double *U)
{
    long B = m / nb;
    double *Meff = (double *)malloc(sizeof(double) * m * n);
    double *Uall = (double *)malloc(sizeof(double) * m * n);
    double *C = (double *)malloc(sizeof(double) * nb * n);
    for (long i = 0; i < m * n; ++i) {
        M[i] = mu * M[i] + G[i];
        Meff[i] = nesterov ? G[i] + mu * M[i] : M[i];
    }
    for (long b = 0; b < B; ++b) {
        const double *Pb = P + b * nb * nb;
        const double *Mb = Meff + b * nb * n;
        for (long i = 0; i < nb; ++i)
            for (long c = 0; c < n; ++c) {
                double s = 0.0;
                for (long p = 0; p < nb; ++p) s += Pb[p * nb + i] * Mb[p * n + c];
                C[i * n + c] = s;
            }
        if (norm == 0) {
            for (long e = 0; e < nb * n; ++e) {
                double c = C[e];
                C[e] = (c > 0.0) ? 1.0 : (c < 0.0) ? -1.0 : (c == 0.0) ? 0.0 : c; /* NaN stays */
            }
        } else if (norm == 2) {
            for (long i = 0; i < nb; ++i) {
                double s = 0.0;
                for (long c = 0; c < n; ++c) s += C[i * n + c] * C[i * n + c];
                double inv = (s > 0.0) ? 1.0 / sqrt(s) : 0.0;
                for (long c = 0; c < n; ++c) C[i * n + c] *= inv;
            }
        }
        for (long p = 0; p < nb; ++p)
            for (long c = 0; c < n; ++c) {
                double s = 0.0;
                for (long i = 0; i < nb; ++i) s += Pb[p * nb + i] * C[i * n + c];
                Uall[(b * nb + p) * n + c] = s;
            }
    }
    for (long i = 0; i < m * n; ++i)
        W[i] = W[i] - lr * (s_eff * Uall[i] + wd * W[i]);
    if (U) memcpy(U, Uall, sizeof(double) * m * n);
    free(Meff); free(Uall); free(C);
}

/* ------------------------------------------------------------------------------------------------
 * Cholesky QR of a square n x n matrix Z (Table 16: "Cholesky" is the faster QR routine of the
 * orthogonal-iteration refresh, next to the principal Householder).  Reading: CholeskyQR2, i.e. two
 * passes of
 *     G = Z^T Z,   G = R^T R (Cholesky, R upper triangular with a positive diagonal),   Z <- Z R^{-1};
 * in exact arithmetic the second pass has R = I, in floating point it restores the orthogonality
 * the first one loses (about cond(Z)^2 u).  The result is the orthonormal factor of the QR with
 * diag(R) > 0 (R = R_2 R_1): the same factor as oracle_householder_qr.  Returns 0, or -1 if a pivot
 * was not positive (Z numerically rank deficient), in which case Q is left undefined.
 * ---------------------------------------------------------------------------------------------- */
int oracle_cholesky_qr2(long n, const double *Z, double *Q)
{
    double *X = (double *)malloc(sizeof(double) * n * n);
    double *G = (double *)malloc(sizeof(double) * n * n);
    int status = 0;
    memcpy(X, Z, sizeof(double) * n * n);
    for (int pass = 0; pass < 2 && status == 0; ++pass) {
        /* G = X^T X */
        for (long i = 0; i < n; ++i)
            for (long j = 0; j < n; ++j) {
                double s = 0.0;
                for (long k = 0; k < n; ++k) s += X[k * n + i] * X[k * n + j];
                G[i * n + j] = s;
            }
        /* Cholesky, row by row: R[i][i] = sqrt(G_ii - sum_k R_ki^2), R[i][j] = (G_ij - sum_k R_ki R_kj) / R_ii;
           R overwrites the upper triangle of G */
        for (long i = 0; i < n && status == 0; ++i) {
            double d = G[i * n + i];
            for (long k = 0; k < i; ++k) d -= G[k * n + i] * G[k * n + i];
            if (!(d > 0.0)) { status = -1; break; }
            double rii = sqrt(d);
            G[i * n + i] = rii;
            for (long j = i + 1; j < n; ++j) {
                double s = G[i * n + j];
                for (long k = 0; k < i; ++k) s -= G[k * n + i] * G[k * n + j];
                G[i * n + j] = s / rii;
            }
        }
        if (status) break;
        /* X <- X R^{-1}: each row x solves y R = x by forward substitution along the columns */
        for (long r = 0; r < n; ++r) {
            double *x = X + r * n;
            for (long j = 0; j < n; ++j) {
                double s = x[j];
                for (long k = 0; k < j; ++k) s -= x[k] * G[k * n + j];
                x[j] = s / G[j * n + j];
            }
        }
    }
    memcpy(Q, X, sizeof(double) * n * n);
    free(X); free(G);
    return status;
}

/* Orthogonal-iteration refresh with the Cholesky QR routine (Table 16): as oracle_orth_iter, with
 * Q <- CholeskyQR2(A_b Q).  Returns 0, or -1 if a Cholesky pivot failed. */
int oracle_orth_iter_cholqr2(long n, const double *A, const double *Qprev, int k, double *Q, double *lam_out)
{
    double *Z = (double *)malloc(sizeof(double) * n * n);
    int status = 0;
    memcpy(Q, Qprev, sizeof(double) * n * n);
    for (int it = 0; it < k && status == 0; ++it) {
        memset(Z, 0, sizeof(double) * n * n);
        for (long i = 0; i < n; ++i)
            for (long l = 0; l < n; ++l)
                for (long j = 0; j < n; ++j)
                    Z[i * n + j] += A[i * n + l] * Q[l * n + j];
        status = oracle_cholesky_qr2(n, Z, Q);
    }
    if (lam_out && status == 0) {
        for (long j = 0; j < n; ++j) {
            double s = 0.0;
            for (long p = 0; p < n; ++p) {
                double aq = 0.0;
                for (long q = 0; q < n; ++q) aq += A[p * n + q] * Q[q * n + j];
                s += Q[p * n + j] * aq;
            }
            lam_out[j] = s;
        }
    }
    free(Z);
    return status;
}
