/*
 * dobb.h -- C ABI of libdobb.so, the MI355X (gfx950) implementation of the Dobb optimizer step
 * described in "Dobb: Shard-Local Preconditioning in Block-Diagonal Eigenbases" (arXiv 2610.39412).
 *
 * For each weight W (m x n, y = W x) the step keeps, per contiguous block b of nb input columns:
 *   A_b  the nb x nb block of the input-activation second moment, as an EMA   (abstract)
 *   Q_b  a complete orthonormal eigenbasis of A_b, refreshed periodically      (abstract; Tables 14-16)
 * and applies  U_b = sign(M_b Q_b) Q_b^T,  W <- W - lr (s U + wd W)              (abstract; Table 9)
 * with M the heavy-ball momentum of the gradient.
 *
 * Conventions shared by every call
 *   Layout    torch layout.  W, G, M, U are m x n row-major (leading dimension n).  Activations X are
 *             N x n row-major with leading dimension ldx >= n (token t is row t).  Block b covers
 *             columns [b*nb, (b+1)*nb); B = n / nb.  A, Q are B consecutive nb x nb row-major
 *             matrices; Q_b holds eigenvectors as COLUMNS (Q_b[p*nb + j] = entry p of vector j).
 *             lambda is B x nb.
 *   Memory    Every data pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA tensor's storage),
 *             owned by the caller.  The library never allocates, frees or keeps any of it.  Scratch
 *             memory is the caller's workspace `ws` of at least dobb_workspace_size(...) bytes,
 *             256-byte aligned; its contents are undefined after a call.
 *   Streams   All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the null
 *             stream).  No call synchronizes the device.  Results are bitwise reproducible for fixed
 *             inputs, shapes and device (no floating-point atomics).
 *   Errors    Arguments are validated on the host BEFORE anything is enqueued; on any error nothing is
 *             launched and the status says why.  DOBB_ERR_HIP reports a failed launch.  Convergence of
 *             the eigensolver is reported per block in the device array `info`, never as a status.
 *             NaN/Inf inputs are not checked; they propagate (sign(NaN) = NaN).
 *   Threads   The library keeps no mutable global state except the optional kernel timer
 *             (dobb_profile_*), which is not thread-safe, and the per-GPU scratch array of
 *             dobb_step_noalloc.  Calls that share a workspace or outputs must be ordered by the
 *             caller.
 */
#ifndef DOBB_H
#define DOBB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DOBB_ABI_VERSION 2

struct ihipStream_t;
typedef struct ihipStream_t *dobb_stream_t; /* the same type as hipStream_t */

typedef enum {
    DOBB_OK = 0,
    DOBB_ERR_INVALID_ARG = -1,   /* NULL pointer, bad enum, beta outside [0,1), N < 1, ... */
    DOBB_ERR_SHAPE = -2,         /* m, n or nb < 1, n % nb != 0, ldx < n, nb too large */
    DOBB_ERR_DTYPE = -3,         /* dtype not supported for that argument */
    DOBB_ERR_WORKSPACE = -4,     /* ws is NULL, misaligned or smaller than dobb_workspace_size */
    DOBB_ERR_HIP = -5,           /* a HIP launch or query failed (no device, bad pointer, ...) */
    DOBB_ERR_NOT_CONVERGED = -6  /* reserved for host-side checks; device results go to info[] */
} dobb_status;

typedef enum { DOBB_F32 = 0, DOBB_BF16 = 1 } dobb_dtype;

typedef enum {
    DOBB_REFRESH_EXACT = 0,      /* Table 15 "Exact eigendecomposition": cyclic Jacobi to tolerance */
    DOBB_REFRESH_ORTH_ITER = 1,  /* Table 15 "k=1 (principal)": k steps Q <- qr(A_b Q).Q, Householder */
    DOBB_REFRESH_ORTH_ITER_CHOLQR = 2  /* Table 16 "Cholesky": the same steps with Cholesky QR */
} dobb_refresh_mode;

typedef enum {
    DOBB_NORM_SIGN = 0,          /* abstract / Table 13: sign normalization of the coefficients */
    DOBB_NORM_IDENTITY = 1,      /* no normalization: U = M Q Q^T (= M); a round-trip test mode */
    DOBB_NORM_COL_L2 = 2         /* Tables 11-12 "Dobb-l2": unit l2 norm per column of C_b */
} dobb_norm;

typedef enum { DOBB_OP_ACCUMULATE = 0, DOBB_OP_REFRESH = 1, DOBB_OP_STEP = 2, DOBB_OP_STEP_G = 3 } dobb_op;

typedef struct {
    int64_t m;   /* output dimension (rows of W) */
    int64_t n;   /* input dimension (columns of W); n % nb == 0 */
    int64_t nb;  /* block width; B = n / nb blocks (1 <= nb <= 1024) */
} dobb_shape;

typedef struct {
    float lr;            /* gamma: W <- W - lr (update_scale * U + weight_decay * W) */
    float weight_decay;  /* lambda (decoupled; uses the weights before the update) */
    float momentum;      /* mu: M <- mu M + G */
    float update_scale;  /* applied scale s_eff on U; tau sqrt(max(m,n)/m) reproduces Table 9's
                            RMS for sign (tau = 0.2 for GPT-2); for COL_L2 Table 9's s = tau sqrt(max(m,n)) */
    int32_t nesterov;    /* 0: project M;  1: project G + mu M (Table 19 ablation) */
    int32_t norm;        /* a dobb_norm */
} dobb_hparams;

/* Bytes of workspace the op needs for `count` matrices of the given shapes.  N (tokens per capture)
 * is used by DOBB_OP_ACCUMULATE only.  For DOBB_OP_STEP, variant is the dobb_norm (sign needs about
 * 1 byte per weight entry, the other norms 4); for DOBB_OP_STEP and DOBB_OP_REFRESH, adding
 * DOBB_WS_BF16_BASIS to variant sizes the call for a bf16 basis (an fp32 copy of each basis in the
 * workspace).  The refresh figure covers every mode.  Returns 0 for bad arguments and for an op that
 * needs no scratch. */
#define DOBB_WS_BF16_BASIS 16
size_t dobb_workspace_size(dobb_op op, int count, const dobb_shape *shapes, int64_t N, int32_t variant);

/* ------------------------------------------------------------------------------------------------
 * Second-moment capture (abstract: input-activation second moment approximated by diagonal blocks;
 * Figure 2 caption: averaged over accumulated mini-batches; Table 17: capture policy is the caller's).
 *   A_b <- beta * A_b + (1 - beta) * (1/N) * sum_t x_{t,b} x_{t,b}^T,   for every block b.
 * X: device, N x n (ldx >= n), fp32 or bf16.  A: device fp32 B x nb x nb, read (when beta > 0) and
 * written in place; the result is exactly symmetric.  0 <= beta < 1 (beta = 0: pure capture, A need
 * not be initialised).  Products are formed in fp32 (exact for bf16), summed in fp32 over at most 64
 * tokens and across those chunks in fp64, so A is close to correctly rounded.
 * -------------------------------------------------------------------------------------------------*/
dobb_status dobb_accumulate_moment(const dobb_shape *s, const void *X, dobb_dtype x_dtype, int64_t N,
                                   int64_t ldx, float beta, float *A, void *ws, size_t ws_bytes,
                                   dobb_stream_t stream);

/* ------------------------------------------------------------------------------------------------
 * Basis refresh (abstract: a complete basis is tracked within each block; Tables 14-16).
 *   EXACT:     Q_b, lambda_b = eig(A_b) by parallel-order cyclic Jacobi: sweeps on an fp32 working
 *              matrix, then fp64 sweeps on V^T A_b V to |a_pq| <= 1e-14 sqrt(|a_pp a_qq|).  Blocks
 *              whose fp32 working matrix exceeds the LDS (nb above about 200) run block Jacobi in
 *              fp64 from the start (index blocks of up to 40 paired by the circle method, one sweep
 *              of each pair's sub-problem per round) to that same threshold.  warm_start = 0 starts
 *              from the identity; warm_start = 1 diagonalises Q_prev^T A_b Q_prev and accumulates
 *              the rotations onto Q_prev.  iters = maximum sweeps of the first stage (<= 0: 30).
 *              tol is the first stage's relative threshold: a pair (p,q) is rotated while
 *              |a_pq| > tol sqrt(|a_pp a_qq|) (<= 0: 1e-7); a stage has converged after a sweep with
 *              no rotation, and info is -1 unless both have.  Output is sorted by descending
 *              eigenvalue, each eigenvector with its largest entry positive.
 *   ORTH_ITER: iters = k >= 1 steps of  Q_b <- qr(A_b Q_b).Q  (Householder, diag(R) > 0) from the
 *              Q passed in (which must hold a basis); lambda_b receives the Rayleigh quotients
 *              q_j^T A_b q_j.  warm_start and tol are ignored.
 *   ORTH_ITER_CHOLQR: the same iteration with the QR by Cholesky (Table 16): two passes of
 *              G = Z^T Z = R^T R, Z <- Z R^{-1} (fp32), the same factor with diag(R) > 0.  A block whose
 *              Gram matrix is not numerically positive definite (Z rank deficient) gets info = -1 and
 *              an unspecified basis.  nb is limited by the LDS (32 (nb + 1) + 3k floats per workgroup:
 *              nb <= 1024 on MI355X); wider blocks return DOBB_ERR_SHAPE.
 * A: device fp32 B x nb x nb (symmetric; only read).  Q: device B x nb x nb, in/out, stored as
 * q_dtype: DOBB_F32, or DOBB_BF16 (Table 18's principal setting, fp32 moments with a bf16 basis: the
 * refresh reads the bf16 basis exactly, computes in fp32/fp64 as above and rounds the result to
 * nearest even once).  lambda: device fp32 B x nb or NULL.  info: device int32 [B] or NULL;
 * receives the sweeps used (EXACT, -1 if iters sweeps did not converge) or k (ORTH_ITER).
 * -------------------------------------------------------------------------------------------------*/
dobb_status dobb_refresh_basis(const dobb_shape *s, const float *A, void *Q, dobb_dtype q_dtype,
                               float *lambda, dobb_refresh_mode mode, int iters, int warm_start, float tol,
                               int32_t *info, void *ws, size_t ws_bytes, dobb_stream_t stream);

/* ------------------------------------------------------------------------------------------------
 * The Dobb step (abstract: project momentum into the block bases, sign-normalise the coefficients,
 * reconstruct; Table 9: update scale; Table 21 note: decoupled weight decay; Table 19: Nesterov).
 *   M <- mu M + G;   P = M (or G + mu M with nesterov);   C_b = P_b Q_b;
 *   U_b = sign(C_b) Q_b^T   (sign(0) = 0);   W <- W - lr (update_scale U + weight_decay W).
 * W: device m x n, fp32 or bf16 (bf16 is updated in fp32 and rounded to nearest even).
 * G: device m x n, fp32 or bf16.  M: device fp32 m x n, in/out.  Q: device B x nb x nb in q_dtype
 * (fp32, or bf16 as stored by dobb_refresh_basis; bf16 entries are used exactly).
 * hp: host pointer.  U_out: device fp32 m x n or NULL (receives U before scaling).
 * C_out: device fp32 m x n or NULL; receives the coefficients C_b = P_b Q_b of every block in block
 * b's columns, as the projection computed them before normalisation (for verification; writing
 * them adds 4 bytes per entry of traffic).
 * -------------------------------------------------------------------------------------------------*/
dobb_status dobb_step(const dobb_shape *s, void *W, dobb_dtype w_dtype, const void *G, dobb_dtype g_dtype,
                      float *M, const void *Q, dobb_dtype q_dtype, const dobb_hparams *hp, float *U_out,
                      float *C_out, void *ws, size_t ws_bytes, dobb_stream_t stream);

/* ------------------------------------------------------------------------------------------------
 * Grouped forms over a matrix set: the same semantics for `count` matrices, enqueued together.
 * shapes, the pointer arrays and hp are HOST arrays of length count whose entries are device
 * pointers (U_out and C_out may be NULL, or arrays with NULL entries; ldx may be NULL for ldx = n).
 * The workspace is sized by dobb_workspace_size(op, count, shapes, N, variant) and shared by the whole
 * group.  All hp entries of one dobb_step_grouped call must share norm and nesterov; all matrices of
 * a call share the dtypes given.
 * -------------------------------------------------------------------------------------------------*/
dobb_status dobb_accumulate_moment_grouped(int count, const dobb_shape *shapes, const void *const *X,
                                           dobb_dtype x_dtype, int64_t N, const int64_t *ldx, float beta,
                                           float *const *A, void *ws, size_t ws_bytes, dobb_stream_t stream);
dobb_status dobb_refresh_basis_grouped(int count, const dobb_shape *shapes, const float *const *A,
                                       void *const *Q, dobb_dtype q_dtype, float *const *lambda,
                                       dobb_refresh_mode mode, int iters, int warm_start, float tol,
                                       int32_t *const *info, void *ws, size_t ws_bytes, dobb_stream_t stream);
dobb_status dobb_step_grouped(int count, const dobb_shape *shapes, void *const *W, dobb_dtype w_dtype,
                              const void *const *G, dobb_dtype g_dtype, float *const *M,
                              const void *const *Q, dobb_dtype q_dtype, const dobb_hparams *hp,
                              float *const *U_out, float *const *C_out, void *ws, size_t ws_bytes,
                              dobb_stream_t stream);

/* ------------------------------------------------------------------------------------------------
 * The Dobb-G step (Tables 12-13: the basis of the output-gradient second moment; Figure 2 caption:
 * that moment is m x m; Table 7: blocks along the output axis, and Dobb-G-l2 normalises along the
 * input axis; Table 9: its update scale).  Blocks are nb consecutive ROWS: s = {m, n, nb} with
 * m % nb == 0 and B = m / nb.  P: device B x nb x nb in p_dtype (fp32 or bf16), the bases of the
 * blocks of the output-gradient moment: capture it with dobb_accumulate_moment on the output
 * gradients (N x m, shape {1, m, nb}) and refresh it with dobb_refresh_basis, unchanged.
 *   M <- mu M + G;  P_eff = M (or G + mu M);  C_b = P_b^T P_eff[rows of b, :]  (nb x n);
 *   U[rows of b, :] = P_b sign(C_b)   (IDENTITY: P_b C_b = M;  COL_L2: P_b diag(1/||c_i||) C_b with
 *   each row c_i of C_b normalised over the n columns: Dobb-G-l2);
 *   W <- W - lr (update_scale U + weight_decay W).
 * Table 9's Dobb-G row gives RMS tau sqrt(max(m,n)/n) for sign (update_scale = tau sqrt(max(m,n)/n))
 * and tau sqrt(max(m,n)) for Dobb-G-l2.  Other arguments, layouts and errors as dobb_step (C_out
 * receives C_b in the rows of block b); the workspace is dobb_workspace_size(DOBB_OP_STEP_G, ...).
 * -------------------------------------------------------------------------------------------------*/
dobb_status dobb_step_g(const dobb_shape *s, void *W, dobb_dtype w_dtype, const void *G, dobb_dtype g_dtype,
                        float *M, const void *P, dobb_dtype p_dtype, const dobb_hparams *hp, float *U_out,
                        float *C_out, void *ws, size_t ws_bytes, dobb_stream_t stream);
dobb_status dobb_step_g_grouped(int count, const dobb_shape *shapes, void *const *W, dobb_dtype w_dtype,
                                const void *const *G, dobb_dtype g_dtype, float *const *M, const void *const *P,
                                dobb_dtype p_dtype, const dobb_hparams *hp, float *const *U_out,
                                float *const *C_out, void *ws, size_t ws_bytes, dobb_stream_t stream);

/* ------------------------------------------------------------------------------------------------
 * The step without a workspace argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The same semantics and
 * kernels as dobb_step; the scratch is a static device array of DOBB_NOALLOC_SCRATCH_BYTES held by
 * the library on each GPU it runs on until the process ends (every matrix of the GPT-2 and 7B-style
 * sets fits with sign normalisation; column-l2 needs 4 bytes per weight entry).  A shape whose
 * workspace (dobb_workspace_size for this op and variant) exceeds it returns DOBB_ERR_WORKSPACE
 * before anything is enqueued.  The call allocates and frees nothing.  The device is the caller's
 * current HIP device, which must be the stream's.  Calls on one GPU share the array: calls that can
 * overlap on one GPU (different streams, different host threads) race and must be ordered by the
 * caller; calls in one stream are ordered by it.
 * -------------------------------------------------------------------------------------------------*/
#define DOBB_NOALLOC_SCRATCH_BYTES (64u << 20)
dobb_status dobb_step_noalloc(const dobb_shape *s, void *W, dobb_dtype w_dtype, const void *G, dobb_dtype g_dtype,
                              float *M, const void *Q, dobb_dtype q_dtype, const dobb_hparams *hp, float *U_out,
                              float *C_out, dobb_stream_t stream);

/* ------------------------------------------------------------------------------------------------
 * Kernel timer (tracing).  While enabled, every kernel the library enqueues is bracketed by a pair
 * of HIP events on its stream; dobb_profile_read synchronizes those events and returns, per kernel
 * name, the launch count and the summed duration in milliseconds.  Names are static strings.
 * Returns the number of distinct kernels (at most cap entries are written).  Not thread-safe.
 * -------------------------------------------------------------------------------------------------*/
void dobb_profile_enable(int on);
int dobb_profile_read(const char **names, int64_t *launches, double *total_ms, int cap);
void dobb_profile_reset(void);

const char *dobb_status_string(dobb_status st);
int dobb_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DOBB_H */
