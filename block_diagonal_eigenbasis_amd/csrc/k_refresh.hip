// Per-block eigenbasis refresh on gfx950.
//
// Dobb paper (arXiv 2610.39412): the abstract has Dobb track a complete basis within each diagonal
// block; Table 15 lists the refresh variants (orthogonal iteration with k = 1, 2, 3 steps, the k = 1
// principal, and an exact eigendecomposition), Table 16 the QR routine (Householder principal) and
// Table 14 the refresh period (a caller parameter).
//
// EXACT     parallel-order cyclic Jacobi.  One launch of k_jacobi_sweep per sweep: one workgroup per
//           block keeps the working matrix in LDS when it fits (nb <= 196) and in the workspace
//           otherwise; the nbp/2 disjoint pairs of each round-robin step are rotated together.  The
//           rotation tangents are computed in fp64, logged, and applied to an fp64 eigenvector
//           accumulator by k_jacobi_rotate_v, spread over many workgroups (rows of V are
//           independent).  k_jacobi_finalize sorts by descending eigenvalue, makes the largest entry
//           of every eigenvector positive and writes fp32 Q, lambda and info.
// ORTH_ITER k times: Z = A_b Q_b (MFMA), Q_b <- qr(Z).Q by Householder (k_householder, Z in LDS
//           when it fits), diag(R) > 0.  Rayleigh quotients go to lambda when requested.
#include "dobb_internal.h"

#include <math.h>

namespace dobb {
namespace {

// ---- batched nb x nb GEMM: C_b = op(A_b) B_b ------------------------------------------------
struct Opnd {
    const float *p[kMaxMats];  // block 0 of every matrix
    int64_t blk_stride;        // elements between consecutive blocks
    int64_t ld;
};
struct OutOpnd {
    float *p[kMaxMats];
    int64_t blk_stride;
    int64_t ld;
};

// grid.x = tiles * tiles * nblk * count
template <bool TRANS_A>
__global__ void __launch_bounds__(256) k_bgemm(int nb, int T, int nblk, Opnd A, Opnd B, OutOpnd C) {
    __shared__ GemmSmem sm;
    const int tile = blockIdx.x % (T * T);
    const int rest = blockIdx.x / (T * T);
    const int b = rest % nblk, mat = rest / nblk;
    const int i0 = (tile / T) * kBM, j0 = (tile % T) * kBN;
    const float *Ab = A.p[mat] + (int64_t)b * A.blk_stride;
    const float *Bb = B.p[mat] + (int64_t)b * B.blk_stride;
    LoadColsK<false> lb{Bb + j0, B.ld, nb - j0, nb};
    f32x16 acc;
    if (TRANS_A) {  // op(A)[i][k] = A[k][i]: already k-major
        LoadColsK<false> la{Ab + i0, A.ld, nb - i0, nb};
        acc = gemm_tile(nb, la, lb, sm);
    } else {
        LoadRowsT<false> la{Ab + (int64_t)i0 * A.ld, A.ld, nb - i0, nb};
        acc = gemm_tile(nb, la, lb, sm);
    }
    float *Cb = C.p[mat] + (int64_t)b * C.blk_stride;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wr = 32 * (w >> 1), wc = 32 * (w & 1);
    const int j = j0 + wc + acc_col(lane);
    if (j < nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + wr + acc_row(r, lane);
            if (i < nb) Cb[(int64_t)i * C.ld + j] = acc[r];
        }
    }
}

// ---- Jacobi ------------------------------------------------------------------------------------
// Round-robin (circle method) pairing of nbp (even) indices: step s, pair k.  Index nbp-1 is fixed;
// over nbp-1 steps every pair (p, q) meets exactly once and the pairs of one step are disjoint.
__device__ __forceinline__ void rr_pair(int nbp, int s, int k, int &p, int &q) {
    const int m = nbp - 1;
    int a, c;
    if (k == 0) { a = s % m; c = m; }
    else { a = (s + k) % m; c = (s - k + m) % m; }
    p = a < c ? a : c;
    q = a < c ? c : a;
}

struct JacTable {
    const float *A[kMaxMats];   // source A_b (cold start)
    const float *Qp[kMaxMats];  // previous basis (warm start)
};

// Aw = symmetric, zero-padded working matrix; V = I (cold) or Q_prev (warm, Aw already holds
// Q_prev^T A Q_prev in its upper triangle); state = 0.  grid.x = nblk * count, block 256.
__global__ void __launch_bounds__(256) k_jacobi_init(int nb, int nbp, int nblk, int warm, JacTable t, float *Aw_all,
                                                     double *V_all, int32_t *state_all) {
    const int g = blockIdx.x;
    const int b = g % nblk, mat = g / nblk;
    float *Aw = Aw_all + (int64_t)g * nbp * nbp;
    double *V = V_all + (int64_t)g * nb * nb;
    const float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const float *Qb = t.Qp[mat] + (int64_t)b * nb * nb;
    for (int64_t e = threadIdx.x; e < (int64_t)nbp * nbp; e += 256) {
        const int i = (int)(e / nbp), j = (int)(e % nbp);
        if (i >= nb || j >= nb) { Aw[e] = 0.f; continue; }
        if (warm) { if (i > j) Aw[e] = Aw[(int64_t)j * nbp + i]; }  // copy upper into lower only
        else Aw[e] = i <= j ? Ab[(int64_t)i * nb + j] : Ab[(int64_t)j * nb + i];
    }
    for (int64_t e = threadIdx.x; e < (int64_t)nb * nb; e += 256) {
        const int i = (int)(e / nb), j = (int)(e % nb);
        V[e] = warm ? (double)Qb[e] : (i == j ? 1.0 : 0.0);
    }
    if (threadIdx.x < 4) state_all[4 * g + threadIdx.x] = 0;
}

// One sweep over all nbp(nbp-1)/2 pairs on a working matrix of element type T (fp32 for the first
// stage, fp64 for the refinement stage); the arithmetic is fp64 either way.  state: [0] sweeps that
// rotated, [1] converged, [2] rotations in this sweep.  grid.x = blocks, block 512.
template <typename T, bool LDS>
__global__ void __launch_bounds__(512) k_jacobi_sweep(int nb, int nbp, float tol, T *Aw_all, double *tlog_all,
                                                      int32_t *state_all) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const int g = blockIdx.x;
    int32_t *st = state_all + 4 * g;
    if (st[1]) {                          // converged in an earlier sweep
        if (threadIdx.x == 0) st[2] = 0;
        return;
    }
    const int npair = nbp / 2;
    double *tsh = (double *)dsm;                          // npair tangents
    int *psh = (int *)(tsh + npair);                      // npair p indices
    int *qsh = psh + npair;                               // npair q indices
    int *nrot_sh = qsh + npair;
    T *Ag = Aw_all + (int64_t)g * nbp * nbp;
    T *A = LDS ? (T *)(dsm + (((size_t)npair * 16 + 4 + 15) / 16) * 16) : Ag;
    double *tl = tlog_all + (int64_t)g * (nbp - 1) * npair;
    const int tid = threadIdx.x, nth = blockDim.x;
    if (LDS) for (int64_t e = tid; e < (int64_t)nbp * nbp; e += nth) A[e] = Ag[e];
    if (tid == 0) *nrot_sh = 0;
    __syncthreads();
    int myrot = 0;
    const double dtol = (double)tol;
    for (int s = 0; s < nbp - 1; ++s) {
        for (int k = tid; k < npair; k += nth) {
            int p, q;
            rr_pair(nbp, s, k, p, q);
            double t = 0.0;
            if (q < nb) {
                const double app = A[(int64_t)p * nbp + p], aqq = A[(int64_t)q * nbp + q];
                const double apq = A[(int64_t)p * nbp + q];
                if (apq != 0.0 && fabs(apq) > dtol * sqrt(fabs(app * aqq))) {
                    const double theta = (aqq - app) / (2.0 * apq);
                    if (fabs(theta) > 1e150) t = 0.5 / theta;
                    else t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(1.0 + theta * theta));
                    ++myrot;
                }
            }
            tsh[k] = t; psh[k] = p; qsh[k] = q;
            tl[(int64_t)s * npair + k] = t;
        }
        __syncthreads();
        // A <- J^T A J, one 2x2 block per (ki <= kj); the transpose block is written from the same values
        for (int it = tid; it < npair * npair; it += nth) {
            const int ki = it / npair, kj = it % npair;
            if (ki > kj) continue;
            const double ti = tsh[ki], tj = tsh[kj];
            if (ti == 0.0 && tj == 0.0) continue;
            const int pi = psh[ki], qi = qsh[ki], pj = psh[kj], qj = qsh[kj];
            if (ki == kj) {
                const double app = A[(int64_t)pi * nbp + pi], aqq = A[(int64_t)qi * nbp + qi];
                const double apq = A[(int64_t)pi * nbp + qi];
                A[(int64_t)pi * nbp + pi] = (T)(app - ti * apq);
                A[(int64_t)qi * nbp + qi] = (T)(aqq + ti * apq);
                A[(int64_t)pi * nbp + qi] = (T)0;
                A[(int64_t)qi * nbp + pi] = (T)0;
            } else {
                const double ci = 1.0 / sqrt(1.0 + ti * ti), si = ti * ci;
                const double cj = 1.0 / sqrt(1.0 + tj * tj), sj = tj * cj;
                const double x00 = A[(int64_t)pi * nbp + pj], x01 = A[(int64_t)pi * nbp + qj];
                const double x10 = A[(int64_t)qi * nbp + pj], x11 = A[(int64_t)qi * nbp + qj];
                const double y00 = ci * x00 - si * x10, y01 = ci * x01 - si * x11;
                const double y10 = si * x00 + ci * x10, y11 = si * x01 + ci * x11;
                const T z00 = (T)(cj * y00 - sj * y01), z01 = (T)(sj * y00 + cj * y01);
                const T z10 = (T)(cj * y10 - sj * y11), z11 = (T)(sj * y10 + cj * y11);
                A[(int64_t)pi * nbp + pj] = z00; A[(int64_t)pi * nbp + qj] = z01;
                A[(int64_t)qi * nbp + pj] = z10; A[(int64_t)qi * nbp + qj] = z11;
                A[(int64_t)pj * nbp + pi] = z00; A[(int64_t)qj * nbp + pi] = z01;
                A[(int64_t)pj * nbp + qi] = z10; A[(int64_t)qj * nbp + qi] = z11;
            }
        }
        __syncthreads();
    }
    if (myrot) atomicAdd(nrot_sh, myrot);  // integer count: order-independent
    if (LDS) for (int64_t e = tid; e < (int64_t)nbp * nbp; e += nth) Ag[e] = A[e];
    __syncthreads();
    if (tid == 0) {
        const int nrot = *nrot_sh;
        st[2] = nrot;
        if (nrot == 0) st[1] = 1;
        else st[0] += 1;
    }
}

// Refinement stage: Aw64 = V^T A V in fp64 (A fp32 widened exactly, V the fp64 eigenvector
// accumulator), zero-padded to nbp; the converged flag is cleared so fp64 sweeps can start.
// Two launches of one kernel: pass 0 forms T64 = A V, pass 1 forms V^T T64.  grid = (tiles^2, blocks),
// 16 x 16 threads, one output entry each, 16-deep K chunks through LDS.
__global__ void __launch_bounds__(256) k_refine_gemm(int nb, int nbp, int nblk, int pass, JacTable t,
                                                     const double *V_all, double *T64_all, double *Aw64_all,
                                                     int32_t *state_all) {
    __shared__ double as[16][17], bs[16][17];
    const int tiles = (nb + 15) / 16;
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    const int ti = blockIdx.x / tiles, tj = blockIdx.x % tiles;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int i = ti * 16 + ty, j = tj * 16 + tx;
    const double *V = V_all + (int64_t)g * nb * nb;
    const float *A = t.A[mat] + (int64_t)b * nb * nb;
    double *T64 = T64_all + (int64_t)g * nb * nb;
    double acc = 0.0;
    for (int k0 = 0; k0 < nb; k0 += 16) {
        const int ka = k0 + tx, kb = k0 + ty;
        // pass 0: lhs = A (row i), rhs = V;  pass 1: lhs = V^T (row i = column i of V), rhs = T64
        double l = 0.0, r = 0.0;
        if (i < nb && ka < nb) l = pass == 0 ? (double)A[(int64_t)i * nb + ka] : V[(int64_t)ka * nb + i];
        if (kb < nb && j < nb) r = pass == 0 ? V[(int64_t)kb * nb + j] : T64[(int64_t)kb * nb + j];
        as[ty][tx] = l;
        bs[ty][tx] = r;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) acc += as[ty][k] * bs[k][tx];
        __syncthreads();
    }
    if (pass == 0) {
        if (i < nb && j < nb) T64[(int64_t)i * nb + j] = acc;
    } else {
        double *Aw = Aw64_all + (int64_t)g * nbp * nbp;
        if (i < nbp && j < nbp) Aw[(int64_t)i * nbp + j] = (i < nb && j < nb) ? acc : 0.0;
        if (blockIdx.x == 0 && threadIdx.x == 0) state_all[4 * g + 1] = 0;
    }
}

// symmetrise the refined matrix from its upper triangle (the two GEMM orders differ in rounding)
__global__ void __launch_bounds__(256) k_symmetrize64(int nbp, double *Aw64_all) {
    double *Aw = Aw64_all + (int64_t)blockIdx.x * nbp * nbp;
    for (int64_t e = threadIdx.x; e < (int64_t)nbp * nbp; e += 256) {
        const int i = (int)(e / nbp), j = (int)(e % nbp);
        if (i > j) Aw[e] = Aw[(int64_t)j * nbp + i];
    }
}

constexpr int kVRows = 8;  // rows of V per workgroup in k_jacobi_rotate_v

// V <- V J_1 J_2 ... for the rotations logged by the last sweep.  grid = (ceil(nb / 8), blocks).
__global__ void __launch_bounds__(256) k_jacobi_rotate_v(int nb, int nbp, double *V_all, const double *tlog_all,
                                                         const int32_t *state_all) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const int g = blockIdx.y;
    if (state_all[4 * g + 2] == 0) return;
    const int npair = nbp / 2;
    const int r0 = blockIdx.x * kVRows;
    const int rows = min(kVRows, nb - r0);
    double *Vs = (double *)dsm;  // rows x nbp (column nbp-1 is the dummy when nb is odd)
    double *V = V_all + (int64_t)g * nb * nb + (int64_t)r0 * nb;
    const double *tl = tlog_all + (int64_t)g * (nbp - 1) * npair;
    for (int e = threadIdx.x; e < rows * nbp; e += 256) {
        const int r = e / nbp, c = e % nbp;
        Vs[e] = c < nb ? V[(int64_t)r * nb + c] : 0.0;
    }
    __syncthreads();
    for (int s = 0; s < nbp - 1; ++s) {
        for (int it = threadIdx.x; it < rows * npair; it += 256) {
            const int r = it / npair, k = it % npair;
            const double t = tl[(int64_t)s * npair + k];
            if (t == 0.0) continue;
            int p, q;
            rr_pair(nbp, s, k, p, q);
            const double c = 1.0 / sqrt(1.0 + t * t), sn = t * c;
            const double vp = Vs[r * nbp + p], vq = Vs[r * nbp + q];
            Vs[r * nbp + p] = c * vp - sn * vq;
            Vs[r * nbp + q] = sn * vp + c * vq;
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < rows * nb; e += 256) {
        const int r = e / nb, c = e % nb;
        V[(int64_t)r * nb + c] = Vs[r * nbp + c];
    }
}

struct OutTable {
    float *Q[kMaxMats];
    float *lam[kMaxMats];
    int32_t *info[kMaxMats];
};

// Sort descending (ties: lower index first), largest-magnitude entry of each vector positive
// (ties: lowest row), write fp32 Q, lambda, info.  grid.x = blocks, block 256.
__global__ void __launch_bounds__(256) k_jacobi_finalize(int nb, int nbp, int nblk, const double *Aw_all,
                                                         const double *V_all, const int32_t *state_all, OutTable t) {
    extern __shared__ __align__(16) unsigned char dsm[];
    float *lam = (float *)dsm;
    int *rank = (int *)(lam + nb);
    const int g = blockIdx.x;
    const int b = g % nblk, mat = g / nblk;
    const double *Aw = Aw_all + (int64_t)g * nbp * nbp;
    const double *V = V_all + (int64_t)g * nb * nb;
    for (int j = threadIdx.x; j < nb; j += 256) lam[j] = (float)Aw[(int64_t)j * nbp + j];
    __syncthreads();
    for (int j = threadIdx.x; j < nb; j += 256) {
        const float lj = lam[j];
        int r = 0;
        for (int i = 0; i < nb; ++i) {
            const float li = lam[i];
            r += (li > lj) || (li == lj && i < j);
        }
        rank[j] = r;
    }
    __syncthreads();
    float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    for (int j = threadIdx.x; j < nb; j += 256) {
        int arg = 0;
        double best = -1.0;
        for (int p = 0; p < nb; ++p) {
            const double a = fabs(V[(int64_t)p * nb + j]);
            if (a > best) { best = a; arg = p; }
        }
        const double sg = V[(int64_t)arg * nb + j] < 0.0 ? -1.0 : 1.0;
        const int rj = rank[j];
        for (int p = 0; p < nb; ++p) Q[(int64_t)p * nb + rj] = (float)(sg * V[(int64_t)p * nb + j]);
        if (t.lam[mat]) t.lam[mat][(int64_t)b * nb + rj] = lam[j];
    }
    if (threadIdx.x == 0 && t.info[mat]) {
        const int32_t *st = state_all + 4 * g;
        t.info[mat][b] = (st[1] && st[3]) ? st[0] : -1;
    }
}

// ---- Householder QR --------------------------------------------------------------------------
// Z (nb x nb, the workspace copy of A_b Q_b) -> Q with diag(R) > 0, written to the Q table.
// Reflector j: H = I - tau v v^T with v_j = 1, v_i = x_i / (x_j + sgn(x_j) ||x||) (i > j) stored
// below the diagonal, tau = 1 + |x_j| / ||x||, R_jj = -sgn(x_j) ||x||.  Q = H_0 ... H_{nb-1} is then
// formed in place from the last reflector to the first, and columns with R_jj < 0 are negated.
// Dot products and updates are computed in fp64 from fp32 storage.  grid.x = blocks, block 256.
template <bool LDS>
__global__ void __launch_bounds__(256) k_householder(int nb, int nblk, float *Z_all, OutTable t) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const int g = blockIdx.x;
    const int b = g % nblk, mat = g / nblk;
    const int tid = threadIdx.x;
    double *tau = (double *)dsm;      // nb
    double *wv = tau + nb;            // nb
    double *red = wv + nb;            // 4 wave partials + 3 scalars
    int8_t *neg = (int8_t *)(red + 8);  // nb
    float *Zg = Z_all + (int64_t)g * nb * nb;
    const int ld = LDS ? nb + 1 : nb;
    float *Z = LDS ? (float *)(dsm + ((size_t)(2 * nb + 8) * 8 + nb + 15) / 16 * 16) : Zg;
    if (LDS) for (int64_t e = tid; e < (int64_t)nb * nb; e += 256) Z[(e / nb) * ld + e % nb] = Zg[e];
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
        double part = 0.0;
        for (int i = j + tid; i < nb; i += 256) { const double x = Z[(int64_t)i * ld + j]; part += x * x; }
        for (int o = 32; o > 0; o >>= 1) part += __shfl_down(part, o, 64);
        if ((tid & 63) == 0) red[tid >> 6] = part;
        __syncthreads();
        if (tid == 0) {
            const double norm2 = red[0] + red[1] + red[2] + red[3];
            const double alpha = sqrt(norm2);
            const double x0 = Z[(int64_t)j * ld + j];
            const double sg = x0 >= 0.0 ? 1.0 : -1.0;
            if (alpha == 0.0) { tau[j] = 0.0; red[4] = 1.0; red[5] = 0.0; }
            else { tau[j] = 1.0 + fabs(x0) / alpha; red[4] = x0 + sg * alpha; red[5] = -sg * alpha; }
        }
        __syncthreads();
        const double tj = tau[j];
        const double u0 = red[4];
        for (int i = j + 1 + tid; i < nb; i += 256) Z[(int64_t)i * ld + j] = (float)((double)Z[(int64_t)i * ld + j] / u0);
        __syncthreads();
        for (int k = j + 1 + tid; k < nb; k += 256) {
            double s = Z[(int64_t)j * ld + k];
            for (int i = j + 1; i < nb; ++i) s += (double)Z[(int64_t)i * ld + j] * (double)Z[(int64_t)i * ld + k];
            wv[k] = tj * s;
        }
        __syncthreads();
        const int w = nb - j - 1;
        for (int64_t e = tid; e < (int64_t)(nb - j) * w; e += 256) {
            const int i = j + (int)(e / w), k = j + 1 + (int)(e % w);
            const double vi = i == j ? 1.0 : (double)Z[(int64_t)i * ld + j];
            Z[(int64_t)i * ld + k] = (float)((double)Z[(int64_t)i * ld + k] - vi * wv[k]);
        }
        if (tid == 0) { neg[j] = red[5] < 0.0; Z[(int64_t)j * ld + j] = (float)red[5]; }
        __syncthreads();
    }
    // form Q in place: for j = nb-1 .. 0, apply H_j to the already formed trailing columns
    for (int j = nb - 1; j >= 0; --j) {
        const double tj = tau[j];
        if (j < nb - 1) {
            for (int k = j + 1 + tid; k < nb; k += 256) {
                double s = Z[(int64_t)j * ld + k];  // row j of a formed column is zero; kept for clarity
                for (int i = j + 1; i < nb; ++i) s += (double)Z[(int64_t)i * ld + j] * (double)Z[(int64_t)i * ld + k];
                wv[k] = tj * s;
            }
            __syncthreads();
            const int w = nb - j - 1;
            for (int64_t e = tid; e < (int64_t)(nb - j) * w; e += 256) {
                const int i = j + (int)(e / w), k = j + 1 + (int)(e % w);
                const double vi = i == j ? 1.0 : (double)Z[(int64_t)i * ld + j];
                Z[(int64_t)i * ld + k] = (float)((double)Z[(int64_t)i * ld + k] - vi * wv[k]);
            }
            __syncthreads();
        }
        for (int i = tid; i < nb; i += 256) {
            if (i > j) Z[(int64_t)i * ld + j] = (float)(-tj * (double)Z[(int64_t)i * ld + j]);
            else if (i == j) Z[(int64_t)i * ld + j] = (float)(1.0 - tj);
            else Z[(int64_t)i * ld + j] = 0.f;
        }
        __syncthreads();
    }
    float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    for (int64_t e = tid; e < (int64_t)nb * nb; e += 256) {
        const int i = (int)(e / nb), j = (int)(e % nb);
        const float v = Z[(int64_t)i * ld + j];
        Q[e] = neg[j] ? -v : v;
    }
}

// lambda_j = q_j^T (A q_j), with T = A Q in the workspace.  grid.x = blocks.
__global__ void __launch_bounds__(256) k_rayleigh(int nb, int nblk, const float *T_all, OutTable t, int k) {
    const int g = blockIdx.x;
    const int b = g % nblk, mat = g / nblk;
    const float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    const float *T = T_all + (int64_t)g * nb * nb;
    for (int j = threadIdx.x; j < nb; j += 256) {
        double s = 0.0;
        for (int p = 0; p < nb; ++p) s += (double)Q[(int64_t)p * nb + j] * (double)T[(int64_t)p * nb + j];
        if (t.lam[mat]) t.lam[mat][(int64_t)b * nb + j] = (float)s;
    }
    if (threadIdx.x == 0 && t.info[mat]) t.info[mat][b] = k;
}

// ---- workspace layout: five regions, each an array of dense per-block records ----------------
inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }
struct Regions {
    size_t aw, v, t, tlog, state, total;
};
Regions regions(int64_t nb, int64_t nblocks) {
    const int64_t nbp = (nb + 1) / 2 * 2;
    Regions R;
    R.aw = al256((size_t)nbp * nbp * 8 * nblocks);  // Aw: nbp x nbp, fp32 (first stage) then fp64
    R.v = al256((size_t)nb * nb * 8 * nblocks);     // V: nb x nb fp64
    R.t = al256((size_t)nb * nb * 8 * nblocks);     // T: nb x nb, fp32 (A Q products) or fp64 (refinement)
    R.tlog = al256((size_t)(nbp - 1) * (nbp / 2) * 8 * nblocks);   // tangents of one sweep
    R.state = al256((size_t)16 * nblocks);                         // 4 ints
    R.total = R.aw + R.v + R.t + R.tlog + R.state;
    return R;
}

size_t jacobi_lds_bytes(int nbp, size_t esz) {
    return (((size_t)(nbp / 2) * 16 + 4 + 15) / 16) * 16 + (size_t)nbp * nbp * esz;
}

constexpr float kTolFp64 = 1e-14f;   // refinement threshold: |a_pq| <= 1e-14 sqrt(|a_pp a_qq|)
constexpr int kMaxFp64Sweeps = 8;

// fp64-stage state: keep whether the fp32 stage converged in state[3]
__global__ void k_stage_flag(int32_t *state_all) {
    const int g = blockIdx.x;
    if (threadIdx.x == 0) state_all[4 * g + 3] = state_all[4 * g + 1];
}
size_t householder_lds_bytes(int nb, bool lds) {
    size_t head = ((size_t)(2 * nb + 8) * 8 + nb + 15) / 16 * 16;
    return head + (lds ? (size_t)nb * (nb + 1) * 4 : 0);
}

}  // namespace

size_t refresh_ws(const dobb_shape &sh, int count) {
    const int cnt = count < kMaxMats ? count : kMaxMats;
    return regions(sh.nb, (sh.n / sh.nb) * cnt).total;
}

hipError_t launch_refresh(const RefreshArgs &a, hipStream_t s) {
    const int nb = (int)a.sh.nb;
    const int nbp = (nb + 1) / 2 * 2;
    const int nblk = (int)(a.sh.n / nb);
    const int T = (nb + kBM - 1) / kBM;
    const int lds_max = max_lds_bytes();
    for (int c0 = 0; c0 < a.count;) {
        const int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        const int64_t nblocks = (int64_t)nblk * cnt;
        const Regions R = regions(nb, nblocks);
        char *base = (char *)a.ws;
        float *Aw = (float *)base;
        double *V = (double *)(base + R.aw);
        float *Tm = (float *)(base + R.aw + R.v);
        double *tlog = (double *)(base + R.aw + R.v + R.t);
        int32_t *state = (int32_t *)(base + R.aw + R.v + R.t + R.tlog);
        const int64_t aw_stride = (int64_t)nbp * nbp, t_stride = (int64_t)nb * nb;

        OutTable ot{};
        Opnd opA{}, opQ{};
        OutOpnd outT{};
        for (int i = 0; i < cnt; ++i) {
            ot.Q[i] = a.Q[c0 + i];
            ot.lam[i] = a.lambda ? a.lambda[c0 + i] : nullptr;
            ot.info[i] = a.info ? a.info[c0 + i] : nullptr;
            opA.p[i] = a.A[c0 + i];
            opQ.p[i] = a.Q[c0 + i];
            outT.p[i] = Tm + (int64_t)i * nblk * t_stride;
        }
        opA.blk_stride = opQ.blk_stride = (int64_t)nb * nb;
        opA.ld = opQ.ld = nb;
        outT.blk_stride = t_stride;
        outT.ld = nb;
        const dim3 ggemm((unsigned)(T * T * nblocks));

        if (a.mode == DOBB_REFRESH_EXACT) {
            if (a.warm) {
                DOBB_LAUNCH("refresh_gemm", s, k_bgemm<false>, ggemm, dim3(256), 0, nb, T, nblk, opA, opQ, outT);
                Opnd opT{};
                OutOpnd outAw{};
                for (int i = 0; i < cnt; ++i) {
                    opT.p[i] = Tm + (int64_t)i * nblk * t_stride;
                    outAw.p[i] = Aw + (int64_t)i * nblk * aw_stride;
                }
                opT.blk_stride = t_stride; opT.ld = nb;
                outAw.blk_stride = aw_stride; outAw.ld = nbp;
                DOBB_LAUNCH("refresh_gemm", s, k_bgemm<true>, ggemm, dim3(256), 0, nb, T, nblk, opQ, opT, outAw);
            }
            JacTable jt{};
            for (int i = 0; i < cnt; ++i) { jt.A[i] = a.A[c0 + i]; jt.Qp[i] = a.Q[c0 + i]; }
            DOBB_LAUNCH("jacobi_init", s, k_jacobi_init, dim3((unsigned)nblocks), dim3(256), 0, nb, nbp, nblk, a.warm, jt,
                        Aw, V, state);
            const int sweeps = a.iters > 0 ? a.iters : 30;
            const dim3 gv((unsigned)((nb + kVRows - 1) / kVRows), (unsigned)nblocks);
            const size_t vsh = (size_t)kVRows * nbp * 8;
            const size_t head = jacobi_lds_bytes(nbp, 0) + 16;
            // stage 1: fp32 working matrix
            {
                const size_t jl = jacobi_lds_bytes(nbp, 4);
                const bool lds = (int64_t)jl <= lds_max;
                if (lds) (void)hipFuncSetAttribute((const void *)k_jacobi_sweep<float, true>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)jl);
                for (int sw = 0; sw < sweeps; ++sw) {
                    if (lds) DOBB_LAUNCH("jacobi_sweep", s, (k_jacobi_sweep<float, true>), dim3((unsigned)nblocks), dim3(512), jl,
                                         nb, nbp, a.tol, Aw, tlog, state);
                    else DOBB_LAUNCH("jacobi_sweep", s, (k_jacobi_sweep<float, false>), dim3((unsigned)nblocks), dim3(512), head,
                                     nb, nbp, a.tol, Aw, tlog, state);
                    DOBB_LAUNCH("jacobi_rotate_v", s, k_jacobi_rotate_v, gv, dim3(256), vsh, nb, nbp, V,
                                (const double *)tlog, (const int32_t *)state);
                }
            }
            // stage 2: V^T A V in fp64, then fp64 sweeps until the relative threshold 1e-14 holds
            {
                double *Aw64 = (double *)Aw;
                double *T64 = (double *)Tm;
                const int tiles = (nb + 15) / 16;
                const dim3 gr((unsigned)(tiles * tiles), (unsigned)nblocks);
                DOBB_LAUNCH("jacobi_stage_flag", s, k_stage_flag, dim3((unsigned)nblocks), dim3(64), 0, state);
                DOBB_LAUNCH("jacobi_refine_gemm", s, k_refine_gemm, gr, dim3(256), 0, nb, nbp, nblk, 0, jt,
                            (const double *)V, T64, Aw64, state);
                DOBB_LAUNCH("jacobi_refine_gemm", s, k_refine_gemm, gr, dim3(256), 0, nb, nbp, nblk, 1, jt,
                            (const double *)V, T64, Aw64, state);
                DOBB_LAUNCH("jacobi_symmetrize", s, k_symmetrize64, dim3((unsigned)nblocks), dim3(256), 0, nbp, Aw64);
                const size_t jl = jacobi_lds_bytes(nbp, 8);
                const bool lds = (int64_t)jl <= lds_max;
                if (lds) (void)hipFuncSetAttribute((const void *)k_jacobi_sweep<double, true>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)jl);
                for (int sw = 0; sw < kMaxFp64Sweeps; ++sw) {
                    if (lds) DOBB_LAUNCH("jacobi_sweep_fp64", s, (k_jacobi_sweep<double, true>), dim3((unsigned)nblocks), dim3(512),
                                         jl, nb, nbp, kTolFp64, Aw64, tlog, state);
                    else DOBB_LAUNCH("jacobi_sweep_fp64", s, (k_jacobi_sweep<double, false>), dim3((unsigned)nblocks), dim3(512),
                                     head, nb, nbp, kTolFp64, Aw64, tlog, state);
                    DOBB_LAUNCH("jacobi_rotate_v", s, k_jacobi_rotate_v, gv, dim3(256), vsh, nb, nbp, V,
                                (const double *)tlog, (const int32_t *)state);
                }
                DOBB_LAUNCH("jacobi_finalize", s, k_jacobi_finalize, dim3((unsigned)nblocks), dim3(256), (size_t)nb * 8, nb,
                            nbp, nblk, (const double *)Aw64, (const double *)V, (const int32_t *)state, ot);
            }
        } else {
            const size_t hl = householder_lds_bytes(nb, true);
            const bool lds = (int64_t)hl <= lds_max;
            const size_t hsh = householder_lds_bytes(nb, lds);
            if (lds) (void)hipFuncSetAttribute((const void *)k_householder<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)hl);
            for (int it = 0; it < a.iters; ++it) {
                DOBB_LAUNCH("refresh_gemm", s, k_bgemm<false>, ggemm, dim3(256), 0, nb, T, nblk, opA, opQ, outT);
                if (lds) DOBB_LAUNCH("householder_qr", s, k_householder<true>, dim3((unsigned)nblocks), dim3(256), hsh, nb, nblk,
                                     Tm, ot);
                else DOBB_LAUNCH("householder_qr", s, k_householder<false>, dim3((unsigned)nblocks), dim3(256), hsh, nb, nblk,
                                 Tm, ot);
            }
            bool want_lam = false, want_info = false;
            for (int i = 0; i < cnt; ++i) { want_lam |= ot.lam[i] != nullptr; want_info |= ot.info[i] != nullptr; }
            if (want_lam) DOBB_LAUNCH("refresh_gemm", s, k_bgemm<false>, ggemm, dim3(256), 0, nb, T, nblk, opA, opQ, outT);
            if (want_lam || want_info)
                DOBB_LAUNCH("rayleigh", s, k_rayleigh, dim3((unsigned)nblocks), dim3(256), 0, nb, nblk, (const float *)Tm, ot,
                            a.iters);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
