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
//           When even the fp32 working matrix exceeds the LDS, block Jacobi in fp64 instead
//           (k_bj_sub / k_bj_apply below): a round touches A and V once instead of nbp - 1 times.
// ORTH_ITER k times: Z = A_b Q_b (MFMA), Q_b <- qr(Z).Q by Householder (k_qr.hip: one launch with
//           Z in LDS for nb <= 128, panel / update / formation launches above), diag(R) > 0.
//           Rayleigh quotients go to lambda when requested.
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

// grid.x = tiles * tiles * nblk * count.  VEC: 16-byte operand loads (nb % 4 == 0, so every row
// and 4-column piece starts 16-byte aligned)
template <bool TRANS_A, bool VEC>
__global__ void __launch_bounds__(256) k_bgemm(int nb, int T, int nblk, Opnd A, Opnd B, OutOpnd C) {
    __shared__ GemmSmem2 sm;
    const int x = xcd_remap(blockIdx.x, gridDim.x);   // the tiles of a block share one XCD's L2
    const int tile = x % (T * T);
    const int rest = x / (T * T);
    const int b = rest % nblk, mat = rest / nblk;
    const int i0 = (tile / T) * kBM, j0 = (tile % T) * kBN;
    const float *Ab = A.p[mat] + (int64_t)b * A.blk_stride;
    const float *Bb = B.p[mat] + (int64_t)b * B.blk_stride;
    LoadColsK<VEC> lb{Bb + j0, B.ld, nb - j0, nb};
    f32x16 acc;
    if (TRANS_A) {  // op(A)[i][k] = A[k][i]: already k-major
        LoadColsK<VEC> la{Ab + i0, A.ld, nb - i0, nb};
        acc = gemm_tile(nb, la, lb, sm);
    } else {
        LoadRowsT<VEC> la{Ab + (int64_t)i0 * A.ld, A.ld, nb - i0, nb};
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

// The same product on 16 x 16 x 4 fp32 MFMA tiles, for widths that a tile of 16 NT fits without
// much padding (NT = 5: 80-wide tiles, 25 per nb = 400 block; nb <= 16 NT: one tile per block, so
// nb = 100 runs as 112 x 112 instead of 128 x 128 with a 112-deep K).  NT waves, wave w computing rows
// 16 w .. 16 w + 15 of the tile against its NT column tiles (the row operand read once per k-step
// for NT products); K in 16-deep chunks, double buffered in LDS with one barrier per chunk, both
// operands k-major there (a[k][i] = op(A)[i][k], b[k][j] = B[k][j]).  The 16 x 16 x 4 lane layout
// (checked on gfx950): A[l % 16][l / 16], B[l / 16][l % 16], D[4 (l / 16) + i][l % 16].
constexpr int kTK = 16;
template <int NT>
struct TileSmem {
    // row pitch 16 or 48 words modulo the 64 banks, so a k-step's four rows of 16 meet no conflict
    static constexpr int P = (16 * NT) % 32 == 0 ? 16 * NT + 16 : 16 * NT;
    float a[2][kTK][P];
    float b[2][kTK][P];
};
// grid.x = tiles * tiles * nblk * count (T = ceil(nb / 16 NT)), block 64 NT
template <int NT, bool TRANS_A, bool VEC>
__global__ void __launch_bounds__(64 * NT) k_bgemm_t(int nb, int T, int nblk, Opnd A, Opnd B, OutOpnd C) {
    constexpr int TILE = 16 * NT, NTH = 64 * NT, Q4 = TILE / 4, K4 = kTK / 4, R = kTK / 16;
    __shared__ __align__(16) TileSmem<NT> sm;
    const int x = xcd_remap(blockIdx.x, gridDim.x);   // the tiles of a block share one XCD's L2
    const int tile = x % (T * T);
    const int rest = x / (T * T);
    const int b = rest % nblk, mat = rest / nblk;
    const int i0 = (tile / T) * TILE, j0 = (tile % T) * TILE;
    const float *Ab = A.p[mat] + (int64_t)b * A.blk_stride;
    const float *Bb = B.p[mat] + (int64_t)b * B.blk_stride;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    // one chunk is TILE x kTK floats of each operand, R float4 pieces of each per thread
    f32x4 va[R], vb[R];
    auto load4 = [&](const float *p, int lim) -> f32x4 {   // p[0..3] that lie below lim, zeros past it
        f32x4 q = f32x4{0.f, 0.f, 0.f, 0.f};
        if (VEC) {
            if (lim > 0) q = *(const f32x4 *)p;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) if (c < lim) q[c] = p[c];
        }
        return q;
    };
    auto fetch = [&](int k0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = t + r * NTH;
            {   // B[k][j]: k = e / Q4, j = 4 (e % Q4) ..
                const int kk = e / Q4, jj = 4 * (e - kk * Q4), k = k0 + kk, j = j0 + jj;
                vb[r] = k < nb ? load4(Bb + (int64_t)k * B.ld + j, nb - j) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if (TRANS_A) {   // op(A)[i][k] = A[k][i]
                const int kk = e / Q4, ii = 4 * (e - kk * Q4), k = k0 + kk, i = i0 + ii;
                va[r] = k < nb ? load4(Ab + (int64_t)k * A.ld + i, nb - i) : f32x4{0.f, 0.f, 0.f, 0.f};
            } else {         // op(A)[i][k] = A[i][k]: i = e / K4, k = 4 (e % K4) ..
                const int ii = e / K4, kk = 4 * (e % K4), i = i0 + ii, k = k0 + kk;
                va[r] = i < nb ? load4(Ab + (int64_t)i * A.ld + k, nb - k) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = t + r * NTH;
            {
                const int kk = e / Q4, jj = 4 * (e - kk * Q4);
                *(f32x4 *)&sm.b[buf][kk][jj] = vb[r];
            }
            if (TRANS_A) {
                const int kk = e / Q4, ii = 4 * (e - kk * Q4);
                *(f32x4 *)&sm.a[buf][kk][ii] = va[r];
            } else {
                const int ii = e / K4, kk = 4 * (e % K4);
#pragma unroll
                for (int c = 0; c < 4; ++c) sm.a[buf][kk + c][ii] = va[r][c];
            }
        }
    };
    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch(0);
    put(0);
    __syncthreads();
    int cur = 0;
    const int r16 = lane & 15, k4 = lane >> 4;
    for (int k0 = 0; k0 < nb; k0 += kTK) {
        const bool more = k0 + kTK < nb;
        if (more) fetch(k0 + kTK);
#pragma unroll
        for (int ks = 0; ks < kTK; ks += 4) {
            const float av = sm.a[cur][ks + k4][16 * w + r16];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const float bv = sm.b[cur][ks + k4][16 * j + r16];
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[j], 0, 0, 0);
            }
        }
        if (more) put(cur ^ 1);   // the other buffer's readers finished before the last barrier
        __syncthreads();
        cur ^= 1;
    }
    float *Cb = C.p[mat] + (int64_t)b * C.blk_stride;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int col = j0 + 16 * j + r16;
        if (col >= nb) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = i0 + 16 * w + 4 * k4 + i;
            if (row < nb) Cb[(int64_t)row * C.ld + col] = acc[j][i];
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

// ---- block Jacobi: working matrices that do not fit the LDS ------------------------------------
// The indices are cut into m (even) index blocks of b (the last ones padded past nb: zero rows and
// columns, never rotated).  A round pairs the index blocks by the circle method, so a sweep is
// m - 1 rounds and meets every pair of index blocks once; in a round the m / 2 pair sets
// S_k = I_k u J_k (2b indices each) are disjoint.  k_bj_sub gives each S_k one cyclic sweep of its
// 2b x 2b sub-problem in LDS, by the rotation rule of k_jacobi_sweep, and keeps the product R_k of
// those rotations (fp64); the swept sub-matrix is A's diagonal tile R_k^T A_{S_k S_k} R_k.
// k_bj_apply carries the round to the rest: A_{S_p S_q} <- R_p^T A_{S_p S_q} R_q for p < q (and its
// transpose), V_{:, S_q} <- V_{:, S_q} R_q.  A round so reads and writes A and V once, where the
// element-wise sweep does so for every one of its nbp - 1 rounds.  All in fp64; the rotation rule
// and threshold are those of the refinement stage, so the result meets the same 1e-14 criterion.
struct BjGeo {
    int m, b;   // index blocks (even), indices per block (a multiple of 4, at most 40)
};
__host__ __device__ inline BjGeo bj_geo(int nb) {
    BjGeo G;
    G.m = 2 * ((nb + 79) / 80);
    const int b = (nb + G.m - 1) / G.m;
    G.b = (b + 3) / 4 * 4;
    return G;
}
// index of local row l (0 .. 2b - 1) of the pair set (I, J)
__device__ __forceinline__ int bj_idx(int l, int I, int J, int b) { return l < b ? I * b + l : J * b + (l - b); }

__host__ __device__ inline size_t bj_sub_lds(int nb) {
    const int b2 = 2 * bj_geo(nb).b;
    return (size_t)2 * b2 * (b2 + 1) * 8 + (size_t)(b2 / 2) * (5 * 8 + 4 + 4) + 16;
}
constexpr int kBjK = 16;   // rows of R per LDS chunk in k_bj_apply
__host__ __device__ inline size_t bj_apply_lds(int nb) {
    const int b2 = 2 * bj_geo(nb).b;
    return (size_t)(b2 + kBjK) * (b2 + 1) * 8;
}

// grid = (m / 2 pair sets, blocks), block 512.  R_all: per block m / 2 matrices 2b x 2b; nrot_all:
// per block and pair set, the rotations of this round (0: R is the identity and was not written).
// B2 = 2b.  One step of the inner sweep is three passes over LDS: the rotations (tangent, cosine
// and sine, computed once by the thread that chooses the pair, with the pair's new diagonal);
// A <- A J and R <- R J; A <- J^T A, which writes the pair's own 2 x 2 block exactly (a_pq = a_qp =
// 0, a_pp - t a_pq, a_qq + t a_pq).  In the two update passes a thread keeps one row (one column)
// index and takes every kBjThreads / B2-th pair, so a wave's lanes touch consecutive rows (columns)
// of the same two columns (rows); the row pitch, B2 + 1 doubles, spreads a column over the banks.
// The two orders of rounding leave A symmetric to rounding only; the angles read the upper entry
// and the swept tile is written back symmetric.
constexpr int kBjThreads = 512;
template <int B2>
__global__ void __launch_bounds__(kBjThreads) k_bj_sub(int nb, int nbp, int round, float tol, double *Aw_all,
                                                       double *R_all, int32_t *nrot_all, int32_t *state_all) {
    extern __shared__ __align__(16) unsigned char dsm[];
    constexpr int b = B2 / 2, np = b, ld = B2 + 1;
    constexpr int kPT = kBjThreads / B2;             // threads per row (column) index
    constexpr int kKP = (np + kPT - 1) / kPT;        // pairs per thread and pass
    const BjGeo G = bj_geo(nb);
    const int k = blockIdx.x, g = blockIdx.y;
    int32_t *st = state_all + 4 * g;
    if (st[1]) return;   // converged
    double *As = (double *)dsm;
    double *Rs = As + B2 * ld;
    double *tsh = Rs + B2 * ld;
    double *csh = tsh + np;
    double *ssh = csh + np;
    double *dp = ssh + np;    // new a_pp
    double *dq = dp + np;     // new a_qq
    int *psh = (int *)(dq + np);
    int *qsh = psh + np;
    int *nrot_sh = qsh + np;
    int I, J;
    rr_pair(G.m, round, k, I, J);
    double *Aw = Aw_all + (int64_t)g * nbp * nbp;
    const int tid = threadIdx.x;
    for (int e = tid; e < B2 * B2; e += kBjThreads) {
        const int r = e / B2, c = e - r * B2;
        const int gi = bj_idx(r, I, J, b), gj = bj_idx(c, I, J, b);
        As[r * ld + c] = (gi < nb && gj < nb) ? Aw[(int64_t)gi * nbp + gj] : 0.0;
        Rs[r * ld + c] = r == c ? 1.0 : 0.0;
    }
    if (tid == 0) *nrot_sh = 0;
    __syncthreads();
    int myrot = 0;
    const double dtol = (double)tol;
    const int ix = tid % B2, kk0 = tid / B2;         // this thread's row (column) and first pair
    const bool worker = kk0 < kPT;
    for (int s = 0; s < B2 - 1; ++s) {
        if (tid < np) {
            int p, q;
            rr_pair(B2, s, tid, p, q);
            double t = 0.0;
            const double app = As[p * ld + p], aqq = As[q * ld + q], apq = As[p * ld + q];
            if (apq != 0.0 && fabs(apq) > dtol * sqrt(fabs(app * aqq))) {
                const double theta = (aqq - app) / (2.0 * apq);
                if (fabs(theta) > 1e150) t = 0.5 / theta;
                else t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(1.0 + theta * theta));
                ++myrot;
            }
            const double c = 1.0 / sqrt(1.0 + t * t);
            tsh[tid] = t; csh[tid] = c; ssh[tid] = t * c; psh[tid] = p; qsh[tid] = q;
            dp[tid] = app - t * apq;
            dq[tid] = aqq + t * apq;
        }
        __syncthreads();
        // columns p, q of A and of R, in row ix
        if (worker) {
#pragma unroll
            for (int i = 0; i < kKP; ++i) {
                const int kk = kk0 + kPT * i;
                if (kk < np && tsh[kk] != 0.0) {
                    const int p = psh[kk], q = qsh[kk];
                    const double c = csh[kk], sn = ssh[kk];
                    const double ap = As[ix * ld + p], aq = As[ix * ld + q];
                    const double rp = Rs[ix * ld + p], rq = Rs[ix * ld + q];
                    As[ix * ld + p] = c * ap - sn * aq;
                    As[ix * ld + q] = sn * ap + c * aq;
                    Rs[ix * ld + p] = c * rp - sn * rq;
                    Rs[ix * ld + q] = sn * rp + c * rq;
                }
            }
        }
        __syncthreads();
        // rows p, q of A, in column ix; the pair's own columns get the exact block
        if (worker) {
#pragma unroll
            for (int i = 0; i < kKP; ++i) {
                const int kk = kk0 + kPT * i;
                if (kk < np && tsh[kk] != 0.0) {
                    const int p = psh[kk], q = qsh[kk];
                    double vp, vq;
                    if (ix == p) { vp = dp[kk]; vq = 0.0; }
                    else if (ix == q) { vp = 0.0; vq = dq[kk]; }
                    else {
                        const double c = csh[kk], sn = ssh[kk];
                        const double yp = As[p * ld + ix], yq = As[q * ld + ix];
                        vp = c * yp - sn * yq;
                        vq = sn * yp + c * yq;
                    }
                    As[p * ld + ix] = vp;
                    As[q * ld + ix] = vq;
                }
            }
        }
        __syncthreads();
    }
    if (myrot) atomicAdd(nrot_sh, myrot);   // integer counts: order-independent
    __syncthreads();
    const int rot = *nrot_sh;
    if (rot) {
        double *R = R_all + ((int64_t)g * (G.m / 2) + k) * B2 * B2;
        for (int e = tid; e < B2 * B2; e += kBjThreads) {
            const int r = e / B2, c = e - r * B2;
            const int gi = bj_idx(r, I, J, b), gj = bj_idx(c, I, J, b);
            // the swept tile, symmetric: the upper entry for both
            const double v = r <= c ? As[r * ld + c] : As[c * ld + r];
            if (gi < nb && gj < nb) Aw[(int64_t)gi * nbp + gj] = v;
            R[e] = Rs[r * ld + c];
        }
    }
    if (tid == 0) {
        nrot_all[(int64_t)g * (G.m / 2) + k] = rot;
        if (rot) atomicAdd(&st[2], rot);
    }
}

// grid = (tiles, blocks), block 256: tiles [0, m/2 (m/2 - 1) / 2) are the pairs p < q of pair sets
// (A_{S_p S_q} <- R_p^T A_{S_p S_q} R_q, written with its transpose), the rest (pair set q, B2-row
// tile) V_{rows, S_q} <- V_{rows, S_q} R_q.  Each thread owns a kT x kT piece of the B2 x B2 result
// (rows ty + 16 i, columns tx + 16 j); the operand X sits in LDS, R comes in kBjK-row chunks.  A pair
// set whose sub-problem rotated nothing has R = I (not read).
template <int B2>
__global__ void __launch_bounds__(256) k_bj_apply(int nb, int nbp, int round, double *Aw_all, double *V_all,
                                                  const double *R_all, const int32_t *nrot_all, const int32_t *state_all) {
    extern __shared__ __align__(16) unsigned char dsm[];
    constexpr int b = B2 / 2, ld = B2 + 1, kT = (B2 + 15) / 16;
    const BjGeo G = bj_geo(nb);
    const int np2 = G.m / 2;
    const int g = blockIdx.y;
    if (state_all[4 * g + 1]) return;
    const int na = np2 * (np2 - 1) / 2;
    const int tile = blockIdx.x;
    int p = 0, q = 0, rt = 0;
    const bool isA = tile < na;
    if (isA) {
        int rem = tile;
        while (rem >= np2 - 1 - p) { rem -= np2 - 1 - p; ++p; }
        q = p + 1 + rem;
    } else {
        const int v = tile - na, nrt = (nb + B2 - 1) / B2;
        q = v / nrt;
        rt = v - q * nrt;
    }
    const int32_t *nr = nrot_all + (int64_t)g * np2;
    const bool rq_id = nr[q] == 0, rp_id = !isA || nr[p] == 0;
    if (rq_id && rp_id) return;
    int Ip = 0, Jp = 0, Iq, Jq;
    rr_pair(G.m, round, q, Iq, Jq);
    if (isA) rr_pair(G.m, round, p, Ip, Jp);
    double *X = (double *)dsm;            // [B2][ld]
    double *Rc = X + B2 * ld;             // [kBjK][ld]
    double *Aw = Aw_all + (int64_t)g * nbp * nbp;
    double *V = V_all + (int64_t)g * nb * nb;
    const double *Rq = R_all + ((int64_t)g * np2 + q) * B2 * B2;
    const double *Rp = isA ? R_all + ((int64_t)g * np2 + p) * B2 * B2 : nullptr;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    // the operand: A_{S_p S_q} or rows rt B2 .. of V's columns S_q (zero outside)
    for (int e = tid; e < B2 * B2; e += 256) {
        const int r = e / B2, c = e - r * B2;
        const int gj = bj_idx(c, Iq, Jq, b);
        double v = 0.0;
        if (isA) {
            const int gi = bj_idx(r, Ip, Jp, b);
            if (gi < nb && gj < nb) v = Aw[(int64_t)gi * nbp + gj];
        } else {
            const int gi = rt * B2 + r;
            if (gi < nb && gj < nb) v = V[(int64_t)gi * nb + gj];
        }
        X[r * ld + c] = v;
    }
    double acc[kT][kT];
    // acc = X R, or (trans_lhs) R^T X; R = I when ident
    auto product = [&](const double *R, bool ident, bool trans_lhs) {
#pragma unroll
        for (int i = 0; i < kT; ++i)
#pragma unroll
            for (int j = 0; j < kT; ++j) acc[i][j] = 0.0;
        for (int k0 = 0; k0 < B2; k0 += kBjK) {
            __syncthreads();   // X complete (first chunk) / the previous chunk's readers are done
            for (int e = tid; e < kBjK * B2; e += 256) {
                const int kr = e / B2, c = e - kr * B2, kk = k0 + kr;
                Rc[kr * ld + c] = kk < B2 ? (ident ? (kk == c ? 1.0 : 0.0) : R[(int64_t)kk * B2 + c]) : 0.0;
            }
            __syncthreads();
#pragma unroll 4
            for (int kr = 0; kr < kBjK; ++kr) {
                if (k0 + kr >= B2) break;
                double xv[kT], rv[kT];
#pragma unroll
                for (int i = 0; i < kT; ++i) {
                    const int r = ty + 16 * i;
                    xv[i] = r < B2 ? (trans_lhs ? Rc[kr * ld + r] : X[r * ld + k0 + kr]) : 0.0;
                }
#pragma unroll
                for (int j = 0; j < kT; ++j) {
                    const int c = tx + 16 * j;
                    rv[j] = c < B2 ? (trans_lhs ? X[(k0 + kr) * ld + c] : Rc[kr * ld + c]) : 0.0;
                }
#pragma unroll
                for (int i = 0; i < kT; ++i)
#pragma unroll
                    for (int j = 0; j < kT; ++j) acc[i][j] = __builtin_fma(xv[i], rv[j], acc[i][j]);
            }
        }
    };
    product(Rq, rq_id, false);
    if (isA) {
        // the partial product X R_q back into X, then R_p^T (X R_q)
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kT; ++i)
#pragma unroll
            for (int j = 0; j < kT; ++j) {
                const int r = ty + 16 * i, c = tx + 16 * j;
                if (r < B2 && c < B2) X[r * ld + c] = acc[i][j];
            }
        product(Rp, rp_id, true);
    }
#pragma unroll
    for (int i = 0; i < kT; ++i)
#pragma unroll
        for (int j = 0; j < kT; ++j) {
            const int r = ty + 16 * i, c = tx + 16 * j;
            if (r >= B2 || c >= B2) continue;
            const int gj = bj_idx(c, Iq, Jq, b);
            if (gj >= nb) continue;
            if (isA) {
                const int gi = bj_idx(r, Ip, Jp, b);
                if (gi >= nb) continue;
                Aw[(int64_t)gi * nbp + gj] = acc[i][j];
                Aw[(int64_t)gj * nbp + gi] = acc[i][j];
            } else {
                const int gi = rt * B2 + r;
                if (gi < nb) V[(int64_t)gi * nb + gj] = acc[i][j];
            }
        }
}

// state: [0] sweeps that rotated, [1] converged, [2] rotations in this sweep, [3] = 1 (one stage)
__global__ void k_bj_begin(int32_t *state_all) {
    if (threadIdx.x == 0) state_all[4 * blockIdx.x + 3] = 1;
}
__global__ void k_bj_sweep_end(int32_t *state_all) {
    int32_t *st = state_all + 4 * blockIdx.x;
    if (threadIdx.x == 0 && !st[1]) {
        if (st[2] == 0) st[1] = 1;
        else st[0] += 1;
        st[2] = 0;
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

// ---- Householder QR, blocked (WY form) ------------------------------------------------------
// Z (nb x nb, the workspace copy of A_b Q_b) -> Q with diag(R) > 0, written to the Q table.
// Panels of kQP = 32 columns.  Each panel is factored column by column in LDS: reflector c is
// H = I - tau v v^T with v_c = 1, v_r = x_r / (x_c + sgn(x_c) ||x||) below, tau = 1 + |x_c| / ||x||,
// R_cc = -sgn(x_c) ||x||.  The panel's reflectors are combined as H_1..H_w = I - V T V^T, with T
// upper triangular from V^T V and the taus; the trailing columns are updated as
// Z <- Z - V T^T (V^T Z) with three fp32 MFMA 32x32x2 products per 32-column tile (one tile per
// wave).  V and T of every panel are kept (V in Z's panel columns, T in the workspace); Q is then
// formed from the identity by applying the block reflectors last to first, Q <- Q - V T (V^T Q), and
// the columns with R_cc < 0 are negated.  Z lives in the workspace.
constexpr int kQP = 32;

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) / 16 * 16; }
// acc (32x32, MFMA layout) -> S[32][33]
__device__ __forceinline__ void acc_to_lds(const f32x16 &acc, float (*S)[33], int lane) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[acc_row(r, lane)][acc_col(lane)] = acc[r];
}

// ---- Householder QR, blocked, one launch per panel step (large blocks) ------------------------
// Panels of 32 columns, split over launches so the trailing updates spread over the whole GPU:
//   k_qr_panel   one workgroup per block factors panel p (32 columns) in LDS, writes V into Z's
//                panel columns, T into the workspace and the signs of R's diagonal;
//   k_qr_update  one workgroup per (block, 64-column tile) applies the panel's block reflector:
//                X <- X - V op(T) (V^T X), with op(T) = T^T while factoring Z and op(T) = T while
//                forming Q from the identity (panels last to first);
//   k_qr_finish  negates the columns of Q with R_cc < 0 and writes info.
struct QrPanelLayout {
    size_t red, tau, gsh, tsd, part, wk, vs, total;
};
__host__ __device__ inline QrPanelLayout qr_panel_layout(int nb) {
    QrPanelLayout L;
    size_t o = 0;
    L.red = o;  o += al16(8 * 8);
    L.tau = o;  o += al16(kQP * 8);
    L.gsh = o;  o += al16(kQP * kQP * 8);
    L.tsd = o;  o += al16(kQP * kQP * 8);
    L.part = o; o += al16(8 * kQP * 8);
    L.wk = o;   o += al16(kQP * 8);
    L.vs = o;   o += al16((size_t)nb * (kQP + 1) * 4);
    L.total = o;
    return L;
}

// grid.x = blocks, block 256
__global__ void __launch_bounds__(256) k_qr_panel(int nb, int p, float *Z_all, float *Tq_all, int8_t *neg_all) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const QrPanelLayout L = qr_panel_layout(nb);
    double *red = (double *)(dsm + L.red);
    double *tau = (double *)(dsm + L.tau);
    double *gsh = (double *)(dsm + L.gsh);
    double *tsd = (double *)(dsm + L.tsd);
    double *part = (double *)(dsm + L.part);
    double *wk = (double *)(dsm + L.wk);
    float(*Vs)[kQP + 1] = (float(*)[kQP + 1])(dsm + L.vs);
    const int g = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int npanel = (nb + kQP - 1) / kQP;
    float *Z = Z_all + (int64_t)g * nb * nb;
    float *Tq = Tq_all + ((int64_t)g * npanel + p) * kQP * kQP;
    int8_t *neg = neg_all + (int64_t)g * nb;
    const int j0 = p * kQP, w = min(kQP, nb - j0), rows = nb - j0;
    for (int e = tid; e < rows * kQP; e += 256) {
        const int r = e / kQP, c = e % kQP;
        Vs[r][c] = c < w ? Z[(int64_t)(j0 + r) * nb + j0 + c] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < w; ++c) {
        double ps = 0.0;
        for (int r = c + tid; r < rows; r += 256) { const double x = Vs[r][c]; ps += x * x; }
        for (int o = 32; o > 0; o >>= 1) ps += __shfl_down(ps, o, 64);
        if (lane == 0) red[wv] = ps;
        __syncthreads();
        if (tid == 0) {
            const double alpha = sqrt(red[0] + red[1] + red[2] + red[3]);
            const double x0 = Vs[c][c];
            const double sg = x0 >= 0.0 ? 1.0 : -1.0;
            if (alpha == 0.0) { tau[c] = 0.0; red[4] = 1.0; red[5] = 0.0; }
            else { tau[c] = 1.0 + fabs(x0) / alpha; red[4] = x0 + sg * alpha; red[5] = -sg * alpha; }
            neg[j0 + c] = red[5] < 0.0;
        }
        __syncthreads();
        const double u0 = red[4], tc = tau[c];
        for (int r = c + 1 + tid; r < rows; r += 256) Vs[r][c] = (float)((double)Vs[r][c] / u0);
        __syncthreads();
        {
            const int k = tid & 31, grp = tid >> 5;
            double sk = 0.0;
            if (k > c && k < w) {
                for (int r = c + grp; r < rows; r += 8) {
                    const double v = r == c ? 1.0 : (double)Vs[r][c];
                    sk += v * (double)Vs[r][k];
                }
            }
            part[grp * kQP + k] = sk;
        }
        __syncthreads();
        if (tid < kQP) {
            double sk = 0.0;
            for (int q = 0; q < 8; ++q) sk += part[q * kQP + tid];
            wk[tid] = tc * sk;
        }
        __syncthreads();
        for (int e = tid; e < (rows - c) * kQP; e += 256) {
            const int r = c + e / kQP, k = e % kQP;
            if (k > c && k < w) {
                const double v = r == c ? 1.0 : (double)Vs[r][c];
                Vs[r][k] = (float)((double)Vs[r][k] - v * wk[k]);
            }
        }
        __syncthreads();
    }
    for (int e = tid; e < rows * kQP; e += 256) {
        const int r = e / kQP, c = e % kQP;
        if (c < w) { if (r == c) Vs[r][c] = 1.f; else if (r < c) Vs[r][c] = 0.f; }
    }
    __syncthreads();
    for (int e = tid; e < kQP * kQP; e += 256) {
        const int i = e / kQP, j = e % kQP;
        double sgv = 0.0;
        if (i < j && j < w)
            for (int r = i; r < rows; ++r) sgv += (double)Vs[r][i] * (double)Vs[r][j];
        gsh[e] = sgv;
        tsd[e] = 0.0;
    }
    __syncthreads();
    for (int j = 0; j < w; ++j) {
        if (tid < j) {
            double sum = 0.0;
            for (int k = tid; k < j; ++k) sum += tsd[tid * kQP + k] * gsh[k * kQP + j];
            tsd[tid * kQP + j] = -tau[j] * sum;
        }
        if (tid == j) tsd[j * kQP + j] = tau[j];
        __syncthreads();
    }
    for (int e = tid; e < kQP * kQP; e += 256) Tq[e] = (float)tsd[e];
    for (int e = tid; e < rows * w; e += 256) {
        const int r = e / w, c = e % w;
        Z[(int64_t)(j0 + r) * nb + j0 + c] = Vs[r][c];
    }
}

// grid = (64-column tiles, blocks), block 256: wave w works on column half h = w & 1 of the tile;
// for V^T X the two waves of a half split the rows, for X -= V Y they split 32-row chunks.
template <bool FACTOR>
__global__ void __launch_bounds__(256) k_qr_update(int nb, int nblk, int p, const float *Z_all, const float *Tq_all,
                                                   OutTable t) {
    __shared__ float Ts[kQP][kQP + 1];
    __shared__ float Wp[2][2][32][33];   // [row half][column half]
    __shared__ float Ysh[2][32][33];
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int h = wv & 1, kp = wv >> 1;
    const int npanel = (nb + kQP - 1) / kQP;
    const int j0 = p * kQP, w = min(kQP, nb - j0), rows = nb - j0;
    const float *Z = Z_all + (int64_t)g * nb * nb;       // V of panel p in columns j0..j0+w
    float *X = FACTOR ? (float *)Z_all + (int64_t)g * nb * nb : t.Q[mat] + (int64_t)b * nb * nb;
    const int first = FACTOR ? j0 + w : j0;
    const int c0 = first + blockIdx.x * 64 + 32 * h;
    const float *Tq = Tq_all + ((int64_t)g * npanel + p) * kQP * kQP;
    for (int e = tid; e < kQP * kQP; e += 256) Ts[e / kQP][e % kQP] = Tq[e];
    const int cc = lane & 31, kr = lane >> 5;
    const bool colok = c0 + cc < nb;
    const bool vok = cc < w;
    // W partial = V[rows of this half]^T X
    {
        const int half = (rows + 1) / 2;
        const int rbeg = kp ? half : 0, rend = kp ? rows : half;
        f32x16 acc = {};
#pragma unroll 8
        for (int k = rbeg; k < rend; k += 2) {
            const int r = k + kr;
            const bool rok = r < rend;
            const float a = (rok && vok) ? Z[(int64_t)(j0 + r) * nb + j0 + cc] : 0.f;
            const float bx = (rok && colok) ? X[(int64_t)(j0 + r) * nb + c0 + cc] : 0.f;
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bx, acc, 0, 0, 0);
        }
        acc_to_lds(acc, Wp[kp][h], lane);
    }
    __syncthreads();
    if (kp == 0) {   // Y = op(T) W for this column half
        f32x16 y = {};
#pragma unroll
        for (int kk = 0; kk < kQP; kk += 2) {
            const int k = kk + kr;
            const float a = FACTOR ? Ts[k][cc] : Ts[cc][k];
            const float wkj = Wp[0][h][k][cc] + Wp[1][h][k][cc];
            y = __builtin_amdgcn_mfma_f32_32x32x2f32(a, wkj, y, 0, 0, 0);
        }
        acc_to_lds(y, Ysh[h], lane);
    }
    __syncthreads();
    // X -= V Y: chunks of 32 rows, alternating between the two waves of this half
    for (int r0 = 32 * kp; r0 < rows; r0 += 64) {
        f32x16 u = {};
        const int rr = r0 + cc;
#pragma unroll
        for (int kk = 0; kk < kQP; kk += 2) {
            const int k = kk + kr;
            const float a = (rr < rows && k < w) ? Z[(int64_t)(j0 + rr) * nb + j0 + k] : 0.f;
            u = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Ysh[h][k][cc], u, 0, 0, 0);
        }
        const int col = c0 + acc_col(lane);
        if (col < nb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = r0 + acc_row(r, lane);
                if (row < rows) X[(int64_t)(j0 + row) * nb + col] -= u[r];
            }
        }
    }
}

// Q := I before the formation sweep.  grid = blocks.
__global__ void __launch_bounds__(256) k_qr_identity(int nb, int nblk, OutTable t) {
    const int g = blockIdx.x;
    float *Q = t.Q[g / nblk] + (int64_t)(g % nblk) * nb * nb;
    for (int64_t e = threadIdx.x; e < (int64_t)nb * nb; e += 256) Q[e] = (e / nb == e % nb) ? 1.f : 0.f;
}

__global__ void __launch_bounds__(256) k_qr_finish(int nb, int nblk, const int8_t *neg_all, OutTable t, int info_value) {
    const int g = blockIdx.x;
    const int b = g % nblk, mat = g / nblk;
    float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    const int8_t *neg = neg_all + (int64_t)g * nb;
    for (int64_t e = threadIdx.x; e < (int64_t)nb * nb; e += 256)
        if (neg[e % nb]) Q[e] = -Q[e];
    if (threadIdx.x == 0 && info_value > 0 && t.info[mat]) t.info[mat][b] = info_value;
}

// lambda_j = q_j^T (A q_j), with T = A Q in the workspace; info = k when k >= 0.  grid.x = blocks.
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
    if (threadIdx.x == 0 && t.info[mat] && k >= 0) t.info[mat][b] = k;   // k < 0: info is written elsewhere
}

// ---- workspace layout: five regions, each an array of dense per-block records ----------------
inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }
struct Regions {
    size_t aw, v, t, tlog, state, tq, neg, total;
};
Regions regions(int64_t nb, int64_t nblocks) {
    const int64_t nbp = (nb + 1) / 2 * 2;
    Regions R;
    R.aw = al256((size_t)nbp * nbp * 8 * nblocks);  // Aw: nbp x nbp, fp32 (first stage) then fp64
    R.v = al256((size_t)nb * nb * 8 * nblocks);     // V: nb x nb fp64
    R.t = al256((size_t)nb * nb * 8 * nblocks);     // T: nb x nb, fp32 (A Q products) or fp64 (refinement),
                                                    // or the block-Jacobi rotations (fewer than nb^2 per block)
    R.tlog = al256((size_t)(nbp - 1) * (nbp / 2) * 8 * nblocks);   // tangents of one sweep
    R.state = al256((size_t)16 * nblocks);                         // 4 ints
    R.tq = al256((size_t)((nb + kQP - 1) / kQP) * kQP * kQP * 4 * nblocks);  // QR panel T factors
    R.neg = al256((size_t)nb * nblocks);                                      // signs of diag(R)
    R.total = R.aw + R.v + R.t + R.tlog + R.state + R.tq + R.neg;
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

}  // namespace

size_t refresh_ws(const dobb_shape &sh, int count) {
    const int cnt = count < kMaxMats ? count : kMaxMats;
    return regions(sh.nb, (sh.n / sh.nb) * cnt).total;
}

// the block-Jacobi sweeps: per sweep m - 1 rounds of k_bj_sub and k_bj_apply, then the bookkeeping
template <int B2>
hipError_t launch_bj(int nb, int nbp, int m, int sweeps, dim3 gs, dim3 ga, size_t ls, size_t la, double *Aw64,
                     double *V, double *Rw, int32_t *nrot, int32_t *state, hipStream_t s) {
    (void)hipFuncSetAttribute((const void *)k_bj_sub<B2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ls);
    (void)hipFuncSetAttribute((const void *)k_bj_apply<B2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)la);
    for (int sw = 0; sw < sweeps; ++sw) {
        for (int r = 0; r < m - 1; ++r) {
            DOBB_LAUNCH("jacobi_block_sub", s, k_bj_sub<B2>, gs, dim3(kBjThreads), ls, nb, nbp, r, kTolFp64, Aw64, Rw, nrot,
                        state);
            DOBB_LAUNCH("jacobi_block_apply", s, k_bj_apply<B2>, ga, dim3(256), la, nb, nbp, r, Aw64, V, (const double *)Rw,
                        (const int32_t *)nrot, (const int32_t *)state);
        }
        DOBB_LAUNCH("jacobi_sweep_end", s, k_bj_sweep_end, dim3(gs.y), dim3(64), 0, state);
    }
    return hipGetLastError();
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
        float *tq = (float *)(base + R.aw + R.v + R.t + R.tlog + R.state);
        int8_t *negs = (int8_t *)(base + R.aw + R.v + R.t + R.tlog + R.state + R.tq);
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
        // the 16 x 16 MFMA tiles where 16 NT fits the width: 80 for multiples of 80, one tile per
        // block up to 128 (the 32 x 32 tiles' 64 x 64 workgroup tiles otherwise)
        const int tnt = nb % 80 == 0 ? 5 : nb <= 48 ? 3 : nb <= 96 ? 6 : nb <= 112 ? 7 : nb <= 128 ? 8 : 0;
        const int tT = tnt ? (nb + 16 * tnt - 1) / (16 * tnt) : 0;
        const dim3 gtile((unsigned)(tT * tT * nblocks));
#define DOBB_BGEMM_T(NT, TR, OA, OB, OC)                                                                          \
    do {                                                                                                          \
        if (nb % 4 == 0) DOBB_LAUNCH("refresh_gemm", s, (k_bgemm_t<NT, TR, true>), gtile, dim3(64 * NT), 0, nb, tT, nblk, OA, OB, OC); \
        else DOBB_LAUNCH("refresh_gemm", s, (k_bgemm_t<NT, TR, false>), gtile, dim3(64 * NT), 0, nb, tT, nblk, OA, OB, OC);         \
    } while (0)
#define DOBB_BGEMM(TR, OA, OB, OC)                                                                               \
    do {                                                                                                         \
        switch (tnt) {                                                                                           \
        case 3: DOBB_BGEMM_T(3, TR, OA, OB, OC); break;                                                         \
        case 5: DOBB_BGEMM_T(5, TR, OA, OB, OC); break;                                                         \
        case 6: DOBB_BGEMM_T(6, TR, OA, OB, OC); break;                                                         \
        case 7: DOBB_BGEMM_T(7, TR, OA, OB, OC); break;                                                         \
        case 8: DOBB_BGEMM_T(8, TR, OA, OB, OC); break;                                                         \
        default:                                                                                                 \
            if (nb % 4 == 0) DOBB_LAUNCH("refresh_gemm", s, (k_bgemm<TR, true>), ggemm, dim3(256), 0, nb, T, nblk, OA, OB, OC); \
            else DOBB_LAUNCH("refresh_gemm", s, (k_bgemm<TR, false>), ggemm, dim3(256), 0, nb, T, nblk, OA, OB, OC);         \
        }                                                                                                        \
    } while (0)

        const bool block_jacobi = a.mode == DOBB_REFRESH_EXACT && (int64_t)jacobi_lds_bytes(nbp, 4) > lds_max;
        if (block_jacobi) {
            // one fp64 stage: Aw64 = V^T A V (V = I or Q_prev, widened), block-Jacobi sweeps to the
            // refinement threshold, then the common finalisation
            JacTable jt{};
            for (int i = 0; i < cnt; ++i) { jt.A[i] = a.A[c0 + i]; jt.Qp[i] = a.Q[c0 + i]; }
            DOBB_LAUNCH("jacobi_init", s, k_jacobi_init, dim3((unsigned)nblocks), dim3(256), 0, nb, nbp, nblk, a.warm, jt,
                        Aw, V, state);
            double *Aw64 = (double *)Aw;
            double *T64 = (double *)Tm;
            const int tiles = (nb + 15) / 16;
            const dim3 gr((unsigned)(tiles * tiles), (unsigned)nblocks);
            DOBB_LAUNCH("jacobi_refine_gemm", s, k_refine_gemm, gr, dim3(256), 0, nb, nbp, nblk, 0, jt, (const double *)V,
                        T64, Aw64, state);
            DOBB_LAUNCH("jacobi_refine_gemm", s, k_refine_gemm, gr, dim3(256), 0, nb, nbp, nblk, 1, jt, (const double *)V,
                        T64, Aw64, state);
            DOBB_LAUNCH("jacobi_symmetrize", s, k_symmetrize64, dim3((unsigned)nblocks), dim3(256), 0, nbp, Aw64);
            DOBB_LAUNCH("jacobi_stage_flag", s, k_bj_begin, dim3((unsigned)nblocks), dim3(64), 0, state);
            const BjGeo G = bj_geo(nb);
            const int b2 = 2 * G.b, np2 = G.m / 2, nrt = (nb + b2 - 1) / b2;
            double *Rw = T64;                        // the rotations of a round: np2 x b2 x b2 per block
            int32_t *nrot = (int32_t *)tlog;         // their counts: np2 per block
            const size_t ls = bj_sub_lds(nb), la = bj_apply_lds(nb);
            const dim3 gs((unsigned)np2, (unsigned)nblocks), ga((unsigned)(np2 * (np2 - 1) / 2 + np2 * nrt), (unsigned)nblocks);
            const int sweeps = a.iters > 0 ? a.iters : 30;
            hipError_t eb = hipSuccess;
            switch (b2) {
#define DOBB_BJ(B2) case B2: eb = launch_bj<B2>(nb, nbp, G.m, sweeps, gs, ga, ls, la, Aw64, V, Rw, nrot, state, s); break;
                DOBB_BJ(8) DOBB_BJ(16) DOBB_BJ(24) DOBB_BJ(32) DOBB_BJ(40) DOBB_BJ(48) DOBB_BJ(56) DOBB_BJ(64)
                DOBB_BJ(72) DOBB_BJ(80)
#undef DOBB_BJ
                default: return hipErrorInvalidValue;
            }
            if (eb != hipSuccess) return eb;
            DOBB_LAUNCH("jacobi_finalize", s, k_jacobi_finalize, dim3((unsigned)nblocks), dim3(256), (size_t)nb * 8, nb, nbp,
                        nblk, (const double *)Aw64, (const double *)V, (const int32_t *)state, ot);
        } else if (a.mode == DOBB_REFRESH_EXACT) {
            if (a.warm) {
                DOBB_BGEMM(false, opA, opQ, outT);
                Opnd opT{};
                OutOpnd outAw{};
                for (int i = 0; i < cnt; ++i) {
                    opT.p[i] = Tm + (int64_t)i * nblk * t_stride;
                    outAw.p[i] = Aw + (int64_t)i * nblk * aw_stride;
                }
                opT.blk_stride = t_stride; opT.ld = nb;
                outAw.blk_stride = aw_stride; outAw.ld = nbp;
                DOBB_BGEMM(true, opQ, opT, outAw);
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
        } else if (a.mode == DOBB_REFRESH_ORTH_ITER_CHOLQR) {
            // Z = A Q in the first half of the T region, the first pass's result in its second half;
            // the Gram matrix (then R) and R^{-1} in the working-matrix region; a flag per block
            float *Q1 = Tm + t_stride * nblocks;
            float *Gm = Aw, *Xm = Aw + t_stride * nblocks;
            Opnd opZ{}, opQ1{}, opX{};
            OutOpnd outG{}, outQ1{}, outQ{};
            for (int i = 0; i < cnt; ++i) {
                const int64_t o = (int64_t)i * nblk * t_stride;
                opZ.p[i] = Tm + o; opQ1.p[i] = Q1 + o; opX.p[i] = Xm + o;
                outG.p[i] = Gm + o; outQ1.p[i] = Q1 + o; outQ.p[i] = a.Q[c0 + i];
            }
            opZ.blk_stride = opQ1.blk_stride = opX.blk_stride = t_stride;
            outG.blk_stride = outQ1.blk_stride = outQ.blk_stride = t_stride;
            opZ.ld = opQ1.ld = opX.ld = outG.ld = outQ1.ld = outQ.ld = nb;
            for (int it = 0; it < a.iters; ++it) {
                DOBB_BGEMM(false, opA, opQ, outT);                                        // Z = A Q
                DOBB_BGEMM(true, opZ, opZ, outG);                                         // Z^T Z
                hipError_t e = launch_chol_inv(nb, (int)nblocks, Gm, Xm, state, it == 0, s);
                if (e != hipSuccess) return e;
                DOBB_BGEMM(false, opZ, opX, outQ1);                                       // Z R^{-1}
                DOBB_BGEMM(true, opQ1, opQ1, outG);                                       // second pass
                e = launch_chol_inv(nb, (int)nblocks, Gm, Xm, state, 0, s);
                if (e != hipSuccess) return e;
                DOBB_BGEMM(false, opQ1, opX, outQ);
            }
            hipError_t e = launch_chol_info(nblk, (int)nblocks, state, ot.info, cnt, a.iters, s);
            if (e != hipSuccess) return e;
            bool want_lam = false;
            for (int i = 0; i < cnt; ++i) want_lam |= ot.lam[i] != nullptr;
            if (want_lam) {
                DOBB_BGEMM(false, opA, opQ, outT);
                DOBB_LAUNCH("rayleigh", s, k_rayleigh, dim3((unsigned)nblocks), dim3(256), 0, nb, nblk, (const float *)Tm, ot,
                            -1);
            }
        } else {
            // blocks up to 512 wide: k_qr.hip's kernels; wider ones: one launch per panel step
            const size_t pl = qr_panel_layout(nb).total;
            (void)hipFuncSetAttribute((const void *)k_qr_panel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl);
            const int npanel = (nb + kQP - 1) / kQP;
            for (int it = 0; it < a.iters; ++it) {
                DOBB_BGEMM(false, opA, opQ, outT);
                const int infov = it == a.iters - 1 ? a.iters : 0;
                if (qr_block_supported(nb)) {
                    const hipError_t e = launch_qr_block(nb, nblk, cnt, Tm, tq, negs, ot.Q, ot.info, infov, s);
                    if (e != hipSuccess) return e;
                    continue;
                }
                for (int p = 0; p < npanel; ++p) {
                    DOBB_LAUNCH("qr_panel", s, k_qr_panel, dim3((unsigned)nblocks), dim3(256), pl, nb, p, Tm, tq, negs);
                    const int first = p * kQP + (nb - p * kQP < kQP ? nb - p * kQP : kQP);
                    const int ntiles = (nb - first + 63) / 64;
                    if (ntiles > 0)
                        DOBB_LAUNCH("qr_update", s, k_qr_update<true>, dim3((unsigned)ntiles, (unsigned)nblocks), dim3(256), 0, nb,
                                    nblk, p, (const float *)Tm, (const float *)tq, ot);
                }
                DOBB_LAUNCH("qr_identity", s, k_qr_identity, dim3((unsigned)nblocks), dim3(256), 0, nb, nblk, ot);
                for (int p = npanel - 1; p >= 0; --p) {
                    const int ntiles = (nb - p * kQP + 63) / 64;
                    DOBB_LAUNCH("qr_form", s, k_qr_update<false>, dim3((unsigned)ntiles, (unsigned)nblocks), dim3(256), 0, nb,
                                nblk, p, (const float *)Tm, (const float *)tq, ot);
                }
                DOBB_LAUNCH("qr_finish", s, k_qr_finish, dim3((unsigned)nblocks), dim3(256), 0, nb, nblk, (const int8_t *)negs,
                            ot, infov);
            }
            bool want_lam = false;
            for (int i = 0; i < cnt; ++i) want_lam |= ot.lam[i] != nullptr;
            if (want_lam) {
                DOBB_BGEMM(false, opA, opQ, outT);
                DOBB_LAUNCH("rayleigh", s, k_rayleigh, dim3((unsigned)nblocks), dim3(256), 0, nb, nblk, (const float *)Tm, ot,
                            a.iters);
            }
        }
        #undef DOBB_BGEMM
        #undef DOBB_BGEMM_T
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
