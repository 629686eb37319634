// Cholesky QR for the orthogonal-iteration refresh (Table 16 of the Dobb paper, arXiv 2610.39412:
// "Cholesky" as the QR routine, next to the principal Householder).  A pass turns Z into Z R^{-1}
// with G = Z^T Z = R^T R; two passes (CholeskyQR2) give the orthonormal factor with diag(R) > 0.
// The products Z^T Z and Z R^{-1} run on the batched GEMM of k_refresh.hip; this file factors the
// Gram matrix and inverts R, one workgroup (4 waves) per block, with the block's matrices in global
// memory (L2) and one 32-row panel in LDS:
//   Cholesky, left-looking by panels of 32 rows of R:
//     T = G[panel rows, p:] - R[:p, panel rows]^T R[:p, p:]      (fp32 MFMA tiles, K = 32 p)
//     T's 32 x 32 diagonal block is factored right-looking in LDS, then every thread solves one column
//     of the rest of the panel, R_pp^T x = t, by forward substitution; the panel's rows of R
//     overwrite those of G.
//   Inverse X = R^{-1}, by panels of 32 columns:
//     thread l < 32 inverts column l of R_pp by back substitution, and
//     X[:p, panel] = -(X[:p, :p] R[:p, panel]) X_pp                (fp32 MFMA tiles, then a 32-wide product)
// A pivot that is not positive (a numerically rank-deficient Z) is replaced by 1 and flagged; the
// refresh then reports info = -1 for the block.
#include "dobb_internal.h"

namespace dobb {
namespace {

constexpr int kCP = 32;   // panel width

struct CholLayout {
    int ldt;                    // pitch of the panel rows (floats)
    size_t tp, yt, xp, xi, total;   // byte offsets: panel [32][ldt], Y tile [64][33], R_pp and X_pp [32][33]
};
__host__ __device__ inline CholLayout chol_layout(int nb) {
    CholLayout L;
    L.ldt = nb + 1;
    size_t o = 0;
    L.tp = o; o += (size_t)kCP * L.ldt * 4;
    o = (o + 15) / 16 * 16;
    L.yt = o; o += (size_t)64 * 33 * 4;
    L.xp = o; o += (size_t)kCP * 33 * 4;
    L.xi = o; o += (size_t)kCP * 33 * 4;
    L.total = o;
    return L;
}

// grid.x = blocks, block 256.  G: nb x nb per block (in: Z^T Z; out: R in its upper triangle and the
// rows' lower parts left as they were); X: nb x nb per block (out: R^{-1}, zero below the diagonal).
__global__ void __launch_bounds__(256) k_chol_inv(int nb, float *G_all, float *X_all, int32_t *flag_all, int first) {
    __shared__ GemmSmem2 sm;
    extern __shared__ __align__(16) unsigned char dsm[];
    const CholLayout L = chol_layout(nb);
    float *tp = (float *)(dsm + L.tp);                 // [32][ldt]
    float (*yt)[33] = (float (*)[33])(dsm + L.yt);     // [64][33]
    float (*xp)[33] = (float (*)[33])(dsm + L.xp);     // [32][33] R_pp
    float (*xi)[33] = (float (*)[33])(dsm + L.xi);     // [32][33] X_pp = R_pp^{-1}
    const int ldt = L.ldt;
    const int g = blockIdx.x;
    float *G = G_all + (int64_t)g * nb * nb;
    float *X = X_all + (int64_t)g * nb * nb;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wr = 32 * (wv >> 1), wc = 32 * (wv & 1);
    const int NP = (nb + kCP - 1) / kCP;
    int bad = 0;   // thread 0

    // ---- Cholesky: R overwrites G's rows, panel by panel ----
    for (int p = 0; p < NP; ++p) {
        const int r0 = kCP * p, w = nb - r0 < kCP ? nb - r0 : kCP, ncol = nb - r0;
        // T = G[r0:r0+w, r0:nb] - R[0:r0, r0:r0+w]^T R[0:r0, r0:nb] -> tp (local column c - r0)
        for (int c0 = r0; c0 < nb; c0 += kBN) {
            LoadColsK<false> la{G + r0, nb, w, r0};             // a[k][i] = R[k][r0 + i]
            LoadColsK<false> lb{G + c0, nb, nb - c0, r0};       // b[k][j] = R[k][c0 + j]
            const f32x16 acc = gemm_tile(r0, la, lb, sm);
            if (wr == 0) {
                const int j = c0 + wc + acc_col(lane);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = acc_row(r, lane);
                    if (i < w && j < nb) tp[i * ldt + (j - r0)] = G[(int64_t)(r0 + i) * nb + j] - acc[r];
                }
            }
        }
        __syncthreads();
        // the 32 x 32 diagonal block, right-looking in LDS: row i is scaled by its pivot, then the rows
        // below it lose r_i^T r_i (upper parts only)
        for (int i = 0; i < w; ++i) {
            const float dii = tp[i * ldt + i];
            const bool ok = dii > 0.f;
            const float rii = ok ? __builtin_sqrtf(dii) : 1.f;
            if (tid == 0 && !ok) bad = 1;
            if (tid >= i && tid < w) tp[i * ldt + tid] = tid == i ? rii : tp[i * ldt + tid] / rii;
            __syncthreads();
            const int rem = w - 1 - i;
            for (int e = tid; e < rem * rem; e += 256) {
                const int j = i + 1 + e / rem, c = i + 1 + e % rem;
                if (c >= j) tp[j * ldt + c] = __builtin_fmaf(-tp[i * ldt + j], tp[i * ldt + c], tp[j * ldt + c]);
            }
            __syncthreads();
        }
        // below the diagonal of the block: zeros
        for (int e = tid; e < w * w; e += 256) {
            const int j = e / w, c = e % w;
            if (c < j) tp[j * ldt + c] = 0.f;
        }
        // the rest of the panel: R_pp^T x = t for each column c >= w (forward substitution, in place)
        for (int cc = w + tid; cc < ncol; cc += 256) {
            for (int i = 0; i < w; ++i) {
                float s = tp[i * ldt + cc];
                for (int k = 0; k < i; ++k) s = __builtin_fmaf(-tp[k * ldt + i], tp[k * ldt + cc], s);
                tp[i * ldt + cc] = s / tp[i * ldt + i];
            }
        }
        __syncthreads();
        // the panel's rows of R (the upper part; the diagonal block's lower part holds zeros)
        for (int e = tid; e < w * ncol; e += 256) {
            const int i = e / ncol, c = e - i * ncol;
            G[(int64_t)(r0 + i) * nb + r0 + c] = tp[i * ldt + c];
        }
        __syncthreads();
    }
    if (tid == 0) flag_all[g] = first ? bad : (flag_all[g] | bad);
    __syncthreads();

    // ---- inverse X = R^{-1}, panel of columns by panel ----
    for (int p = 0; p < NP; ++p) {
        const int r0 = kCP * p, w = nb - r0 < kCP ? nb - r0 : kCP;
        // R_pp -> xp; lanes l < w of wave 0 each solve R_pp x = e_l (back substitution) into column l of xi
        for (int e = tid; e < kCP * kCP; e += 256) {
            const int i = e / kCP, j = e - i * kCP;
            xp[i][j] = (i < w && j < w && j >= i) ? G[(int64_t)(r0 + i) * nb + r0 + j] : (i == j ? 1.f : 0.f);
        }
        __syncthreads();
        if (tid < w) {
            const int l = tid;
            for (int i = kCP - 1; i >= 0; --i) {
                float v = 0.f;
                if (i <= l) {
                    float s = i == l ? 1.f : 0.f;
                    for (int k = i + 1; k <= l; ++k) s = __builtin_fmaf(-xp[i][k], xi[k][l], s);
                    v = s / xp[i][i];
                }
                xi[i][l] = v;
            }
        }
        __syncthreads();
        // rows above the panel: X[i0:i0+64, r0:r0+w] = -(X[i0:, 0:r0] R[0:r0, r0:r0+w]) X_pp
        for (int i0 = 0; i0 < r0; i0 += kBM) {
            const int rows = r0 - i0 < kBM ? r0 - i0 : kBM;
            LoadRowsT<false> la{X + (int64_t)i0 * nb, nb, rows, r0};   // a[k][i] = X[i0 + i][k]
            LoadColsK<false> lb{G + r0, nb, w, r0};                     // b[k][j] = R[k][r0 + j]
            const f32x16 acc = gemm_tile(r0, la, lb, sm);
            if (wc == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) yt[wr + acc_row(r, lane)][acc_col(lane)] = acc[r];
            }
            __syncthreads();
            for (int e = tid; e < rows * w; e += 256) {
                const int i = e / w, j = e - i * w;
                float s = 0.f;
                for (int k = 0; k <= j; ++k) s = __builtin_fmaf(yt[i][k], xi[k][j], s);
                X[(int64_t)(i0 + i) * nb + r0 + j] = -s;
            }
            __syncthreads();
        }
        // the panel's own rows: zero left of the diagonal, X_pp on it
        for (int e = tid; e < w * (r0 + w); e += 256) {
            const int i = e / (r0 + w), c = e - i * (r0 + w);
            X[(int64_t)(r0 + i) * nb + c] = c < r0 + i ? 0.f : xi[i][c - r0];
        }
        __syncthreads();
    }
}

struct InfoTable {
    int32_t *info[kMaxMats];
};
__global__ void k_chol_info(int nblk, int nblocks, const int32_t *flag_all, InfoTable t, int info_value) {
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= nblocks) return;
    int32_t *inf = t.info[g / nblk];
    if (inf) inf[g % nblk] = flag_all[g] ? -1 : info_value;
}

}  // namespace

bool chol_supported(int64_t nb) { return nb >= 1 && (int64_t)chol_layout((int)nb).total + (int64_t)sizeof(GemmSmem2) <= max_lds_bytes(); }

hipError_t launch_chol_inv(int nb, int nblocks, float *G, float *X, int32_t *flag, int first, hipStream_t s) {
    const size_t lds = chol_layout(nb).total;
    (void)hipFuncSetAttribute((const void *)k_chol_inv, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    DOBB_LAUNCH("cholqr_factor", s, k_chol_inv, dim3((unsigned)nblocks), dim3(256), lds, nb, G, X, flag, first);
    return hipGetLastError();
}

hipError_t launch_chol_info(int nblk, int nblocks, const int32_t *flag, int32_t *const *info, int cnt, int info_value,
                            hipStream_t s) {
    InfoTable t{};
    for (int i = 0; i < cnt; ++i) t.info[i] = info[i];
    DOBB_LAUNCH("cholqr_info", s, k_chol_info, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, nblk, nblocks, flag,
                t, info_value);
    return hipGetLastError();
}

}  // namespace dobb
