// The Dobb step on gfx950: momentum, projection into the block eigenbases with the sign epilogue,
// and reconstruction with the fused decoupled-weight-decay update.
//
// Dobb paper (arXiv 2610.39412), abstract: momentum is projected into the per-block bases, the
// coefficients are sign-normalised and the update is reconstructed; Table 9 fixes the update scale,
// Table 21's note the decoupled weight decay (it reads only the weights), Table 19 the Nesterov
// ablation and Tables 11-12 the column-l2 variant (Dobb-l2).
//
// Kernels (one launch each per group of equally shaped matrices):
//   k_momentum     M <- mu M + G                           HBM-bound elementwise pass
//   k_project      C_b = P_b Q_b, S = sign(C) as int8     fp32 MFMA 32x32x2, K = nb
//   k_colnorm      colscale_j = 1/||C[:, j]||             (column-l2 variant only; 16 row groups per column)
//   k_reconstruct  U_b = S_b Q_b^T, W <- W - lr (s U + wd W)   fp32 MFMA, K = nb
#include "dobb_internal.h"

namespace dobb {
namespace {

struct MomTable {
    const void *G[kMaxMats];
    float *M[kMaxMats];
    float mu[kMaxMats];
};

template <bool GBF16, bool VEC>
__global__ void __launch_bounds__(256) k_momentum(int64_t numel, MomTable t) {
    const int mat = blockIdx.y;
    float *__restrict__ M = t.M[mat];
    const float mu = t.mu[mat];
    const int64_t stride = (int64_t)gridDim.x * 256;
    if (VEC) {
        const int64_t nv = numel >> 2;
        for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nv; v += stride) {
            f32x4 m = ((const f32x4 *)M)[v];
            f32x4 g;
            if (GBF16) {
                uint2 h = ((const uint2 *)t.G[mat])[v];
                g[0] = bf16_to_f32((uint16_t)(h.x & 0xffff)); g[1] = bf16_to_f32((uint16_t)(h.x >> 16));
                g[2] = bf16_to_f32((uint16_t)(h.y & 0xffff)); g[3] = bf16_to_f32((uint16_t)(h.y >> 16));
            } else {
                g = ((const f32x4 *)t.G[mat])[v];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) m[c] = __builtin_fmaf(mu, m[c], g[c]);
            ((f32x4 *)M)[v] = m;
        }
        // tail (numel % 4) handled by the scalar loop below starting at 4*nv
        for (int64_t e = (nv << 2) + (int64_t)blockIdx.x * 256 + threadIdx.x; e < numel; e += stride) {
            float g = GBF16 ? bf16_to_f32(((const uint16_t *)t.G[mat])[e]) : ((const float *)t.G[mat])[e];
            M[e] = __builtin_fmaf(mu, M[e], g);
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < numel; e += stride) {
            float g = GBF16 ? bf16_to_f32(((const uint16_t *)t.G[mat])[e]) : ((const float *)t.G[mat])[e];
            M[e] = __builtin_fmaf(mu, M[e], g);
        }
    }
}

struct ProjTable {
    const float *M[kMaxMats];
    const void *G[kMaxMats];
    const float *Q[kMaxMats];
    int8_t *S[kMaxMats];
    float *C[kMaxMats];
    float *Cout[kMaxMats];     // NULL or m x n fp32: the coefficients (verification output)
    float mu[kMaxMats];
};

// a[k][i] = G + mu M  (Nesterov input), from the momentum already updated by k_momentum
template <bool GBF16>
struct LoadNesterovT {
    const float *M; const void *G; int64_t off; int64_t ld; int rows; int K; float mu;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, i = t >> 2, k = k0 + 4 * (t & 3);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v[c] = 0.f;
            if (i < rows && k + c < K) {
                int64_t e = off + (int64_t)i * ld + k + c;
                float g = GBF16 ? bf16_to_f32(((const uint16_t *)G)[e]) : ((const float *)G)[e];
                v[c] = __builtin_fmaf(mu, M[e], g);
            }
        }
    }
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBM]) const {
        const int t = threadIdx.x, i = t >> 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[4 * (t & 3) + c][i ^ gemm_swz(4 * (t & 3) + c)] = v[c];
    }
};

// grid.x = col_tiles * B * count (column tile fastest), grid.y = row tiles of 64
template <bool VEC, int NEST /*0 none, 1 G fp32, 2 G bf16*/, bool SIGN>
__global__ void __launch_bounds__(256) k_project(int64_t m, int64_t n, int nb, int col_tiles, int nblk, ProjTable t) {
    __shared__ GemmSmem2 sm;
    const int ct = blockIdx.x % col_tiles;
    const int rest = blockIdx.x / col_tiles;
    const int b = rest % nblk, mat = rest / nblk;
    const int64_t r0 = (int64_t)blockIdx.y * kBM;
    const int c0 = ct * kBN;
    const int rows = (int)min<int64_t>(kBM, m - r0);
    const int cols = nb - c0;
    const int64_t off = r0 * n + (int64_t)b * nb;
    const float *Qb = t.Q[mat] + (int64_t)b * nb * nb + c0;
    LoadColsK<VEC> lb{Qb, nb, cols, nb};
    f32x16 acc;
    if (NEST == 0) {
        LoadRowsT<VEC> la{t.M[mat] + off, n, rows, nb};
        acc = gemm_tile(nb, la, lb, sm);
    } else {
        LoadNesterovT<NEST == 2> la{t.M[mat], t.G[mat], off, n, rows, nb, t.mu[mat]};
        acc = gemm_tile(nb, la, lb, sm);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wr = 32 * (w >> 1), wc = 32 * (w & 1);
    const int col = wc + acc_col(lane);
    if (col < cols) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wr + acc_row(r, lane);
            if (row < rows) {
                const int64_t e = off + (int64_t)row * n + c0 + col;
                if (SIGN) t.S[mat][e] = sign_code(acc[r]);
                else t.C[mat][e] = acc[r];
                if (t.Cout[mat]) t.Cout[mat][e] = acc[r];
            }
        }
    }
}

struct ColTable {
    float *C[kMaxMats];
    float *cs[kMaxMats];
};

// colscale_j = 1 / ||C[:, j]||_2 (0 for a zero column), summed in fp64.  grid = (ceil(n / 64), matrices),
// block 1024: thread (g, c) sums column 64 blockIdx.x + c over rows g, g + 16, ... (64 consecutive
// columns per row: 256-byte reads), then the 16 partial sums are added in g order (deterministic).
constexpr int kCnCols = 64, kCnGroups = 16;
__global__ void __launch_bounds__(kCnCols * kCnGroups) k_colnorm(int64_t m, int64_t n, ColTable t) {
    __shared__ double part[kCnGroups][kCnCols];
    const int mat = blockIdx.y;
    const int c = threadIdx.x % kCnCols, g = threadIdx.x / kCnCols;
    const int64_t j = (int64_t)blockIdx.x * kCnCols + c;
    const float *C = t.C[mat];
    double s = 0.0;
    if (j < n)
        for (int64_t r = g; r < m; r += kCnGroups) {
            const double v = C[r * n + j];
            s += v * v;
        }
    part[g][c] = s;
    __syncthreads();
    if (g == 0 && j < n) {
        double tot = 0.0;
#pragma unroll
        for (int q = 0; q < kCnGroups; ++q) tot += part[q][c];
        t.cs[mat][j] = tot > 0.0 ? (float)(1.0 / sqrt(tot)) : 0.f;
    }
}

struct ReconTable {
    const int8_t *S[kMaxMats];
    const float *C[kMaxMats];
    const float *cs[kMaxMats];
    const float *Q[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};

// a[k][i] = sign code decoded, from S (int8, row-major)
template <bool VEC>
struct LoadSignT {
    const int8_t *src; int64_t ld; int rows; int K;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, i = t >> 2, k = k0 + 4 * (t & 3);
        v[0] = v[1] = v[2] = v[3] = 0.f;
        if (i < rows) {
            const int8_t *p = src + (int64_t)i * ld + k;
            if (VEC) {
                if (k < K) {
                    uint32_t q = *(const uint32_t *)p;
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = sign_decode((int8_t)((q >> (8 * c)) & 0xff));
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) if (k + c < K) v[c] = sign_decode(p[c]);
            }
        }
    }
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBM]) const {
        const int t = threadIdx.x, i = t >> 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[4 * (t & 3) + c][i ^ gemm_swz(4 * (t & 3) + c)] = v[c];
    }
};

// a[k][i] = C * colscale (column-l2) or C (identity).  VEC: nb and n multiples of 4, and C and the
// scales in the 256-byte-aligned workspace, so a row's four k sit in one 16-byte piece
template <bool SCALED, bool VEC>
struct LoadCoefT {
    const float *src; const float *cs; int64_t ld; int rows; int K;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, i = t >> 2, k = k0 + 4 * (t & 3);
        if (VEC) {
            f32x4 q = {0.f, 0.f, 0.f, 0.f};
            if (i < rows && k < K) {
                q = *(const f32x4 *)(src + (int64_t)i * ld + k);
                if (SCALED) {
                    const f32x4 c4 = *(const f32x4 *)(cs + k);
#pragma unroll
                    for (int c = 0; c < 4; ++c) q[c] *= c4[c];
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = q[c];
            return;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v[c] = 0.f;
            if (i < rows && k + c < K) {
                v[c] = src[(int64_t)i * ld + k + c];
                if (SCALED) v[c] *= cs[k + c];
            }
        }
    }
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBM]) const {
        const int t = threadIdx.x, i = t >> 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[4 * (t & 3) + c][i ^ gemm_swz(4 * (t & 3) + c)] = v[c];
    }
};

template <bool VEC, int AMODE /*0 sign codes, 1 C, 2 C*colscale*/, bool WBF16>
__global__ void __launch_bounds__(256) k_reconstruct(int64_t m, int64_t n, int nb, int col_tiles, int nblk, ReconTable t) {
    __shared__ GemmSmem2 sm;
    const int ct = blockIdx.x % col_tiles;
    const int rest = blockIdx.x / col_tiles;
    const int b = rest % nblk, mat = rest / nblk;
    const int64_t r0 = (int64_t)blockIdx.y * kBM;
    const int c0 = ct * kBN;
    const int rows = (int)min<int64_t>(kBM, m - r0);
    const int cols = nb - c0;
    const int64_t off = r0 * n + (int64_t)b * nb;
    // B operand: b[k][j] = Q_b[c0 + j][k]  (Q_b^T), a row-major read of Q_b's rows c0..c0+63
    LoadRowsT<VEC> lb{t.Q[mat] + (int64_t)b * nb * nb + (int64_t)c0 * nb, nb, cols, nb};
    f32x16 acc;
    if (AMODE == 0) {
        LoadSignT<VEC> la{t.S[mat] + off, n, rows, nb};
        acc = gemm_tile(nb, la, lb, sm);
    } else {
        LoadCoefT<AMODE == 2, VEC> la{t.C[mat] + off, t.cs[mat] + (int64_t)b * nb, n, rows, nb};
        acc = gemm_tile(nb, la, lb, sm);
    }
    const float lr = t.lr[mat], wd = t.wd[mat], sc = t.scale[mat];
    float *U = t.U[mat];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wr = 32 * (w >> 1), wc = 32 * (w & 1);
    const int col = wc + acc_col(lane);
    if (col < cols) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wr + acc_row(r, lane);
            if (row < rows) {
                const int64_t e = off + (int64_t)row * n + c0 + col;
                const float u = acc[r];
                if (U) U[e] = u;
                if (WBF16) {
                    uint16_t *W = (uint16_t *)t.W[mat];
                    const float wv = bf16_to_f32(W[e]);
                    W[e] = f32_to_bf16(wv - lr * __builtin_fmaf(sc, u, wd * wv));
                } else {
                    float *W = (float *)t.W[mat];
                    const float wv = W[e];
                    W[e] = wv - lr * __builtin_fmaf(sc, u, wd * wv);
                }
            }
        }
    }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_momentum(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    const int64_t numel = a.sh.m * a.sh.n;
    MomTable t{};
    bool vec = numel % 4 == 0;
    for (int i = 0; i < cnt; ++i) {
        t.G[i] = a.G[c0 + i]; t.M[i] = a.M[c0 + i]; t.mu[i] = a.hp[c0 + i].momentum;
        vec = vec && aligned16(t.G[i]) && aligned16(t.M[i]);
    }
    const int64_t want = (numel / 4 + 255) / 256;
    const int gx = (int)(want < 2048 ? (want > 0 ? want : 1) : 2048);
    const dim3 grid(gx, cnt);
    if (a.g_dtype == DOBB_BF16) {
        if (vec) DOBB_LAUNCH("momentum", s, (k_momentum<true, true>), grid, dim3(256), 0, numel, t);
        else DOBB_LAUNCH("momentum", s, (k_momentum<true, false>), grid, dim3(256), 0, numel, t);
    } else {
        if (vec) DOBB_LAUNCH("momentum", s, (k_momentum<false, true>), grid, dim3(256), 0, numel, t);
        else DOBB_LAUNCH("momentum", s, (k_momentum<false, false>), grid, dim3(256), 0, numel, t);
    }
    return hipGetLastError();
}

hipError_t launch_colnorm(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    ColTable t{};
    for (int i = 0; i < cnt; ++i) { t.C[i] = a.C[c0 + i]; t.cs[i] = a.colscale[c0 + i]; }
    dim3 grid((unsigned)((a.sh.n + kCnCols - 1) / kCnCols), cnt);
    DOBB_LAUNCH("colnorm", s, k_colnorm, grid, dim3(kCnCols * kCnGroups), 0, a.sh.m, a.sh.n, t);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const int col_tiles = (nb + kBN - 1) / kBN;
    const int row_tiles = (int)((m + kBM - 1) / kBM);
    for (int c0 = 0; c0 < a.count;) {
        // chunk: at most kMaxMats matrices, and blocks * matrices within grid.x limits
        int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        // column-l2 with nb <= 128: the split-fp16 rows kernels do momentum, projection, column norms
        // and reconstruction
        if (a.hp[c0].norm == DOBB_NORM_COL_L2 && a.colpart && proj_l2_rows_eligible(a.sh)) {
            bool al = true;
            for (int i = 0; i < cnt; ++i)
                al = al && aligned16(a.M[c0 + i]) &&
                     ((uintptr_t)a.G[c0 + i] & (a.g_dtype == DOBB_BF16 ? 7u : 15u)) == 0;
            if (al) {
                hipError_t e = launch_proj_l2_rows(a, c0, cnt, s);
                if (e == hipSuccess) e = launch_recon_l2_rows(a, c0, cnt, s);
                if (e != hipSuccess) return e;
                c0 += cnt;
                continue;
            }
        }
        // column-l2 with 128 < nb <= 416: the split-fp16 wide kernels (basis streamed in k-slices)
        if (a.hp[c0].norm == DOBB_NORM_COL_L2 && a.planes && a.planes[c0] && step_wide_eligible(a.sh)) {
            bool al = true;
            for (int i = 0; i < cnt; ++i)
                al = al && aligned16(a.M[c0 + i]) &&
                     ((uintptr_t)a.G[c0 + i] & (a.g_dtype == DOBB_BF16 ? 7u : 15u)) == 0 &&
                     ((uintptr_t)a.W[c0 + i] & (a.w_dtype == DOBB_BF16 ? 7u : 15u)) == 0 &&
                     (!a.U || aligned16(a.U[c0 + i])) && (!a.Cout || aligned16(a.Cout[c0 + i]));
            if (al) {
                const hipError_t e = launch_step_wide_l2(a, c0, cnt, s);
                if (e != hipSuccess) return e;
                c0 += cnt;
                continue;
            }
        }
        // momentum
        {
            const hipError_t e = launch_momentum(a, c0, cnt, s);
            if (e != hipSuccess) return e;
        }
        const int norm = a.hp[c0].norm;
        const int nest = a.hp[c0].nesterov ? (a.g_dtype == DOBB_BF16 ? 2 : 1) : 0;
        // projection (+ sign)
        {
            ProjTable t{};
            bool vec = (n % 4 == 0) && (nb % 4 == 0);
            for (int i = 0; i < cnt; ++i) {
                t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.Q[i] = a.Q[c0 + i];
                t.S[i] = a.S[c0 + i]; t.C[i] = a.C[c0 + i]; t.mu[i] = a.hp[c0 + i].momentum;
                t.Cout[i] = a.Cout ? a.Cout[c0 + i] : nullptr;
                vec = vec && aligned16(t.M[i]) && aligned16(t.Q[i]);
            }
            dim3 grid((unsigned)(col_tiles * nblk * cnt), (unsigned)row_tiles);
            const bool sign = norm == DOBB_NORM_SIGN;
#define DOBB_PROJ(V, N, SG) DOBB_LAUNCH("project", s, (k_project<V, N, SG>), grid, dim3(256), 0, m, n, nb, col_tiles, nblk, t)
            if (vec) {
                if (nest == 0) { if (sign) DOBB_PROJ(true, 0, true); else DOBB_PROJ(true, 0, false); }
                else if (nest == 1) { if (sign) DOBB_PROJ(true, 1, true); else DOBB_PROJ(true, 1, false); }
                else { if (sign) DOBB_PROJ(true, 2, true); else DOBB_PROJ(true, 2, false); }
            } else {
                if (nest == 0) { if (sign) DOBB_PROJ(false, 0, true); else DOBB_PROJ(false, 0, false); }
                else if (nest == 1) { if (sign) DOBB_PROJ(false, 1, true); else DOBB_PROJ(false, 1, false); }
                else { if (sign) DOBB_PROJ(false, 2, true); else DOBB_PROJ(false, 2, false); }
            }
#undef DOBB_PROJ
        }
        if (norm == DOBB_NORM_COL_L2) {
            const hipError_t e = launch_colnorm(a, c0, cnt, s);
            if (e != hipSuccess) return e;
        }
        // reconstruction + parameter update (column-l2 with nb <= 128: the split-fp16 rows kernel)
        if (norm == DOBB_NORM_COL_L2 && recon_l2_rows_eligible(a.sh)) {
            const hipError_t e = launch_recon_l2_rows(a, c0, cnt, s);
            if (e != hipSuccess) return e;
        } else {
            ReconTable t{};
            bool vec = (n % 4 == 0) && (nb % 4 == 0);
            for (int i = 0; i < cnt; ++i) {
                const dobb_hparams &h = a.hp[c0 + i];
                t.S[i] = a.S[c0 + i]; t.C[i] = a.C[c0 + i]; t.cs[i] = a.colscale[c0 + i];
                t.Q[i] = a.Q[c0 + i]; t.W[i] = a.W[c0 + i]; t.U[i] = a.U ? a.U[c0 + i] : nullptr;
                t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
                vec = vec && aligned16(t.Q[i]);
            }
            dim3 grid((unsigned)(col_tiles * nblk * cnt), (unsigned)row_tiles);
            const int amode = norm == DOBB_NORM_SIGN ? 0 : norm == DOBB_NORM_IDENTITY ? 1 : 2;
            const bool wbf = a.w_dtype == DOBB_BF16;
#define DOBB_REC(V, AM, WB) DOBB_LAUNCH("reconstruct", s, (k_reconstruct<V, AM, WB>), grid, dim3(256), 0, m, n, nb, col_tiles, nblk, t)
            if (vec) {
                if (amode == 0) { if (wbf) DOBB_REC(true, 0, true); else DOBB_REC(true, 0, false); }
                else if (amode == 1) { if (wbf) DOBB_REC(true, 1, true); else DOBB_REC(true, 1, false); }
                else { if (wbf) DOBB_REC(true, 2, true); else DOBB_REC(true, 2, false); }
            } else {
                if (amode == 0) { if (wbf) DOBB_REC(false, 0, true); else DOBB_REC(false, 0, false); }
                else if (amode == 1) { if (wbf) DOBB_REC(false, 1, true); else DOBB_REC(false, 1, false); }
                else { if (wbf) DOBB_REC(false, 2, true); else DOBB_REC(false, 2, false); }
            }
#undef DOBB_REC
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
