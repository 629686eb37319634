// The Dobb-G step: the basis of the output-gradient second moment, blocks of nb consecutive rows.
//
// Dobb paper (arXiv 2610.39412): Tables 12-13 (the output-gradient second moment as the basis
// source: Dobb-G, Dobb-G-l2), Figure 2 caption (that moment is m x m), Table 7 (blocks along the
// output axis; Dobb-G-l2 normalises each coefficient row over the input axis), Table 9 (Dobb-G's
// update scale).  For block b (rows R_b = [b nb, (b+1) nb)) with basis P_b:
//   C_b = P_b^T M_b  (nb x n),  S_b = sign(C_b) | C_b | diag(1/||c_i||) C_b,  U[R_b, :] = P_b S_b,
//   W <- W - lr (s U + wd W).
// A block is nb whole rows of the weight, so both products read and write along rows: each output
// tile is 64 (basis index, or row of the block) x 64 (columns of W), with K = nb, on the fp32 MFMA
// tile core of dobb_internal.h (both operands staged k-major in LDS).
//   k_project_g      C_b tile = P_b^T M_b: P_b rows and M_b rows are both k-major already
//   k_rownorm_g      Dobb-G-l2: rs_r = 1 / ||C[r, :]|| (fp64 sum over the n columns, one wave per row)
//   k_reconstruct_g  U tile = P_b S_b: P_b transposed into LDS, S (or C scaled by rs) k-major;
//                    W <- W - lr (s U + wd W) in the epilogue
// The momentum M <- mu M + G runs first (k_step.hip's elementwise kernel).
#include "dobb_internal.h"

namespace dobb {
namespace {

struct ProjGTable {
    const float *M[kMaxMats];
    const void *G[kMaxMats];
    const float *P[kMaxMats];
    int8_t *S[kMaxMats];
    float *C[kMaxMats];
    float *Cout[kMaxMats];     // NULL or m x n fp32: the coefficients (verification output)
    float mu[kMaxMats];
};

// b[k][j] = G + mu M at element off + k ld + j (the Nesterov operand, from the updated momentum)
template <bool GBF16, bool VEC>
struct LoadNestColsK {
    const float *M; const void *G; int64_t off; int64_t ld; int cols; int K; float mu;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15), k = k0 + kk;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = 0.f;
        if (k >= K) return;
        const int64_t e = off + (int64_t)k * ld + j;
        if (VEC) {
            if (j < cols) {
                const f32x4 mv = *(const f32x4 *)(M + e);
                f32x4 gv;
                if (GBF16) {
                    const uint2 h = *(const uint2 *)((const uint16_t *)G + e);
                    gv = f32x4{bf16_to_f32((uint16_t)h.x), bf16_to_f32((uint16_t)(h.x >> 16)),
                               bf16_to_f32((uint16_t)h.y), bf16_to_f32((uint16_t)(h.y >> 16))};
                } else {
                    gv = *(const f32x4 *)((const float *)G + e);
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = __builtin_fmaf(mu, mv[c], gv[c]);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (j + c < cols) {
                    const float g = GBF16 ? bf16_to_f32(((const uint16_t *)G)[e + c]) : ((const float *)G)[e + c];
                    v[c] = __builtin_fmaf(mu, M[e + c], g);
                }
        }
    }
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBN]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15);
        *(f32x4 *)&dst[kk][j ^ gemm_swz(kk)] = f32x4{v[0], v[1], v[2], v[3]};
    }
};

// grid.x = column tiles of 64, grid.y = (64-row tiles of the basis index) x blocks x matrices
template <bool VEC, int NEST /*0 none, 1 G fp32, 2 G bf16*/, bool SIGN>
__global__ void __launch_bounds__(256) k_project_g(int64_t m, int64_t n, int nb, int itiles, int nblk, ProjGTable t) {
    __shared__ GemmSmem2 sm;
    const int c0 = blockIdx.x * kBN;
    int rest = blockIdx.y;
    const int it = rest % itiles;
    rest /= itiles;
    const int b = rest % nblk, mat = rest / nblk;
    const int i0 = it * kBM;
    const int64_t off = (int64_t)b * nb * n + c0;            // element (row b nb, column c0)
    // A operand a[k][i] = P_b[k][i0 + i] (row-major P_b is k-major already)
    LoadColsK<VEC> la{t.P[mat] + (int64_t)b * nb * nb + i0, nb, nb - i0, nb};
    f32x16 acc;
    if (NEST == 0) {
        LoadColsK<VEC> lb{t.M[mat] + off, n, (int)(n - c0 < kBN ? n - c0 : kBN), nb};
        acc = gemm_tile(nb, la, lb, sm);
    } else {
        LoadNestColsK<NEST == 2, VEC> lb{t.M[mat], t.G[mat], off, n, (int)(n - c0 < kBN ? n - c0 : kBN), nb, t.mu[mat]};
        acc = gemm_tile(nb, la, lb, sm);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wr = 32 * (w >> 1), wc = 32 * (w & 1);
    const int64_t col = c0 + wc + acc_col(lane);
    if (col < n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + wr + acc_row(r, lane);
            if (i < nb) {
                const int64_t e = ((int64_t)b * nb + i) * n + col;
                if (SIGN) t.S[mat][e] = sign_code(acc[r]);
                else t.C[mat][e] = acc[r];
                if (t.Cout[mat]) t.Cout[mat][e] = acc[r];
            }
        }
    }
}

// Dobb-G-l2: rs_r = 1 / ||C[r, :]||_2 (0 for a zero row), summed in fp64 by one wave per row in a
// fixed order (lane partial sums, then a butterfly).  grid = (ceil(m / 4), matrices), block 256.
struct RowNormTable {
    const float *C[kMaxMats];
    float *rs[kMaxMats];
};
__global__ void __launch_bounds__(256) k_rownorm_g(int64_t m, int64_t n, RowNormTable t) {
    const int mat = blockIdx.y;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= m) return;
    const float *C = t.C[mat] + r * n;
    double s = 0.0;
    for (int64_t c = lane; c < n; c += 64) {
        const double v = C[c];
        s += v * v;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) t.rs[mat][r] = s > 0.0 ? (float)(1.0 / sqrt(s)) : 0.f;
}

struct ReconGTable {
    const int8_t *S[kMaxMats];
    const float *C[kMaxMats];
    const float *rs[kMaxMats];
    const float *P[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};

// b[k][j] = sign code decoded at src[k ld + j]
template <bool VEC>
struct LoadSignColsK {
    const int8_t *src; int64_t ld; int cols; int K;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15), k = k0 + kk;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = 0.f;
        if (k >= K) return;
        const int8_t *p = src + (int64_t)k * ld + j;
        if (VEC) {
            if (j < cols) {
                const uint32_t q = *(const uint32_t *)p;
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = sign_decode((int8_t)((q >> (8 * c)) & 0xff));
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) if (j + c < cols) v[c] = sign_decode(p[c]);
        }
    }
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBN]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15);
        *(f32x4 *)&dst[kk][j ^ gemm_swz(kk)] = f32x4{v[0], v[1], v[2], v[3]};
    }
};

// b[k][j] = C[k ld + j] (identity) or C[k ld + j] rs[k] (Dobb-G-l2: row k of the block scaled)
template <bool SCALED, bool VEC>
struct LoadCoefColsK {
    const float *src; const float *rs; int64_t ld; int cols; int K;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15), k = k0 + kk;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = 0.f;
        if (k >= K) return;
        const float *p = src + (int64_t)k * ld + j;
        const float sc = SCALED ? rs[k] : 1.f;
        if (VEC) {
            if (j < cols) {
                const f32x4 q = *(const f32x4 *)p;
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = SCALED ? q[c] * sc : q[c];
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) if (j + c < cols) v[c] = SCALED ? p[c] * sc : p[c];
        }
    }
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBN]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15);
        *(f32x4 *)&dst[kk][j ^ gemm_swz(kk)] = f32x4{v[0], v[1], v[2], v[3]};
    }
};

// grid.x = column tiles of 64, grid.y = (64-row tiles of the block) x blocks x matrices
template <bool VEC, int AMODE /*0 sign codes, 1 C, 2 C scaled by rs*/, bool WBF16>
__global__ void __launch_bounds__(256) k_reconstruct_g(int64_t m, int64_t n, int nb, int ptiles, int nblk,
                                                       ReconGTable t) {
    __shared__ GemmSmem2 sm;
    const int c0 = blockIdx.x * kBN;
    int rest = blockIdx.y;
    const int pt = rest % ptiles;
    rest /= ptiles;
    const int b = rest % nblk, mat = rest / nblk;
    const int p0 = pt * kBM;
    const int64_t off = (int64_t)b * nb * n + c0;
    const int cols = (int)(n - c0 < kBN ? n - c0 : kBN);
    // A operand a[k][i] = P_b[p0 + i][k]: row-major P_b transposed into the k-major layout
    LoadRowsT<VEC> la{t.P[mat] + (int64_t)b * nb * nb + (int64_t)p0 * nb, nb, nb - p0, nb};
    f32x16 acc;
    if (AMODE == 0) {
        LoadSignColsK<VEC> lb{t.S[mat] + off, n, cols, nb};
        acc = gemm_tile(nb, la, lb, sm);
    } else {
        LoadCoefColsK<AMODE == 2, VEC> lb{t.C[mat] + off, t.rs[mat] + (int64_t)b * nb, n, cols, nb};
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
            const int p = p0 + wr + acc_row(r, lane);
            if (p < nb) {
                const int64_t e = off + (int64_t)(p) * n + col;
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

bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t step_g_ws_one(const dobb_shape &sh, int norm) {
    const size_t mn = (size_t)sh.m * (size_t)sh.n;
    if (norm == DOBB_NORM_SIGN) return al256(mn);                  // int8 sign codes
    return al256(mn * 4) + al256((size_t)sh.m * 4);                // fp32 coefficients + row scales
}

hipError_t launch_step_g(const StepArgs &a, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(m / nb);
    const int cnt = a.count;
    const int itiles = (nb + kBM - 1) / kBM;
    const unsigned col_tiles = (unsigned)((n + kBN - 1) / kBN);
    if (cnt < 1 || cnt > kMaxMats || (int64_t)itiles * nblk * cnt > 65535) return hipErrorInvalidValue;
    hipError_t e = launch_momentum(a, 0, cnt, s);
    if (e != hipSuccess) return e;
    const int norm = a.hp[0].norm;
    const int nest = a.hp[0].nesterov ? (a.g_dtype == DOBB_BF16 ? 2 : 1) : 0;
    const dim3 grid(col_tiles, (unsigned)(itiles * nblk * cnt));
    bool vec = n % 4 == 0 && nb % 4 == 0;
    {
        ProjGTable t{};
        for (int i = 0; i < cnt; ++i) {
            t.M[i] = a.M[i]; t.G[i] = a.G[i]; t.P[i] = a.Q[i]; t.S[i] = a.S[i]; t.C[i] = a.C[i];
            t.Cout[i] = a.Cout ? a.Cout[i] : nullptr; t.mu[i] = a.hp[i].momentum;
            vec = vec && al16(t.M[i]) && al16(t.P[i]) &&
                  ((uintptr_t)t.G[i] & (a.g_dtype == DOBB_BF16 ? 7u : 15u)) == 0;
        }
        const bool sign = norm == DOBB_NORM_SIGN;
#define DOBB_PG(V, N, SG) DOBB_LAUNCH("project_g", s, (k_project_g<V, N, SG>), grid, dim3(256), 0, m, n, nb, itiles, nblk, t)
        if (vec) {
            if (nest == 0) { if (sign) DOBB_PG(true, 0, true); else DOBB_PG(true, 0, false); }
            else if (nest == 1) { if (sign) DOBB_PG(true, 1, true); else DOBB_PG(true, 1, false); }
            else { if (sign) DOBB_PG(true, 2, true); else DOBB_PG(true, 2, false); }
        } else {
            if (nest == 0) { if (sign) DOBB_PG(false, 0, true); else DOBB_PG(false, 0, false); }
            else if (nest == 1) { if (sign) DOBB_PG(false, 1, true); else DOBB_PG(false, 1, false); }
            else { if (sign) DOBB_PG(false, 2, true); else DOBB_PG(false, 2, false); }
        }
#undef DOBB_PG
    }
    if (norm == DOBB_NORM_COL_L2) {
        RowNormTable t{};
        for (int i = 0; i < cnt; ++i) { t.C[i] = a.C[i]; t.rs[i] = a.colscale[i]; }
        DOBB_LAUNCH("rownorm_g", s, k_rownorm_g, dim3((unsigned)((m + 3) / 4), (unsigned)cnt), dim3(256), 0, m, n, t);
    }
    {
        ReconGTable t{};
        for (int i = 0; i < cnt; ++i) {
            const dobb_hparams &h = a.hp[i];
            t.S[i] = a.S[i]; t.C[i] = a.C[i]; t.rs[i] = a.colscale[i]; t.P[i] = a.Q[i]; t.W[i] = a.W[i];
            t.U[i] = a.U ? a.U[i] : nullptr;
            t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
            vec = vec && al16(a.C[i]);
        }
        const int amode = norm == DOBB_NORM_SIGN ? 0 : norm == DOBB_NORM_IDENTITY ? 1 : 2;
        const bool wbf = a.w_dtype == DOBB_BF16;
#define DOBB_RG(V, AM, WB) DOBB_LAUNCH("reconstruct_g", s, (k_reconstruct_g<V, AM, WB>), grid, dim3(256), 0, m, n, nb, itiles, nblk, t)
        if (vec) {
            if (amode == 0) { if (wbf) DOBB_RG(true, 0, true); else DOBB_RG(true, 0, false); }
            else if (amode == 1) { if (wbf) DOBB_RG(true, 1, true); else DOBB_RG(true, 1, false); }
            else { if (wbf) DOBB_RG(true, 2, true); else DOBB_RG(true, 2, false); }
        } else {
            if (amode == 0) { if (wbf) DOBB_RG(false, 0, true); else DOBB_RG(false, 0, false); }
            else if (amode == 1) { if (wbf) DOBB_RG(false, 1, true); else DOBB_RG(false, 1, false); }
            else { if (wbf) DOBB_RG(false, 2, true); else DOBB_RG(false, 2, false); }
        }
#undef DOBB_RG
    }
    return hipGetLastError();
}

}  // namespace dobb
