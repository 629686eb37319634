// Block-diagonal second-moment capture with EMA on gfx950.
//
// Dobb paper (arXiv 2610.39412), abstract: the input-activation second moment is approximated by its
// diagonal blocks; Figure 2 caption: second moments are averaged over accumulated mini-batches.
//   A_b <- beta A_b + (1 - beta) (1/N) X_b^T X_b      (X_b = the nb columns of block b, N tokens)
//
// k_syrk: one workgroup per (upper-triangle 64x64 tile pair, block, matrix, token split).  The
// products are formed by v_mfma_f32_32x32x2_f32 (exact for bf16 inputs), summed in fp32 over 64
// tokens and folded into fp64 registers, so the sum over N tokens is close to correctly rounded.
// Without a token split the EMA is fused into the epilogue; with one, fp64 partials go to the
// workspace and k_syrk_reduce adds them in split order (deterministic, no atomics).  Each result is
// written at (i, j) and (j, i) from the same value, so A is exactly symmetric.
#include "dobb_internal.h"

namespace dobb {
namespace {

struct AccTable {
    const void *X[kMaxMats];
    float *A[kMaxMats];
    int64_t ldx[kMaxMats];
};

// dst[kk][j] = X[(k0 + kk) * ld + j] as fp32 (zero outside kk + k0 < K, j < cols); bf16 or fp32.
template <bool XBF16, bool VEC>
struct LoadTokens {
    const void *src; int64_t ld; int cols; int K;
    __device__ __forceinline__ void operator()(int k0, float (*dst)[kBN + kPad]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15), k = k0 + kk;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (k < K) {
            const int64_t e = (int64_t)k * ld + j;
            if (XBF16) {
                const uint16_t *p = (const uint16_t *)src + e;
                if (VEC) {
                    if (j < cols) {
                        uint2 h = *(const uint2 *)p;
                        v[0] = bf16_to_f32((uint16_t)(h.x & 0xffff)); v[1] = bf16_to_f32((uint16_t)(h.x >> 16));
                        v[2] = bf16_to_f32((uint16_t)(h.y & 0xffff)); v[3] = bf16_to_f32((uint16_t)(h.y >> 16));
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) if (j + c < cols) v[c] = bf16_to_f32(p[c]);
                }
            } else {
                const float *p = (const float *)src + e;
                if (VEC) {
                    if (j < cols) { f32x4 q = *(const f32x4 *)p; v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3]; }
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) if (j + c < cols) v[c] = p[c];
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[kk][j + c] = v[c];
    }
};

__device__ __forceinline__ void tile_pair(int p, int T, int &ti, int &tj) {
    ti = 0;
    while (p >= T - ti) { p -= T - ti; ++ti; }
    tj = ti + p;
}

constexpr int kFoldChunks = 4;  // fold the fp32 accumulator into fp64 every 4 x 16 = 64 tokens

// grid.x = npairs * nblk * count, grid.y = token splits
template <bool XBF16, bool VEC>
__global__ void __launch_bounds__(256) k_syrk(int64_t N, int nb, int T, int npairs, int nblk, int64_t tok_per_split,
                                              int nsplit, float beta, AccTable t, double *partial) {
    __shared__ GemmSmem sm;
    const int pair = blockIdx.x % npairs;
    const int rest = blockIdx.x / npairs;
    const int b = rest % nblk, mat = rest / nblk;
    int ti, tj;
    tile_pair(pair, T, ti, tj);
    const int i0 = ti * kBM, j0 = tj * kBN;
    const int64_t tb = (int64_t)blockIdx.y * tok_per_split;
    const int64_t te = min<int64_t>(N, tb + tok_per_split);
    const int K = (int)(te - tb);
    const int64_t ld = t.ldx[mat];
    const size_t esz = XBF16 ? 2 : 4;
    const char *base = (const char *)t.X[mat] + (size_t)(tb * ld + (int64_t)b * nb) * esz;
    LoadTokens<XBF16, VEC> la{base + (size_t)i0 * esz, ld, nb - i0, K};
    LoadTokens<XBF16, VEC> lb{base + (size_t)j0 * esz, ld, nb - j0, K};

    f32x16 acc = {};
    double accd[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) accd[r] = 0.0;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wr = 32 * (w >> 1), wc = 32 * (w & 1);
    int chunk = 0;
    for (int k0 = 0; k0 < K; k0 += kBK) {
        la(k0, sm.a);
        lb(k0, sm.b);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 2) {
            float a = sm.a[kk + (lane >> 5)][wr + (lane & 31)];
            float bb = sm.b[kk + (lane >> 5)][wc + (lane & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bb, acc, 0, 0, 0);
        }
        __syncthreads();
        if (++chunk == kFoldChunks) {
#pragma unroll
            for (int r = 0; r < 16; ++r) { accd[r] += (double)acc[r]; acc[r] = 0.f; }
            chunk = 0;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) accd[r] += (double)acc[r];

    const int gj = j0 + wc + acc_col(lane);
    const double invN = 1.0 / (double)N;
    const double bd = (double)beta;
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const int64_t tot_blocks = gridDim.x / npairs;  // nblk * matrices in this launch
    double *Pb = partial ? partial + ((int64_t)blockIdx.y * tot_blocks + rest) * nb * nb : nullptr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int gi = i0 + wr + acc_row(r, lane);
        if (gi >= nb || gj >= nb || gi > gj) continue;  // only the upper triangle (gi <= gj)
        if (nsplit == 1) {
            const double old = beta > 0.f ? (double)Ab[(int64_t)gi * nb + gj] : 0.0;
            const float v = (float)(bd * old + (1.0 - bd) * (accd[r] * invN));
            Ab[(int64_t)gi * nb + gj] = v;
            Ab[(int64_t)gj * nb + gi] = v;
        } else {
            Pb[(int64_t)gi * nb + gj] = accd[r];
        }
    }
}

// Sum the token-split partials in split order, apply the EMA, write both triangles.
// grid.x over nb*nb entries of a block, grid.y = block index within the launch (nblk * count).
__global__ void __launch_bounds__(256) k_syrk_reduce(int64_t N, int nb, int nblk, int nsplit, int64_t tot_blocks,
                                                     float beta, AccTable t, const double *partial) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)nb * nb) return;
    const int i = (int)(e / nb), j = (int)(e % nb);
    if (i > j) return;
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    double s = 0.0;
    for (int sp = 0; sp < nsplit; ++sp) s += partial[((int64_t)sp * tot_blocks + g) * nb * nb + e];
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const double bd = (double)beta;
    const double old = beta > 0.f ? (double)Ab[e] : 0.0;
    const float v = (float)(bd * old + (1.0 - bd) * (s / (double)N));
    Ab[(int64_t)i * nb + j] = v;
    Ab[(int64_t)j * nb + i] = v;
}

}  // namespace

// Token split plan: enough workgroups for >= 4 per CU, >= 256 tokens per split, split length a
// multiple of 64 tokens (the fp64 fold period).  Returns the number of splits; *tps its length.
int accumulate_plan(const dobb_shape &sh, int64_t N, int count, int64_t *tps) {
    const int nb = (int)sh.nb;
    const int T = (nb + kBM - 1) / kBM;
    const int64_t tiles = (int64_t)T * (T + 1) / 2 * (sh.n / nb) * (count < kMaxMats ? count : kMaxMats);
    int64_t nsplit = (1024 + tiles - 1) / tiles;
    const int64_t cap = N / 256;
    if (nsplit > cap) nsplit = cap;
    if (nsplit < 1) nsplit = 1;
    if (nsplit > 64) nsplit = 64;
    const int64_t len = ((N + nsplit - 1) / nsplit + 63) / 64 * 64;
    if (tps) *tps = len;
    return (int)((N + len - 1) / len);
}

int accumulate_splits(const dobb_shape &sh, int64_t N, int count) { return accumulate_plan(sh, N, count, nullptr); }

size_t accumulate_ws(const dobb_shape &sh, int64_t N, int count) {
    const int nsplit = accumulate_splits(sh, N, count);
    if (nsplit <= 1) return 0;
    const int cnt = count < kMaxMats ? count : kMaxMats;
    return (size_t)nsplit * cnt * (size_t)(sh.n / sh.nb) * sh.nb * sh.nb * sizeof(double);
}

hipError_t launch_accumulate(const AccumulateArgs &a, hipStream_t s) {
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(a.sh.n / nb);
    const int T = (nb + kBM - 1) / kBM;
    const int npairs = T * (T + 1) / 2;
    int64_t tps = a.N;
    const int nsplit = accumulate_plan(a.sh, a.N, a.count, &tps);
    if (nsplit <= 1) tps = a.N;
    const bool xbf = a.x_dtype == DOBB_BF16;
    for (int c0 = 0; c0 < a.count;) {
        const int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        AccTable t{};
        bool vec = nb % 4 == 0;
        for (int i = 0; i < cnt; ++i) {
            t.X[i] = a.X[c0 + i]; t.A[i] = a.A[c0 + i]; t.ldx[i] = a.ldx[c0 + i];
            vec = vec && (t.ldx[i] % 4 == 0) && (((uintptr_t)t.X[i] & (xbf ? 7u : 15u)) == 0);
        }
        dim3 grid((unsigned)(npairs * nblk * cnt), (unsigned)nsplit);
        double *part = nsplit > 1 ? a.partial : nullptr;
#define DOBB_SYRK(XB, V) DOBB_LAUNCH("accumulate_syrk", s, (k_syrk<XB, V>), grid, dim3(256), 0, a.N, nb, T, npairs, nblk, tps, nsplit, a.beta, t, part)
        if (xbf) { if (vec) DOBB_SYRK(true, true); else DOBB_SYRK(true, false); }
        else { if (vec) DOBB_SYRK(false, true); else DOBB_SYRK(false, false); }
#undef DOBB_SYRK
        if (nsplit > 1) {
            const int64_t tot = (int64_t)nblk * cnt;
            dim3 g2((unsigned)(((int64_t)nb * nb + 255) / 256), (unsigned)tot);
            DOBB_LAUNCH("accumulate_reduce", s, k_syrk_reduce, g2, dim3(256), 0, a.N, nb, nblk, nsplit, tot, a.beta, t,
                        (const double *)part);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
