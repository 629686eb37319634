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

// ---- bf16 inputs: v_mfma_f32_32x32x16_bf16 --------------------------------------------------
// Output tile 128 x 128 per workgroup of 8 waves (wave w owns the 32 x 64 piece at rows 32*(w/2),
// cols 64*(w%2), as 1 x 2 MFMA tiles).  Both MFMA operands want 8 consecutive tokens of one column per
// lane, so each 128-token chunk is transposed on the way into LDS: each thread loads 8 tokens x 8
// columns, transposes the 8 x 8 block in registers and writes one 16-byte row per column into
// xs[strip][col][token].  The products of bf16 values are exact in fp32; the fp32 sums of every 256
// tokens are folded into fp64 registers.  Diagonal tile pairs load one strip and skip the quarter below the
// diagonal.  Workgroups are renumbered so the tile pairs of one block run on the same XCD (the
// dispatcher deals workgroup ids round-robin over the 8 XCDs) and share its L2.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kST = 128, kSK = 128;
// LDS row j (one column of X) holds the chunk's 128 tokens as 16 groups of 8; group g sits in slot
// g ^ swz(j).  The transposed writes (16 lanes: rows 8*cg + c, same g) and the MFMA reads (16
// consecutive rows, same g) then each touch 16 distinct 16-byte slots of the 256-byte bank window.
__device__ __forceinline__ int swz(int j) { return (j ^ (j >> 3)) & 15; }
constexpr int kSFold = 2;  // fold fp32 sums into fp64 every 2 chunks (256 tokens)

__device__ __forceinline__ int xcd_remap(int x, int G) {
    if (G % 8) return x;
    return (x % 8) * (G / 8) + x / 8;
}

// 8 consecutive bf16 of one row (valid > 0 of them in range).  VEC = 8: nb % 8 == 0 and 16-byte
// alignment, so valid >= 8; VEC = 4: nb % 4 == 0 and 8-byte alignment, so valid is a multiple of 4.
template <int VEC>
__device__ __forceinline__ void load_row8(const uint16_t *p, int valid, uint32_t d[4]) {
    if (VEC == 8) {
        const uint4 v = *(const uint4 *)p;
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else if (VEC == 4) {
        const uint2 v0 = *(const uint2 *)p;
        const uint2 v1 = valid >= 8 ? *(const uint2 *)(p + 4) : uint2{0u, 0u};
        d[0] = v0.x; d[1] = v0.y; d[2] = v1.x; d[3] = v1.y;
    } else {
        uint16_t h[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) h[c] = c < valid ? p[c] : (uint16_t)0;
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = (uint32_t)h[2 * q] | ((uint32_t)h[2 * q + 1] << 16);
    }
}

template <int VEC>
__global__ void __launch_bounds__(512) k_syrk_bf16(int64_t N, int nb, int T, int npairs, int nblk, int64_t tok_per_split,
                                                      int nsplit, float beta, AccTable t, double *partial) {
    __shared__ __align__(16) uint16_t xs[2][kST][kSK];
    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int pair = x % npairs;
    const int rest = x / npairs;
    const int b = rest % nblk, mat = rest / nblk;
    int ti, tj;
    tile_pair(pair, T, ti, tj);
    const bool diag = ti == tj;
    const int i0 = ti * kST, j0 = tj * kST;
    const int wi = min(kST, nb - i0), wj = min(kST, nb - j0);
    const int64_t tb = (int64_t)blockIdx.y * tok_per_split;
    const int64_t te = min<int64_t>(N, tb + tok_per_split);
    const int64_t ld = t.ldx[mat];
    const uint16_t *Xb = (const uint16_t *)t.X[mat] + (int64_t)b * nb;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // loader role: strip ls, columns 8*cg.., tokens 8*tg.. of the chunk (16 x 16 blocks per strip);
    // cg varies fastest, so each load instruction of a wave reads 4 rows x 256 contiguous bytes
    const int ls = tid >> 8, cg = tid & 15, tg = (tid & 255) >> 4;
    const bool loader = !(diag && ls == 1);
    const int lcol0 = (ls ? j0 : i0) + 8 * cg;
    const int lvalid = (ls ? wj : wi) - 8 * cg;
    // compute role
    const int wr = 32 * (w >> 1), wc = 64 * (w & 1);
    const bool skip = diag && wr >= wc + 64;  // strictly below the diagonal: mirrored from above
    const int sj = diag ? 0 : 1;

    f32x16 acc[2];
    double accd[2][16];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        acc[c] = (f32x16){};
#pragma unroll
        for (int r = 0; r < 16; ++r) accd[c][r] = 0.0;
    }

    uint32_t d[8][4];
    auto gload = [&](int64_t t0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t row = t0 + 8 * tg + r;
            if (loader && row < te && lvalid > 0) load_row8<VEC>(Xb + row * ld + lcol0, lvalid, d[r]);
            else { d[r][0] = d[r][1] = d[r][2] = d[r][3] = 0u; }
        }
    };
    // software pipeline: the global loads of chunk c+1 are issued before the MFMAs of chunk c
    if (tb < te) gload(tb);
    int nchunk = 0;
    for (int64_t t0 = tb; t0 < te; t0 += kSK) {
        __syncthreads();  // previous chunk's MFMA reads are done
        if (loader) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                uint4 o;
                uint32_t e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = d[2 * q][c >> 1], hi = d[2 * q + 1][c >> 1];
                    e[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                o.x = e[0]; o.y = e[1]; o.z = e[2]; o.w = e[3];
                const int j = 8 * cg + c;
                *(uint4 *)&xs[ls][j][8 * (tg ^ swz(j))] = o;
            }
        }
        __syncthreads();
        if (t0 + kSK < te) gload(t0 + kSK);
        if (!skip) {
#pragma unroll
            for (int kk = 0; kk < kSK; kk += 16) {
                const int g = (kk >> 3) + (lane >> 5);
                const int ja = wr + (lane & 31), jb0 = wc + (lane & 31), jb1 = jb0 + 32;
                bf16x8 a0 = *(const bf16x8 *)&xs[0][ja][8 * (g ^ swz(ja))];
                bf16x8 b0 = *(const bf16x8 *)&xs[sj][jb0][8 * (g ^ swz(jb0))];
                bf16x8 b1 = *(const bf16x8 *)&xs[sj][jb1][8 * (g ^ swz(jb1))];
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[1], 0, 0, 0);
            }
            if (++nchunk == kSFold) {
                nchunk = 0;
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int r = 0; r < 16; ++r) { accd[c][r] += (double)acc[c][r]; acc[c][r] = 0.f; }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) accd[c][r] += (double)acc[c][r];
    if (skip) return;

    const double invN = 1.0 / (double)N;
    const double bd = (double)beta;
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const int64_t tot_blocks = gridDim.x / npairs;
    double *Pb = partial ? partial + ((int64_t)blockIdx.y * tot_blocks + rest) * nb * nb : nullptr;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int gj = j0 + wc + 32 * c + acc_col(lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int gi = i0 + wr + acc_row(r, lane);
            if (gi >= nb || gj >= nb || gi > gj) continue;
            if (nsplit == 1) {
                const double old = beta > 0.f ? (double)Ab[(int64_t)gi * nb + gj] : 0.0;
                const float v = (float)(bd * old + (1.0 - bd) * (accd[c][r] * invN));
                Ab[(int64_t)gi * nb + gj] = v;
                Ab[(int64_t)gj * nb + gi] = v;
            } else {
                Pb[(int64_t)gi * nb + gj] = accd[c][r];
            }
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
int accumulate_plan(const dobb_shape &sh, int64_t N, int count, int64_t *tps, bool bf16) {
    const int nb = (int)sh.nb;
    const int tile = bf16 ? kST : kBM;
    const int T = (nb + tile - 1) / tile;
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

int accumulate_splits(const dobb_shape &sh, int64_t N, int count, bool bf16) {
    return accumulate_plan(sh, N, count, nullptr, bf16);
}

size_t accumulate_ws(const dobb_shape &sh, int64_t N, int count) {
    const int nsplit = accumulate_splits(sh, N, count, false) > accumulate_splits(sh, N, count, true)
                           ? accumulate_splits(sh, N, count, false) : accumulate_splits(sh, N, count, true);
    if (nsplit <= 1) return 0;
    const int cnt = count < kMaxMats ? count : kMaxMats;
    return (size_t)nsplit * cnt * (size_t)(sh.n / sh.nb) * sh.nb * sh.nb * sizeof(double);
}

hipError_t launch_accumulate(const AccumulateArgs &a, hipStream_t s) {
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(a.sh.n / nb);
    const bool xbf = a.x_dtype == DOBB_BF16;
    const int tile = xbf ? kST : kBM;
    const int T = (nb + tile - 1) / tile;
    const int npairs = T * (T + 1) / 2;
    int64_t tps = a.N;
    const int nsplit = accumulate_plan(a.sh, a.N, a.count, &tps, xbf);
    if (nsplit <= 1) tps = a.N;
    for (int c0 = 0; c0 < a.count;) {
        const int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        AccTable t{};
        bool vec4 = nb % 4 == 0, vec8 = nb % 8 == 0;
        for (int i = 0; i < cnt; ++i) {
            t.X[i] = a.X[c0 + i]; t.A[i] = a.A[c0 + i]; t.ldx[i] = a.ldx[c0 + i];
            const uintptr_t p = (uintptr_t)t.X[i];
            vec4 = vec4 && (t.ldx[i] % 4 == 0) && ((p & (xbf ? 7u : 15u)) == 0);
            vec8 = vec8 && (t.ldx[i] % 8 == 0) && ((p & 15u) == 0);
        }
        dim3 grid((unsigned)(npairs * nblk * cnt), (unsigned)nsplit);
        double *part = nsplit > 1 ? a.partial : nullptr;
        if (xbf) {
#define DOBB_SYRKB(V) DOBB_LAUNCH("accumulate_syrk_bf16", s, (k_syrk_bf16<V>), grid, dim3(512), 0, a.N, nb, T, npairs, nblk, tps, nsplit, a.beta, t, part)
            if (vec8) DOBB_SYRKB(8); else if (vec4) DOBB_SYRKB(4); else DOBB_SYRKB(1);
#undef DOBB_SYRKB
        } else {
#define DOBB_SYRK(V) DOBB_LAUNCH("accumulate_syrk", s, (k_syrk<false, V>), grid, dim3(256), 0, a.N, nb, T, npairs, nblk, tps, nsplit, a.beta, t, part)
            if (vec4) DOBB_SYRK(true); else DOBB_SYRK(false);
#undef DOBB_SYRK
        }
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
