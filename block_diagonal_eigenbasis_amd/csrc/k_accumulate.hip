// Block-diagonal second-moment capture with EMA on gfx950.
//
// Dobb paper (arXiv 2610.39412), abstract: the input-activation second moment is approximated by its
// diagonal blocks; Figure 2 caption: second moments are averaged over accumulated mini-batches.
//   A_b <- beta A_b + (1 - beta) (1/N) X_b^T X_b      (X_b = the nb columns of block b, N tokens)
//
// k_syrk (fp32 activations): one workgroup per (upper-triangle 64x64 tile pair, block, matrix, token
// split).  The products are exact in fp64 and summed in fp64, so A is correctly rounded but for near
// ties.  Without a token split the EMA is fused into the epilogue; with one, fp64 partials go to the
// workspace and k_syrk_reduce adds them in split order (deterministic, no atomics).  Each result is
// written at (i, j) and (j, i) from the same value, so A is exactly symmetric.
// bf16 activations: k_syrk_narrow_dma (blocks of 33 .. 128 columns), k_syrk_wide_dma (up to 416)
// and k_syrk_wide (up to 512) take each block whole, so that its activations are read from HBM
// once; k_syrk_bf16 (128 x 128 tile pairs) takes the rest (all described below).
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

// fp32 activations: grid.x = npairs * nblk * count, grid.y = token splits.  Products of fp32 values
// are exact in fp64 and the sums run in fp64 (v_fma_f64), so the sum over a split is within a few
// units of 2^-53 of the exact one and A comes out correctly rounded to fp32 but for near ties.
// Thread t owns the 4 x 4 outputs at rows 4 (t / 16) .., columns 4 (t % 16) .. of the 64 x 64 tile;
// each 16-token chunk is staged in LDS as fp32, token-major.
template <bool VEC>
__global__ void __launch_bounds__(256) k_syrk(int64_t N, int nb, int T, int npairs, int nblk, int64_t tok_per_split,
                                              int nsplit, float beta, AccTable t, double *partial) {
    __shared__ __align__(16) GemmSmem sm;
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
    const char *base = (const char *)t.X[mat] + (size_t)(tb * ld + (int64_t)b * nb) * 4;
    LoadTokens<false, VEC> la{base + (size_t)i0 * 4, ld, nb - i0, K};
    LoadTokens<false, VEC> lb{base + (size_t)j0 * 4, ld, nb - j0, K};

    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    double acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
    for (int k0 = 0; k0 < K; k0 += kBK) {
        la(k0, sm.a);
        lb(k0, sm.b);
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < kBK; ++kk) {
            const f32x4 av = *(const f32x4 *)&sm.a[kk][4 * ty];
            const f32x4 bv = *(const f32x4 *)&sm.b[kk][4 * tx];
            double ad[4], bd[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) { ad[c] = (double)av[c]; bd[c] = (double)bv[c]; }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fma(ad[r], bd[c], acc[r][c]);
        }
        __syncthreads();
    }

    const double invN = 1.0 / (double)N;
    const double bd = (double)beta;
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const int64_t tot_blocks = gridDim.x / npairs;  // nblk * matrices in this launch
    double *Pb = partial ? partial + ((int64_t)blockIdx.y * tot_blocks + rest) * nb * nb : nullptr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int gi = i0 + 4 * ty + r, gj = j0 + 4 * tx + c;
            if (gi >= nb || gj >= nb || gi > gj) continue;  // only the upper triangle (gi <= gj)
            if (nsplit == 1) {
                const double old = beta > 0.f ? (double)Ab[(int64_t)gi * nb + gj] : 0.0;
                const float v = (float)(bd * old + (1.0 - bd) * (acc[r][c] * invN));
                Ab[(int64_t)gi * nb + gj] = v;
                Ab[(int64_t)gj * nb + gi] = v;
            } else {
                Pb[(int64_t)gi * nb + gj] = acc[r][c];
            }
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

// ---- wide blocks (bf16 X, 128 < nb <= 512) ------------------------------------------------------
// One workgroup stages a 64-token chunk of ALL nb columns of block b in LDS, so X is read from HBM
// once.  The upper triangle of X_b^T X_b is covered by groups of 2 x 4 tiles of 32 x 32 (row tiles
// 2p, 2p+1; column tiles from 2p on, four at a time); each wave owns one group and keeps its eight
// accumulators in registers for the whole token split (8 MFMAs per 6 LDS operand reads).  The
// groups of a block are spread over ceil(groups / 8) adjacent workgroups, which read the same chunks
// close together in time, so the repeated reads are served by L2.
// A chunk is loaded into registers (8 tokens x 8 columns per thread), transposed 8 x 8 on the way
// into LDS ([column][token], 16-byte slots swizzled against bank conflicts), double buffered.
// The sums stay fp32 over a split of at most 4096 tokens (256 MFMA steps); splits are added in fp64
// by k_syrk_reduce<float> in split order.  The diagonal entries are sums of squares, every term
// positive, and would collect the largest fp32 rounding error that way (about 5e-7 of max|A_b| at
// 4096 tokens): the waves whose group holds the two diagonal tiles move them into fp64 registers
// every kWFold chunks (fp32 runs of 16 MFMA steps), one entry per lane and tile.
constexpr int kWK = 64;          // tokens per LDS chunk
constexpr int kWMaxGroups = 32;  // 2 x 4 tile groups for up to 16 tile rows (20 needed)
constexpr int64_t kWSplitMax = 4096;
constexpr unsigned kWOff = 0xffffffffu;   // buffer offset past the end: the load returns zeros
constexpr int kWFold = 4;        // chunks between moves of the diagonal entries into fp64

struct WideGroups {
    uint8_t r0[kWMaxGroups], c0[kWMaxGroups];
};

// 16-byte slot of 8 tokens within a 128-byte column row: conflict-free for 8- and 16-lane phases
__device__ __forceinline__ int wswz(int c) { return (c ^ (c >> 3)) & 7; }

// grid.x = wgs (fastest) x blocks x matrices, renumbered per XCD; grid.y = token splits; block 512
__global__ void __launch_bounds__(512) k_syrk_wide(int64_t N, int nb, int T32, int ngroups, int wgs, int nblk,
                                                   int64_t tok_per_split, int nsplit, float beta, AccTable t,
                                                   WideGroups grp, float *partial) {
    extern __shared__ __align__(16) uint16_t xw[];   // [2][32 T32][kWK]
    const int nbp = 32 * T32;
    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int wg = x % wgs, rest = x / wgs;
    const int b = rest % nblk, mat = rest / nblk;
    const int64_t tb = (int64_t)blockIdx.y * tok_per_split;
    const int64_t te = min<int64_t>(N, tb + tok_per_split);
    const int64_t ld = t.ldx[mat];
    const uint16_t *Xb = (const uint16_t *)t.X[mat] + (int64_t)b * nb;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // columns [nb, nbp) of both buffers stay zero (they only feed discarded entries)
    for (int e = tid; e < 2 * (nbp - nb) * (kWK / 8); e += 512) {
        const int bb = e / ((nbp - nb) * (kWK / 8)), r = e % ((nbp - nb) * (kWK / 8));
        const int c = nb + r / (kWK / 8), sl = r % (kWK / 8);
        *(uint4 *)&xw[((size_t)bb * nbp + c) * kWK + 8 * sl] = uint4{0u, 0u, 0u, 0u};
    }

    // loader role: token group tg (8 tokens), column group cg (8 columns); cg fastest.  Buffer loads
    // with an offset past the end for idle lanes and tokens >= te read zeros without a branch.
    const int ncg = nb / 8;
    const int tg = tid / ncg, cg = tid - tg * ncg;
    const bool loader = tid < ncg * (kWK / 8);
    const __amdgpu_buffer_rsrc_t rX =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(Xb), (short)0, (int)((N * ld - (int64_t)b * nb) * 2), 0x00020000);
    uint32_t d[8][4];
    auto gload = [&](int64_t t0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t row = t0 + 8 * tg + r;
            const unsigned off = (loader && row < te) ? (unsigned)((row * ld + 8 * cg) * 2) : kWOff;
            const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
            d[r][0] = v.x; d[r][1] = v.y; d[r][2] = v.z; d[r][3] = v.w;
        }
    };

    // compute role: group g -> row tiles R0, R0 + 1 and column tiles C0 .. C0 + 3 (wave-uniform).
    // All eight products are issued; tiles past the grid (operand strip 0) or below the diagonal
    // are discarded in the epilogue.
    const int g = wg * 8 + w;
    const bool active = g < ngroups;
    const int R0 = active ? grp.r0[g] : 0, C0 = active ? grp.c0[g] : 0;
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
    int acol[2], bcol[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) acol[i] = 32 * (R0 + i < T32 ? R0 + i : 0) + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) bcol[j] = 32 * (C0 + j < T32 ? C0 + j : 0) + (lane & 31);

    // a diagonal group (C0 == R0) holds tiles (R0, R0) and (R0 + 1, R0 + 1) at acc[0][0] and acc[1][1];
    // lane l has the diagonal entry of each in register rd (when 8 (rd / 4) + rd % 4 =
    // l % 32 - 4 (l / 32) has a solution), and keeps its fp64 sums in dg[]
    const bool dgroup = active && C0 == R0;
    const int dt = (lane & 31) - 4 * (lane >> 5);
    const int rd = (dt >= 0 && (dt & 7) < 4) ? 4 * (dt >> 3) + (dt & 7) : -1;
    double dg[2] = {0.0, 0.0};
    auto fold_diag = [&]() {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float v = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                v = r == rd ? acc[k][k][r] : v;
                acc[k][k][r] = r == rd ? 0.f : acc[k][k][r];
            }
            dg[k] += (double)v;
        }
    };

    if (tb < te) gload(tb);
    int cur = 0;
    int chunk = 0;
    for (int64_t t0 = tb; t0 < te; t0 += kWK) {
        uint16_t *xs = xw + (size_t)cur * nbp * kWK;
        if (loader) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                uint32_t e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = d[2 * q][c >> 1], hi = d[2 * q + 1][c >> 1];
                    e[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                const int col = 8 * cg + c;
                *(uint4 *)&xs[(size_t)col * kWK + 8 * (tg ^ wswz(col))] = uint4{e[0], e[1], e[2], e[3]};
            }
        }
        __syncthreads();   // this chunk is staged; the other buffer's readers finished last trip
        if (t0 + kWK < te) gload(t0 + kWK);
        if (active) {
#pragma unroll
            for (int kk = 0; kk < kWK; kk += 16) {
                const int gq = (kk >> 3) + (lane >> 5);
                bf16x8 a[2], bv[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8 *)&xs[(size_t)acol[i] * kWK + 8 * (gq ^ wswz(acol[i]))];
#pragma unroll
                for (int j = 0; j < 4; ++j) bv[j] = *(const bf16x8 *)&xs[(size_t)bcol[j] * kWK + 8 * (gq ^ wswz(bcol[j]))];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bv[j], acc[i][j], 0, 0, 0);
            }
        }
        if (dgroup && ++chunk == kWFold) {
            fold_diag();
            chunk = 0;
        }
        cur ^= 1;
    }
    if (dgroup) fold_diag();
    if (!active) return;

    const int64_t tot_blocks = (int64_t)nblk * (gridDim.x / (wgs * nblk));
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    float *Pb = partial ? partial + ((int64_t)blockIdx.y * tot_blocks + rest) * nb * nb : nullptr;
    const double invN = 1.0 / (double)N, bd = (double)beta;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (R0 + i >= T32 || C0 + j >= T32 || C0 + j < R0 + i) continue;
            const int gj = 32 * (C0 + j) + acc_col(lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = 32 * (R0 + i) + acc_row(r, lane);
                if (gi >= nb || gj >= nb || gi > gj) continue;
                // the diagonal entries of a diagonal group are all in dg (acc holds 0 there)
                const double sum = (dgroup && i == j && r == rd) ? dg[i] : (double)acc[i][j][r];
                if (Pb) {
                    Pb[(int64_t)gi * nb + gj] = (float)sum;
                } else {
                    const double old = beta > 0.f ? (double)Ab[(int64_t)gi * nb + gj] : 0.0;
                    const float v = (float)(bd * old + (1.0 - bd) * (sum * invN));
                    Ab[(int64_t)gi * nb + gj] = v;
                    Ab[(int64_t)gj * nb + gi] = v;
                }
            }
        }
}

// The same tile groups, with X staged by the memory engine: each wave's buffer loads write their
// 16 bytes per lane straight into LDS (no registers, no repacking), so three 64-token chunks fit
// in LDS and two are in flight while the third is multiplied.  LDS keeps X's own layout, rows of
// PC columns (PC = 32 mod 128, so that the four rows one half-wave reads fall in disjoint banks);
// columns nb .. PC - 1 and tokens past the split are loaded from an offset past the end of the
// buffer, i.e. as zeros.  The MFMA operands (8 tokens of one column per lane) come from gfx950's
// transposing LDS read: ds_read_b64_tr_b16 gives lane i of each 16-lane group, as its element j,
// element i % 4 of the 8 bytes addressed by lane 4 j + i / 4, so lanes that address 4 tokens x 4
// four-column pieces receive 4 tokens of one column each; two reads make an operand.
// The three buffers are separate LDS arrays and the loop is unrolled over them, so that the
// compiler sees which buffer each load writes and each read reads, and waits before a read only
// for the loads into that buffer; the barrier is written out (waits on this wave's own loads of
// the next chunk, then s_barrier) so that it does not wait for the loads still in flight.  Every wave
// issues the same number of loads in every step (a chunk's 16-byte pieces come in PC / 8 loads of
// 1 KiB, 4 mod 8 of them: waves 4..7 repeat their previous load, same bytes to the same place),
// including loads of chunks past the split's end (all lanes out of range: zeros, no memory
// traffic), so that the compiler's count of loads in flight is exact on every path.
constexpr int kWDMaxCols = 416;    // 3 x 64 x 416 x 2 B = 156 KiB of LDS

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4;
typedef __attribute__((address_space(3))) void *lds_void;

__device__ __forceinline__ bf16x8 tr_operand(const uint8_t *p, int pitch4) {
    // two transposing reads, 4 tokens apart: the lane's 8 tokens of one column
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p + pitch4));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// s_waitcnt vmcnt(N), expcnt and lgkmcnt left alone (N < 16)
template <int N>
__device__ __forceinline__ void vm_wait() { __builtin_amdgcn_s_waitcnt(0x0f70 | N); }

// The staging plan of one workgroup of NW waves: a chunk's kWK token rows of PC / 8 16-byte pieces
// are PC / 8 loads of 1 KiB; wave w issues loads w, w + NW, ... (the last one again where that
// passes the count, so that every wave issues kNld per chunk); load r fills LDS bytes
// [1 KiB r, 1 KiB (r + 1)) of the buffer, lane l the piece P = 64 r + l: token P / (PC / 8), piece
// P % (PC / 8) of that token's row.  Pieces from column nb on, and tokens from the split's end on,
// load from an offset past the end of the buffer (zeros).  A piece that runs past column nb (nb % 8
// = 4) brings 4 columns of the next block, which only feed discarded entries.
template <int PC, int NW>
struct DmaPlan {
    static constexpr int kPitch = 2 * PC;                 // bytes per token row
    static constexpr int kBytes = kWK * kPitch;           // one chunk
    static constexpr int kPpr = PC / 8;                   // pieces per row = loads per chunk
    static constexpr int kNld = (kPpr + NW - 1) / NW;     // loads per chunk and wave
    static_assert(PC % 128 == 32 && kPpr >= NW, "rows of 32 mod 128 columns, one load per wave at least");
    __amdgpu_buffer_rsrc_t rX;
    int64_t ld, te;
    int ldr[kNld], tkn[kNld];
    unsigned boff[kNld];
    __device__ __forceinline__ DmaPlan(const uint16_t *Xb, int64_t range, int64_t ld_, int nb, int64_t te_, int w, int lane)
        : ld(ld_), te(te_) {
        rX = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(Xb), (short)0, (int)(range * 2), 0x00020000);
#pragma unroll
        for (int i = 0; i < kNld; ++i) {
            const int r = w + NW * i < kPpr ? w + NW * i : w + NW * (i - 1);
            const int P = 64 * r + lane;
            const int tk = P / kPpr, pc = P - tk * kPpr;
            ldr[i] = r;
            tkn[i] = 8 * pc < nb ? tk : kWK;   // padding columns: never in range
            boff[i] = (unsigned)(((int64_t)tk * ld + 8 * pc) * 2);
        }
    }
    // the chunk of tokens t0 .. t0 + kWK - 1 into buf (all zeros when t0 >= te)
    __device__ __forceinline__ void issue(int64_t t0, uint8_t *buf) const {
        const int lim = (int)max<int64_t>(-1, min<int64_t>(kWK, te - t0));
        const unsigned base = lim > 0 ? (unsigned)(t0 * ld * 2) : 0u;
#pragma unroll
        for (int i = 0; i < kNld; ++i) {
            const unsigned off = tkn[i] < lim ? base + boff[i] : kWOff;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (lds_void)(buf + 1024 * ldr[i]), 16, off, 0, 0, 0);
        }
    }
};

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// body(cur) for the chunks t0 = tb, tb + kWK, .. < te, each in LDS at cur, with NBUF chunk buffers
// (NBUF - 1 chunks in flight).  A step refills the previous chunk's buffer with the chunk NBUF - 1
// ahead, runs the body, waits for this wave's loads of the next chunk (those of the chunks after it
// stay in flight) and meets the barrier (every wave's loads of the next chunk have landed and every
// wave is done with cur).  Unrolled twice over the buffers: the compiler's count of loads in flight
// merges less precisely at the loop head, where its first read also waits for the next chunk.  On
// return no load is in flight.
template <int NBUF, class Plan, class Body>
__device__ __forceinline__ void dma_chunks(const Plan &L, int64_t tb, int64_t te, uint8_t *const (&buf)[NBUF],
                                           Body &&body) {
    static_assert((NBUF - 2) * Plan::kNld < 16, "vmcnt immediate");
    auto step = [&](int64_t t0, const uint8_t *cur, uint8_t *nxt) {
        L.issue(t0 + (NBUF - 1) * kWK, nxt);
        body(cur);
        if (t0 + kWK < te) vm_wait<(NBUF - 2) * Plan::kNld>(); else vm_wait<0>();
        lds_barrier();
    };
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k) L.issue(tb + k * kWK, buf[k]);
    vm_wait<(NBUF - 2) * Plan::kNld>();
    lds_barrier();
    for (int64_t t0 = tb; t0 < te; t0 += 2 * NBUF * kWK) {
#pragma unroll
        for (int k = 0; k < 2 * NBUF; ++k) {
            if (t0 + k * kWK >= te) break;
            step(t0 + k * kWK, buf[k % NBUF], buf[(k + NBUF - 1) % NBUF]);
        }
    }
    vm_wait<0>();   // the loads past the end: none may land after the workgroup has ended
}

// operand address within a chunk buffer: lane (group G = lane / 16, q = lane % 16) points at token
// 8 (G / 2) + q / 4 and columns 16 (G % 2) + 4 (q % 4) .. + 3 of 32-column tile `tile`
template <int PITCH>
__device__ __forceinline__ int tr_lane_offset(int lane, int tile) {
    const int G = lane >> 4, q = lane & 15;
    return (8 * (G >> 1) + (q >> 2)) * PITCH + 2 * (16 * (G & 1) + 4 * (q & 3)) + 64 * tile;
}

// grid.x = wgs (fastest) x blocks x matrices, renumbered per XCD; grid.y = token splits; block 512
template <int PC>
__global__ void __launch_bounds__(512) k_syrk_wide_dma(int64_t N, int nb, int T32, int ngroups, int wgs, int nblk,
                                                       int64_t tok_per_split, int nsplit, float beta, AccTable t,
                                                       WideGroups grp, float *partial) {
    using D = DmaPlan<PC, 8>;
    __shared__ __align__(16) uint8_t xb0[D::kBytes], xb1[D::kBytes], xb2[D::kBytes];
    uint8_t *const bufs[3] = {xb0, xb1, xb2};
    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int wg = x % wgs, rest = x / wgs;
    const int b = rest % nblk, mat = rest / nblk;
    const int64_t tb = (int64_t)blockIdx.y * tok_per_split;
    const int64_t te = min<int64_t>(N, tb + tok_per_split);
    const int64_t ld = t.ldx[mat];
    const uint16_t *Xb = (const uint16_t *)t.X[mat] + (int64_t)b * nb;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const D L(Xb, N * ld - (int64_t)b * nb, ld, nb, te, w, lane);

    const int g = wg * 8 + w;
    const bool active = g < ngroups;
    const int R0 = active ? grp.r0[g] : 0, C0 = active ? grp.c0[g] : 0;
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
    int aof[2], bof[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) aof[i] = tr_lane_offset<D::kPitch>(lane, R0 + i < T32 ? R0 + i : 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) bof[j] = tr_lane_offset<D::kPitch>(lane, C0 + j < T32 ? C0 + j : 0);

    const bool dgroup = active && C0 == R0;
    const int dt = (lane & 31) - 4 * (lane >> 5);
    const int rd = (dt >= 0 && (dt & 7) < 4) ? 4 * (dt >> 3) + (dt & 7) : -1;
    double dg[2] = {0.0, 0.0};
    auto fold_diag = [&]() {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float v = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                v = r == rd ? acc[k][k][r] : v;
                acc[k][k][r] = r == rd ? 0.f : acc[k][k][r];
            }
            dg[k] += (double)v;
        }
    };
    int chunk = 0;
    dma_chunks(L, tb, te, bufs, [&](const uint8_t *cur) {
        if (active) {
#pragma unroll
            for (int kk = 0; kk < kWK; kk += 16) {
                bf16x8 a[2], bv[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) a[i] = tr_operand(cur + aof[i] + kk * D::kPitch, 4 * D::kPitch);
#pragma unroll
                for (int j = 0; j < 4; ++j) bv[j] = tr_operand(cur + bof[j] + kk * D::kPitch, 4 * D::kPitch);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bv[j], acc[i][j], 0, 0, 0);
            }
        }
        if (dgroup && ++chunk == kWFold) {
            fold_diag();
            chunk = 0;
        }
    });
    if (dgroup) fold_diag();
    if (!active) return;

    const int64_t tot_blocks = (int64_t)nblk * (gridDim.x / (wgs * nblk));
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    float *Pb = partial ? partial + ((int64_t)blockIdx.y * tot_blocks + rest) * nb * nb : nullptr;
    const double invN = 1.0 / (double)N, bd = (double)beta;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (R0 + i >= T32 || C0 + j >= T32 || C0 + j < R0 + i) continue;
            const int gj = 32 * (C0 + j) + acc_col(lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = 32 * (R0 + i) + acc_row(r, lane);
                if (gi >= nb || gj >= nb || gi > gj) continue;
                const double sum = (dgroup && i == j && r == rd) ? dg[i] : (double)acc[i][j][r];
                if (Pb) {
                    Pb[(int64_t)gi * nb + gj] = (float)sum;
                } else {
                    const double old = beta > 0.f ? (double)Ab[(int64_t)gi * nb + gj] : 0.0;
                    const float v = (float)(bd * old + (1.0 - bd) * (sum * invN));
                    Ab[(int64_t)gi * nb + gj] = v;
                    Ab[(int64_t)gj * nb + gi] = v;
                }
            }
        }
}

// Blocks of 33 .. 128 columns, bf16 X (nb % 4 == 0), the same staging with four waves: one
// workgroup per block and token split, two per CU (a fourth chunk buffer, three chunks in flight,
// measured no faster: 2.05 against 2.03 ms for the GPT-2 XL nb = 100 set).  The upper triangle's T32 (T32 + 1) / 2 tiles
// of 32 x 32 (at most 10) go to the waves in turn, at most 3 per wave; every 4 chunks (256
// tokens) the fp32 sums move into fp64 registers, so a split needs no fp32 length limit and the
// bf16 token-split plan applies (one split for the GPT-2 XL set, the EMA fused in the epilogue).
constexpr int kNMaxTiles = 3;
__global__ void __launch_bounds__(256) k_syrk_narrow_dma(int64_t N, int nb, int T32, int nblk, int64_t tok_per_split,
                                                         int nsplit, float beta, AccTable t, double *partial) {
    using D = DmaPlan<160, 4>;
    __shared__ __align__(16) uint8_t xb0[D::kBytes], xb1[D::kBytes], xb2[D::kBytes];
    uint8_t *const bufs[3] = {xb0, xb1, xb2};
    const int rest = xcd_remap(blockIdx.x, gridDim.x);
    const int b = rest % nblk, mat = rest / nblk;
    const int64_t tb = (int64_t)blockIdx.y * tok_per_split;
    const int64_t te = min<int64_t>(N, tb + tok_per_split);
    const int64_t ld = t.ldx[mat];
    const uint16_t *Xb = (const uint16_t *)t.X[mat] + (int64_t)b * nb;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const D L(Xb, N * ld - (int64_t)b * nb, ld, nb, te, w, lane);

    // tiles w, w + 4, w + 8 of the row-major upper triangle
    const int ntiles = T32 * (T32 + 1) / 2;
    int ti[kNMaxTiles], tj[kNMaxTiles], aof[kNMaxTiles], bof[kNMaxTiles];
    bool has[kNMaxTiles];
    f32x16 acc[kNMaxTiles];
    double accd[kNMaxTiles][16];
#pragma unroll
    for (int k = 0; k < kNMaxTiles; ++k) {
        has[k] = w + 4 * k < ntiles;
        tile_pair(has[k] ? w + 4 * k : 0, T32, ti[k], tj[k]);
        aof[k] = tr_lane_offset<D::kPitch>(lane, ti[k]);
        bof[k] = tr_lane_offset<D::kPitch>(lane, tj[k]);
        acc[k] = (f32x16){};
#pragma unroll
        for (int r = 0; r < 16; ++r) accd[k][r] = 0.0;
    }
    int chunk = 0;
    dma_chunks(L, tb, te, bufs, [&](const uint8_t *cur) {
#pragma unroll
        for (int kk = 0; kk < kWK; kk += 16) {
#pragma unroll
            for (int k = 0; k < kNMaxTiles; ++k) {
                if (!has[k]) continue;
                const bf16x8 a = tr_operand(cur + aof[k] + kk * D::kPitch, 4 * D::kPitch);
                const bf16x8 bv = tr_operand(cur + bof[k] + kk * D::kPitch, 4 * D::kPitch);
                acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[k], 0, 0, 0);
            }
        }
        if (++chunk == 4) {
            chunk = 0;
#pragma unroll
            for (int k = 0; k < kNMaxTiles; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r) { accd[k][r] += (double)acc[k][r]; acc[k][r] = 0.f; }
        }
    });

    const double invN = 1.0 / (double)N, bd = (double)beta;
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const int64_t tot_blocks = gridDim.x;
    double *Pb = partial ? partial + ((int64_t)blockIdx.y * tot_blocks + rest) * nb * nb : nullptr;
#pragma unroll
    for (int k = 0; k < kNMaxTiles; ++k) {
        if (!has[k]) continue;
        const int gj = 32 * tj[k] + acc_col(lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int gi = 32 * ti[k] + acc_row(r, lane);
            if (gi >= nb || gj >= nb || gi > gj) continue;
            const double sum = accd[k][r] + (double)acc[k][r];
            if (nsplit == 1) {
                const double old = beta > 0.f ? (double)Ab[(int64_t)gi * nb + gj] : 0.0;
                const float v = (float)(bd * old + (1.0 - bd) * (sum * invN));
                Ab[(int64_t)gi * nb + gj] = v;
                Ab[(int64_t)gj * nb + gi] = v;
            } else {
                Pb[(int64_t)gi * nb + gj] = sum;
            }
        }
    }
}

// Sum the token-split partials in split order, apply the EMA, write both triangles.  One
// workgroup per 32 x 32 tile (I, J), I <= J, of a block: the partials of the upper triangle are
// read along rows, and the mirrored tile (J, I) goes out through LDS, also along rows.
// grid.x = T32 (T32 + 1) / 2 tile pairs, grid.y = block index within the launch (nblk * count).
template <typename PT>
__global__ void __launch_bounds__(256) k_syrk_reduce(int64_t N, int nb, int nblk, int nsplit, int64_t tot_blocks,
                                                     float beta, AccTable t, const PT *partial) {
    __shared__ float tile[32][33];
    const int T32 = (nb + 31) / 32;
    int I, J;
    tile_pair(blockIdx.x, T32, I, J);
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const double bd = (double)beta, invN = 1.0 / (double)N;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = tid + 256 * k, r = e >> 5, c = e & 31;
        const int i = 32 * I + r, j = 32 * J + c;
        float v = 0.f;
        if (i < nb && j < nb && i <= j) {
            const int64_t off = (int64_t)i * nb + j;
            double s = 0.0;
            for (int sp = 0; sp < nsplit; ++sp) s += (double)partial[((int64_t)sp * tot_blocks + g) * nb * nb + off];
            const double old = beta > 0.f ? (double)Ab[off] : 0.0;
            v = (float)(bd * old + (1.0 - bd) * (s * invN));
            Ab[off] = v;
        }
        tile[r][c] = v;
    }
    __syncthreads();
    // mirror: A[32 J + r][32 I + c] = tile[c][r] for entries strictly below the diagonal
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = tid + 256 * k, r = e >> 5, c = e & 31;
        const int i = 32 * J + r, j = 32 * I + c;
        if (i < nb && j < nb && j < i) Ab[(int64_t)i * nb + j] = tile[c][r];
    }
}

// The same for the fp32 partials of the wide kernels when nb % 4 == 0 and A is 16-byte aligned: one
// four-column piece of a tile row per thread, the partials of up to kRedBatch splits loaded before
// they are added (in split order, as above).  In a diagonal tile the pieces straddling the diagonal
// read partials below it (never written) but keep only the entries on and above it.  (One
// workgroup per 32-row band going over its tiles measured slower: 3.62 against 3.59 ms for the
// nb = 400 capture with this reduce.)
constexpr int kRedBatch = 8;
__global__ void __launch_bounds__(256) k_syrk_reduce4(int64_t N, int nb, int nblk, int nsplit, int64_t tot_blocks,
                                                      float beta, AccTable t, const float *partial) {
    __shared__ float tile[32][33];
    const int T32 = (nb + 31) / 32;
    int I, J;
    tile_pair(blockIdx.x, T32, I, J);
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    float *Ab = t.A[mat] + (int64_t)b * nb * nb;
    const double bd = (double)beta, invN = 1.0 / (double)N;
    const int tid = threadIdx.x, r = tid >> 3, c = 4 * (tid & 7);
    const int i = 32 * I + r, j = 32 * J + c;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < nb && j < nb) {   // nb % 4 == 0: the whole piece is in range
        const int64_t off = (int64_t)i * nb + j;
        const int64_t pstride = tot_blocks * nb * nb;
        const float *p = partial + (int64_t)g * nb * nb + off;
        double sum[4] = {0.0, 0.0, 0.0, 0.0};
        for (int sp0 = 0; sp0 < nsplit; sp0 += kRedBatch) {
            f32x4 q[kRedBatch];
#pragma unroll
            for (int k = 0; k < kRedBatch; ++k)
                q[k] = sp0 + k < nsplit ? *(const f32x4 *)(p + (int64_t)(sp0 + k) * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < kRedBatch; ++k)
                if (sp0 + k < nsplit) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum[e] += (double)q[k][e];
                }
        }
        const f32x4 old = beta > 0.f ? *(const f32x4 *)(Ab + off) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (float)(bd * (double)old[e] + (1.0 - bd) * (sum[e] * invN));
        if (I < J) {
            *(f32x4 *)(Ab + off) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (i <= j + e) Ab[off + e] = v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[r][c + e] = v[e];
    __syncthreads();
    // mirror: A[32 J + r][32 I + c + e] = tile[c + e][r] for entries strictly below the diagonal
    const int i2 = 32 * J + r, j2 = 32 * I + c;
    if (i2 < nb && j2 < nb) {
        const f32x4 m = {tile[c][r], tile[c + 1][r], tile[c + 2][r], tile[c + 3][r]};
        float *dst = Ab + (int64_t)i2 * nb + j2;
        if (I < J) {
            *(f32x4 *)dst = m;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j2 + e < i2) dst[e] = m[e];
        }
    }
}

}  // namespace

// 2 x 4 tile groups over the upper triangle of a T32 x T32 grid of 32 x 32 tiles
static int wide_groups(int T32, WideGroups *g) {
    int n = 0;
    for (int r = 0; r < T32; r += 2)
        for (int c = r; c < T32; c += 4) {
            if (g && n < kWMaxGroups) { g->r0[n] = (uint8_t)r; g->c0[n] = (uint8_t)c; }
            ++n;
        }
    return n;
}

static bool wide_shape(int64_t nb) { return nb > 128 && nb <= 512 && nb % 8 == 0; }

// LDS row width of k_syrk_wide_dma for T32 tiles: the least width >= 32 T32 that is 32 mod 128
static int dma_cols(int T32) {
    const int c = 32 * T32;
    return c + ((32 - c % 128) + 128) % 128;
}


// Split plan of the wide kernel: at most kWSplitMax tokens per split (the fp32 sum length), enough
// workgroups for about four per CU, at least 256 tokens per split, lengths a multiple of kWK.
static int wide_plan(const dobb_shape &sh, int64_t N, int count, int64_t *tps) {
    const int nb = (int)sh.nb, T32 = (nb + 31) / 32;
    const int wgs = (wide_groups(T32, nullptr) + 7) / 8;
    const int64_t wgtot = (int64_t)wgs * (sh.n / nb) * (count < kMaxMats ? count : kMaxMats);
    int64_t nsplit = (1024 + wgtot - 1) / wgtot;
    if (nsplit > N / 256) nsplit = N / 256;
    const int64_t need = (N + kWSplitMax - 1) / kWSplitMax;
    if (nsplit < need) nsplit = need;
    if (nsplit < 1) nsplit = 1;
    const int64_t len = ((N + nsplit - 1) / nsplit + kWK - 1) / kWK * kWK;
    if (tps) *tps = len;
    return (int)((N + len - 1) / len);
}

// Token split plan: enough workgroups for >= 4 per CU, >= 256 tokens per split, split length a
// multiple of 64 tokens (the fp64 fold period).  Returns the number of splits; *tps its length.
int accumulate_plan(const dobb_shape &sh, int64_t N, int count, int64_t *tps, bool bf16) {
    const int nb = (int)sh.nb;
    const int tile = bf16 ? kST : kBM;
    const int T = (nb + tile - 1) / tile;
    const int64_t tiles = (int64_t)T * (T + 1) / 2 * (sh.n / nb) * (count < kMaxMats ? count : kMaxMats);
    // bf16: 512 tile pairs already fill the chip (the fp64 fold makes a split unnecessary for accuracy)
    const int64_t target = bf16 ? 512 : 1024;
    int64_t nsplit = (target + tiles - 1) / tiles;
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
    const int cnt = count < kMaxMats ? count : kMaxMats;
    const size_t per = (size_t)cnt * (size_t)(sh.n / sh.nb) * sh.nb * sh.nb;
    size_t bytes = nsplit > 1 ? (size_t)nsplit * per * sizeof(double) : 0;
    if (wide_shape(sh.nb)) {   // fp32 partials of the wide kernel
        const int ws = wide_plan(sh, N, count, nullptr);
        if (ws > 1 && (size_t)ws * per * sizeof(float) > bytes) bytes = (size_t)ws * per * sizeof(float);
    }
    return bytes;
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
        bool vec4 = nb % 4 == 0, vec8 = nb % 8 == 0, wide_ok = true;
        for (int i = 0; i < cnt; ++i) {
            t.X[i] = a.X[c0 + i]; t.A[i] = a.A[c0 + i]; t.ldx[i] = a.ldx[c0 + i];
            const uintptr_t p = (uintptr_t)t.X[i];
            vec4 = vec4 && (t.ldx[i] % 4 == 0) && ((p & (xbf ? 7u : 15u)) == 0);
            vec8 = vec8 && (t.ldx[i] % 8 == 0) && ((p & 15u) == 0);
            wide_ok = wide_ok && a.N * t.ldx[i] * 2 < ((int64_t)1 << 31);   // 32-bit buffer offsets
        }
        if (xbf && vec8 && wide_ok && wide_shape(nb)) {
            const int T32 = (nb + 31) / 32;
            WideGroups grp{};
            const int ngroups = wide_groups(T32, &grp);
            const int wgs = (ngroups + 7) / 8;
            int64_t wtps = a.N;
            const int wsplit = wide_plan(a.sh, a.N, a.count, &wtps);
            float *wpart = wsplit > 1 ? (float *)a.partial : nullptr;
            dim3 grid((unsigned)(wgs * nblk * cnt), (unsigned)wsplit);
            const int pcols = dma_cols(T32);
            if (pcols <= kWDMaxCols) {
#define DOBB_WDMA(PC) DOBB_LAUNCH("accumulate_syrk_wide", s, k_syrk_wide_dma<PC>, grid, dim3(512), 0, a.N, nb, T32, ngroups, wgs, nblk, wtps, wsplit, a.beta, t, grp, wpart)
                if (pcols == 160) DOBB_WDMA(160); else if (pcols == 288) DOBB_WDMA(288); else DOBB_WDMA(416);
#undef DOBB_WDMA
            } else {
                const size_t lds = (size_t)2 * 32 * T32 * kWK * sizeof(uint16_t);
                (void)hipFuncSetAttribute((const void *)k_syrk_wide, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                DOBB_LAUNCH("accumulate_syrk_wide", s, k_syrk_wide, grid, dim3(512), lds, a.N, nb, T32, ngroups, wgs, nblk,
                            wtps, wsplit, a.beta, t, grp, wpart);
            }
            if (wsplit > 1) {
                const int64_t tot = (int64_t)nblk * cnt;
                dim3 g2((unsigned)(T32 * (T32 + 1) / 2), (unsigned)tot);
                bool a16 = true;
                for (int i = 0; i < cnt; ++i) a16 = a16 && ((uintptr_t)t.A[i] & 15u) == 0;
                if (a16)   // nb % 8 == 0 here
                    DOBB_LAUNCH("accumulate_reduce", s, k_syrk_reduce4, g2, dim3(256), 0, a.N, nb, nblk, wsplit, tot,
                                a.beta, t, (const float *)wpart);
                else
                    DOBB_LAUNCH("accumulate_reduce", s, k_syrk_reduce<float>, g2, dim3(256), 0, a.N, nb, nblk, wsplit, tot,
                                a.beta, t, (const float *)wpart);
            }
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            c0 += cnt;
            continue;
        }
        dim3 grid((unsigned)(npairs * nblk * cnt), (unsigned)nsplit);
        double *part = nsplit > 1 ? a.partial : nullptr;
        if (xbf && vec4 && wide_ok && nb > 32 && nb <= 128) {
            DOBB_LAUNCH("accumulate_syrk_bf16", s, k_syrk_narrow_dma, grid, dim3(256), 0, a.N, nb, (nb + 31) / 32, nblk,
                        tps, nsplit, a.beta, t, part);
        } else if (xbf) {
#define DOBB_SYRKB(V) DOBB_LAUNCH("accumulate_syrk_bf16", s, (k_syrk_bf16<V>), grid, dim3(512), 0, a.N, nb, T, npairs, nblk, tps, nsplit, a.beta, t, part)
            if (vec8) DOBB_SYRKB(8); else if (vec4) DOBB_SYRKB(4); else DOBB_SYRKB(1);
#undef DOBB_SYRKB
        } else {
#define DOBB_SYRK(V) DOBB_LAUNCH("accumulate_syrk_f64", s, (k_syrk<V>), grid, dim3(256), 0, a.N, nb, T, npairs, nblk, tps, nsplit, a.beta, t, part)
            if (vec4) DOBB_SYRK(true); else DOBB_SYRK(false);
#undef DOBB_SYRK
        }
        if (nsplit > 1) {
            const int64_t tot = (int64_t)nblk * cnt;
            const int T32 = (nb + 31) / 32;
            dim3 g2((unsigned)(T32 * (T32 + 1) / 2), (unsigned)tot);
            DOBB_LAUNCH("accumulate_reduce", s, k_syrk_reduce<double>, g2, dim3(256), 0, a.N, nb, nblk, nsplit, tot, a.beta, t,
                        (const double *)part);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
