// The Dobb-l2 step (column-l2 normalisation of the coefficients) for block widths nb <= 128,
// nb % 4 == 0: row tiles staged through LDS.
//
// Dobb paper (arXiv 2610.39412): Tables 11-12 (Dobb-l2: every column of C_b scaled to unit l2 norm
// over the rows), abstract (projection and reconstruction in the block bases), Table 9 (update
// scale), Table 21 caption (decoupled weight decay), Table 19 (Nesterov).  The sign step of these
// widths runs in one pass (k_step_fused.hip); the column norms need every row's coefficients before
// any row can be reconstructed, so this step takes two passes with C in the workspace.
//
// C = P Q with both operands split into two fp16 parts (three products: hi*hi, hi*lo, lo*hi).  The
// rows of P are first scaled by a power of two (exact) that puts each row's largest magnitude in
// [2^13, 2^14), so the fp16 parts neither overflow nor lose the row's scale; C is stored unscaled.
// U = C~ Q^T with C~ = C diag(colscale), |C~| <= 1, split into two fp16 parts, and Q split into two
// (three products).
//
// Layout of the work: a workgroup (8 waves) owns one block b; it splits Q_b into LDS once and then
// streams tiles of TR rows.  Every global access walks along rows (consecutive lanes take
// consecutive 16- or 8-byte pieces of a row's nb-wide slice).  The MFMA operands are read from LDS
// tiles:
//   k_proj_rows   M, G rows -> M <- mu M + G (written back), P -> LDS (fp32);
//                 waves take (32-row tile, column chunks): C^T = Q^T P^T; C -> LDS -> rows, with
//                 each tile's column sums of squares (fp64)
//   k_colscale    the column scales 1 / ||C[:, j]|| from the tiles' sums
//   k_recon_rows  C rows -> C~ in LDS; U^T = Q C~^T; U -> LDS -> rows, where
//                 W <- W - lr (s U + wd W) is applied to the W rows loaded one tile ahead
// The next tile's rows are loaded while the current tile's products run.
#include "step_common.h"

#include <type_traits>

namespace dobb {
namespace {
using namespace stepk;

constexpr int kRT = 512;    // threads per workgroup (8 waves)
constexpr int kKS = 16;     // k per MFMA step
constexpr int kPadK = 8;    // Q plane row padding (2-byte elements)

// LDS geometry shared by host and device
struct RowsGeo {
    int KS, kpad, qld, pld, uld, NCH;
};
__host__ __device__ inline RowsGeo rows_geo(int nb) {
    RowsGeo g;
    g.KS = (nb + kKS - 1) / kKS;
    g.kpad = g.KS * kKS;
    g.qld = g.kpad + kPadK;     // Q planes: 2-byte elements per row
    g.pld = g.kpad + 4;         // P tile: fp32 per row; (pld / 4) odd keeps 16 rows on distinct banks
    g.uld = nb + 4 + ((nb / 4) % 2 == 0 ? 0 : 4);   // U tile: fp32 per row, (uld / 4) odd
    g.NCH = (nb + 31) / 32;
    return g;
}
__host__ __device__ inline size_t a16(size_t x) { return (x + 15) / 16 * 16; }

// ---- projection ----------------------------------------------------------------------------------
struct ProjRowsTable {
    float *M[kMaxMats];
    const void *G[kMaxMats];
    const float *Q[kMaxMats];
    float *C[kMaxMats];        // the coefficients (m x n fp32)
    double *part[kMaxMats];    // per row tile, the column sums of squares ([tiles][n])
    float *Cout[kMaxMats];     // NULL or m x n fp32: the coefficients (verification output)
    float mu[kMaxMats];
};
// LDS: Q_b^T (two fp16 planes) and the P tile (fp32), which later holds the C tile
__host__ __device__ inline size_t proj_rows_lds(int nb, int TR) {
    const RowsGeo g = rows_geo(nb);
    return a16((size_t)2 * nb * g.qld * 2) + a16((size_t)TR * g.pld * 4);
}

// grid.x = tile groups x blocks x matrices (block fastest, renumbered per XCD), block 512.
// TR = 128 or 64 rows per tile; the 8 waves take (32-row tile rt, group cg of column chunks).
// The epilogue writes C (unscaled by the row's power of two) along the rows through the P tile's
// LDS, also to t.Cout when given (a verification output), and each tile's column sums of squares
// in fp64.
template <int NCH, int TR, int NEST, bool GBF16>
__global__ void __launch_bounds__(512) k_proj_rows(int64_t m, int64_t n, int nb, int nblk, int ngroups, int tpg,
                                                   ProjRowsTable t) {
    extern __shared__ __align__(16) unsigned char lds[];
    const RowsGeo geo = rows_geo(nb);
    const int KS = geo.KS, kpad = geo.kpad, qld = geo.qld, pld = geo.pld;
    uint16_t *qs = (uint16_t *)lds;                                          // [2][nb][qld]
    float *ps = (float *)(lds + a16((size_t)2 * nb * qld * 2));              // [TR][pld]

    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int b = x % nblk, rest = x / nblk;
    const int tg = rest % ngroups, mat = rest / ngroups;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t ntile = (m + TR - 1) / TR;
    const int64_t t_begin = (int64_t)tg * tpg;
    const int64_t t_end = t_begin + tpg < ntile ? t_begin + tpg : ntile;

    // Q_b^T split into two fp16 planes (element (p, j) of Q at plane[j][p]); zero for p in [nb, kpad)
    {
        const float *Q = t.Q[mat] + (int64_t)b * nb * nb;
        const int total = kpad * nb;
        for (int e0 = 0; e0 < total; e0 += kRT * 8) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + tid + kRT * i;
                v[i] = (e < total && e < nb * nb) ? Q[e] : 0.f;   // e = p * nb + j
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + tid + kRT * i;
                if (e < total) {
                    const int p = e / nb, j = e - p * nb;
                    uint16_t h, l;
                    split2h(v[i], h, l);
                    qs[(0 * nb + j) * qld + p] = h;
                    qs[(1 * nb + j) * qld + p] = l;
                }
            }
        }
        // the P tiles' columns [nb, kpad) stay zero
        for (int e = tid; e < TR * (kpad - nb); e += kRT) {
            const int r = e / (kpad - nb), c = nb + e % (kpad - nb);
            ps[r * pld + c] = 0.f;
        }
    }

    // row pieces: piece e -> row e / q, columns 4 (e % q) .. + 3 of the block slice
    const int q = nb / 4;
    constexpr int kIPT = (TR * 32 + kRT - 1) / kRT;   // pieces per thread for q <= 32
    float *M = t.M[mat] + (int64_t)b * nb;
    const void *Gv = t.G[mat];
    const float mu = t.mu[mat];
    f32x4 mr[kIPT], gr[kIPT];
    auto load_tile = [&](int64_t tile) {
#pragma unroll
        for (int i = 0; i < kIPT; ++i) {
            const int e = tid + kRT * i;
            const int r = e / q, c = 4 * (e - r * q);
            const int64_t row = tile * TR + r;
            mr[i] = gr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (tile < t_end && e < TR * q && row < m) {
                const int64_t off = row * n + c;
                mr[i] = *(const f32x4 *)(M + off);
                if (GBF16) {
                    const uint2 hb = *(const uint2 *)((const uint16_t *)Gv + (int64_t)b * nb + off);
                    gr[i] = f32x4{bf16_to_f32((uint16_t)hb.x), bf16_to_f32((uint16_t)(hb.x >> 16)),
                                  bf16_to_f32((uint16_t)hb.y), bf16_to_f32((uint16_t)(hb.y >> 16))};
                } else {
                    gr[i] = *(const f32x4 *)((const float *)Gv + (int64_t)b * nb + off);
                }
            }
        }
    };

    constexpr int kRTiles = TR / 32;              // 32-row tiles per tile
    constexpr int kGroups = 8 / kRTiles;          // column-chunk groups
    constexpr int kCPG = (NCH + kGroups - 1) / kGroups;
    const int rt = wv % kRTiles, cg = wv / kRTiles;
    const int kh = 8 * (lane >> 5);

    load_tile(t_begin);
    for (int64_t tile = t_begin; tile < t_end; ++tile) {
        // momentum (written back along the rows) and P into the LDS tile (its last readers passed the
        // previous tile's second barrier)
        float *pc = ps;
#pragma unroll
        for (int i = 0; i < kIPT; ++i) {
            const int e = tid + kRT * i;
            const int r = e / q, c = 4 * (e - r * q);
            const int64_t row = tile * TR + r;
            f32x4 mn, pv;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                mn[cc] = __builtin_fmaf(mu, mr[i][cc], gr[i][cc]);
                pv[cc] = NEST ? __builtin_fmaf(mu, mn[cc], gr[i][cc]) : mn[cc];
            }
            if (e < TR * q) {
                if (row < m) *(f32x4 *)(M + row * n + c) = mn;
                *(f32x4 *)(pc + r * pld + c) = pv;   // rows past m hold zeros (their loads read zero)
            }
        }
        load_tile(tile + 1);
        __syncthreads();
        // the scale of this lane's row: its half of the row (k = 16 ks + kh ..), then the other half
        // from lane ^ 32
        int sexp;
        {
            const float *pr = pc + (32 * rt + (lane & 31)) * pld + kh;
            uint32_t mx = 0u;
            for (int ks = 0; ks < KS; ++ks) {
                const f32x4 p0 = *(const f32x4 *)(pr + ks * kKS), p1 = *(const f32x4 *)(pr + ks * kKS + 4);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const uint32_t u0 = __float_as_uint(p0[cc]) & 0x7fffffffu;
                    const uint32_t u1 = __float_as_uint(p1[cc]) & 0x7fffffffu;
                    mx = u0 > mx ? u0 : mx;
                    mx = u1 > mx ? u1 : mx;
                }
            }
            const uint32_t o = (uint32_t)__shfl_xor((int)mx, 32);
            sexp = row_scale_exp(o > mx ? o : mx);
        }
        // C^T = Q^T P^T for 32-row tile rt and this wave's column chunks
        f32x16 acc[kCPG];
#pragma unroll
        for (int j = 0; j < kCPG; ++j) acc[j] = (f32x16){};
        for (int ks = 0; ks < KS; ++ks) {
            const float *pr = pc + (32 * rt + (lane & 31)) * pld + ks * kKS + kh;
            const f32x4 p0 = *(const f32x4 *)pr, p1 = *(const f32x4 *)(pr + 4);
            uint16_t hh[8], hl[8];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                split2s(__builtin_amdgcn_ldexpf(p0[cc], sexp), hh[cc], hl[cc]);
                split2s(__builtin_amdgcn_ldexpf(p1[cc], sexp), hh[cc + 4], hl[cc + 4]);
            }
            const uint4 uh = {pack2(hh[0], hh[1]), pack2(hh[2], hh[3]), pack2(hh[4], hh[5]), pack2(hh[6], hh[7])};
            const uint4 ul = {pack2(hl[0], hl[1]), pack2(hl[2], hl[3]), pack2(hl[4], hl[5]), pack2(hl[6], hl[7])};
            const f16x8 ah = __builtin_bit_cast(f16x8, uh), al = __builtin_bit_cast(f16x8, ul);
            f16x8 Qh[kCPG], Ql[kCPG];
#pragma unroll
            for (int j = 0; j < kCPG; ++j) {
                const int ch = cg * kCPG + j;
                const int col = 32 * ch + (lane & 31);
                const bool ok = ch < NCH && col < nb;
                const int cs = ok ? col : 0;
                uint4 bh = *(const uint4 *)&qs[(0 * nb + cs) * qld + ks * kKS + kh];
                uint4 bl = *(const uint4 *)&qs[(1 * nb + cs) * qld + ks * kKS + kh];
                if (!ok) bh = bl = uint4{0u, 0u, 0u, 0u};
                Qh[j] = __builtin_bit_cast(f16x8, bh);
                Ql[j] = __builtin_bit_cast(f16x8, bl);
            }
#pragma unroll
            for (int j = 0; j < kCPG; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh[j], ah, acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kCPG; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ql[j], ah, acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kCPG; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh[j], al, acc[j], 0, 0, 0);
        }
        {
            // C tile -> the P tile's LDS (every wave is past its products), then rows out and the
            // tile's column sums of squares (rows past m are zero)
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kCPG; ++j) {
                const int ch = cg * kCPG + j;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int col = 32 * ch + 4 * (lane >> 5) + 8 * qq;
                    if (ch < NCH && col < nb)
                        *(f32x4 *)(pc + (32 * rt + (lane & 31)) * pld + col) =
                            f32x4{__builtin_amdgcn_ldexpf(acc[j][4 * qq], -sexp),
                                  __builtin_amdgcn_ldexpf(acc[j][4 * qq + 1], -sexp),
                                  __builtin_amdgcn_ldexpf(acc[j][4 * qq + 2], -sexp),
                                  __builtin_amdgcn_ldexpf(acc[j][4 * qq + 3], -sexp)};
                }
            }
            __syncthreads();
            float *Cb = t.C[mat] + (int64_t)b * nb;
            float *Co = t.Cout[mat] ? t.Cout[mat] + (int64_t)b * nb : nullptr;
            for (int e = tid; e < TR * q; e += kRT) {
                const int r = e / q, c = 4 * (e - r * q);
                const int64_t row = tile * TR + r;
                if (row < m) {
                    const f32x4 cv = *(const f32x4 *)(pc + r * pld + c);
                    *(f32x4 *)(Cb + row * n + c) = cv;
                    if (Co) *(f32x4 *)(Co + row * n + c) = cv;
                }
            }
            if (tid < nb) {
                double sq = 0.0;
                const int rows = m - tile * TR < TR ? (int)(m - tile * TR) : TR;
                for (int r = 0; r < rows; ++r) {
                    const double v = pc[r * pld + tid];
                    sq += v * v;
                }
                t.part[mat][tile * n + (int64_t)b * nb + tid] = sq;
            }
            __syncthreads();   // the next tile's staging overwrites the P tile
        }
    }
}

// ---- reconstruction ------------------------------------------------------------------------------
struct ReconRowsTable {
    const float *C[kMaxMats];    // the coefficients C (m x n fp32) and the column scales
    const float *cs[kMaxMats];
    const float *Q[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};
// the tile of scaled coefficients, fp32 with pitch kpad + 4 ((pitch / 4) odd), then the block's
// kpad column scales (zero past nb)
__host__ __device__ inline int rows_cpitch(int nb) { return rows_geo(nb).kpad + 4; }
__host__ __device__ inline size_t recon_rows_tile(int nb, int TR) {
    return a16((size_t)TR * rows_cpitch(nb) * 4 + (size_t)rows_geo(nb).kpad * 4);
}
__host__ __device__ inline size_t recon_rows_lds(int nb, int TR) {
    const RowsGeo g = rows_geo(nb);
    return a16((size_t)2 * nb * g.qld * 2) + recon_rows_tile(nb, TR) + a16((size_t)TR * g.uld * 4);
}

// The tile holds C~ = C diag(colscale) in fp32; |C~| <= 1, so it splits into two fp16 parts without
// a scale and U = C~ Q^T takes three products (hi hi, lo(Q) hi, hi lo(C~)).
template <int NCH, int TR, bool WBF16>
__global__ void __launch_bounds__(512) k_recon_rows(int64_t m, int64_t n, int nb, int nblk, int ngroups, int tpg,
                                                    ReconRowsTable t) {
    extern __shared__ __align__(16) unsigned char lds[];
    const RowsGeo geo = rows_geo(nb);
    const int KS = geo.KS, kpad = geo.kpad, qld = geo.qld, uld = geo.uld;
    uint16_t *qs = (uint16_t *)lds;                                          // [2][nb][qld]
    const int cpitch = rows_cpitch(nb);
    float *ct = (float *)(lds + a16((size_t)2 * nb * qld * 2));              // [TR][cpitch]
    float *csl = ct + TR * cpitch;                                           // [kpad]
    float *us = (float *)(lds + a16((size_t)2 * nb * qld * 2) + recon_rows_tile(nb, TR));   // [TR][uld]

    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int b = x % nblk, rest = x / nblk;
    const int tg = rest % ngroups, mat = rest / ngroups;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t ntile = (m + TR - 1) / TR;
    const int64_t t_begin = (int64_t)tg * tpg;
    const int64_t t_end = t_begin + tpg < ntile ? t_begin + tpg : ntile;

    // Q_b split into two fp16 planes in its natural layout (element (p, c) at plane[p][c]); zero for c >= nb
    {
        const float *Q = t.Q[mat] + (int64_t)b * nb * nb;
        const int total = nb * kpad;
        for (int e0 = 0; e0 < total; e0 += kRT * 8) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + tid + kRT * i;
                const int p = e / kpad, c = e - p * kpad;
                v[i] = (e < total && c < nb) ? Q[p * nb + c] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + tid + kRT * i;
                if (e < total) {
                    const int p = e / kpad, c = e - p * kpad;
                    uint16_t h, l;
                    split2h(v[i], h, l);
                    qs[(0 * nb + p) * qld + c] = h;
                    qs[(1 * nb + p) * qld + c] = l;
                }
            }
        }
    }

    // the block's column scales, and zero tile columns [nb, kpad) (the staging writes c < nb only)
    for (int c = tid; c < kpad; c += kRT) csl[c] = c < nb ? t.cs[mat][(int64_t)b * nb + c] : 0.f;
    for (int e = tid; e < TR * (kpad - nb); e += kRT) {
        const int r = e / (kpad - nb), c = nb + e % (kpad - nb);
        ct[r * cpitch + c] = 0.f;
    }
    __syncthreads();
    const float *Cm = t.C[mat];
    const float lr = t.lr[mat], wd = t.wd[mat], sc = t.scale[mat];
    void *const Wv = t.W[mat];
    float *const U = t.U[mat];
    // C and W rows: 4-element pieces, nb / 4 per row
    const int q = nb / 4;
    constexpr int kWPT = (TR * 32 + kRT - 1) / kRT;   // pieces per thread (nb <= 128)
    using WVec = typename std::conditional<WBF16, uint2, f32x4>::type;
    f32x4 cr[kWPT];
    WVec wr[kWPT];
    auto load_tile = [&](int64_t tile) {
#pragma unroll
        for (int i = 0; i < kWPT; ++i) {
            const int e = tid + kRT * i;
            const int r = e / q, c = 4 * (e - r * q);
            const int64_t row = tile * TR + r;
            cr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (tile < t_end && e < TR * q && row < m)
                cr[i] = *(const f32x4 *)(Cm + row * n + (int64_t)b * nb + c);
        }
#pragma unroll
        for (int i = 0; i < kWPT; ++i) {
            const int e = tid + kRT * i;
            const int r = e / q, c = 4 * (e - r * q);
            const int64_t row = tile * TR + r;
            if (tile < t_end && e < TR * q && row < m)
                wr[i] = *(const WVec *)((const char *)Wv + ((row * n + (int64_t)b * nb + c) * (WBF16 ? 2 : 4)));
        }
    };

    constexpr int kRTiles = TR / 32;
    constexpr int kGroups = 8 / kRTiles;
    constexpr int kCPG = (NCH + kGroups - 1) / kGroups;
    const int rt = wv % kRTiles, cg = wv / kRTiles;
    const int kh = 8 * (lane >> 5);

    load_tile(t_begin);
    for (int64_t tile = t_begin; tile < t_end; ++tile) {
#pragma unroll
        for (int i = 0; i < kWPT; ++i) {
            const int e = tid + kRT * i;
            const int r = e / q, c = 4 * (e - r * q);
            if (e < TR * q) {
                const f32x4 sv = *(const f32x4 *)(csl + c);
                *(f32x4 *)(ct + r * cpitch + c) =
                    f32x4{cr[i][0] * sv[0], cr[i][1] * sv[1], cr[i][2] * sv[2], cr[i][3] * sv[3]};
            }
        }
        WVec wcur[kWPT];
#pragma unroll
        for (int i = 0; i < kWPT; ++i) wcur[i] = wr[i];
        load_tile(tile + 1);
        __syncthreads();
        // U^T = Q C~^T for 32-row tile rt and this wave's column chunks
        f32x16 acc[kCPG];
#pragma unroll
        for (int j = 0; j < kCPG; ++j) acc[j] = (f32x16){};
        for (int ks = 0; ks < KS; ++ks) {
            f16x8 as, al;
            {
                const float *cp = ct + (32 * rt + (lane & 31)) * cpitch + ks * kKS + kh;
                const f32x4 c0 = *(const f32x4 *)cp, c1 = *(const f32x4 *)(cp + 4);
                uint16_t hh[8], hl[8];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    split2h(c0[cc], hh[cc], hl[cc]);
                    split2h(c1[cc], hh[cc + 4], hl[cc + 4]);
                }
                as = __builtin_bit_cast(f16x8, uint4{pack2(hh[0], hh[1]), pack2(hh[2], hh[3]), pack2(hh[4], hh[5]), pack2(hh[6], hh[7])});
                al = __builtin_bit_cast(f16x8, uint4{pack2(hl[0], hl[1]), pack2(hl[2], hl[3]), pack2(hl[4], hl[5]), pack2(hl[6], hl[7])});
            }
            f16x8 Bh[kCPG], Bl[kCPG];
#pragma unroll
            for (int j = 0; j < kCPG; ++j) {
                const int ch = cg * kCPG + j;
                const int p = 32 * ch + (lane & 31);
                const bool ok = ch < NCH && p < nb;
                const int ps = ok ? p : 0;
                uint4 bh = *(const uint4 *)&qs[(0 * nb + ps) * qld + ks * kKS + kh];
                uint4 bl = *(const uint4 *)&qs[(1 * nb + ps) * qld + ks * kKS + kh];
                if (!ok) bh = bl = uint4{0u, 0u, 0u, 0u};
                Bh[j] = __builtin_bit_cast(f16x8, bh);
                Bl[j] = __builtin_bit_cast(f16x8, bl);
            }
#pragma unroll
            for (int j = 0; j < kCPG; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Bh[j], as, acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kCPG; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Bl[j], as, acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kCPG; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Bh[j], al, acc[j], 0, 0, 0);
        }
        // U tile -> LDS: lane holds row 32 rt + l % 32, columns 32 ch + 4 (l / 32) + 8 qq + t
#pragma unroll
        for (int j = 0; j < kCPG; ++j) {
            const int ch = cg * kCPG + j;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int col = 32 * ch + 4 * (lane >> 5) + 8 * qq;
                if (ch < NCH && col < nb)
                    *(f32x4 *)(us + (32 * rt + (lane & 31)) * uld + col) =
                        f32x4{acc[j][4 * qq], acc[j][4 * qq + 1], acc[j][4 * qq + 2], acc[j][4 * qq + 3]};
            }
        }
        __syncthreads();
        // W <- W - lr (s U + wd W) along the rows
#pragma unroll
        for (int i = 0; i < kWPT; ++i) {
            const int e = tid + kRT * i;
            const int r = e / q, c = 4 * (e - r * q);
            const int64_t row = tile * TR + r;
            if (e < TR * q && row < m) {
                const f32x4 u = *(const f32x4 *)(us + r * uld + c);
                const int64_t off = row * n + (int64_t)b * nb + c;
                float w0[4];
                if constexpr (WBF16) {
                    const uint2 hb = wcur[i];
                    w0[0] = bf16_to_f32((uint16_t)hb.x); w0[1] = bf16_to_f32((uint16_t)(hb.x >> 16));
                    w0[2] = bf16_to_f32((uint16_t)hb.y); w0[3] = bf16_to_f32((uint16_t)(hb.y >> 16));
                } else {
                    w0[0] = wcur[i][0]; w0[1] = wcur[i][1]; w0[2] = wcur[i][2]; w0[3] = wcur[i][3];
                }
                float nw[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) nw[cc] = w0[cc] - lr * __builtin_fmaf(sc, u[cc], wd * w0[cc]);
                if (U) *(f32x4 *)(U + off) = u;
                if constexpr (WBF16) {
                    *(uint2 *)((uint16_t *)Wv + off) =
                        uint2{(uint32_t)f32_to_bf16(nw[0]) | ((uint32_t)f32_to_bf16(nw[1]) << 16),
                              (uint32_t)f32_to_bf16(nw[2]) | ((uint32_t)f32_to_bf16(nw[3]) << 16)};
                } else {
                    *(f32x4 *)((float *)Wv + off) = f32x4{nw[0], nw[1], nw[2], nw[3]};
                }
            }
        }
    }
}

struct ColScaleTable {
    const double *part[kMaxMats];
    float *cs[kMaxMats];
};
__global__ void __launch_bounds__(256) k_colscale(int64_t n, int64_t ntile, ColScaleTable t) {
    const int mat = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    double s = 0.0;
    for (int64_t tl = 0; tl < ntile; ++tl) s += t.part[mat][tl * n + j];
    t.cs[mat][j] = s > 0.0 ? (float)(1.0 / sqrt(s)) : 0.f;
}

// Column-l2 projection: momentum, C = P Q (split fp16 products), C to the workspace with the tiles'
// column sums of squares, then the column scales.  128-row tiles, one tile group per block.
template <int NCH>
hipError_t launch_proj_l2_cfg(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    constexpr int TR = 128;
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const int64_t ntile = (m + TR - 1) / TR;
    const int64_t blocks = (int64_t)nblk * cnt;
    int64_t tpg = (ntile * blocks + 1023) / 1024;
    if (tpg < 4) tpg = 4;
    if (tpg > ntile) tpg = ntile;
    const int ngroups = (int)((ntile + tpg - 1) / tpg);
    const dim3 grid((unsigned)(ngroups * blocks));
    ProjRowsTable t{};
    for (int i = 0; i < cnt; ++i) {
        t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.Q[i] = a.Q[c0 + i];
        t.C[i] = a.C[c0 + i]; t.part[i] = a.colpart[c0 + i]; t.mu[i] = a.hp[c0 + i].momentum;
        t.Cout[i] = a.Cout ? a.Cout[c0 + i] : nullptr;
    }
    const size_t sh = proj_rows_lds(nb, TR);
    const bool gbf = a.g_dtype == DOBB_BF16;
    const bool nest = a.hp[c0].nesterov != 0;
#define DOBB_PL2(NE, GB)                                                                                         \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_proj_rows<NCH, TR, NE, GB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("project_l2_f16x3", s, (k_proj_rows<NCH, TR, NE, GB>), grid, dim3(kRT), sh, m, n, nb, nblk,   \
                    ngroups, (int)tpg, t);                                                                       \
    } while (0)
    if (!nest) { if (gbf) DOBB_PL2(0, true); else DOBB_PL2(0, false); }
    else { if (gbf) DOBB_PL2(1, true); else DOBB_PL2(1, false); }
#undef DOBB_PL2
    ColScaleTable ct{};
    for (int i = 0; i < cnt; ++i) { ct.part[i] = a.colpart[c0 + i]; ct.cs[i] = a.colscale[c0 + i]; }
    DOBB_LAUNCH("colscale", s, k_colscale, dim3((unsigned)((n + 255) / 256), (unsigned)cnt), dim3(256), 0, n, ntile, ct);
    return hipGetLastError();
}

// Column-l2 reconstruction (C and the column scales already in the workspace), 64-row tiles.
template <int NCH>
hipError_t launch_recon_l2_cfg(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    constexpr int TR = 64;
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const int64_t ntile = (m + TR - 1) / TR;
    const int64_t blocks = (int64_t)nblk * cnt;
    int64_t tpg = (ntile * blocks + 1023) / 1024;
    if (tpg < 4) tpg = 4;
    if (tpg > ntile) tpg = ntile;
    const int ngroups = (int)((ntile + tpg - 1) / tpg);
    const dim3 grid((unsigned)(ngroups * blocks));
    ReconRowsTable t{};
    for (int i = 0; i < cnt; ++i) {
        const dobb_hparams &h = a.hp[c0 + i];
        t.C[i] = a.C[c0 + i]; t.cs[i] = a.colscale[c0 + i]; t.Q[i] = a.Q[c0 + i]; t.W[i] = a.W[c0 + i];
        t.U[i] = a.U ? a.U[c0 + i] : nullptr;
        t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
    }
    const size_t sh = recon_rows_lds(nb, TR);
#define DOBB_RL2(WB)                                                                                             \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_recon_rows<NCH, TR, WB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("reconstruct_l2_f16x3", s, (k_recon_rows<NCH, TR, WB>), grid, dim3(kRT), sh, m, n, nb, nblk,  \
                    ngroups, (int)tpg, t);                                                                       \
    } while (0)
    if (a.w_dtype == DOBB_BF16) DOBB_RL2(true); else DOBB_RL2(false);
#undef DOBB_RL2
    return hipGetLastError();
}

}  // namespace

bool recon_l2_rows_eligible(const dobb_shape &sh) {
    return sh.nb <= 128 && sh.nb % 4 == 0 && sh.n % 4 == 0 &&
           (int64_t)recon_rows_lds((int)sh.nb, 64) <= max_lds_bytes();
}

bool proj_l2_rows_eligible(const dobb_shape &sh) {
    return recon_l2_rows_eligible(sh) &&
           (int64_t)proj_rows_lds((int)sh.nb, 128) <= max_lds_bytes();
}

hipError_t launch_proj_l2_rows(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    const int nct = (int)((a.sh.nb + 31) / 32);
    if (nct <= 1) return launch_proj_l2_cfg<1>(a, c0, cnt, s);
    if (nct <= 2) return launch_proj_l2_cfg<2>(a, c0, cnt, s);
    if (nct <= 3) return launch_proj_l2_cfg<3>(a, c0, cnt, s);
    return launch_proj_l2_cfg<4>(a, c0, cnt, s);
}

hipError_t launch_recon_l2_rows(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    const int nct = (int)((a.sh.nb + 31) / 32);
    if (nct <= 1) return launch_recon_l2_cfg<1>(a, c0, cnt, s);
    if (nct <= 2) return launch_recon_l2_cfg<2>(a, c0, cnt, s);
    if (nct <= 3) return launch_recon_l2_cfg<3>(a, c0, cnt, s);
    return launch_recon_l2_cfg<4>(a, c0, cnt, s);
}

}  // namespace dobb
