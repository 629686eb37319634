// The Dobb step (sign normalisation) for block widths 128 < nb <= 416: row tiles staged through LDS.
//
// Dobb paper (arXiv 2610.39412): abstract (project momentum into the block bases, sign-normalise,
// reconstruct), Table 9 (update scale), Table 21 caption (decoupled weight decay), Table 19
// (Nesterov).
//
// Same arithmetic as the narrow-block kernels: C = P Q with both operands split into two fp16 parts
// (three products), each row of P scaled by a power of two that keeps its largest magnitude in
// [2^13, 2^14); U = S Q^T with Q split into two fp16 parts (S is exact in fp16).  P streams through
// in column chunks, so a row's scale is the one its largest entry so far asks for: when a later chunk
// lowers it, the row's accumulators are rescaled by the (exact) power of two before its products.  A block's basis is too large to stay in LDS, so it is streamed one 16-deep k-slice at a
// time from planes that k_split_wide lays out slice by slice (each slice one contiguous copy, with
// the LDS swizzle already applied).  All row data moves along rows:
//   k_proj_wide   M, G rows (64-column chunks) -> M <- mu M + G (written back), P -> LDS (scaled per
//                 row, split into two fp16 planes once);
//                 waves take (32-row tile, every second 32-column chunk): C^T = Q^T P^T;
//                 sign bytes -> LDS -> rows
//   k_recon_wide  64-row tiles, two workgroups per CU: sign-byte rows -> LDS once; waves take
//                 (32-row tile, every fourth chunk): U = S Q^T; U -> LDS (32 rows at a time) -> rows,
//                 where W <- W - lr (s U + wd W) is applied
// Column-l2 normalisation (Dobb-l2, Tables 11-12) takes the same two kernels with L2 set: the
// projection writes C (unscaled by the row's power of two) to the workspace instead of sign bytes,
// k_colnorm (k_step.hip) turns C into the column scales 1 / ||C[:, j]||, and the reconstruction
// stages, with each basis slice, the 16 columns of C~ = C diag(colscale) the slice multiplies
// (|C~| <= 1: two fp16 parts without a scale, three products hi hi, hi lo(Q), lo hi).
// The workgroups of one block are adjacent in launch order, so they run together on one XCD and
// read the basis slices from its L2.
#include "step_common.h"

#include <type_traits>

namespace dobb {
namespace {
using namespace stepk;

constexpr int kWT = 512;        // threads per workgroup (8 waves)
constexpr int kTR = 128;        // rows per tile
constexpr int kKSD = 16;        // k per MFMA step
constexpr int kKC = 64;         // projection: columns of P per LDS chunk (4 k-steps)
constexpr int kPLD = kKC + 8;   // P plane pitch in bf16 (144 bytes: 16 rows on distinct 16-byte slots)
constexpr int kSPC = kKC / 16;  // k-steps per P chunk

struct WideGeo {
    int KS, nct, R;   // k-steps, 32-column chunks, staged rows (32 nct)
};
__host__ __device__ inline WideGeo wide_geo(int nb) {
    WideGeo g;
    g.KS = (nb + kKSD - 1) / kKSD;
    g.nct = (nb + 31) / 32;
    g.R = 32 * g.nct;
    return g;
}
// 2-byte elements of one plane of one block: KS slices of R rows x 16 k
__host__ __device__ inline int64_t wide_plane_elems(int nb) {
    const WideGeo g = wide_geo(nb);
    return (int64_t)g.KS * g.R * kKSD;
}
// physical 16-byte half of logical half h of row j of a slice (32 bytes per row): rows 4 apart
// alternate, so 8 or 16 consecutive rows read the same logical half from distinct banks
__host__ __device__ inline int qswz(int j) { return ((j >> 2) ^ (j >> 3)) & 1; }
__host__ __device__ inline size_t a16(size_t x) { return (x + 15) / 16 * 16; }
// the largest of v over the 16 lanes of a DPP row, in every lane of it: the partners within a quad
// (quad_perm [1,0,3,2], [2,3,0,1]), the other quad of the half-row (row_half_mirror) and the other
// half (row_mirror), register to register
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    return max(v, dpp_u32<0x140>(v));
}

// ---- basis planes --------------------------------------------------------------------------------
// planes (4 per matrix, each nblk x KS x R x 16 two-byte elements, slice-major):
//   0, 1  fp16 hi / lo of Q_b:    slice ks, row p, k: Q_b[p][16 ks + k]
//   2, 3  fp16 hi / lo of Q_b^T:  slice ks, row j, k: Q_b[16 ks + k][j]
// zero where a row or k index is >= nb.
struct SplitWideTable {
    const float *Q[kMaxMats];
    uint16_t *planes[kMaxMats];
};

// grid = (KS, blocks x matrices), block 256.  Workgroup ks reads rows 16 ks .. 16 ks + 15 of Q_b
// once (along rows, into LDS) and writes from them Q^T slice ks (all rows j) and, for every slice
// s, the 16 rows p = 16 ks .. of the Q slices; the last one also zeroes the Q slices' rows past
// 16 KS (padding up to R).
__global__ void __launch_bounds__(256) k_split_wide(int nb, int nblk, SplitWideTable t) {
    __shared__ float tile[kKSD * 513];   // [16][R + 1], R <= 512
    const WideGeo geo = wide_geo(nb);
    const int R = geo.R, KS = geo.KS;
    const int ks = blockIdx.x, g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    const float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    const int64_t PE = wide_plane_elems(nb), plane = (int64_t)nblk * PE;
    uint16_t *Pb = t.planes[mat] + (int64_t)b * PE;
    const int tid = threadIdx.x, k0 = kKSD * ks;
    if (((uintptr_t)Q & 15u) == 0) {   // nb % 4 == 0: rows start 16-byte aligned, 16-byte loads
        const int R4 = R / 4;
        for (int e = tid; e < kKSD * R4; e += 256) {
            const int kk = e / R4, j = 4 * (e - kk * R4);
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (k0 + kk < nb && j < nb) v = *(const f32x4 *)(Q + (int64_t)(k0 + kk) * nb + j);
#pragma unroll
            for (int c = 0; c < 4; ++c) tile[kk * (R + 1) + j + c] = v[c];
        }
    } else {
        for (int e = tid; e < kKSD * R; e += 256) {
            const int kk = e / R, j = e - kk * R;
            tile[kk * (R + 1) + j] = (k0 + kk < nb && j < nb) ? Q[(int64_t)(k0 + kk) * nb + j] : 0.f;
        }
    }
    __syncthreads();
    // Q^T slice ks: row j, k: Q[k0 + k][j]
    uint16_t *P = Pb + (int64_t)ks * R * kKSD;
    for (int e = tid; e < 2 * R; e += 256) {
        const int j = e >> 1, hs = e & 1, h = hs ^ qswz(j);
        uint16_t ph[8], pl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) split2h(tile[(8 * h + i) * (R + 1) + j], ph[i], pl[i]);
        const int64_t o = (int64_t)j * kKSD + 8 * hs;
        *(uint4 *)(P + 2 * plane + o) = uint4{pack2(ph[0], ph[1]), pack2(ph[2], ph[3]), pack2(ph[4], ph[5]), pack2(ph[6], ph[7])};
        *(uint4 *)(P + 3 * plane + o) = uint4{pack2(pl[0], pl[1]), pack2(pl[2], pl[3]), pack2(pl[4], pl[5]), pack2(pl[6], pl[7])};
    }
    // Q slices s, rows p = k0 + kk: Q[p][16 s + k] (the tile holds those rows; zero past nb)
    for (int e = tid; e < KS * kKSD * 2; e += 256) {
        const int sl = e / (2 * kKSD), rem = e - sl * 2 * kKSD;
        const int kk = rem >> 1, hs = rem & 1, p = k0 + kk, h = hs ^ qswz(p);
        uint16_t qh[8], ql[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) split2h(tile[kk * (R + 1) + kKSD * sl + 8 * h + i], qh[i], ql[i]);
        const int64_t o = ((int64_t)sl * R + p) * kKSD + 8 * hs;
        *(uint4 *)(Pb + o) = uint4{pack2(qh[0], qh[1]), pack2(qh[2], qh[3]), pack2(qh[4], qh[5]), pack2(qh[6], qh[7])};
        *(uint4 *)(Pb + plane + o) = uint4{pack2(ql[0], ql[1]), pack2(ql[2], ql[3]), pack2(ql[4], ql[5]), pack2(ql[6], ql[7])};
    }
    // padding rows [16 KS, R) of every Q slice
    if (ks == KS - 1) {
        const int pad = R - kKSD * KS;
        for (int e = tid; e < KS * pad * 2; e += 256) {
            const int sl = e / (2 * pad), rem = e - sl * 2 * pad;
            const int64_t o = ((int64_t)sl * R + kKSD * KS + (rem >> 1)) * kKSD + 8 * (rem & 1);
            *(uint4 *)(Pb + o) = uint4{0u, 0u, 0u, 0u};
            *(uint4 *)(Pb + plane + o) = uint4{0u, 0u, 0u, 0u};
        }
    }
}

// ---- projection ----------------------------------------------------------------------------------
struct ProjWideTable {
    float *M[kMaxMats];
    const void *G[kMaxMats];
    const uint16_t *planes[kMaxMats];
    uint8_t *S[kMaxMats];
    float *Cout[kMaxMats];     // NULL or m x n fp32: the coefficients (verification output)
    float *C[kMaxMats];        // column-l2: the coefficients (m x n fp32 workspace)
    float mu[kMaxMats];
};
// LDS: two Q^T slices (2 planes each; the sign tile overlays them after the products), the P chunk
// split into two fp16 planes, and the tile's per-row scale exponents
__host__ __device__ inline size_t proj_wide_qregion(int nb, int ldp) {
    const WideGeo g = wide_geo(nb);
    const size_t q = (size_t)2 * 2 * g.R * kKSD * 2, s = (size_t)kTR * ldp;
    return a16(q > s ? q : s);
}
__host__ __device__ inline size_t proj_wide_lds(int nb, int ldp) {
    return proj_wide_qregion(nb, ldp) + (size_t)2 * kTR * kPLD * 2 + (size_t)kTR * 4;
}

// grid.x = tile groups (fastest) x blocks x matrices, renumbered per XCD; block 512.
// NCT = ceil(nb / 32).  Wave w: 32-row tile rt = w % 4, column chunks cg + 2 j (cg = w / 4).
// CO: also write the coefficients to t.Cout (a verification output; off in the timed path).
// L2: column-l2 normalisation: C to t.C instead of the sign bytes.
template <int NCT, int NEST, bool GBF16, bool CO = false, bool L2 = false>
__global__ void __launch_bounds__(512) k_proj_wide(int64_t m, int64_t n, int nb, int nblk, int ngroups, int tpg,
                                                   int ldp, ProjWideTable t) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int NCW = (NCT + 1) / 2, R = 32 * NCT, nct = NCT;
    const int KS = (nb + kKSD - 1) / kKSD;
    uint16_t *qs = (uint16_t *)lds;                                   // [2][2][R][16]
    uint8_t *ss = lds;                                                // [kTR][ldp], after the products
    uint16_t *ps = (uint16_t *)(lds + proj_wide_qregion(nb, ldp));    // [2][kTR][kPLD]
    int *rs = (int *)(ps + 2 * kTR * kPLD);                           // [kTR] row scale exponents

    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int tg = x % ngroups, rest = x / ngroups;
    const int b = rest % nblk, mat = rest / nblk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = w & 3, cg = w >> 2;
    const int64_t ntile = (m + kTR - 1) / kTR;
    const int64_t t_begin = (int64_t)tg * tpg;
    const int64_t t_end = t_begin + tpg < ntile ? t_begin + tpg : ntile;

    constexpr int kGS = GBF16 ? 2 : 4;
    const int64_t mn_el = m * n - (int64_t)b * nb;
    const __amdgpu_buffer_rsrc_t rM = make_rsrc(t.M[mat] + (int64_t)b * nb, mn_el * 4);
    const __amdgpu_buffer_rsrc_t rG = make_rsrc((const char *)t.G[mat] + (int64_t)b * nb * kGS, mn_el * kGS);
    const int64_t sld = (int64_t)nblk * ldp;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(t.S[mat] + (int64_t)b * ldp, m * sld - (int64_t)b * ldp);
    const int64_t PE = wide_plane_elems(nb), plane = (int64_t)nblk * PE;
    const uint16_t *QT = t.planes[mat] + 2 * plane + (int64_t)b * PE;
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(QT, (plane + PE) * 2);
    const float mu = t.mu[mat];

    // M / G chunk pieces: kTR rows x 20 four-column pieces, 5 per thread
    constexpr int kMP = kTR * (kKC / 4) / kWT;
    f32x4 mr[kMP], gr[kMP];
    auto mg_off = [&](int i, int64_t tile, int kc0) -> unsigned {
        const int e = tid + kWT * i;
        const int r = e / (kKC / 4), c = kc0 + 4 * (e - r * (kKC / 4));
        const int64_t row = tile * kTR + r;
        return (tile < t_end && row < m && c < nb) ? (unsigned)row * (unsigned)n + (unsigned)c : kOff;
    };
    auto load_mg = [&](int64_t tile, int kc0) {
#pragma unroll
        for (int i = 0; i < kMP; ++i) {
            const unsigned o = mg_off(i, tile, kc0);
            mr[i] = bload4(rM, boff(o, 4));
            if constexpr (GBF16) {
                const uint2 hb = bload2u(rG, boff(o, 2));
                gr[i] = f32x4{bf16_to_f32((uint16_t)hb.x), bf16_to_f32((uint16_t)(hb.x >> 16)),
                              bf16_to_f32((uint16_t)hb.y), bf16_to_f32((uint16_t)(hb.y >> 16))};
            } else {
                gr[i] = bload4(rG, boff(o, 4));
            }
        }
    };
    // momentum written back along the rows; P scaled by its row's power of two and split once into
    // two fp16 planes of the LDS chunk (zeros past m and nb).  The 16 lanes of a row are consecutive,
    // so the chunk's row maximum is a 16-lane reduction; the row's exponent is the smaller of the
    // chunk's and the one in rs (the first chunk of a tile starts afresh).
    auto stage_p = [&](int64_t tile, int kc0, bool first) {
#pragma unroll
        for (int i = 0; i < kMP; ++i) {
            const int e = tid + kWT * i;
            const int r = e / (kKC / 4), c = 4 * (e - r * (kKC / 4));
            f32x4 mn, pv;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                mn[cc] = __builtin_fmaf(mu, mr[i][cc], gr[i][cc]);
                pv[cc] = NEST ? __builtin_fmaf(mu, mn[cc], gr[i][cc]) : mn[cc];
            }
            bstore4(mn, rM, boff(mg_off(i, tile, kc0), 4));
            uint32_t mx = __float_as_uint(pv[0]) & 0x7fffffffu;
#pragma unroll
            for (int cc = 1; cc < 4; ++cc) {
                const uint32_t u = __float_as_uint(pv[cc]) & 0x7fffffffu;
                mx = u > mx ? u : mx;
            }
            mx = row16_max(mx);
            int se = row_scale_exp(mx);
            if (!first) {
                const int so = rs[r];
                se = so < se ? so : se;
            }
            if ((tid & 15) == 0) rs[r] = se;
            uint16_t h[4], l[4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) split2s(__builtin_amdgcn_ldexpf(pv[cc], se), h[cc], l[cc]);
            uint16_t *pp = ps + r * kPLD + c;
            *(uint2 *)pp = uint2{pack2(h[0], h[1]), pack2(h[2], h[3])};
            *(uint2 *)(pp + kTR * kPLD) = uint2{pack2(l[0], l[1]), pack2(l[2], l[3])};
        }
    };
    // Q^T slice pieces: 2 planes x R rows x 2 halves of 16 bytes
    constexpr int kQP = (4 * R + kWT - 1) / kWT;
    uint4 qr[kQP];
    auto load_q = [&](int ks) {
#pragma unroll
        for (int i = 0; i < kQP; ++i) {
            const int e = tid + kWT * i;
            const int pl = e / (2 * R), rem = e - pl * 2 * R;
            const unsigned o = e < 4 * R ? (unsigned)(pl * plane + (int64_t)ks * R * kKSD + 8 * rem) : kOff;
            qr[i] = bload4u(rQ, boff(o, 2));
        }
    };
    auto store_q = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kQP; ++i) {
            const int e = tid + kWT * i;
            if (e < 4 * R) *(uint4 *)(qs + (size_t)buf * 2 * R * kKSD + 8 * e) = qr[i];
        }
    };

    const int kh = 8 * (lane >> 5);
    // this lane's Q^T slice offset for chunk cg; chunk cg + 2 j is 64 j rows further (qswz depends on
    // row bits 2 and 3 only, so the swizzle is the same)
    const int qrow = 32 * cg + (lane & 31);
    const int qoff = qrow * kKSD + 8 * ((lane >> 5) ^ qswz(qrow));
    const int nchunk = (KS + kSPC - 1) / kSPC;
    int par = 0;
    load_mg(t_begin, 0);
    load_q(0);
    const int prow = 32 * rt + (lane & 31);   // the P row (tile row) of this lane's accumulators
    for (int64_t tile = t_begin; tile < t_end; ++tile) {
        f32x16 acc[NCW];
#pragma unroll
        for (int j = 0; j < NCW; ++j) acc[j] = (f32x16){};
        int sreg = 0;   // the scale exponent acc holds its row at
        for (int c = 0; c < nchunk; ++c) {
            const int kc0 = c * kKC;
            __syncthreads();   // the last chunk's products are done with ps, the sign drain with qs
            stage_p(tile, kc0, c == 0);
            if (c + 1 < nchunk) load_mg(tile, kc0 + kKC);
            else load_mg(tile + 1, 0);
            const int s_end = KS - kSPC * c < kSPC ? KS - kSPC * c : kSPC;
            for (int s = 0; s < s_end; ++s) {
                const int ks = kSPC * c + s;
                store_q(par);
                load_q(ks + 1 < KS ? ks + 1 : 0);   // the next tile starts over at slice 0
                __syncthreads();
                if (s == 0) {
                    // this chunk's scale of the lane's row: rescale what acc holds when it dropped
                    const int se = rs[prow];
                    const int d = c == 0 ? 0 : se - sreg;
                    if (__any(d != 0)) {
#pragma unroll
                        for (int j = 0; j < NCW; ++j)
#pragma unroll
                            for (int i = 0; i < 16; ++i) acc[j][i] = __builtin_amdgcn_ldexpf(acc[j][i], d);
                    }
                    sreg = se;
                }
                const uint16_t *pr = ps + prow * kPLD + kKSD * s + kh;
                const f16x8 ah = *(const f16x8 *)pr;
                const f16x8 al = *(const f16x8 *)(pr + kTR * kPLD);
                const uint16_t *qb = qs + (size_t)par * 2 * R * kKSD + qoff;
                // chunks two at a time, their products interleaved so that consecutive MFMAs are
                // independent
#pragma unroll
                for (int j = 0; j < NCW; j += 2) {
                    const bool two = j + 1 < NCW && cg + 2 * (j + 1) < nct;
                    if (cg + 2 * j < nct) {
                        const uint16_t *q0 = qb + 2 * j * 32 * kKSD;
                        const uint16_t *q1 = q0 + 2 * 32 * kKSD;
                        const f16x8 Qh0 = *(const f16x8 *)q0, Ql0 = *(const f16x8 *)(q0 + R * kKSD);
                        if (two) {
                            const f16x8 Qh1 = *(const f16x8 *)q1, Ql1 = *(const f16x8 *)(q1 + R * kKSD);
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, ah, acc[j], 0, 0, 0);
                            acc[j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh1, ah, acc[j + 1], 0, 0, 0);
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ql0, ah, acc[j], 0, 0, 0);
                            acc[j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ql1, ah, acc[j + 1], 0, 0, 0);
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, al, acc[j], 0, 0, 0);
                            acc[j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh1, al, acc[j + 1], 0, 0, 0);
                        } else {
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, ah, acc[j], 0, 0, 0);
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ql0, ah, acc[j], 0, 0, 0);
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, al, acc[j], 0, 0, 0);
                        }
                    }
                }
                par ^= 1;
            }
        }
        const int64_t crow = tile * kTR + prow;
        if constexpr (L2) {
            // C, unscaled, along the lane's row: columns 32 ch + 8 qq + 4 (l / 32) + 0..3
            float *const Cw = t.C[mat] + (int64_t)b * nb;
            float *const Co = t.Cout[mat] ? t.Cout[mat] + (int64_t)b * nb : nullptr;
#pragma unroll
            for (int j = 0; j < NCW; ++j) {
                const int ch = cg + 2 * j;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int col = 32 * ch + 8 * qq + 4 * (lane >> 5);
                    if (ch < nct && col < nb && crow < m) {
                        const f32x4 cv = {__builtin_amdgcn_ldexpf(acc[j][4 * qq], -sreg),
                                          __builtin_amdgcn_ldexpf(acc[j][4 * qq + 1], -sreg),
                                          __builtin_amdgcn_ldexpf(acc[j][4 * qq + 2], -sreg),
                                          __builtin_amdgcn_ldexpf(acc[j][4 * qq + 3], -sreg)};
                        *(f32x4 *)(Cw + crow * n + col) = cv;
                        if (Co) *(f32x4 *)(Co + crow * n + col) = cv;
                    }
                }
            }
            continue;
        }
        // sign bytes: lane holds row 32 rt + l % 32, columns 32 ch + 8 qq + 4 (l / 32) + 0..3 -> LDS
        __syncthreads();   // every wave is done with the Q slices that the sign tile overlays
        float *const Co = CO ? t.Cout[mat] : nullptr;
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            const int ch = cg + 2 * j;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int col = 32 * ch + 8 * qq + 4 * (lane >> 5);   // nb % 4 == 0: all 4 valid or none
                const uint32_t w4 = sign_byte(acc[j][4 * qq]) | (sign_byte(acc[j][4 * qq + 1]) << 8) |
                                    (sign_byte(acc[j][4 * qq + 2]) << 16) | (sign_byte(acc[j][4 * qq + 3]) << 24);
                if (ch < nct && col < nb) *(uint32_t *)(ss + (32 * rt + (lane & 31)) * ldp + col) = w4;
                if (CO && Co && ch < nct && col < nb && crow < m)
                    *(f32x4 *)(Co + crow * n + (int64_t)b * nb + col) =
                        f32x4{__builtin_amdgcn_ldexpf(acc[j][4 * qq], -sreg), __builtin_amdgcn_ldexpf(acc[j][4 * qq + 1], -sreg),
                              __builtin_amdgcn_ldexpf(acc[j][4 * qq + 2], -sreg), __builtin_amdgcn_ldexpf(acc[j][4 * qq + 3], -sreg)};
            }
        }
        __syncthreads();
        // sign rows out in 8-byte pieces (bytes [nb, ldp) of a row are padding, never read as signs)
        const int q8 = ldp / 8;
        for (int e = tid; e < kTR * q8; e += kWT) {
            const int r = e / q8, c = 8 * (e - r * q8);
            const int64_t row = tile * kTR + r;
            bstore2u(*(const uint2 *)(ss + r * ldp + c), rS, row < m ? (unsigned)(row * sld + c) : kOff);
        }
    }
}

// ---- reconstruction ------------------------------------------------------------------------------
struct ReconWideTable {
    const uint8_t *S[kMaxMats];
    const float *C[kMaxMats];    // column-l2: the coefficients (m x n fp32) and the column scales
    const float *cs[kMaxMats];
    const uint16_t *planes[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};
// sign tile pitch: the k extent 16 KS rounded up to an odd number of 8-byte units (rows on distinct
// banks).  The tile holds every k the products read, zero past nb (zero times the basis' zero
// padding: a stale byte there could decode to an infinite fp16 value and give NaN).
__host__ __device__ inline int wide_spitch(int nb) { return kKSD * ((nb + kKSD - 1) / kKSD) + 8; }
// U staging pitch in floats: R + 8 (R = 32 ceil(nb / 32)), 8 mod 16, so that the two rows written by
// the half-waves of one accumulator register fall in opposite bank halves
__host__ __device__ inline int wide_uld(int nb) { return wide_geo(nb).R + 8; }
constexpr int kRTR = 64;   // reconstruction: rows per workgroup
constexpr int kCSP = kKSD + 8;   // column-l2: C~ slice plane pitch in 2-byte elements (3 16-byte units)
// LDS: region 0 holds two Q slices (2 planes each) during the products, then 32 rows of U at a time;
// region 1 the tile's sign rows, or (column-l2) two C~ slices of kRTR rows x 16 columns, each split
// into two fp16 planes.  At most
// 81408 bytes (nb <= 416): two workgroups fit on a CU.
__host__ __device__ inline size_t recon_wide_qregion(int nb) {
    const size_t q = (size_t)2 * 2 * wide_geo(nb).R * kKSD * 2, u = (size_t)32 * wide_uld(nb) * 4;
    return a16(q > u ? q : u);
}
__host__ __device__ inline size_t recon_wide_lds(int nb, int ldp, bool l2 = false) {
    (void)ldp;
    return recon_wide_qregion(nb) + (l2 ? a16((size_t)2 * 2 * kRTR * kCSP * 2) : a16((size_t)kRTR * wide_spitch(nb)));
}

// grid.x = tiles of kRTR rows (fastest) x blocks x matrices, renumbered per XCD; block 512, two
// workgroups per CU (four waves per SIMD), so that one's products overlap the other's row traffic.
// NCT = ceil(nb / 32).  Wave w: 32-row tile rt = w / 4, column chunks cg + 4 j (cg = w % 4).
// L2: column-l2 normalisation (C~ slices instead of the sign tile, three products).
template <int NCT, bool WBF16, bool L2 = false>
__global__ void __launch_bounds__(512, 4) k_recon_wide(int64_t m, int64_t n, int nb, int nblk, int ntile, int ldp,
                                                       ReconWideTable t) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int NCW = (NCT + 3) / 4, R = 32 * NCT, nct = NCT;
    constexpr int uld = R + 8;   // wide_uld
    const int KS = (nb + kKSD - 1) / kKSD;
    const int spitch = wide_spitch(nb);
    uint16_t *qs = (uint16_t *)lds;                        // [2][2][R][16], then U rows [32][uld] fp32
    float *us = (float *)lds;
    uint8_t *ss = lds + recon_wide_qregion(nb);             // [kRTR][spitch]
    uint16_t *cbuf = (uint16_t *)(lds + recon_wide_qregion(nb));   // L2: [2 slices][2 planes][kRTR][kCSP]

    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = x % ntile, rest = x / ntile;
    const int b = rest % nblk, mat = rest / nblk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = w >> 2, cg = w & 3;
    const int64_t row0 = (int64_t)tile * kRTR;

    constexpr int kWS = WBF16 ? 2 : 4;
    const int64_t mn_el = m * n - (int64_t)b * nb;
    const __amdgpu_buffer_rsrc_t rW = make_rsrc((const char *)t.W[mat] + (int64_t)b * nb * kWS, mn_el * kWS);
    float *const U = t.U[mat];
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(U ? (const void *)(U + (int64_t)b * nb) : t.W[mat], U ? mn_el * 4 : 0);
    const int64_t sld = (int64_t)nblk * ldp;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(L2 ? (const void *)t.W[mat] : (const void *)(t.S[mat] + (int64_t)b * ldp),
                                                L2 ? 0 : m * sld - (int64_t)b * ldp);
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(L2 ? (const void *)(t.C[mat] + (int64_t)b * nb) : (const void *)t.W[mat],
                                                L2 ? mn_el * 4 : 0);
    const int64_t PE = wide_plane_elems(nb), plane = (int64_t)nblk * PE;
    const uint16_t *QN = t.planes[mat] + (int64_t)b * PE;
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(QN, (plane + PE) * 2);
    const float lr = t.lr[mat], wd = t.wd[mat], sc = t.scale[mat];

    // e / d for 0 <= e < 2^16, 0 < d < 2^10: the float quotient is within one of the exact one
    auto divu = [](int e, int d, float inv) -> int {
        int r = (int)((float)e * inv);
        r -= r * d > e;
        r += (r + 1) * d <= e;
        return r;
    };
    // Q slice pieces: 2 planes x R rows x 2 halves
    constexpr int kQP = (4 * R + kWT - 1) / kWT;
    uint4 qr[kQP];
    auto load_q = [&](int ks) {
#pragma unroll
        for (int i = 0; i < kQP; ++i) {
            const int e = tid + kWT * i;
            const int pl = e / (2 * R), rem = e - pl * 2 * R;
            const unsigned o = e < 4 * R ? (unsigned)(pl * plane + (int64_t)ks * R * kKSD + 8 * rem) : kOff;
            qr[i] = bload4u(rQ, boff(o, 2));
        }
    };
    auto store_q = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kQP; ++i) {
            const int e = tid + kWT * i;
            if (e < 4 * R) *(uint4 *)(qs + (size_t)buf * 2 * R * kKSD + 8 * e) = qr[i];
        }
    };

    // column-l2: piece e < 4 kRTR of a C~ slice: row e / 4, columns 4 (e % 4) .. + 3 of the slice,
    // C times its column scales (zero past m and nb)
    f32x4 cpc = {0.f, 0.f, 0.f, 0.f};
    auto load_c = [&](int ks) {
        if constexpr (L2) {
            const int e = tid, r = e >> 2, c = kKSD * ks + 4 * (e & 3);
            const int64_t row = row0 + r;
            const bool ok = e < 4 * kRTR && row < m && c < nb;
            cpc = bload4(rC, boff(ok ? (unsigned)(row * n + c) : kOff, 4));
            if (ok) {
                const f32x4 sv = *(const f32x4 *)(t.cs[mat] + (int64_t)b * nb + c);
                cpc = f32x4{cpc[0] * sv[0], cpc[1] * sv[1], cpc[2] * sv[2], cpc[3] * sv[3]};
            }
        }
    };
    // split once at staging (|C~| <= 1: two fp16 parts, no scale)
    auto store_c = [&](int buf) {
        if constexpr (L2) {
            if (tid < 4 * kRTR) {
                uint16_t h[4], l[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) split2h(cpc[cc], h[cc], l[cc]);
                uint16_t *d = cbuf + ((size_t)2 * buf * kRTR + (tid >> 2)) * kCSP + 4 * (tid & 3);
                *(uint2 *)d = uint2{pack2(h[0], h[1]), pack2(h[2], h[3])};
                *(uint2 *)(d + kRTR * kCSP) = uint2{pack2(l[0], l[1]), pack2(l[2], l[3])};
            }
        }
    };

    load_q(0);
    load_c(0);
    // sign rows of the tile -> LDS in 8-byte pieces, k = 0 .. 16 KS - 1 (zero at and past nb)
    if constexpr (!L2) {
        constexpr int kSP = (kRTR * (R / 8) + kWT - 1) / kWT;
        const int q8 = 2 * KS;
        const float inv_q8 = 1.0f / (float)q8;
        uint2 sv[kSP];
#pragma unroll
        for (int i = 0; i < kSP; ++i) {
            const int e = tid + kWT * i;
            const int r = divu(e, q8, inv_q8), c = 8 * (e - r * q8);
            const int64_t row = row0 + r;
            // c < nb <= ldp and both multiples of 8 (ldp) or 4 (nb): the piece lies inside the row
            sv[i] = bload2u(rS, (e < kRTR * q8 && row < m && c < nb) ? (unsigned)(row * sld + c) : kOff);
            if (c + 4 >= nb) sv[i].y = 0u;
        }
#pragma unroll
        for (int i = 0; i < kSP; ++i) {
            const int e = tid + kWT * i;
            const int r = divu(e, q8, inv_q8), c = 8 * (e - r * q8);
            if (e < kRTR * q8) *(uint2 *)(ss + r * spitch + c) = sv[i];
        }
    }

    // U = S Q^T for 32-row tile rt and this wave's column chunks
    const int kh = 8 * (lane >> 5);
    f32x16 acc[NCW];
#pragma unroll
    for (int j = 0; j < NCW; ++j) acc[j] = (f32x16){};
    int par = 0;
    for (int ks = 0; ks < KS; ++ks) {
        store_q(par);
        store_c(par);
        if (ks + 1 < KS) {
            load_q(ks + 1);
            load_c(ks + 1);
        }
        __syncthreads();
        f16x8 as, al;
        if constexpr (L2) {
            const uint16_t *cp = cbuf + ((size_t)2 * par * kRTR + 32 * rt + (lane & 31)) * kCSP + kh;
            as = __builtin_bit_cast(f16x8, *(const uint4 *)cp);
            al = __builtin_bit_cast(f16x8, *(const uint4 *)(cp + kRTR * kCSP));
        } else {
            as = signs_f16x8(*(const uint2 *)(ss + (32 * rt + (lane & 31)) * spitch + kKSD * ks + kh));
            al = as;
        }
        const uint16_t *qb = qs + (size_t)par * 2 * R * kKSD;
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            const int ch = cg + 4 * j;
            if (ch < nct) {
                const int p = 32 * ch + (lane & 31);
                const int o = p * kKSD + 8 * ((lane >> 5) ^ qswz(p));
                const f16x8 Bh = *(const f16x8 *)(qb + o);
                const f16x8 Bl = *(const f16x8 *)(qb + R * kKSD + o);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as, Bh, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as, Bl, acc[j], 0, 0, 0);
                if constexpr (L2) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, Bh, acc[j], 0, 0, 0);
            }
            // one chunk's operands at a time (the other waves of the SIMD cover the LDS latency)
            __builtin_amdgcn_sched_barrier(0);
        }
        par ^= 1;
    }

    // W <- W - lr (s U + wd W), one 32-row tile at a time: its waves write U to the LDS (lane: column
    // 32 ch + l % 32 of rows 8 (r / 4) + 4 (l / 32) + r % 4), then every thread updates 16-byte
    // pieces along the rows.  The W pieces of a half are loaded before its U is staged, and each
    // register is refilled with the second half's piece as soon as it is used.
    const int nq = nb >> 2;
    const float inv_nq = 1.0f / (float)nq;
    constexpr int kUP = (32 * (R / 4) + kWT - 1) / kWT;   // pieces per thread and half
    using WVec = typename std::conditional<WBF16, uint2, f32x4>::type;
    auto piece_off = [&](int h, int k) -> unsigned {       // element offset of piece k of half h
        const int e = tid + kWT * k;
        const int r = divu(e, nq, inv_nq), c = 4 * (e - r * nq);
        const int64_t row = row0 + 32 * h + r;
        return (e < 32 * nq && row < m) ? (unsigned)row * (unsigned)n + (unsigned)c : kOff;
    };
    auto load_piece_w = [&](int h, int k) -> WVec {
        const unsigned o = piece_off(h, k);
        if constexpr (WBF16) return bload2u(rW, boff(o, 2));
        else return bload4(rW, boff(o, 4));
    };
    auto write_u = [&]() {
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            const int ch = cg + 4 * j;
            const int col = 32 * ch + (lane & 31);
            if (ch < nct && col < nb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) us[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * uld + col] = acc[j][r];
            }
        }
    };
    WVec wv[kUP];
    auto update = [&](int h) {
#pragma unroll
        for (int k = 0; k < kUP; ++k) {
            const int e = tid + kWT * k;
            const int r = divu(e, nq, inv_nq), c = 4 * (e - r * nq);
            const unsigned o = piece_off(h, k);
            if (e < 32 * nq) {
                const f32x4 u = *(const f32x4 *)(us + r * uld + c);
                float w0[4];
                if constexpr (WBF16) {
                    const uint2 hb = wv[k];
                    w0[0] = bf16_to_f32((uint16_t)hb.x); w0[1] = bf16_to_f32((uint16_t)(hb.x >> 16));
                    w0[2] = bf16_to_f32((uint16_t)hb.y); w0[3] = bf16_to_f32((uint16_t)(hb.y >> 16));
                } else {
                    w0[0] = wv[k][0]; w0[1] = wv[k][1]; w0[2] = wv[k][2]; w0[3] = wv[k][3];
                }
                float nw[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) nw[cc] = w0[cc] - lr * __builtin_fmaf(sc, u[cc], wd * w0[cc]);
                if (U) bstore4(u, rU, boff(o, 4));
                if constexpr (WBF16)
                    bstore2u(uint2{(uint32_t)f32_to_bf16(nw[0]) | ((uint32_t)f32_to_bf16(nw[1]) << 16),
                                   (uint32_t)f32_to_bf16(nw[2]) | ((uint32_t)f32_to_bf16(nw[3]) << 16)},
                             rW, boff(o, 2));
                else bstore4(f32x4{nw[0], nw[1], nw[2], nw[3]}, rW, boff(o, 4));
            }
            if (h == 0) wv[k] = load_piece_w(1, k);
            __builtin_amdgcn_sched_barrier(0);   // one piece at a time (register pressure)
        }
    };
#pragma unroll
    for (int k = 0; k < kUP; ++k) wv[k] = load_piece_w(0, k);
    __syncthreads();   // every wave is done with the Q slices
    if (rt == 0) write_u();
    __syncthreads();
    update(0);
    __syncthreads();   // every thread is done reading the first half
    if (rt == 1) write_u();
    __syncthreads();
    update(1);
}

// ---- the whole step in one pass --------------------------------------------------------------------
// k_step_wide_fused: one 128-row tile of one block per workgroup.  Momentum and the projection run as
// in k_proj_wide (P chunks staged in LDS, Q^T slices streamed); the signs go to an LDS tile that stays
// for the reconstruction, which runs U = S Q^T over the same 128 rows with the Q slices streamed in
// turn (wave w: 32-row tile w % 4, every second 32-column chunk from w / 4, the projection's split);
// W is updated straight from the accumulators.  The sign bytes never reach HBM, and each
// basis slice serves 128 rows in both products.  Templated on the chunks per wave (NCW = ceil(nct / 2),
// nct = ceil(nb / 32) at run time) to keep the instances few.
struct FusedWideTable {
    float *M[kMaxMats];
    const void *G[kMaxMats];
    const uint16_t *planes[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float mu[kMaxMats], lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};
// LDS, static per instance (nb <= RM): a ring of four basis-slice stages (2 planes each), one region
// that holds the P chunk planes during the projection and the sign tile (rows of wide_spitch bytes)
// after it, and the tile's row scale exponents.  At RM = 416: 4 x 26624 + 54272 + 512 = 161280 bytes.
template <int NCW>
struct RingGeo {
    static constexpr int RM = 64 * NCW < 416 ? 64 * NCW : 416;   // staged rows at most
    static constexpr int KSM = (RM + kKSD - 1) / kKSD;           // k-steps at most
    static constexpr int kStage = 2 * RM * kKSD;                 // 2-byte elements of one stage
    static constexpr int kP = 2 * kTR * kPLD * 2, kS = kTR * (kKSD * KSM + 8);
    static constexpr int kPS = kP > kS ? kP : kS;                // bytes of the P / sign region
    static constexpr int kND = (2 * (RM / 32) + 7) / 8;          // slice loads per wave and stage
};
// s_waitcnt vmcnt(N) (this wave's memory operations older than the last N are done), then lgkmcnt(0)
// and the workgroup barrier, in one asm block so that no memory operation moves across it
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
typedef __attribute__((address_space(3))) void *lds_void;
// one 16-byte piece per lane from buffer offset off into LDS at dst + 16 lane (zeros past the range);
// a function of its own: the builtin written inside the kernel's lambdas kept the host pass from
// emitting the kernel's launch stub
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void *dst, unsigned off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void)dst, 16, off, 0, 0, 0);
}

// grid.x = 128-row tiles (fastest) x blocks x matrices, renumbered per XCD; block 512.
// The basis slices reach LDS by loads that write it directly: the projection's KS slices of Q^T and
// the reconstruction's KS slices of Q form one sequence of slots, each phase padded to 4 nchunk slots
// (empty ones load zeros and skip the products), slot t in stage t % 4; the loads of slot t + 3 are
// issued once every wave has passed the barrier of slot t (so stage (t + 3) % 4 = (t - 1) % 4 is free),
// three slices in flight.  Each wave issues kND 1 KiB loads per slot (piece w + 8 i of the stage's
// 2 nct pieces, piece w again past the count), and a chunk start adds 12 buffer operations (the
// momentum stores and the next chunk's M and G loads, issued for every chunk so that the count is
// fixed): before the barrier of slot t a wave waits until its operations older than the last
// 2 kND (+ 12 where a chunk start lies between) are done, which covers its loads of slot t.
template <int NCW, int NEST, bool GBF16, bool WBF16>
__global__ void __launch_bounds__(512) k_step_wide_fused(int64_t m, int64_t n, int nb, int nblk, int ntile,
                                                         FusedWideTable t) {
    using L = RingGeo<NCW>;
    __shared__ __align__(16) uint16_t qst0[L::kStage], qst1[L::kStage], qst2[L::kStage], qst3[L::kStage];
    __shared__ __align__(16) uint8_t pss[L::kPS];
    __shared__ int rs[kTR];   // row scale exponents
    uint16_t *const qst[4] = {qst0, qst1, qst2, qst3};
    const WideGeo geo = wide_geo(nb);
    const int nct = geo.nct, R = geo.R, KS = geo.KS;
    const int spitch = wide_spitch(nb);
    uint16_t *const ps = (uint16_t *)pss;   // [2][kTR][kPLD] during the projection
    uint8_t *const ss = pss;                // [kTR][spitch] sign bytes after it

    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = x % ntile, rest = x / ntile;
    const int b = rest % nblk, mat = rest / nblk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = w & 3, cg = w >> 2;
    const int64_t row0 = (int64_t)tile * kTR;

    constexpr int kGS = GBF16 ? 2 : 4, kWS = WBF16 ? 2 : 4;
    const int64_t mn_el = m * n - (int64_t)b * nb;
    const __amdgpu_buffer_rsrc_t rM = make_rsrc(t.M[mat] + (int64_t)b * nb, mn_el * 4);
    const __amdgpu_buffer_rsrc_t rG = make_rsrc((const char *)t.G[mat] + (int64_t)b * nb * kGS, mn_el * kGS);
    float *const U = t.U[mat];
    const int64_t PE = wide_plane_elems(nb), plane = (int64_t)nblk * PE;
    const __amdgpu_buffer_rsrc_t rQN = make_rsrc(t.planes[mat] + (int64_t)b * PE, (plane + PE) * 2);              // Q
    const __amdgpu_buffer_rsrc_t rQT = make_rsrc(t.planes[mat] + 2 * plane + (int64_t)b * PE, (plane + PE) * 2);  // Q^T
    const float mu = t.mu[mat], lr = t.lr[mat], wd = t.wd[mat], sc = t.scale[mat];

    // ---- momentum and P: M / G chunk pieces, kTR rows x 16 four-column pieces, 4 per thread ----
    constexpr int kMP = kTR * (kKC / 4) / kWT;
    static_assert(kMP == 4, "a chunk start issues 3 kMP = 12 buffer operations");
    f32x4 mr[kMP], gr[kMP];
    auto mg_off = [&](int i, int kc0) -> unsigned {
        const int e = tid + kWT * i;
        const int r = e / (kKC / 4), c = kc0 + 4 * (e - r * (kKC / 4));
        const int64_t row = row0 + r;
        return (row < m && c < nb) ? (unsigned)row * (unsigned)n + (unsigned)c : kOff;
    };
    auto load_mg = [&](int kc0) {
#pragma unroll
        for (int i = 0; i < kMP; ++i) {
            const unsigned o = mg_off(i, kc0);
            mr[i] = bload4(rM, boff(o, 4));
            if constexpr (GBF16) {
                const uint2 hb = bload2u(rG, boff(o, 2));
                gr[i] = f32x4{bf16_to_f32((uint16_t)hb.x), bf16_to_f32((uint16_t)(hb.x >> 16)),
                              bf16_to_f32((uint16_t)hb.y), bf16_to_f32((uint16_t)(hb.y >> 16))};
            } else {
                gr[i] = bload4(rG, boff(o, 4));
            }
        }
    };
    // momentum written back along the rows; P scaled by its row's power of two and split once into two
    // fp16 planes of the LDS chunk (as in k_proj_wide)
    // (the kMP pieces are rows 32 i + tid / 16, one 16-lane group each: their row maxima, the reads of
    // the rows' previous exponents and the writes go as independent batches, not one chain per piece)
    auto stage_p = [&](int kc0, bool first) {
        f32x4 pv[kMP];
        int se[kMP];
#pragma unroll
        for (int i = 0; i < kMP; ++i) {
            f32x4 mn;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                mn[cc] = __builtin_fmaf(mu, mr[i][cc], gr[i][cc]);
                pv[i][cc] = NEST ? __builtin_fmaf(mu, mn[cc], gr[i][cc]) : mn[cc];
            }
            bstore4(mn, rM, boff(mg_off(i, kc0), 4));
            uint32_t mx = __float_as_uint(pv[i][0]) & 0x7fffffffu;
#pragma unroll
            for (int cc = 1; cc < 4; ++cc) {
                const uint32_t u = __float_as_uint(pv[i][cc]) & 0x7fffffffu;
                mx = u > mx ? u : mx;
            }
            se[i] = row_scale_exp(row16_max(mx));
        }
        const int r0 = tid / (kKC / 4), c = 4 * (tid - r0 * (kKC / 4));   // row r0 + 32 i, columns c ..
        if (!first) {
            int so[kMP];
#pragma unroll
            for (int i = 0; i < kMP; ++i) so[i] = rs[r0 + 32 * i];
#pragma unroll
            for (int i = 0; i < kMP; ++i) se[i] = so[i] < se[i] ? so[i] : se[i];
        }
#pragma unroll
        for (int i = 0; i < kMP; ++i) {
            const int r = r0 + 32 * i;
            if ((tid & 15) == 0) rs[r] = se[i];
            uint16_t h[4], l[4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) split2s(__builtin_amdgcn_ldexpf(pv[i][cc], se[i]), h[cc], l[cc]);
            uint16_t *pp = ps + r * kPLD + c;
            *(uint2 *)pp = uint2{pack2(h[0], h[1]), pack2(h[2], h[3])};
            *(uint2 *)(pp + kTR * kPLD) = uint2{pack2(l[0], l[1]), pack2(l[2], l[3])};
        }
    };
    // ---- the slice loads: this wave's pieces (stage bytes 1024 p .. + 1023; plane p / nct) ----
    const int nchunk = (KS + kSPC - 1) / kSPC;
    const int PS = kSPC * nchunk;   // slots per phase
    unsigned dof[L::kND];
    int dlds[L::kND];
#pragma unroll
    for (int i = 0; i < L::kND; ++i) {
        const int p = w + 8 * i < 2 * nct ? w + 8 * i : w;
        const int pl = p >= nct;
        dof[i] = (unsigned)(pl * plane * 2) + 1024u * (unsigned)(p - pl * nct) + 16u * (unsigned)lane;
        dlds[i] = 1024 * p;
    }
    // the loads of slot tl into stage st: Q^T slice tl (projection), Q slice tl - PS (reconstruction),
    // zeros for the padding slots and past the end
    auto issue = [&](int tl, uint16_t *st) {
        const bool proj = tl < PS;
        const int ks = proj ? tl : tl - PS;
        const bool real = ks < KS && tl < 2 * PS;
        const __amdgpu_buffer_rsrc_t rq = proj ? rQT : rQN;
        const unsigned sb = (unsigned)ks * (unsigned)(R * kKSD * 2);
#pragma unroll
        for (int i = 0; i < L::kND; ++i)
            lds_load16(rq, (uint8_t *)st + dlds[i], real ? sb + dof[i] : kOff);
    };

    const int kh = 8 * (lane >> 5);
    const int prow = 32 * rt + (lane & 31);   // the tile row of this lane's accumulators
    load_mg(0);
    issue(0, qst[0]);
    issue(1, qst[1]);
    issue(2, qst[2]);
    f32x16 acc[NCW];
#pragma unroll
    for (int j = 0; j < NCW; ++j) acc[j] = (f32x16){};

    // ---- C^T = Q^T P^T ----
    {
        const int qrow = 32 * cg + (lane & 31);
        const int qoff = qrow * kKSD + 8 * ((lane >> 5) ^ qswz(qrow));
        int sreg = 0;   // the scale exponent acc holds its row at
        for (int c = 0; c < nchunk; ++c) {
            const int kc0 = c * kKC;
#pragma unroll
            for (int s = 0; s < kSPC; ++s) {
                const int ks = kSPC * c + s;
                if (s == 1 || s == 2) vm_wait_barrier<2 * L::kND + 3 * kMP>();
                else vm_wait_barrier<2 * L::kND>();   // slot ks in LDS; every wave done with slot ks - 1
                if (s == 0) {
                    stage_p(kc0, c == 0);
                    load_mg(kc0 + kKC);   // past nb on the last chunk: zeros, no memory traffic
                    lds_barrier();
                }
                issue(ks + 3, qst[(s + 3) % 4]);
                if (ks < KS) {
                    if (s == 0) {
                        const int se = rs[prow];
                        const int d = c == 0 ? 0 : se - sreg;
                        if (__any(d != 0)) {
#pragma unroll
                            for (int j = 0; j < NCW; ++j)
#pragma unroll
                                for (int i = 0; i < 16; ++i) acc[j][i] = __builtin_amdgcn_ldexpf(acc[j][i], d);
                        }
                        sreg = se;
                    }
                    const uint16_t *pr = ps + prow * kPLD + kKSD * s + kh;
                    const f16x8 ah = *(const f16x8 *)pr;
                    const f16x8 al = *(const f16x8 *)(pr + kTR * kPLD);
                    const uint16_t *qb = qst[s] + qoff;
#pragma unroll
                    for (int j = 0; j < NCW; j += 2) {
                        // nct is 2 NCW - 1 or 2 NCW: only the last chunk of a wave can lie past it
                        const bool two = j + 1 < NCW && (j + 1 < NCW - 1 || cg + 2 * (j + 1) < nct);
                        if (j < NCW - 1 || cg + 2 * j < nct) {
                            const uint16_t *q0 = qb + 2 * j * 32 * kKSD;
                            const uint16_t *q1 = q0 + 2 * 32 * kKSD;
                            const f16x8 Qh0 = *(const f16x8 *)q0, Ql0 = *(const f16x8 *)(q0 + R * kKSD);
                            if (two) {
                                const f16x8 Qh1 = *(const f16x8 *)q1, Ql1 = *(const f16x8 *)(q1 + R * kKSD);
                                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, ah, acc[j], 0, 0, 0);
                                acc[j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh1, ah, acc[j + 1], 0, 0, 0);
                                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ql0, ah, acc[j], 0, 0, 0);
                                acc[j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ql1, ah, acc[j + 1], 0, 0, 0);
                                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, al, acc[j], 0, 0, 0);
                                acc[j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh1, al, acc[j + 1], 0, 0, 0);
                            } else {
                                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, ah, acc[j], 0, 0, 0);
                                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ql0, ah, acc[j], 0, 0, 0);
                                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qh0, al, acc[j], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        }
    }
    lds_barrier();   // every wave is done with the P planes the sign tile overwrites
    // ---- the signs -> the sign tile: lane holds row prow, columns 32 ch + 8 qq + 4 (l / 32) + 0..3;
    // bytes at and past nb stay zero (written here for the chunks past nb, below for the row tail) ----
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
        const int ch = cg + 2 * j;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int col = 32 * ch + 8 * qq + 4 * (lane >> 5);   // nb % 4 == 0: all 4 valid or none
            const uint32_t w4 = sign_byte(acc[j][4 * qq]) | (sign_byte(acc[j][4 * qq + 1]) << 8) |
                                (sign_byte(acc[j][4 * qq + 2]) << 16) | (sign_byte(acc[j][4 * qq + 3]) << 24);
            if (ch < nct && col < nb) *(uint32_t *)(ss + prow * spitch + col) = w4;
        }
    }
    // zero the row tails [nb, 16 KS) that the products read (nb % 4 == 0: whole 4-byte words)
    for (int e = tid; e < kTR * ((kKSD * KS - nb) / 4); e += kWT) {
        const int q4 = (kKSD * KS - nb) / 4;
        const int r = e / q4, c = nb + 4 * (e - r * q4);
        *(uint32_t *)(ss + r * spitch + c) = 0u;
    }

    // ---- W <- W - lr (s U + wd W) straight from the accumulators: lane holds column 32 ch + l % 32 of
    // rows 8 (r / 4) + 4 (l / 32) + r % 4 of its 32-row tile, so one 4-byte access per lane covers two
    // 128-byte row pieces.  The descriptors start at the tile's first row and end with its last one,
    // so rows past m are dropped by the hardware; a chunk's W loads are issued two chunks ahead (the
    // first two during the last reconstruction slots) ----
    const int64_t trows = m - row0 < kTR ? m - row0 : kTR;
    const int64_t tile_el = (trows - 1) * n + nb;      // elements from (row0, b nb) to the tile's last one
    const int64_t tbase = row0 * n + (int64_t)b * nb;
    const __amdgpu_buffer_rsrc_t rWt = make_rsrc((const char *)t.W[mat] + tbase * kWS, tile_el * kWS);
    const __amdgpu_buffer_rsrc_t rUt = make_rsrc(U ? (const void *)(U + tbase) : t.W[mat], U ? tile_el * 4 : 0);
    const unsigned rbase = (unsigned)((32 * rt + 4 * (lane >> 5)) * n);   // row offset of r = 0
    const unsigned r8 = (unsigned)(8 * n);
    auto col_off = [&](int j) -> unsigned {
        const int col = 32 * (cg + 2 * j) + (lane & 31);
        return cg + 2 * j < nct && col < nb ? rbase + (unsigned)col : kOff;
    };
    // element offset of register r of a chunk whose row-0 offset is c0 (kOff stays kOff)
    auto el = [&](unsigned c0, int r) -> unsigned {
        return c0 == kOff ? kOff : c0 + (unsigned)(r >> 2) * r8 + (unsigned)(r & 3) * (unsigned)n;
    };
    using WEl = typename std::conditional<WBF16, uint16_t, float>::type;
    WEl wv[3][16];
    auto load_w = [&](int j, WEl (&d)[16]) {
        const unsigned c0 = col_off(j);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (WBF16) d[r] = bload1h(rWt, boff(el(c0, r), 2));
            else d[r] = bload1(rWt, boff(el(c0, r), 4));
        }
    };
    // ---- U = S Q^T over the same rows ----
#pragma unroll
    for (int j = 0; j < NCW; ++j) acc[j] = (f32x16){};
    auto recon_slice = [&](int ks, const uint16_t *qb) {
        const f16x8 as = signs_f16x8(*(const uint2 *)(ss + prow * spitch + kKSD * ks + kh));
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            const int ch = cg + 2 * j;
            if (j < NCW - 1 || ch < nct) {
                const int p = 32 * ch + (lane & 31);
                const int o = p * kKSD + 8 * ((lane >> 5) ^ qswz(p));
                const f16x8 Bh = *(const f16x8 *)(qb + o);
                const f16x8 Bl = *(const f16x8 *)(qb + R * kKSD + o);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as, Bh, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as, Bl, acc[j], 0, 0, 0);
            }
        }
    };
    for (int g = 0; g < nchunk - 1; ++g) {
#pragma unroll
        for (int s = 0; s < kSPC; ++s) {
            const int ks = kSPC * g + s;
            vm_wait_barrier<2 * L::kND>();   // the slice and (first slot) every wave's signs are in LDS
            issue(PS + ks + 3, qst[(s + 3) % 4]);
            if (ks < KS) recon_slice(ks, qst[s]);
        }
    }
    // the last group of four slots: only its first slot has a slice left to load (the last one); after
    // it come the W loads of the update's first two chunks (2 x 16 per lane), which stay in flight
    // through the remaining products
    {
        const int k0 = kSPC * (nchunk - 1);
        vm_wait_barrier<2 * L::kND>();
        issue(PS + k0 + 3, qst[3]);
        asm volatile("" ::: "memory");   // the W loads stay behind the slice loads: the waits below count on it
        __builtin_amdgcn_sched_barrier(0);
        load_w(0, wv[0]);
        load_w(1, wv[1]);
        if (k0 < KS) recon_slice(k0, qst[0]);
        vm_wait_barrier<2 * L::kND + 32>();
        if (k0 + 1 < KS) recon_slice(k0 + 1, qst[1]);
        vm_wait_barrier<L::kND + 32>();
        if (k0 + 2 < KS) recon_slice(k0 + 2, qst[2]);
        vm_wait_barrier<32>();   // the last slice loads of this wave: none lands after the workgroup ends
        if (k0 + 3 < KS) recon_slice(k0 + 3, qst[3]);
    }

#pragma unroll
    for (int j = 0; j < NCW; ++j) {
        if (j + 2 < NCW) load_w(j + 2, wv[(j + 2) % 3]);
        const unsigned c0 = col_off(j);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const unsigned o = el(c0, r);
            float w0;
            if constexpr (WBF16) w0 = bf16_to_f32(wv[j % 3][r]);
            else w0 = wv[j % 3][r];
            const float u = acc[j][r];
            const float nw = w0 - lr * __builtin_fmaf(sc, u, wd * w0);
            if (U) bstore1(u, rUt, boff(o, 4));
            if constexpr (WBF16) bstore1h(f32_to_bf16(nw), rWt, boff(o, 2));
            else bstore1(nw, rWt, boff(o, 4));
        }
    }
}

// One 128-row tile per workgroup: the workgroups of a block are then as many as its tiles and run
// together on one XCD, sharing its basis slices in L2.
int64_t wide_tpg(int64_t, int64_t) { return 1; }

template <int NCT>
hipError_t launch_wide_cfg(const StepArgs &a, int c0, int cnt, int ldp, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const WideGeo geo = wide_geo(nb);
    {
        SplitWideTable t{};
        for (int i = 0; i < cnt; ++i) { t.Q[i] = a.Q[c0 + i]; t.planes[i] = a.planes[c0 + i]; }
        DOBB_LAUNCH("split_q", s, k_split_wide, dim3((unsigned)geo.KS, (unsigned)(nblk * cnt)), dim3(256), 0, nb, nblk, t);
    }
    const int64_t ntile = (m + kTR - 1) / kTR;
    const int64_t tpg = wide_tpg(ntile, (int64_t)nblk * cnt);
    const int ngroups = (int)((ntile + tpg - 1) / tpg);
    const dim3 grid((unsigned)((int64_t)ngroups * nblk * cnt));
    {
        ProjWideTable t{};
        for (int i = 0; i < cnt; ++i) {
            t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.planes[i] = a.planes[c0 + i];
            t.S[i] = (uint8_t *)a.S[c0 + i]; t.mu[i] = a.hp[c0 + i].momentum;
            t.Cout[i] = a.Cout ? a.Cout[c0 + i] : nullptr;
        }
        const size_t sh = proj_wide_lds(nb, ldp);
        const bool gbf = a.g_dtype == DOBB_BF16;
        const bool nest = a.hp[c0].nesterov != 0;
        bool co = false;
        for (int i = 0; i < cnt; ++i) co = co || t.Cout[i] != nullptr;
#define DOBB_PWIDE(NE, GB, CO)                                                                                   \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_proj_wide<NCT, NE, GB, CO>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("project_f16x3", s, (k_proj_wide<NCT, NE, GB, CO>), grid, dim3(kWT), sh, m, n, nb, nblk, ngroups,  \
                    (int)tpg, ldp, t);                                                                           \
    } while (0)
        if (co) {
            if (!nest) { if (gbf) DOBB_PWIDE(0, true, true); else DOBB_PWIDE(0, false, true); }
            else { if (gbf) DOBB_PWIDE(1, true, true); else DOBB_PWIDE(1, false, true); }
        } else {
            if (!nest) { if (gbf) DOBB_PWIDE(0, true, false); else DOBB_PWIDE(0, false, false); }
            else { if (gbf) DOBB_PWIDE(1, true, false); else DOBB_PWIDE(1, false, false); }
        }
#undef DOBB_PWIDE
    }
    {
        ReconWideTable t{};
        for (int i = 0; i < cnt; ++i) {
            const dobb_hparams &h = a.hp[c0 + i];
            t.S[i] = (const uint8_t *)a.S[c0 + i]; t.planes[i] = a.planes[c0 + i]; t.W[i] = a.W[c0 + i];
            t.U[i] = a.U ? a.U[c0 + i] : nullptr;
            t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
        }
        const size_t sh = recon_wide_lds(nb, ldp);
        const int rtiles = (int)((m + kRTR - 1) / kRTR);
        const dim3 rgrid((unsigned)((int64_t)rtiles * nblk * cnt));
#define DOBB_RWIDE(WB)                                                                                           \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_recon_wide<NCT, WB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("reconstruct_f16x2", s, (k_recon_wide<NCT, WB>), rgrid, dim3(kWT), sh, m, n, nb, nblk, rtiles, \
                    ldp, t);                                                                                     \
    } while (0)
        if (a.w_dtype == DOBB_BF16) DOBB_RWIDE(true); else DOBB_RWIDE(false);
#undef DOBB_RWIDE
    }
    return hipGetLastError();
}

// The one-pass sign step: the basis planes, then one workgroup per 128-row tile of every block.
template <int NCW>
hipError_t launch_wide_fused_cfg(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const WideGeo geo = wide_geo(nb);
    {
        SplitWideTable t{};
        for (int i = 0; i < cnt; ++i) { t.Q[i] = a.Q[c0 + i]; t.planes[i] = a.planes[c0 + i]; }
        DOBB_LAUNCH("split_q", s, k_split_wide, dim3((unsigned)geo.KS, (unsigned)(nblk * cnt)), dim3(256), 0, nb, nblk, t);
    }
    if (geo.R > RingGeo<NCW>::RM) return hipErrorInvalidValue;   // the static stages hold RM rows (nb <= 416)
    const int ntile = (int)((m + kTR - 1) / kTR);
    const dim3 grid((unsigned)((int64_t)ntile * nblk * cnt));
    FusedWideTable t{};
    for (int i = 0; i < cnt; ++i) {
        const dobb_hparams &h = a.hp[c0 + i];
        t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.planes[i] = a.planes[c0 + i]; t.W[i] = a.W[c0 + i];
        t.U[i] = a.U ? a.U[c0 + i] : nullptr;
        t.mu[i] = h.momentum; t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
    }
    const bool gbf = a.g_dtype == DOBB_BF16, wbf = a.w_dtype == DOBB_BF16;
    const bool nest = a.hp[c0].nesterov != 0;
#define DOBB_WF(NE, GB, WB)                                                                                      \
    DOBB_LAUNCH("step_wide_fused_f16", s, (k_step_wide_fused<NCW, NE, GB, WB>), grid, dim3(kWT), 0, m, n, nb, nblk, ntile, t)
    if (!nest) {
        if (gbf) { if (wbf) DOBB_WF(0, true, true); else DOBB_WF(0, true, false); }
        else { if (wbf) DOBB_WF(0, false, true); else DOBB_WF(0, false, false); }
    } else {
        if (gbf) { if (wbf) DOBB_WF(1, true, true); else DOBB_WF(1, true, false); }
        else { if (wbf) DOBB_WF(1, false, true); else DOBB_WF(1, false, false); }
    }
#undef DOBB_WF
    return hipGetLastError();
}

// Column-l2: the basis planes, C (with momentum) into the workspace, the column scales, then the
// reconstruction of C~ with the W update.
template <int NCT>
hipError_t launch_wide_l2_cfg(const StepArgs &a, int c0, int cnt, int ldp, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const WideGeo geo = wide_geo(nb);
    {
        SplitWideTable t{};
        for (int i = 0; i < cnt; ++i) { t.Q[i] = a.Q[c0 + i]; t.planes[i] = a.planes[c0 + i]; }
        DOBB_LAUNCH("split_q", s, k_split_wide, dim3((unsigned)geo.KS, (unsigned)(nblk * cnt)), dim3(256), 0, nb, nblk, t);
    }
    const int64_t ntile = (m + kTR - 1) / kTR;
    const int64_t tpg = wide_tpg(ntile, (int64_t)nblk * cnt);
    const int ngroups = (int)((ntile + tpg - 1) / tpg);
    const dim3 grid((unsigned)((int64_t)ngroups * nblk * cnt));
    {
        ProjWideTable t{};
        for (int i = 0; i < cnt; ++i) {
            t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.planes[i] = a.planes[c0 + i];
            t.C[i] = a.C[c0 + i]; t.mu[i] = a.hp[c0 + i].momentum;
            t.Cout[i] = a.Cout ? a.Cout[c0 + i] : nullptr;
        }
        const size_t sh = proj_wide_lds(nb, ldp);
        const bool gbf = a.g_dtype == DOBB_BF16;
        const bool nest = a.hp[c0].nesterov != 0;
#define DOBB_PWL2(NE, GB)                                                                                        \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_proj_wide<NCT, NE, GB, false, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("project_l2_f16x3", s, (k_proj_wide<NCT, NE, GB, false, true>), grid, dim3(kWT), sh, m, n, nb, nblk, \
                    ngroups, (int)tpg, ldp, t);                                                                  \
    } while (0)
        if (!nest) { if (gbf) DOBB_PWL2(0, true); else DOBB_PWL2(0, false); }
        else { if (gbf) DOBB_PWL2(1, true); else DOBB_PWL2(1, false); }
#undef DOBB_PWL2
    }
    {
        const hipError_t e = launch_colnorm(a, c0, cnt, s);
        if (e != hipSuccess) return e;
    }
    {
        ReconWideTable t{};
        for (int i = 0; i < cnt; ++i) {
            const dobb_hparams &h = a.hp[c0 + i];
            t.C[i] = a.C[c0 + i]; t.cs[i] = a.colscale[c0 + i];
            t.planes[i] = a.planes[c0 + i]; t.W[i] = a.W[c0 + i];
            t.U[i] = a.U ? a.U[c0 + i] : nullptr;
            t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
        }
        const size_t sh = recon_wide_lds(nb, ldp, true);
        const int rtiles = (int)((m + kRTR - 1) / kRTR);
        const dim3 rgrid((unsigned)((int64_t)rtiles * nblk * cnt));
#define DOBB_RWL2(WB)                                                                                            \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_recon_wide<NCT, WB, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("reconstruct_l2_f16x3", s, (k_recon_wide<NCT, WB, true>), rgrid, dim3(kWT), sh, m, n, nb, nblk,  \
                    rtiles, ldp, t);                                                                             \
    } while (0)
        if (a.w_dtype == DOBB_BF16) DOBB_RWL2(true); else DOBB_RWL2(false);
#undef DOBB_RWL2
    }
    return hipGetLastError();
}

}  // namespace

bool step_wide_eligible(const dobb_shape &sh) {
    // the launcher instantiates 5 <= ceil(nb / 32) <= 13
    if (sh.nb <= 128 || sh.nb > 416 || sh.nb % 4 != 0) return false;
    const int ldp = step_bf16_ldp(sh.nb);
    // 32-bit buffer offsets: the largest byte offset into M, G, W, U or the sign codes
    const int64_t big = sh.m * sh.n * 4 > sh.m * (sh.n / sh.nb) * ldp ? sh.m * sh.n * 4 : sh.m * (sh.n / sh.nb) * ldp;
    if (big >= ((int64_t)1 << 31)) return false;
    return (int64_t)proj_wide_lds((int)sh.nb, ldp) <= max_lds_bytes() &&
           (int64_t)recon_wide_lds((int)sh.nb, ldp) <= max_lds_bytes();
}

size_t step_wide_planes_bytes(const dobb_shape &sh) {
    return (size_t)4 * (size_t)(sh.n / sh.nb) * (size_t)wide_plane_elems((int)sh.nb) * 2;
}

hipError_t launch_step_wide_l2(const StepArgs &a, int c0, int cnt, hipStream_t s) {
    const int ldp = step_bf16_ldp(a.sh.nb);
    switch ((int)((a.sh.nb + 31) / 32)) {
        case 5: return launch_wide_l2_cfg<5>(a, c0, cnt, ldp, s);
        case 6: return launch_wide_l2_cfg<6>(a, c0, cnt, ldp, s);
        case 7: return launch_wide_l2_cfg<7>(a, c0, cnt, ldp, s);
        case 8: return launch_wide_l2_cfg<8>(a, c0, cnt, ldp, s);
        case 9: return launch_wide_l2_cfg<9>(a, c0, cnt, ldp, s);
        case 10: return launch_wide_l2_cfg<10>(a, c0, cnt, ldp, s);
        case 11: return launch_wide_l2_cfg<11>(a, c0, cnt, ldp, s);
        case 12: return launch_wide_l2_cfg<12>(a, c0, cnt, ldp, s);
        case 13: return launch_wide_l2_cfg<13>(a, c0, cnt, ldp, s);
        default: return hipErrorInvalidValue;   // see step_wide_eligible
    }
}

hipError_t launch_step_wide(const StepArgs &a, int ldp, hipStream_t s) {
    const int nct = (int)((a.sh.nb + 31) / 32);
    for (int c0 = 0; c0 < a.count;) {
        const int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        hipError_t e;
        // the one-pass kernel unless the coefficients are asked for (the two-kernel path writes them)
        bool co = false;
        for (int i = 0; i < cnt; ++i) co = co || (a.Cout && a.Cout[c0 + i]);
        if (!co) {   // the one-pass kernel's static LDS fits every nb <= 416
            switch ((nct + 1) / 2) {
                case 3: e = launch_wide_fused_cfg<3>(a, c0, cnt, s); break;
                case 4: e = launch_wide_fused_cfg<4>(a, c0, cnt, s); break;
                case 5: e = launch_wide_fused_cfg<5>(a, c0, cnt, s); break;
                case 6: e = launch_wide_fused_cfg<6>(a, c0, cnt, s); break;
                case 7: e = launch_wide_fused_cfg<7>(a, c0, cnt, s); break;
                default: return hipErrorInvalidValue;   // see step_wide_eligible
            }
            if (e != hipSuccess) return e;
            c0 += cnt;
            continue;
        }
        switch (nct) {
            case 5: e = launch_wide_cfg<5>(a, c0, cnt, ldp, s); break;
            case 6: e = launch_wide_cfg<6>(a, c0, cnt, ldp, s); break;
            case 7: e = launch_wide_cfg<7>(a, c0, cnt, ldp, s); break;
            case 8: e = launch_wide_cfg<8>(a, c0, cnt, ldp, s); break;
            case 9: e = launch_wide_cfg<9>(a, c0, cnt, ldp, s); break;
            case 10: e = launch_wide_cfg<10>(a, c0, cnt, ldp, s); break;
            case 11: e = launch_wide_cfg<11>(a, c0, cnt, ldp, s); break;
            case 12: e = launch_wide_cfg<12>(a, c0, cnt, ldp, s); break;
            case 13: e = launch_wide_cfg<13>(a, c0, cnt, ldp, s); break;
            default: return hipErrorInvalidValue;   // nb > 416 does not fit the LDS (see step_wide_eligible)
        }
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
