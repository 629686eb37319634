// The Dobb step (sign normalisation) in one pass for block widths nb <= 128, nb % 4 == 0.
//
// Dobb paper (arXiv 2610.39412): abstract (project momentum into the block bases, sign-normalise,
// reconstruct), Table 9 (update scale), Table 21 caption (decoupled weight decay), Table 19
// (Nesterov).
//
// One workgroup of 8 waves per (block, row range): the block's basis is split once into two fp16
// planes (Q = h + l, |Q| <= 1) in both orientations and stays in LDS; after that single barrier every
// wave works on its own 16-row tiles with no further synchronisation:
//   - M and G rows come straight from HBM into the registers of the MFMA operand layout, the new
//     momentum goes back from the same registers, and each row is scaled by a power of two (from its
//     largest |P|, a two-step shuffle over the row's four lane groups) and split into fp16 hi + lo;
//   - C^T = Q^T P^T as three fp16 products per 16 x 16 x 32 step (Qh Ph + Ql Ph + Qh Pl);
//   - the contraction index of both products runs in the order
//       kappa = 32 s + 8 g + i  <->  p = 32 s + 4 g + (i mod 4) + 16 (i div 4)
//     (s the step, g the lane group, i the lane's k slot), the order in which the projection's
//     accumulators hold C: lane (r, g) ends with C[r][16 ch + 4 g + 0..3] for every 16-column chunk
//     ch, which is exactly its slot of the reconstruction's operand sign(C)^T. The signs never leave
//     the registers, and the basis planes in LDS are stored in that order;
//   - U^T = Q sign(C)^T as two fp16 products (Qh S + Ql S, signs exact in fp16), and lane (r, g) ends
//     with U[r][16 ch + 4 g + 0..3], the W entries it updates and stores.
// HBM traffic is the method's: G and W read, M read and written, W written. The next tile's M and G
// and the current tile's W are in flight while the products run.
#include "step_common.h"

namespace dobb {
using namespace stepk;
namespace {

constexpr int kFT = 512;   // threads per workgroup (8 waves)

struct FusedGeo {
    int nc;     // 16-column chunks of the block
    int ks;     // 32-deep contraction steps (both products)
    int rows;   // basis rows held: 16 nc
    int ld;     // plane pitch in 2-byte elements: 32 ks + 16, i.e. 2 mod 4 in 16-byte units, the pitches
                // at which the 16-byte reads of 16 rows x 4 lane groups run without bank conflicts
                // on gfx950 (odd pitches give two-way conflicts for this pattern)
};
__host__ __device__ inline FusedGeo fused_geo(int nb) {
    FusedGeo g;
    g.nc = (nb + 15) / 16;
    g.ks = (nb + 31) / 32;
    g.rows = 16 * g.nc;
    g.ld = 32 * g.ks + 16;
    return g;
}
__host__ __device__ inline size_t fused_lds(int nb) {
    const FusedGeo g = fused_geo(nb);
    return (size_t)4 * g.rows * g.ld * 2;   // two orientations x two planes
}
// contraction slot kappa -> basis index p (see the file comment)
__host__ __device__ inline int fused_perm(int kappa) {
    return 32 * (kappa >> 5) + 4 * ((kappa >> 3) & 3) + (kappa & 3) + 16 * ((kappa >> 2) & 1);
}

struct FusedTable {
    float *M[kMaxMats];
    const void *G[kMaxMats];
    const float *Q[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float *C[kMaxMats];
    float mu[kMaxMats], lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};

// grid.x = row groups x blocks x matrices (block fastest, renumbered per XCD), block 512.
// NC, KS: fused_geo(nb).nc and .ks; NEST: Nesterov momentum; CO: also write C (a verification
// output: the unscaled coefficients P Q_b in fp32).
template <int NC, int KS, int NEST, bool GBF16, bool WBF16, bool CO>
__global__ void __launch_bounds__(kFT) k_step_fused(int64_t m, int64_t n, int nb, int nblk, int ngroups, int tpg,
                                                    FusedTable t) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int ROWS = 16 * NC, LD = 32 * KS + 16, PLANE = ROWS * LD;
    uint16_t *qa = (uint16_t *)lds;          // [2][ROWS][LD]: (j, kappa) -> Q[perm(kappa)][j]   (projection)
    uint16_t *qb = qa + 2 * PLANE;           // [2][ROWS][LD]: (c, kappa) -> Q[c][perm(kappa)]   (reconstruction)

    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int b = x % nblk, rest = x / nblk;
    const int tg = rest % ngroups, mat = rest / ngroups;
    const int tid = threadIdx.x;

    // ---- the block's basis: both orientations, both planes, contraction order kappa ----
    {
        const float *Q = t.Q[mat] + (int64_t)b * nb * nb;
        constexpr int K8 = 4 * KS;                     // 8-slot groups per row
        for (int e = tid; e < ROWS * K8; e += kFT) {
            const int r = e % ROWS, k0 = 8 * (e / ROWS);   // r fastest: coalesced reads of Q[p][r]
            uint16_t ah[8], al[8], bh[8], bl[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int p = fused_perm(k0 + i);
                const bool in = r < nb && p < nb;
                split2h(in ? Q[(int64_t)p * nb + r] : 0.f, ah[i], al[i]);
                split2h(in ? Q[(int64_t)r * nb + p] : 0.f, bh[i], bl[i]);
            }
            uint16_t *a0 = qa + r * LD + k0, *b0 = qb + r * LD + k0;
            *(uint4 *)a0 = uint4{pack2(ah[0], ah[1]), pack2(ah[2], ah[3]), pack2(ah[4], ah[5]), pack2(ah[6], ah[7])};
            *(uint4 *)(a0 + PLANE) = uint4{pack2(al[0], al[1]), pack2(al[2], al[3]), pack2(al[4], al[5]), pack2(al[6], al[7])};
            *(uint4 *)b0 = uint4{pack2(bh[0], bh[1]), pack2(bh[2], bh[3]), pack2(bh[4], bh[5]), pack2(bh[6], bh[7])};
            *(uint4 *)(b0 + PLANE) = uint4{pack2(bl[0], bl[1]), pack2(bl[2], bl[3]), pack2(bl[4], bl[5]), pack2(bl[6], bl[7])};
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t ntile = (m + 15) / 16;
    const int64_t t_begin = (int64_t)tg * tpg;
    const int64_t t_end = t_begin + tpg < ntile ? t_begin + tpg : ntile;
    float *const M = t.M[mat];
    const char *const Gv = (const char *)t.G[mat];
    char *const Wv = (char *)t.W[mat];
    float *const U = t.U[mat];
    float *const Cq = t.C[mat];
    const float mu = t.mu[mat], lrate = t.lr[mat], wd = t.wd[mat], sc = t.scale[mat];
    constexpr int GS = GBF16 ? 2 : 4, WS = WBF16 ? 2 : 4;
    const int col0 = b * nb;
    // Global accesses go through buffer descriptors that cover one 16-row tile (rows past m, or past
    // the range, have no bytes): a lane with nothing to read gets zeros and its stores are dropped,
    // with no branch around the instruction. Element offsets within a tile: lr n + col0 + p < 16 n.
    // lane (lr, lg) of step s holds P[row][32 s + 4 lg + 0..3] (half 0) and P[row][32 s + 16 + 4 lg + 0..3]
    // (half 1): two four-column pieces, each valid as a whole (nb % 4 == 0)
    unsigned eo[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int p = 32 * s + 16 * h + 4 * lg;
            eo[s][h] = p < nb ? (unsigned)(lr * (int)n + col0 + p) : kOff;
        }
    // W, U and C: lane (lr, lg) holds columns 16 ch + 4 lg + 0..3
    unsigned wo[NC];
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
        const int c = 16 * ch + 4 * lg;
        wo[ch] = c < nb ? (unsigned)(lr * (int)n + col0 + c) : kOff;
    }
    auto tile_rows = [&](int64_t tl) -> int64_t {
        if (tl >= t_end) return 0;
        const int64_t r = m - tl * 16;
        return r < 16 ? r : 16;
    };

    // M and G of two tiles in flight where the registers allow it (up to 112 basis rows; 248 VGPRs at
    // 128 rows, where one tile ahead is kept): buffer BUF (a compile-time index) holds tile tl
    constexpr bool kTwo = NC <= 7;
    f32x4 pm[kTwo ? 2 : 1][KS][2], pg[kTwo ? 2 : 1][KS][2];
    auto load_mg = [&](int64_t tl, auto BUF) {
        constexpr int B_ = decltype(BUF)::value;
        const int64_t rows = tile_rows(tl), r0 = tl * 16;
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(M + r0 * n, rows * n * 4);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(Gv + r0 * n * GS, rows * n * GS);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) pm[B_][s][h] = bload4(rm, boff(eo[s][h], 4));
        __builtin_amdgcn_sched_barrier(0);   // all of the tile's M rows, then its G rows (2 % faster
                                             // on the GPT-2 XL shapes than interleaving the two)
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (GBF16) {
                    const uint2 hb = bload2u(rg, boff(eo[s][h], 2));
                    pg[B_][s][h] = f32x4{bf16_to_f32((uint16_t)hb.x), bf16_to_f32((uint16_t)(hb.x >> 16)),
                                     bf16_to_f32((uint16_t)hb.y), bf16_to_f32((uint16_t)(hb.y >> 16))};
                } else {
                    pg[B_][s][h] = bload4(rg, boff(eo[s][h], 4));
                }
            }
    };

    auto do_tile = [&](int64_t tile, auto BUF) {
        constexpr int B_ = decltype(BUF)::value;
        const int64_t rows = tile_rows(tile), r0 = tile * 16;
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(M + r0 * n, rows * n * 4);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(Wv + r0 * n * WS, rows * n * WS);
        // momentum (written back), the row's scale, P scaled and split into the B operands
        f16x8 ph[KS], pl[KS];
        uint32_t mx = 0u;
        f32x4 pv[KS][2];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 mn;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    mn[cc] = __builtin_fmaf(mu, pm[B_][s][h][cc], pg[B_][s][h][cc]);
                    pv[s][h][cc] = NEST ? __builtin_fmaf(mu, mn[cc], pg[B_][s][h][cc]) : mn[cc];
                    const uint32_t u = __float_as_uint(pv[s][h][cc]) & 0x7fffffffu;
                    mx = u > mx ? u : mx;
                }
                bstore4(mn, rm, boff(eo[s][h], 4));
            }
        // the row's largest magnitude over the wave's four 16-lane rows: the lane swaps between rows
        // (whichever way a swap goes, the two results of a lane are its own value and its partner's)
        {
            const auto a = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
            mx = max(a[0], a[1]);
            const auto b = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
            mx = max(b[0], b[1]);
        }
        const int sexp = row_scale_exp(mx);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint16_t hh[8], hl[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) split2s(__builtin_amdgcn_ldexpf(pv[s][i >> 2][i & 3], sexp), hh[i], hl[i]);
            ph[s] = __builtin_bit_cast(f16x8, uint4{pack2(hh[0], hh[1]), pack2(hh[2], hh[3]), pack2(hh[4], hh[5]), pack2(hh[6], hh[7])});
            pl[s] = __builtin_bit_cast(f16x8, uint4{pack2(hl[0], hl[1]), pack2(hl[2], hl[3]), pack2(hl[4], hl[5]), pack2(hl[6], hl[7])});
        }
        // the M and G of this buffer's next tile (two tiles on, or the next one), this tile's W
        load_mg(tile + (kTwo ? 16 : 8), BUF);
        using WVec = typename std::conditional<WBF16, uint2, f32x4>::type;
        WVec wcur[NC];
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            if constexpr (WBF16) wcur[ch] = bload2u(rw, boff(wo[ch], 2));
            else wcur[ch] = bload4(rw, boff(wo[ch], 4));
        }
        // C^T = Q^T P^T: chunk ch of lane (lr, lg) = C[row][16 ch + 4 lg + 0..3] (scaled by 2^sexp)
        f32x4 acc[NC];
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) acc[ch] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int ch = 0; ch < NC; ++ch) {
                const uint16_t *qp = qa + (16 * ch + lr) * LD + 32 * s + 8 * lg;
                const f16x8 ah = __builtin_bit_cast(f16x8, *(const uint4 *)qp);
                const f16x8 al = __builtin_bit_cast(f16x8, *(const uint4 *)(qp + PLANE));
                acc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ph[s], acc[ch], 0, 0, 0);
                acc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, ph[s], acc[ch], 0, 0, 0);
                acc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, pl[s], acc[ch], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep each step's operand loads inside the step
        }
        if constexpr (CO) {
            if (Cq) {
                const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cq + r0 * n, rows * n * 4);
#pragma unroll
                for (int ch = 0; ch < NC; ++ch)
                    bstore4(f32x4{__builtin_amdgcn_ldexpf(acc[ch][0], -sexp), __builtin_amdgcn_ldexpf(acc[ch][1], -sexp),
                                  __builtin_amdgcn_ldexpf(acc[ch][2], -sexp), __builtin_amdgcn_ldexpf(acc[ch][3], -sexp)},
                            rc, boff(wo[ch], 4));
            }
        }
        // sign(C) as the reconstruction's B operand: slots 0..3 of step s from chunk 2 s, 4..7 from
        // chunk 2 s + 1 (zero past the last chunk; zero columns of the basis give C = 0 past nb)
        f16x8 sg[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint32_t w[4];
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                const int ch = 2 * s + hq;
                if (ch < NC) {
                    w[2 * hq] = (sign_byte(acc[ch][0]) << 8) | (sign_byte(acc[ch][1]) << 24);
                    w[2 * hq + 1] = (sign_byte(acc[ch][2]) << 8) | (sign_byte(acc[ch][3]) << 24);
                } else {
                    w[2 * hq] = w[2 * hq + 1] = 0u;
                }
            }
            sg[s] = __builtin_bit_cast(f16x8, uint4{w[0], w[1], w[2], w[3]});
        }
        // U^T = Q sign(C)^T: chunk ch of lane (lr, lg) = U[row][16 ch + 4 lg + 0..3]
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) acc[ch] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int ch = 0; ch < NC; ++ch) {
                const uint16_t *qp = qb + (16 * ch + lr) * LD + 32 * s + 8 * lg;
                const f16x8 bh = __builtin_bit_cast(f16x8, *(const uint4 *)qp);
                const f16x8 bl = __builtin_bit_cast(f16x8, *(const uint4 *)(qp + PLANE));
                acc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, sg[s], acc[ch], 0, 0, 0);
                acc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bl, sg[s], acc[ch], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // W <- W - lr (s U + wd W)
        if (U) {
            const __amdgpu_buffer_rsrc_t ru = make_rsrc(U + r0 * n, rows * n * 4);
#pragma unroll
            for (int ch = 0; ch < NC; ++ch) bstore4(acc[ch], ru, boff(wo[ch], 4));
        }
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            f32x4 w0;
            if constexpr (WBF16)
                w0 = f32x4{bf16_to_f32((uint16_t)wcur[ch].x), bf16_to_f32((uint16_t)(wcur[ch].x >> 16)),
                           bf16_to_f32((uint16_t)wcur[ch].y), bf16_to_f32((uint16_t)(wcur[ch].y >> 16))};
            else
                w0 = wcur[ch];
            float nw[4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) nw[cc] = w0[cc] - lrate * __builtin_fmaf(sc, acc[ch][cc], wd * w0[cc]);
            if constexpr (WBF16) {
                bstore2u(uint2{(uint32_t)f32_to_bf16(nw[0]) | ((uint32_t)f32_to_bf16(nw[1]) << 16),
                               (uint32_t)f32_to_bf16(nw[2]) | ((uint32_t)f32_to_bf16(nw[3]) << 16)},
                         rw, boff(wo[ch], 2));
            } else {
                bstore4(f32x4{nw[0], nw[1], nw[2], nw[3]}, rw, boff(wo[ch], 4));
            }
        }
        };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int64_t tile = t_begin + wv;
    load_mg(tile, I0{});
    if constexpr (kTwo) load_mg(tile + 8, I1{});
    // the first tile's rows, waited for here: the loop head then has no loads of its own to wait for
    // and does not wait for the previous tile's stores
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (kTwo) {
        for (; tile < t_end; tile += 16) {
            do_tile(tile, I0{});
            if (tile + 8 < t_end) do_tile(tile + 8, I1{});
        }
    } else {
        for (; tile < t_end; tile += 8) do_tile(tile, I0{});
    }

}

template <int NC, int KS>
hipError_t launch_fused_cfg(const StepArgs &a, int c0, int cnt, bool co, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const int64_t ntile = (m + 15) / 16;
    const int64_t blocks = (int64_t)nblk * cnt;
    // about 4096 workgroups (16 per CU, one resident at a time) over the launch: a block's rows in
    // the nearest whole number of equal groups (measured on the GPT-2 XL shapes: 1024 workgroups
    // run 8 % slower, 2048 1.5 %, 8192 2 %)
    int64_t ngroups = (4096 + blocks / 2) / blocks;
    if (ngroups < 1) ngroups = 1;
    if (ngroups > ntile) ngroups = ntile;
    const int64_t tpg = (ntile + ngroups - 1) / ngroups;
    ngroups = (ntile + tpg - 1) / tpg;
    if (ngroups * blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(ngroups * blocks));
    FusedTable t{};
    for (int i = 0; i < cnt; ++i) {
        const dobb_hparams &h = a.hp[c0 + i];
        t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.Q[i] = a.Q[c0 + i]; t.W[i] = a.W[c0 + i];
        t.U[i] = a.U ? a.U[c0 + i] : nullptr;
        t.C[i] = a.Cout ? a.Cout[c0 + i] : nullptr;
        t.mu[i] = h.momentum; t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
    }
    const size_t sh = fused_lds(nb);
    const bool gbf = a.g_dtype == DOBB_BF16, wbf = a.w_dtype == DOBB_BF16;
    const bool nest = a.hp[c0].nesterov != 0;
#define DOBB_F(NE, GB, WB, C)                                                                                    \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_step_fused<NC, KS, NE, GB, WB, C>,                             \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);                          \
        DOBB_LAUNCH("step_fused_f16", s, (k_step_fused<NC, KS, NE, GB, WB, C>), grid, dim3(kFT), sh, m, n, nb,  \
                    nblk, (int)ngroups, (int)tpg, t);                                                            \
    } while (0)
#define DOBB_F2(NE, C)                                                                                           \
    do {                                                                                                         \
        if (gbf) { if (wbf) DOBB_F(NE, true, true, C); else DOBB_F(NE, true, false, C); }                        \
        else { if (wbf) DOBB_F(NE, false, true, C); else DOBB_F(NE, false, false, C); }                          \
    } while (0)
    if (co) { if (nest) DOBB_F2(1, true); else DOBB_F2(0, true); }
    else { if (nest) DOBB_F2(1, false); else DOBB_F2(0, false); }
#undef DOBB_F2
#undef DOBB_F
    return hipGetLastError();
}

}  // namespace

bool step_fused_eligible(const dobb_shape &sh) {
    // 32-bit byte offsets within a 16-row tile: 64 n < 2^32
    return sh.nb >= 4 && sh.nb <= 128 && sh.nb % 4 == 0 && sh.n % 4 == 0 && sh.n < ((int64_t)1 << 25) &&
           (int64_t)fused_lds((int)sh.nb) <= max_lds_bytes();
}

hipError_t launch_step_fused(const StepArgs &a, hipStream_t s) {
    const FusedGeo g = fused_geo((int)a.sh.nb);
    for (int c0 = 0; c0 < a.count;) {
        const int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        bool co = false;
        for (int i = 0; i < cnt; ++i) co = co || (a.Cout && a.Cout[c0 + i]);
        hipError_t e;
        switch (g.nc) {
            case 1: e = launch_fused_cfg<1, 1>(a, c0, cnt, co, s); break;
            case 2: e = launch_fused_cfg<2, 1>(a, c0, cnt, co, s); break;
            case 3: e = launch_fused_cfg<3, 2>(a, c0, cnt, co, s); break;
            case 4: e = launch_fused_cfg<4, 2>(a, c0, cnt, co, s); break;
            case 5: e = launch_fused_cfg<5, 3>(a, c0, cnt, co, s); break;
            case 6: e = launch_fused_cfg<6, 3>(a, c0, cnt, co, s); break;
            case 7: e = launch_fused_cfg<7, 4>(a, c0, cnt, co, s); break;
            case 8: e = launch_fused_cfg<8, 4>(a, c0, cnt, co, s); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
