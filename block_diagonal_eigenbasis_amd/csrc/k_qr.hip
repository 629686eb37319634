// Householder QR of every block of a launch: Q_b <- qr(Z_b).Q with diag(R) > 0.
//
// Dobb paper (arXiv 2610.39412), Tables 15-16: the orthogonal-iteration refresh orthonormalises
// Z = A_b Q_b with a QR routine, Householder being the principal one.
//
// Blocked Householder with 32-column panels.  Reflector c of a panel is H = I - tau v v^T with
// v_c = 1, v_r = x_r / (x_c + sgn(x_c) ||x||), tau = 1 + |x_c| / ||x||, R_cc = -sgn(x_c) ||x||; the
// panel's reflectors combine as H_1 ... H_w = I - V T V^T (compact WY).  Factoring applies
// I - V T^T V^T to the trailing columns; Q is formed from the identity by applying I - V T V^T for
// the panels last to first on rows and columns >= the panel start, the last application also
// negating the columns whose R_cc < 0.
//
// Panel factorisation (factor_panel): the panel lives in registers, thread 8 k + g holding column k
// at rows g RPT .. g RPT + RPT - 1, so a column's threads share a wave; each column costs one
// workgroup barrier.  Norms, the cross-thread sums and T are kept in fp64, the per-element work is
// fp32.  The dot products
// v_c^T x_k of a column step also give v_k^T v_c for the earlier columns k, from which T is built
// one column behind.
//
// nb <= 128 (k_qr_block): one workgroup per block with Z in LDS does every panel, trailing update
// and formation step in one launch.
// nb > 128: per panel one k_qr_panel launch (one workgroup per block) and one k_qr_apply launch
// (one workgroup per 64-column tile per block); formation is a single k_qr_form launch that carries
// each 64-column tile of Q through all panels.  A wave keeps its 32 x (rows/2) share of a tile in
// registers from load to store, in the MFMA accumulator layout (rows are fed to the V^T X products
// in that order), so the tile is read and written once; V is staged in LDS.
#include "dobb_internal.h"

#include <math.h>

namespace dobb {
namespace {

constexpr int kPW = 32;             // panel width
constexpr int kQT = 256;            // threads per workgroup
constexpr int kGroups = kQT / kPW;  // row groups of a panel
constexpr int kVRows = 576;         // floats of a published column buffer (kGroups x (RPT + 4), RPT <= 64)

struct QrBlockOut {
    float *Q[kMaxMats];
    int32_t *info[kMaxMats];
};

__host__ __device__ inline size_t a16(size_t x) { return (x + 15) / 16 * 16; }

// ---- panel factorisation ------------------------------------------------------------------------
struct PanelLds {
    size_t gs, td, vcol, red, part, tau, total;
};
__host__ __device__ inline PanelLds panel_lds(int nb, size_t o) {
    PanelLds L;
    L.gs = o;   o += a16((size_t)kPW * kPW * 8);      // v_k^T v_c (k < c)
    L.td = o;   o += a16((size_t)kPW * kPW * 8);      // T, fp64
    L.vcol = o; o += a16((size_t)2 * kVRows * 4);     // column c, double buffered by c parity
    L.red = o;  o += a16((size_t)2 * kGroups * 8);
    L.part = o; o += a16((size_t)kGroups * kPW * 8);
    L.tau = o;  o += a16((size_t)kPW * 8);
    L.total = o;
    return L;
}

struct PanelPtrs {
    double (*Gs)[kPW];
    double (*Td)[kPW];
    float *vcol;
    double *red;
    double (*part)[kPW];
    double *tau;
};
__device__ inline PanelPtrs panel_ptrs(unsigned char *dsm, const PanelLds &L) {
    return PanelPtrs{(double(*)[kPW])(dsm + L.gs), (double(*)[kPW])(dsm + L.td), (float *)(dsm + L.vcol),
                     (double *)(dsm + L.red), (double(*)[kPW])(dsm + L.part), (double *)(dsm + L.tau)};
}

// v from lane l's partner under a DPP lane pattern (both 32-bit halves moved)
template <int CTRL>
__device__ __forceinline__ double dpp_double(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// sum over the 8 lanes of a column (lanes 8 k .. 8 k + 7 of a wave), in registers: the quad's
// partners by quad_perm [1,0,3,2] and [2,3,0,1], then the other quad of the 8 by row_half_mirror
// (lane i of a half-row of 8 takes lane 7 - i)
__device__ __forceinline__ double col_sum(double v) {
    v += dpp_double<0xB1>(v);
    v += dpp_double<0x4E>(v);
    v += dpp_double<0x141>(v);
    return v;
}

// Factor the panel held in P (thread tid = 8 k + grp: column k, rows grp RPT + i of the rows x w
// panel, zero at rows >= rows).  On return P holds column k of V (0 above row k), negf[c] = 1 where
// R_cc < 0, and S.Td (fp64, upper triangle of the leading w x w) holds T once the caller has passed
// a barrier.
// A column's 8 threads share a wave, so its cross-thread sums are shuffles and a column step has
// one workgroup barrier.  Column c is published by its own wave with its rows above c zeroed and
// row c replaced by x_c + sgn(x_c) ||x||, so that v = x / (x_c + sgn(x_c) ||x||) is one scaling of
// the published column on every row (v_c = 1 up to one fp32 rounding, and that same v is stored
// and used everywhere); ||x|| and x_c go along in fp64 for tau = 1 + |x_c| / ||x|| and the sign.
template <int RPT>
__device__ __forceinline__ void factor_panel(float (&P)[RPT], int w, int rows, int k, int grp, const PanelPtrs &S,
                                             int8_t *negf) {
    static_assert(RPT % 4 == 0 && kGroups * (RPT + 4) <= kVRows, "panel rows");
    // a published column keeps group g's rows at [g (RPT + 4), + RPT): the 4-float gap between
    // groups puts the 8 groups of a wave's reads on distinct banks
    constexpr int kGS = RPT + 4;
    const int rbase = grp * RPT, lbase = grp * kGS;
    auto lds_row = [](int r) { return (r / RPT) * kGS + r % RPT; };
    auto publish = [&](int c) {
        float *vc = S.vcol + (c & 1) * kVRows;
        double ss[4] = {0.0, 0.0, 0.0, 0.0};   // exact squares, four chains
        float x[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            x[i] = rbase + i >= c ? P[i] : 0.f;
            ss[i & 3] = __builtin_fma((double)x[i], (double)x[i], ss[i & 3]);
        }
#pragma unroll
        for (int i = 0; i < RPT; i += 4) *(f32x4 *)(vc + lbase + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
        const double alpha = sqrt(col_sum((ss[0] + ss[1]) + (ss[2] + ss[3])));
        if (grp == 0) {   // row c was stored by this wave: LDS operations of a wave are in order
            const double x0 = (double)vc[lds_row(c)];
            S.red[(c & 1) * 2] = alpha;
            S.red[(c & 1) * 2 + 1] = x0;
            vc[lds_row(c)] = (float)(x0 + (x0 >= 0.0 ? alpha : -alpha));
        }
    };
    if (k == 0) publish(0);
    for (int c = 0; c < w; ++c) {
        const int buf = c & 1;
        const float *vc = S.vcol + buf * kVRows;
        __syncthreads();   // column c published; Gs, tau and T of earlier columns visible
        const double alpha = S.red[buf * 2], x0 = S.red[buf * 2 + 1];
        const double sg = x0 >= 0.0 ? 1.0 : -1.0;
        const double tc = alpha == 0.0 ? 0.0 : 1.0 + fabs(x0) / alpha;
        const float inv = alpha == 0.0 ? 1.f : (float)(1.0 / (x0 + sg * alpha));
        // column c-1 of T: its Gram entries and tau became visible at the barrier above.  Entry
        // (k, c-1) is a sum over l = k .. c-2, split over the column's 8 threads (l = k + grp + 8 i)
        if (c >= 2) {   // uniform: every lane takes part in the shuffles
            double part = 0.0;
            if (k < c - 1)
                for (int l = k + grp; l < c - 1; l += 8) part += S.Td[k][l] * S.Gs[l][c - 1];
            const double sum = col_sum(part);
            if (grp == 0 && k < c - 1) S.Td[k][c - 1] = -S.tau[c - 1] * sum;
        }
        // v^T P_k = inv (x^T P_k) on this thread's rows, summed over the column's 8 threads
        float x[RPT];
#pragma unroll
        for (int i = 0; i < RPT; i += 4) {
            const f32x4 q = *(const f32x4 *)(vc + lbase + i);
            x[i] = q[0]; x[i + 1] = q[1]; x[i + 2] = q[2]; x[i + 3] = q[3];
        }
        float sd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) sd[i & 3] = __builtin_fmaf(x[i], P[i], sd[i & 3]);
        const double tot =
            col_sum((double)inv * (((double)sd[0] + (double)sd[1]) + ((double)sd[2] + (double)sd[3])));
        if (k > c && k < w) {
            const float a = (float)(tc * tot) * inv;   // P_k -= tc (v^T P_k) v
#pragma unroll
            for (int i = 0; i < RPT; ++i) P[i] = __builtin_fmaf(-a, x[i], P[i]);
            if (k == c + 1) publish(c + 1);
        } else if (k == c) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) P[i] = inv * x[i];   // v: 0 above row c
            if (grp == 0) {
                S.tau[c] = tc;
                S.Td[c][c] = tc;
                negf[c] = (alpha != 0.0 && sg > 0.0) ? 1 : 0;   // R_cc = -sg alpha < 0
            }
        } else if (k < c && grp == 0) {
            S.Gs[k][c] = tot;   // v_k^T v_c
        }
    }
    __syncthreads();
    if (w >= 2) {
        double part = 0.0;
        if (k < w - 1)
            for (int l = k + grp; l < w - 1; l += 8) part += S.Td[k][l] * S.Gs[l][w - 1];
        const double sum = col_sum(part);
        if (grp == 0 && k < w - 1) S.Td[k][w - 1] = -S.tau[w - 1] * sum;
    }
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- one wave applies a block reflector to a 32-column tile held in LDS ----------------------------
//   X[j0 + r, c0 + j] -= (V op(T) V^T X)[r, j],  r < rows, j < 32 (columns >= ncols are skipped)
// op(T) = T^T while factoring, T while forming Q.  W: this wave's 32 x 33 LDS scratch.  FLIP negates
// the stored column col where neg[col] is set.
template <bool TRANS_T, bool FLIP>
__device__ void wy_wave(float *X, int ldx, int ncols, int j0, int rows, int c0, const float (*Vs)[kPW + 1],
                        const float (*Ts)[kPW + 1], float (*W)[33], const int8_t *neg, int lane) {
    const int kr = lane >> 5, cc = lane & 31;
    const bool colok = c0 + cc < ncols;
    const int ccl = colok ? c0 + cc : 0;
    f32x16 acc = {};
    for (int kb = 0; kb < rows; kb += 16) {
        float a[8], bx[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = kb + 2 * u + kr;
            const bool ok = r < rows;
            const int rs = ok ? r : 0;
            const float av = Vs[rs][cc];
            const float xv = X[(int64_t)(j0 + rs) * ldx + ccl];
            a[u] = ok ? av : 0.f;
            bx[u] = (ok && colok) ? xv : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], bx[u], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) W[acc_row(r, lane)][acc_col(lane)] = acc[r];
    wave_sync_lds();
    f32x16 y = {};
#pragma unroll
    for (int kk = 0; kk < kPW; kk += 2) {
        const int k = kk + kr;
        const float a = TRANS_T ? Ts[k][cc] : Ts[cc][k];
        y = __builtin_amdgcn_mfma_f32_32x32x2f32(a, W[k][cc], y, 0, 0, 0);
    }
    wave_sync_lds();
#pragma unroll
    for (int r = 0; r < 16; ++r) W[acc_row(r, lane)][acc_col(lane)] = y[r];
    wave_sync_lds();
    const int col = c0 + acc_col(lane);
    const float sgn = (FLIP && colok && neg[col]) ? -1.f : 1.f;
    for (int r0 = 0; r0 < rows; r0 += 32) {
        f32x16 u = {};
#pragma unroll
        for (int kk = 0; kk < kPW; kk += 2) {
            const int k = kk + kr, rr = r0 + cc;
            const float a = rr < rows ? Vs[rr < rows ? rr : 0][k] : 0.f;
            u = __builtin_amdgcn_mfma_f32_32x32x2f32(a, W[k][cc], u, 0, 0, 0);
        }
        if (!colok) continue;
        float *xc = X + (int64_t)(j0 + r0) * ldx + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = r0 + acc_row(r, lane);
            if (row < rows) {
                const float v = xc[(int64_t)acc_row(r, lane) * ldx] - u[r];
                xc[(int64_t)acc_row(r, lane) * ldx] = FLIP ? sgn * v : v;
            }
        }
    }
}

// ---- nb <= 128: one workgroup per block, Z in LDS ----------------------------------------------------
struct BlockLds {
    size_t vs, ts, wsc, neg, zs, total;
    PanelLds pn;
};
__host__ __device__ inline BlockLds block_lds(int nb) {
    BlockLds L;
    size_t o = 0;
    L.vs = o; o += a16((size_t)nb * (kPW + 1) * 4);
    L.ts = o; o += a16((size_t)kPW * (kPW + 1) * 4);
    L.pn = panel_lds(nb, o);                    // panel scratch, reused as the waves' update scratch
    L.wsc = o;
    const size_t wend = o + a16((size_t)4 * 32 * 33 * 4);
    o = L.pn.total > wend ? L.pn.total : wend;
    L.neg = o; o += a16((size_t)nb);
    L.zs = o;  o += a16((size_t)nb * (nb + 1) * 4);
    L.total = o;
    return L;
}

// grid.x = blocks of the launch, block 256; RPT >= ceil(nb / 8).  T of panel p goes to Tq (workspace).
template <int RPT>
__global__ void __launch_bounds__(256) k_qr_block(int nb, int nblk, const float *Z_all, float *Tq_all, QrBlockOut t,
                                                  int info_value) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const BlockLds L = block_lds(nb);
    float(*Vs)[kPW + 1] = (float(*)[kPW + 1])(dsm + L.vs);
    float(*Ts)[kPW + 1] = (float(*)[kPW + 1])(dsm + L.ts);
    float(*Wsc)[32][33] = (float(*)[32][33])(dsm + L.wsc);
    int8_t *neg = (int8_t *)(dsm + L.neg);
    const PanelPtrs S = panel_ptrs(dsm, L.pn);
    const int ldz = nb + 1;
    float *Z = (float *)(dsm + L.zs);

    const int g = blockIdx.x;
    const int b = g % nblk, mat = g / nblk;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int k = tid >> 3, grp = tid & (kGroups - 1);   // tid = 8 k + grp
    const int npanel = (nb + kPW - 1) / kPW;
    const float *Zg = Z_all + (int64_t)g * nb * nb;
    float *Tq = Tq_all + (int64_t)g * npanel * kPW * kPW;
    for (int r = wv; r < nb; r += kQT / 64)
        for (int c = lane; c < nb; c += 64) Z[r * ldz + c] = Zg[(int64_t)r * nb + c];
    __syncthreads();

    for (int p = 0; p < npanel; ++p) {
        const int j0 = p * kPW, w = min(kPW, nb - j0), rows = nb - j0;
        float P[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = grp * RPT + i;
            P[i] = (k < w && r < rows) ? Z[(int64_t)(j0 + r) * ldz + j0 + k] : 0.f;
        }
        factor_panel<RPT>(P, w, rows, k, grp, S, neg + j0);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = grp * RPT + i;
            if (r < rows) {
                Vs[r][k] = k < w ? P[i] : 0.f;
                if (k < w) Z[(int64_t)(j0 + r) * ldz + j0 + k] = P[i];
            }
        }
        __syncthreads();
        for (int e = tid; e < kPW * kPW; e += kQT) {
            const int i = e / kPW, j = e % kPW;
            const float tv = (i <= j && j < w) ? (float)S.Td[i][j] : 0.f;
            Ts[i][j] = tv;
            Tq[(int64_t)p * kPW * kPW + e] = tv;
        }
        __syncthreads();
        const int first = j0 + w;
        const int ntiles = (nb - first + 31) / 32;
        for (int tile = wv; tile < ntiles; tile += 4)
            wy_wave<true, false>(Z, ldz, nb, j0, rows, first + 32 * tile, Vs, Ts, Wsc[wv], neg, lane);
        __syncthreads();
    }

    // Q formed in place over Z (as LAPACK's orgqr does): panels last to first.  When panel p comes,
    // columns >= j0 + w already hold Q's columns as the later panels left them (their rows < j0 + w
    // untouched so far), columns j0 .. j0 + w - 1 still hold V_p, and columns < j0 the earlier V.
    // V_p goes to Vs, its columns restart as identity columns, the R entries in rows j0 .. j0 + w - 1
    // right of the panel become the zeros Q has there before H_p, and H_p = I - V_p T_p V_p^T is
    // applied to rows and columns >= j0.
    for (int p = npanel - 1; p >= 0; --p) {
        const int j0 = p * kPW, w = min(kPW, nb - j0), rows = nb - j0;
        for (int e = tid; e < rows * kPW; e += kQT) {
            const int r = e / kPW, c = e % kPW;
            Vs[r][c] = c < w ? Z[(int64_t)(j0 + r) * ldz + j0 + c] : 0.f;
        }
        for (int e = tid; e < kPW * kPW; e += kQT) Ts[e / kPW][e % kPW] = Tq[(int64_t)p * kPW * kPW + e];
        __syncthreads();   // V_p staged: its columns can be overwritten
        for (int e = tid; e < nb * w; e += kQT) {   // the panel's columns: identity columns
            const int r = e / w, c = e - r * w;
            Z[r * ldz + j0 + c] = r == j0 + c ? 1.f : 0.f;
        }
        for (int e = tid; e < w * (nb - j0 - w); e += kQT) {   // its rows right of the panel: zero
            const int r = e / (nb - j0 - w), c = e - r * (nb - j0 - w);
            Z[(j0 + r) * ldz + j0 + w + c] = 0.f;
        }
        __syncthreads();
        const int ntiles = (nb - j0 + 31) / 32;
        for (int tile = wv; tile < ntiles; tile += 4) {
            if (p == 0) wy_wave<false, true>(Z, ldz, nb, j0, rows, j0 + 32 * tile, Vs, Ts, Wsc[wv], neg, lane);
            else wy_wave<false, false>(Z, ldz, nb, j0, rows, j0 + 32 * tile, Vs, Ts, Wsc[wv], neg, lane);
        }
        __syncthreads();
    }
    float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    for (int r = wv; r < nb; r += kQT / 64)
        for (int c = lane; c < nb; c += 64) Q[(int64_t)r * nb + c] = Z[r * ldz + c];
    if (tid == 0 && info_value > 0 && t.info[mat]) t.info[mat][b] = info_value;
}

// ---- nb > 128: panel launch ------------------------------------------------------------------------
// grid.x = blocks, block 256.  Writes V into Z's panel columns, T (fp32) to Tq, diag(R) signs to negs.
template <int RPT>
__global__ void __launch_bounds__(256) k_qr_panel(int nb, int p, float *Z_all, float *Tq_all, int8_t *neg_all) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const PanelLds L = panel_lds(nb, 0);
    const PanelPtrs S = panel_ptrs(dsm, L);
    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int k = tid >> 3, grp = tid & (kGroups - 1);   // tid = 8 k + grp
    const int npanel = (nb + kPW - 1) / kPW;
    const int j0 = p * kPW, w = min(kPW, nb - j0), rows = nb - j0;
    float *Z = Z_all + (int64_t)g * nb * nb;
    float *Tq = Tq_all + ((int64_t)g * npanel + p) * kPW * kPW;
    float P[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = grp * RPT + i;
        P[i] = (k < w && r < rows) ? Z[(int64_t)(j0 + r) * nb + j0 + k] : 0.f;
    }
    factor_panel<RPT>(P, w, rows, k, grp, S, neg_all + (int64_t)g * nb + j0);
    if (k < w) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = grp * RPT + i;
            if (r < rows) Z[(int64_t)(j0 + r) * nb + j0 + k] = P[i];
        }
    }
    __syncthreads();
    for (int e = tid; e < kPW * kPW; e += kQT) {
        const int i = e / kPW, j = e % kPW;
        Tq[e] = (i <= j && j < w) ? (float)S.Td[i][j] : 0.f;
    }
}

// ---- nb > 128: apply a panel's block reflector -------------------------------------------------------
// grid = (64-column tiles, blocks), block 256.  Wave (kp, h): column half h of the tile, row half kp.
// A wave's rows are processed in 32-row chunks; chunk rows are fed to the V^T X products in the
// order of the MFMA accumulator layout (k-step s of half-wave q uses row 8 (s/4) + 4 q + s % 4), so
// the chunk loaded for those products is already laid out as the X - V Y result.
// FACTOR: X = Z (columns after the panel), op(T) = T^T.  Otherwise X = Q (columns from the panel
// start), op(T) = T, and with FLIP (first panel) the columns whose R_cc < 0 are negated.
// Vs[r][c] = V[r][c] for r < rows, c < 32 (zero for c >= w) from Z's panel columns, and zero rows
// from rows up to the next multiple of 32.  8 threads per row, eight rows per thread in flight.
template <int CH, int NT = kQT>
__device__ __forceinline__ void stage_v(float (*Vs)[kPW + 1], const float *Z, int nb, int j0, int w, int rows, int tid) {
    constexpr int kPasses = 2 * CH;   // NT / 8 rows per pass
    const int c4 = 4 * (tid & 7), r0 = tid >> 3;
    const int rpad = (rows + 31) & ~31;
    const bool vec = (nb & 3) == 0 && c4 + 4 <= w;
    const float *Zp = Z + (int64_t)j0 * nb + j0;
#pragma unroll
    for (int b0 = 0; b0 < kPasses; b0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = r0 + (NT / 8) * (b0 + i);
            const bool ok = b0 + i < kPasses && r < rows;
            const float *src = Zp + (ok ? r : 0) * nb + c4;
            if (vec) {
                v[i] = *(const f32x4 *)src;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[i][q] = c4 + q < w ? src[q] : 0.f;
            }
            if (!ok) v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = r0 + (NT / 8) * (b0 + i);
            if (b0 + i < kPasses && r < rpad) {
#pragma unroll
                for (int q = 0; q < 4; ++q) Vs[r][c4 + q] = v[i][q];
            }
        }
    }
}

struct ApplyLds {
    size_t vs, ts, wp, total;
};
__host__ __device__ inline ApplyLds apply_lds(int nb) {
    ApplyLds L;
    size_t o = 0;
    L.vs = o; o += a16((size_t)((nb + 31) & ~31) * (kPW + 1) * 4);
    L.ts = o; o += a16((size_t)kPW * (kPW + 1) * 4);
    L.wp = o; o += a16((size_t)2 * 2 * 32 * 33 * 4);   // [row half][column half]
    L.total = o;
    return L;
}

// TWO (factoring only): apply panel p's block reflector and then panel p + 1's to the columns from
// 32 (p + 2) on, reading and writing the tile once for both; the columns of panel p + 1 get panel
// p's reflector alone, from a launch limited by cend (columns from cend on are left alone), before
// panel p + 1 is factored.  Each column sees the same products in the same order either way.
template <int CH, bool FACTOR, bool FLIP, bool TWO = false>
__global__ void __launch_bounds__(256) k_qr_apply(int nb, int nblk, int p, const float *Z_all, const float *Tq_all,
                                                  const int8_t *neg_all, QrBlockOut t, int info_value,
                                                  int cend = 1 << 30) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const ApplyLds L = apply_lds(nb);
    float(*Vs)[kPW + 1] = (float(*)[kPW + 1])(dsm + L.vs);
    float(*Ts)[kPW + 1] = (float(*)[kPW + 1])(dsm + L.ts);
    float(*Wp)[2][32][33] = (float(*)[2][32][33])(dsm + L.wp);
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int h = wv & 1, kp = wv >> 1;
    const int kr = lane >> 5, cc = lane & 31;
    const int npanel = (nb + kPW - 1) / kPW;
    const int j0 = p * kPW, w = min(kPW, nb - j0), rows = nb - j0;
    const float *Z = Z_all + (int64_t)g * nb * nb;
    float *X = FACTOR ? (float *)Z_all + (int64_t)g * nb * nb : t.Q[mat] + (int64_t)b * nb * nb;
    const int first = FACTOR ? (TWO ? j0 + 2 * kPW : j0 + w) : j0;
    const int c0 = first + blockIdx.x * 64 + 32 * h;
    const bool colok = c0 + cc < nb && c0 + cc < cend;
    const int ccl = colok ? c0 + cc : 0;
    // rows of this wave: [rb, re), at most CH chunks of 32
    const int half = ((rows + 63) / 64) * 32;
    const int rb = kp ? half : 0, re = kp ? rows : (half < rows ? half : rows);
    // element (row, col) of the tile lives at Xr[row * nb + col]; this lane's rows within a chunk are
    // 4 kr + {0, 1, 2, 3, 8, ..., 27}: offsets from one 32-bit lane offset
    float *Xr = X + (int64_t)j0 * nb;
    const unsigned lo = (unsigned)((rb + 4 * kr) * nb + ccl);
    const unsigned unb = (unsigned)nb;
    // this wave's share of the tile, accumulator layout; rows >= re and columns >= nb read as 0
    f32x16 x[CH];
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
        const int r0 = rb + 32 * ch;
        if (r0 + 32 <= re && colok) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[ch][r] = Xr[lo + (unsigned)(32 * ch + 8 * (r >> 2) + (r & 3)) * unb];
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = r0 + acc_row(r, lane);
                const bool ok = row < re && colok;
                const float v = Xr[ok ? lo + (unsigned)(32 * ch + 8 * (r >> 2) + (r & 3)) * unb : 0u];
                x[ch][r] = ok ? v : 0.f;
            }
        }
    }
    // V (zero rows up to a multiple of 32) and T
    stage_v<CH>(Vs, Z, nb, j0, w, rows, tid);
    const float *Tq = Tq_all + ((int64_t)g * npanel + p) * kPW * kPW;
    {
        float tv[kPW * kPW / kQT];
#pragma unroll
        for (int i = 0; i < kPW * kPW / kQT; ++i) tv[i] = Tq[tid + kQT * i];
#pragma unroll
        for (int i = 0; i < kPW * kPW / kQT; ++i) Ts[(tid + kQT * i) / kPW][(tid + kQT * i) % kPW] = tv[i];
    }
    __syncthreads();
    // W partial = V[this wave's rows]^T X (rows past `rows` have V = 0)
    f32x16 acc = {};
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
        const int r0 = rb + 32 * ch;
        if (r0 >= re) break;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const float a = Vs[r0 + 8 * (s >> 2) + 4 * kr + (s & 3)][cc];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, x[ch][s], acc, 0, 0, 0);
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Wp[kp][h][acc_row(r, lane)][acc_col(lane)] = acc[r];
    __syncthreads();
    // Y = op(T) (W_0 + W_1), computed by both waves of the column half
    f32x16 y = {};
#pragma unroll
    for (int kk = 0; kk < kPW; kk += 2) {
        const int kx = kk + kr;
        const float a = FACTOR ? Ts[kx][cc] : Ts[cc][kx];
        y = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Wp[0][h][kx][cc] + Wp[1][h][kx][cc], y, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) Wp[kp][h][acc_row(r, lane)][acc_col(lane)] = y[r];
    wave_sync_lds();
    float yb[kPW / 2];   // B operands of the V Y products, the same for every chunk
#pragma unroll
    for (int kk = 0; kk < kPW; kk += 2) yb[kk / 2] = Wp[kp][h][kk + kr][cc];
    // X -= V Y on this wave's rows (kept in registers when panel p + 1 follows)
    const float sgn = (FLIP && colok && neg_all[(int64_t)g * nb + ccl]) ? -1.f : 1.f;
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
        const int r0 = rb + 32 * ch;
        if (r0 >= re) break;
        f32x16 u = {};
#pragma unroll
        for (int kk = 0; kk < kPW; kk += 2)
            u = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[r0 + cc][kk + kr], yb[kk / 2], u, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) x[ch][r] -= u[r];
    }
    if constexpr (TWO) {
        // panel p + 1: its rows start 32 rows down the tile, so it acts on chunks r0 >= 32
        const int j1 = j0 + kPW, w1 = min(kPW, nb - j1), rows1 = nb - j1;
        __syncthreads();   // panel p's readers of Vs, Ts and Wp are done
        stage_v<CH>(Vs, Z, nb, j1, w1, rows1, tid);
        {
            const float *Tq1 = Tq_all + ((int64_t)g * npanel + p + 1) * kPW * kPW;
            float tv[kPW * kPW / kQT];
#pragma unroll
            for (int i = 0; i < kPW * kPW / kQT; ++i) tv[i] = Tq1[tid + kQT * i];
#pragma unroll
            for (int i = 0; i < kPW * kPW / kQT; ++i) Ts[(tid + kQT * i) / kPW][(tid + kQT * i) % kPW] = tv[i];
        }
        __syncthreads();
        f32x16 acc1 = {};
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int r0 = rb + 32 * ch;
            if (r0 >= re) break;
            if (r0 < kPW) continue;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float a = Vs[r0 - kPW + 8 * (s >> 2) + 4 * kr + (s & 3)][cc];
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, x[ch][s], acc1, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Wp[kp][h][acc_row(r, lane)][acc_col(lane)] = acc1[r];
        __syncthreads();
        f32x16 y1 = {};
#pragma unroll
        for (int kk = 0; kk < kPW; kk += 2) {
            const int kx = kk + kr;
            y1 = __builtin_amdgcn_mfma_f32_32x32x2f32(Ts[kx][cc], Wp[0][h][kx][cc] + Wp[1][h][kx][cc], y1, 0, 0, 0);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) Wp[kp][h][acc_row(r, lane)][acc_col(lane)] = y1[r];
        wave_sync_lds();
#pragma unroll
        for (int kk = 0; kk < kPW; kk += 2) yb[kk / 2] = Wp[kp][h][kk + kr][cc];
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int r0 = rb + 32 * ch;
            if (r0 >= re) break;
            if (r0 < kPW) continue;
            f32x16 u = {};
#pragma unroll
            for (int kk = 0; kk < kPW; kk += 2) {
                const int rr = r0 - kPW + cc;
                u = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[rr][kk + kr], yb[kk / 2], u, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) x[ch][r] -= u[r];
        }
    }
    if (colok) {
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int r0 = rb + 32 * ch;
            if (r0 >= re) break;
            if (r0 + 32 <= re) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = x[ch][r];
                    Xr[lo + (unsigned)(32 * ch + 8 * (r >> 2) + (r & 3)) * unb] = FLIP ? sgn * v : v;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (r0 + acc_row(r, lane) < re) {
                        const float v = x[ch][r];
                        Xr[lo + (unsigned)(32 * ch + 8 * (r >> 2) + (r & 3)) * unb] = FLIP ? sgn * v : v;
                    }
                }
            }
        }
    }
    if (FLIP && blockIdx.x == 0 && tid == 0 && info_value > 0 && t.info[mat]) t.info[mat][b] = info_value;
}

// ---- nb > 128: formation of Q in one launch ---------------------------------------------------------
// A workgroup owns a 64-column tile of Q_b over all nb rows and keeps it in registers (accumulator
// layout, as in k_qr_apply) from the identity to the final store.  Its 8 waves split the tile into
// two column halves by four row sets, so a wave holds at most 4 x 32 rows and two waves share each
// SIMD.  It applies the block reflectors
// I - V_p T_p V_p^T for p = min(npanel - 1, last column / 32) down to 0 (panels starting past the
// tile's last column leave its identity columns unchanged), each with V_p and T_p staged in LDS, and
// stores the tile once with the columns whose R_cc < 0 negated.  Wave (kp, h): column half h, the
// 32-row chunks kp, kp + 4, kp + 8, ... (interleaved, so that the chunks a panel touches stay spread
// over the waves); chunks lying wholly above a panel's first row are skipped (V = 0).
// grid = (ceil(nb / 64) tiles, blocks), block 512.  CH = ceil(ceil(nb / 32) / 4).
constexpr int kFP = 4;                 // formation: row parts
constexpr int kFT = 2 * 64 * kFP;      // formation: threads per workgroup
__host__ __device__ inline ApplyLds form_lds(int nb) {
    ApplyLds L;
    size_t o = 0;
    L.vs = o; o += a16((size_t)((nb + 31) & ~31) * (kPW + 1) * 4);
    L.ts = o; o += a16((size_t)kPW * (kPW + 1) * 4);
    L.wp = o; o += a16((size_t)kFP * 2 * 32 * 33 * 4);   // [row part][column half]
    L.total = o;
    return L;
}
// stage_v in two halves, so that a panel's V rows can be loaded while the previous panel's products
// run: load_v_regs reads the rows (zeros past `rows` and past the panel width) into registers,
// store_v_regs writes them to Vs (rows up to the next multiple of 32).  2 CH passes of NT / 8 rows.
template <int CH, int NT>
__device__ __forceinline__ void load_v_regs(f32x4 (&v)[2 * CH], const float *Z, int nb, int j0, int w, int rows,
                                            int tid) {
    const int c4 = 4 * (tid & 7), r0 = tid >> 3;
    const bool vec = (nb & 3) == 0 && c4 + 4 <= w;
    const float *Zp = Z + (int64_t)j0 * nb + j0;
#pragma unroll
    for (int i = 0; i < 2 * CH; ++i) {
        const int r = r0 + (NT / 8) * i;
        const bool ok = r < rows;
        const float *src = Zp + (ok ? r : 0) * nb + c4;
        if (vec) {
            v[i] = *(const f32x4 *)src;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[i][q] = c4 + q < w ? src[q] : 0.f;
        }
        if (!ok) v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}
template <int CH, int NT>
__device__ __forceinline__ void store_v_regs(float (*Vs)[kPW + 1], const f32x4 (&v)[2 * CH], int rows, int tid) {
    const int c4 = 4 * (tid & 7), r0 = tid >> 3;
    const int rpad = (rows + 31) & ~31;
#pragma unroll
    for (int i = 0; i < 2 * CH; ++i) {
        const int r = r0 + (NT / 8) * i;
        if (r < rpad) {
#pragma unroll
            for (int q = 0; q < 4; ++q) Vs[r][c4 + q] = v[i][q];
        }
    }
}

template <int CH>
__global__ void __launch_bounds__(kFT) k_qr_form(int nb, int nblk, const float *Z_all, const float *Tq_all,
                                                 const int8_t *neg_all, QrBlockOut t, int info_value) {
    extern __shared__ __align__(16) unsigned char dsm[];
    const ApplyLds L = form_lds(nb);
    float(*Vs)[kPW + 1] = (float(*)[kPW + 1])(dsm + L.vs);
    float(*Ts)[kPW + 1] = (float(*)[kPW + 1])(dsm + L.ts);
    float(*Wp)[2][32][33] = (float(*)[2][32][33])(dsm + L.wp);
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int h = wv & 1, kp = wv >> 1;
    const int kr = lane >> 5, cc = lane & 31;
    const int npanel = (nb + kPW - 1) / kPW;
    const float *Z = Z_all + (int64_t)g * nb * nb;
    float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    const int c0 = blockIdx.x * 64 + 32 * h;
    const bool colok = c0 + cc < nb;
    const int ccl = colok ? c0 + cc : 0;
    // this wave's 32-row chunks: 32 (kp + kFP ch), interleaved over the row sets so that the chunks
    // at or below a panel's first row stay evenly spread as the panels advance
    auto chunk_row = [&](int ch) { return 32 * (kp + kFP * ch); };
    const unsigned lo = (unsigned)((32 * kp + 4 * kr) * nb + ccl);
    const unsigned unb = (unsigned)nb;
    // the identity columns of the tile
    f32x16 x[CH];
#pragma unroll
    for (int ch = 0; ch < CH; ++ch)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = chunk_row(ch) + acc_row(r, lane);
            x[ch][r] = (colok && row < nb && row == ccl) ? 1.f : 0.f;
        }
    const int plast = (blockIdx.x * 64 + 63) / kPW < npanel - 1 ? (blockIdx.x * 64 + 63) / kPW : npanel - 1;
    // panel p's V rows and T, loaded one panel ahead into registers
    static_assert(2 * CH * (kFT / 8) >= 32 * kFP * CH, "the V passes cover the row parts");
    f32x4 vpre[2 * CH];
    float tpre[kPW * kPW / kFT];
    auto fetch = [&](int p) {
        const int j0 = p * kPW;
        load_v_regs<CH, kFT>(vpre, Z, nb, j0, min(kPW, nb - j0), nb - j0, tid);
        const float *Tq = Tq_all + ((int64_t)g * npanel + p) * kPW * kPW;
#pragma unroll
        for (int i = 0; i < kPW * kPW / kFT; ++i) tpre[i] = Tq[tid + kFT * i];
    };
    fetch(plast);
    for (int p = plast; p >= 0; --p) {
        const int j0 = p * kPW, rows = nb - j0;
        __syncthreads();   // the last panel's readers of Vs, Ts and Wp are done
        store_v_regs<CH, kFT>(Vs, vpre, rows, tid);
#pragma unroll
        for (int i = 0; i < kPW * kPW / kFT; ++i) Ts[(tid + kFT * i) / kPW][(tid + kFT * i) % kPW] = tpre[i];
        if (p > 0) fetch(p - 1);
        __syncthreads();
        // W partial = V^T X over this wave's chunks at rows >= j0 (chunks are 32-aligned, as is j0)
        f32x16 acc = {};
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int r0 = chunk_row(ch);
            if (r0 >= nb) break;
            if (r0 < j0) continue;
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) {
                const float a = Vs[r0 - j0 + 8 * (s2 >> 2) + 4 * kr + (s2 & 3)][cc];
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, x[ch][s2], acc, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Wp[kp][h][acc_row(r, lane)][acc_col(lane)] = acc[r];
        __syncthreads();
        // Y = T (W_0 + W_1 + W_2 + W_3)
        f32x16 y = {};
#pragma unroll
        for (int kk = 0; kk < kPW; kk += 2) {
            const int kx = kk + kr;
            float wsum = Wp[0][h][kx][cc];
#pragma unroll
            for (int q = 1; q < kFP; ++q) wsum += Wp[q][h][kx][cc];
            y = __builtin_amdgcn_mfma_f32_32x32x2f32(Ts[cc][kx], wsum, y, 0, 0, 0);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) Wp[kp][h][acc_row(r, lane)][acc_col(lane)] = y[r];
        wave_sync_lds();
        float yb[kPW / 2];
#pragma unroll
        for (int kk = 0; kk < kPW; kk += 2) yb[kk / 2] = Wp[kp][h][kk + kr][cc];
        // X -= V Y on this wave's chunks at rows >= j0
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int r0 = chunk_row(ch);
            if (r0 >= nb) break;
            if (r0 < j0) continue;
            f32x16 u = {};
#pragma unroll
            for (int kk = 0; kk < kPW; kk += 2)
                u = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[r0 - j0 + cc][kk + kr], yb[kk / 2], u, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) x[ch][r] -= u[r];
        }
    }
    // store, negating the columns whose R_cc < 0
    if (colok) {
        const float sgn = neg_all[(int64_t)g * nb + ccl] ? -1.f : 1.f;
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int r0 = chunk_row(ch);
            if (r0 >= nb) break;
            const unsigned cb = lo + (unsigned)(32 * kFP * ch) * unb;
            if (r0 + 32 <= nb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Q[cb + (unsigned)(8 * (r >> 2) + (r & 3)) * unb] = sgn * x[ch][r];
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (r0 + acc_row(r, lane) < nb) Q[cb + (unsigned)(8 * (r >> 2) + (r & 3)) * unb] = sgn * x[ch][r];
            }
        }
    }
    if (blockIdx.x == 0 && tid == 0 && info_value > 0 && t.info[mat]) t.info[mat][b] = info_value;
}


template <int RPT>
hipError_t launch_block(int nb, int nblk, int nblocks, const float *Z, float *tq, const QrBlockOut &o, int infov,
                        hipStream_t s) {
    const size_t sh = block_lds(nb).total;
    (void)hipFuncSetAttribute((const void *)k_qr_block<RPT>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
    DOBB_LAUNCH("qr_block", s, (k_qr_block<RPT>), dim3((unsigned)nblocks), dim3(kQT), sh, nb, nblk, Z, tq, o, infov);
    return hipGetLastError();
}

template <int RPT, int CH>
hipError_t launch_panels(int nb, int nblk, int nblocks, float *Z, float *tq, int8_t *negs, const QrBlockOut &o,
                         int infov, hipStream_t s) {
    const size_t ps = panel_lds(nb, 0).total;
    const size_t as = apply_lds(nb).total;
    (void)hipFuncSetAttribute((const void *)k_qr_panel<RPT>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ps);
    (void)hipFuncSetAttribute((const void *)k_qr_panel<8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ps);
    (void)hipFuncSetAttribute((const void *)k_qr_panel<16>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ps);
    (void)hipFuncSetAttribute((const void *)k_qr_panel<32>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ps);
    (void)hipFuncSetAttribute((const void *)k_qr_apply<CH, true, false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)as);
    (void)hipFuncSetAttribute((const void *)k_qr_apply<CH, true, false, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)as);
    const int npanel = (nb + kPW - 1) / kPW;
    auto factor = [&](int p) {
        const int rows = nb - p * kPW;   // rows per thread: ceil(rows / 8), rounded up to a template size
        if (rows <= 64 && RPT > 8)
            DOBB_LAUNCH("qr_panel", s, (k_qr_panel<8>), dim3((unsigned)nblocks), dim3(kQT), ps, nb, p, Z, tq, negs);
        else if (rows <= 128 && RPT > 16)
            DOBB_LAUNCH("qr_panel", s, (k_qr_panel<16>), dim3((unsigned)nblocks), dim3(kQT), ps, nb, p, Z, tq, negs);
        else if (rows <= 256 && RPT > 32)
            DOBB_LAUNCH("qr_panel", s, (k_qr_panel<32>), dim3((unsigned)nblocks), dim3(kQT), ps, nb, p, Z, tq, negs);
        else
            DOBB_LAUNCH("qr_panel", s, (k_qr_panel<RPT>), dim3((unsigned)nblocks), dim3(kQT), ps, nb, p, Z, tq, negs);
    };
    // panels in pairs: panel p's reflector goes to panel p + 1's columns alone, panel p + 1 is
    // factored, and both reflectors then go to the remaining columns in one pass (the trailing part
    // of the block is read and written once per two panels); an odd last panel updates alone
    for (int p = 0; p < npanel;) {
        factor(p);
        const int j0 = p * kPW;
        if (p + 1 < npanel) {
            DOBB_LAUNCH("qr_update", s, (k_qr_apply<CH, true, false>), dim3(1u, (unsigned)nblocks), dim3(kQT), as, nb, nblk,
                        p, (const float *)Z, (const float *)tq, (const int8_t *)negs, o, 0, j0 + 2 * kPW);
            factor(p + 1);
            const int ntiles = (nb - (j0 + 2 * kPW) + 63) / 64;
            if (ntiles > 0)
                DOBB_LAUNCH("qr_update", s, (k_qr_apply<CH, true, false, true>), dim3((unsigned)ntiles, (unsigned)nblocks),
                            dim3(kQT), as, nb, nblk, p, (const float *)Z, (const float *)tq, (const int8_t *)negs, o, 0,
                            1 << 30);
            p += 2;
        } else {
            const int first = j0 + (nb - j0 < kPW ? nb - j0 : kPW);
            const int ntiles = (nb - first + 63) / 64;
            if (ntiles > 0)
                DOBB_LAUNCH("qr_update", s, (k_qr_apply<CH, true, false>), dim3((unsigned)ntiles, (unsigned)nblocks),
                            dim3(kQT), as, nb, nblk, p, (const float *)Z, (const float *)tq, (const int8_t *)negs, o, 0,
                            1 << 30);
            p += 1;
        }
    }
    // formation: each wave ceil(ceil(nb / 32) / 4) chunks of 32 rows, i.e. CH / 2
    const size_t fs = form_lds(nb).total;
    (void)hipFuncSetAttribute((const void *)k_qr_form<CH / 2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)fs);
    DOBB_LAUNCH("qr_form", s, (k_qr_form<CH / 2>), dim3((unsigned)((nb + 63) / 64), (unsigned)nblocks), dim3(kFT), fs,
                nb, nblk, (const float *)Z, (const float *)tq, (const int8_t *)negs, o, infov);
    return hipGetLastError();
}

}  // namespace

bool qr_block_supported(int64_t nb) { return nb >= 1 && nb <= 512; }

hipError_t launch_qr_block(int nb, int nblk, int cnt, float *Z, float *tq, int8_t *negs, float *const *Q,
                           int32_t *const *info, int info_value, hipStream_t s) {
    QrBlockOut o{};
    for (int i = 0; i < cnt; ++i) { o.Q[i] = Q[i]; o.info[i] = info ? info[i] : nullptr; }
    const int nblocks = nblk * cnt;
    if (nb <= 128 && (int64_t)block_lds(nb).total <= max_lds_bytes()) {
        if (nb <= 64) return launch_block<8>(nb, nblk, nblocks, Z, tq, o, info_value, s);
        return launch_block<16>(nb, nblk, nblocks, Z, tq, o, info_value, s);
    }
    // panel rows per thread: ceil(nb / 8); 32-row chunks per apply wave: ceil(nb / 64)
    if (nb <= 128) return launch_panels<16, 2>(nb, nblk, nblocks, Z, tq, negs, o, info_value, s);
    if (nb <= 256) return launch_panels<32, 4>(nb, nblk, nblocks, Z, tq, negs, o, info_value, s);
    return launch_panels<64, 8>(nb, nblk, nblocks, Z, tq, negs, o, info_value, s);
}

}  // namespace dobb
