// The Dobb step (sign normalisation) with fp32-accurate products on bf16 matrix cores.
//
// Dobb paper (arXiv 2610.39412): abstract (project momentum into the block bases, sign-normalise,
// reconstruct), Table 9 (update scale), Table 21 note (decoupled weight decay), Table 19 (Nesterov).
//
// gfx950 has no fp32-input fast MFMA, so fp32 operands are split into bf16 parts:
//   x = x_h + x_m + x_l,  x_h = bf16(x), x_m = bf16(x - x_h), x_l = bf16(x - x_h - x_m),
// each subtraction exact in fp32, the remainder below 2^-26 |x|.  Products of bf16 parts are exact
// in fp32 and accumulate in fp32.
//   projection     C = P Q with P, Q split three ways: the six products of order <= 2
//                  (hh, hm, mh, hl, mm, lh); the dropped terms are O(2^-26) of |P||Q|.
//   reconstruction U = S Q^T with S in {-1, 0, +1} exact in fp16 and Q (entries in [-1, 1]) split into
//                  two fp16 parts (remainder below 2^-22): two products (S Qh, S Ql).
// Kernels (one launch each per group of equally shaped matrices, nb <= 512):
//   k_split_q      Q_b -> fp16 hi/lo planes of Q_b (for U), bf16 h/m/l planes of Q_b^T (for C)
//   k_proj_bf16    M <- mu M + G fused; C = P Q (P = M or G + mu M); S = sign(C) as int8 codes
//   k_recon_bf16   U = S Q^T;  W <- W - lr (s U + wd W)
// A workgroup owns 128 rows x the whole block width, so it writes its rows of M exactly once.
// Signs travel from the projection to the reconstruction as one byte each: the high byte of the
// fp16 value (+1 -> 0x3c, -1 -> 0xbc, 0 -> 0x00, NaN -> 0x7e), so a byte permute rebuilds fp16.
// Workgroup ids are renumbered so the row tiles of one block run on one XCD and share Q_b in L2.
#include "dobb_internal.h"

namespace dobb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kKS = 16;        // k per MFMA step

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// split v into three bf16 parts (v_cvt_pk_bf16_f32 rounds to nearest even; each residual is exact)
__device__ __forceinline__ void split3(float v, uint16_t &h, uint16_t &m, uint16_t &l) {
    h = bf16_bits(v);
    const float r1 = v - bf16_to_f32(h);
    m = bf16_bits(r1);
    const float r2 = r1 - bf16_to_f32(m);
    l = bf16_bits(r2);
}

struct SplitTable {
    const float *Q[kMaxMats];
    uint16_t *planes[kMaxMats];  // 5 planes of B x nb x ldp: natural fp16 hi, lo; transposed bf16 h, m, l
};

// Q entries lie in [-1, 1]: two fp16 parts keep ~22 bits, the remainder is below 2^-22 in absolute terms
__device__ __forceinline__ void split2h(float v, uint16_t &h, uint16_t &l) {
    const _Float16 a = (_Float16)v;
    h = __builtin_bit_cast(uint16_t, a);
    l = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)a));
}

__device__ __forceinline__ uint8_t sign_f16_hi(float c) {
    return c > 0.f ? (uint8_t)0x3c : c < 0.f ? (uint8_t)0xbc : c == 0.f ? (uint8_t)0 : (uint8_t)0x7e;
}

// grid = (tiles^2 over nb x ldp, blocks * matrices), block 256 (32 x 8)
__global__ void __launch_bounds__(256) k_split_q(int nb, int ldp, int nblk, SplitTable t) {
    __shared__ float tile[32][33];
    const int g = blockIdx.y;
    const int b = g % nblk, mat = g / nblk;
    const int tpr = (ldp + 31) / 32;
    const int ti = blockIdx.x / tpr, tj = blockIdx.x % tpr;
    const float *Q = t.Q[mat] + (int64_t)b * nb * nb;
    const int64_t plane = (int64_t)nblk * nb * ldp;
    uint16_t *P = t.planes[mat] + (int64_t)b * nb * ldp;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int y = ty; y < 32; y += 8) {
        const int r = ti * 32 + y, c = tj * 32 + tx;
        tile[y][tx] = (r < nb && c < nb) ? Q[(int64_t)r * nb + c] : 0.f;
    }
    __syncthreads();
    for (int y = ty; y < 32; y += 8) {
        // natural: row r = ti*32 + y, column c = tj*32 + tx (c < ldp)
        int r = ti * 32 + y, c = tj * 32 + tx;
        if (r < nb && c < ldp) {
            uint16_t h, l;
            split2h(tile[y][tx], h, l);
            const int64_t e = (int64_t)r * ldp + c;
            P[e] = h; P[plane + e] = l;
        }
        // transposed: row c' = tj*32 + y holds column c' of Q, entries k = ti*32 + tx
        r = tj * 32 + y; c = ti * 32 + tx;
        if (r < nb && c < ldp) {
            uint16_t h, m, l;
            split3(tile[tx][y], h, m, l);
            const int64_t e = (int64_t)r * ldp + c;
            P[2 * plane + e] = h; P[3 * plane + e] = m; P[4 * plane + e] = l;
        }
    }
}

// ---- GEMM kernels ----------------------------------------------------------------------------
// A workgroup of 8 waves owns 128 rows x the whole block width.  Waves form RW = 8/CW row groups of
// 32*RT rows (RT = CW/2 row tiles of 32) and CW column groups; column group cg owns the 32-column
// chunks cg, cg + CW, cg + 2 CW, ... (at most NCW of them).  Each 16-deep k-step stages, in LDS:
//   A: the left operand for all 128 rows (the split of P = M or G + mu M for the projection, the
//      sign codes for the reconstruction), [plane][row][k];
//   B: the right operand for all columns, [plane][column][k], 16-byte pieces.
// LDS is double buffered: the global loads of step s+1 are issued before the MFMAs of step s and
// written to the other buffer after them, so each step has one barrier.
constexpr int kThreads = 512, kRows = 128, kWavesPerWg = 8;
constexpr int kRowLd = kKS + 8;  // bf16 per staged row (16 k + 8 pad = 48 bytes)

template <int CW, int NCW>
struct Cfg {
    static constexpr int RT = CW / 2;                 // row tiles per wave
    static constexpr int kCols = 32 * CW * NCW;       // staged columns
    static constexpr int kBPieces = 3 * kCols * 2;    // 16-byte pieces of B per k-step
    static constexpr int kBPer = (kBPieces + kThreads - 1) / kThreads;
    static constexpr int kAElems = 3 * kRows * kRowLd;  // bf16 per A buffer (3 planes)
};
// bf16 per B buffer (3 planes of ncols = 32 * chunks staged columns)
__host__ __device__ inline int b_elems(int ncols) { return 3 * ncols * kRowLd; }

template <int NPL, int COLS>
struct BStage {  // right operand pieces for one k-step
    static constexpr int kPieces = NPL * COLS * 2;
    static constexpr int kPer = (kPieces + kThreads - 1) / kThreads;
    uint4 v[kPer];
    // rows [0, ncols) of each plane are staged (ncols <= COLS, a multiple of 32); LDS stride ncols
    __device__ __forceinline__ void fetch(const uint16_t *p0, int64_t plane, int nrows_valid, int ldp, int k0,
                                          int ncols) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + kThreads * i;
            const int half = e & 1, row = (e >> 1) % COLS, pl = (e >> 1) / COLS;
            const int k = k0 + 8 * half;
            v[i] = uint4{0u, 0u, 0u, 0u};
            if (e < kPieces && row < nrows_valid && row < ncols && k < ldp)
                v[i] = *(const uint4 *)(p0 + pl * plane + (int64_t)row * ldp + k);
        }
    }
    __device__ __forceinline__ void store(uint16_t *qs, int ncols) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + kThreads * i;
            const int half = e & 1, row = (e >> 1) % COLS, pl = (e >> 1) / COLS;
            if (e < kPieces && row < ncols) *(uint4 *)(qs + ((size_t)pl * ncols + row) * kRowLd + 8 * half) = v[i];
        }
    }
};

__device__ __forceinline__ bf16x8 frag(const uint16_t *base, int rows_per_plane, int pl, int r, int koff) {
    return *(const bf16x8 *)(base + ((size_t)pl * rows_per_plane + r) * kRowLd + koff);
}

struct ProjTable16 {
    float *M[kMaxMats];
    const void *G[kMaxMats];
    const uint16_t *planes[kMaxMats];
    uint8_t *S[kMaxMats];
    float *Cout[kMaxMats];     // NULL or m x n fp32: the coefficients (verification output)
    float mu[kMaxMats];
};

// grid.x = row tiles (128 rows) * blocks * matrices, renumbered per XCD; block 512.
template <int CW, int NCW, int NEST, bool GBF16>
__global__ void __launch_bounds__(512) k_proj_bf16(int64_t m, int64_t n, int nb, int ldp, int rtiles, int nblk,
                                                   ProjTable16 t) {
    using C = Cfg<CW, NCW>;
    extern __shared__ __align__(16) uint16_t lds[];
    const int nct = (nb + 31) / 32, ncols = 32 * nct;
    uint16_t *const Abase = lds;                    // two A buffers of C::kAElems
    uint16_t *const Bbase = lds + 2 * C::kAElems;   // two B buffers of b_elems(ncols)
#define ABUF(i) (Abase + (i) * C::kAElems)
#define BBUF(i) (Bbase + (i) * b_elems(ncols))
    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int rt = x % rtiles, rest = x / rtiles;
    const int b = rest % nblk, mat = rest / nblk;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rg = w / CW, cg = w % CW;
    const int kh = 8 * (lane >> 5);
    const int64_t r0 = (int64_t)rt * kRows;
    float *const __restrict__ M = t.M[mat] + (int64_t)b * nb;
    const void *const __restrict__ Gv = t.G[mat];
    const float mu = t.mu[mat];
    const int64_t plane = (int64_t)nblk * nb * ldp;
    const uint16_t *QT = t.planes[mat] + 2 * plane + (int64_t)b * nb * ldp;  // transposed planes

    // A staging role: row ar, k offset ak (4 consecutive k)
    const int ar = tid >> 2, ak = 4 * (tid & 3);
    const int64_t arow = r0 + ar;
    const bool arok = arow < m;
    f32x4 mv, gv;   // operands of the next k-step to be staged
    auto fetch_a = [&](int k0) {
        const int kq = k0 + ak;
        mv = f32x4{0.f, 0.f, 0.f, 0.f};
        gv = f32x4{0.f, 0.f, 0.f, 0.f};
        if (arok && kq < nb) {
            const int64_t e = arow * n + kq;
            mv = *(const f32x4 *)(M + e);
            if (GBF16) {
                const uint2 hb = *(const uint2 *)((const uint16_t *)Gv + (int64_t)b * nb + e);
                gv[0] = bf16_to_f32((uint16_t)(hb.x & 0xffff)); gv[1] = bf16_to_f32((uint16_t)(hb.x >> 16));
                gv[2] = bf16_to_f32((uint16_t)(hb.y & 0xffff)); gv[3] = bf16_to_f32((uint16_t)(hb.y >> 16));
            } else {
                gv = *(const f32x4 *)((const float *)Gv + (int64_t)b * nb + e);
            }
        }
    };
    // momentum update of the fetched values, written back once; their split goes to LDS
    auto store_a = [&](int k0, uint16_t *A) {
        const int kq = k0 + ak;
        f32x4 mn;
#pragma unroll
        for (int c = 0; c < 4; ++c) mn[c] = __builtin_fmaf(mu, mv[c], gv[c]);
        if (arok && kq < nb) *(f32x4 *)(M + arow * n + kq) = mn;
        uint16_t h[4], md[4], l[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float pv = NEST ? __builtin_fmaf(mu, mn[c], gv[c]) : mn[c];
            split3(pv, h[c], md[c], l[c]);
        }
        uint2 vh = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
        uint2 vm = {(uint32_t)md[0] | ((uint32_t)md[1] << 16), (uint32_t)md[2] | ((uint32_t)md[3] << 16)};
        uint2 vl = {(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
        *(uint2 *)(A + ((size_t)0 * kRows + ar) * kRowLd + ak) = vh;
        *(uint2 *)(A + ((size_t)1 * kRows + ar) * kRowLd + ak) = vm;
        *(uint2 *)(A + ((size_t)2 * kRows + ar) * kRowLd + ak) = vl;
    };

    f32x16 acc[C::RT][NCW];
#pragma unroll
    for (int i = 0; i < C::RT; ++i)
#pragma unroll
        for (int c = 0; c < NCW; ++c) acc[i][c] = (f32x16){};

    BStage<3, C::kCols> bs;
    bs.fetch(QT, plane, nb, ldp, 0, ncols);
    fetch_a(0);
    bs.store(BBUF(0), ncols);
    store_a(0, ABUF(0));
    fetch_a(kKS);
    __syncthreads();
    int cur = 0;
    for (int k0 = 0; k0 < nb; k0 += kKS) {
        const bool more = k0 + kKS < nb;
        if (more) bs.fetch(QT, plane, nb, ldp, k0 + kKS, ncols);
        const uint16_t *A = ABUF(cur), *B = BBUF(cur);
        bf16x8 ah[C::RT], am[C::RT], al[C::RT];
#pragma unroll
        for (int i = 0; i < C::RT; ++i) {
            const int r = (rg * C::RT + i) * 32 + (lane & 31);
            ah[i] = frag(A, kRows, 0, r, kh); am[i] = frag(A, kRows, 1, r, kh); al[i] = frag(A, kRows, 2, r, kh);
        }
#pragma unroll
        for (int c = 0; c < NCW; ++c) {
            const int ch = cg + CW * c;
            if (ch >= nct) break;
            const int col = 32 * ch + (lane & 31);
            const bf16x8 Bh = frag(B, ncols, 0, col, kh);
            const bf16x8 Bm = frag(B, ncols, 1, col, kh);
            const bf16x8 Bl = frag(B, ncols, 2, col, kh);
#pragma unroll
            for (int i = 0; i < C::RT; ++i) {
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], Bh, acc[i][c], 0, 0, 0);
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], Bm, acc[i][c], 0, 0, 0);
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[i], Bh, acc[i][c], 0, 0, 0);
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], Bl, acc[i][c], 0, 0, 0);
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[i], Bm, acc[i][c], 0, 0, 0);
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], Bh, acc[i][c], 0, 0, 0);
            }
        }
        if (more) {
            bs.store(BBUF(cur ^ 1), ncols);
            store_a(k0 + kKS, ABUF(cur ^ 1));
            fetch_a(k0 + 2 * kKS);   // lands during the next step's products
        }
        __syncthreads();
        cur ^= 1;
    }
#undef ABUF
#undef BBUF
    // sign bytes, stored with row stride nblk * ldp (block b at column offset b * ldp)
    uint8_t *const __restrict__ S = t.S[mat] + (int64_t)b * ldp;
    const int64_t lds_ = (int64_t)nblk * ldp;
    float *const Cout = t.Cout[mat];
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
        const int col = 32 * (cg + CW * c) + acc_col(lane);
        if (col >= nb) continue;
#pragma unroll
        for (int i = 0; i < C::RT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t rr = r0 + (rg * C::RT + i) * 32 + acc_row(r, lane);
                if (rr < m) {
                    S[rr * lds_ + col] = sign_f16_hi(acc[i][c][r]);
                    if (Cout) Cout[rr * n + (int64_t)b * nb + col] = acc[i][c][r];
                }
            }
    }
}

struct ReconTable16 {
    const uint8_t *S[kMaxMats];
    const uint16_t *planes[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// two consecutive sign bytes (bytes 2j, 2j+1 of x) -> two fp16 values
template <int J>
__device__ __forceinline__ uint32_t signs_f16x2(uint32_t x) {
    return __builtin_amdgcn_perm(0u, x, J == 0 ? 0x010c000cu : 0x030c020cu);
}

// W <- W - lr (s U + wd W) for the accumulator tiles of one wave.  Lane l of a 32 x 32 tile holds
// column l % 32 and rows 4 (l / 32) + 8 (r / 4) + r % 4, so each lane walks one column with
// compile-time row offsets from its own row pointer.  FULL: every row of the workgroup is < m.
template <bool FULL, int RT, int NCW, int CW, bool WBF16>
__device__ __forceinline__ void recon_epilogue(const f32x16 (&acc)[RT][NCW], void *Wv, float *U, int64_t m,
                                               int64_t n, int nb, int b, int64_t r0, int rg, int cg, int lane,
                                               float lr, float wd, float sc) {
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
        const int col = 32 * (cg + CW * c) + acc_col(lane);
        if (col >= nb) continue;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const int64_t rl = r0 + (rg * RT + i) * 32 + 4 * (lane >> 5);   // this lane's first row
            const int64_t base = rl * n + (int64_t)b * nb + col;
            const int64_t vr = m - rl;                                     // rows left from rl on
            // loads of rows past m read a valid row instead: rl if rl < m, else row 0
            const int64_t lbase = FULL || vr > 0 ? base : (int64_t)b * nb + col;
            float wv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ro = 8 * (r >> 2) + (r & 3);
                const int64_t e = lbase + (FULL || ro < vr ? (int64_t)ro * n : 0);
                wv[r] = WBF16 ? bf16_to_f32(((const uint16_t *)Wv)[e]) : ((const float *)Wv)[e];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ro = 8 * (r >> 2) + (r & 3);
                if (!FULL && ro >= vr) continue;
                const int64_t e = base + (int64_t)ro * n;
                const float u = acc[i][c][r];
                if (U) U[e] = u;
                const float nw = wv[r] - lr * __builtin_fmaf(sc, u, wd * wv[r]);
                if (WBF16) ((uint16_t *)Wv)[e] = f32_to_bf16(nw);
                else ((float *)Wv)[e] = nw;
            }
        }
    }
}

// U = S Q^T with Q = Qh + Ql (fp16 parts) and S in {-1, 0, +1, NaN}: two f16 MFMAs per tile and k-step.
// Waves: RW = 8/CW row groups of 32*RT rows (RT = 4/RW) and CW column groups.  The sign codes of a
// row tile (8 bytes per lane per k-step) are read straight from global memory, two k-steps ahead;
// only Q's planes are staged in LDS (double buffered).
template <int CW, int NCW, bool WBF16>
__global__ void __launch_bounds__(512) k_recon_bf16(int64_t m, int64_t n, int nb, int ldp, int rtiles, int nblk,
                                                    ReconTable16 t) {
    constexpr int RW = kWavesPerWg / CW, RT = 4 / RW;
    constexpr int kColsMax = 32 * CW * NCW;
    extern __shared__ __align__(16) uint16_t lds[];
    const int x = xcd_remap(blockIdx.x, gridDim.x);
    const int rt = x % rtiles, rest = x / rtiles;
    const int b = rest % nblk, mat = rest / nblk;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rg = w / CW, cg = w % CW;
    const int kh = 8 * (lane >> 5);
    const int64_t r0 = (int64_t)rt * kRows;
    const int64_t lds_ = (int64_t)nblk * ldp;
    const uint8_t *S = t.S[mat] + (int64_t)b * ldp;
    const int64_t plane = (int64_t)nblk * nb * ldp;
    const uint16_t *Qn = t.planes[mat] + (int64_t)b * nb * ldp;  // natural fp16 planes: row p, entries c
    const int nct = (nb + 31) / 32, ncols = 32 * nct;
    const int belems = 2 * ncols * kRowLd;

    // sign bytes of the current and the next k-step (rows past m and k past nb read as 0)
    uint2 sa[RT], sb[RT];
    auto fetch_s = [&](int k0, uint2 *sq) {
        const int k = k0 + kh;   // multiple of 8; nb is a multiple of 4, so k < nb means k + 4 <= nb
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const int64_t row = r0 + (rg * RT + i) * 32 + (lane & 31);
            sq[i] = uint2{0u, 0u};
            if (row < m && k < nb) {
                sq[i] = *(const uint2 *)(S + row * lds_ + k);
                if (k + 4 >= nb) sq[i].y = 0u;
            }
        }
    };

    f32x16 acc[RT][NCW];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int c = 0; c < NCW; ++c) acc[i][c] = (f32x16){};

    BStage<2, kColsMax> bs;
    bs.fetch(Qn, plane, nb, ldp, 0, ncols);
    fetch_s(0, sa);
    fetch_s(kKS, sb);
    bs.store(lds, ncols);
    __syncthreads();
    int cur = 0;
    for (int k0 = 0; k0 < nb; k0 += kKS) {
        const bool more = k0 + kKS < nb;
        if (more) bs.fetch(Qn, plane, nb, ldp, k0 + kKS, ncols);
        const uint16_t *B = lds + cur * belems;
        f16x8 as[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const uint4 v = {signs_f16x2<0>(sa[i].x), signs_f16x2<1>(sa[i].x), signs_f16x2<0>(sa[i].y),
                             signs_f16x2<1>(sa[i].y)};
            as[i] = __builtin_bit_cast(f16x8, v);
        }
#pragma unroll
        for (int c = 0; c < NCW; ++c) {
            const int ch = cg + CW * c;
            if (ch >= nct) break;
            const int col = 32 * ch + (lane & 31);
            const f16x8 Bh = __builtin_bit_cast(f16x8, frag(B, ncols, 0, col, kh));
            const f16x8 Bl = __builtin_bit_cast(f16x8, frag(B, ncols, 1, col, kh));
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as[i], Bh, acc[i][c], 0, 0, 0);
                acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as[i], Bl, acc[i][c], 0, 0, 0);
            }
        }
        if (more) {
            bs.store(lds + (cur ^ 1) * belems, ncols);
#pragma unroll
            for (int i = 0; i < RT; ++i) sa[i] = sb[i];
            fetch_s(k0 + 2 * kKS, sb);
        }
        __syncthreads();
        cur ^= 1;
    }
    // epilogue: per 32-row tile, all 16 loads of W are issued before any store
    const float lr = t.lr[mat], wd = t.wd[mat], sc = t.scale[mat];
    if (r0 + kRows <= m)
        recon_epilogue<true, RT, NCW, CW, WBF16>(acc, t.W[mat], t.U[mat], m, n, nb, b, r0, rg, cg, lane, lr, wd, sc);
    else
        recon_epilogue<false, RT, NCW, CW, WBF16>(acc, t.W[mat], t.U[mat], m, n, nb, b, r0, rg, cg, lane, lr, wd, sc);
}

template <int CW, int NCW>
hipError_t launch_cfg(const StepArgs &a, int c0, int cnt, int ldp, hipStream_t s) {
    using C = Cfg<CW, NCW>;
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const int rtiles = (int)((m + kRows - 1) / kRows);
    {
        SplitTable t{};
        for (int i = 0; i < cnt; ++i) { t.Q[i] = a.Q[c0 + i]; t.planes[i] = a.planes[c0 + i]; }
        const int tiles = ((nb + 31) / 32) * ((ldp + 31) / 32);
        DOBB_LAUNCH("split_q", s, k_split_q, dim3((unsigned)tiles, (unsigned)(nblk * cnt)), dim3(256), 0, nb, ldp, nblk, t);
    }
    const dim3 grid((unsigned)(rtiles * nblk * cnt));
    {
        ProjTable16 t{};
        for (int i = 0; i < cnt; ++i) {
            t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.planes[i] = a.planes[c0 + i];
            t.S[i] = (uint8_t *)a.S[c0 + i]; t.mu[i] = a.hp[c0 + i].momentum;
            t.Cout[i] = a.Cout ? a.Cout[c0 + i] : nullptr;
        }
        const bool gbf = a.g_dtype == DOBB_BF16;
        const bool nest = a.hp[c0].nesterov != 0;
        const size_t sh = (size_t)2 * (C::kAElems + b_elems(32 * ((nb + 31) / 32))) * 2;
#define DOBB_PROJ3(NE, GB)                                                                                       \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_proj_bf16<CW, NCW, NE, GB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("project_bf16x6", s, (k_proj_bf16<CW, NCW, NE, GB>), grid, dim3(kThreads), sh, m, n, nb, ldp, rtiles, nblk, t); \
    } while (0)
        if (!nest) { if (gbf) DOBB_PROJ3(0, true); else DOBB_PROJ3(0, false); }
        else { if (gbf) DOBB_PROJ3(1, true); else DOBB_PROJ3(1, false); }
#undef DOBB_PROJ3
    }
    return hipGetLastError();
}

template <int CW, int NCW>
hipError_t launch_recon(const StepArgs &a, int c0, int cnt, int ldp, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const int rtiles = (int)((m + kRows - 1) / kRows);
    const dim3 grid((unsigned)(rtiles * nblk * cnt));
    ReconTable16 t{};
    for (int i = 0; i < cnt; ++i) {
        const dobb_hparams &h = a.hp[c0 + i];
        t.S[i] = (const uint8_t *)a.S[c0 + i]; t.planes[i] = a.planes[c0 + i]; t.W[i] = a.W[c0 + i];
        t.U[i] = a.U ? a.U[c0 + i] : nullptr;
        t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
    }
    const size_t sh = (size_t)2 * (2 * 32 * ((nb + 31) / 32) * kRowLd) * 2;
#define DOBB_REC3(WB)                                                                                            \
    do {                                                                                                         \
        (void)hipFuncSetAttribute((const void *)k_recon_bf16<CW, NCW, WB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("reconstruct_f16x2", s, (k_recon_bf16<CW, NCW, WB>), grid, dim3(kThreads), sh, m, n, nb, ldp, rtiles, nblk, t); \
    } while (0)
    if (a.w_dtype == DOBB_BF16) DOBB_REC3(true); else DOBB_REC3(false);
#undef DOBB_REC3
    return hipGetLastError();
}

}  // namespace

int step_bf16_ldp(int64_t nb) { return (int)((nb + 7) / 8 * 8); }

bool step_bf16_eligible(const dobb_shape &sh, int norm) {
    if (norm != DOBB_NORM_SIGN || sh.nb % 4 != 0 || sh.nb > 512 || sh.n % 4 != 0) return false;
    const int ncols = 32 * (int)((sh.nb + 31) / 32);
    const size_t lds = (size_t)2 * (Cfg<4, 1>::kAElems + b_elems(ncols)) * 2;  // the projection's LDS
    return (int64_t)lds <= max_lds_bytes();
}

size_t step_bf16_ws_one(const dobb_shape &sh) {
    const int64_t ldp = step_bf16_ldp(sh.nb), nblk = sh.n / sh.nb;
    const size_t s_bytes = (size_t)sh.m * nblk * ldp;
    size_t p_bytes = (size_t)5 * nblk * sh.nb * ldp * 2;
    if (step_wide_planes_bytes(sh) > p_bytes) p_bytes = step_wide_planes_bytes(sh);
    return (s_bytes + 255) / 256 * 256 + (p_bytes + 255) / 256 * 256;
}

hipError_t launch_step_bf16(const StepArgs &a, hipStream_t s) {
    const int nb = (int)a.sh.nb;
    const int ldp = step_bf16_ldp(nb);
    if (step_fused_eligible(a.sh)) return launch_step_fused(a, s);
    if (step_wide_eligible(a.sh)) return launch_step_wide(a, ldp, s);
    const int nct = (nb + 31) / 32;   // 32-column chunks of a block
    for (int c0 = 0; c0 < a.count;) {
        const int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        hipError_t e;
        if (nct <= 2) e = launch_cfg<2, 1>(a, c0, cnt, ldp, s);
        else if (nct <= 4) e = launch_cfg<4, 1>(a, c0, cnt, ldp, s);
        else if (nct <= 8) e = launch_cfg<4, 2>(a, c0, cnt, ldp, s);
        else if (nct <= 12) e = launch_cfg<4, 3>(a, c0, cnt, ldp, s);
        else e = launch_cfg<4, 4>(a, c0, cnt, ldp, s);
        if (e != hipSuccess) return e;
        if (nct <= 2) e = launch_recon<2, 1>(a, c0, cnt, ldp, s);
        else if (nct <= 4) e = launch_recon<4, 1>(a, c0, cnt, ldp, s);
        else if (nct <= 8) e = launch_recon<8, 1>(a, c0, cnt, ldp, s);
        else e = launch_recon<8, 2>(a, c0, cnt, ldp, s);
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
