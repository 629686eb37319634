// The Dobb step (sign normalisation) for block widths nb <= 128, with the block's basis resident
// in LDS.
//
// Dobb paper (arXiv 2610.39412): abstract (project momentum into the block bases, sign-normalise,
// reconstruct), Table 9 (update scale), Table 21 caption (decoupled weight decay), Table 19
// (Nesterov).
//
// Same arithmetic as the staged kernels of k_step_bf16.hip: the projection C = P Q splits both
// operands into three bf16 parts and issues the six products of order <= 2; the reconstruction
// U = S Q^T splits Q into two fp16 parts (S is exact in fp16).  Signs travel as the high byte of
// their fp16 value (+1 -> 0x3c, -1 -> 0xbc, 0 -> 0x00, NaN -> 0x7e).
//
// A workgroup (4 waves) owns one block b and a range of 32-row slabs.  It first writes the split
// basis into LDS (from fp32 Q: no separate split pass), then every wave streams its slabs on its
// own, with no workgroup barrier: the operands of k-step j + 2 are loaded while k-step j runs.
//   k_proj_res   M <- mu M + G; C = P Q (P = M, or G + mu M with Nesterov); sign bytes out
//   k_recon_res  U = S Q^T; W <- W - lr (s U + wd W); the slab's W is loaded one slab ahead
#include "dobb_internal.h"

#include <type_traits>

namespace dobb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));

constexpr int kRT = 256;    // threads per workgroup
constexpr int kKS = 16;     // k per MFMA step
constexpr int kPadK = 8;    // LDS row padding (bf16/fp16 elements)

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ void split3(float v, uint16_t &h, uint16_t &m, uint16_t &l) {
    h = bf16_bits(v);
    const float r1 = v - bf16_to_f32(h);
    m = bf16_bits(r1);
    l = bf16_bits(r1 - bf16_to_f32(m));
}
__device__ __forceinline__ void split2h(float v, uint16_t &h, uint16_t &l) {
    const _Float16 a = (_Float16)v;
    h = __builtin_bit_cast(uint16_t, a);
    l = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)a));
}
// high byte of the fp16 value of sign(c), from the bits of c without branches:
// +1 -> 0x3c, -1 -> 0xbc, +-0 -> 0x00, NaN -> 0x7e
__device__ __forceinline__ uint32_t sign_byte(float c) {
    const uint32_t u = __float_as_uint(c);
    const uint32_t mag = u & 0x7fffffffu;
    const uint32_t sb = 0x3cu | ((u >> 24) & 0x80u);
    const uint32_t nz = mag > 0x7f800000u ? 0x7eu : sb;
    return mag == 0u ? 0u : nz;
}
template <int J>
__device__ __forceinline__ uint32_t signs_f16x2(uint32_t x) {
    return __builtin_amdgcn_perm(0u, x, J == 0 ? 0x010c000cu : 0x030c020cu);
}
__device__ __forceinline__ int xcd_remap(int x, int G) {
    if (G % 8) return x;
    return (x % 8) * (G / 8) + x / 8;
}
__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }

// Buffer descriptor over [base, base + bytes).  Accesses through it are never branched around: a
// lane with nothing to do gets the offset kOff, past the end, so its load returns 0 and its store is
// dropped.  With every memory instruction unconditional the compiler can count the outstanding
// ones exactly and wait only for the operands a step needs (a branched access makes it wait for
// all of them).
constexpr unsigned kOff = 0xffffffffu;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---- projection ----------------------------------------------------------------------------------
struct ProjResTable {
    float *M[kMaxMats];
    const void *G[kMaxMats];
    const float *Q[kMaxMats];
    uint8_t *S[kMaxMats];
    float mu[kMaxMats];
};

// One k-step's operands for one lane: row l % 32 of the slab, k = 16 ks + 8 (l / 32) .. + 7.
struct PStep {
    f32x4 m0, m1, g0, g1;
};

// LDS: three planes (bf16 h, m, l of Q) x nb columns j x qld (k = row p of Q), i.e. Q^T.
// grid.x = blocks x slab groups x matrices (renumbered per XCD), block 256.
template <int NCH, int NEST, bool GBF16>
__global__ void __launch_bounds__(256) k_proj_res(int64_t m, int64_t n, int nb, int nblk, int ngroups, int spg,
                                                  int ldp, ProjResTable t) {
    extern __shared__ __align__(16) uint16_t qs[];
    const int KS = (nb + kKS - 1) / kKS, kpad = KS * kKS, qld = kpad + kPadK;
    const int x = xcd_remap(blockIdx.x, gridDim.x);
    // block index fastest: the workgroups that run together on one XCD cover every block of the
    // same rows, so each row of M, G (or W) is read in one sweep
    const int b = x % nblk, rest = x / nblk;
    const int grp = rest % ngroups, mat = rest / ngroups;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t nslab = (m + 31) / 32;
    const int64_t s_begin = (int64_t)grp * spg;
    const int64_t s_end = s_begin + spg < nslab ? s_begin + spg : nslab;

    // split Q_b^T into the three planes: element (p, j) of Q -> plane[j][p]; zero for p in [nb, kpad)
    {
        const float *Q = t.Q[mat] + (int64_t)b * nb * nb;
        const int total = kpad * nb;
        for (int e0 = 0; e0 < total; e0 += kRT * 8) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + tid + kRT * i;
                const int p = e / nb;
                v[i] = (e < total && p < nb) ? Q[e] : 0.f;   // e = p * nb + j
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + tid + kRT * i;
                if (e < total) {
                    const int p = e / nb, j = e - p * nb;
                    uint16_t h, md, l;
                    split3(v[i], h, md, l);
                    qs[(0 * nb + j) * qld + p] = h;
                    qs[(1 * nb + j) * qld + p] = md;
                    qs[(2 * nb + j) * qld + p] = l;
                }
            }
        }
    }
    __syncthreads();

    float *M = t.M[mat] + (int64_t)b * nb;
    const void *Gv = t.G[mat];
    const float mu = t.mu[mat];
    const int kh = 8 * (lane >> 5);
    const int nsl = (int)((s_end - s_begin - wv + 3) / 4);   // this wave's slabs: s_begin + wv + 4 i
    const int nsteps = nsl > 0 ? nsl * KS : 0;

    // descriptors over this block's columns of M, G and the sign bytes (row-major, rows < m)
    const int64_t ncut = (int64_t)b * nb;
    const __amdgpu_buffer_rsrc_t rM = make_rsrc(M, (m * n - ncut) * 4);
    const __amdgpu_buffer_rsrc_t rG = make_rsrc((const char *)Gv + ncut * (GBF16 ? 2 : 4), (m * n - ncut) * (GBF16 ? 2 : 4));
    // element offset of (row, k) within the block, or kOff (row >= m, step past the end, k >= nb)
    auto elem_off = [&](int idx, int k4) -> unsigned {
        const int sl = idx / KS, ks = idx - sl * KS;
        const int64_t row = (s_begin + wv + 4 * (int64_t)sl) * 32 + (lane & 31);
        const int k = ks * kKS + kh + k4;
        return (idx < nsteps && row < m && k < nb) ? (unsigned)(row * n + k) : kOff;
    };
    auto load = [&](int idx, PStep &d) {
        const unsigned e0 = elem_off(idx, 0), e1 = elem_off(idx, 4);
        d.m0 = bload4(rM, e0 == kOff ? kOff : e0 * 4);
        d.m1 = bload4(rM, e1 == kOff ? kOff : e1 * 4);
        if (GBF16) {
            const uint2 h0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rG, e0 == kOff ? kOff : e0 * 2, 0, 0));
            const uint2 h1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rG, e1 == kOff ? kOff : e1 * 2, 0, 0));
            d.g0 = f32x4{bf16_to_f32((uint16_t)h0.x), bf16_to_f32((uint16_t)(h0.x >> 16)),
                         bf16_to_f32((uint16_t)h0.y), bf16_to_f32((uint16_t)(h0.y >> 16))};
            d.g1 = f32x4{bf16_to_f32((uint16_t)h1.x), bf16_to_f32((uint16_t)(h1.x >> 16)),
                         bf16_to_f32((uint16_t)h1.y), bf16_to_f32((uint16_t)(h1.y >> 16))};
        } else {
            d.g0 = bload4(rG, e0 == kOff ? kOff : e0 * 4);
            d.g1 = bload4(rG, e1 == kOff ? kOff : e1 * 4);
        }
    };

    uint8_t *S = t.S[mat] + (int64_t)b * ldp;
    const int64_t sld = (int64_t)nblk * ldp;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(S, m * sld - (int64_t)b * ldp);
    f32x16 acc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = (f32x16){};

    // one k-step: uses the operands in `cur` and refills `fill` with those of step idx + 2.  Memory
    // instructions are issued even past the last step (offset kOff), so their count never depends
    // on a branch; only the arithmetic of a step past the end is skipped.
    auto step = [&](int idx, PStep &cur, PStep &fill) {
        load(idx + 2, fill);
        const unsigned e0 = elem_off(idx, 0), e1 = elem_off(idx, 4);
        f32x4 mn0, mn1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            mn0[c] = __builtin_fmaf(mu, cur.m0[c], cur.g0[c]);
            mn1[c] = __builtin_fmaf(mu, cur.m1[c], cur.g1[c]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, mn0), rM, e0 == kOff ? kOff : e0 * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, mn1), rM, e1 == kOff ? kOff : e1 * 4, 0, 0);
        if (idx >= nsteps) return;
        const int sl = idx / KS, ks = idx - sl * KS;
        float pv[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pv[c] = NEST ? __builtin_fmaf(mu, mn0[c], cur.g0[c]) : mn0[c];
            pv[c + 4] = NEST ? __builtin_fmaf(mu, mn1[c], cur.g1[c]) : mn1[c];
        }
        uint16_t hh[8], hm[8], hl[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) split3(pv[c], hh[c], hm[c], hl[c]);
        const uint4 uh = {pack2(hh[0], hh[1]), pack2(hh[2], hh[3]), pack2(hh[4], hh[5]), pack2(hh[6], hh[7])};
        const uint4 um = {pack2(hm[0], hm[1]), pack2(hm[2], hm[3]), pack2(hm[4], hm[5]), pack2(hm[6], hm[7])};
        const uint4 ul = {pack2(hl[0], hl[1]), pack2(hl[2], hl[3]), pack2(hl[4], hl[5]), pack2(hl[6], hl[7])};
        const bf16x8 ah = __builtin_bit_cast(bf16x8, uh), am = __builtin_bit_cast(bf16x8, um),
                     al = __builtin_bit_cast(bf16x8, ul);
        bf16x8 Qh[NCH], Qm[NCH], Ql[NCH];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            const int j = 32 * ch + (lane & 31);
            const bool jok = ch < NCH - 1 || j < nb;   // only the last chunk can reach past nb
            const int js = jok ? j : 0;
            uint4 bh = *(const uint4 *)&qs[(0 * nb + js) * qld + ks * kKS + kh];
            uint4 bm = *(const uint4 *)&qs[(1 * nb + js) * qld + ks * kKS + kh];
            uint4 bl = *(const uint4 *)&qs[(2 * nb + js) * qld + ks * kKS + kh];
            if (ch == NCH - 1 && !jok) bh = bm = bl = uint4{0u, 0u, 0u, 0u};
            Qh[ch] = __builtin_bit_cast(bf16x8, bh);
            Qm[ch] = __builtin_bit_cast(bf16x8, bm);
            Ql[ch] = __builtin_bit_cast(bf16x8, bl);
        }
        // C^T = Q^T P^T: the accumulator holds row l % 32 of the slab and columns
        // 32 ch + 4 (l / 32) + 8 q + t in register 4 q + t.  Products are issued chunk-interleaved so
        // consecutive MFMAs never share an accumulator.
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Qh[ch], ah, acc[ch], 0, 0, 0);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Qm[ch], ah, acc[ch], 0, 0, 0);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Qh[ch], am, acc[ch], 0, 0, 0);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ql[ch], ah, acc[ch], 0, 0, 0);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Qm[ch], am, acc[ch], 0, 0, 0);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Qh[ch], al, acc[ch], 0, 0, 0);
        if (ks == KS - 1) {   // slab done: four sign bytes per store, then a fresh accumulator
            const int64_t row = (s_begin + wv + 4 * (int64_t)sl) * 32 + (lane & 31);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = 32 * ch + 4 * (lane >> 5) + 8 * q;   // nb % 4 == 0: all 4 valid or none
                    const uint32_t w4 = sign_byte(acc[ch][4 * q]) | (sign_byte(acc[ch][4 * q + 1]) << 8) |
                                        (sign_byte(acc[ch][4 * q + 2]) << 16) | (sign_byte(acc[ch][4 * q + 3]) << 24);
                    const unsigned off = (row < m && col < nb) ? (unsigned)(row * sld + col) : kOff;
                    __builtin_amdgcn_raw_buffer_store_b32(w4, rS, off, 0, 0);
                }
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) acc[ch] = (f32x16){};
        }
    };

    PStep d0, d1, d2;
    load(0, d0);
    load(1, d1);
    for (int idx = 0; idx < nsteps; idx += 3) {   // three steps per trip: the operand buffers rotate by name
        step(idx, d0, d2);
        step(idx + 1, d1, d0);
        step(idx + 2, d2, d1);
    }
}

// ---- reconstruction ------------------------------------------------------------------------------
struct ReconResTable {
    const uint8_t *S[kMaxMats];
    const float *Q[kMaxMats];
    void *W[kMaxMats];
    float *U[kMaxMats];
    float lr[kMaxMats], wd[kMaxMats], scale[kMaxMats];
};

// LDS: two planes (fp16 hi, lo of Q) x nb rows p x qld (k = column c of Q), Q's natural layout.
template <int NCH, bool WBF16>
__global__ void __launch_bounds__(256) k_recon_res(int64_t m, int64_t n, int nb, int nblk, int ngroups, int spg,
                                                   int ldp, ReconResTable t) {
    extern __shared__ __align__(16) uint16_t qs[];
    const int KS = (nb + kKS - 1) / kKS, kpad = KS * kKS, qld = kpad + kPadK;
    const int x = xcd_remap(blockIdx.x, gridDim.x);
    // block index fastest: the workgroups that run together on one XCD cover every block of the
    // same rows, so each row of M, G (or W) is read in one sweep
    const int b = x % nblk, rest = x / nblk;
    const int grp = rest % ngroups, mat = rest / ngroups;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t nslab = (m + 31) / 32;
    const int64_t s_begin = (int64_t)grp * spg;
    const int64_t s_end = s_begin + spg < nslab ? s_begin + spg : nslab;

    // split Q_b into the two planes: element (p, c) -> plane[p][c]; zero for c in [nb, kpad)
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
    __syncthreads();

    const int kh = 8 * (lane >> 5);
    const int nsl = (int)((s_end - s_begin - wv + 3) / 4);
    const uint8_t *S = t.S[mat] + (int64_t)b * ldp;
    const int64_t sld = (int64_t)nblk * ldp;
    const float lr = t.lr[mat], wd = t.wd[mat], sc = t.scale[mat];
    void *const Wv = t.W[mat];
    float *const U = t.U[mat];

    const int64_t ncut = (int64_t)b * nb;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(S, m * sld - (int64_t)b * ldp);
    constexpr int kEs = WBF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rW = make_rsrc((const char *)Wv + ncut * kEs, (m * n - ncut) * kEs);
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(U ? (const void *)(U + ncut) : (const void *)Wv, U ? (m * n - ncut) * 4 : 0);
    // sign bytes of slab sl for this lane: row l % 32, k = 16 ks + 8 (l / 32) .. + 7 for ks < KS
    // (at most 8 k-steps); rows past m and k past nb read as 0
    auto load_s = [&](int sl, uint2 (&sv)[8]) {
        const int64_t row = (s_begin + wv + 4 * (int64_t)sl) * 32 + (lane & 31);
        const bool rok = sl < nsl && row < m;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int k = ks * kKS + kh;   // multiple of 8; nb % 4 == 0, so k < nb means k + 4 <= nb
            const unsigned off = (rok && ks < KS && k < nb) ? (unsigned)(row * sld + k) : kOff;
            sv[ks] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rS, off, 0, 0));
            if (k + 4 >= nb) sv[ks].y = 0u;
        }
    };
    // U^T = Q S^T: the accumulator holds row l % 32 of the slab and columns 32 ch + 4 (l / 32) + 8 q + t
    // in register 4 q + t, so W moves in 4-column pieces; pieces of rows past m or columns past nb get
    // the offset kOff (loads read 0, stores are dropped)
    using WVec = typename std::conditional<WBF16, uint2, f32x4>::type;
    auto woff = [&](int sl, int c) -> unsigned {   // element offset of this lane's piece at column c + 4 (l / 32)
        const int64_t row = (s_begin + wv + 4 * (int64_t)sl) * 32 + (lane & 31);
        const int col = c + 4 * (lane >> 5);
        return (sl < nsl && row < m && col < nb) ? (unsigned)(row * n + col) : kOff;
    };

    uint2 scur[8], snext[8];
    load_s(0, scur);
    for (int sl = 0; sl < nsl; ++sl) {
        // this slab's W and the next slab's sign bytes are in flight during this slab's products
        WVec wcur[NCH][4];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const unsigned eo = woff(sl, 32 * ch + 8 * q);
                const unsigned bo = eo == kOff ? kOff : eo * kEs;
                if constexpr (WBF16) wcur[ch][q] = __builtin_bit_cast(WVec, __builtin_amdgcn_raw_buffer_load_b64(rW, bo, 0, 0));
                else wcur[ch][q] = __builtin_bit_cast(WVec, __builtin_amdgcn_raw_buffer_load_b128(rW, bo, 0, 0));
            }
        load_s(sl + 1, snext);
        f32x16 acc[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) acc[c] = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks >= KS) break;
            const uint4 av = {signs_f16x2<0>(scur[ks].x), signs_f16x2<1>(scur[ks].x), signs_f16x2<0>(scur[ks].y),
                              signs_f16x2<1>(scur[ks].y)};
            const f16x8 as = __builtin_bit_cast(f16x8, av);
            f16x8 Bh[NCH], Bl[NCH];
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int p = 32 * ch + (lane & 31);
                const bool pok = ch < NCH - 1 || p < nb;   // only the last chunk can reach past nb
                const int ps = pok ? p : 0;
                uint4 bh = *(const uint4 *)&qs[(0 * nb + ps) * qld + ks * kKS + kh];
                uint4 bl = *(const uint4 *)&qs[(1 * nb + ps) * qld + ks * kKS + kh];
                if (ch == NCH - 1 && !pok) bh = bl = uint4{0u, 0u, 0u, 0u};
                Bh[ch] = __builtin_bit_cast(f16x8, bh);
                Bl[ch] = __builtin_bit_cast(f16x8, bl);
            }
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Bh[ch], as, acc[ch], 0, 0, 0);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) acc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Bl[ch], as, acc[ch], 0, 0, 0);
        }
        // W <- W - lr (s U + wd W)
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const unsigned eo = woff(sl, 32 * ch + 8 * q);
                float w0[4], nw[4];
                if (WBF16) {
                    const uint2 hb = *(const uint2 *)&wcur[ch][q];
                    w0[0] = bf16_to_f32((uint16_t)hb.x); w0[1] = bf16_to_f32((uint16_t)(hb.x >> 16));
                    w0[2] = bf16_to_f32((uint16_t)hb.y); w0[3] = bf16_to_f32((uint16_t)(hb.y >> 16));
                } else {
                    const f32x4 fv = *(const f32x4 *)&wcur[ch][q];
                    w0[0] = fv[0]; w0[1] = fv[1]; w0[2] = fv[2]; w0[3] = fv[3];
                }
                f32x4 uv;
#pragma unroll
                for (int t2 = 0; t2 < 4; ++t2) {
                    const float u = acc[ch][4 * q + t2];
                    uv[t2] = u;
                    nw[t2] = w0[t2] - lr * __builtin_fmaf(sc, u, wd * w0[t2]);
                }
                if (U) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, uv), rU, eo == kOff ? kOff : eo * 4, 0, 0);
                if (WBF16) {
                    const v2u32 o = {(uint32_t)f32_to_bf16(nw[0]) | ((uint32_t)f32_to_bf16(nw[1]) << 16),
                                     (uint32_t)f32_to_bf16(nw[2]) | ((uint32_t)f32_to_bf16(nw[3]) << 16)};
                    __builtin_amdgcn_raw_buffer_store_b64(o, rW, eo == kOff ? kOff : eo * 2, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, f32x4{nw[0], nw[1], nw[2], nw[3]}), rW,
                                                          eo == kOff ? kOff : eo * 4, 0, 0);
                }
            }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) scur[ks] = snext[ks];
    }
}

template <int NCH>
hipError_t launch_res(const StepArgs &a, int c0, int cnt, int ldp, hipStream_t s) {
    const int64_t m = a.sh.m, n = a.sh.n;
    const int nb = (int)a.sh.nb;
    const int nblk = (int)(n / nb);
    const int KS = (nb + kKS - 1) / kKS, qld = KS * kKS + kPadK;
    const int64_t nslab = (m + 31) / 32;
    // slabs per workgroup: enough workgroups to fill the chip about four times over, at least 4
    const int64_t blocks = (int64_t)nblk * cnt;
    int64_t spg = (nslab * blocks + 4 * 1024 - 1) / (4 * 1024);
    if (spg < 4) spg = 4;
    spg = (spg + 3) / 4 * 4;
    if (spg > nslab) spg = (nslab + 3) / 4 * 4;
    const int ngroups = (int)((nslab + spg - 1) / spg);
    const dim3 grid((unsigned)(ngroups * blocks));
    {
        ProjResTable t{};
        for (int i = 0; i < cnt; ++i) {
            t.M[i] = a.M[c0 + i]; t.G[i] = a.G[c0 + i]; t.Q[i] = a.Q[c0 + i];
            t.S[i] = (uint8_t *)a.S[c0 + i]; t.mu[i] = a.hp[c0 + i].momentum;
        }
        const size_t sh = (size_t)3 * nb * qld * 2;
        const bool gbf = a.g_dtype == DOBB_BF16;
        const bool nest = a.hp[c0].nesterov != 0;
#define DOBB_PRES(NE, GB)                                                                                         \
    do {                                                                                                          \
        (void)hipFuncSetAttribute((const void *)k_proj_res<NCH, NE, GB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("project_bf16x6", s, (k_proj_res<NCH, NE, GB>), grid, dim3(kRT), sh, m, n, nb, nblk, ngroups, (int)spg, \
                    ldp, t);                                                                                      \
    } while (0)
        if (!nest) { if (gbf) DOBB_PRES(0, true); else DOBB_PRES(0, false); }
        else { if (gbf) DOBB_PRES(1, true); else DOBB_PRES(1, false); }
#undef DOBB_PRES
    }
    {
        ReconResTable t{};
        for (int i = 0; i < cnt; ++i) {
            const dobb_hparams &h = a.hp[c0 + i];
            t.S[i] = (const uint8_t *)a.S[c0 + i]; t.Q[i] = a.Q[c0 + i]; t.W[i] = a.W[c0 + i];
            t.U[i] = a.U ? a.U[c0 + i] : nullptr;
            t.lr[i] = h.lr; t.wd[i] = h.weight_decay; t.scale[i] = h.update_scale;
        }
        const size_t sh = (size_t)2 * nb * qld * 2;
#define DOBB_RRES(WB)                                                                                             \
    do {                                                                                                          \
        (void)hipFuncSetAttribute((const void *)k_recon_res<NCH, WB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh); \
        DOBB_LAUNCH("reconstruct_f16x2", s, (k_recon_res<NCH, WB>), grid, dim3(kRT), sh, m, n, nb, nblk, ngroups, (int)spg, \
                    ldp, t);                                                                                      \
    } while (0)
        if (a.w_dtype == DOBB_BF16) DOBB_RRES(true); else DOBB_RRES(false);
#undef DOBB_RRES
    }
    return hipGetLastError();
}

}  // namespace

bool step_res_eligible(const dobb_shape &sh) { return sh.nb <= 128; }

hipError_t launch_step_res(const StepArgs &a, int ldp, hipStream_t s) {
    const int nct = (int)((a.sh.nb + 31) / 32);
    for (int c0 = 0; c0 < a.count;) {
        const int cnt = a.count - c0 < kMaxMats ? a.count - c0 : kMaxMats;
        hipError_t e;
        if (nct <= 1) e = launch_res<1>(a, c0, cnt, ldp, s);
        else if (nct <= 2) e = launch_res<2>(a, c0, cnt, ldp, s);
        else if (nct <= 3) e = launch_res<3>(a, c0, cnt, ldp, s);
        else e = launch_res<4>(a, c0, cnt, ldp, s);
        if (e != hipSuccess) return e;
        c0 += cnt;
    }
    return hipSuccess;
}

}  // namespace dobb
