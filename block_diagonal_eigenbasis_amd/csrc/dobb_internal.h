// Internal definitions shared by the libdobb kernels and the C-ABI layer (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dobb.h"

namespace dobb {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Matrices handled by one launch.  Kernels receive a table of per-matrix device pointers by value
// (kernel arguments are copied at launch, so nothing is staged in device memory); the matrices of
// one table share a shape.  Launchers split longer lists into chunks of kMaxMats.
constexpr int kMaxMats = 48;

// ---- bf16 helpers (round-to-nearest-even on store; NaN kept quiet) ----
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : rne);  // NaN stays NaN
}

// sign with sign(0) = 0 and NaN kept; encoded in int8 as -1, 0, 1 and 0x7f for NaN
__device__ __forceinline__ int8_t sign_code(float c) {
    return c > 0.f ? (int8_t)1 : c < 0.f ? (int8_t)-1 : c == 0.f ? (int8_t)0 : (int8_t)127;
}
__device__ __forceinline__ float sign_decode(int8_t s) { return s == 127 ? __builtin_nanf("") : (float)s; }

// ---- tiled fp32 MFMA GEMM core -------------------------------------------------------------
// One 256-thread workgroup computes a 64 x 64 output tile; wave w owns the 32 x 32 sub-tile at rows
// 32*(w/2), cols 32*(w%2) with v_mfma_f32_32x32x2_f32.  Operands are staged through LDS one
// 16-deep K-chunk at a time, both k-major: a[k][i] (output row i) and b[k][j] (output column j), so
// every MFMA operand read is 32 consecutive floats.  Lane layout of the 32x32 accumulator (checked
// on gfx950): register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
constexpr int kBM = 64, kBN = 64, kBK = 16, kPad = 4;

struct GemmSmem {
    float a[kBK][kBM + kPad];
    float b[kBK][kBN + kPad];
};

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
// Workgroup ids renumbered so that each XCD (ids are dealt round-robin over the 8 XCDs) runs a
// contiguous range of logical ids: neighbours in logical order then share one XCD's L2.
__device__ __forceinline__ int xcd_remap(int x, int G) {
    if (G % 8) return x;
    return (x % 8) * (G / 8) + x / 8;
}
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Two LDS buffers for gemm_tile: the next K-chunk is fetched into registers before the products of
// the current one and stored to the other buffer after them, so each chunk costs one barrier.
// Column index swizzled by row (gemm_swz): the two rows read by the half-waves of an MFMA operand
// load fall in opposite bank halves, and the four rows a loader wave writes in one instruction
// spread over all 64 banks.
struct __align__(16) GemmSmem2 {
    float a[2][kBK][kBM];
    float b[2][kBK][kBN];
};
__device__ __forceinline__ int gemm_swz(int row) { return ((row & 1) << 5) ^ (((row >> 2) & 3) << 4); }

template <typename LoadA, typename LoadB>
__device__ __forceinline__ f32x16 gemm_tile(int K, const LoadA &la, const LoadB &lb, GemmSmem2 &sm) {
    f32x16 acc = {};
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wr = 32 * (w >> 1), wc = 32 * (w & 1);
    float va[4], vb[4];
    la.fetch(0, va);
    lb.fetch(0, vb);
    la.put(va, sm.a[0]);
    lb.put(vb, sm.b[0]);
    __syncthreads();
    int cur = 0;
    for (int k0 = 0; k0 < K; k0 += kBK) {
        const bool more = k0 + kBK < K;
        if (more) {
            la.fetch(k0 + kBK, va);
            lb.fetch(k0 + kBK, vb);
        }
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 2) {
            const int kr = kk + (lane >> 5);
            float a = sm.a[cur][kr][(wr + (lane & 31)) ^ gemm_swz(kr)];
            float b = sm.b[cur][kr][(wc + (lane & 31)) ^ gemm_swz(kr)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
        if (more) {   // the other buffer's readers finished before the last barrier
            la.put(va, sm.a[cur ^ 1]);
            lb.put(vb, sm.b[cur ^ 1]);
        }
        __syncthreads();
        cur ^= 1;
    }
    return acc;
}

// Loader: a[k][i] = src[(r0 + i) * ld + k0 + k] (row-major operand that must be transposed into the
// k-major LDS layout).  Zero outside rows < rows, k < K.  Thread t loads row t/4, k = 4*(t%4)..+3.
template <bool VEC>
struct LoadRowsT {
    const float *src; int64_t ld; int rows; int K;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, i = t >> 2, k = k0 + 4 * (t & 3);
        v[0] = v[1] = v[2] = v[3] = 0.f;
        if (i < rows) {
            const float *p = src + (int64_t)i * ld + k;
            if (VEC) {
                if (k < K) { f32x4 q = *(const f32x4 *)p; v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3]; }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) if (k + c < K) v[c] = p[c];
            }
        }
    }
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBM]) const {
        const int t = threadIdx.x, i = t >> 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[4 * (t & 3) + c][i ^ gemm_swz(4 * (t & 3) + c)] = v[c];
    }
};

// Loader: b[k][j] = src[(k0 + k) * ld + j] (already k-major).  Zero outside k < K, j < cols.
// Thread t loads k = t/16, j = 4*(t%16)..+3.
template <bool VEC>
struct LoadColsK {
    const float *src; int64_t ld; int cols; int K;
    __device__ __forceinline__ void fetch(int k0, float (&v)[4]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15), k = k0 + kk;
        v[0] = v[1] = v[2] = v[3] = 0.f;
        if (k < K) {
            const float *p = src + (int64_t)k * ld + j;
            if (VEC) {
                if (j < cols) { f32x4 q = *(const f32x4 *)p; v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3]; }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) if (j + c < cols) v[c] = p[c];
            }
        }
    }
    // the swizzle flips column bits 4 and 5 only, so the four columns stay contiguous: one 16-byte
    // store per lane (four 4-byte stores at stride 4 put a wave's 64 lanes on 16 banks)
    __device__ __forceinline__ void put(const float (&v)[4], float (*dst)[kBN]) const {
        const int t = threadIdx.x, kk = t >> 4, j = 4 * (t & 15);
        *(f32x4 *)&dst[kk][j ^ gemm_swz(kk)] = f32x4{v[0], v[1], v[2], v[3]};
    }
};

// ---- kernel launchers (one translation unit each); arrays are host arrays of length count ----
void prof_before(const char *name, hipStream_t s);  // event pair around each launch when profiling
void prof_after(hipStream_t s);
int max_lds_bytes();

struct StepArgs {
    int count;
    dobb_shape sh;
    dobb_dtype w_dtype, g_dtype;
    const dobb_hparams *hp;           // per matrix
    const void *const *G;
    float *const *M;
    void *const *W;
    float *const *U;                  // entries may be NULL
    float *const *Cout;               // coefficients C = P Q before normalisation; entries may be NULL
    const float *const *Q;
    // workspace regions per matrix
    int8_t *const *S;                 // sign codes m x n
    float *const *C;                  // fp32 coefficients m x n (identity / column-l2 norms)
    float *const *colscale;           // n column scales (column-l2)
    double *const *colpart;           // column-l2, nb <= 128: per 128-row tile, column sums of squares
    uint16_t *const *planes;          // bf16 planes of Q (bf16 path)
};
hipError_t launch_step(const StepArgs &a, hipStream_t s);
// M <- mu M + G for matrices c0 .. c0 + cnt - 1 of a (k_step.hip)
hipError_t launch_momentum(const StepArgs &a, int c0, int cnt, hipStream_t s);
// The Dobb-G step (k_step_g.hip): blocks of sh.nb rows, bases a.Q = P (m / nb blocks); cnt <= kMaxMats.
// Workspace per matrix: sign codes (m x n bytes), or fp32 coefficients (m x n) and row scales (m).
size_t step_g_ws_one(const dobb_shape &sh, int norm);
hipError_t launch_step_g(const StepArgs &a, hipStream_t s);
// bf16 basis <-> fp32 copy (k_basis.hip): cnt <= kMaxMats matrices of `elems` entries each
hipError_t launch_basis_convert(int cnt, const void *const *src, void *const *dst, int64_t elems, bool to_f32,
                                hipStream_t s);
// fp32-accurate bf16-split path for the sign norm (nb <= 512, nb % 4 == 0)
bool step_bf16_eligible(const dobb_shape &sh, int norm);
size_t step_bf16_ws_one(const dobb_shape &sh);
int step_bf16_ldp(int64_t nb);
hipError_t launch_step_bf16(const StepArgs &a, hipStream_t s);
// nb <= 128 (nb % 4 == 0): the whole sign step in one pass, the block's basis resident in LDS and
// every wave on its own 16-row tiles (k_step_fused.hip); 16-byte aligned M, G, W, U, C (8 bytes for
// bf16 G and W)
bool step_fused_eligible(const dobb_shape &sh);
hipError_t launch_step_fused(const StepArgs &a, hipStream_t s);
// column-l2 reconstruction for nb <= 128 (nb % 4 == 0) from C and the column scales, split fp16 products
bool recon_l2_rows_eligible(const dobb_shape &sh);
hipError_t launch_recon_l2_rows(const StepArgs &a, int c0, int cnt, hipStream_t s);
// column-l2 projection for the same shapes: momentum, C, the tiles' column sums of squares, the scales
bool proj_l2_rows_eligible(const dobb_shape &sh);
hipError_t launch_proj_l2_rows(const StepArgs &a, int c0, int cnt, hipStream_t s);
// 128 < nb <= 512: basis streamed in k-slices from slice-major planes, row tiles staged in LDS
bool step_wide_eligible(const dobb_shape &sh);
size_t step_wide_planes_bytes(const dobb_shape &sh);
hipError_t launch_step_wide(const StepArgs &a, int ldp, hipStream_t s);
// column-l2 for the same widths (k_step_wide.hip): matrices c0 .. c0 + cnt - 1 of a (cnt <= kMaxMats),
// a.planes the basis planes (step_wide_planes_bytes each), a.C / a.colscale as for the fp32 kernels
hipError_t launch_step_wide_l2(const StepArgs &a, int c0, int cnt, hipStream_t s);
// the column scales 1 / ||C[:, j]|| of a.C into a.colscale (k_step.hip)
hipError_t launch_colnorm(const StepArgs &a, int c0, int cnt, hipStream_t s);

struct AccumulateArgs {
    int count;
    dobb_shape sh;
    dobb_dtype x_dtype;
    int64_t N;
    const int64_t *ldx;               // per matrix
    const void *const *X;
    float *const *A;
    float beta;
    double *partial;                  // split-K partial sums (whole group), may be NULL if nsplit == 1
    int nsplit;
};
int accumulate_splits(const dobb_shape &sh, int64_t N, int count, bool bf16);
size_t accumulate_ws(const dobb_shape &sh, int64_t N, int count);
hipError_t launch_accumulate(const AccumulateArgs &a, hipStream_t s);

struct RefreshArgs {
    int count;
    dobb_shape sh;
    const float *const *A;
    float *const *Q;
    float *const *lambda;             // entries may be NULL
    int32_t *const *info;             // entries may be NULL
    dobb_refresh_mode mode;
    int iters;
    int warm;
    float tol;
    void *ws;                         // scratch for the whole group
};
size_t refresh_ws(const dobb_shape &sh, int count);
hipError_t launch_refresh(const RefreshArgs &a, hipStream_t s);
// Householder QR of every block of a launch, nb <= 512.  Z: the blocks of the launch, dense nb x nb
// each (overwritten); tq: npanel x 32 x 32 fp32 per block; negs: nb bytes per block.
bool qr_block_supported(int64_t nb);
// Cholesky QR (k_cholqr.hip): per block, R with R^T R = G overwrites G's upper part and X = R^{-1};
// flag[g] records a non-positive pivot (first: set, else or-ed in)
bool chol_supported(int64_t nb);
hipError_t launch_chol_inv(int nb, int nblocks, float *G, float *X, int32_t *flag, int first, hipStream_t s);
hipError_t launch_chol_info(int nblk, int nblocks, const int32_t *flag, int32_t *const *info, int cnt, int info_value,
                            hipStream_t s);
hipError_t launch_qr_block(int nb, int nblk, int cnt, float *Z, float *tq, int8_t *negs, float *const *Q,
                           int32_t *const *info, int info_value, hipStream_t s);

}  // namespace dobb

#define DOBB_LAUNCH(name, stream, kernel, grid, block, shmem, ...)                          \
    do {                                                                                    \
        ::dobb::prof_before(name, stream);                                                  \
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                \
        ::dobb::prof_after(stream);                                                         \
    } while (0)
