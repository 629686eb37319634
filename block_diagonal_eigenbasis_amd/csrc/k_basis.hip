// Basis storage in bf16 (Table 18 of the Dobb paper, arXiv 2610.39412: fp32 second moments with a
// bf16 basis is the principal precision setting).  The refresh and step kernels compute with an fp32
// basis; a bf16 basis is widened exactly into an fp32 copy in the workspace before them and, after a
// refresh, rounded back to bf16 (nearest even) once.
#include "dobb_internal.h"

namespace dobb {
namespace {

struct ConvTable {
    const void *src[kMaxMats];
    void *dst[kMaxMats];
};

// grid = (chunks of 1024 elements, matrices), block 256: 4 consecutive elements per thread
template <bool TO_F32>
__global__ void __launch_bounds__(256) k_basis_convert(int64_t elems, ConvTable t) {
    const int mat = blockIdx.y;
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (TO_F32) {
        const uint16_t *s = (const uint16_t *)t.src[mat];
        float *d = (float *)t.dst[mat];
        if (e0 + 4 <= elems && (elems & 3) == 0) {
            const uint2 h = *(const uint2 *)(s + e0);
            *(f32x4 *)(d + e0) = f32x4{bf16_to_f32((uint16_t)h.x), bf16_to_f32((uint16_t)(h.x >> 16)),
                                       bf16_to_f32((uint16_t)h.y), bf16_to_f32((uint16_t)(h.y >> 16))};
        } else {
            for (int64_t e = e0; e < e0 + 4 && e < elems; ++e) d[e] = bf16_to_f32(s[e]);
        }
    } else {
        const float *s = (const float *)t.src[mat];
        uint16_t *d = (uint16_t *)t.dst[mat];
        if (e0 + 4 <= elems && (elems & 3) == 0) {
            const f32x4 v = *(const f32x4 *)(s + e0);
            *(uint2 *)(d + e0) = uint2{(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                                       (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
        } else {
            for (int64_t e = e0; e < e0 + 4 && e < elems; ++e) d[e] = f32_to_bf16(s[e]);
        }
    }
}

}  // namespace

hipError_t launch_basis_convert(int cnt, const void *const *src, void *const *dst, int64_t elems, bool to_f32,
                                hipStream_t s) {
    if (cnt < 1 || cnt > kMaxMats || elems < 1) return hipErrorInvalidValue;
    ConvTable t{};
    for (int i = 0; i < cnt; ++i) { t.src[i] = src[i]; t.dst[i] = dst[i]; }
    const dim3 grid((unsigned)((elems + 1023) / 1024), (unsigned)cnt);
    if (to_f32) DOBB_LAUNCH("basis_widen", s, k_basis_convert<true>, grid, dim3(256), 0, elems, t);
    else DOBB_LAUNCH("basis_narrow", s, k_basis_convert<false>, grid, dim3(256), 0, elems, t);
    return hipGetLastError();
}

}  // namespace dobb
