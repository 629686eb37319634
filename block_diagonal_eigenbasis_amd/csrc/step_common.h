// Device helpers shared by the step kernels (k_step_fused.hip, k_step_rows.hip,
// k_step_wide.hip): the operand splits, sign codes and buffer-descriptor access.
#pragma once
#include "dobb_internal.h"

namespace dobb {
namespace stepk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// v = h + m + l in bf16 (round to nearest even; each residual is exact in fp32)
__device__ __forceinline__ void split3(float v, uint16_t &h, uint16_t &m, uint16_t &l) {
    h = bf16_bits(v);
    const float r1 = v - bf16_to_f32(h);
    m = bf16_bits(r1);
    l = bf16_bits(r1 - bf16_to_f32(m));
}
// v = h + l in fp16 (|v| <= 1 for the entries of an orthonormal basis)
__device__ __forceinline__ void split2h(float v, uint16_t &h, uint16_t &l) {
    const _Float16 a = (_Float16)v;
    h = __builtin_bit_cast(uint16_t, a);
    l = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)a));
}
// power-of-two exponent that scales a row whose largest magnitude has fp32 bits `bits` into
// [2^13, 2^14): 14 minus the frexp exponent (biased exponent - 126).  A zero row gets 140 (its
// entries stay zero); an infinite or NaN maximum gets -115 (the row's coefficients become NaN, as
// they would unscaled).
__device__ __forceinline__ int row_scale_exp(uint32_t bits) { return 140 - (int)(bits >> 23); }
// v (already scaled by its row's power of two, |v| < 2^14) = h + l in fp16; the residual v - h is
// exact in fp32, and |v - h - l| <= 2^-22 |v| where l is normal
__device__ __forceinline__ void split2s(float v, uint16_t &h, uint16_t &l) {
    const _Float16 a = (_Float16)v;
    h = __builtin_bit_cast(uint16_t, a);
    l = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)a));
}
// high byte of the fp16 value of sign(c), from the bits of c without branches:
// +1 -> 0x3c, -1 -> 0xbc, 0 -> 0x00, NaN -> 0x7e
__device__ __forceinline__ uint32_t sign_byte(float c) {
    const uint32_t u = __float_as_uint(c);
    const uint32_t mag = u & 0x7fffffffu;
    const uint32_t sb = 0x3cu | ((u >> 24) & 0x80u);
    const uint32_t nz = mag > 0x7f800000u ? 0x7eu : sb;
    return mag == 0u ? 0u : nz;
}
// sign bytes 2J, 2J + 1 of x -> two fp16 values (the byte is the high byte, the low byte is 0)
template <int J>
__device__ __forceinline__ uint32_t signs_f16x2(uint32_t x) {
    return __builtin_amdgcn_perm(0u, x, J == 0 ? 0x010c000cu : 0x030c020cu);
}
// eight sign bytes -> an fp16x8 MFMA operand
__device__ __forceinline__ f16x8 signs_f16x8(uint2 sv) {
    const uint4 av = {signs_f16x2<0>(sv.x), signs_f16x2<1>(sv.x), signs_f16x2<0>(sv.y), signs_f16x2<1>(sv.y)};
    return __builtin_bit_cast(f16x8, av);
}
__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }
// eight fp32 values -> three bf16x8 parts
__device__ __forceinline__ void split3x8(f32x4 p0, f32x4 p1, bf16x8 &ah, bf16x8 &am, bf16x8 &al) {
    uint16_t hh[8], hm[8], hl[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        split3(p0[c], hh[c], hm[c], hl[c]);
        split3(p1[c], hh[c + 4], hm[c + 4], hl[c + 4]);
    }
    ah = __builtin_bit_cast(bf16x8, uint4{pack2(hh[0], hh[1]), pack2(hh[2], hh[3]), pack2(hh[4], hh[5]), pack2(hh[6], hh[7])});
    am = __builtin_bit_cast(bf16x8, uint4{pack2(hm[0], hm[1]), pack2(hm[2], hm[3]), pack2(hm[4], hm[5]), pack2(hm[6], hm[7])});
    al = __builtin_bit_cast(bf16x8, uint4{pack2(hl[0], hl[1]), pack2(hl[2], hl[3]), pack2(hl[4], hl[5]), pack2(hl[6], hl[7])});
}

// Buffer-descriptor access: a lane with nothing to do passes kOff, past the end of the buffer, so
// its load returns zeros and its store is dropped, without a branch around the instruction.
constexpr unsigned kOff = 0xffffffffu;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ unsigned boff(unsigned elem, unsigned size) { return elem == kOff ? kOff : elem * size; }
__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 bload2u(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint4 bload4u(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void bstore4(f32x4 v, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore2u(uint2 v, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore1(float v, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore1h(uint16_t v, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint16_t bload1h(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

}  // namespace stepk
}  // namespace dobb
