// Device helpers shared by the matrix-core decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vk {
namespace mfma {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A product rounded to fp32 and never fused into a later add, so the running
// max and the exponent argument see the same score.
__device__ __forceinline__ float mul_rounded(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

__device__ __forceinline__ floatx4 mfma32(const uint4& a, const uint4& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                   __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(const uint2& a, const uint2& b, const floatx4& c) {
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                  __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
}

// K and V are read exactly once per step: nontemporal (streaming) loads.  On
// MI355X a plain streaming read tops out near 6.0 TB/s and a nontemporal one
// near 6.5 TB/s.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int W>
__device__ __forceinline__ uint32_t word(const uint4& v) {
    return W == 0 ? v.x : W == 1 ? v.y : W == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    half2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Two weights as an fp16 pair (round to nearest even) and the fp16 pair of
// what that rounding left.  a - fp16(a) is exact in fp32 (the two are within
// a factor 2), so hi + lo is within 2^-22 relative of the weight, or 2^-25
// absolute where the residual falls below fp16's normal range (2^-14; 2^-14
// if subnormal operands were flushed).  Callers scale the weights so that
// the largest is between 2^7 and 2^15 (the fp16 range ends at 65504), which
// makes that absolute term negligible next to the largest.  A PV product in
// fp16 takes both pairs (two matrix products): one fp16 weight alone is off
// by up to 2^-11 relative.
__device__ __forceinline__ void pack_half2_split(float a, float b, uint32_t& hi, uint32_t& lo) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const half2_t h = {(_Float16)a, (_Float16)b};
    hi = __builtin_bit_cast(uint32_t, h);
    const half2_t l = {(_Float16)(a - (float)h.x), (_Float16)(b - (float)h.y)};
    lo = __builtin_bit_cast(uint32_t, l);
}

// Max over the four 16-lane rows of a wave (lanes i, i + 16, i + 32, i + 48:
// one matrix-core column), with gfx950's row-swapping permutes: VALU only, no
// LDS round trip as for a shuffle.  permlane32_swap(v, v) leaves lane l with
// v[l] in one result and v[l ^ 32] in the other (rows 0-1 and 2-3 swapped),
// permlane16_swap the same for l ^ 16 (rows 0 and 1, 2 and 3).
__device__ __forceinline__ float max_rows4(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto h = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const float m = fmaxf(__builtin_bit_cast(float, h[0]), __builtin_bit_cast(float, h[1]));
    const uint32_t mb = __builtin_bit_cast(uint32_t, m);
    const auto q = __builtin_amdgcn_permlane16_swap(mb, mb, false, false);
    return fmaxf(__builtin_bit_cast(float, q[0]), __builtin_bit_cast(float, q[1]));
}

// fp32 element type: one k-slot per lane group.
__device__ __forceinline__ floatx4 mfma4_f32(uint32_t a, uint32_t b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a),
                                                 __builtin_bit_cast(float, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma4_f32(float a, float b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 element type (K, V and q as bfloat16): the same products on the bf16
// matrix instructions.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma32_bf16(const uint4& a, const uint4& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16_bf16(const uint2& a, const uint2& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                      __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}

// Two weights as a bf16 pair (round to nearest even) and the pair of what
// that rounding left (a - bf16(a), itself rounded): hi + lo carries a weight
// to about 2^-16 relative, so the PV product done as two bf16 products keeps
// the weights about as exact as the fp16 path does.
__device__ __forceinline__ void pack_bf16_split(float a, float b, uint32_t& hi, uint32_t& lo) {
    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
    const bf2_t h = {(__bf16)a, (__bf16)b};
    hi = __builtin_bit_cast(uint32_t, h);
    const float ah = __builtin_bit_cast(float, hi << 16);
    const float bh = __builtin_bit_cast(float, hi & 0xFFFF0000u);
    const bf2_t l = {(__bf16)(a - ah), (__bf16)(b - bh)};
    lo = __builtin_bit_cast(uint32_t, l);
}

// 4x8 fp16 transpose step for the 16x16x16 product: dim e of the lane
// group's 4 tokens.
template <int E>
__device__ __forceinline__ uint2 vt_operand4(const uint4 (&v)[4]) {
    constexpr uint32_t sel = (E & 1) ? 0x07060302u : 0x05040100u;
    uint2 a;
    a.x = __builtin_amdgcn_perm(word<E / 2>(v[1]), word<E / 2>(v[0]), sel);
    a.y = __builtin_amdgcn_perm(word<E / 2>(v[3]), word<E / 2>(v[2]), sel);
    return a;
}


}  // namespace mfma
}  // namespace vk
