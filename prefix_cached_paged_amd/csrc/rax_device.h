// Device-side helpers shared by the librax kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rax {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kWave = 64;

// log2(e): scores are scaled by sm_scale * log2(e) once so that the softmax uses exp2.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 -> packed bf16x2 (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Pick 16-bit element `e` (0..7, compile-time) out of a 16-byte register quad.
template <int E>
__device__ __forceinline__ uint32_t half_of(const uint4& v) {
    const uint32_t w = (E / 2 == 0) ? v.x : (E / 2 == 1) ? v.y : (E / 2 == 2) ? v.z : v.w;
    return (E & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Same for a 4-element (8-byte) register pair.
template <int E>
__device__ __forceinline__ uint32_t half_of(const uint2& v) {
    const uint32_t w = (E / 2 == 0) ? v.x : v.y;
    return (E & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Column E of an 8x8 (rows r[0..7]) block of 16-bit values, as one 16-byte operand:
// out element j = r[j] element E. Pure register moves (byte permutes).
template <int E, typename Row>
__device__ __forceinline__ uint4 column8(const Row (&r)[8]) {
    uint4 o;
    o.x = half_of<E>(r[0]) | (half_of<E>(r[1]) << 16);
    o.y = half_of<E>(r[2]) | (half_of<E>(r[3]) << 16);
    o.z = half_of<E>(r[4]) | (half_of<E>(r[5]) << 16);
    o.w = half_of<E>(r[6]) | (half_of<E>(r[7]) << 16);
    return o;
}

// The values of lanes l and l ^ 32 (pair32) or l ^ 16 (pair16), in some order, in every lane:
// the gfx950 permlane swaps of a register with itself, one VALU operation, no LDS.
__device__ __forceinline__ void pair32(float v, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_pair32(float v) { float a, b; pair32(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max_pair16(float v) { float a, b; pair16(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_pair32(float v) { float a, b; pair32(v, a, b); return a + b; }
__device__ __forceinline__ float sum_pair16(float v) { float a, b; pair16(v, a, b); return a + b; }

// FP8 E4M3 -> bf16: every E4M3 value (finite or NaN) is exactly a bf16 value, so the widening
// rounds nothing. bf16x2_of_e4m3<HI> widens bytes 2 HI, 2 HI + 1 of w in one gfx950
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 (the same bits as v_cvt_pk_f32_fp8 followed by
// v_cvt_pk_bf16_f32, for all 2^16 byte pairs of either half); widen8 turns 8 bytes into 8 bf16
// in byte order.
template <bool HI>
__device__ __forceinline__ uint32_t bf16x2_of_e4m3(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}
__device__ __forceinline__ uint4 widen8(uint2 x) {
    return make_uint4(bf16x2_of_e4m3<false>(x.x), bf16x2_of_e4m3<true>(x.x),
                      bf16x2_of_e4m3<false>(x.y), bf16x2_of_e4m3<true>(x.y));
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, kWave));
}

}  // namespace rax
