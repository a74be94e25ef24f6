// common.h -- device helpers shared by the gfx950 kernels of the routed expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

#define MOE_WAVE 64

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed BF16 (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16(f, 0.0f) & 0xFFFFu; }

// sigmoid(z) = 1 / (1 + 2^(-z log2 e)) with the hardware exp2 and reciprocal
// (about 1 ulp each); for very negative z the exponential overflows to +inf and
// the reciprocal gives 0, so silu(z) = z sigmoid(z) tends to -0, and to z for large z.
__device__ __forceinline__ float sigmoid_f(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// erf(x) by Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// for x >= 0, erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2) with
// t = 1 / (1 + p x), absolute error at most 1.5e-7; odd in x.  One reciprocal, one exp2
// and five FMAs, about the cost of a sigmoid (the device library's erff made the GeGLU
// epilogue 20 % slower than the SwiGLU one).
__device__ __forceinline__ float erf_as(float x) {
    const float ax = __builtin_fabsf(x);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
    float poly = 1.061405429f;
    poly = __builtin_fmaf(poly, t, -1.453152027f);
    poly = __builtin_fmaf(poly, t, 1.421413741f);
    poly = __builtin_fmaf(poly, t, -0.284496736f);
    poly = __builtin_fmaf(poly, t, 0.254829592f);
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * ax * ax);
    const float r = 1.0f - poly * t * e;
    return __builtin_copysignf(r, x);
}

// Gated activations of the W13 output (nvfp4moe README, "Supported kernel surface":
// SwiGLU, GeGLU and ReGLU FC1 epilogues): a = f(g) * u with f = silu, the exact (erf)
// GELU z Phi(z), or max(z, 0); act_df is f' for the backward (Phi(z) + z phi(z) for the
// GELU, with erf_as and the hardware exp2).
constexpr int kActSwiGLU = 0, kActGeGLU = 1, kActReGLU = 2;
template <int kAct> __device__ __forceinline__ float act_f(float z) {
    if constexpr (kAct == kActGeGLU) return 0.5f * z * (1.0f + erf_as(z * 0.70710678118654752f));
    else if constexpr (kAct == kActReGLU) return z > 0.0f ? z : 0.0f;
    else return silu_f(z);
}
// f and f' together (the GELU's Phi computed once)
template <int kAct> __device__ __forceinline__ void act_f_df(float z, float& f, float& df) {
    if constexpr (kAct == kActGeGLU) {
        const float cdf = 0.5f * (1.0f + erf_as(z * 0.70710678118654752f));
        f = z * cdf;
        df = cdf + z * 0.39894228040143268f * __builtin_amdgcn_exp2f(-0.72134752044448170f * z * z);
    } else if constexpr (kAct == kActReGLU) {
        f = z > 0.0f ? z : 0.0f;
        df = z > 0.0f ? 1.0f : 0.0f;
    } else {
        const float sg = sigmoid_f(z);
        f = z * sg;
        df = sg * (1.0f + z * (1.0f - sg));
    }
}
template <int kAct> __device__ __forceinline__ float act_df(float z) {
    if constexpr (kAct == kActGeGLU)
        return 0.5f * (1.0f + erf_as(z * 0.70710678118654752f)) +
               z * 0.39894228040143268f * __builtin_amdgcn_exp2f(-0.72134752044448170f * z * z);
    else if constexpr (kAct == kActReGLU) return z > 0.0f ? 1.0f : 0.0f;
    else {
        const float sg = sigmoid_f(z);
        return sg * (1.0f + z * (1.0f - sg));
    }
}

// OCP MX conversion (E4M3 elements, E8M0 block scale) shared by the quantizer and
// the MXFP8 W13 epilogue.
// E4M3 (OCP "E4M3FN") codes of four finite floats, nearest even, saturating at +-448,
// packed little-endian (a in bits 0..7): gfx950's f32 -> FP8 conversion (OCP E4M3 on
// this target), two values per instruction, after a med3 clamp to +-448.  The plain
// definition it stands for: from 2^-6 up, round the mantissa to 3 bits (a carry steps
// the exponent) and rebias the exponent from 127 to 7, saturating past 448; below 2^-6,
// the nearest-even count of 2^-9 steps; the sign bit is kept, also on zero.  The two
// agree on every finite float (all 2^32 patterns were compared on the GPU, with this
// library's compile flags, against that definition written out in integer arithmetic).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    auto sat = [](float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
    return (uint32_t)w;
}

// E8M0 byte of a block whose largest magnitude is amax (any finite float): the smallest
// power of two X with amax / X <= 448 (E4M3's largest normal), so no element saturates.
// With amax = m 2^e, m in [1, 2): log2 X = e - 8, or e - 7 when m > 1.75 (the significand
// field above 0x600000), biased by 127 and clamped to [0, 254]; zero and FP32 subnormals
// give 0
__device__ __forceinline__ uint32_t e8m0_scale(float amax) {
    const uint32_t bits = __float_as_uint(amax);
    const int ef = (int)((bits >> 23) & 0xFF);   // 0 for zero / subnormal
    if (ef == 0) return 0u;
    int b = ef - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);   // (ef - 127) - 8 [+ 1] + 127
    b = b < 0 ? 0 : (b > 254 ? 254 : b);
    return (uint32_t)b;
}

// Streaming (non-temporal) store of 16 bytes, for whole-line outputs no nearby kernel
// reads back from cache: written through L2 as ordinary stores, they evict operand
// lines the other workgroups of the XCD are still reading.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(void* p, uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    uint32_t l = __lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}
