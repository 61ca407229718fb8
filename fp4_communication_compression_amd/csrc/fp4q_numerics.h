// fp4q_numerics.h -- the scalar operations on which the kernels' agreement with
// the method's fp32 definition rests.  The kernels (fp4q.hip) use them, and the
// test suite's exhaustive instruction checks run the same functions over every
// input pattern of their domains.
//
// What each promises (and the checks confirm on the GPU):
//   rcp_rn        correctly rounded 1/x for 2^-125 <= |x| < 2^125;
//   div_rn        correctly rounded a/b for a >= 2^-99 and b in rcp_rn's range,
//                 given y = rcp_rn(b);
//   coarse_scale  correctly rounded A/2688 for A >= 2^-100;
//   e4m3_pair     OCP E4M3FN round-to-nearest-even of values in [0, 448];
//   e2m1_pair     E2M1 round-to-nearest-even of v / scale (scale a power of
//                 two, 1 in the dual-scale kernels), saturating at 6, keeping
//                 the sign of v;
//   e2m1_values / e4m3_value   exact decodes;
//   e2m1_halves   the same E2M1 values as binary16 (exact: every E2M1 value
//                 times a power of two in [2^-14, 2^4] is a binary16 normal);
//   fma_half      fma(h, b, c) of a binary16 h and binary32 b, c, rounded once
//                 to binary32, exactly as fmaf((float)h, b, c);
//   bf16_rne_pair round-to-nearest-even to bfloat16.
#pragma once

#include <hip/hip_runtime.h>

namespace fp4q_num {

// Hardware reciprocal estimate and one Newton step.
__device__ __forceinline__ float rcp_rn(float x) {
    const float y = __builtin_amdgcn_rcpf(x);
    const float e = fmaf(-x, y, 1.0f);
    return fmaf(e, y, y);
}

// q = a y, then one remainder correction; the remainder a - q b is exact for
// a >= 2^-99 and normal b.
__device__ __forceinline__ float div_rn(float a, float b, float y) {
    const float q = a * y;
    const float r = fmaf(-q, b, a);
    return fmaf(r, y, q);
}

// 2688 = 6 * 448: the block's largest micro-group takes the top of the E4M3 range.
constexpr float kScaleDivisor = 2688.0f;
__device__ __forceinline__ float coarse_scale(float A) {
    return div_rn(A, kScaleDivisor, 1.0f / kScaleDivisor);
}

// Largest finite E4M3FN value; the conversion itself gives NaN above 464, so
// callers clamp to this first.
constexpr float kE4M3Max = 448.0f;

// E4M3 codes of t0, t1 (in [0, 448]) into bytes 0, 1 (kHi = false) or 2, 3 of old.
template <bool kHi>
__device__ __forceinline__ unsigned e4m3_pair(unsigned old, float t0, float t1) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, old, kHi);
}

// The value of E4M3 byte kByte of w.
template <int kByte>
__device__ __forceinline__ float e4m3_value(unsigned w) {
    return __builtin_amdgcn_cvt_f32_fp8(w, kByte);
}

// E2M1 codes of v0 / scale (low nibble) and v1 / scale into byte kSel of old.
template <int kSel>
__device__ __forceinline__ unsigned e2m1_pair(unsigned old, float v0, float v1, float scale = 1.0f) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, v0, v1, scale, kSel);
}

// Values of the two E2M1 codes in byte kSel of w (low nibble first), times scale.
template <int kSel>
__device__ __forceinline__ auto e2m1_values(unsigned w, float scale = 1.0f) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, kSel);
}

// Values of the two E2M1 codes in byte kSel of w as binary16 (low nibble in
// element 0), times scale (a power of two keeping them binary16 normals).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <int kSel>
__device__ __forceinline__ f16x2 e2m1_halves(unsigned w, float scale = 1.0f) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, kSel);
}

// fma with a binary16 first factor (one mixed-precision instruction): the
// conversion of h is exact, so the result is fmaf((float)h, b, c).
__device__ __forceinline__ float fma_half(_Float16 h, float b, float c) {
    return __builtin_fmaf((float)h, b, c);
}

// Two fp32 values rounded to nearest-even bfloat16, lo in the low half
// (denormals kept, as the whole library is built).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned bf16_rne_pair(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

}  // namespace fp4q_num
