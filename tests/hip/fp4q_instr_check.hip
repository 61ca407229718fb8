// fp4q_instr_check.hip -- TEST-ONLY library: exhaustive GPU checks of the scalar
// operations in fp4q_numerics.h, the functions the kernels use for every
// rounding decision.  Each sweep runs the function under test over a range of
// fp32 bit patterns (or counter-based random operands) on the GPU and compares
// it there with an expectation the host supplies from the oracle (rounding
// thresholds) or with the IEEE operation it must equal.  Mismatches are counted
// in a device result {count, first mismatching pattern}; the host stops at the
// first chunk that reports one.
//
// Every kernel reads only its arguments and its small input arrays (bounds
// checked) and writes only its result words or its bounded output arrays.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fp4q_numerics.h"

namespace {

using namespace fp4q_num;

constexpr int kThreads = 256;
constexpr int kPer = 16;  // patterns per thread

struct Result {
    unsigned long long count;
    unsigned long long first;
};

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

__device__ __forceinline__ void report(Result *res, unsigned long long bad, unsigned long long first) {
    if (bad) {
        atomicAdd(&res->count, bad);
        atomicMin(&res->first, first);
    }
}

// Expected E2M1 code of x / 2^k from the oracle's thresholds: thr[m - 1] is the
// smallest magnitude that rounds to magnitude code m (m = 1..7), in fp64 and
// already multiplied by 2^k; the sign bit follows the sign of x (neg_zero: the
// code of a negative value whose magnitude rounds to 0).
struct E2M1Thresholds {
    double thr[7];
    int neg_zero;
};

__device__ __forceinline__ unsigned e2m1_expect(float x, const E2M1Thresholds &T) {
    const double u = fabs((double)x);
    unsigned mag = 0;
#pragma unroll
    for (int m = 0; m < 7; ++m) mag += u >= T.thr[m] ? 1u : 0u;
    if (signbit(x)) return mag ? (mag | 8u) : (unsigned)T.neg_zero;
    return mag;
}

// All finite fp32 patterns in [begin, begin + count): e2m1_pair at scale 2^k
// (the kernels' E2M1 rounding) against the thresholds.
__global__ __launch_bounds__(kThreads) void e2m1_sweep(uint64_t begin, uint64_t count, float scale,
                                                        E2M1Thresholds T, Result *res) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    unsigned long long bad = 0, first = ~0ull;
#pragma unroll
    for (int j = 0; j < kPer; j += 2) {
        const uint64_t i0 = base + j, i1 = base + j + 1;
        if (i0 >= count) break;
        const uint32_t u0 = (uint32_t)(begin + i0), u1 = i1 < count ? (uint32_t)(begin + i1) : u0;
        const float x0 = as_f(u0), x1 = as_f(u1);
        const unsigned c = e2m1_pair<0>(0u, x0, x1, scale) & 0xFFu;
        const bool fin0 = (u0 & 0x7F800000u) != 0x7F800000u, fin1 = (u1 & 0x7F800000u) != 0x7F800000u;
        if (fin0 && (c & 15u) != e2m1_expect(x0, T)) {
            ++bad;
            first = first < begin + i0 ? first : begin + i0;
        }
        if (i1 < count && fin1 && (c >> 4) != e2m1_expect(x1, T)) {
            ++bad;
            first = first < begin + i1 ? first : begin + i1;
        }
    }
    report(res, bad, first);
}

// E4M3 of t >= 0 as the compress kernel takes it: fminf(t, 448), then the
// conversion; expected: the number of oracle thresholds (126, ascending: the
// smallest t of each code 1..126) at or below t.
__device__ __forceinline__ unsigned e4m3_expect(float t, const float *__restrict__ thr) {
    int lo = 0, hi = 126;  // count of thr[i] <= t lies in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (thr[mid - 1] <= t) lo = mid; else hi = mid - 1;
    }
    return (unsigned)lo;
}

__global__ __launch_bounds__(kThreads) void e4m3_sweep(uint64_t begin, uint64_t count,
                                                        const float *__restrict__ thr, Result *res) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    unsigned long long bad = 0, first = ~0ull;
#pragma unroll
    for (int j = 0; j < kPer; j += 2) {
        const uint64_t i0 = base + j, i1 = base + j + 1;
        if (i0 >= count) break;
        const uint32_t u0 = (uint32_t)(begin + i0), u1 = i1 < count ? (uint32_t)(begin + i1) : u0;
        const float t0 = as_f(u0), t1 = as_f(u1);
        const unsigned c = e4m3_pair<false>(0u, fminf(t0, kE4M3Max), fminf(t1, kE4M3Max));
        if ((c & 0xFFu) != e4m3_expect(t0, thr)) {
            ++bad;
            first = first < begin + i0 ? first : begin + i0;
        }
        if (i1 < count && ((c >> 8) & 0xFFu) != e4m3_expect(t1, thr)) {
            ++bad;
            first = first < begin + i1 ? first : begin + i1;
        }
    }
    report(res, bad, first);
}

// rcp_rn(x) against IEEE 1/x, bit for bit.
__global__ __launch_bounds__(kThreads) void rcp_sweep(uint64_t begin, uint64_t count, Result *res) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    unsigned long long bad = 0, first = ~0ull;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint64_t i = base + j;
        if (i >= count) break;
        const float x = as_f((uint32_t)(begin + i));
        if (as_u(rcp_rn(x)) != as_u(1.0f / x)) {
            ++bad;
            first = first < begin + i ? first : begin + i;
        }
    }
    report(res, bad, first);
}

// coarse_scale(A) against IEEE A / 2688, bit for bit.
__global__ __launch_bounds__(kThreads) void scale_sweep(uint64_t begin, uint64_t count, Result *res) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    unsigned long long bad = 0, first = ~0ull;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint64_t i = base + j;
        if (i >= count) break;
        const float A = as_f((uint32_t)(begin + i));
        if (as_u(coarse_scale(A)) != as_u(A / kScaleDivisor)) {
            ++bad;
            first = first < begin + i ? first : begin + i;
        }
    }
    report(res, bad, first);
}

__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// The micro-scale division as compress makes it, on random blocks: a block
// maximum A in [2^-80, 2^122) (exponent uniform, random significand), a group
// maximum a in [0, A] (exponent uniform over the 48 binades below A's, random
// significand, or a = A exactly one time in 16), d6 = 6 coarse_scale(A),
// t = div_rn(a, d6, rcp_rn(d6)).  For a >= 2^-99, t must equal IEEE a / d6 bit
// for bit; below (where the remainder may round), its E4M3 code must equal the
// code of the IEEE quotient.  res->first records the random index.
__global__ __launch_bounds__(kThreads) void micro_div_random(uint64_t seed, uint64_t begin, uint64_t count,
                                                              Result *res) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    unsigned long long bad = 0, first = ~0ull;
#pragma unroll 4
    for (int j = 0; j < kPer; ++j) {
        const uint64_t i = base + j;
        if (i >= count) break;
        const uint64_t r0 = splitmix64(seed ^ (2 * (begin + i))), r1 = splitmix64(seed ^ (2 * (begin + i) + 1));
        const int eA = -80 + (int)((r0 >> 32) % 202u);           // [-80, 121]
        const float A = as_f(((uint32_t)(eA + 127) << 23) | ((uint32_t)r0 & 0x7FFFFFu));
        float a;
        if (((r1 >> 60) & 15u) == 0) {
            a = A;
        } else {
            const int ea = eA - (int)((r1 >> 32) % 48u);
            const uint32_t m = (uint32_t)r1 & 0x7FFFFFu;
            a = ea >= -126 ? as_f(((uint32_t)(ea + 127) << 23) | m) : as_f(m >> (-126 - ea > 23 ? 23 : -126 - ea));
            a = fminf(a, A);
        }
        const float d6 = 6.0f * coarse_scale(A);
        const float t = div_rn(a, d6, rcp_rn(d6));
        const float ref = a / d6;
        bool ok;
        if (a >= 0x1p-99f) {
            ok = as_u(t) == as_u(ref);
        } else {
            const unsigned c1 = e4m3_pair<false>(0u, fminf(t, kE4M3Max), 0.0f) & 0xFFu;
            const unsigned c2 = e4m3_pair<false>(0u, fminf(ref, kE4M3Max), 0.0f) & 0xFFu;
            ok = c1 == c2;
        }
        if (!ok) {
            ++bad;
            first = first < begin + i ? first : begin + i;
        }
    }
    report(res, bad, first);
}

// The binary16 decode and mixed-precision fused multiply-add against the
// binary32 ones, on random operands: code c (4 bits), b and c with random bit
// patterns (finite), decoded at scale 2^k for k in {0, -4}.  Checks, bit for bit
// (NaN against NaN): fma_half(h, b, c) == fmaf(v, b, c) and
// fma_half(h, b, -0) == v * b, where h and v are the binary16 and binary32
// decodes of the same code.
__device__ __forceinline__ bool same_bits(float a, float b) {
    return as_u(a) == as_u(b) || (a != a && b != b);
}

__device__ __forceinline__ float random_finite(uint64_t r) {
    uint32_t u = (uint32_t)r;
    if ((u & 0x7F800000u) == 0x7F800000u) u ^= 0x40000000u;  // no Inf or NaN
    // one draw in four from a narrower, typical exponent range [2^-40, 2^40)
    if (((r >> 32) & 3u) == 0) u = (u & 0x807FFFFFu) | ((uint32_t)(87 + ((r >> 40) % 80u)) << 23);
    return as_f(u);
}

__global__ __launch_bounds__(kThreads) void half_fma_random(uint64_t seed, uint64_t begin, uint64_t count,
                                                             Result *res) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    unsigned long long bad = 0, first = ~0ull;
#pragma unroll 4
    for (int j = 0; j < kPer; ++j) {
        const uint64_t i = base + j;
        if (i >= count) break;
        const uint64_t r0 = splitmix64(seed ^ (3 * (begin + i))), r1 = splitmix64(seed ^ (3 * (begin + i) + 1)),
                       r2 = splitmix64(seed ^ (3 * (begin + i) + 2));
        const unsigned code = (unsigned)(r2 >> 60) & 15u;
        const float scale = (r2 >> 59) & 1u ? 0.0625f : 1.0f;
        const float b = random_finite(r0), c = ((r2 >> 58) & 1u) ? random_finite(r1) : ((r2 >> 57) & 1u ? -0.0f : 0.0f);
        const float v = e2m1_values<0>(code | (code << 4), scale)[0];
        const _Float16 h = e2m1_halves<0>(code | (code << 4), scale)[0];
        const bool ok = same_bits(fma_half(h, b, c), fmaf(v, b, c)) && same_bits(fma_half(h, b, -0.0f), v * b) &&
                        same_bits((float)h, v);
        if (!ok) {
            ++bad;
            first = first < begin + i ? first : begin + i;
        }
    }
    report(res, bad, first);
}

// bf16_rne_pair against integer round-to-nearest-even on the bit pattern
// (finite inputs; overflow rounds to infinity, as the integer form gives).
__device__ __forceinline__ unsigned bf16_expect(uint32_t u) {
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kThreads) void bf16_sweep(uint64_t begin, uint64_t count, Result *res) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    unsigned long long bad = 0, first = ~0ull;
#pragma unroll
    for (int j = 0; j < kPer; j += 2) {
        const uint64_t i0 = base + j, i1 = base + j + 1;
        if (i0 >= count) break;
        const uint32_t u0 = (uint32_t)(begin + i0), u1 = i1 < count ? (uint32_t)(begin + i1) : u0;
        const unsigned r = bf16_rne_pair(as_f(u0), as_f(u1));
        const bool fin0 = (u0 & 0x7F800000u) != 0x7F800000u, fin1 = (u1 & 0x7F800000u) != 0x7F800000u;
        if (fin0 && (r & 0xFFFFu) != bf16_expect(u0)) {
            ++bad;
            first = first < begin + i0 ? first : begin + i0;
        }
        if (i1 < count && fin1 && (r >> 16) != bf16_expect(u1)) {
            ++bad;
            first = first < begin + i1 ? first : begin + i1;
        }
    }
    report(res, bad, first);
}

// Element-wise evaluation for the host's cross-checks against the oracle:
// what = 0: E2M1 code at scale 1;  1: E4M3 code of fminf(t, 448);  2: rcp_rn;
// 3: bf16 rounding.  out[i] holds the code, or the result's bit pattern.
__global__ __launch_bounds__(kThreads) void eval_kernel(int what, const float *__restrict__ in, int64_t n,
                                                         uint32_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const float x = in[i];
    uint32_t r;
    switch (what) {
        case 0: r = e2m1_pair<0>(0u, x, 0.0f) & 15u; break;
        case 1: r = e4m3_pair<false>(0u, fminf(x, kE4M3Max), 0.0f) & 0xFFu; break;
        case 2: r = as_u(rcp_rn(x)); break;
        default: r = bf16_rne_pair(x, 0.0f) & 0xFFFFu; break;
    }
    out[i] = r;
}

// Decode tables: out[0..255] = e4m3_value of every byte; then, for each of
// nscales scales, the 16 E2M1 values at that scale; then the same through the
// binary16 decode (meaningful where the values are binary16 normals).  One
// thread per entry.
__global__ __launch_bounds__(kThreads) void decode_kernel(const float *__restrict__ scales, int nscales,
                                                           float *__restrict__ out) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < 256) {
        out[i] = e4m3_value<0>((unsigned)i);
    } else if (i < 256 + 16 * nscales) {
        const int s = (i - 256) / 16, c = (i - 256) % 16;
        // code c in both nibbles of byte 0: the low one decodes to f[0]
        const auto f = e2m1_values<0>((unsigned)(c | (c << 4)), scales[s]);
        out[i] = f[0];
    } else if (i < 256 + 32 * nscales) {
        const int s = (i - 256 - 16 * nscales) / 16, c = (i - 256) % 16;
        out[i] = (float)e2m1_halves<0>((unsigned)(c | (c << 4)), scales[s])[0];
    }
}

int launch_sweep(const void *fn, void **args, uint64_t count, void *stream) {
    const uint64_t per_block = (uint64_t)kThreads * kPer;
    const uint64_t blocks = (count + per_block - 1) / per_block;
    if (count == 0 || blocks > 0x7FFFFFFFull) return -1;
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0,
                                         (hipStream_t)stream);
    return e == hipSuccess ? 0 : -2;
}

}  // namespace

extern "C" {

// Each sweep: patterns (or random indices) [begin, begin + count), count <= 2^32;
// res: device pointer to {count, first} (the caller clears count and sets first
// to all ones).  Returns 0, or -1 for bad arguments, -2 for a failed launch.
int ic_e2m1_sweep(uint64_t begin, uint64_t count, float scale, const double *thr7, int neg_zero,
                  void *res, void *stream) {
    if (!thr7 || !res || count > (1ull << 32)) return -1;
    E2M1Thresholds T;
    for (int m = 0; m < 7; ++m) T.thr[m] = thr7[m];
    T.neg_zero = neg_zero;
    void *args[] = {&begin, &count, &scale, &T, &res};
    return launch_sweep((const void *)&e2m1_sweep, args, count, stream);
}

int ic_e4m3_sweep(uint64_t begin, uint64_t count, const float *thr126_dev, void *res, void *stream) {
    if (!thr126_dev || !res || count > (1ull << 32)) return -1;
    void *args[] = {&begin, &count, &thr126_dev, &res};
    return launch_sweep((const void *)&e4m3_sweep, args, count, stream);
}

int ic_rcp_sweep(uint64_t begin, uint64_t count, void *res, void *stream) {
    if (!res || count > (1ull << 32)) return -1;
    void *args[] = {&begin, &count, &res};
    return launch_sweep((const void *)&rcp_sweep, args, count, stream);
}

int ic_scale_sweep(uint64_t begin, uint64_t count, void *res, void *stream) {
    if (!res || count > (1ull << 32)) return -1;
    void *args[] = {&begin, &count, &res};
    return launch_sweep((const void *)&scale_sweep, args, count, stream);
}

int ic_micro_div_random(uint64_t seed, uint64_t begin, uint64_t count, void *res, void *stream) {
    if (!res || count > (1ull << 32)) return -1;
    void *args[] = {&seed, &begin, &count, &res};
    return launch_sweep((const void *)&micro_div_random, args, count, stream);
}

int ic_half_fma_random(uint64_t seed, uint64_t begin, uint64_t count, void *res, void *stream) {
    if (!res || count > (1ull << 32)) return -1;
    void *args[] = {&seed, &begin, &count, &res};
    return launch_sweep((const void *)&half_fma_random, args, count, stream);
}

int ic_bf16_sweep(uint64_t begin, uint64_t count, void *res, void *stream) {
    if (!res || count > (1ull << 32)) return -1;
    void *args[] = {&begin, &count, &res};
    return launch_sweep((const void *)&bf16_sweep, args, count, stream);
}

int ic_eval(int what, const float *in_dev, int64_t n, uint32_t *out_dev, void *stream) {
    if (!in_dev || !out_dev || n <= 0 || n > (1ll << 30) || what < 0 || what > 3) return -1;
    void *args[] = {&what, &in_dev, &n, &out_dev};
    const hipError_t e = hipLaunchKernel((const void *)&eval_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                                         dim3(kThreads), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? 0 : -2;
}

// out_dev: 256 + 32 * nscales floats.
int ic_decode_tables(const float *scales_dev, int nscales, float *out_dev, void *stream) {
    if (!scales_dev || !out_dev || nscales < 0 || nscales > 4096) return -1;
    const int n = 256 + 32 * nscales;
    void *args[] = {&scales_dev, &nscales, &out_dev};
    const hipError_t e = hipLaunchKernel((const void *)&decode_kernel, dim3((n + kThreads - 1) / kThreads),
                                         dim3(kThreads), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? 0 : -2;
}

}  // extern "C"
