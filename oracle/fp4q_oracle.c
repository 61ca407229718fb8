/*
 * fp4q_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow CPU oracle of the FP4Quant compress / decompress transform.
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load it;
 * the product path never does.  It shares no code with the HIP library.
 *
 * What it follows ("FP4Quant: Efficient 4-Bit Communication Compression for
 * Model-Parallel LLM Training", abstract): a tensor is cut into blocks, each
 * block goes through a two-level fast Walsh-Hadamard transform (FWHT) to reduce
 * quantisation error, then micro-grouped dual-scale FP4 quantisation (one coarse
 * scale per block, one fine scale per micro-group; the zot.news digest: small
 * clusters of values share scaling factors), then packing two 4-bit codes per
 * byte (zot.news digest).  The receiver dequantises, undoes the transform and,
 * as in a tensor-parallel AllReduce (zot.news digest, "Read it as"), sums the
 * payloads of k peers.
 *
 * Constants of this library: block 256 = 16 x 16, FWHT normalised by 1/16,
 * micro-group 16, coarse scale fp32, micro-scale OCP E4M3FN, element code E2M1
 * (values 0, 0.5, 1, 1.5, 2, 3, 4, 6) rounded to nearest-even, low nibble =
 * even element.  Readings of points the pages leave open are listed beside the
 * code that takes them.
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, built with
 * -ffp-contract=off and no fast-math, so every fp32 operation below is one
 * correctly rounded operation in the order written.  The accumulate reference
 * and the error metric are binary64.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLOCK 256
#define GROUP 16
#define NGROUP (BLOCK / GROUP)

/* ------------------------------------------------------------------ threads */
static int g_threads = 1;
void fp4q_ref_set_threads(int n) { g_threads = n > 0 ? n : 1; }
int fp4q_ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------- bf16 input */
static float widen_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16; /* a bfloat16 is the top half of a binary32 */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------- E2M1 format
 * 4 bits: sign | 2-bit exponent (bias 1) | 1-bit mantissa.  Exponent 0 is
 * subnormal: value m * 0.5.  Otherwise 2^(e-1) * (1 + m/2).  No Inf or NaN. */
float fp4q_ref_e2m1_decode(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -mag : mag;
}

/* Round to nearest E2M1 value, ties to the even mantissa, saturating at 6.
 * Reading: the code keeps the sign of its input, as a float conversion does, so
 * a negative value whose magnitude rounds to 0 gives 0x8 (-0). */
int fp4q_ref_e2m1_encode(float v) {
    float u = fabsf(v);
    int mag = 0;
    for (int c = 0; c < 7; ++c) {
        float lo = fp4q_ref_e2m1_decode(c), hi = fp4q_ref_e2m1_decode(c + 1);
        float mid = 0.5f * (lo + hi); /* exact: grid values have 2 significant bits */
        /* go up past the midpoint; on the midpoint go up only if c has an odd mantissa */
        if (u > mid || (u == mid && (c & 1)))
            mag = c + 1;
        else
            break;
    }
    return mag | (signbit(v) ? 8 : 0);
}

/* ------------------------------------------------------------- E4M3 format
 * OCP E4M3FN: sign | 4-bit exponent (bias 7) | 3-bit mantissa.  Exponent 0 is
 * subnormal: m * 2^-9.  Otherwise 2^(e-7) * (1 + m/8).  0x7F / 0xFF are NaN;
 * there is no Inf; the largest finite value is 0x7E = 448. */
float fp4q_ref_e4m3_decode(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    float mag;
    if (e == 15 && m == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

/* Round a finite t >= 0 to nearest E4M3, ties to the even mantissa, saturating
 * at 448 (never NaN).  Works in binary64, where every step below is exact. */
int fp4q_ref_e4m3_encode(float t) {
    double u = (double)t;
    if (!(u > 0.0)) return 0;
    if (u >= 448.0) return 0x7E;
    int e2;
    (void)frexp(u, &e2);      /* u = f * 2^e2 with f in [0.5, 1) */
    int E = e2 - 1;           /* u = (2f) * 2^E with 2f in [1, 2) */
    if (E < -6) {             /* below the smallest normal 2^-6: spacing 2^-9 */
        double q = nearbyint(ldexp(u, 9)); /* ties to even in the default mode */
        return (int)q;        /* q == 8 is exactly the smallest normal, code 0x08 */
    }
    double q = nearbyint(ldexp(u, 3 - E)); /* 8 <= q <= 16: 1.mmm scaled by 8 */
    int m = (int)q - 8, ex = E + 7;
    if (m == 8) { m = 0; ex += 1; }
    int code = (ex << 3) | m;
    return code > 0x7E ? 0x7E : code; /* u < 448 never rounds past 448 */
}

/* ------------------------------------------------------------------- FWHT
 * y = H x / 16 with H[i][j] = (-1)^popcount(i & j) (natural Sylvester order).
 * Reading: radix-2 butterflies on pairs (i, i+h) -> (a+b, a-b), stride h going
 * 1, 2, ..., 128, then one multiply by 1/16.  Strides 1..8 are the first level
 * (index bits 0-3), 16..128 the second (bits 4-7). */
void fp4q_ref_fwht256(float *y) {
    for (int h = 1; h < BLOCK; h <<= 1)
        for (int i = 0; i < BLOCK; ++i)
            if ((i & h) == 0) {
                float a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
    for (int i = 0; i < BLOCK; ++i) y[i] *= 0.0625f;
}

void fp4q_ref_fwht256_f64(double *y) {
    for (int h = 1; h < BLOCK; h <<= 1)
        for (int i = 0; i < BLOCK; ++i)
            if ((i & h) == 0) {
                double a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
    for (int i = 0; i < BLOCK; ++i) y[i] *= 0.0625;
}

/* ------------------------------------------------------------- compress
 * One 256-block.  Outputs: 128 code bytes, 16 micro-scale bytes, 1 fp32 block
 * scale; optionally the pre-rounding values v (256) and t (16) for the parity
 * checker.  Steps and readings:
 *   y   = FWHT(x) (or x itself when fwht == 0)
 *   A   = max |y|;  s = A / 2688            (2688 = 6 * 448: the largest group
 *                                            of a block uses the whole E4M3 range)
 *   a_g = max |y| over group g;  t_g = a_g / (6 s) with 6 s rounded first;
 *   m_g = E4M3(t_g)  (A == 0 gives s = 0 and every m_g = 0)
 *   S_g = s * E4M3value(m_g);  r_g = 1 / S_g, taken as 0 when S_g == 0 and as
 *         FLT_MAX when 1 / S_g overflows (S_g below 2^-128)
 *   v_i = y_i * r_g;  code_i = E2M1(v_i)
 *   byte k = code[2k] | code[2k+1] << 4
 * quantize_block performs every step after the transform. */
static void quantize_block(const float *y, uint8_t *codes, uint8_t *micro, float *block,
                           float *v_out, float *t_out) {
    uint8_t code[BLOCK];
    float A = 0.0f;
    for (int i = 0; i < BLOCK; ++i) A = fmaxf(A, fabsf(y[i]));
    float s = A / 2688.0f;
    *block = s;

    for (int g = 0; g < NGROUP; ++g) {
        const float *yg = y + GROUP * g;
        float a = 0.0f;
        for (int i = 0; i < GROUP; ++i) a = fmaxf(a, fabsf(yg[i]));
        float t = 0.0f;
        int m = 0;
        if (s != 0.0f) {
            float d = 6.0f * s;
            t = a / d;
            m = fp4q_ref_e4m3_encode(t);
        }
        micro[g] = (uint8_t)m;
        if (t_out) t_out[g] = t;

        float S = s * fp4q_ref_e4m3_decode(m);
        float r = (S == 0.0f) ? 0.0f : 1.0f / S;
        if (r > FLT_MAX) r = FLT_MAX;
        for (int i = 0; i < GROUP; ++i) {
            float v = yg[i] * r;
            code[GROUP * g + i] = (uint8_t)fp4q_ref_e2m1_encode(v);
            if (v_out) v_out[GROUP * g + i] = v;
        }
    }
    for (int k = 0; k < BLOCK / 2; ++k)
        codes[k] = (uint8_t)(code[2 * k] | (code[2 * k + 1] << 4));
}

static void compress_block(const uint16_t *x, int fwht, uint8_t *codes, uint8_t *micro,
                           float *block, float *v_out, float *t_out) {
    float y[BLOCK];
    for (int i = 0; i < BLOCK; ++i) y[i] = widen_bf16(x[i]);
    if (fwht) fp4q_ref_fwht256(y);
    quantize_block(y, codes, micro, block, v_out, t_out);
}

/* Flat block order: block b holds elements [256 b, 256 b + 256) of the row-major
 * tensor; payload arrays are flat in the same order. */
void fp4q_ref_compress(const uint16_t *x, int64_t nblocks, int fwht, uint8_t *codes,
                       uint8_t *micro, float *block, float *v_out, float *t_out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t b = 0; b < nblocks; ++b)
        compress_block(x + BLOCK * b, fwht, codes + (BLOCK / 2) * b, micro + NGROUP * b,
                       block + b, v_out ? v_out + BLOCK * b : NULL,
                       t_out ? t_out + NGROUP * b : NULL);
}

/* ----------------------------------------------------------- decompress
 * yhat_i = E2M1value(code_i) * S_g with S_g = s * E4M3value(m_g) computed as in
 * compress; then the same FWHT (H / 16 is its own inverse). */
static void decompress_block(const uint8_t *codes, const uint8_t *micro, float s, int fwht,
                             float *out) {
    for (int g = 0; g < NGROUP; ++g) {
        float S = s * fp4q_ref_e4m3_decode(micro[g]);
        for (int i = 0; i < GROUP; ++i) {
            int e = GROUP * g + i;
            int c = (codes[e >> 1] >> (4 * (e & 1))) & 15;
            out[e] = fp4q_ref_e2m1_decode(c) * S;
        }
    }
    if (fwht) fp4q_ref_fwht256(out);
}

void fp4q_ref_decompress(const uint8_t *codes, const uint8_t *micro, const float *block,
                         int64_t nblocks, int fwht, float *out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t b = 0; b < nblocks; ++b)
        decompress_block(codes + (BLOCK / 2) * b, micro + NGROUP * b, block[b], fwht,
                         out + BLOCK * b);
}

/* Binary64 decompress: the payload's value code * micro * block is exact in
 * binary64 (2 + 4 + 24 significant bits), and so is the transform's input. */
static void decompress_block_f64(const uint8_t *codes, const uint8_t *micro, float s, int fwht,
                                 double *out) {
    for (int g = 0; g < NGROUP; ++g) {
        double S = (double)s * (double)fp4q_ref_e4m3_decode(micro[g]);
        for (int i = 0; i < GROUP; ++i) {
            int e = GROUP * g + i;
            int c = (codes[e >> 1] >> (4 * (e & 1))) & 15;
            out[e] = (double)fp4q_ref_e2m1_decode(c) * S;
        }
    }
    if (fwht) fp4q_ref_fwht256_f64(out);
}

void fp4q_ref_decompress_f64(const uint8_t *codes, const uint8_t *micro, const float *block,
                             int64_t nblocks, int fwht, double *out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t b = 0; b < nblocks; ++b)
        decompress_block_f64(codes + (BLOCK / 2) * b, micro + NGROUP * b, block[b], fwht,
                             out + BLOCK * b);
}

/* Receiver-side reduce: out = sum over peers p = 0..k-1 of decompress(payload p),
 * every peer's decompress and the sum in binary64. */
void fp4q_ref_accumulate_f64(int k, const uint8_t *const *codes, const uint8_t *const *micro,
                             const float *const *block, int64_t nblocks, int fwht,
                             double *out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t b = 0; b < nblocks; ++b) {
        double acc[BLOCK], d[BLOCK];
        for (int i = 0; i < BLOCK; ++i) acc[i] = 0.0;
        for (int p = 0; p < k; ++p) {
            decompress_block_f64(codes[p] + (BLOCK / 2) * b, micro[p] + NGROUP * b,
                                 block[p][b], fwht, d);
            for (int i = 0; i < BLOCK; ++i) acc[i] += d[i];
        }
        memcpy(out + BLOCK * b, acc, sizeof acc);
    }
}

/* Receiver step of a compressed AllReduce split into a reduce-scatter and an
 * all-gather: the k payloads a rank receives for its slice are summed, together
 * with the rank's own uncompressed part of that slice when one is given, and
 * the sum is quantised again for the all-gather.  Reading: the sum is taken
 * where the payloads live, in the transform domain (decompressing k payloads,
 * summing and compressing again would apply H/16 twice, and H/16 is its own
 * inverse), in fp32.  The accumulator starts at the local part transformed
 * exactly as compress transforms its input (fwht = 0: the local part as is),
 * or at +0 without one; each peer's term E2M1value(code) * S_g, as in
 * decompress, is then added in peer order p = 0 .. k-1 (a rounded product and
 * a rounded sum); then the quantisation steps of compress (block maximum
 * onwards) apply to the sum.  With no peer the result is compress(local). */
void fp4q_ref_requantize_ex(int k, const uint8_t *const *codes, const uint8_t *const *micro,
                            const float *const *block, const uint16_t *local, int fwht,
                            int64_t nblocks, uint8_t *out_codes, uint8_t *out_micro,
                            float *out_block, float *v_out, float *t_out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t b = 0; b < nblocks; ++b) {
        float acc[BLOCK], d[BLOCK];
        if (local) {
            for (int i = 0; i < BLOCK; ++i) acc[i] = widen_bf16(local[BLOCK * b + i]);
            if (fwht) fp4q_ref_fwht256(acc);
        } else {
            for (int i = 0; i < BLOCK; ++i) acc[i] = 0.0f;
        }
        for (int p = 0; p < k; ++p) {
            decompress_block(codes[p] + (BLOCK / 2) * b, micro[p] + NGROUP * b, block[p][b], 0, d);
            for (int i = 0; i < BLOCK; ++i) acc[i] = acc[i] + d[i];
        }
        quantize_block(acc, out_codes + (BLOCK / 2) * b, out_micro + NGROUP * b, out_block + b,
                       v_out ? v_out + BLOCK * b : NULL, t_out ? t_out + NGROUP * b : NULL);
    }
}

void fp4q_ref_requantize(int k, const uint8_t *const *codes, const uint8_t *const *micro,
                         const float *const *block, int64_t nblocks, uint8_t *out_codes,
                         uint8_t *out_micro, float *out_block, float *v_out, float *t_out) {
    fp4q_ref_requantize_ex(k, codes, micro, block, NULL, 1, nblocks, out_codes, out_micro,
                           out_block, v_out, t_out);
}

/* ------------------------------------------------ MXFP4-style variant
 * The microscaling FP4 format named on the gist.science page ("Practical FP4
 * Training for Large-Scale MoE Models on Hopper GPUs", Problemstellung item 2:
 * blocks of 32, E2M1 elements), as an alternative to the dual scale: after the
 * same transform, every 32 consecutive values share one power-of-two scale 2^e
 * stored as an E8M0 byte (e + 127), with no coarse scale.  Following the OCP
 * microscaling rule, e = floor(log2(max |y| over the 32)) - 2 (2 = the largest
 * E2M1 exponent), clamped to [-127, 127]; a zero group takes e = -127.  Each
 * element is v = y / 2^e (exact: a power-of-two scaling of a value below 8)
 * rounded to E2M1 as in compress.  4.25 bits per element. */
#define MXGROUP 32
#define MXNGROUP (BLOCK / MXGROUP)

static int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    int e2;
    (void)frexpf(amax, &e2); /* amax = f 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
    int e = (e2 - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

static void compress_block_mx(const uint16_t *x, int fwht, uint8_t *codes, uint8_t *scales,
                              float *v_out) {
    float y[BLOCK];
    uint8_t code[BLOCK];
    for (int i = 0; i < BLOCK; ++i) y[i] = widen_bf16(x[i]);
    if (fwht) fp4q_ref_fwht256(y);
    for (int g = 0; g < MXNGROUP; ++g) {
        const float *yg = y + MXGROUP * g;
        float a = 0.0f;
        for (int i = 0; i < MXGROUP; ++i) a = fmaxf(a, fabsf(yg[i]));
        int e = mx_exponent(a);
        scales[g] = (uint8_t)(e + 127);
        for (int i = 0; i < MXGROUP; ++i) {
            float v = (float)ldexp((double)yg[i], -e); /* exact */
            code[MXGROUP * g + i] = (uint8_t)fp4q_ref_e2m1_encode(v);
            if (v_out) v_out[MXGROUP * g + i] = v;
        }
    }
    for (int k = 0; k < BLOCK / 2; ++k)
        codes[k] = (uint8_t)(code[2 * k] | (code[2 * k + 1] << 4));
}

void fp4q_ref_compress_mx(const uint16_t *x, int64_t nblocks, int fwht, uint8_t *codes,
                          uint8_t *scales, float *v_out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t b = 0; b < nblocks; ++b)
        compress_block_mx(x + BLOCK * b, fwht, codes + (BLOCK / 2) * b, scales + MXNGROUP * b,
                          v_out ? v_out + BLOCK * b : NULL);
}

/* yhat_i = E2M1value(code_i) * 2^e (exact), then the same transform. */
void fp4q_ref_decompress_mx(const uint8_t *codes, const uint8_t *scales, int64_t nblocks,
                            int fwht, float *out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t b = 0; b < nblocks; ++b) {
        float *o = out + BLOCK * b;
        for (int e = 0; e < BLOCK; ++e) {
            int c = (codes[(BLOCK / 2) * b + (e >> 1)] >> (4 * (e & 1))) & 15;
            int ex = (int)scales[MXNGROUP * b + e / MXGROUP] - 127;
            o[e] = (float)ldexp((double)fp4q_ref_e2m1_decode(c), ex);
        }
        if (fwht) fp4q_ref_fwht256(o);
    }
}

/* ------------------------------------------------ bfloat16 output option
 * The receiver may write bfloat16 instead of binary32: each binary32 result is
 * rounded to the nearer of its two neighbouring bfloat16 values (the one that
 * keeps its top 16 bits, and the next one away from zero), ties to the even
 * significand.  Past the largest finite bfloat16 the next value is taken as
 * 2^128, so that overflow rounds as IEEE rounding does.  Finite inputs. */
uint16_t fp4q_ref_bf16_round(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t lo = (uint16_t)(u >> 16), hi = (uint16_t)(lo + 1);
    if ((u & 0xFFFFu) == 0) return lo;                    /* already a bfloat16 */
    double x = fabs((double)f), a = fabs((double)widen_bf16(lo));
    double b = ((hi & 0x7F80u) == 0x7F80u) ? ldexp(1.0, 128) : fabs((double)widen_bf16(hi));
    if (x - a < b - x) return lo;
    if (x - a > b - x) return hi;
    return (lo & 1u) ? hi : lo;
}

/* ------------------------------------------------- vectorised scalar helpers */
void fp4q_ref_e2m1_encode_n(const float *v, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)fp4q_ref_e2m1_encode(v[i]);
}

void fp4q_ref_e4m3_encode_n(const float *t, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)fp4q_ref_e4m3_encode(t[i]);
}

void fp4q_ref_fwht256_n(float *y, int64_t nblocks) {
    for (int64_t b = 0; b < nblocks; ++b) fp4q_ref_fwht256(y + BLOCK * b);
}

void fp4q_ref_bf16_round_n(const float *x, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t i = 0; i < n; ++i) out[i] = fp4q_ref_bf16_round(x[i]);
}
