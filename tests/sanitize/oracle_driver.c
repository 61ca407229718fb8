/* Runs every oracle routine on random and edge-case inputs of a few shapes, for
 * a build under AddressSanitizer and UndefinedBehaviorSanitizer (tests only).
 * Exit status 0 when every call returned; the sanitizers abort on a finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void fp4q_ref_set_threads(int n);
float fp4q_ref_e2m1_decode(int code);
int fp4q_ref_e2m1_encode(float v);
float fp4q_ref_e4m3_decode(int code);
int fp4q_ref_e4m3_encode(float t);
void fp4q_ref_fwht256(float *y);
void fp4q_ref_fwht256_f64(double *y);
void fp4q_ref_compress(const uint16_t *x, int64_t nblocks, int fwht, uint8_t *codes,
                       uint8_t *micro, float *block, float *v_out, float *t_out);
void fp4q_ref_decompress(const uint8_t *codes, const uint8_t *micro, const float *block,
                         int64_t nblocks, int fwht, float *out);
void fp4q_ref_decompress_f64(const uint8_t *codes, const uint8_t *micro, const float *block,
                             int64_t nblocks, int fwht, double *out);
void fp4q_ref_accumulate_f64(int k, const uint8_t *const *codes, const uint8_t *const *micro,
                             const float *const *block, int64_t nblocks, int fwht, double *out);
void fp4q_ref_requantize_ex(int k, const uint8_t *const *codes, const uint8_t *const *micro,
                            const float *const *block, const uint16_t *local, int fwht,
                            int64_t nblocks, uint8_t *out_codes, uint8_t *out_micro,
                            float *out_block, float *v_out, float *t_out);
void fp4q_ref_compress_mx(const uint16_t *x, int64_t nblocks, int fwht, uint8_t *codes,
                          uint8_t *scales, float *v_out);
void fp4q_ref_decompress_mx(const uint8_t *codes, const uint8_t *scales, int64_t nblocks,
                            int fwht, float *out);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng; }

/* bf16 bit patterns: mostly normal-range values, some zeros, tiny, huge, and
 * (with special) NaN and infinities */
static void fill(uint16_t *x, int64_t n, int special) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r = next();
        uint16_t e = (uint16_t)(100 + (r >> 8) % 60);          /* exponents 2^-27 .. 2^32 */
        uint16_t v = (uint16_t)((r & 0x8000u) | (e << 7) | ((r >> 16) & 0x7F));
        switch ((r >> 24) % 16) {
            case 0: v = 0; break;
            case 1: v = (uint16_t)(r & 0x807F); break;             /* subnormal */
            case 2: v = (uint16_t)((r & 0x8000u) | (0xF0u << 7)); break; /* 2^113 */
            default: break;
        }
        if (special && (r >> 20) % 97 == 0) v = (r & 1) ? 0x7FC0 : 0xFF80;
        x[i] = v;
    }
}

static int run(int64_t nblocks, int fwht, int special) {
    const int64_t n = 256 * nblocks;
    enum { K = 16 };
    uint16_t *x = malloc(2 * n), *loc = malloc(2 * n);
    uint8_t *codes[K], *micro[K];
    float *block[K];
    float *v = malloc(4 * n), *t = malloc(4 * (n / 16)), *out = malloc(4 * n);
    double *outd = malloc(8 * n);
    uint8_t *oc = malloc(n / 2), *om = malloc(n / 16), *mxc = malloc(n / 2), *mxs = malloc(n / 32);
    float *ob = malloc(4 * nblocks);
    fill(loc, n, special);
    for (int p = 0; p < K; ++p) {
        codes[p] = malloc(n / 2);
        micro[p] = malloc(n / 16);
        block[p] = malloc(4 * nblocks);
        fill(x, n, special);
        fp4q_ref_compress(x, nblocks, fwht, codes[p], micro[p], block[p], v, t);
    }
    fp4q_ref_decompress(codes[0], micro[0], block[0], nblocks, fwht, out);
    fp4q_ref_decompress_f64(codes[0], micro[0], block[0], nblocks, fwht, outd);
    fp4q_ref_accumulate_f64(K, (const uint8_t *const *)codes, (const uint8_t *const *)micro,
                            (const float *const *)block, nblocks, fwht, outd);
    for (int k = 0; k <= K; k += 5)
        fp4q_ref_requantize_ex(k, (const uint8_t *const *)codes, (const uint8_t *const *)micro,
                               (const float *const *)block, k % 2 ? NULL : loc, fwht, nblocks,
                               oc, om, ob, v, t);
    fp4q_ref_requantize_ex(1, (const uint8_t *const *)codes, (const uint8_t *const *)micro,
                           (const float *const *)block, NULL, fwht, nblocks, oc, om, ob, NULL, NULL);
    fp4q_ref_compress_mx(loc, nblocks, fwht, mxc, mxs, v);
    fp4q_ref_decompress_mx(mxc, mxs, nblocks, fwht, out);
    for (int p = 0; p < K; ++p) {
        free(codes[p]);
        free(micro[p]);
        free(block[p]);
    }
    free(x); free(loc); free(v); free(t); free(out); free(outd);
    free(oc); free(om); free(mxc); free(mxs); free(ob);
    return 0;
}

int main(void) {
    fp4q_ref_set_threads(1);
    for (int c = 0; c < 16; ++c) fp4q_ref_e2m1_decode(c);
    for (int c = 0; c < 256; ++c) fp4q_ref_e4m3_decode(c);
    const float probe[] = {0.0f, -0.0f, 0.25f, 5.0f, 6.5f, 1e30f, -1e-30f, 448.0f, 464.0f, 1e-10f,
                           INFINITY, -INFINITY, NAN};
    for (unsigned i = 0; i < sizeof probe / sizeof probe[0]; ++i) {
        fp4q_ref_e2m1_encode(probe[i]);
        fp4q_ref_e4m3_encode(fabsf(probe[i]));
    }
    float y[256];
    double yd[256];
    for (int i = 0; i < 256; ++i) y[i] = yd[i] = (float)(next() % 1000) - 500.0f;
    fp4q_ref_fwht256(y);
    fp4q_ref_fwht256_f64(yd);
    const int64_t shapes[] = {1, 3, 16, 43};
    for (unsigned s = 0; s < 4; ++s)
        for (int fwht = 0; fwht < 2; ++fwht)
            for (int special = 0; special < 2; ++special) run(shapes[s], fwht, special);
    printf("oracle driver ok\n");
    return 0;
}
