/*
 * qig_oracle.c -- plain, slow, CPU oracle for the k-quant prefill MMQ.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * HIP library.  Floating-point results are accumulated in fp64; the
 * quantizer is a defined fp32 procedure and is done in fp32 on purpose.
 *
 * Sources (the four "minfer CUDA optimization steps" pages):
 *   [r43]  "46 . r43 -- PC-sampling attribution + pre-expand-B parity FAIL"
 *   [r44]  "47 . r44 -- W_exp stride mismatch root cause"
 *   [r20]  "25 . r20: Split-phase A staging"
 *   [r21]  "26 . r21 -- Coalesced block-linear A staging"
 *
 * Where the pages are silent the reading taken is stated at the function.
 * Parity status: every function below is pinned by the CPU tests, except
 * the q4_K block *byte layout* (super-block with fp16 d, fp16 dmin, twelve
 * bytes of packed 6-bit scale/min pairs and 128 bytes of nibbles), which the
 * pages never print: it is the GGUF q4_K layout restated from the format's
 * public definition.  Its decoding is pinned to hand-derived fixtures, but it
 * is "parity unpinned" against any real model file.
 *
 * Build: gcc -O2 -fopenmp -std=c11 -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* IEEE binary16                                                             */
/* ------------------------------------------------------------------------ */

/* binary16 -> double, exact, subnormals kept.  The scale fields d/dmin of
 * both weight formats and d of the activation block are fp16 ([r44] s2.2
 * lists "d[2]" as the last field of block_q6_K; [r21] s2.1 gives a 2-byte d
 * in the pad40 block). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* float -> binary16, round to nearest, ties to even, subnormals kept.
 * Written on doubles so every step is exact except the one rounding. */
uint16_t oracle_float_to_half_rne(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double v = fabs((double)f);
    if (isnan(f))
        return sign | 0x7e00;
    if (v >= 65520.0)                  /* halfway to 2^16 rounds up to inf */
        return sign | 0x7c00;
    if (v < ldexp(1.0, -14)) {         /* subnormal range: units of 2^-24 */
        double n = nearbyint(ldexp(v, 24));   /* default mode: ties to even */
        return sign | (uint16_t)n;            /* n == 1024 is the smallest normal */
    }
    int e;
    frexp(v, &e);                      /* v = f * 2^e, f in [0.5, 1) */
    e -= 1;                            /* v in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(v, 10 - e));   /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* ------------------------------------------------------------------------ */
/* Activation quantization into q8 "pad40" blocks                            */
/* ------------------------------------------------------------------------ */
/*
 * One block per (token t, 32-wide chunk c) at byte offset (t*nb32 + c)*40,
 * nb32 = id/32 ([r20] s3.2 addressing of the A plane; [r21] s2.1 layout
 * diagram): bytes 0-1 fp16 d, bytes 4-35 the 32 int8 quants, bytes 36-39
 * ssum, pitch 40.
 *
 * The pages never print how the fields are filled.  Reading taken:
 *   amax = max |x_i| over the chunk, d32 = amax / 127 (fp32 division),
 *   q_i  = clamp(roundf(x_i / d32), -127, 127)   (fp32 division, ties away
 *          from zero), all q_i = 0 when d32 == 0,
 *   d    = fp16_rne(d32) stored at bytes 0-1, bytes 2-3 zero,
 *   ssum = (float)d * sum(q_i) as fp32 (exact: 11-bit times 12-bit).
 * The page code reads the +36 word as an integer sum; this oracle stores the
 * scaled fp32 form instead, which carries the same integer (ssum / d).
 */
void oracle_quantize_q8_pad40(const float *x, int64_t nt, int64_t id,
                              int64_t ldx, uint8_t *q8)
{
    const int64_t nb32 = id / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nt; ++t) {
        for (int64_t c = 0; c < nb32; ++c) {
            const float *xs = x + t * ldx + 32 * c;
            uint8_t *blk = q8 + (t * nb32 + c) * 40;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xs[i]);
                if (a > amax)
                    amax = a;
            }
            float d32 = amax / 127.0f;
            int8_t qs[32];
            int sum = 0;
            for (int i = 0; i < 32; ++i) {
                int q = 0;
                if (d32 != 0.0f) {
                    float r = roundf(xs[i] / d32);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    q = (int)r;
                }
                qs[i] = (int8_t)q;
                sum += q;
            }
            uint16_t dh = oracle_float_to_half_rne(d32);
            float ssum = (float)(oracle_half_to_double(dh) * (double)sum);
            memset(blk, 0, 40);
            blk[0] = (uint8_t)(dh & 0xff);
            blk[1] = (uint8_t)(dh >> 8);
            memcpy(blk + 4, qs, 32);
            memcpy(blk + 36, &ssum, 4);
        }
    }
}

/* Read one pad40 block back: d (fp16 decoded), the 32 quants, ssum. */
static void q8_read(const uint8_t *blk, double *d, const int8_t **qs, float *ssum)
{
    uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8));
    *d = oracle_half_to_double(h);
    *qs = (const int8_t *)(blk + 4);
    memcpy(ssum, blk + 36, 4);
}

/* ------------------------------------------------------------------------ */
/* q6_K                                                                      */
/* ------------------------------------------------------------------------ */
/*
 * block_q6_K ([r44] s2.2): 128 bytes ql, 64 bytes qh, 16 int8 sub-block
 * scales, fp16 d -- 210 content bytes at offsets 0 / 128 / 192 / 208 (ql and
 * qh offsets from the raw-W staging loads in [r44] s3.2, the scale at +192
 * from the I2F.S8 consumer in [r43] s3.1).  256 elements in 16 sub-blocks of
 * 16, each with its own signed scale ([r44] s1.1).  A row of raw W holds
 * nsb = id/256 blocks at stride bstride (224 when padded for 16-byte
 * alignment, [r44] s2.2).
 *
 * Element e of a block, in the terms of the element decoder of [r44] s3.2:
 * the block's 256 elements form two halves of 128; within a half, the
 * element's position n splits into a quarter (n / 32) and a lane (n % 32).
 * Quarters 0 and 1 take the low nibble, quarters 2 and 3 the high nibble, of
 * ql byte (64*half + 32*(quarter & 1) + lane); the two high bits come from
 * qh byte (32*half + lane), 2-bit field number `quarter`.  The stored 6-bit
 * value minus 32 is the centred weight in [-32, 31] ([r43] s3.3 shows the
 * -32..31 range; the "+-127" of [r44] s2.1 is read as garbled).
 */
static int q6k_element(const uint8_t *blk, int e)
{
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    int half = e / 128;
    int n = e % 128;
    int quarter = n / 32;
    int lane = n % 32;
    int qlbyte = ql[64 * half + 32 * (quarter & 1) + lane];
    int low4 = (quarter < 2) ? (qlbyte & 15) : (qlbyte >> 4);
    int high2 = (qh[32 * half + lane] >> (2 * quarter)) & 3;
    return low4 + 16 * high2 - 32;
}

void oracle_q6k_decode(const uint8_t *blk, int8_t c6[256], int8_t sc[16], double *d)
{
    for (int e = 0; e < 256; ++e)
        c6[e] = (int8_t)q6k_element(blk, e);
    for (int s = 0; s < 16; ++s)
        sc[s] = (int8_t)blk[192 + s];
    *d = oracle_half_to_double((uint16_t)(blk[208] | (blk[209] << 8)));
}

/*
 * expand_q6k_dense: the registration-time dense centred-int8 plane W_exp
 * ([r43] s3.2, [r44] s2.2 and s3.2): od x id bytes, row stride id,
 * super-block stride 256, out[j*id + 256*sb + e] = element e of block sb of
 * row j.  The input is the padded raw plane (row stride nsb*bstride).
 *
 * This is deliberately written the other way round from q6k_element: it walks
 * the source bytes and scatters their bits, following the byte-pair view of
 * the expander on those pages (each ql byte feeds two elements 64 apart, each
 * qh byte feeds four elements 32 apart), so that the two listings check each
 * other.
 */
void oracle_expand_q6k_dense(const uint8_t *W, int64_t bstride, int64_t od,
                             int64_t id, int8_t *out)
{
    const int64_t nsb = id / 256;
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < od; ++j) {
        for (int64_t sb = 0; sb < nsb; ++sb) {
            const uint8_t *blk = W + j * nsb * bstride + sb * bstride;
            int8_t *o = out + j * id + 256 * sb;
            int v[256];
            for (int e = 0; e < 256; ++e)
                v[e] = 0;
            /* ql byte b: half b/64, r = b%64 -> elements 128*half + r (low
             * nibble) and 128*half + r + 64 (high nibble). */
            for (int b = 0; b < 128; ++b) {
                int base = 128 * (b / 64) + (b % 64);
                v[base] |= blk[b] & 15;
                v[base + 64] |= blk[b] >> 4;
            }
            /* qh byte b: half b/32, lane b%32 -> four elements 32 apart,
             * field f at bits 2f..2f+1 is the top of element 128*half +
             * lane + 32*f. */
            for (int b = 0; b < 64; ++b) {
                int base = 128 * (b / 32) + (b % 32);
                for (int f = 0; f < 4; ++f)
                    v[base + 32 * f] |= ((blk[128 + b] >> (2 * f)) & 3) << 4;
            }
            for (int e = 0; e < 256; ++e)
                o[e] = (int8_t)(v[e] - 32);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* q4_K (layout not on the pages: GGUF block_q4_K restated)                 */
/* ------------------------------------------------------------------------ */
/*
 * 144 bytes: fp16 d at 0, fp16 dmin at 2, scale bytes S[0..11] at 4, 128
 * bytes of nibbles at 16.  Eight sub-blocks of 32; sub-block b has a 6-bit
 * scale sc_b and a 6-bit min m_b:
 *   b < 4 : sc = S[b] & 63,                      m = S[b+4] & 63
 *   b >= 4: sc = (S[b+4] & 15) | (S[b-4] >> 6) << 4,
 *           m  = (S[b+4] >> 4) | (S[b]   >> 6) << 4
 * Nibble byte 32*g + i (g = 0..3) holds element 64*g + i in its low nibble
 * and element 64*g + 32 + i in its high nibble.  Weight = d*sc*q - dmin*m.
 */
void oracle_q4k_decode(const uint8_t *blk, uint8_t q[256], uint8_t sc[8],
                       uint8_t m[8], double *d, double *dmin)
{
    const uint8_t *S = blk + 4;
    const uint8_t *qs = blk + 16;
    *d = oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    *dmin = oracle_half_to_double((uint16_t)(blk[2] | (blk[3] << 8)));
    for (int b = 0; b < 8; ++b) {
        if (b < 4) {
            sc[b] = S[b] & 63;
            m[b] = S[b + 4] & 63;
        } else {
            sc[b] = (uint8_t)((S[b + 4] & 15) | ((S[b - 4] >> 6) << 4));
            m[b] = (uint8_t)((S[b + 4] >> 4) | ((S[b] >> 6) << 4));
        }
    }
    for (int g = 0; g < 4; ++g) {
        for (int i = 0; i < 32; ++i) {
            q[64 * g + i] = qs[32 * g + i] & 15;
            q[64 * g + 32 + i] = qs[32 * g + i] >> 4;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Sub-block integer partials and the fp64 GEMM                              */
/* ------------------------------------------------------------------------ */
/*
 * Shapes: W has od rows of nsb = id/256 super-blocks; the activation plane
 * has nt tokens of nb32 = id/32 pad40 blocks; y is [nt][od].
 *
 * q6_K ([r44] s1.1, s2.1): sixteen 16-element sub-blocks, each with its own
 * d*sc; the pad40 chunk of sub-block s of super-block sb is 8*sb + s/2.
 *   P6(t,j,sb,s) = sum_{e in s} qa(t, 256 sb + e) * c6(j, sb, e)
 *   y(t,j)       = sum_sb sum_s da(t, 8 sb + s/2) * d(j,sb) * sc(j,sb,s) * P6
 * q4_K: eight 32-element sub-blocks, one per pad40 chunk:
 *   P4(t,j,sb,b) = sum_{e in b} qa(t, 256 sb + e) * q4(j, sb, e)
 *   y(t,j)       = sum_sb sum_b [ da * d * sc * P4 - dmin * m * ssum(t, 8 sb + b) ]
 * where da and ssum are the stored fp16 d and fp32 ssum of the pad40 block.
 */

typedef struct {
    int64_t nsb, nb32;
} shape_t;

/* decode the whole activation plane once: qa[t][id], da[t][nb32], ss[t][nb32] */
static void q8_plane(const uint8_t *q8, int64_t nt, int64_t id,
                     int8_t *qa, double *da, double *ss)
{
    const int64_t nb32 = id / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nt; ++t) {
        for (int64_t c = 0; c < nb32; ++c) {
            double d;
            const int8_t *qs;
            float s;
            q8_read(q8 + (t * nb32 + c) * 40, &d, &qs, &s);
            memcpy(qa + t * id + 32 * c, qs, 32);
            da[t * nb32 + c] = d;
            ss[t * nb32 + c] = (double)s;
        }
    }
}

static int64_t idot(const int8_t *a, const int8_t *b, int n)
{
    int64_t s = 0;
    for (int i = 0; i < n; ++i)
        s += (int64_t)a[i] * (int64_t)b[i];
    return s;
}

/* one decoded q6_K row: c6[id], sc[16*nsb], d[nsb] */
static void q6k_row(const uint8_t *W, int64_t bstride, int64_t id, int64_t j,
                    int8_t *c6, int8_t *sc, double *d)
{
    const int64_t nsb = id / 256;
    for (int64_t sb = 0; sb < nsb; ++sb)
        oracle_q6k_decode(W + j * nsb * bstride + sb * bstride, c6 + 256 * sb,
                          sc + 16 * sb, d + sb);
}

static void q4k_row(const uint8_t *W, int64_t id, int64_t j, int8_t *q4,
                    uint8_t *sc, uint8_t *m, double *d, double *dmin)
{
    const int64_t nsb = id / 256;
    for (int64_t sb = 0; sb < nsb; ++sb) {
        uint8_t qq[256];
        oracle_q4k_decode(W + j * nsb * 144 + sb * 144, qq, sc + 8 * sb, m + 8 * sb,
                          d + sb, dmin + sb);
        for (int e = 0; e < 256; ++e)
            q4[256 * sb + e] = (int8_t)qq[e];
    }
}

/* Returns 0, or -1 if a partial does not fit int32 (it always does for valid
 * blocks: |P| <= 32 * 127 * 32). */
int oracle_q6k_partials(const uint8_t *W, int64_t bstride, int64_t od, int64_t id,
                        const uint8_t *q8, int64_t nt, int64_t t0, int64_t t1,
                        int64_t j0, int64_t j1, int32_t *P)
{
    const int64_t nsb = id / 256, nb32 = id / 32, nw = j1 - j0;
    int8_t *qa = malloc((size_t)(t1 - t0) * id);
    double *da = malloc(sizeof(double) * (size_t)(t1 - t0) * nb32);
    double *ss = malloc(sizeof(double) * (size_t)(t1 - t0) * nb32);
    int bad = 0;
    (void)od; (void)nt;
    q8_plane(q8 + t0 * nb32 * 40, t1 - t0, id, qa, da, ss);
    #pragma omp parallel for schedule(dynamic) reduction(|:bad)
    for (int64_t j = j0; j < j1; ++j) {
        int8_t *c6 = malloc((size_t)id);
        int8_t *sc = malloc((size_t)(16 * nsb));
        double *d = malloc(sizeof(double) * (size_t)nsb);
        q6k_row(W, bstride, id, j, c6, sc, d);
        for (int64_t t = t0; t < t1; ++t)
            for (int64_t s = 0; s < 16 * nsb; ++s) {
                int64_t p = idot(qa + (t - t0) * id + 16 * s, c6 + 16 * s, 16);
                if (p > INT32_MAX || p < INT32_MIN) bad = 1;
                P[((t - t0) * nw + (j - j0)) * 16 * nsb + s] = (int32_t)p;
            }
        free(c6); free(sc); free(d);
    }
    free(qa); free(da); free(ss);
    return bad ? -1 : 0;
}

int oracle_q4k_partials(const uint8_t *W, int64_t od, int64_t id,
                        const uint8_t *q8, int64_t nt, int64_t t0, int64_t t1,
                        int64_t j0, int64_t j1, int32_t *P)
{
    const int64_t nsb = id / 256, nb32 = id / 32, nw = j1 - j0;
    int8_t *qa = malloc((size_t)(t1 - t0) * id);
    double *da = malloc(sizeof(double) * (size_t)(t1 - t0) * nb32);
    double *ss = malloc(sizeof(double) * (size_t)(t1 - t0) * nb32);
    int bad = 0;
    (void)od; (void)nt;
    q8_plane(q8 + t0 * nb32 * 40, t1 - t0, id, qa, da, ss);
    #pragma omp parallel for schedule(dynamic) reduction(|:bad)
    for (int64_t j = j0; j < j1; ++j) {
        int8_t *q4 = malloc((size_t)id);
        uint8_t *sc = malloc((size_t)(8 * nsb)), *m = malloc((size_t)(8 * nsb));
        double *d = malloc(sizeof(double) * (size_t)nsb);
        double *dmin = malloc(sizeof(double) * (size_t)nsb);
        q4k_row(W, id, j, q4, sc, m, d, dmin);
        for (int64_t t = t0; t < t1; ++t)
            for (int64_t b = 0; b < 8 * nsb; ++b) {
                int64_t p = idot(qa + (t - t0) * id + 32 * b, q4 + 32 * b, 32);
                if (p > INT32_MAX || p < INT32_MIN) bad = 1;
                P[((t - t0) * nw + (j - j0)) * 8 * nsb + b] = (int32_t)p;
            }
        free(q4); free(sc); free(m); free(d); free(dmin);
    }
    free(qa); free(da); free(ss);
    return bad ? -1 : 0;
}

/* y6 for the (t, j) pairs listed: n points, or the full [nt][od] grid when
 * tt == NULL (then out is y[nt][od]). */
static void mmq_q6k_impl(const uint8_t *W, int64_t bstride, int64_t od, int64_t id,
                         const uint8_t *q8, int64_t nt, const int64_t *tt,
                         const int64_t *jj, int64_t n, double *out)
{
    const int64_t nsb = id / 256, nb32 = id / 32;
    int8_t *qa = malloc((size_t)nt * id);
    double *da = malloc(sizeof(double) * (size_t)nt * nb32);
    double *ss = malloc(sizeof(double) * (size_t)nt * nb32);
    q8_plane(q8, nt, id, qa, da, ss);
    if (tt == NULL) {
        #pragma omp parallel for schedule(dynamic)
        for (int64_t j = 0; j < od; ++j) {
            int8_t *c6 = malloc((size_t)id);
            int8_t *sc = malloc((size_t)(16 * nsb));
            double *d = malloc(sizeof(double) * (size_t)nsb);
            q6k_row(W, bstride, id, j, c6, sc, d);
            for (int64_t t = 0; t < nt; ++t) {
                double y = 0.0;
                for (int64_t s = 0; s < 16 * nsb; ++s) {
                    int64_t p = idot(qa + t * id + 16 * s, c6 + 16 * s, 16);
                    y += da[t * nb32 + s / 2] * d[s / 16] * (double)sc[s] * (double)p;
                }
                out[t * od + j] = y;
            }
            free(c6); free(sc); free(d);
        }
    } else {
        #pragma omp parallel for schedule(dynamic)
        for (int64_t k = 0; k < n; ++k) {
            int64_t t = tt[k], j = jj[k];
            int8_t *c6 = malloc((size_t)id);
            int8_t *sc = malloc((size_t)(16 * nsb));
            double *d = malloc(sizeof(double) * (size_t)nsb);
            q6k_row(W, bstride, id, j, c6, sc, d);
            double y = 0.0;
            for (int64_t s = 0; s < 16 * nsb; ++s) {
                int64_t p = idot(qa + t * id + 16 * s, c6 + 16 * s, 16);
                y += da[t * nb32 + s / 2] * d[s / 16] * (double)sc[s] * (double)p;
            }
            out[k] = y;
            free(c6); free(sc); free(d);
        }
    }
    free(qa); free(da); free(ss);
}

static void mmq_q4k_impl(const uint8_t *W, int64_t od, int64_t id, const uint8_t *q8,
                         int64_t nt, const int64_t *tt, const int64_t *jj, int64_t n,
                         double *out)
{
    const int64_t nsb = id / 256, nb32 = id / 32;
    int8_t *qa = malloc((size_t)nt * id);
    double *da = malloc(sizeof(double) * (size_t)nt * nb32);
    double *ss = malloc(sizeof(double) * (size_t)nt * nb32);
    q8_plane(q8, nt, id, qa, da, ss);
    int64_t count = (tt == NULL) ? od : n;
    #pragma omp parallel for schedule(dynamic)
    for (int64_t k = 0; k < count; ++k) {
        int64_t j = (tt == NULL) ? k : jj[k];
        int8_t *q4 = malloc((size_t)id);
        uint8_t *sc = malloc((size_t)(8 * nsb)), *m = malloc((size_t)(8 * nsb));
        double *d = malloc(sizeof(double) * (size_t)nsb);
        double *dmin = malloc(sizeof(double) * (size_t)nsb);
        q4k_row(W, id, j, q4, sc, m, d, dmin);
        int64_t tb = (tt == NULL) ? 0 : tt[k];
        int64_t te = (tt == NULL) ? nt : tt[k] + 1;
        for (int64_t t = tb; t < te; ++t) {
            double y = 0.0;
            for (int64_t b = 0; b < 8 * nsb; ++b) {
                int64_t p = idot(qa + t * id + 32 * b, q4 + 32 * b, 32);
                y += da[t * nb32 + b] * d[b / 8] * (double)sc[b] * (double)p
                   - dmin[b / 8] * (double)m[b] * ss[t * nb32 + b];
            }
            if (tt == NULL)
                out[t * od + j] = y;
            else
                out[k] = y;
        }
        free(q4); free(sc); free(m); free(d); free(dmin);
    }
    free(qa); free(da); free(ss);
}

void oracle_mmq_q6k(const uint8_t *W, int64_t bstride, int64_t od, int64_t id,
                    const uint8_t *q8, int64_t nt, double *y)
{
    mmq_q6k_impl(W, bstride, od, id, q8, nt, NULL, NULL, 0, y);
}

void oracle_mmq_q4k(const uint8_t *W, int64_t od, int64_t id, const uint8_t *q8,
                    int64_t nt, double *y)
{
    mmq_q4k_impl(W, od, id, q8, nt, NULL, NULL, 0, y);
}

void oracle_mmq_q6k_points(const uint8_t *W, int64_t bstride, int64_t od, int64_t id,
                           const uint8_t *q8, int64_t nt, const int64_t *tt,
                           const int64_t *jj, int64_t n, double *out)
{
    mmq_q6k_impl(W, bstride, od, id, q8, nt, tt, jj, n, out);
}

void oracle_mmq_q4k_points(const uint8_t *W, int64_t od, int64_t id, const uint8_t *q8,
                           int64_t nt, const int64_t *tt, const int64_t *jj, int64_t n,
                           double *out)
{
    mmq_q4k_impl(W, od, id, q8, nt, tt, jj, n, out);
}

/*
 * q6_K GEMM whose quants are read from a dense centred plane at the given
 * strides: element e of super-block sb of row j is plane[j*row_stride +
 * sb*sb_stride + e] (reads past plane_bytes count as 0); d and the scales
 * still come from the raw blocks.  With the dense plane's own strides (id,
 * 256) this is oracle_mmq_q6k; with the padded raw-W strides (nsb*bstride,
 * bstride) it reproduces the consumer mistake analysed on the r44 page
 * ("W_exp stride mismatch root cause", s2.3), which the tests use as a
 * mutant that parity must reject.
 */
void oracle_mmq_q6k_from_plane(const int8_t *plane, int64_t plane_bytes, int64_t row_stride,
                               int64_t sb_stride, const uint8_t *W, int64_t bstride, int64_t od,
                               int64_t id, const uint8_t *q8, int64_t nt, double *y)
{
    const int64_t nsb = id / 256, nb32 = id / 32;
    int8_t *qa = malloc((size_t)nt * id);
    double *da = malloc(sizeof(double) * (size_t)nt * nb32);
    double *ss = malloc(sizeof(double) * (size_t)nt * nb32);
    q8_plane(q8, nt, id, qa, da, ss);
    #pragma omp parallel for schedule(dynamic)
    for (int64_t j = 0; j < od; ++j) {
        int8_t *c6 = malloc((size_t)id);
        int8_t *sc = malloc((size_t)(16 * nsb));
        double *d = malloc(sizeof(double) * (size_t)nsb);
        q6k_row(W, bstride, id, j, c6, sc, d);          /* scales and d from W */
        for (int64_t sb = 0; sb < nsb; ++sb)
            for (int e = 0; e < 256; ++e) {
                int64_t off = j * row_stride + sb * sb_stride + e;
                c6[256 * sb + e] = (off >= 0 && off < plane_bytes) ? plane[off] : 0;
            }
        for (int64_t t = 0; t < nt; ++t) {
            double acc = 0.0;
            for (int64_t s = 0; s < 16 * nsb; ++s) {
                int64_t p = idot(qa + t * id + 16 * s, c6 + 16 * s, 16);
                acc += da[t * nb32 + s / 2] * d[s / 16] * (double)sc[s] * (double)p;
            }
            y[t * od + j] = acc;
        }
        free(c6); free(sc); free(d);
    }
    free(qa); free(da); free(ss);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Harness control, not arithmetic: the thread count of later calls (n <= 0
 * restores the OpenMP default).  Timings of the oracle on one thread use it. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    static int dflt = 0;
    if (dflt == 0) dflt = omp_get_max_threads();
    omp_set_num_threads(n > 0 ? n : dflt);
#else
    (void)n;
#endif
}
