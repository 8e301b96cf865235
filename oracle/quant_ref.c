/*
 * Reference quantizers for the routed-expert weight formats.
 *
 * TEST INFRASTRUCTURE ONLY: this file belongs to the oracle.  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code with the HIP library.
 *
 * What is quantized and to which format follows the pages: only the routed
 * experts are quantized; their up/gate projections go to a 2-bit codebook
 * format (the pages call theirs IQ2_XXS) and down goes to Q2_K ("DwarfStar"
 * README, section on model weights; deep-dive article, section 3.4.3 on the
 * quantization strategy).  The pages give no bit layouts; the layouts below
 * are this project's own, with 256 weights per block:
 *
 *   CB2  38 B: [0:2) fp16 d | [2:6) eight 4-bit sub-block scales s_j (s_j in
 *        bits 4*(j%2).. of byte 2+j/2) | [6:38) 32 codebook indices, one per
 *        group of 8 weights.  w[8g+i] = d * s_{g/4} * C[idx_g][i].
 *   CB2S 66 B (the signed codebook format, 2.0625 bits per weight, the byte
 *        budget of the pages' IQ2_XXS): [0:2) fp16 d | eight 8-byte sub-block
 *        records at [2+8j, 10+8j): bytes 0..3 the grid indices of groups
 *        4j..4j+3, bytes 4..7 a little-endian word holding, for group 4j+u,
 *        the negative-sign flags of its weights 0..6 at bits 7u..7u+6 and
 *        s_j at bits 28..31.  Weight 7's flag is the parity of the other
 *        seven (every group has an even number of negative weights).  The
 *        grid G holds non-negative magnitudes.
 *        w[8g+i] = d * s_{g/4} * (-1)^{neg_gi} * G[idx_g][i].
 *   Q2_K 84 B: [0:2) fp16 d | [2:4) fp16 dmin | [4:20) byte j = sc_j | m_j<<4
 *        (16 sub-blocks of 16) | [20:84) 2-bit q_i in bits 2*(i%4) of byte i/4.
 *        w_i = d*sc_j*q_i - dmin*m_j, j = i/16.
 *   Q4_K 144 B: [0:2) d | [2:4) dmin | [4:16) sixteen 6-bit fields in one
 *        little-endian 96-bit stream (field n at bits 6n..6n+5; n<8: sc_n,
 *        n>=8: m_{n-8}) | [16:144) 4-bit q_i in bits 4*(i%2) of byte i/2.
 *        w_i = d*sc_j*q_i - dmin*m_j, j = i/32.
 *   Q5_K 176 B: as Q4_K with 5-bit codes: [0:16) as Q4_K | [16:144) the low
 *        4 bits of q_i in bits 4*(i%2) of byte 16+i/2 | [144:176) bit 4 of q_i
 *        in bit i%8 of byte 144+i/8.  w_i = d*sc_j*q_i - dmin*m_j, j = i/32.
 *   Q6_K 210 B: [0:2) fp16 d | [2:18) sixteen int8 sub-block scales sc_j
 *        (two's complement; 16 sub-blocks of 16) | [18:146) the low 4 bits of
 *        u_i = q_i + 32 in bits 4*(i%2) of byte 18+i/2 | [146:210) the high 2
 *        bits of u_i in bits 2*(i%4) of byte 146+i/4.  w_i = d*sc_j*q_i,
 *        q_i in -32..31, j = i/16 (symmetric: no min term).
 *
 * The pages name Q5_K and Q6_K among the routed layouts of other models'
 * files ("ds4" README mirror, section on model weights, GLM layouts: gate/up
 * Q2_K/Q4_K/Q5_K, down Q2_K/Q4_K/Q5_K/Q6_K); as with the others, the byte
 * layouts are this project's own.
 *
 * Arithmetic: IEEE fp32, round-half-to-even for every rounding (rintf in the
 * default rounding mode; fp16 conversion written out below), no contraction
 * (built with -ffp-contract=off).  A row whose length K is not a multiple of
 * 256 is padded with zeros to the next multiple.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 256

/* fp32 -> fp16 bit pattern, round to nearest, ties to even.
 * The value is rounded to the nearest multiple of the fp16 spacing of its
 * binade (2^(E-10) for normal E, 2^-24 in the subnormal range); an exact
 * double division by a power of two keeps this free of double rounding. */
uint16_t ref_f32_to_f16_bits(float f)
{
    if (isnan(f)) return 0x7e00;
    uint16_t s = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (a == 0.0) return s;
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < -14) E = -14;
    double ulp = ldexp(1.0, E - 10);
    double r = nearbyint(a / ulp);
    if (r * ulp > 65504.0) return s | 0x7c00;
    if (E == -14 && r < 1024.0) return s | (uint16_t)r;      /* subnormal */
    if (r == 2048.0) { r = 1024.0; E += 1; }
    return s | (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
}

float ref_f16_bits_to_f32(uint16_t h)
{
    int s = h >> 15, E = (h >> 10) & 31, m = h & 1023;
    double v;
    if (E == 0) v = ldexp((double)m, -24);
    else if (E == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + m, E - 25);
    return (float)(s ? -v : v);
}


static void put_f16(uint8_t *p, uint16_t h) { p[0] = (uint8_t)(h & 0xff); p[1] = (uint8_t)(h >> 8); }

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Copy one row into a zero-padded buffer of nb*256 floats. */
static void padded_row(const float *w, int K, int nb, float *buf)
{
    memset(buf, 0, sizeof(float) * (size_t)nb * QK);
    memcpy(buf, w, sizeof(float) * (size_t)K);
}

/* ---------------------------------------------------------------- Q2_K/Q4_K
 * Affine "scale + min" formats.  Per sub-block j of n weights:
 *   lo = min(0, min w), hi = max w, scale_j = (hi - lo)/L, mn_j = -lo
 * (L = largest code).  Per block: d = fp16(max_j scale_j / S),
 * dmin = fp16(max_j mn_j / S) (S = largest sub-block scale code).  Then
 *   sc_j = rint(scale_j / d), m_j = rint(mn_j / dmin)          (clamped to 0..S)
 *   q_i  = rint((w_i + dmin*m_j) / (d*sc_j))                    (clamped to 0..L)
 * with a zero divisor giving code 0. */
static void affine_block(const float *w, int nsub, int n, int L, int S,
                         uint16_t *d_bits, uint16_t *dmin_bits, int *sc, int *m, int *q)
{
    float scale[16], mn[16];
    float max_scale = 0.0f, max_mn = 0.0f;
    for (int j = 0; j < nsub; ++j) {
        float lo = 0.0f, hi = w[j * n];
        for (int i = 0; i < n; ++i) {
            float v = w[j * n + i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        scale[j] = (hi - lo) / (float)L;
        mn[j] = -lo;
        if (scale[j] > max_scale) max_scale = scale[j];
        if (mn[j] > max_mn) max_mn = mn[j];
    }
    *d_bits = ref_f32_to_f16_bits(max_scale / (float)S);
    *dmin_bits = ref_f32_to_f16_bits(max_mn / (float)S);
    float d = ref_f16_bits_to_f32(*d_bits), dmin = ref_f16_bits_to_f32(*dmin_bits);
    for (int j = 0; j < nsub; ++j) {
        sc[j] = d > 0.0f ? clampi((int)rintf(scale[j] / d), 0, S) : 0;
        m[j] = dmin > 0.0f ? clampi((int)rintf(mn[j] / dmin), 0, S) : 0;
        float step = d * (float)sc[j];
        float off = dmin * (float)m[j];
        for (int i = 0; i < n; ++i) {
            float v = w[j * n + i];
            q[j * n + i] = step > 0.0f ? clampi((int)rintf((v + off) / step), 0, L) : 0;
        }
    }
}

void ref_quant_q2k_row(const float *w, int K, uint8_t *out)
{
    int nb = (K + QK - 1) / QK;
    float *buf = (float *)malloc(sizeof(float) * (size_t)nb * QK);
    padded_row(w, K, nb, buf);
    for (int b = 0; b < nb; ++b) {
        uint16_t db, dmb;
        int sc[16], m[16], q[QK];
        affine_block(buf + (size_t)b * QK, 16, 16, 3, 15, &db, &dmb, sc, m, q);
        uint8_t *p = out + (size_t)b * 84;
        memset(p, 0, 84);
        put_f16(p, db);
        put_f16(p + 2, dmb);
        for (int j = 0; j < 16; ++j) p[4 + j] = (uint8_t)(sc[j] | (m[j] << 4));
        for (int i = 0; i < QK; ++i) p[20 + i / 4] |= (uint8_t)(q[i] << (2 * (i % 4)));
    }
    free(buf);
}

void ref_quant_q4k_row(const float *w, int K, uint8_t *out)
{
    int nb = (K + QK - 1) / QK;
    float *buf = (float *)malloc(sizeof(float) * (size_t)nb * QK);
    padded_row(w, K, nb, buf);
    for (int b = 0; b < nb; ++b) {
        uint16_t db, dmb;
        int sc[16], m[16], q[QK];
        affine_block(buf + (size_t)b * QK, 8, 32, 15, 63, &db, &dmb, sc, m, q);
        uint8_t *p = out + (size_t)b * 144;
        memset(p, 0, 144);
        put_f16(p, db);
        put_f16(p + 2, dmb);
        /* sixteen 6-bit fields, field n at stream bits 6n..6n+5 */
        for (int n = 0; n < 16; ++n) {
            int f = n < 8 ? sc[n] : m[n - 8];
            for (int t = 0; t < 6; ++t) {
                int bit = 6 * n + t;
                if ((f >> t) & 1) p[4 + bit / 8] |= (uint8_t)(1u << (bit % 8));
            }
        }
        for (int i = 0; i < QK; ++i) p[16 + i / 2] |= (uint8_t)(q[i] << (4 * (i % 2)));
    }
    free(buf);
}

void ref_quant_q5k_row(const float *w, int K, uint8_t *out)
{
    int nb = (K + QK - 1) / QK;
    float *buf = (float *)malloc(sizeof(float) * (size_t)nb * QK);
    padded_row(w, K, nb, buf);
    for (int b = 0; b < nb; ++b) {
        uint16_t db, dmb;
        int sc[16], m[16], q[QK];
        affine_block(buf + (size_t)b * QK, 8, 32, 31, 63, &db, &dmb, sc, m, q);
        uint8_t *p = out + (size_t)b * 176;
        memset(p, 0, 176);
        put_f16(p, db);
        put_f16(p + 2, dmb);
        for (int n = 0; n < 16; ++n) {
            int f = n < 8 ? sc[n] : m[n - 8];
            for (int t = 0; t < 6; ++t) {
                int bit = 6 * n + t;
                if ((f >> t) & 1) p[4 + bit / 8] |= (uint8_t)(1u << (bit % 8));
            }
        }
        for (int i = 0; i < QK; ++i) {
            p[16 + i / 2] |= (uint8_t)((q[i] & 15) << (4 * (i % 2)));
            p[144 + i / 8] |= (uint8_t)((q[i] >> 4) << (i % 8));
        }
    }
    free(buf);
}

/* Q6_K, symmetric.  Per sub-block j of 16 weights: scale_j = max|w| / 31.
 * Per block: d = fp16(max_j scale_j / 127); sc_j = rint(scale_j / d) clamped
 * to 0..127 (0 if d == 0); q_i = rint(w_i / (d*sc_j)) clamped to -32..31 (0 if
 * d*sc_j == 0).  d*sc_j needs at most 18 significant bits and its product with
 * q at most 24, so the dequantized value is exact in fp32. */
void ref_quant_q6k_row(const float *w, int K, uint8_t *out)
{
    int nb = (K + QK - 1) / QK;
    float *buf = (float *)malloc(sizeof(float) * (size_t)nb * QK);
    padded_row(w, K, nb, buf);
    for (int b = 0; b < nb; ++b) {
        const float *x = buf + (size_t)b * QK;
        float scale[16], max_scale = 0.0f;
        for (int j = 0; j < 16; ++j) {
            float amax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(x[16 * j + i]);
                if (a > amax) amax = a;
            }
            scale[j] = amax / 31.0f;
            if (scale[j] > max_scale) max_scale = scale[j];
        }
        uint16_t db = ref_f32_to_f16_bits(max_scale / 127.0f);
        float d = ref_f16_bits_to_f32(db);
        uint8_t *p = out + (size_t)b * 210;
        memset(p, 0, 210);
        put_f16(p, db);
        for (int j = 0; j < 16; ++j) {
            int sc = d > 0.0f ? clampi((int)rintf(scale[j] / d), 0, 127) : 0;
            p[2 + j] = (uint8_t)(int8_t)sc;
            float step = d * (float)sc;
            for (int i = 0; i < 16; ++i) {
                int k = 16 * j + i;
                int q = step > 0.0f ? clampi((int)rintf(x[k] / step), -32, 31) : 0;
                int u = q + 32;
                p[18 + k / 2] |= (uint8_t)((u & 15) << (4 * (k % 2)));
                p[146 + k / 4] |= (uint8_t)((u >> 4) << (2 * (k % 4)));
            }
        }
    }
    free(buf);
}

/* -------------------------------------------------------------------- CB2
 * Per sub-block j of 32 weights: sigma_j = max|w| / 3.  Per block:
 * d = fp16(max_j sigma_j / 15), s_j = rint(sigma_j / d) clamped to 0..15.
 * Per group of 8 weights with step = d*s_j > 0: the target t_i =
 * rint(w_i / step * 4096) (int32) and the chosen index minimises the integer
 * distance sum_i (t_i - 4096*C[idx][i])^2, lowest index on ties; a zero step
 * gives index 0. */
void ref_quant_cb2_row(const float *w, int K, const int8_t *cb, uint8_t *out)
{
    int nb = (K + QK - 1) / QK;
    float *buf = (float *)malloc(sizeof(float) * (size_t)nb * QK);
    padded_row(w, K, nb, buf);
    for (int b = 0; b < nb; ++b) {
        const float *x = buf + (size_t)b * QK;
        float sigma[8], max_sigma = 0.0f;
        for (int j = 0; j < 8; ++j) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(x[32 * j + i]);
                if (a > amax) amax = a;
            }
            sigma[j] = amax / 3.0f;
            if (sigma[j] > max_sigma) max_sigma = sigma[j];
        }
        uint16_t db = ref_f32_to_f16_bits(max_sigma / 15.0f);
        float d = ref_f16_bits_to_f32(db);
        uint8_t *p = out + (size_t)b * 38;
        memset(p, 0, 38);
        put_f16(p, db);
        for (int j = 0; j < 8; ++j) {
            int s = d > 0.0f ? clampi((int)rintf(sigma[j] / d), 0, 15) : 0;
            p[2 + j / 2] |= (uint8_t)(s << (4 * (j % 2)));
            float step = d * (float)s;
            for (int gg = 0; gg < 4; ++gg) {
                int g = 4 * j + gg;
                int best = 0;
                if (step > 0.0f) {
                    int32_t t[8];
                    for (int i = 0; i < 8; ++i) t[i] = (int32_t)rintf(x[8 * g + i] / step * 4096.0f);
                    int64_t best_dist = -1;
                    for (int c = 0; c < 256; ++c) {
                        int64_t dist = 0;
                        for (int i = 0; i < 8; ++i) {
                            int64_t diff = (int64_t)t[i] - 4096 * (int64_t)cb[8 * c + i];
                            dist += diff * diff;
                        }
                        if (best_dist < 0 || dist < best_dist) { best_dist = dist; best = c; }
                    }
                }
                p[6 + g] = (uint8_t)best;
            }
        }
    }
    free(buf);
}

/* ------------------------------------------------------------------- CB2S
 * Per sub-block j: sigma_j = max|w| / 5 (5 is the grid's largest magnitude);
 * d and s_j as for CB2.  Per group of 8 with step = d*s_j > 0: the magnitude
 * targets a_i = rint(|w_i| / step * 4096) (int32) and the natural signs
 * neg_i = (w_i < 0).  For grid entry c the cost is the integer distance
 * sum_i (a_i - 4096*G[c][i])^2; when the number of negative weights is odd,
 * one sign must flip, and flipping weight p adds 4 * a_p * 4096*G[c][p], so
 * the cheapest p (lowest on ties) is added to c's cost.  The chosen entry
 * has the lowest cost (lowest index on ties) and its flip, if any, is
 * applied.  A zero step gives index 0 and no negative flags. */
void ref_quant_cb2s_row(const float *w, int K, const uint8_t *grid, uint8_t *out)
{
    int nb = (K + QK - 1) / QK;
    float *buf = (float *)malloc(sizeof(float) * (size_t)nb * QK);
    padded_row(w, K, nb, buf);
    for (int b = 0; b < nb; ++b) {
        const float *x = buf + (size_t)b * QK;
        float sigma[8], max_sigma = 0.0f;
        for (int j = 0; j < 8; ++j) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(x[32 * j + i]);
                if (a > amax) amax = a;
            }
            sigma[j] = amax / 5.0f;
            if (sigma[j] > max_sigma) max_sigma = sigma[j];
        }
        uint16_t db = ref_f32_to_f16_bits(max_sigma / 15.0f);
        float d = ref_f16_bits_to_f32(db);
        uint8_t *p = out + (size_t)b * 66;
        memset(p, 0, 66);
        put_f16(p, db);
        for (int j = 0; j < 8; ++j) {
            int s = d > 0.0f ? clampi((int)rintf(sigma[j] / d), 0, 15) : 0;
            float step = d * (float)s;
            uint32_t word = (uint32_t)s << 28;
            for (int u = 0; u < 4; ++u) {
                int g = 4 * j + u;
                int best = 0, neg[8] = {0};
                if (step > 0.0f) {
                    int64_t a[8];
                    int nneg = 0;
                    for (int i = 0; i < 8; ++i) {
                        a[i] = (int64_t)rintf(fabsf(x[8 * g + i]) / step * 4096.0f);
                        neg[i] = x[8 * g + i] < 0.0f;
                        nneg += neg[i];
                    }
                    int64_t best_cost = -1;
                    int best_flip = -1;
                    for (int c = 0; c < 256; ++c) {
                        int64_t cost = 0;
                        for (int i = 0; i < 8; ++i) {
                            int64_t diff = a[i] - 4096 * (int64_t)grid[8 * c + i];
                            cost += diff * diff;
                        }
                        int flip = -1;
                        if (nneg & 1) {
                            int64_t fc = -1;
                            for (int i = 0; i < 8; ++i) {
                                int64_t f = 4 * a[i] * 4096 * (int64_t)grid[8 * c + i];
                                if (fc < 0 || f < fc) { fc = f; flip = i; }
                            }
                            cost += fc;
                        }
                        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = c; best_flip = flip; }
                    }
                    if (best_flip >= 0) neg[best_flip] ^= 1;
                }
                p[2 + 8 * j + u] = (uint8_t)best;
                for (int i = 0; i < 7; ++i) word |= (uint32_t)neg[i] << (7 * u + i);
            }
            for (int t = 0; t < 4; ++t) p[2 + 8 * j + 4 + t] = (uint8_t)(word >> (8 * t));
        }
    }
    free(buf);
}

/* Quantize rows [r0, r1) of a row-major [rows][K] matrix into the packed
 * output (row r occupies nb*block_bytes bytes at r*nb*block_bytes).
 * fmt: 1 = CB2, 2 = Q2_K, 3 = Q4_K, 5 = Q5_K, 6 = Q6_K, 7 = CB2S (cb is then
 * the uint8 magnitude grid).  Returns 0 on success, -1 on a bad fmt. */
int ref_quant_rows(int fmt, const float *w, int64_t r0, int64_t r1, int K, const int8_t *cb, uint8_t *out)
{
    int nb = (K + QK - 1) / QK;
    int bb = fmt == 1 ? 38 : fmt == 2 ? 84 : fmt == 3 ? 144 : fmt == 5 ? 176 : fmt == 6 ? 210 : fmt == 7 ? 66 : 0;
    if (!bb) return -1;
    for (int64_t r = r0; r < r1; ++r) {
        const float *row = w + r * (int64_t)K;
        uint8_t *o = out + r * (int64_t)nb * bb;
        if (fmt == 1) ref_quant_cb2_row(row, K, cb, o);
        else if (fmt == 2) ref_quant_q2k_row(row, K, o);
        else if (fmt == 3) ref_quant_q4k_row(row, K, o);
        else if (fmt == 5) ref_quant_q5k_row(row, K, o);
        else if (fmt == 7) ref_quant_cb2s_row(row, K, (const uint8_t *)cb, o);
        else ref_quant_q6k_row(row, K, o);
    }
    return 0;
}
