// q2_pack: host-side quantizer for the routed-expert block formats (see
// include/moe.h for the layouts and the exact quantization rule).  The rule
// follows the formats the pages name for the routed experts (2-bit codebook
// for up/gate, Q2_K for down, Q4_K as the wider variant: "DwarfStar" README,
// section on model weights); the arithmetic is strict IEEE fp32 with
// round-half-to-even, so the bytes are reproducible and independent of the
// thread count.
#pragma STDC FP_CONTRACT OFF
#pragma clang fp contract(off)

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "moe.h"
#include "status.h"

namespace {

inline uint16_t half_bits(float f)
{
    _Float16 h = (_Float16)f;                 // IEEE conversion, round to nearest even
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

inline float half_value(uint16_t b)
{
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (float)h;
}

inline int rne_clamp(float v, int hi) { return std::min(std::max((int)std::nearbyint(v), 0), hi); }

inline void store_half(uint8_t *p, uint16_t b) { p[0] = (uint8_t)b; p[1] = (uint8_t)(b >> 8); }

// Affine "scale + min" block (Q2_K: 16 x 16, codes 0..3, scales 0..15;
// Q4_K: 8 x 32, codes 0..15, scales 0..63).
struct Affine {
    uint16_t d, dmin;
    int sc[16], m[16];
    uint8_t q[256];
};

void affine(const float *x, int nsub, int sub, int qmax, int smax, Affine &a)
{
    float scale[16], mn[16], top_scale = 0.f, top_mn = 0.f;
    for (int j = 0; j < nsub; ++j) {
        const float *v = x + j * sub;
        float lo = std::min(0.f, *std::min_element(v, v + sub));
        float hi = *std::max_element(v, v + sub);
        scale[j] = (hi - lo) / (float)qmax;
        mn[j] = -lo;
        top_scale = std::max(top_scale, scale[j]);
        top_mn = std::max(top_mn, mn[j]);
    }
    a.d = half_bits(top_scale / (float)smax);
    a.dmin = half_bits(top_mn / (float)smax);
    const float d = half_value(a.d), dmin = half_value(a.dmin);
    for (int j = 0; j < nsub; ++j) {
        a.sc[j] = d > 0.f ? rne_clamp(scale[j] / d, smax) : 0;
        a.m[j] = dmin > 0.f ? rne_clamp(mn[j] / dmin, smax) : 0;
        const float step = d * (float)a.sc[j];
        const float shift = dmin * (float)a.m[j];
        for (int i = 0; i < sub; ++i)
            a.q[j * sub + i] = step > 0.f ? (uint8_t)rne_clamp((x[j * sub + i] + shift) / step, qmax) : 0;
    }
}

void block_q2k(const float *x, uint8_t *o)
{
    Affine a;
    affine(x, 16, 16, 3, 15, a);
    std::memset(o, 0, 84);
    store_half(o, a.d);
    store_half(o + 2, a.dmin);
    for (int j = 0; j < 16; ++j) o[4 + j] = (uint8_t)(a.sc[j] | (a.m[j] << 4));
    for (int b = 0; b < 64; ++b)
        o[20 + b] = (uint8_t)(a.q[4 * b] | (a.q[4 * b + 1] << 2) | (a.q[4 * b + 2] << 4) | (a.q[4 * b + 3] << 6));
}

void block_q4k(const float *x, uint8_t *o)
{
    Affine a;
    affine(x, 8, 32, 15, 63, a);
    std::memset(o, 0, 144);
    store_half(o, a.d);
    store_half(o + 2, a.dmin);
    // 16 six-bit fields in a 96-bit little-endian stream: sc_0..7 then m_0..7
    uint64_t lo = 0, hi = 0;                       // bits 0..63 and 64..95
    for (int n = 0; n < 16; ++n) {
        const uint64_t f = (uint64_t)(n < 8 ? a.sc[n] : a.m[n - 8]);
        const int bit = 6 * n;
        if (bit + 6 <= 64) lo |= f << bit;
        else if (bit >= 64) hi |= f << (bit - 64);
        else { lo |= f << bit; hi |= f >> (64 - bit); }
    }
    for (int b = 0; b < 8; ++b) o[4 + b] = (uint8_t)(lo >> (8 * b));
    for (int b = 0; b < 4; ++b) o[12 + b] = (uint8_t)(hi >> (8 * b));
    for (int b = 0; b < 128; ++b) o[16 + b] = (uint8_t)(a.q[2 * b] | (a.q[2 * b + 1] << 4));
}

// Q5_K: the Q4_K block with 5-bit codes (8 x 32, codes 0..31, scales 0..63);
// the low nibbles as in Q4_K, bit 4 of every code in a 32-byte bit plane.
void block_q5k(const float *x, uint8_t *o)
{
    Affine a;
    affine(x, 8, 32, 31, 63, a);
    std::memset(o, 0, 176);
    store_half(o, a.d);
    store_half(o + 2, a.dmin);
    uint64_t lo = 0, hi = 0;
    for (int n = 0; n < 16; ++n) {
        const uint64_t f = (uint64_t)(n < 8 ? a.sc[n] : a.m[n - 8]);
        const int bit = 6 * n;
        if (bit + 6 <= 64) lo |= f << bit;
        else if (bit >= 64) hi |= f << (bit - 64);
        else { lo |= f << bit; hi |= f >> (64 - bit); }
    }
    for (int b = 0; b < 8; ++b) o[4 + b] = (uint8_t)(lo >> (8 * b));
    for (int b = 0; b < 4; ++b) o[12 + b] = (uint8_t)(hi >> (8 * b));
    for (int b = 0; b < 128; ++b) o[16 + b] = (uint8_t)((a.q[2 * b] & 15) | ((a.q[2 * b + 1] & 15) << 4));
    for (int b = 0; b < 32; ++b) {
        uint8_t plane = 0;
        for (int t = 0; t < 8; ++t) plane |= (uint8_t)(((a.q[8 * b + t] >> 4) & 1) << t);
        o[144 + b] = plane;
    }
}

// Q6_K: symmetric, 16 x 16, signed codes -32..31 stored as u = q + 32 (low
// nibbles, then the high two bits four to a byte), int8 sub-block scales.
void block_q6k(const float *x, uint8_t *o)
{
    float scale[16], top = 0.f;
    for (int j = 0; j < 16; ++j) {
        float amax = 0.f;
        for (int i = 0; i < 16; ++i) amax = std::max(amax, std::fabs(x[16 * j + i]));
        scale[j] = amax / 31.f;
        top = std::max(top, scale[j]);
    }
    const uint16_t db = half_bits(top / 127.f);
    const float d = half_value(db);
    std::memset(o, 0, 210);
    store_half(o, db);
    uint8_t u[256];
    for (int j = 0; j < 16; ++j) {
        const int sc = d > 0.f ? rne_clamp(scale[j] / d, 127) : 0;
        o[2 + j] = (uint8_t)sc;
        const float step = d * (float)sc;
        for (int i = 0; i < 16; ++i) {
            const int q = step > 0.f ? std::min(std::max((int)std::nearbyint(x[16 * j + i] / step), -32), 31) : 0;
            u[16 * j + i] = (uint8_t)(q + 32);
        }
    }
    for (int b = 0; b < 128; ++b) o[18 + b] = (uint8_t)((u[2 * b] & 15) | ((u[2 * b + 1] & 15) << 4));
    for (int b = 0; b < 64; ++b)
        o[146 + b] = (uint8_t)((u[4 * b] >> 4) | ((u[4 * b + 1] >> 4) << 2) | ((u[4 * b + 2] >> 4) << 4) |
                               ((u[4 * b + 3] >> 4) << 6));
}

// CB2: nearest codeword in the integer metric.  With t the fixed-point target
// and c a codeword, |t - 4096c|^2 = |t|^2 - 8192 (t.c - 2048 |c|^2), so the
// argmin over c only needs v(c) = 2048 |c|^2 - t.c.  |t_i| <= 4.5*4096 and
// |c_i| <= 3, so v fits in int32 exactly; a strict '<' over increasing c keeps
// the lowest index on ties.  The codebook is stored transposed so that the
// 256 candidate values of one group are computed as wide integer vectors.
struct Codebook {
    int32_t ct[8][256];                             // ct[i][c] = C[c][i]
    int32_t base[256];                              // 2048 |c|^2
    explicit Codebook(const int8_t *cb)
    {
        for (int e = 0; e < 256; ++e) {
            int32_t n = 0;
            for (int i = 0; i < 8; ++i) { ct[i][e] = cb[8 * e + i]; n += (int32_t)cb[8 * e + i] * cb[8 * e + i]; }
            base[e] = 2048 * n;
        }
    }
};

__attribute__((target_clones("avx2", "default")))
int nearest_codeword(const int32_t t[8], const Codebook &C)
{
    int32_t v[256];
    for (int e = 0; e < 256; ++e) v[e] = C.base[e];
    for (int i = 0; i < 8; ++i) {
        const int32_t ti = t[i];
        for (int e = 0; e < 256; ++e) v[e] -= ti * C.ct[i][e];
    }
    int best = 0;
    int32_t best_v = v[0];
    for (int e = 1; e < 256; ++e)
        if (v[e] < best_v) { best_v = v[e]; best = e; }
    return best;
}

void block_cb2(const float *x, const Codebook &C, uint8_t *o)
{
    float sigma[8], top = 0.f;
    for (int j = 0; j < 8; ++j) {
        float amax = 0.f;
        for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(x[32 * j + i]));
        sigma[j] = amax / 3.f;
        top = std::max(top, sigma[j]);
    }
    const uint16_t db = half_bits(top / 15.f);
    const float d = half_value(db);
    std::memset(o, 0, 38);
    store_half(o, db);
    for (int j = 0; j < 8; ++j) {
        const int s = d > 0.f ? rne_clamp(sigma[j] / d, 15) : 0;
        o[2 + j / 2] |= (uint8_t)(s << (4 * (j & 1)));
        const float step = d * (float)s;
        for (int g = 4 * j; g < 4 * j + 4; ++g) {
            int best = 0;
            if (step > 0.f) {
                int32_t t[8];
                for (int i = 0; i < 8; ++i) t[i] = (int32_t)std::nearbyint(x[8 * g + i] / step * 4096.f);
                best = nearest_codeword(t, C);
            }
            o[6 + g] = (uint8_t)best;
        }
    }
}

// CB2S: the same integer metric on magnitudes.  With a the fixed-point
// magnitude targets, |a - 4096G|^2 = |a|^2 - 8192 (a.G - 2048 |G|^2), and a
// sign flip at p adds 4 a_p 4096 G_p = 8192 (2 a_p G_p), so every candidate's
// cost is |a|^2 + 8192 u(c) with u(c) = 2048 |G_c|^2 - a.G_c (+ 2 min_p a_p
// G_cp when the count of negatives is odd).  a_i <= 7.5*4096 and G <= 15
// keep u in int32.  Strict '<' over increasing c (and over p) keeps the
// lowest index on ties.
struct Grid {
    int32_t gt[8][256];                             // gt[i][c] = G[c][i]
    int32_t base[256];                              // 2048 |G_c|^2
    explicit Grid(const uint8_t *g)
    {
        for (int e = 0; e < 256; ++e) {
            int32_t n = 0;
            for (int i = 0; i < 8; ++i) { gt[i][e] = g[8 * e + i]; n += (int32_t)g[8 * e + i] * g[8 * e + i]; }
            base[e] = 2048 * n;
        }
    }
};

__attribute__((target_clones("avx2", "default")))
int best_signed_entry(const int32_t a[8], bool odd, const Grid &G)
{
    int32_t u[256], m[256];
    for (int e = 0; e < 256; ++e) { u[e] = G.base[e]; m[e] = INT32_MAX; }
    for (int i = 0; i < 8; ++i) {
        const int32_t ai = a[i];
        for (int e = 0; e < 256; ++e) {
            const int32_t p = ai * G.gt[i][e];
            u[e] -= p;
            m[e] = std::min(m[e], p);
        }
    }
    if (odd)
        for (int e = 0; e < 256; ++e) u[e] += 2 * m[e];
    int best = 0;
    for (int e = 1; e < 256; ++e)
        if (u[e] < u[best]) best = e;
    return best;
}

void block_cb2s(const float *x, const Grid &G, uint8_t *o)
{
    float sigma[8], top = 0.f;
    for (int j = 0; j < 8; ++j) {
        float amax = 0.f;
        for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(x[32 * j + i]));
        sigma[j] = amax / 5.f;
        top = std::max(top, sigma[j]);
    }
    const uint16_t db = half_bits(top / 15.f);
    const float d = half_value(db);
    std::memset(o, 0, 66);
    store_half(o, db);
    for (int j = 0; j < 8; ++j) {
        const int s = d > 0.f ? rne_clamp(sigma[j] / d, 15) : 0;
        const float step = d * (float)s;
        uint8_t *rec = o + 2 + 8 * j;
        uint32_t word = (uint32_t)s << 28;
        for (int u = 0; u < 4; ++u) {
            const float *v = x + 32 * j + 8 * u;
            int idx = 0;
            uint32_t neg = 0;                                   // bit i: weight i negative
            if (step > 0.f) {
                int32_t a[8];
                for (int i = 0; i < 8; ++i) {
                    a[i] = (int32_t)std::nearbyint(std::fabs(v[i]) / step * 4096.f);
                    neg |= (uint32_t)(v[i] < 0.f) << i;
                }
                const bool odd = __builtin_popcount(neg) & 1;
                idx = best_signed_entry(a, odd, G);
                if (odd) {
                    int p = 0;
                    for (int i = 1; i < 8; ++i)
                        if (a[i] * G.gt[i][idx] < a[p] * G.gt[p][idx]) p = i;
                    neg ^= 1u << p;
                }
            }
            rec[u] = (uint8_t)idx;
            word |= (neg & 0x7fu) << (7 * u);
        }
        for (int t = 0; t < 4; ++t) rec[4 + t] = (uint8_t)(word >> (8 * t));
    }
}

}  // namespace

extern "C" int q2_pack(int fmt, const float *w_host, int64_t rows, int K, const int8_t *codebook_host, void *out_host)
{
    using moe::set_error;
    if (fmt != MOE_FMT_CB2 && fmt != MOE_FMT_Q2K && fmt != MOE_FMT_Q4K && fmt != MOE_FMT_Q5K && fmt != MOE_FMT_Q6K &&
        fmt != MOE_FMT_CB2S)
        return set_error(MOE_ERR_INVALID_ARG, "q2_pack: fmt=%d is not CB2, CB2S, Q2K, Q4K, Q5K or Q6K", fmt);
    if (rows < 0 || K < 1) return set_error(MOE_ERR_INVALID_ARG, "q2_pack: rows=%lld K=%d", (long long)rows, K);
    if (rows == 0) return MOE_OK;
    if (!w_host || !out_host) return set_error(MOE_ERR_INVALID_ARG, "q2_pack: NULL input or output");
    if ((fmt == MOE_FMT_CB2 || fmt == MOE_FMT_CB2S) && !codebook_host)
        return set_error(MOE_ERR_INVALID_ARG, "q2_pack: CB2 needs a codebook, CB2S its grid");
    const int nb = (K + 255) / 256;
    const int bb = fmt == MOE_FMT_CB2 ? 38 : fmt == MOE_FMT_Q2K ? 84 : fmt == MOE_FMT_Q4K ? 144
                 : fmt == MOE_FMT_Q5K ? 176 : fmt == MOE_FMT_CB2S ? 66 : 210;
    Codebook *cbp = fmt == MOE_FMT_CB2 ? new Codebook(codebook_host) : nullptr;
    Grid *gp = fmt == MOE_FMT_CB2S ? new Grid((const uint8_t *)codebook_host) : nullptr;
    auto work = [&](int64_t r0, int64_t r1) {
        std::vector<float> row((size_t)nb * 256);
        for (int64_t r = r0; r < r1; ++r) {
            std::fill(row.begin(), row.end(), 0.f);
            std::memcpy(row.data(), w_host + r * (int64_t)K, sizeof(float) * (size_t)K);
            uint8_t *o = (uint8_t *)out_host + r * (int64_t)nb * bb;
            for (int b = 0; b < nb; ++b) {
                const float *x = row.data() + 256 * b;
                if (fmt == MOE_FMT_CB2) block_cb2(x, *cbp, o + (int64_t)b * bb);
                else if (fmt == MOE_FMT_Q2K) block_q2k(x, o + (int64_t)b * bb);
                else if (fmt == MOE_FMT_Q4K) block_q4k(x, o + (int64_t)b * bb);
                else if (fmt == MOE_FMT_Q5K) block_q5k(x, o + (int64_t)b * bb);
                else if (fmt == MOE_FMT_CB2S) block_cb2s(x, *gp, o + (int64_t)b * bb);
                else block_q6k(x, o + (int64_t)b * bb);
            }
        }
    };
    unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    if ((int64_t)nt > rows) nt = (unsigned)rows;
    std::vector<std::thread> pool;
    const int64_t chunk = (rows + nt - 1) / nt;
    for (unsigned i = 0; i < nt; ++i) {
        const int64_t r0 = i * chunk, r1 = std::min(rows, r0 + chunk);
        if (r0 < r1) pool.emplace_back(work, r0, r1);
    }
    for (auto &th : pool) th.join();
    delete cbp;
    delete gp;
    return MOE_OK;
}
