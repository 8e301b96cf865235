// Expert FFN on gfx950: grouped GEMMs over the routed experts (2-bit codebook
// gate/up, Q2_K down, or Q4_K) and the bf16 shared expert, SwiGLU, and the
// routing-weighted combine.
//
// Only the routed experts are quantized (gate/up 2-bit codebook, down Q2_K),
// while the shared expert stays at full precision ("DwarfStar" README, section
// on model weights; deep-dive article, section 3.4.3).  Decode reads each
// routed weight once per token step while compute idles, which is why several
// sessions' decode rows are packed into one call ("Part 5: serving layer",
// section 6 on session batching): the decode kernels here take any number of
// rows per expert in the MFMA N dimension at no extra weight traffic.
//
// Work decomposition: a tiny schedule kernel turns the device-side segment
// offsets into a list of (group, first row) tiles, shared expert first so that
// its long tiles start early; each GEMM work-group takes one tile and one
// slice of output features.  Nothing is read back to the host.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// ============================================================== schedule
int ffn_max_tiles(int T, int k, int E, int has_shared, int BM, int BMsh, int KSsh)
{
    if (BMsh <= 0) BMsh = BM;
    const int64_t tk = (int64_t)T * k;
    const int64_t routed = (tk + BM - 1) / BM + std::min<int64_t>(E, tk);
    const int64_t sh = has_shared ? (int64_t)((T + BMsh - 1) / BMsh) * std::max(KSsh, 1) : 0;
    return (int)(routed + sh);
}

__global__ __launch_bounds__(1024) void ffn_schedule(const int32_t *offsets, int T, int k, int E, int has_shared,
                                                     int BM, int BMsh, int KSsh, int max_tiles, int32_t *sched)
{
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int G = E + (has_shared ? 1 : 0);
    const int per = (G + 1023) / 1024;               // 1 or 2 (E <= 1024)
    int cnt[2] = {0, 0}, mine = 0;
    for (int i = 0; i < per; ++i) {
        const int o = tid * per + i;
        if (o < G) {
            const int g = has_shared ? (o == 0 ? E : o - 1) : o;
            // routing from moe_route is consistent; clamp anyway so that a bad
            // caller-supplied offsets array cannot push tiles out of range
            const int Tk = T * k;
            const int n = g == E ? T : min(max(offsets[g + 1], 0), Tk) - min(max(offsets[g], 0), Tk);
            const int bm = g == E ? BMsh : BM;
            cnt[i] = n > 0 ? ((n + bm - 1) / bm) * (g == E ? KSsh : 1) : 0;
            mine += cnt[i];
        }
    }
    part[tid] = mine;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int start = part[tid] - mine;
    for (int i = 0; i < per; ++i) {
        const int o = tid * per + i;
        if (o < G) {
            const int g = has_shared ? (o == 0 ? E : o - 1) : o;
            const int bm = g == E ? BMsh : BM, ks = g == E ? KSsh : 1;
            // shared K parts of one row tile are consecutive: group id E + part
            for (int c = 0; c < cnt[i] && start + c < max_tiles; ++c) {
                sched[1 + 2 * (start + c)] = g + c % ks;
                sched[2 + 2 * (start + c)] = (c / ks) * bm;
            }
            start += cnt[i];
        }
    }
    if (tid == 1023) sched[0] = min(part[1023], max_tiles);
}

void launch_ffn_schedule(const int32_t *offsets, int T, int k, int E, int has_shared, int BM, int32_t *sched,
                         hipStream_t s, int BMsh, int KSsh)
{
    if (BMsh <= 0) BMsh = BM;
    KSsh = std::max(KSsh, 1);
    ffn_schedule<<<1, 1024, 0, s>>>(offsets, T, k, E, has_shared, BM, BMsh, KSsh,
                                    ffn_max_tiles(T, k, E, has_shared, BM, BMsh, KSsh), sched);
}

// h of the shared rows (positions Tk + t) from the K-part partial sums of g
// and u, added in part order
__global__ __launch_bounds__(256) void sh_finalize_kernel(const float *part, int KS, int T, int I, int Tk,
                                                          uint16_t *h_bf16, float *h_f32, int hstride)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * I) return;
    const int t = (int)(i / I), n = (int)(i % I);
    float g = 0.f, u = 0.f;
    for (int q = 0; q < KS; ++q) {
        g += part[(((int64_t)q * 2 + 0) * T + t) * I + n];
        u += part[(((int64_t)q * 2 + 1) * T + t) * I + n];
    }
    const float h = g / (1.0f + expf(-g)) * u;
    const int64_t o = (int64_t)(Tk + t) * hstride + n;
    if (h_f32) h_f32[o] = h;
    else h_bf16[o] = (uint16_t)f32_to_bf16_rne(h);
}

void launch_sh_finalize(const float *part, int KS, int T, int I, int Tk, uint16_t *h_bf16, float *h_f32, int hstride,
                        hipStream_t s)
{
    const int64_t n = (int64_t)T * I;
    sh_finalize_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, KS, T, I, Tk, h_bf16, h_f32, hstride);
}

// ============================================================== tile helpers
struct Tile {
    int g, m0, n0, Ng, Kg, row0, nvalid;
    int w;                                         // index of the routed group's matrices in w0 / w1
    bool sh;
};

// Returns false when this work-group has no work (uniform over the group).
__device__ __forceinline__ bool tile_of(const FfnPass &p, int BM, int BN, Tile &t)
{
    const int tau = blockIdx.x;
    if (tau >= p.sched[0]) return false;
    t.g = p.sched[1 + 2 * tau];
    t.m0 = p.sched[2 + 2 * tau];
    t.sh = t.g == p.E;
    t.Ng = t.sh ? p.Nsh : p.N;
    t.n0 = blockIdx.y * BN;
    if (t.n0 >= t.Ng) return false;
    t.Kg = t.sh ? p.Ksh : p.K;
    int pb, pe;
    const int Tk = p.T * p.k;
    if (t.sh) { pb = Tk; pe = pb + p.T; }
    else { pb = min(max(p.offsets[t.g], 0), Tk); pe = min(max(p.offsets[t.g + 1], pb), Tk); }
    t.row0 = pb + t.m0;
    t.nvalid = min(BM, pe - t.row0);
    t.w = t.sh ? 0 : p.slot ? max(p.slot[t.g], 0) : t.g;
    return t.nvalid > 0;
}

// activation row of tile row i (i < nvalid)
__device__ __forceinline__ int64_t act_row(const FfnPass &p, const Tile &t, int i)
{
    const int pos = t.row0 + i;
    if (!p.act_by_token) return pos;
    if (t.sh) return pos - p.T * p.k;
    int tok = p.perm[pos] / p.k;
    return min(max(tok, 0), p.T - 1);              // in bounds even for corrupt routing
}

__device__ __forceinline__ const uint8_t *wrow(const FfnPass &p, int m, int g, int r)
{
    const uint8_t *base = m == 0 ? p.w0 : p.w1;
    return base + (int64_t)g * p.w_expert_bytes + (int64_t)r * p.w_row_bytes;
}

__device__ __forceinline__ const uint16_t *srow(const FfnPass &p, int m, int Kg, int r)
{
    return (m == 0 ? p.s0 : p.s1) + (int64_t)r * Kg;
}

// 32 bf16 activations at [k, k+32) of a bf16 row (zero beyond Kg)
__device__ __forceinline__ void load32_bf16(const uint16_t *row, int k, int Kg, uint32_t out[16])
{
    if (k + 32 <= Kg) {
        const u32x4 *src = (const u32x4 *)(row + k);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 v = src[c];
            out[4 * c] = v.x; out[4 * c + 1] = v.y; out[4 * c + 2] = v.z; out[4 * c + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t lo = k + 2 * e < Kg ? row[k + 2 * e] : 0u;
            const uint32_t hi = k + 2 * e + 1 < Kg ? row[k + 2 * e + 1] : 0u;
            out[e] = lo | (hi << 16);
        }
    }
}

__device__ __forceinline__ void store32(uint16_t *dst, const uint32_t v[16])
{
    u32x4 *d = (u32x4 *)dst;
#pragma unroll
    for (int c = 0; c < 4; ++c) d[c] = u32x4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
}

__device__ __forceinline__ void zero16(uint32_t v[16])
{
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ============================================================== decode
// Exact-weight path.  Weights enter the bf16 MFMA as integer codes with the
// sub-block scale folded in (exact), fp32 activations as two bf16 terms, and
// the per-row block scale d multiplies the fp32 partial sum of each 128-wide
// K step.  Q2_K's min term sum_j m_j * (sum of the sub-block's activations) is
// one more MFMA per K step.  A work-group owns 16 rows (positions) x 16 output
// features; its four waves split K and are summed in a fixed order at the end.
template <bool GATEUP, bool ACTF32, int FMTW>
struct DecLds {
    static constexpr int NMAT = GATEUP ? 2 : 1;
    uint16_t a_hi[16 * LROW];
    uint16_t a_lo[ACTF32 ? 16 * LROW : 2];
    uint16_t b[NMAT][16 * LROW];
    float scale[NMAT][16];
    float dmin[16];
    uint16_t xmin[FMTW == FMT_Q2K ? 16 * 32 : 2];
    uint16_t mmin[FMTW == FMT_Q2K ? 16 * 32 : 2];
};

template <int FMTW, bool GATEUP, bool ACTF32, typename L>
__device__ __forceinline__ void decode_tile(const FfnPass &p, const Tile &t, L *lds_all)
{
    constexpr int NMAT = GATEUP ? 2 : 1;
    constexpr int BB = block_bytes(FMTW);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    L &lds = lds_all[wave];
    const int nsteps = (t.Kg + KS - 1) / KS;
    f32x4 acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int sbase = 0; sbase < nsteps; sbase += 4) {
        const int s = sbase + wave;
        const bool active = s < nsteps;
        if (active) {
            // ---- activations: lane -> (row i, quarter q), 32 values at k = 128 s + 32 q
            const int i = lane >> 2, q = lane & 3;
            const int k = s * KS + 32 * q;
            uint32_t hi[16], lo[16];
            float xs0 = 0.f, xs1 = 0.f;                   // sums of the two 16-wide halves
            if (i < t.nvalid) {
                const int64_t ar = act_row(p, t, i);
                if (ACTF32) {
                    const float *row = (const float *)p.act + ar * p.act_stride;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float v0 = k + 2 * e < t.Kg ? row[k + 2 * e] : 0.f;
                        const float v1 = k + 2 * e + 1 < t.Kg ? row[k + 2 * e + 1] : 0.f;
                        const uint32_t h0 = f32_to_bf16_rne(v0), h1 = f32_to_bf16_rne(v1);
                        const uint32_t l0 = f32_to_bf16_rne(v0 - bf16_bits_to_f32(h0));
                        const uint32_t l1 = f32_to_bf16_rne(v1 - bf16_bits_to_f32(h1));
                        hi[e] = h0 | (h1 << 16);
                        lo[e] = l0 | (l1 << 16);
                        if (e < 8) xs0 += v0 + v1; else xs1 += v0 + v1;
                    }
                } else {
                    load32_bf16((const uint16_t *)p.act + ar * p.act_stride, k, t.Kg, hi);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float v = bf16_bits_to_f32(hi[e] & 0xffffu) + bf16_bits_to_f32(hi[e] >> 16);
                        if (e < 8) xs0 += v; else xs1 += v;
                    }
                    zero16(lo);
                }
            } else {
                zero16(hi);
                zero16(lo);
            }
            store32(&lds.a_hi[i * LROW + 32 * q], hi);
            if (ACTF32) store32(&lds.a_lo[i * LROW + 32 * q], lo);
            if (FMTW == FMT_Q2K) {
                // min-term operand: slots 0..7 = hi of the 8 sub-block sums, 8..15 = lo, rest 0
                uint16_t *xm = &lds.xmin[i * 32];
                const uint32_t h0 = f32_to_bf16_rne(xs0), h1 = f32_to_bf16_rne(xs1);
                xm[2 * q] = (uint16_t)h0;
                xm[2 * q + 1] = (uint16_t)h1;
                xm[8 + 2 * q] = (uint16_t)f32_to_bf16_rne(xs0 - bf16_bits_to_f32(h0));
                xm[8 + 2 * q + 1] = (uint16_t)f32_to_bf16_rne(xs1 - bf16_bits_to_f32(h1));
#pragma unroll
                for (int z = 0; z < 4; ++z) xm[16 + 4 * q + z] = 0;
            }
            // ---- weights: lane -> (feature rr, quarter q)
            const int rr = lane >> 2;
            const int r = t.n0 + rr;
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                uint32_t v[16];
                float dsc = 0.f, dmn = 0.f;
                int m2[2] = {0, 0};
                if (r < t.Ng) {
                    if (FMTW == FMT_BF16) {
                        load32_bf16(srow(p, m, t.Kg, r), s * KS + 32 * q, t.Kg, v);
                        dsc = 1.f;
                    } else {
                        const uint8_t *blk = wrow(p, m, t.w, r) + (int64_t)(s >> 1) * BB;
                        const int k0 = (s & 1) * KS + 32 * q;
                        if (FMTW == FMT_CB2) unit_cb2<true>(blk, k0, p.codebook, v, &dsc);
                        else unit_q2k<true>(blk, k0, v, &dsc, &dmn, m2);
                    }
                } else {
                    zero16(v);
                }
                store32(&lds.b[m][rr * LROW + 32 * q], v);
                if (q == 0) lds.scale[m][rr] = dsc;
                if (FMTW == FMT_Q2K && m == 0) {
                    if (q == 0) lds.dmin[rr] = dmn;
                    uint16_t *mm = &lds.mmin[rr * 32];
                    const uint16_t b0 = (uint16_t)f32_to_bf16_exact((float)m2[0]);
                    const uint16_t b1 = (uint16_t)f32_to_bf16_exact((float)m2[1]);
                    mm[2 * q] = b0; mm[2 * q + 1] = b1;
                    mm[8 + 2 * q] = b0; mm[8 + 2 * q + 1] = b1;
#pragma unroll
                    for (int z = 0; z < 4; ++z) mm[16 + 4 * q + z] = 0;
                }
            }
        }
        __syncthreads();
        if (active) {
            const int fr = lane & 15, fk = 8 * (lane >> 4);
            f32x4 P[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 a = *(const bf16x8 *)&lds.a_hi[fr * LROW + 32 * kk + fk];
                bf16x8 al;
                if (ACTF32) al = *(const bf16x8 *)&lds.a_lo[fr * LROW + 32 * kk + fk];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const bf16x8 b = *(const bf16x8 *)&lds.b[m][fr * LROW + 32 * kk + fk];
                    P[m] = mfma16x16x32(a, b, P[m]);
                    if (ACTF32) P[m] = mfma16x16x32(al, b, P[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const float sc = lds.scale[m][fr];
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[m][v] += sc * P[m][v];
            }
            if (FMTW == FMT_Q2K) {
                const bf16x8 xa = *(const bf16x8 *)&lds.xmin[fr * 32 + fk];
                const bf16x8 mb = *(const bf16x8 *)&lds.mmin[fr * 32 + fk];
                const f32x4 Mt = mfma16x16x32(xa, mb, f32x4{0.f, 0.f, 0.f, 0.f});
                const float dm = lds.dmin[fr];
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[0][v] -= dm * Mt[v];
            }
        }
        __syncthreads();
    }

    // ---- sum the four waves in a fixed order, then the epilogue on wave 0
    float *red = (float *)&lds_all[0];                 // reuse: [wave][m][lane][4]
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wave * NMAT + m) * 64 + lane) * 4 + v] = acc[m][v];
    __syncthreads();
    if (wave != 0) return;
    float tot[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sum = red[((0 * NMAT + m) * 64 + lane) * 4 + v];
#pragma unroll
            for (int w = 1; w < 4; ++w) sum += red[((w * NMAT + m) * 64 + lane) * 4 + v];
            tot[m][v] = sum;
        }
    const int n = t.n0 + (lane & 15);
    if (n >= t.Ng) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int i = 4 * (lane >> 4) + v;
        if (i >= t.nvalid) continue;
        const int64_t pos = t.row0 + i;
        float r;
        if (GATEUP) r = silu_mul(tot[0][v], tot[1][v]);
        else r = tot[0][v];
        ((float *)p.out)[pos * p.out_stride + n] = r;
    }
}

template <int FMT, bool GATEUP, bool ACTF32>
__global__ __launch_bounds__(256) void ffn_decode_kernel(FfnPass p)
{
    // one LDS layout big enough for both the routed and the shared (bf16) body
    using LR = DecLds<GATEUP, ACTF32, FMT>;
    using LS = DecLds<GATEUP, ACTF32, FMT_BF16>;
    constexpr size_t BYTES = sizeof(LR) > sizeof(LS) ? sizeof(LR) : sizeof(LS);
    static_assert(4 * sizeof(LS) >= (size_t)(GATEUP ? 2 : 1) * 4 * 64 * 4 * 4, "reduction buffer");
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * BYTES];
    Tile t;
    if (!tile_of(p, DEC_BM, DEC_BN, t)) return;
    // the bf16 (shared expert) layout is never larger, so its four per-wave
    // regions fit in the same buffer
    if (t.sh) decode_tile<FMT_BF16, GATEUP, ACTF32>(p, t, (LS *)smem);
    else decode_tile<FMT, GATEUP, ACTF32>(p, t, (LR *)smem);
}

hipError_t launch_ffn_decode(const FfnPass &p, bool gateup, hipStream_t s)
{
    const int has_sh = p.Nsh > 0;
    dim3 grid(ffn_max_tiles(p.T, p.k, p.E, has_sh, DEC_BM), (std::max(p.N, p.Nsh) + DEC_BN - 1) / DEC_BN);
    if (gateup) {
        if (p.fmt != FMT_CB2) return hipErrorInvalidValue;
        if (p.act_f32) ffn_decode_kernel<FMT_CB2, true, true><<<grid, 256, 0, s>>>(p);
        else ffn_decode_kernel<FMT_CB2, true, false><<<grid, 256, 0, s>>>(p);
    } else {
        if (p.fmt != FMT_Q2K || !p.act_f32) return hipErrorInvalidValue;
        ffn_decode_kernel<FMT_Q2K, false, true><<<grid, 256, 0, s>>>(p);
    }
    return hipGetLastError();
}

// ============================================================== prefill
// bf16 path: dequantized weights rounded to bf16 (RNE) while they are staged
// into LDS, bf16 activations, MFMA 16x16x32 with fp32 accumulation.  A
// work-group computes 64 positions x 64 features (x2 for gate and up); the
// four waves form a 2 x 2 grid of 32 x 32 sub-tiles.
template <int FMTW, bool GATEUP>
__device__ __forceinline__ void prefill_tile(const FfnPass &p, const Tile &t, uint16_t *a_s, uint16_t *b_s)
{
    constexpr int NMAT = GATEUP ? 2 : 1;
    constexpr int BB = block_bytes(FMTW);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int nsteps = (t.Kg + KS - 1) / KS;
    f32x4 acc[NMAT][2][2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[m][a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int i = tid >> 2, q = tid & 3;
    const int64_t ar = i < t.nvalid ? act_row(p, t, i) : 0;
    const int r = t.n0 + i;

    for (int s = 0; s < nsteps; ++s) {
        __syncthreads();
        {
            uint32_t v[16];
            if (i < t.nvalid) load32_bf16((const uint16_t *)p.act + ar * p.act_stride, s * KS + 32 * q, t.Kg, v);
            else zero16(v);
            store32(&a_s[i * LROW + 32 * q], v);
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            uint32_t v[16];
            if (r < t.Ng) {
                if (FMTW == FMT_BF16) {
                    load32_bf16(srow(p, m, t.Kg, r), s * KS + 32 * q, t.Kg, v);
                } else {
                    const uint8_t *blk = wrow(p, m, t.w, r) + (int64_t)(s >> 1) * BB;
                    const int k0 = (s & 1) * KS + 32 * q;
                    float dd, dm;
                    int m2[2];
                    if (FMTW == FMT_CB2) unit_cb2<false>(blk, k0, p.codebook, v, &dd);
                    else if (FMTW == FMT_Q2K) unit_q2k<false>(blk, k0, v, &dd, &dm, m2);
                    else unit_q4k_bf16(blk, k0, v);
                }
            } else {
                zero16(v);
            }
            store32(&b_s[m * 64 * LROW + i * LROW + 32 * q], v);
        }
        __syncthreads();
        const int fr = lane & 15, fk = 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 af[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) af[a] = *(const bf16x8 *)&a_s[(32 * wm + 16 * a + fr) * LROW + 32 * kk + fk];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const bf16x8 bf = *(const bf16x8 *)&b_s[m * 64 * LROW + (32 * wn + 16 * b + fr) * LROW + 32 * kk + fk];
#pragma unroll
                    for (int a = 0; a < 2; ++a) acc[m][a][b] = mfma16x16x32(af[a], bf, acc[m][a][b]);
                }
        }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int n = t.n0 + 32 * wn + 16 * b + (lane & 15);
            if (n >= t.Ng) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ii = 32 * wm + 16 * a + 4 * (lane >> 4) + v;
                if (ii >= t.nvalid) continue;
                const int64_t pos = t.row0 + ii;
                if (GATEUP) {
                    const float h = silu_mul(acc[0][a][b][v], acc[1][a][b][v]);
                    ((uint16_t *)p.out)[pos * p.out_stride + n] = (uint16_t)f32_to_bf16_rne(h);
                } else {
                    ((float *)p.out)[pos * p.out_stride + n] = acc[0][a][b][v];
                }
            }
        }
}

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void ffn_prefill_kernel(FfnPass p)
{
    __shared__ __attribute__((aligned(16))) uint16_t a_s[PRE_BM * LROW];
    __shared__ __attribute__((aligned(16))) uint16_t b_s[(GATEUP ? 2 : 1) * PRE_BN * LROW];
    Tile t;
    if (!tile_of(p, PRE_BM, PRE_BN, t)) return;
    if (t.sh) prefill_tile<FMT_BF16, GATEUP>(p, t, a_s, b_s);
    else prefill_tile<FMT, GATEUP>(p, t, a_s, b_s);
}

hipError_t launch_ffn_prefill(const FfnPass &p, bool gateup, hipStream_t s)
{
    const int has_sh = p.Nsh > 0;
    dim3 grid(ffn_max_tiles(p.T, p.k, p.E, has_sh, PRE_BM), (std::max(p.N, p.Nsh) + PRE_BN - 1) / PRE_BN);
    if (p.act_f32 || p.out_f32 == gateup) return hipErrorInvalidValue;
    if (gateup) {
        if (p.fmt == FMT_CB2) ffn_prefill_kernel<FMT_CB2, true><<<grid, 256, 0, s>>>(p);
        else if (p.fmt == FMT_Q4K) ffn_prefill_kernel<FMT_Q4K, true><<<grid, 256, 0, s>>>(p);
        else return hipErrorInvalidValue;
    } else {
        if (p.fmt == FMT_Q2K) ffn_prefill_kernel<FMT_Q2K, false><<<grid, 256, 0, s>>>(p);
        else if (p.fmt == FMT_Q4K) ffn_prefill_kernel<FMT_Q4K, false><<<grid, 256, 0, s>>>(p);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ============================================================== combine
// y[t] = shared(t) + sum_{j<k} w[t,j] * O[inv[t*k+j]], j in top-k order, with
// shared(t) = sum_q sh[q][t] over the shared expert's K parts in order (one
// part: its O rows); fp32, four features per thread.  Atomic-free: each
// output element is written by exactly one thread.
__global__ __launch_bounds__(256) void combine_kernel(const float *O, const int32_t *inv, const float *topk_w,
                                                      int T, int k, int H, int sh_parts, const float *sh, float *y)
{
    const int t = blockIdx.x, n = 1024 * blockIdx.y + 4 * threadIdx.x;
    const int Tk = T * k;
    if (n >= H) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < sh_parts; ++q) acc += *(const f32x4 *)&sh[((int64_t)q * T + t) * H + n];
    // eight slots' rows requested together (each read once: non-temporal),
    // then added in slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
        f32x4 o[8];
        float w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = min(j0 + i, k - 1);
            const int pos = min(max(inv[t * k + j], 0), Tk - 1);
            o[i] = __builtin_nontemporal_load((const f32x4 *)&O[(int64_t)pos * H + n]);
            w[i] = topk_w[t * k + j];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (j0 + i < k) acc += w[i] * o[i];
    }
    *(f32x4 *)&y[(int64_t)t * H + n] = acc;
}

void launch_combine(const float *O, const int32_t *inv, const float *topk_w, int T, int k, int H, int sh_parts,
                    const float *sh, float *y, hipStream_t s)
{
    combine_kernel<<<dim3(T, (H + 1023) / 1024), 256, 0, s>>>(O, inv, topk_w, T, k, H, sh_parts, sh, y);
}

// ============================================================== unpack
// One thread per 32-weight unit; exact fp32 values (see moe.h).
__global__ __launch_bounds__(256) void unpack_kernel(int fmt, const uint8_t *packed, int64_t rows, int K, int nb,
                                                     const int8_t *cb, float *out)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t units_per_row = (int64_t)nb * 8;
    if (u >= rows * units_per_row) return;
    const int64_t r = u / units_per_row;
    const int ur = (int)(u % units_per_row);
    const int b = ur >> 3, k0 = (ur & 7) * 32;
    const int kbase = b * QK + k0;
    if (kbase >= K) return;
    const int BB = block_bytes(fmt);
    const uint8_t *blk = packed + (r * nb + b) * BB;
    float v[32];
    const float d = f16_bits_to_f32(ld_u16(blk));
    if (fmt == FMT_CB2) {
        const int j = k0 >> 5;
        const int s = (blk[2 + (j >> 1)] >> (4 * (j & 1))) & 15;
        const float step = d * (float)s;
        for (int g = 0; g < 4; ++g) {
            const int8_t *c = cb + 8 * blk[6 + 4 * j + g];
            for (int i = 0; i < 8; ++i) v[8 * g + i] = step * (float)c[i];
        }
    } else if (fmt == FMT_CB2S) {
        // sub-block record: 4 grid indices, then signs (7 per group) and s_j
        const int j = k0 >> 5;
        const uint8_t *rec = blk + 2 + 8 * j;
        const uint32_t word = (uint32_t)rec[4] | ((uint32_t)rec[5] << 8) | ((uint32_t)rec[6] << 16) |
                              ((uint32_t)rec[7] << 24);
        const float step = d * (float)(word >> 28);
        const uint8_t *grid = (const uint8_t *)cb;
        for (int g = 0; g < 4; ++g) {
            uint32_t neg = (word >> (7 * g)) & 0x7fu;
            neg |= (uint32_t)(__builtin_popcount(neg) & 1) << 7;
            const uint8_t *c = grid + 8 * rec[g];
            for (int i = 0; i < 8; ++i) v[8 * g + i] = step * ((neg >> i) & 1 ? -(float)c[i] : (float)c[i]);
        }
    } else if (fmt == FMT_Q2K) {
        const float dmin = f16_bits_to_f32(ld_u16(blk + 2));
        for (int e = 0; e < 32; ++e) {
            const int i = k0 + e, j = i >> 4;
            const int sm = blk[4 + j];
            const int q = (blk[20 + (i >> 2)] >> (2 * (i & 3))) & 3;
            v[e] = (d * (float)(sm & 15)) * (float)q - dmin * (float)(sm >> 4);
        }
    } else if (fmt == FMT_Q6K) {
        for (int e = 0; e < 32; ++e) {
            const int i = k0 + e;
            const float mul = d * (float)(int8_t)blk[2 + (i >> 4)];
            const int u = ((blk[18 + (i >> 1)] >> (4 * (i & 1))) & 15) | (((blk[146 + (i >> 2)] >> (2 * (i & 3))) & 3) << 4);
            v[e] = mul * (float)(u - 32);
        }
    } else {
        const float dmin = f16_bits_to_f32(ld_u16(blk + 2));
        const int j = k0 >> 5;
        const float mul = d * (float)q4k_field(blk, j), off = dmin * (float)q4k_field(blk, 8 + j);
        for (int e = 0; e < 32; ++e) {
            const int i = k0 + e;
            int q = (blk[16 + (i >> 1)] >> (4 * (i & 1))) & 15;
            if (fmt == FMT_Q5K) q |= ((blk[144 + (i >> 3)] >> (i & 7)) & 1) << 4;
            v[e] = mul * (float)q - off;
        }
    }
    float *o = out + r * K + kbase;
    for (int e = 0; e < 32; ++e)
        if (kbase + e < K) o[e] = v[e];
}

hipError_t launch_unpack(int fmt, const uint8_t *packed, int64_t rows, int K, const int8_t *codebook, float *out,
                         hipStream_t s)
{
    const int nb = (K + QK - 1) / QK;
    const int64_t units = rows * nb * 8;
    const int64_t blocks = (units + 255) / 256;
    unpack_kernel<<<(unsigned)blocks, 256, 0, s>>>(fmt, packed, rows, K, nb, codebook, out);
    return hipGetLastError();
}

}  // namespace moe
