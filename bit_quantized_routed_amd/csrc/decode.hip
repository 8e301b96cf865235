// Single-token decode (T = 1): the memory-bound case the pages describe for
// decode, where every routed weight is read once per token step while compute
// idles ("Part 5: 服务层", section 6).  Two launches after the router:
//
//   dec_gateup: each routed 16-row tile of one expert is one contiguous byte
//     range (gate and up, 2 x 16 x 1064 B at H = 7168); a work-group loads it
//     whole with 16-byte loads, all in flight, then eight waves split K.
//     Codebook entries are exact bf16 MFMA operands; the fp32 sub-block
//     scale d*s_j multiplies each 32-wide partial sum.  The epilogue writes
//     h = silu(g)*u as two bf16 terms (hi + lo, relative error below 2^-17)
//     and, per 16-row sub-block, the sums of h that Q2_K's min term needs.
//     The bf16 shared expert runs as four K quarters that write partial sums.
//   dec_down: 64 output rows per work-group and group; Q2_K codes become
//     exact bf16 values sc*q through a 32 KB LDS table indexed by (sc, code
//     byte); the block scale d and the min term dmin * sum_j m_j X_j apply to
//     the fp32 sums of each 256-wide block.  The shared expert's work-groups
//     first add the four gate/up quarters (in order) and form their slice of h.
//   dec_combine: y = sum of the shared expert's K parts + the routed outputs
//     weighted in top-k order.
//
// Work-groups of one launch never wait for each other: on this chip a
// device-scope release/acquire writes back and invalidates the L2 of an XCD,
// so results pass between work-groups only across launches.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int DD_ROWS = 64;        // output rows per down work-group
constexpr int DD_KPART = 512;      // shared-expert K part of the down pass

// ---------------------------------------------------------------- helpers
// With one token, the k selected experts sit at positions sorted by expert
// id: slot s is the expert of stable rank s among topk_idx[0..k) (rank = number
// of smaller ids plus equal ids earlier in the list, a permutation of 0..k-1
// even if a corrupt routing repeated an expert).  All threads call it.
__device__ __forceinline__ int rank_expert(const int32_t *topk_idx, int k, int slot, int *lds)
{
    if ((int)threadIdx.x < k) lds[threadIdx.x] = topk_idx[threadIdx.x];
    __syncthreads();
    int g = -1;
    for (int j = 0; j < k; ++j) {
        const int ej = lds[j];
        int rank = 0;
        for (int i = 0; i < k; ++i) rank += (lds[i] < ej) || (i < j && lds[i] == ej);
        if (rank == slot) g = ej;
    }
    __syncthreads();
    return g;
}

__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo)
{
    hi = f32_to_bf16_rne(v);
    lo = f32_to_bf16_rne(v - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ u32x4 pack8(const uint32_t h[8])
{
    return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// h for 16 feature rows r0.. of one position, from the fp32 gate/up sums
// g[16], u[16]; with `routed`, also the sub-block sum for Q2_K's min term.
// Threads 0..15 (one wave) do the work.
__device__ __forceinline__ void finalize_h(const DecPass &p, int64_t pos, int r0, int ncols, bool routed,
                                           const float *g, const float *u)
{
    const int tid = threadIdx.x;
    if (tid < 16) {
        const int n = r0 + tid;
        const float gv = g[tid], uv = u[tid];
        const float h = n < ncols ? gv / (1.0f + expf(-gv)) * uv : 0.f;
        uint32_t hi, lo;
        split_bf16(h, hi, lo);
        if (n < ncols) {
            p.h_hi[pos * p.hstride + n] = (uint16_t)hi;
            p.h_lo[pos * p.hstride + n] = (uint16_t)lo;
        }
        if (routed) {
            float s = h;                            // rows r0..r0+15 = one 16-wide sub-block of down's K
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 16);
            if (tid == 0) {
                uint32_t shi, slo;
                split_bf16(s, shi, slo);
                uint16_t *xr = p.X + (pos * p.nbI + (r0 >> 8)) * 32;
                xr[(r0 & 255) >> 4] = (uint16_t)shi;
                xr[16 + ((r0 & 255) >> 4)] = (uint16_t)slo;
            }
        }
    }
}

// ============================================================== gate / up
constexpr int DG_KQ = 4;           // shared-expert K quarters

template <bool XF32>
__global__ __launch_bounds__(512) void dec_gateup_kernel(DecPass p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ float gsum[16], usum[16];
    __shared__ int kidx[64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4;
    const int n_sh_items = p.Ish > 0 ? (p.Ish / 16) * DG_KQ : 0;
    int item = blockIdx.x;

    if (item < n_sh_items) {
        // ---------------------------------------------- shared expert, one K quarter
        const int rt = item / DG_KQ, q = item % DG_KQ;
        const int r0 = rt * 16;
        const int KQ = p.H / DG_KQ, k0 = q * KQ;
        const int nsteps = KQ / 32;
        uint16_t *xh = (uint16_t *)dsm;             // [KQ] hi
        uint16_t *xl = xh + KQ;                     // [KQ] lo (fp32 x only)
        float *red = (float *)(dsm + 4 * KQ);       // [8 waves][2][64*4]
        // B fragments straight from HBM: wave w takes K steps w, w+8, ...
        constexpr int MAXS = 9;
        u32x4 bg[MAXS], bu[MAXS];
        const uint16_t *rg = p.sg + (int64_t)(r0 + fr) * p.H + k0 + 8 * fc;
        const uint16_t *ru = p.su + (int64_t)(r0 + fr) * p.H + k0 + 8 * fc;
#pragma unroll
        for (int j = 0; j < MAXS; ++j) {
            const int st = wave + 8 * j;
            if (st < nsteps) {
                bg[j] = *(const u32x4 *)(rg + 32 * st);
                bu[j] = *(const u32x4 *)(ru + 32 * st);
            }
        }
        for (int i = tid; i < KQ / 8; i += 512) {
            if (XF32) {
                const float *src = (const float *)p.x + k0 + 8 * i;
                uint32_t h[8], l[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) split_bf16(src[e], h[e], l[e]);
                *(u32x4 *)&xh[8 * i] = pack8(h);
                *(u32x4 *)&xl[8 * i] = pack8(l);
            } else {
                *(u32x4 *)&xh[8 * i] = *(const u32x4 *)((const uint16_t *)p.x + k0 + 8 * i);
            }
        }
        __syncthreads();
        f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < MAXS; ++j) {
            const int st = wave + 8 * j;
            if (st >= nsteps) break;
            const int k = 32 * st + 8 * fc;
            bf16x8 a = {};
            if (fr == 0) a = *(const bf16x8 *)&xh[k];          // A row 0 = the token
            const bf16x8 Bg = __builtin_bit_cast(bf16x8, bg[j]), Bu = __builtin_bit_cast(bf16x8, bu[j]);
            ag = mfma16x16x32(a, Bg, ag);
            au = mfma16x16x32(a, Bu, au);
            if (XF32) {
                bf16x8 al = {};
                if (fr == 0) al = *(const bf16x8 *)&xl[k];
                ag = mfma16x16x32(al, Bg, ag);
                au = mfma16x16x32(al, Bu, au);
            }
        }
        // D element (slot 0, feature fr) sits in lane fr (fc = 0), element 0
        if (fc == 0) { red[(wave * 2 + 0) * 16 + fr] = ag[0]; red[(wave * 2 + 1) * 16 + fr] = au[0]; }
        __syncthreads();
        if (tid < 16) {
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) { g += red[(w * 2 + 0) * 16 + tid]; u += red[(w * 2 + 1) * 16 + tid]; }
            p.part_sh[(int64_t)(q * 2 + 0) * p.Ish + r0 + tid] = g;
            p.part_sh[(int64_t)(q * 2 + 1) * p.Ish + r0 + tid] = u;
        }
        return;
    }

    // -------------------------------------------------- routed expert tile
    item -= n_sh_items;
    const int n_rt = p.I / 16;
    const int slot = item / n_rt, rt = item % n_rt;
    const int g = rank_expert(p.topk_idx, p.k, slot, kidx);
    if (g < 0 || g >= p.E) return;
    const int64_t pos = min(max(p.offsets[g], 0), p.k - 1);
    const int r0 = rt * 16;
    const int rb = p.gu_row_bytes;
    uint8_t *wt = dsm;                                   // [2][16][rb]
    uint16_t *xh = (uint16_t *)(dsm + 32 * rb);          // [H] hi
    uint16_t *cbt = xh + p.H;                            // [256][8] bf16 codewords
    {
        const int n16 = rb;                              // 16 rows * rb bytes / 16
        const u32x4 *sg4 = (const u32x4 *)(p.wg + (int64_t)g * p.gu_expert_bytes + (int64_t)r0 * rb);
        const u32x4 *su4 = (const u32x4 *)(p.wu + (int64_t)g * p.gu_expert_bytes + (int64_t)r0 * rb);
        constexpr int MAXL = 5;                          // 2 * n16 <= 2560
        u32x4 buf[MAXL];
#pragma unroll
        for (int j = 0; j < MAXL; ++j) {
            const int i = tid + 512 * j;
            if (i < n16) buf[j] = sg4[i];
            else if (i < 2 * n16) buf[j] = su4[i - n16];
        }
        for (int i = tid; i < p.H / 8; i += 512) {
            u32x4 v;
            if (XF32) {
                const float *src = (const float *)p.x + 8 * i;
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = f32_to_bf16_rne(src[e]);
                v = pack8(h);
            } else {
                v = *(const u32x4 *)((const uint16_t *)p.x + 8 * i);
            }
            *(u32x4 *)&xh[8 * i] = v;
        }
        for (int i = tid; i < 256 * 8; i += 512) cbt[i] = (uint16_t)f32_to_bf16_exact((float)p.codebook[i]);
#pragma unroll
        for (int j = 0; j < MAXL; ++j) {
            const int i = tid + 512 * j;
            if (i < 2 * n16) *(u32x4 *)(wt + 16 * i) = buf[j];
        }
    }
    __syncthreads();
    const int nbH = rb / 38;
    const int b0 = (nbH * wave) / 8, b1 = (nbH * (wave + 1)) / 8;
    f32x4 acc_g = {0.f, 0.f, 0.f, 0.f}, acc_u = {0.f, 0.f, 0.f, 0.f};
    const uint8_t *rowg = wt + fr * rb, *rowu = wt + 16 * rb + fr * rb;
    for (int b = b0; b < b1; ++b) {
        const uint8_t *bkg = rowg + 38 * b, *bku = rowu + 38 * b;
        const float dg = f16_bits_to_f32(bkg[0] | (bkg[1] << 8));
        const float du = f16_bits_to_f32(bku[0] | (bku[1] << 8));
#pragma unroll
        for (int sb = 0; sb < 8; ++sb) {
            const int sgv = (bkg[2 + (sb >> 1)] >> (4 * (sb & 1))) & 15;
            const int suv = (bku[2 + (sb >> 1)] >> (4 * (sb & 1))) & 15;
            const bf16x8 Bg = *(const bf16x8 *)&cbt[8 * bkg[6 + 4 * sb + fc]];
            const bf16x8 Bu = *(const bf16x8 *)&cbt[8 * bku[6 + 4 * sb + fc]];
            const int k = 256 * b + 32 * sb + 8 * fc;
            bf16x8 a = {};
            if (fr == 0) a = *(const bf16x8 *)&xh[k];
            f32x4 Pg = mfma16x16x32(a, Bg, f32x4{0.f, 0.f, 0.f, 0.f});
            f32x4 Pu = mfma16x16x32(a, Bu, f32x4{0.f, 0.f, 0.f, 0.f});
            if (XF32) {
                uint32_t lo[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (fr == 0) {
                    const float *src = (const float *)p.x + k;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        uint32_t hi;
                        split_bf16(src[e], hi, lo[e]);
                    }
                }
                const bf16x8 al = __builtin_bit_cast(bf16x8, pack8(lo));
                Pg = mfma16x16x32(al, Bg, Pg);
                Pu = mfma16x16x32(al, Bu, Pu);
            }
            // D columns are features: this lane's column is feature fr, whose
            // block and sub-block scale this lane read itself
            acc_g += (dg * (float)sgv) * Pg;
            acc_u += (du * (float)suv) * Pu;
        }
    }
    __syncthreads();                                     // wt is reused for the reduction
    float *red = (float *)wt;                            // [8 waves][2][16]
    if (fc == 0) { red[(wave * 2 + 0) * 16 + fr] = acc_g[0]; red[(wave * 2 + 1) * 16 + fr] = acc_u[0]; }
    __syncthreads();
    if (tid < 16) {
        float gg = 0.f, uu = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) { gg += red[(w * 2 + 0) * 16 + tid]; uu += red[(w * 2 + 1) * 16 + tid]; }
        gsum[tid] = gg;
        usum[tid] = uu;
    }
    __syncthreads();
    finalize_h(p, pos, r0, p.I, true, gsum, usum);
}

// ============================================================== down + combine
// 512 threads: wave w owns output rows 16*(w&3).. of the tile and the K half
// w>>2; the two halves are added in a fixed order before the write.
__global__ __launch_bounds__(512) void dec_down_kernel(DecPass p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ float red[4][16];
    __shared__ int kidx[64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4;
    const int rg = wave & 3, kh = wave >> 2;
    const int n_ot = (p.H + DD_ROWS - 1) / DD_ROWS;
    const int KPD = p.Ish > 0 ? p.Ish / DD_KPART : 0;
    const int n_sh_items = n_ot * KPD;
    int item = blockIdx.x;
    const bool sh = item < n_sh_items;
    int ot, part = 0, g = -1;
    if (sh) {
        ot = item / KPD;
        part = item % KPD;
    } else {
        item -= n_sh_items;
        const int slot = item / n_ot;
        ot = item % n_ot;
        g = rank_expert(p.topk_idx, p.k, slot, kidx);
        if (g < 0 || g >= p.E) return;
    }
    const int row = ot * DD_ROWS + 16 * rg + fr;       // this lane's output feature
    const bool row_ok = row < p.H;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int64_t pos = 0;

    if (sh) {
        // ---------------------------------------------- shared expert K part
        const int k0 = part * DD_KPART;
        uint16_t *hh = (uint16_t *)dsm, *hl = hh + DD_KPART;
        u32x4 bw[8];                                    // K steps 8*kh .. 8*kh+7 of 32
        const uint16_t *rw = p.sd + (int64_t)(row_ok ? row : 0) * p.Ish + k0 + 8 * fc;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            bw[s] = row_ok ? *(const u32x4 *)(rw + 32 * (8 * kh + s)) : u32x4{0, 0, 0, 0};
        // this part's slice of the shared expert's h: add the gate/up quarters
        // in order, then silu(g) * u, split into two bf16 terms
        for (int i = tid; i < DD_KPART; i += 512) {
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int q = 0; q < DG_KQ; ++q) {
                g += p.part_sh[(int64_t)(q * 2 + 0) * p.Ish + k0 + i];
                u += p.part_sh[(int64_t)(q * 2 + 1) * p.Ish + k0 + i];
            }
            const float h = g / (1.0f + expf(-g)) * u;
            uint32_t hi, lo;
            split_bf16(h, hi, lo);
            hh[i] = (uint16_t)hi;
            hl[i] = (uint16_t)lo;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int k = 32 * (8 * kh + s) + 8 * fc;
            bf16x8 ah = {}, al = {};
            if (fr == 0) {
                ah = *(const bf16x8 *)&hh[k];
                al = *(const bf16x8 *)&hl[k];
            }
            const bf16x8 B = __builtin_bit_cast(bf16x8, bw[s]);
            acc = mfma16x16x32(ah, B, acc);
            acc = mfma16x16x32(al, B, acc);
        }
    } else {
        // ---------------------------------------------- routed Q2_K rows
        pos = min(max(p.offsets[g], 0), p.k - 1);
        const int nb = p.nbI;
        const int nbh = (nb + 1) / 2;
        const int bb0 = kh * nbh, bb1 = min(nb, bb0 + nbh);
        uint16_t *tab = (uint16_t *)dsm;                  // [16 sc][256 bytes][4]
        uint16_t *hh = tab + 16 * 256 * 4;                // [nb*256] hi
        uint16_t *hl = hh + nb * 256;                     // [nb*256] lo
        uint16_t *xm = hl + nb * 256;                     // [nb][32]
        const uint8_t *wrow = p.wd + (int64_t)g * p.d_expert_bytes + (int64_t)(row_ok ? row : 0) * p.d_row_bytes;
        constexpr int MAXB = 4;
        u32x4 codes[MAXB], scl[MAXB];
        uint32_t dd[MAXB];
#pragma unroll
        for (int j = 0; j < MAXB; ++j) {
            const int b = bb0 + j;
            if (b < bb1 && row_ok) {
                const uint8_t *blk = wrow + 84 * b;
                codes[j] = *(const u32x4 *)(blk + 20 + 16 * fc);
                scl[j] = *(const u32x4 *)(blk + 4);
                dd[j] = *(const uint32_t *)blk;
            } else {
                codes[j] = u32x4{0, 0, 0, 0};
                scl[j] = u32x4{0, 0, 0, 0};
                dd[j] = 0;
            }
        }
        for (int i = tid; i < 16 * 256; i += 512) {
            const int sc = i >> 8, byte = i & 255;
            uint32_t v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = f32_to_bf16_exact((float)(sc * ((byte >> (2 * t)) & 3)));
            *(uint2 *)&tab[4 * i] = uint2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
        }
        for (int i = tid; i < nb * 32; i += 512) {
            *(u32x4 *)&hh[8 * i] = *(const u32x4 *)(p.h_hi + pos * p.hstride + 8 * i);
            *(u32x4 *)&hl[8 * i] = *(const u32x4 *)(p.h_lo + pos * p.hstride + 8 * i);
            xm[i] = p.X[pos * nb * 32 + i];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < MAXB; ++j) {
            const int b = bb0 + j;
            if (b >= bb1) break;
            // lane (fr, fc) owns K positions [64 fc, 64 fc + 64) of block b, i.e.
            // sub-blocks 4fc..4fc+3 and code bytes 16fc..16fc+15
            const uint32_t cw[4] = {codes[j].x, codes[j].y, codes[j].z, codes[j].w};
            const uint32_t sw[4] = {scl[j].x, scl[j].y, scl[j].z, scl[j].w};
            const uint32_t scw = sw[fc];
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int sc = (scw >> (8 * (m >> 1))) & 15;
                const uint32_t word = cw[m >> 1];
                const int by0 = (word >> (16 * (m & 1))) & 255, by1 = (word >> (16 * (m & 1) + 8)) & 255;
                const uint2 t0 = *(const uint2 *)&tab[4 * (sc * 256 + by0)];
                const uint2 t1 = *(const uint2 *)&tab[4 * (sc * 256 + by1)];
                const bf16x8 B = __builtin_bit_cast(bf16x8, u32x4{t0.x, t0.y, t1.x, t1.y});
                const int k = 256 * b + 64 * fc + 8 * m;
                bf16x8 ah = {}, al = {};
                if (fr == 0) {
                    ah = *(const bf16x8 *)&hh[k];
                    al = *(const bf16x8 *)&hl[k];
                }
                P = mfma16x16x32(ah, B, P);
                P = mfma16x16x32(al, B, P);
            }
            // min term over the block's 16 sub-blocks: k-slots 0..15 carry X_hi
            // with m_0..15, slots 16..31 carry X_lo with the same m
            uint32_t mv[4];
            {
                const uint32_t w0 = sw[2 * (fc & 1)], w1 = sw[2 * (fc & 1) + 1];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t w = q ? w1 : w0;
                    mv[2 * q] = f32_to_bf16_exact((float)((w >> 4) & 15)) |
                                (f32_to_bf16_exact((float)((w >> 12) & 15)) << 16);
                    mv[2 * q + 1] = f32_to_bf16_exact((float)((w >> 20) & 15)) |
                                    (f32_to_bf16_exact((float)((w >> 28) & 15)) << 16);
                }
            }
            bf16x8 xa = {};
            if (fr == 0) xa = *(const bf16x8 *)&xm[b * 32 + 8 * fc];
            const f32x4 Mt = mfma16x16x32(xa, __builtin_bit_cast(bf16x8, u32x4{mv[0], mv[1], mv[2], mv[3]}),
                                          f32x4{0.f, 0.f, 0.f, 0.f});
            // this lane's D column is its own feature `row`, whose d and dmin it read
            const float d = f16_bits_to_f32(dd[j] & 0xffffu), dmin = f16_bits_to_f32(dd[j] >> 16);
            acc += d * P - dmin * Mt;
        }
    }
    // add the two K halves in a fixed order: slot 0 of feature fr is lane fr, v = 0
    if (kh == 1 && fc == 0) red[rg][fr] = acc[0];
    __syncthreads();
    if (kh == 0 && fc == 0 && row_ok) {
        const float v = acc[0] + red[rg][fr];
        if (sh) p.O_sh[(int64_t)part * p.H + row] = v;
        else p.O[pos * p.H + row] = v;
    }

}

// y = the shared expert's K parts in order, then the routed outputs in top-k order
__global__ __launch_bounds__(256) void dec_combine_kernel(DecPass p)
{
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= p.H) return;
    const int KPD = p.Ish > 0 ? p.Ish / DD_KPART : 0;
    float y = 0.f;
    for (int q = 0; q < KPD; ++q) y += p.O_sh[(int64_t)q * p.H + n];
    for (int j = 0; j < p.k; ++j) {
        const int ps = min(max(p.inv[j], 0), p.k - 1);
        y += p.topk_w[j] * p.O[(int64_t)ps * p.H + n];
    }
    p.y[n] = y;
}

// ============================================================== launchers
size_t dec_single_lds_gateup(int H, int gu_row_bytes) { return 32 * (size_t)gu_row_bytes + 2 * (size_t)H + 4096; }

bool dec_single_ok(int T, int H, int I, int Ish, int k, int gu_row_bytes)
{
    return T == 1 && k <= 64 && H % 512 == 0 && (Ish == 0 || Ish % DD_KPART == 0) && I % 256 == 0 &&
           I / 256 <= 8 && gu_row_bytes * 2 <= 2560 && H / DG_KQ / 32 <= 8 * 9 &&
           dec_single_lds_gateup(H, gu_row_bytes) <= 64 * 1024;
}

hipError_t launch_dec_gateup(const DecPass &p, hipStream_t s)
{
    const int grid = (p.Ish > 0 ? (p.Ish / 16) * DG_KQ : 0) + p.k * (p.I / 16);
    const size_t lds = dec_single_lds_gateup(p.H, p.gu_row_bytes);
    if (p.x_f32) dec_gateup_kernel<true><<<grid, 512, lds, s>>>(p);
    else dec_gateup_kernel<false><<<grid, 512, lds, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_dec_down(const DecPass &p, hipStream_t s)
{
    const int n_ot = (p.H + DD_ROWS - 1) / DD_ROWS;
    const int KPD = p.Ish > 0 ? p.Ish / DD_KPART : 0;
    const int grid = n_ot * KPD + p.k * n_ot;
    const size_t lds = 16 * 256 * 4 * 2 + 2 * (size_t)p.nbI * 256 * 2 + (size_t)p.nbI * 32 * 2;
    dec_down_kernel<<<grid, 512, lds, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_dec_combine(const DecPass &p, hipStream_t s)
{
    dec_combine_kernel<<<(p.H + 255) / 256, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
