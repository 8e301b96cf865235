// Device pieces of the single-token router used both by the router launches
// (route.hip) and by the fused single-token layer (decode.hip), so that the
// two compute the same partial logits and the same selection bit for bit.
// The router is kept at full precision ("DwarfStar" README, section on model
// weights; deep-dive article, section 3.4.3): fp64 accumulation, ties to the
// lower expert index.
#pragma once
#include "common.h"

namespace moe {

// One wave's item of the partial logits: EW experts x TB tokens over one H
// chunk (item < (E / EW) * ceil(T / TB) * NC), written to part[c][t][e].
template <int EW, int TB, bool XBF16>
__device__ __forceinline__ void route_partial_item(const void *x, const float *wr, int T, int H, int E, int NC, int HC,
                                                   int item, int lane, double *part)
{
    (void)E;
    const int n_tg = (T + TB - 1) / TB;
    const int c = item % NC;
    const int tg = (item / NC) % n_tg;
    const int eg = item / (NC * n_tg);
    const int t0 = tg * TB, nt = min(TB, T - t0);
    const int h_begin = c * HC, h_end = min(H, h_begin + HC);
    double acc[EW][TB];
#pragma unroll
    for (int a = 0; a < EW; ++a)
#pragma unroll
        for (int b = 0; b < TB; ++b) acc[a][b] = 0.0;
    // batches of SB steps of 256 h: every load of a batch is issued before any use
    constexpr int SB = TB == 1 ? 8 : 2;
    for (int h0 = h_begin + 4 * lane; h0 < h_end; h0 += 256 * SB) {
        f32x4 w4[SB][EW];
        uint2 xb[SB][TB];
        f32x4 xf[SB][TB];
#pragma unroll
        for (int st = 0; st < SB; ++st) {
            const int h = h0 + 256 * st;
            if (h < h_end) {
#pragma unroll
                for (int a = 0; a < EW; ++a) w4[st][a] = *(const f32x4 *)&wr[(size_t)(eg * EW + a) * H + h];
#pragma unroll
                for (int b = 0; b < TB; ++b)
                    if (b < nt) {
                        if (XBF16) xb[st][b] = *(const uint2 *)&((const uint16_t *)x)[(size_t)(t0 + b) * H + h];
                        else xf[st][b] = *(const f32x4 *)&((const float *)x)[(size_t)(t0 + b) * H + h];
                    }
            }
        }
#pragma unroll
        for (int st = 0; st < SB; ++st) {
            if (h0 + 256 * st >= h_end) break;
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                if (b < nt) {
                    double xv[4];
                    if (XBF16) {
                        const uint2 u = xb[st][b];
                        xv[0] = bf16_bits_to_f32(u.x & 0xffffu); xv[1] = bf16_bits_to_f32(u.x >> 16);
                        xv[2] = bf16_bits_to_f32(u.y & 0xffffu); xv[3] = bf16_bits_to_f32(u.y >> 16);
                    } else {
                        const f32x4 f = xf[st][b];
                        xv[0] = f.x; xv[1] = f.y; xv[2] = f.z; xv[3] = f.w;
                    }
#pragma unroll
                    for (int a = 0; a < EW; ++a)
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[a][b] = fma(xv[q], (double)w4[st][a][q], acc[a][b]);
                }
            }
        }
    }
#pragma unroll
    for (int a = 0; a < EW; ++a)
#pragma unroll
        for (int b = 0; b < TB; ++b) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) acc[a][b] += __shfl_xor(acc[a][b], off, 64);
        }
#pragma unroll
    for (int a = 0; a < EW; ++a)
#pragma unroll
        for (int b = 0; b < TB; ++b)
            if (lane == a * TB + b && b < nt) part[((size_t)c * T + t0 + b) * E + eg * EW + a] = acc[a][b];
}

// A single-token item (T = 1, EW = TB = 1, bf16 x) whose H chunk fits one
// batch of eight 256-wide steps (HC <= 2048), split into two halves of four
// steps, each its router-weight loads and then its arithmetic, so that a
// caller can keep other loads in flight in between (x comes from a copy of its
// bits, e.g. in LDS).  The arithmetic is route_partial_item's for that case,
// operation for operation (the fp64 sum runs over the steps in order, across
// the halves), so both give the same bits.
struct RouteItem1 {
    f32x4 w4[4];
    double acc;
    int c, e, h0, h_end;
};

__device__ __forceinline__ void route_item1_begin(int H, int NC, int HC, int item, int lane, RouteItem1 &r)
{
    r.c = item % NC;
    r.e = item / NC;
    const int h_begin = r.c * HC;
    r.h_end = min(H, h_begin + HC);
    r.h0 = h_begin + 4 * lane;
    r.acc = 0.0;
}

// loads of half hf (steps 4 hf .. 4 hf + 3); steps past the chunk re-read its
// last step and are not used, so every load is unconditional
__device__ __forceinline__ void route_item1_load(const float *wr, int H, int hf, RouteItem1 &r)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = min(r.h0 + 256 * (4 * hf + i), r.h_end - 4);
        r.w4[i] = *(const f32x4 *)&wr[(size_t)r.e * H + h];
    }
}

__device__ __forceinline__ void route_item1_step(const uint16_t *xbits, int hf, RouteItem1 &r)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = r.h0 + 256 * (4 * hf + i);
        if (h >= r.h_end) break;
        const uint2 u = *(const uint2 *)&xbits[h];
        const double xv[4] = {bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16),
                              bf16_bits_to_f32(u.y & 0xffffu), bf16_bits_to_f32(u.y >> 16)};
#pragma unroll
        for (int q = 0; q < 4; ++q) r.acc = fma(xv[q], (double)r.w4[i][q], r.acc);
    }
}

__device__ __forceinline__ void route_item1_end(const RouteItem1 &r, int E, int lane, double *part)
{
    double acc = r.acc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) part[(size_t)r.c * E + r.e] = acc;
}

// Wave-wide reductions by DPP: four steps (swap neighbours, swap pairs,
// mirror the half-rows, mirror the rows) leave each 16-lane row's result in
// every lane of the row; the four row results are read from lanes 0, 16, 32,
// 48.  Straight-line code: no exec-mask branches between the steps.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double readlane_f64(double v, int l)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}

// largest value of the wave (no NaN among the inputs)
__device__ __forceinline__ double wave_max_f64(double v)
{
    v = fmax(v, dpp_f64<0xB1>(v));      // quad_perm [1,0,3,2]
    v = fmax(v, dpp_f64<0x4E>(v));      // quad_perm [2,3,0,1]
    v = fmax(v, dpp_f64<0x141>(v));     // row_half_mirror
    v = fmax(v, dpp_f64<0x140>(v));     // row_mirror
    return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

__device__ __forceinline__ int wave_min_i32(int v)
{
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Wave-wide arg-max over (value descending, expert ascending): the largest
// value, then the lowest expert among the lanes holding it (a ballot names the
// lane when only one does, the usual case; equal values take a min-reduction).
// Lanes without a candidate hold (-inf, INT_MAX).  Returns uniform values.
__device__ __forceinline__ void wave_argmax(double &bv, int &be)
{
    const double m = wave_max_f64(bv);
    const uint64_t tie = __ballot(bv == m);
    int e;
    if (__popcll(tie) == 1) e = __builtin_amdgcn_readlane(be, __ffsll((unsigned long long)tie) - 1);
    else e = wave_min_i32(bv == m ? be : 0x7fffffff);
    bv = m;
    be = e;
}

// Candidate logit of expert e at T == 1: its NC (<= 4) partials, all loaded
// together and added in chunk order, plus the bias; NaN ranks below every
// number.
__device__ __forceinline__ double select_logit(const double *part, const float *bias, int E, int NC, int e)
{
    double c4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) c4[c] = c < NC ? part[(size_t)c * E + e] : 0.0;
    const double bv = bias ? (double)bias[e] : 0.0;
    double s = c4[0];
#pragma unroll
    for (int c = 1; c < 4; ++c) if (c < NC) s += c4[c];
    if (bias) s += bv;
    return s != s ? -INFINITY : s;
}

// The end of a T == 1 selection, in one wave: lane j < k holds slot j's
// expert my_e and logit my_l; bit i of taken says whether expert lane + 64 i
// was selected.  Weights are the sigmoids of the selected logits over their
// sum (fp64).  The grouping of one token is the selection sorted by expert
// id: offsets come from ballots of the taken flags, and the position of slot
// j is the number of selected ids below its own.  With write false only kid /
// kw (when non-null: the selected experts and their weights in top-k order,
// e.g. in LDS) are filled.
template <int MAXPL>
__device__ __forceinline__ void select_finish(int E, int k, int lane, int my_e, double my_l, uint32_t taken,
                                              int32_t *topk_idx, float *topk_w, int32_t *offsets, int32_t *perm,
                                              int32_t *inv, bool write, int32_t *kid, float *kw)
{
    double sg = lane < k ? 1.0 / (1.0 + exp(-my_l)) : 0.0;
    double ssum = sg;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ssum += __shfl_xor(ssum, off, 64);
    uint64_t mk[MAXPL];
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) mk[i] = 64 * i < E ? __ballot((taken >> i) & 1u) : 0ull;
    const int es = my_e >> 6, el = my_e & 63;
    int below = 0;
#pragma unroll
    for (int i = 0; i < MAXPL; ++i)
        below += i < es ? __popcll(mk[i]) : i == es ? __popcll(mk[i] & ((1ull << el) - 1ull)) : 0;
    if (lane < k) {
        const float wj = (float)(sg / ssum);
        if (kid) kid[lane] = my_e;
        if (kw) kw[lane] = wj;
        if (write) {
            topk_idx[lane] = my_e;
            topk_w[lane] = wj;
            perm[below] = lane;
            inv[lane] = below;
        }
    }
    if (!write) return;
    int base = 0;
    const uint64_t lower = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) {
        if (64 * i >= E) break;
        const int e = lane + 64 * i;
        if (e < E) offsets[e] = base + __popcll(mk[i] & lower);
        base += __popcll(mk[i]);
    }
    if (lane == 0) offsets[E] = base;
}

// T == 1: one wave selects and groups.  Lane l holds experts l, l+64, ...;
// k rounds of a wave-wide arg-max over (logit descending, expert ascending)
// pick k distinct experts in top-k order.  No LDS, no barriers.
template <int MAXPL>                              // experts per lane: E <= 64 * MAXPL
__device__ __forceinline__ void select_one(const double *part, const float *bias, int E, int k, int NC, int lane,
                                           int32_t *topk_idx, float *topk_w, int32_t *offsets, int32_t *perm,
                                           int32_t *inv, bool write, int32_t *kid, float *kw)
{
    double v[MAXPL];
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = 64 * i < E && e < E ? select_logit(part, bias, E, NC, e) : -INFINITY;
    }
    uint32_t taken = 0;
    int my_e = 0;
    double my_l = 0.0;
    for (int j = 0; j < k; ++j) {
        double bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < MAXPL; ++i) {
            if (64 * i >= E) break;
            const int e = lane + 64 * i;
            // e grows with i, so a strict '>' keeps the lowest expert among equals
            if (e < E && !((taken >> i) & 1u) && (be == 0x7fffffff || v[i] > bv)) { bv = v[i]; be = e; }
        }
        wave_argmax(bv, be);
        if ((be & 63) == lane && be < E) taken |= 1u << (be >> 6);
        if (lane == j) { my_e = be; my_l = bv; }
    }
    select_finish<MAXPL>(E, k, lane, my_e, my_l, taken, topk_idx, topk_w, offsets, perm, inv, write, kid, kw);
}

}  // namespace moe
