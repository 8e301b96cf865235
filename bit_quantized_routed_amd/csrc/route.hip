// Router on gfx950: fp64 logits, per-token top-k with normalised sigmoid
// weights, and a stable counting sort of the assignments by expert.
//
// The pages keep the router unquantized so that routing decisions stay
// reliable (deep-dive article on DwarfStar, section 3.4.3) and need "special
// dispatch logic" for the expert activation pattern (same article, section
// 3.2.1).  Selection here is exact: logits accumulate in fp64 in one fixed
// order for every expert, ties go to the lower expert index, and the grouping
// is a counting sort whose ranks come from per-expert token bitmasks, so the
// result does not depend on thread timing.
#include "common.h"
#include "route.h"
#include "route_dev.h"

#include <algorithm>

namespace moe {

// ---------------------------------------------------------------- logits
// Small T: one wave per (expert, chunk of 8 tokens).  Each lane strides over
// h, then a fixed butterfly reduces the 64 partial sums.
template <bool XBF16>
__global__ __launch_bounds__(64) void route_logits_small(const void *x, const float *wr,
                                                          const float *bias, int T, int H, int E,
                                                          double *logits)
{
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * 8;
    const int lane = threadIdx.x;
    const int nt = min(8, T - t0);
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    const float *w = wr + (size_t)e * H;
    for (int h = lane; h < H; h += 64) {
        const double wv = (double)w[h];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < nt) {
                double xv;
                if (XBF16) xv = (double)bf16_bits_to_f32(((const uint16_t *)x)[(size_t)(t0 + i) * H + h]);
                else xv = (double)((const float *)x)[(size_t)(t0 + i) * H + h];
                acc[i] = fma(xv, wv, acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc[i] += __shfl_xor(acc[i], off, 64);
    }
    if (lane < nt) {
        double v = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) if (i == lane) v = acc[i];
        if (bias) v += (double)bias[e];
        logits[(size_t)(t0 + lane) * E + e] = v;
    }
}

// Large T: a 64-token x 64-expert tile per work-group, H staged through LDS in
// chunks of 32; each thread owns 4 tokens x 4 experts and accumulates them in
// h order (the same order for every expert).
template <bool XBF16>
__global__ __launch_bounds__(256) void route_logits_tiled(const void *x, const float *wr,
                                                           const float *bias, int T, int H, int E,
                                                           double *logits)
{
    constexpr int TT = 64, TE = 64, HC = 32;
    __shared__ double xs[HC][TT + 1];
    __shared__ double ws[HC][TE + 1];
    const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
    const int tid = threadIdx.x;
    const int tt = (tid & 15) * 4, te = (tid >> 4) * 4;
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
    for (int h0 = 0; h0 < H; h0 += HC) {
        __syncthreads();
        for (int i = tid; i < TT * HC; i += 256) {
            const int r = i / HC, c = i % HC;
            const int t = t0 + r, h = h0 + c;
            double v = 0.0;
            if (t < T && h < H) {
                if (XBF16) v = (double)bf16_bits_to_f32(((const uint16_t *)x)[(size_t)t * H + h]);
                else v = (double)((const float *)x)[(size_t)t * H + h];
            }
            xs[c][r] = v;
            const int e = e0 + r;
            ws[c][r] = (e < E && h < H) ? (double)wr[(size_t)e * H + h] : 0.0;
        }
        __syncthreads();
#pragma unroll 4
        for (int c = 0; c < HC; ++c) {
            double xv[4], wv[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) xv[a] = xs[c][tt + a];
#pragma unroll
            for (int b = 0; b < 4; ++b) wv[b] = ws[c][te + b];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = fma(xv[a], wv[b], acc[a][b]);
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int t = t0 + tt + a, e = e0 + te + b;
            if (t < T && e < E) logits[(size_t)t * E + e] = acc[a][b] + (bias ? (double)bias[e] : 0.0);
        }
}

// Large T on the fp64 matrix cores: a 64-token x 64-expert tile and one of
// ROUTE_KPARTS parts of H per work-group, written as partial logits
// [part][T][E] that the top-k kernel adds in part order.  Bigger token tiles
// read W_r fewer times (T/64 instead of T/32 passes over its 7.34 MB); the K
// split keeps the work-group count up (512 at T = 2048, E = 256).  H is staged through LDS in chunks of 32
// as fp64 (x and W_r widened exactly); each wave owns 16 experts and the
// four 16-token quarters (four independent v_mfma_f64_16x16x4f64 chains),
// and the raw values of chunk c + 1 are loaded into registers while chunk c
// is computed.  Rows of the LDS tiles are padded to 33 doubles so the 16
// lanes of one read hit 16 different bank pairs.  Needs H % (32 * ROUTE_KPARTS) == 0.
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <bool XBF16>
__global__ __launch_bounds__(256) void route_logits_mfma(const void *x, const float *wr, int T, int H, int E,
                                                          double *part)
{
    constexpr int TT = 64, TE = 64, HC = 32, LD = HC + 1;
    __shared__ double xs[TT][LD];
    __shared__ double ws[TE][LD];
    const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE, kp = blockIdx.z;
    const int HP = H / ROUTE_KPARTS, hb = kp * HP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fk = lane >> 4;
    f64x4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f64x4{0.0, 0.0, 0.0, 0.0};
    // staging maps: 8 x values and 8 W_r values per thread (64 rows x 32 each)
    const int sr = tid >> 2, sk = (tid & 3) * 8;
    const bool xok = t0 + sr < T, wok = e0 + sr < E;
    // rows past T or E load row 0 (in bounds) and stage zeros
    const size_t xoff = (size_t)(xok ? t0 + sr : 0) * H + hb + sk, woff = (size_t)(wok ? e0 + sr : 0) * H + hb + sk;
    u32x4 xraw[XBF16 ? 1 : 2];
    f32x4 wraw[2];
    auto gload = [&](int h0) {
        if (XBF16) xraw[0] = *(const u32x4 *)((const uint16_t *)x + xoff + h0);
        else {
#pragma unroll
            for (int i = 0; i < 2; ++i) xraw[i] = *(const u32x4 *)((const float *)x + xoff + h0 + 4 * i);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) wraw[i] = *(const f32x4 *)&wr[woff + h0 + 4 * i];
    };
    gload(0);
    for (int h0 = 0; h0 < HP; h0 += HC) {
        __syncthreads();                                   // previous chunk consumed
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            double v;
            if (XBF16) v = (double)bf16_bits_to_f32((xraw[0][i >> 1] >> (16 * (i & 1))) & 0xffffu);
            else v = (double)__uint_as_float(xraw[i >> 2][i & 3]);
            xs[sr][sk + i] = xok ? v : 0.0;
            ws[sr][sk + i] = wok ? (double)wraw[i >> 2][i & 3] : 0.0;
        }
        __syncthreads();
        gload(min(h0 + HC, HP - HC));                      // next chunk in flight (the last re-reads its own)
#pragma unroll
        for (int kk = 0; kk < HC / 4; ++kk) {
            // A: lane (fr, fk) holds x[token fr][h 4kk + fk]; B: W_r[expert fr][h 4kk + fk]
            const double b = ws[wave * 16 + fr][4 * kk + fk];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f64_16x16x4f64(xs[mt * 16 + fr][4 * kk + fk], b, acc[mt], 0, 0, 0);
        }
    }
    // D: lane (fr, fk) holds rows fk + 4i (tokens) of column fr (expert); the
    // fp64 16x16x4 result interleaves rows across lane groups, unlike the
    // fp32-output shapes
    const int e = e0 + wave * 16 + fr;
    if (e < E) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + mt * 16 + fk + 4 * i;
                if (t < T) part[((size_t)kp * T + t) * E + e] = acc[mt][i];
            }
    }
}

// ---------------------------------------------------------------- top-k
// One wave selects the k best experts of one token: k rounds of a wave-wide
// arg-max over (logit desc, expert asc).  Each lane holds experts lane+64*i.
// l: the token's logits, or its first partial-logit row when nparts > 1 (the
// parts, pstride apart, are added in part order, then the bias)
template <int MAXPL = 16>                        // experts per lane: E <= 64 * MAXPL
__device__ __forceinline__ void wave_topk(const double *l, int E, int k, int lane, int32_t *idx_out,
                                          float *w_out, int32_t *idx_lds, int nparts = 1, size_t pstride = 0,
                                          const float *bias = nullptr)
{
    // the same sum wherever a logit is needed (selection and normalisation)
    auto logit = [&](int e) {
        double s = l[e];
        for (int c = 1; c < nparts; ++c) s += l[c * pstride + e];
        if (bias) s += (double)bias[e];
        return s;
    };
    double v[MAXPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) {
        const int e = lane + 64 * i;
        const double s = e < E ? logit(e) : -INFINITY;
        v[i] = s != s ? -INFINITY : s;            // NaN ranks below every number, so every lane agrees
    }
    double ssum = 0.0;
    for (int j = 0; j < k; ++j) {
        double bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < MAXPL; ++i) {
            const int e = lane + 64 * i;
            // e grows with i, so a strict '>' keeps the lowest expert among equals
            if (e < E && !((taken >> i) & 1u) && (be == 0x7fffffff || v[i] > bv)) { bv = v[i]; be = e; }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const double ov = __shfl_xor(bv, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        if (be < 0 || be >= E) be = 0;            // only reachable with non-finite logits
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        const double s = 1.0 / (1.0 + exp(-bv));
        ssum += s;
        if (lane == 0) {
            idx_out[j] = be;
            if (idx_lds) idx_lds[j] = be;
            w_out[j] = (float)s;                   // provisional: score, normalised below
        }
    }
    // normalise (lane 0 owns the k outputs); recompute each score exactly as above
    if (lane == 0) {
        for (int j = 0; j < k; ++j) {
            const int e = idx_out[j];
            const double s = 1.0 / (1.0 + exp(-logit(e)));
            w_out[j] = (float)(s / ssum);
        }
    }
}

template <int MAXPL>
__global__ __launch_bounds__(256) void route_topk(const double *logits, const float *bias, int nparts, int T,
                                                  int E, int k, int32_t *topk_idx, float *topk_w)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    wave_topk<MAXPL>(logits + (size_t)t * E, E, k, lane, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, nullptr,
              nparts, (size_t)T * E, bias);
}

// ---------------------------------------------------------------- grouping
// Large T.  rank: one wave per tile of 64 tokens; bit t of mask[e] is set when
// token t of the tile selected expert e, so the rank of (t, e) inside the tile
// is popcount(mask[e] below bit t).
__global__ __launch_bounds__(64) void route_rank(const int32_t *topk_idx, int T, int E, int k,
                                                 int32_t *rank, int32_t *tile_counts)
{
    extern __shared__ uint32_t mask[];           // [E][2]
    const int lane = threadIdx.x;
    const int tile = blockIdx.x;
    for (int i = lane; i < 2 * E; i += 64) mask[i] = 0;
    __syncthreads();
    const int t = tile * 64 + lane;
    if (t < T)
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[(size_t)t * k + j];
            atomicOr(&mask[2 * e + (lane >> 5)], 1u << (lane & 31));
        }
    __syncthreads();
    if (t < T) {
        const uint64_t below = lane ? ((1ull << lane) - 1ull) : 0ull;
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[(size_t)t * k + j];
            const uint64_t m = (uint64_t)mask[2 * e] | ((uint64_t)mask[2 * e + 1] << 32);
            rank[(size_t)t * k + j] = __popcll(m & below);
        }
    }
    for (int e = lane; e < E; e += 64)
        tile_counts[(size_t)tile * E + e] = __popc(mask[2 * e]) + __popc(mask[2 * e + 1]);
}

// one work-group of 1024 threads: per-expert running sums over the tiles, then
// an exclusive scan over the experts
__global__ __launch_bounds__(1024) void route_scan(int ntiles, int E, int Tk, int32_t *tile_counts,
                                                   int32_t *offsets)
{
    __shared__ int32_t part[1024];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E)
        for (int t0 = 0; t0 < ntiles; t0 += 16) {
            // sixteen tiles' counts requested together, then the running sum
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = t0 + i < ntiles ? tile_counts[(size_t)(t0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (t0 + i < ntiles) {
                    tile_counts[(size_t)(t0 + i) * E + e] = run;   // becomes the tile base
                    run += c[i];
                }
        }
    part[e] = e < E ? run : 0;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {        // inclusive Hillis-Steele scan
        const int v = e >= off ? part[e - off] : 0;
        __syncthreads();
        part[e] += v;
        __syncthreads();
    }
    if (e < E) offsets[e] = part[e] - run;
    if (e == 0) offsets[E] = Tk;
}

__global__ __launch_bounds__(256) void route_scatter(const int32_t *topk_idx, const int32_t *rank,
                                                     const int32_t *tile_base, const int32_t *offsets,
                                                     int T, int E, int k, int32_t *perm, int32_t *inv)
{
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= T * k) return;
    const int t = a / k;
    const int e = topk_idx[a];
    const int pos = offsets[e] + tile_base[(size_t)(t >> 6) * E + e] + rank[a];
    perm[pos] = a;
    inv[a] = pos;
}

// Small T (T <= 64): one work-group does top-k, counting, scan and scatter.
__global__ __launch_bounds__(256) void route_select_small(const double *logits, int T, int E, int k,
                                                          int32_t *topk_idx, float *topk_w,
                                                          int32_t *offsets, int32_t *perm, int32_t *inv)
{
    __shared__ uint32_t mask[2 * 1024];
    __shared__ int32_t cnt[1024];
    __shared__ int32_t sidx[64 * 32];            // T*k <= 2048
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < 2 * E; i += 256) mask[i] = 0;
    for (int t = wave; t < T; t += 4)
        wave_topk(logits + (size_t)t * E, E, k, lane, topk_idx + (size_t)t * k, topk_w + (size_t)t * k,
                  sidx + t * k);
    __syncthreads();
    for (int a = tid; a < T * k; a += 256) {
        const int t = a / k, e = sidx[a];
        atomicOr(&mask[2 * e + (t >> 5)], 1u << (t & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) cnt[e] = __popc(mask[2 * e]) + __popc(mask[2 * e + 1]);
    __syncthreads();
    if (tid == 0) {                               // E <= 1024 serial prefix sum
        int run = 0;
        for (int e = 0; e < E; ++e) { const int c = cnt[e]; cnt[e] = run; offsets[e] = run; run += c; }
        offsets[E] = run;
    }
    __syncthreads();
    for (int a = tid; a < T * k; a += 256) {
        const int t = a / k, e = sidx[a];
        const uint64_t m = (uint64_t)mask[2 * e] | ((uint64_t)mask[2 * e + 1] << 32);
        const uint64_t below = t ? ((1ull << t) - 1ull) : 0ull;
        const int pos = cnt[e] + __popcll(m & below);
        perm[pos] = a;
        inv[a] = pos;
    }
}

// ---------------------------------------------------------------- launchers
void launch_route_logits(const void *x, bool xbf16, const float *wr, const float *bias, int T, int H, int E,
                         double *logits, hipStream_t s)
{
    if (T <= 64) {
        dim3 grid(E, (T + 7) / 8);
        if (xbf16) route_logits_small<true><<<grid, 64, 0, s>>>(x, wr, bias, T, H, E, logits);
        else route_logits_small<false><<<grid, 64, 0, s>>>(x, wr, bias, T, H, E, logits);
    } else if (route_logits_parts(T, H) > 1) {
        dim3 grid((T + 63) / 64, (E + 63) / 64, ROUTE_KPARTS);
        if (xbf16) route_logits_mfma<true><<<grid, 256, 0, s>>>(x, wr, T, H, E, logits);
        else route_logits_mfma<false><<<grid, 256, 0, s>>>(x, wr, T, H, E, logits);
    } else {
        dim3 grid((T + 63) / 64, (E + 63) / 64);
        if (xbf16) route_logits_tiled<true><<<grid, 256, 0, s>>>(x, wr, bias, T, H, E, logits);
        else route_logits_tiled<false><<<grid, 256, 0, s>>>(x, wr, bias, T, H, E, logits);
    }
}

void launch_route_select_small(const double *logits, int T, int E, int k, int32_t *topk_idx, float *topk_w,
                               int32_t *offsets, int32_t *perm, int32_t *inv, hipStream_t s)
{
    route_select_small<<<1, 256, 0, s>>>(logits, T, E, k, topk_idx, topk_w, offsets, perm, inv);
}

void launch_route_topk(const double *logits, const float *bias, int T, int H, int E, int k, int32_t *topk_idx,
                       float *topk_w, hipStream_t s)
{
    // the fp64 MFMA logits leave partial sums without the bias; the other
    // logits kernels leave finished logits
    const int np = route_logits_parts(T, H);
    // unrolled for the experts each lane holds (E <= 64 * MAXPL)
#define MOE_TOPK(pl) route_topk<pl><<<(T + 3) / 4, 256, 0, s>>>(logits, np > 1 ? bias : nullptr, np, T, E, k, topk_idx, topk_w)
    if (E <= 64) MOE_TOPK(1);
    else if (E <= 128) MOE_TOPK(2);
    else if (E <= 256) MOE_TOPK(4);
    else if (E <= 512) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
}

int route_logits_parts(int T, int H) { return T > 64 && H % (32 * ROUTE_KPARTS) == 0 ? ROUTE_KPARTS : 1; }

void launch_route_rank(const int32_t *topk_idx, int T, int E, int k, int32_t *rank, int32_t *tile_counts,
                       hipStream_t s)
{
    route_rank<<<(T + 63) / 64, 64, 2 * E * sizeof(uint32_t), s>>>(topk_idx, T, E, k, rank, tile_counts);
}

void launch_route_scan(int T, int E, int k, int32_t *tile_counts, int32_t *offsets, hipStream_t s)
{
    route_scan<<<1, 1024, 0, s>>>((T + 63) / 64, E, T * k, tile_counts, offsets);
}

void launch_route_scatter(const int32_t *topk_idx, const int32_t *rank, const int32_t *tile_base,
                          const int32_t *offsets, int T, int E, int k, int32_t *perm, int32_t *inv, hipStream_t s)
{
    route_scatter<<<(T * k + 255) / 256, 256, 0, s>>>(topk_idx, rank, tile_base, offsets, T, E, k, perm, inv);
}

}  // namespace moe

// ============================================================================
// Small-T router (T <= 64, k <= 64, E <= 1024) in two launches.
//
// route_partial: every wave computes fp64 partial logits for EW experts x TB
// tokens over one H chunk (16-byte loads of W_r rows, 8-byte loads of bf16 x,
// all loads of a batch issued before the arithmetic) and writes
// partial[c][t][e].  Selection: a work-group per token sums the chunks in
// order and ranks the experts; T == 1 then groups in the same work-group,
// otherwise one more work-group builds offsets, perm and inv.  Every expert's logit is summed in the same order, so equal rows of
// W_r give equal logits and ties resolve to the lower index exactly as in a
// sequential evaluation.  (A single launch that lets its last work-group do
// the selection needs a device-scope release/acquire in every work-group;
// on this chip those write back and invalidate the L2 of each XCD and cost
// far more than the second launch.)
// ============================================================================
namespace moe {

template <int EW, int TB, bool XBF16>
__global__ __launch_bounds__(256) void route_partial(const void *x, const float *wr, int T, int H, int E, int NC,
                                                     int HC, double *part)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave;
    if (item >= (E / EW) * ((T + TB - 1) / TB) * NC) return;
    route_partial_item<EW, TB, XBF16>(x, wr, T, H, E, NC, HC, item, lane, part);
}

// Exact top-k of one token by rank counting: thread e counts the experts that
// beat it (larger logit, or equal logit and lower index); rank < k selects it.
// The ranks are a permutation of 0..E-1 (no NaN reaches here), so exactly k
// distinct experts are selected.
// All threads read the same logit at a time (LDS broadcast).  Writes the
// selections in rank order and their normalised sigmoid weights.  256 threads.
__device__ void rank_topk(const double *lg, int E, int k, int32_t *idx_out, float *w_out, int32_t *sel_e,
                          double *sel_l)
{
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) {
        const double le = lg[e];
        int r = 0;
        int f = 0;
        for (; f + 4 <= E; f += 4) {
            const double l0 = lg[f], l1 = lg[f + 1], l2 = lg[f + 2], l3 = lg[f + 3];
            r += (l0 > le) || (l0 == le && f < e);
            r += (l1 > le) || (l1 == le && f + 1 < e);
            r += (l2 > le) || (l2 == le && f + 2 < e);
            r += (l3 > le) || (l3 == le && f + 3 < e);
        }
        for (; f < E; ++f) r += (lg[f] > le) || (lg[f] == le && f < e);
        if (r < k) { sel_e[r] = e; sel_l[r] = le; }
    }
    __syncthreads();
    if (tid < 64) {
        // weights: sigmoid of the selected logits over their sum (fp64)
        double s = 0.0;
        for (int j = tid; j < k; j += 64) s += 1.0 / (1.0 + exp(-sel_l[j]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        for (int j = tid; j < k; j += 64) {
            idx_out[j] = sel_e[j];
            w_out[j] = (float)((1.0 / (1.0 + exp(-sel_l[j]))) / s);
        }
    }
}

__device__ __forceinline__ void token_logits(const double *part, const float *bias, int T, int E, int NC, int t,
                                             double *lg)
{
    for (int e = threadIdx.x; e < E; e += 256) {
        double v = part[(size_t)t * E + e];
        for (int c = 1; c < NC; ++c) v += part[((size_t)c * T + t) * E + e];
        if (bias) v += (double)bias[e];
        lg[e] = v != v ? -INFINITY : v;   // NaN ranks below every number, so ranks stay a permutation
    }
    __syncthreads();
}

// counts, offsets, perm and inv from the selections (T <= 64); 256 threads
__device__ void group_small(const int32_t *sidx, int T, int E, int k, int32_t *offsets, int32_t *perm, int32_t *inv,
                            uint32_t *mask, int32_t *cnt)
{
    const int tid = threadIdx.x;
    for (int i = tid; i < 2 * E; i += 256) mask[i] = 0;
    __syncthreads();
    for (int a = tid; a < T * k; a += 256) {
        const int t = a / k, e = sidx[a];
        atomicOr(&mask[2 * e + (t >> 5)], 1u << (t & 31));
    }
    __syncthreads();
    int local[4], run = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        local[i] = e < E ? __popc(mask[2 * e]) + __popc(mask[2 * e + 1]) : 0;
        run += local[i];
    }
    cnt[tid] = run;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int v = tid >= off ? cnt[tid - off] : 0;
        __syncthreads();
        cnt[tid] += v;
        __syncthreads();
    }
    int base = cnt[tid] - run;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        if (e < E) { cnt[e] = base; offsets[e] = base; }
        base += local[i];
    }
    if (tid == 255) offsets[E] = base;
    __syncthreads();
    for (int a = tid; a < T * k; a += 256) {
        const int t = a / k, e = sidx[a];
        const uint64_t m = (uint64_t)mask[2 * e] | ((uint64_t)mask[2 * e + 1] << 32);
        const uint64_t below = t ? ((1ull << t) - 1ull) : 0ull;
        const int pos = cnt[e] + __popcll(m & below);
        perm[pos] = a;
        inv[a] = pos;
    }
}

template <int MAXPL>
__global__ __launch_bounds__(64) void route_select_one(const double *part, const float *bias, int E, int k, int NC,
                                                       int32_t *topk_idx, float *topk_w, int32_t *offsets,
                                                       int32_t *perm, int32_t *inv)
{
    select_one<MAXPL>(part, bias, E, k, NC, threadIdx.x, topk_idx, topk_w, offsets, perm, inv, true, nullptr, nullptr);
}

// 1 < T <= 64: one work-group per token selects ...
__global__ __launch_bounds__(256) void route_select_tok(const double *part, const float *bias, int T, int E, int k,
                                                        int NC, int32_t *topk_idx, float *topk_w)
{
    __shared__ double lg[1024];
    __shared__ double sel_l[64];
    __shared__ int32_t sel_e[64];
    const int t = blockIdx.x;
    token_logits(part, bias, T, E, NC, t, lg);
    rank_topk(lg, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, sel_e, sel_l);
}

// ... and one work-group groups them
__global__ __launch_bounds__(256) void route_group_small(const int32_t *topk_idx, int T, int E, int k,
                                                         int32_t *offsets, int32_t *perm, int32_t *inv)
{
    __shared__ int32_t sidx[64 * 64];
    __shared__ uint32_t mask[2 * 1024];
    __shared__ int32_t cnt[1024];
    for (int a = threadIdx.x; a < T * k; a += 256) sidx[a] = topk_idx[a];
    __syncthreads();
    group_small(sidx, T, E, k, offsets, perm, inv, mask, cnt);
}

int route_decode_chunks(int T, int H)
{
    // enough waves to spread the W_r stream over the chip at small T; the
    // split depends on H only, so a token's logits do not depend on T
    (void)T;
    const int steps = (H + 255) / 256;
    return std::min(4, steps);
}

void launch_route_partial(const void *x, bool xbf16, const float *wr, int T, int H, int E, double *part, hipStream_t s)
{
    const int NC = route_decode_chunks(T, H);
    const int steps = (H + 255) / 256;
    const int HC = ((steps + NC - 1) / NC) * 256;
    const int EW = (T > 8 && E % 4 == 0) ? 4 : 1;
    const int TB = T <= 2 ? 1 : 8;
    const int items = (E / EW) * ((T + TB - 1) / TB) * NC;
    const int grid = (items + 3) / 4;
#define MOE_RP(ew, tb, xb) route_partial<ew, tb, xb><<<grid, 256, 0, s>>>(x, wr, T, H, E, NC, HC, part)
    if (EW == 4) { if (xbf16) MOE_RP(4, 8, true); else MOE_RP(4, 8, false); }
    else if (TB == 8) { if (xbf16) MOE_RP(1, 8, true); else MOE_RP(1, 8, false); }
    else { if (xbf16) MOE_RP(1, 1, true); else MOE_RP(1, 1, false); }
#undef MOE_RP
}

void launch_route_select(const double *part, const float *bias, int T, int H, int E, int k, int32_t *topk_idx,
                         float *topk_w, int32_t *offsets, int32_t *perm, int32_t *inv, hipStream_t s)
{
    const int NC = route_decode_chunks(T, H);
    if (T == 1) {
        if (E <= 64) route_select_one<1><<<1, 64, 0, s>>>(part, bias, E, k, NC, topk_idx, topk_w, offsets, perm, inv);
        else if (E <= 128) route_select_one<2><<<1, 64, 0, s>>>(part, bias, E, k, NC, topk_idx, topk_w, offsets, perm, inv);
        else if (E <= 256) route_select_one<4><<<1, 64, 0, s>>>(part, bias, E, k, NC, topk_idx, topk_w, offsets, perm, inv);
        else if (E <= 512) route_select_one<8><<<1, 64, 0, s>>>(part, bias, E, k, NC, topk_idx, topk_w, offsets, perm, inv);
        else route_select_one<16><<<1, 64, 0, s>>>(part, bias, E, k, NC, topk_idx, topk_w, offsets, perm, inv);
    } else {
        route_select_tok<<<T, 256, 0, s>>>(part, bias, T, E, k, NC, topk_idx, topk_w);
        route_group_small<<<1, 256, 0, s>>>(topk_idx, T, E, k, offsets, perm, inv);
    }
}

}  // namespace moe
