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
#include "kernels.h"

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

// ---------------------------------------------------------------- top-k
// One wave selects the k best experts of one token: k rounds of a wave-wide
// arg-max over (logit desc, expert asc).  Each lane holds experts lane+64*i.
__device__ __forceinline__ void wave_topk(const double *l, int E, int k, int lane, int32_t *idx_out,
                                          float *w_out, int32_t *idx_lds)
{
    constexpr int MAXPL = 16;                    // E <= 1024
    double v[MAXPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? l[e] : -INFINITY;
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
            const double s = 1.0 / (1.0 + exp(-l[e]));
            w_out[j] = (float)(s / ssum);
        }
    }
}

__global__ __launch_bounds__(256) void route_topk(const double *logits, int T, int E, int k,
                                                  int32_t *topk_idx, float *topk_w)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    wave_topk(logits + (size_t)t * E, E, k, lane, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, nullptr);
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
        for (int tile = 0; tile < ntiles; ++tile) {
            const int c = tile_counts[(size_t)tile * E + e];
            tile_counts[(size_t)tile * E + e] = run;    // becomes the tile base
            run += c;
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

void launch_route_topk(const double *logits, int T, int E, int k, int32_t *topk_idx, float *topk_w, hipStream_t s)
{
    route_topk<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
}

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
