// Single-token decode (T = 1): the memory-bound case the pages describe for
// decode, where every routed weight is read once per token step while compute
// idles ("Part 5: 服务层", section 6).  After the router:
//
//   dec1_gateup: gate/up GEMVs.  One persistent work-group of 16 waves per
//     CU (the waves share one routed table); each takes one role.  Shared-expert units are 16 bf16 rows x one K
//     eighth, loaded straight into MFMA B registers, x as the A operand.  The
//     routed role is a table lookup: a work-group owns one 1024-wide K chunk,
//     builds T[g][c] = codeword c . x[8g .. 8g+7] for the chunk's 128 groups
//     and all 256 codewords once (fp32, from MFMA with exact operands), then
//     streams row tiles of the selected experts through it, one 4-byte LDS
//     read per 8 weights, with the fp32 sub-block scale s_j and block scale d
//     applied to the sums.  It writes one fp32 partial per row and chunk; the
//     shared expert writes fp32 partial sums of its K eighths.
//   dec1_hform + dec1_down_fused (k <= 8, I <= 2048, sh_inter <= 2048):
//     dec1_hform forms h = silu(g) * u once -- the routed chunk partials and
//     the shared K parts added in order -- as two bf16 terms (hi + lo,
//     relative error below 2^-17), with the per-16 sums Q2_K's min term needs.
//     dec1_down_fused: a work-group of 16 waves owns 32 output rows; each wave
//     takes 16 of them for one top-k slot (Q2_K) and one K eighth of the bf16
//     shared down, so each CU mixes table lookups with streaming; the wave sums meet
//     in LDS and y is written directly.  Q2_K codes become exact bf16 values
//     sc*q through a 32 KB LDS table indexed by (sc, code byte); the block
//     scale d and the min term dmin * sum_j m_j X_j apply to the fp32 sums of
//     each 256-wide block.
//   Other shapes: dec1_down (persistent; a routed work-group forms h for its
//     slots itself; a unit is 128 output rows of one slot's Q2_K down or of
//     one 512-wide K part of the shared down) and dec1_combine (y = the
//     shared expert's K parts in order + the routed outputs weighted in top-k
//     order).
//
// The role split gives each role work-groups in proportion to its measured
// cost per byte.  Routed buffers are indexed by top-k slot j (partials, O),
// so no kernel needs the grouping arrays at T = 1.  Activation terms (x or h
// as hi + lo bf16) enter as rows 0 and 1 of an MFMA A operand, so one MFMA
// covers both.  Work-groups of one launch never wait for each other: results
// pass between work-groups only across launches.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "decode.h"
#include "devcache.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

constexpr int D1_THREADS = 512;
constexpr int GU_THREADS = 1024;   // gate/up: 16 waves share one routed table per CU
constexpr int GU_WAVES = GU_THREADS / 64;
constexpr int SH_KQ = DEC_SH_KQ;   // K parts of the shared gate/up
constexpr int SH_MAXS = 2;         // shared gate/up K steps (of 32) per wave and unit
constexpr int DN_ROWS = 128;       // output rows of a down unit (16 per wave)
constexpr int DN_KPART = 512;      // K part of a shared down unit
constexpr int DN_MAXB = 8;         // Q2_K blocks per row of a routed down unit (I <= 2048)
constexpr int DN_MAXKC = 8;        // K chunks of the routed gate/up tables (H <= 8192)
constexpr int DF_SHSEG = 4;        // 512-wide K segments of the staged shared down (sh_inter <= 2048)
constexpr size_t LDS_MAX = 160 * 1024;
// Routed gate/up tiles per work-group in the register ring (2..6).  Measured
// on decode1: 2 (the next tile in flight while one is computed) is fastest;
// deeper rings put more scattered row windows in flight at once and were
// slower (63.1 / 65.5 / 67.5 / 69.1 us per step for 2 / 3 / 4 / 5).
constexpr int GU_PF = 2;
static_assert(GU_PF >= 2 && GU_PF <= 6, "ring of 2 to 6 register sets");
static_assert(256 * DEC_LUT_KB * DN_MAXKC / 8 <= GU_THREADS, "stage 1 stages x with one 8-value piece per thread");

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo)
{
    hi = f32_to_bf16_rne(v);
    lo = f32_to_bf16_rne(v - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ u32x4 pack8(const uint32_t h[8])
{
    return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// A operand of one token's activation terms: row 0 = hi, row 1 = lo (when
// there are two terms), other rows zero.  Lane (fr, fc) supplies 8 values at k.
template <bool TWO>
__device__ __forceinline__ bf16x8 act_rows(const uint16_t *hi, const uint16_t *lo, int k, int fr)
{
    bf16x8 a = {};
    if (fr == 0) a = *(const bf16x8 *)&hi[k];
    else if (TWO && fr == 1) a = *(const bf16x8 *)&lo[k];
    return a;
}

// The eight A fragments k0, k0 + step, ... of one block for rows 0 (and 1 with
// two terms), read in one masked region.  Rows 2..15 of A only feed rows 2..15
// of D, which no caller reads, so they are left as they are.
template <bool TWO>
__device__ __forceinline__ void act_block(const uint16_t *row, int k0, int step, int fr, bf16x8 (&a)[8])
{
    if (fr < (TWO ? 2 : 1)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) a[m] = *(const bf16x8 *)&row[k0 + step * m];
    }
}

__device__ __forceinline__ int clamp_expert(int g, int E) { return min(max(g, 0), E - 1); }
// index of expert e's matrices in the routed weight arrays (an expert cache
// view maps experts to slots)
__device__ __forceinline__ int expert_matrix(const DecPass &p, int e) { return p.slot ? max(p.slot[e], 0) : e; }

// ============================================================== gate / up
// One kernel, four launch modes:
//   GU_SPLIT   work-groups [0, gu_sh_wg) take shared-expert gate/up units
//              u = wg, wg + gu_sh_wg, ...; the others take routed units.
//   GU_STAGE1  every work-group first takes router items (fp64 partial logits
//              of one expert over one H chunk, when p.route), then shared
//              gate/up units.
//   GU_STAGE1R the same with bf16 x and at most one item per wave: a wave's
//              item overlaps its first shared rows.
//   GU_STAGE2  every work-group takes routed gate/up units.  Before them,
//              wave 0 selects the experts from the partial logits when
//              p.route (every work-group selects, the first also writes the
//              routing outputs), waves 8..15 build the work-group's table,
//              and waves 1..15 stream rows of the shared down (the shared h
//              is complete after stage 1), so the selection's latency is
//              spent on bytes the step needs anyway.
enum { GU_SPLIT = 0, GU_STAGE1 = 1, GU_STAGE2 = 2, GU_STAGE1R = 3 };

// Whole-row GEMV pieces of the staged layer's shared expert.  A wave streams
// rows from HBM in 512-wide K segments (64 lanes x 8 bf16, 1 KB contiguous per
// load instruction), so every row is read front to back; the activation's
// matching 8 values sit in the lane's registers (or come from LDS), and pairs
// of bf16 products accumulate in fp32 (v_dot2c_f32_bf16: the products of
// bf16 values are exact).  One wave reduction per row.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t w, uint32_t a, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, a), acc, false);
}

// the elements are copied out first: a bit cast of a vector element (w.y)
// would reinterpret the storage from the vector's start
__device__ __forceinline__ float dot8(const u32x4 &w, const u32x4 &a, float acc)
{
    const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w, a0 = a.x, a1 = a.y, a2 = a.z, a3 = a.w;
    acc = dot2(w0, a0, acc);
    acc = dot2(w1, a1, acc);
    acc = dot2(w2, a2, acc);
    acc = dot2(w3, a3, acc);
    return acc;
}

// sum over the 64 lanes (in a fixed butterfly order; every lane gets it)
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Stage 1, shared gate/up: unit = one feature and one half of K; waves 2i and
// 2i + 1 of a work-group take the two halves of feature 8 (round * G + wg) + i.
// The halves meet in LDS and the first wave writes the feature's
// h = silu(g) * u as two bf16 terms (sh_hi, sh_lo).  x (one or two bf16 terms)
// was staged in LDS by the caller.
// hook(i), i = 0, 1: called once each per wave, in order, right after the
// wave's i-th batch of shared loads is requested (at the start or the end when
// the wave has fewer batches), for work that should run while those loads are
// in flight; it may use wave-wide operations.  Every load here is
// unconditional (a wave past sh_inter re-reads the last row and does not use
// it), so the compiler can wait for exactly the loads a use needs.
template <bool XF32, typename Hook>
__device__ __forceinline__ void dec1_shared_gateup_rows(const DecPass &p, const uint16_t *xh, const uint16_t *xl,
                                                        float *red, int G, Hook &&hook)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int H = p.H, ns = H / 512, half = wave & 1, nlo = ns / 2;
    const int s0 = half ? nlo : 0, s1 = half ? ns : nlo;
    const int rounds = (p.Ish + 8 * G - 1) / (8 * G);
    constexpr int B = 4;                                          // segments requested together
    const int nb0 = rounds > 0 ? (s1 - s0 + B - 1) / B : 0;       // round 0's batches (uniform over the wave)
    if (nb0 == 0) {
        hook(0);
        hook(1);
    }
    for (int rd = 0; rd < rounds; ++rd) {
        const int f = 8 * (rd * G + (int)blockIdx.x) + (wave >> 1);
        const int fl = min(f, p.Ish - 1);
        float ag = 0.f, au = 0.f;
        const uint16_t *rg = p.sg + (int64_t)fl * H + 8 * lane, *ru = p.su + (int64_t)fl * H + 8 * lane;
        for (int sb = s0; sb < s1; sb += B) {
            u32x4 g4[B], u4[B];
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const int sg = min(sb + i, s1 - 1);               // past the half: re-read, not used
                g4[i] = *(const u32x4 *)(rg + 512 * sg);
                u4[i] = *(const u32x4 *)(ru + 512 * sg);
            }
            if (rd == 0 && sb == s0) hook(0);                     // uniform over the wave
            if (rd == 0 && sb == s0 + B) hook(1);
#pragma unroll
            for (int i = 0; i < B; ++i) {
                if (sb + i >= s1) break;
                const int k = 512 * (sb + i) + 8 * lane;
                const u32x4 a = *(const u32x4 *)&xh[k];
                ag = dot8(g4[i], a, ag);
                au = dot8(u4[i], a, au);
                if (XF32) {
                    const u32x4 al = *(const u32x4 *)&xl[k];
                    ag = dot8(g4[i], al, ag);
                    au = dot8(u4[i], al, au);
                }
            }
        }
        ag = wave_sum(ag);
        au = wave_sum(au);
        if (half && lane == 0) { red[2 * (wave >> 1)] = ag; red[2 * (wave >> 1) + 1] = au; }
        __syncthreads();
        if (!half && lane == 0 && f < p.Ish) {
            const float g = ag + red[2 * (wave >> 1)], uu = au + red[2 * (wave >> 1) + 1];
            const float h = g / (1.0f + expf(-g)) * uu;
            uint32_t hi, lo;
            split_bf16(h, hi, lo);
            p.sh_hi[f] = (uint16_t)hi;
            p.sh_lo[f] = (uint16_t)lo;
        }
        __syncthreads();
    }
    if (nb0 == 1) hook(1);
}

// Stage 2, shared down: wave slot n of NW streams output rows n, n + NW, ...
// over all of sh_inter, with the shared h for its lanes' K positions (two bf16
// terms per value) in registers; the row's sum goes to O_sh[row] (one part).
// Two rows are in flight per wave.  Waves need not meet: no barrier.
__device__ __forceinline__ void dec1_shared_down_rows(const DecPass &p, int n, int NW)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int H = p.H, ns = p.Ish / 512;                          // <= DF_SHSEG segments
    u32x4 hh[DF_SHSEG], hl[DF_SHSEG];
#pragma unroll
    for (int s = 0; s < DF_SHSEG; ++s) {
        const int k = 512 * min(s, ns - 1) + 8 * lane;
        hh[s] = *(const u32x4 *)(p.sh_hi + k);
        hl[s] = *(const u32x4 *)(p.sh_lo + k);
    }
    u32x4 Wa[DF_SHSEG], Wb[DF_SHSEG];
    auto load = [&](int r, u32x4 (&W4)[DF_SHSEG]) {
        const uint16_t *rw = p.sd + (int64_t)min(r, H - 1) * p.Ish + 8 * lane;
#pragma unroll
        for (int s = 0; s < DF_SHSEG; ++s) W4[s] = *(const u32x4 *)(rw + 512 * min(s, ns - 1));
    };
    auto row = [&](int r, const u32x4 (&W4)[DF_SHSEG]) {
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < DF_SHSEG; ++s) {
            if (s < ns) {
                acc = dot8(W4[s], hh[s], acc);
                acc = dot8(W4[s], hl[s], acc);
            }
        }
        acc = wave_sum(acc);
        if (lane == 0 && r < H) p.O_sh[r] = acc;
    };
    if (n >= H) return;                                           // uniform over the wave
    // two register sets in turn; the prefetch past the last row re-reads it
    load(n, Wa);
    for (int r = n;;) {
        load(r + NW < H ? r + NW : r, Wb);
        row(r, Wa);
        if ((r += NW) >= H) break;
        load(r + NW < H ? r + NW : r, Wa);
        row(r, Wb);
        if ((r += NW) >= H) break;
    }
}

// Work-groups go to the chip's 8 XCDs in turn (work-group b to XCD b % 8),
// and each XCD has its own L2.  Numbering the G work-groups XCD by XCD (all
// of XCD 0 first, in launch order, then XCD 1, ...) puts consecutive numbers
// on one XCD: the K chunks of one row tile, whose 152-byte pieces of a row
// share cache lines at their edges, then fetch those lines through one L2.
// A bijection of [0, G) for any G.
__device__ __forceinline__ int xcd_major(int b, int G)
{
    const int x = b & 7;
    int below = 0;                                                // work-groups on XCDs 0 .. x - 1
    for (int y = 0; y < x; ++y) below += (G - y + 7) >> 3;
    return below + (b >> 3);
}

template <bool XF32, int MODE = GU_SPLIT, int MAXPL = 4>
__global__ __launch_bounds__(GU_THREADS) void dec1_gateup_kernel(DecPass p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int kid[64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4;
    const int H = p.H;

    bool shared_role;
    int G, u;
    if constexpr (MODE == GU_STAGE1 || MODE == GU_STAGE1R) {
        shared_role = true;
        G = gridDim.x;
        u = blockIdx.x;
    } else if constexpr (MODE == GU_STAGE2) {
        shared_role = false;                                      // the shared down runs inside the routed role
        G = gridDim.x;
        u = xcd_major(blockIdx.x, G);
    } else {
        const int na = p.gu_sh_wg;
        shared_role = (int)blockIdx.x < na;
        G = shared_role ? na : p.gu_rt_wg;
        u = shared_role ? (int)blockIdx.x : (int)blockIdx.x - na;
    }
    if constexpr (MODE == GU_STAGE1 || MODE == GU_STAGE1R) {
        // x (hi, and lo for fp32 x) into LDS, the router's partial logits
        // (the same items and arithmetic as the router's own partial-logit
        // launch), then whole shared gate/up rows.
        uint16_t *xh = (uint16_t *)dsm;                           // [H] and a spare 8-value slot
        uint16_t *xl = xh + H + 8;                                // [H] (fp32 x only)
        float *red = (float *)(dsm + (XF32 ? 4 : 2) * (size_t)(H + 8));   // [8 features][2]
        const int nw = (int)gridDim.x * GU_WAVES, item = (int)blockIdx.x + (int)gridDim.x * wave;
        if constexpr (MODE == GU_STAGE1R) {
            // bf16 x, one router item per wave at most, in one batch (the
            // launcher checks): the wave requests x, then its item's router
            // weights, and does the item's arithmetic (x from LDS) once its
            // first shared rows are requested too, so the three streams
            // overlap.  Loads are unconditional (past the end they re-read the
            // last piece or item), so the compiler waits for exactly the loads
            // each use needs.  H / 8 <= GU_THREADS: one 8-value piece of x per
            // thread.
            static_assert(!XF32, "the overlapped router items read bf16 x from LDS");
            const int nitems = p.E * p.rnc;
            const u32x4 xb = *(const u32x4 *)((const uint16_t *)p.x + 8 * min(tid, H / 8 - 1));
            RouteItem1 ri;
            route_item1_begin(H, p.rnc, p.rhc, min(item, nitems - 1), lane, ri);
            route_item1_load(p.wr, H, 0, ri);
            // every thread stores (those past H / 8 into a spare slot), so the
            // x load is not moved behind the router loads into a branch
            *(u32x4 *)&xh[tid < H / 8 ? 8 * tid : H] = xb;
            __syncthreads();
            const bool mine = item < nitems;                      // uniform over the wave
            // first half of the item under the first shared batch, its second
            // half's loads then, its arithmetic under the second batch
            dec1_shared_gateup_rows<false>(p, xh, xl, red, G, [&](int i) {
                if (i == 0) {
                    if (mine) route_item1_step(xh, 0, ri);
                    route_item1_load(p.wr, H, 1, ri);
                } else if (mine) {
                    route_item1_step(xh, 1, ri);
                    route_item1_end(ri, p.E, lane, p.rpart);
                }
            });
        } else {
            // the items first, spread over the whole grid
            if (p.route) {
                for (int it = item; it < p.E * p.rnc; it += nw)
                    route_partial_item<1, 1, !XF32>(p.x, p.wr, 1, H, p.E, p.rnc, p.rhc, it, lane, p.rpart);
            }
            for (int i = tid; i < H / 8; i += GU_THREADS) {
                if (XF32) {
                    const float *src = (const float *)p.x + 8 * i;
                    uint32_t h[8], l[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) split_bf16(src[e], h[e], l[e]);
                    *(u32x4 *)&xh[8 * i] = pack8(h);
                    *(u32x4 *)&xl[8 * i] = pack8(l);
                } else {
                    *(u32x4 *)&xh[8 * i] = *(const u32x4 *)((const uint16_t *)p.x + 8 * i);
                }
            }
            __syncthreads();
            dec1_shared_gateup_rows<XF32>(p, xh, xl, red, G, [](int) {});
        }
        return;
    }
    if (shared_role) {
        // ---------------------------------------------- shared expert
        const int n_units = (p.Ish / 16) * SH_KQ;
        if (u >= n_units) return;                                 // uniform over the work-group
        uint16_t *xh = (uint16_t *)dsm;                           // [H]
        uint16_t *xl = xh + H;                                    // [H] (fp32 x only)
        float *red = (float *)(dsm + (XF32 ? 4 : 2) * (size_t)H); // [16 waves][2][16]
        // x (hi, and lo for fp32 x) into LDS once
        for (int i = tid; i < H / 8; i += GU_THREADS) {
            if (XF32) {
                const float *src = (const float *)p.x + 8 * i;
                uint32_t h[8], l[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) split_bf16(src[e], h[e], l[e]);
                *(u32x4 *)&xh[8 * i] = pack8(h);
                *(u32x4 *)&xl[8 * i] = pack8(l);
            } else {
                *(u32x4 *)&xh[8 * i] = *(const u32x4 *)((const uint16_t *)p.x + 8 * i);
            }
        }
        const int KQ = H / SH_KQ, nsteps = KQ / 32;
        u32x4 ga[SH_MAXS], ua[SH_MAXS], gb[SH_MAXS], ub[SH_MAXS];
        auto load = [&](int uu, u32x4 (&G4)[SH_MAXS], u32x4 (&U4)[SH_MAXS]) {
            const int r0 = (uu / SH_KQ) * 16, k0 = (uu % SH_KQ) * KQ;
            const uint16_t *rg = p.sg + (int64_t)(r0 + fr) * H + k0 + 8 * fc;
            const uint16_t *ru = p.su + (int64_t)(r0 + fr) * H + k0 + 8 * fc;
            // unconditional loads (steps past the end re-read the last one and
            // are never used): a load under a branch makes the compiler wait for it
#pragma unroll
            for (int j = 0; j < SH_MAXS; ++j) {
                const int st = min(wave + GU_WAVES * j, nsteps - 1);
                G4[j] = *(const u32x4 *)(rg + 32 * st);
                U4[j] = *(const u32x4 *)(ru + 32 * st);
            }
        };
        auto unit = [&](int uu, const u32x4 (&G4)[SH_MAXS], const u32x4 (&U4)[SH_MAXS]) {
            const int r0 = (uu / SH_KQ) * 16, q = uu % SH_KQ, k0 = q * KQ;
            f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
            // every step consumes its registers (steps past the end with a zero
            // A operand): a register left unread on some path keeps its load
            // pending there, and the next load into it would wait for it
#pragma unroll
            for (int j = 0; j < SH_MAXS; ++j) {
                const int st = wave + GU_WAVES * j;
                bf16x8 a = act_rows<XF32>(xh, xl, k0 + 32 * min(st, nsteps - 1) + 8 * fc, fr);
                if (st >= nsteps) a = bf16x8{};
                ag = mfma16x16x32(a, __builtin_bit_cast(bf16x8, G4[j]), ag);
                au = mfma16x16x32(a, __builtin_bit_cast(bf16x8, U4[j]), au);
            }
            // D[0][n] (x hi) and D[1][n] (x lo) of feature n sit in lane n, elements 0 and 1
            if (fc == 0) {
                red[(wave * 2 + 0) * 16 + fr] = XF32 ? ag[0] + ag[1] : ag[0];
                red[(wave * 2 + 1) * 16 + fr] = XF32 ? au[0] + au[1] : au[0];
            }
            __syncthreads();
            if (tid < 32) {
                const int m = tid >> 4, n = tid & 15;
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < GU_WAVES; ++w) sum += red[(w * 2 + m) * 16 + n];
                p.part_sh[(int64_t)(q * 2 + m) * p.Ish + r0 + n] = sum;
            }
            __syncthreads();
        };
        // the prefetch is unconditional (the last unit re-reads its own bytes,
        // which the L2 still holds): a load under a branch makes every later
        // wait assume the shorter path and wait for the prefetch as well
        load(u, ga, ua);
        __syncthreads();                                          // x staged
        for (;;) {
            load(u + G < n_units ? u + G : u, gb, ub);
            unit(u, ga, ua);
            u += G;
            if (u >= n_units) break;
            load(u + G < n_units ? u + G : u, ga, ua);
            unit(u, gb, ub);
            u += G;
            if (u >= n_units) break;
        }
        return;
    }

    // -------------------------------------------------- routed experts
    // Work-group r owns K chunk kc = r % nkc (DEC_LUT_KB blocks of 256) and
    // takes the tiles r / nkc, r / nkc + R, ... (R = work-groups per chunk).
    // Tile t is 128 features of one top-k slot, their gate and up rows.  The
    // work-group first builds the chunk's table T[g][c] = sum_v C[c][v]
    // x[8g + v] for its 32 * DEC_LUT_KB groups g and all 256 codewords c, one
    // MFMA per 32 x 32 tile (K = 16: x hi in K 0..7, x lo in K 8..15, the
    // codeword in both); then each 8-weight group of a row costs one 4-byte LDS
    // read.  A row's blocks of the chunk go to four adjacent lanes, straight
    // into registers; their sums meet in the quad and one fp32 partial per row
    // and chunk goes to part_rt; the down launch adds them in chunk order.
    // (stage 2 launches exactly R * nkc work-groups, so none returns here and
    // every one takes its share of the shared down)
    const int nkc = p.nkc, R = G / nkc;
    const int kc = u % nkc, j0 = u / nkc;
    if (j0 >= R) return;                                          // uniform over the work-group
    const int nbH = H >> 8, rb = p.gu_row_bytes;
    const int kb = min(DEC_LUT_KB, nbH - DEC_LUT_KB * kc);        // blocks in this chunk (2 or 4: H % 512 == 0)
    float *tab = (float *)dsm;                                    // [32 * DEC_LUT_KB groups][256 codewords]
    // The chunk's table and the expert ids are independent: waves 8..15
    // build the table (wave w: codewords 32 (w % 8) .. + 31 against every
    // 32-group tile of the chunk) while wave 0 selects the experts, so the
    // selection's latency covers the table's
    if (wave >= 8) {
        const int c = 32 * (wave & 7) + (lane & 31), hl = lane >> 5;
        const uint64_t cw = *(const uint64_t *)(p.codebook + 8 * c);
        f32x4 xv4[DEC_LUT_KB][2];
        bf16x8 xa[DEC_LUT_KB];
#pragma unroll
        for (int gt = 0; gt < DEC_LUT_KB; ++gt) {
            // tiles past a short chunk re-read its last one and are not built
            const int k = 256 * (DEC_LUT_KB * kc + min(gt, kb - 1)) + 8 * (lane & 31);
            if (XF32) {
                xv4[gt][0] = *(const f32x4 *)((const float *)p.x + k);
                xv4[gt][1] = *(const f32x4 *)((const float *)p.x + k + 4);
            } else {
                xa[gt] = *(const bf16x8 *)((const uint16_t *)p.x + k);
            }
        }
        uint32_t cb[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) cb[v] = f32_to_bf16_exact((float)(int8_t)(cw >> (8 * v)));
        const bf16x8 Bc = __builtin_bit_cast(bf16x8, pack8(cb));
#pragma unroll
        for (int gt = 0; gt < DEC_LUT_KB; ++gt) {
            if (gt >= kb) break;                                  // uniform over the work-group
            bf16x8 A = {};
            if (XF32) {
                const float xv[8] = {xv4[gt][0][0], xv4[gt][0][1], xv4[gt][0][2], xv4[gt][0][3],
                                     xv4[gt][1][0], xv4[gt][1][1], xv4[gt][1][2], xv4[gt][1][3]};
                uint32_t h8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t hi, lo;
                    split_bf16(xv[e], hi, lo);
                    h8[e] = hl ? lo : hi;
                }
                A = __builtin_bit_cast(bf16x8, pack8(h8));
            } else if (hl == 0) {
                A = xa[gt];
            }
            f32x16 D = {};
            D = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bc, D, 0, 0, 0);
            // D element v of lane l: group 8 (v / 4) + 4 (l / 32) + v % 4 of the tile, codeword c
#pragma unroll
            for (int v = 0; v < 16; ++v) tab[(32 * gt + 8 * (v >> 2) + 4 * hl + (v & 3)) * 256 + c] = D[v];
        }
    }
    if constexpr (MODE == GU_STAGE2) {
        // stage 2: waves 1..15 of every work-group stream the shared down's
        // rows (independent of the selection) while wave 0 selects
        if (wave > 0 && p.Ish > 0) dec1_shared_down_rows(p, u * (GU_WAVES - 1) + wave - 1, G * (GU_WAVES - 1));
    }
    if (MODE == GU_STAGE2 && p.route) {
        // every routed work-group selects the same experts from the partial
        // logits; the first one also writes the routing outputs
        if (wave == 0)
            select_one<MAXPL>(p.rpart, p.bias, p.E, p.k, p.rnc, lane, p.o_idx, p.o_w, p.o_off, p.o_perm, p.o_inv,
                              u == 0, kid, nullptr);
    } else if (tid < p.k) {
        kid[tid] = expert_matrix(p, clamp_expert(p.topk_idx[tid], p.E));
    }
    __syncthreads();                                              // expert ids and table staged
    // Lane (r, b) of wave w, r = lane / 4, b = lane % 4: block b of the chunk
    // in row 16 (w / 2) + r of the tile's gate (w even) or up (w odd)
    // features.  The four blocks of a row sit in adjacent lanes, so one load
    // instruction reads the row's whole chunk and its cache lines are used
    // at once; lanes past a short chunk re-read its last block and their
    // sums are not added.  Blocks start 2-byte aligned (rows are 4-byte
    // aligned): the 40-byte window from the aligned address at or below the
    // block covers it, and stays in the row (a block at a dword boundary is
    // never the last one, since every row has an even number of blocks).
    const int bl = lane & 3, hr = wave & 1, fo = 16 * (wave >> 1) + (lane >> 2);
    const int B = DEC_LUT_KB * kc + min(bl, kb - 1);
    const int boff = (38 * B) & ~3;
    const bool odd = B & 1;                                       // the block starts 2 bytes into its window
    const float *tb = tab + 32 * 256 * min(bl, kb - 1);
    const int nft = p.I / 128, ntile = p.k * nft;
    const uint8_t *wmat = hr ? p.wu : p.wg;
    auto rowp = [&](int t) -> const uint32_t * {
        const int s = t / nft, f = 128 * (t - s * nft) + fo;
        return (const uint32_t *)(wmat + (int64_t)kid[s] * p.gu_expert_bytes + (int64_t)f * rb + boff);
    };
    // GU_PF register sets in a ring: while one tile is computed, the next
    // GU_PF - 1 tiles of this work-group are in flight.  Loads past the last
    // tile re-read the first one and are never used.
    uint32_t W[GU_PF][10];
    auto load = [&](int t, uint32_t (&Wr)[10]) {
        const uint32_t *src = rowp(t);
#pragma unroll
        for (int e = 0; e < 10; ++e) Wr[e] = src[e];
    };
    int t = j0;
#pragma unroll
    for (int i = 0; i < GU_PF; ++i) load(t + i * R < ntile ? t + i * R : t, W[i]);
    // one row's block: sum over sub-blocks of s_j * (four table entries), times d
    auto task = [&](const uint32_t (&W)[10]) -> float {
        const uint32_t d16 = odd ? W[0] >> 16 : W[0] & 0xffffu;
        const uint32_t sc = odd ? W[1] : __builtin_amdgcn_alignbyte(W[1], W[0], 2);
        float acc = 0.f;
#pragma unroll
        for (int sb = 0; sb < 8; ++sb) {
            const uint32_t w = odd ? W[2 + sb] : __builtin_amdgcn_alignbyte(W[2 + sb], W[1 + sb], 2);
            const float *t4 = tb + 4 * sb * 256;
            const float tv = (t4[w & 255u] + t4[256 + ((w >> 8) & 255u)]) + (t4[512 + ((w >> 16) & 255u)] + t4[768 + (w >> 24)]);
            acc += (float)((sc >> (4 * sb)) & 15u) * tv;
        }
        return f16_bits_to_f32(d16) * acc;
    };
    const int64_t cstride = (int64_t)2 * p.k * p.I;               // one K chunk of part_rt
    // a row's block sums meet in the quad's first lane (quad_perm moves),
    // added in block order; that lane writes the row's partial
    auto quad_get = [](float v, auto j) -> float {
        constexpr int J = decltype(j)::value;
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), J * 0x55, 0xF, 0xF, false));
    };
    auto tile = [&](int tt, const uint32_t (&W)[10]) {
        const float v = task(W);
        const float v1 = quad_get(v, std::integral_constant<int, 1>{});
        const float v2 = quad_get(v, std::integral_constant<int, 2>{});
        const float v3 = quad_get(v, std::integral_constant<int, 3>{});
        if (bl == 0) {
            float sum = v;
            if (kb > 1) sum += v1;
            if (kb > 2) sum += v2;
            if (kb > 3) sum += v3;
            const int s = tt / nft, f0 = 128 * (tt - s * nft);
            p.part_rt[kc * cstride + (int64_t)(2 * s + hr) * p.I + f0 + fo] = sum;
        }
    };
    // the ring, unrolled so every register set has a fixed name: a tile is
    // computed from its set, which then takes the tile GU_PF steps later (an
    // unconditional load).  Waves do not meet: no barrier per tile.
#define MOE_GU_STEP(i)                                                             \
    if constexpr ((i) < GU_PF) {                                                   \
        tile(t, W[i]);                                                             \
        load(t + GU_PF * R < ntile ? t + GU_PF * R : t, W[i]);                     \
        if ((t += R) >= ntile) break;                                              \
    }
    for (;;) {
        MOE_GU_STEP(0)
        MOE_GU_STEP(1)
        MOE_GU_STEP(2)
        MOE_GU_STEP(3)
        MOE_GU_STEP(4)
        MOE_GU_STEP(5)
    }
#undef MOE_GU_STEP
}

// ============================================================== down
// Wave w computes output rows 16w.. of the unit's 128 over the whole K, so no
// reduction between waves is needed.  Each work-group takes a contiguous range
// of units, so the LDS copy of the activation (one slot's h, or one K part of
// the shared h) changes rarely.
__global__ __launch_bounds__(D1_THREADS) void dec1_down_kernel(DecPass p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int kid[64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4;
    const int H = p.H;
    const int n_ot = (H + DN_ROWS - 1) / DN_ROWS;
    const bool shared_role = (int)blockIdx.x < p.dn_sh_wg;
    const int G = shared_role ? p.dn_sh_wg : p.dn_rt_wg;
    const int w = shared_role ? (int)blockIdx.x : (int)blockIdx.x - p.dn_sh_wg;
    const int n_units = shared_role ? n_ot * (p.Ish / DN_KPART) : p.k * n_ot;
    const int u_begin = (int)(((int64_t)n_units * w) / G), u_end = (int)(((int64_t)n_units * (w + 1)) / G);
    if (u_begin >= u_end) return;                                  // uniform over the work-group

    if (shared_role) {
        // ---------------------------------------------- shared expert K parts
        uint16_t *hh = (uint16_t *)dsm, *hl = hh + DN_KPART;
        u32x4 wa[16], wb[16];                                      // two buffers in turn
        auto load = [&](int uu, u32x4 (&W4)[16]) {
            const int part = uu / n_ot, row = min((uu % n_ot) * DN_ROWS + 16 * wave + fr, H - 1);
            const uint16_t *rw = p.sd + (int64_t)row * p.Ish + part * DN_KPART + 8 * fc;
#pragma unroll
            for (int s = 0; s < 16; ++s) W4[s] = *(const u32x4 *)(rw + 32 * s);
        };
        int cur_part = -1;
        auto unit = [&](int uu, const u32x4 (&W4)[16]) {
            const int part = uu / n_ot, ot = uu % n_ot;
            if (part != cur_part) {
                // this part's slice of the shared h: add the gate/up K parts in
                // order, then silu(g) * u, split into two bf16 terms
                __syncthreads();
                const int k0 = part * DN_KPART;
                for (int i = tid; i < DN_KPART; i += D1_THREADS) {
                    float g = 0.f, uv = 0.f;
#pragma unroll
                    for (int q = 0; q < SH_KQ; ++q) {
                        g += p.part_sh[(int64_t)(q * 2 + 0) * p.Ish + k0 + i];
                        uv += p.part_sh[(int64_t)(q * 2 + 1) * p.Ish + k0 + i];
                    }
                    const float h = g / (1.0f + expf(-g)) * uv;
                    uint32_t hi, lo;
                    split_bf16(h, hi, lo);
                    hh[i] = (uint16_t)hi;
                    hl[i] = (uint16_t)lo;
                }
                __syncthreads();
                cur_part = part;
            }
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const bf16x8 a = act_rows<true>(hh, hl, 32 * s + 8 * fc, fr);
                P = mfma16x16x32(a, __builtin_bit_cast(bf16x8, W4[s]), P);
            }
            const int row = ot * DN_ROWS + 16 * wave + fr;
            if (fc == 0 && row < H) p.O_sh[(int64_t)part * H + row] = P[0] + P[1];
        };
        load(u_begin, wa);
        for (int u = u_begin;;) {                                  // unconditional prefetch, as above
            load(min(u + 1, u_end - 1), wb);
            unit(u, wa);
            if (++u >= u_end) break;
            load(min(u + 1, u_end - 1), wa);
            unit(u, wb);
            if (++u >= u_end) break;
        }
        return;
    }

    // -------------------------------------------------- routed Q2_K rows
    const int nb = p.nbI;
    // every slot's h (hi, lo) and min-term sums are staged once, so no load
    // of the unit loop has to wait behind a staging load
    uint16_t *tab = (uint16_t *)dsm;                               // [16 sc][256 bytes][4]
    uint16_t *hh = tab + 16 * 256 * 4;                             // [k][nb*256] hi
    uint16_t *hl = hh + p.k * nb * 256;                            // [k][nb*256] lo
    float *xm = (float *)(hl + p.k * nb * 256);                    // [k][nb][16] sub-block sums of h
    if (tid < p.k) kid[tid] = expert_matrix(p, clamp_expert(p.topk_idx[tid], p.E));
    __syncthreads();
    // two register buffers in turn, per block: this lane's 16 code bytes, the
    // sc|m bytes of its four sub-blocks, and d|dmin.  While one unit is
    // computed, the next is in flight.
    u32x4 ca[DN_MAXB], cb[DN_MAXB];
    uint32_t sa[DN_MAXB], sb[DN_MAXB], da[DN_MAXB], db[DN_MAXB];
    // unconditional loads (rows past H and blocks past nb re-read valid bytes
    // that are never used): a load under a branch makes the compiler wait for it
    auto load = [&](int uu, u32x4 (&C4)[DN_MAXB], uint32_t (&S4)[DN_MAXB], uint32_t (&D4)[DN_MAXB]) {
        const int slot = uu / n_ot, row = min((uu % n_ot) * DN_ROWS + 16 * wave + fr, H - 1);
        const uint8_t *wrow = p.wd + (int64_t)kid[slot] * p.d_expert_bytes + (int64_t)row * p.d_row_bytes;
#pragma unroll
        for (int b = 0; b < DN_MAXB; ++b) {
            const uint8_t *blk = wrow + 84 * min(b, nb - 1);
            C4[b] = *(const u32x4 *)(blk + 20 + 16 * fc);
            S4[b] = *(const uint32_t *)(blk + 4 + 4 * fc);
            D4[b] = *(const uint32_t *)blk;
        }
    };
    const uint16_t *arow = (fr & 1) ? hl : hh;                      // this lane's A row (rows 0, 1 used)
    auto unit = [&](int uu, const u32x4 (&C4)[DN_MAXB], const uint32_t (&S4)[DN_MAXB], const uint32_t (&D4)[DN_MAXB]) {
        const int slot = uu / n_ot, ot = uu % n_ot;
        const uint16_t *sa_row = arow + slot * nb * 256;
        const float *sx = xm + slot * nb * 16;
        float acc = 0.f, accm = 0.f;
        // every block consumes its registers; blocks past nb (re-reads of the
        // last block) read in-range LDS and add zero
#pragma unroll
        for (int bl = 0; bl < DN_MAXB; ++bl) {
            const int b = min(bl, nb - 1);
            // lane (fr, fc) owns K positions [64 fc, 64 fc + 64) of block b, i.e.
            // sub-blocks 4fc..4fc+3 and code bytes 16fc..16fc+15
            const uint32_t cw[4] = {C4[bl].x, C4[bl].y, C4[bl].z, C4[bl].w};
            const uint32_t scw = S4[bl];
            // all LDS reads of the block (A rows, 16 table entries) go out before its MFMAs
            bf16x8 a[8];
            act_block<true>(sa_row, 256 * b + 64 * fc, 8, fr, a);
            u32x4 Bq[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int sc = (scw >> (8 * (m >> 1))) & 15;
                const uint32_t word = cw[m >> 1];
                const int by0 = (word >> (16 * (m & 1))) & 255, by1 = (word >> (16 * (m & 1) + 8)) & 255;
                const uint2 t0 = *(const uint2 *)&tab[4 * (sc * 256 + by0)];
                const uint2 t1 = *(const uint2 *)&tab[4 * (sc * 256 + by1)];
                Bq[m] = u32x4{t0.x, t0.y, t1.x, t1.y};
            }
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 8; ++m) P = mfma16x16x32(a[m], __builtin_bit_cast(bf16x8, Bq[m]), P);
            // min term of this lane's four sub-blocks: sum_j m_j X_j (fp32)
            const f32x4 xv = *(const f32x4 *)&sx[b * 16 + 4 * fc];
            float mt = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) mt += (float)((scw >> (8 * i + 4)) & 15) * xv[i];
            // column fr of D is this lane's own feature, whose d and dmin it read;
            // rows 0 and 1 (h hi and lo) sit in lanes with fc == 0
            const float d = f16_bits_to_f32(D4[bl] & 0xffffu), dmin = f16_bits_to_f32(D4[bl] >> 16);
            acc += bl < nb ? d * (P[0] + P[1]) : 0.f;
            accm += bl < nb ? dmin * mt : 0.f;
        }
        // the four lanes of a feature hold its min term in four parts
        accm += __shfl_xor(accm, 16, 64);
        accm += __shfl_xor(accm, 32, 64);
        const int row = ot * DN_ROWS + 16 * wave + fr;
        if (fc == 0 && row < H) p.O[(int64_t)slot * H + row] = acc - accm;
    };
    // h of the slots this work-group's units use: the gate and up partial sums
    // of the K chunks added in chunk order, then silu(g) * u as two bf16 terms,
    // and the per-16 sums of h for the min term.  Four features per thread and
    // pass; I % 256 == 0 keeps whole waves in or out of a pass (the four lanes
    // of a 16-wide sub-block are adjacent).  The first pass's partials go out
    // before the first unit's weights, so waiting for them waits for nothing
    // else; the code table is built while both are in flight.
    const int I = p.I, s0 = u_begin / n_ot, s1 = (u_end - 1) / n_ot;
    const int nq = (s1 - s0 + 1) * (I / 4);
    const int64_t cstride = (int64_t)2 * p.k * I;                 // one K chunk of part_rt
    f32x4 gv[DN_MAXKC], uv[DN_MAXKC];
    auto h_load = [&](int q) {
        const int slot = s0 + q / (I / 4), f = 4 * (q % (I / 4));
        const float *pg = p.part_rt + (int64_t)2 * slot * I + f;
#pragma unroll
        for (int c = 0; c < DN_MAXKC; ++c) {
            const int64_t o = cstride * min(c, p.nkc - 1);
            gv[c] = *(const f32x4 *)(pg + o);
            uv[c] = *(const f32x4 *)(pg + o + I);
        }
    };
    auto h_form = [&](int q) {
        const int slot = s0 + q / (I / 4), f = 4 * (q % (I / 4));
        f32x4 g = gv[0], uu = uv[0];
#pragma unroll
        for (int c = 1; c < DN_MAXKC; ++c)
            if (c < p.nkc) { g += gv[c]; uu += uv[c]; }
        uint32_t hi[4], lo[4];
        float hs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float h = g[e] / (1.0f + expf(-g[e])) * uu[e];
            split_bf16(h, hi[e], lo[e]);
            hs += h;
        }
        *(uint2 *)&hh[slot * I + f] = uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
        *(uint2 *)&hl[slot * I + f] = uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
        hs += __shfl_xor(hs, 1, 64);
        hs += __shfl_xor(hs, 2, 64);
        if ((lane & 3) == 0) xm[slot * nb * 16 + (f >> 4)] = hs;
    };
    // pass 0 covers quads [0, 512): nq >= I / 4 >= 64, so at least wave 0 is in it
    h_load(min(tid, nq - 1));
    load(u_begin, ca, sa, da);
    for (int i = tid; i < 16 * 256; i += D1_THREADS) {
        const int sc = i >> 8, byte = i & 255;
        uint32_t v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = f32_to_bf16_exact((float)(sc * ((byte >> (2 * t)) & 3)));
        *(uint2 *)&tab[4 * i] = uint2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
    }
    if (tid < nq) h_form(tid);                                     // uniform over each wave
    for (int q0 = D1_THREADS; q0 < nq; q0 += D1_THREADS) {
        const int q = q0 + tid;
        if (q >= nq) break;                                        // uniform over each wave
        h_load(q);
        h_form(q);
    }
    __syncthreads();
    for (int u = u_begin;;) {                                      // unconditional prefetch, as above
        load(min(u + 1, u_end - 1), cb, sb, db);
        unit(u, ca, sa, da);
        if (++u >= u_end) break;
        load(min(u + 1, u_end - 1), ca, sa, da);
        unit(u, cb, sb, db);
        if (++u >= u_end) break;
    }
}

// y = the shared expert's K parts in order, then the routed outputs in top-k order
__global__ __launch_bounds__(64) void dec1_combine_kernel(DecPass p)
{
    // four outputs per lane; every load of a lane is issued before the first
    // sum (indices clamped, the extra terms masked), so the kernel waits for
    // one memory latency rather than one per term
    const int n = 4 * (blockIdx.x * 64 + threadIdx.x);
    if (n >= p.H) return;
    const int KPD = p.Ish / DN_KPART;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < KPD; q0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = *(const f32x4 *)&p.O_sh[(int64_t)min(q0 + i, KPD - 1) * p.H + n];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (q0 + i < KPD) y += v[i];
    }
    for (int j0 = 0; j0 < p.k; j0 += 8) {
        f32x4 v[8];
        float w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = min(j0 + i, p.k - 1);
            v[i] = *(const f32x4 *)&p.O[(int64_t)j * p.H + n];
            w[i] = p.topk_w[j];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (j0 + i < p.k) y += w[i] * v[i];
    }
    *(f32x4 *)&p.y[n] = y;
}

// ============================================================== fused down
// For k <= DF_MAXK slots, I <= 2048 and sh_inter <= 2048, h is formed once
// (dec1_hform) and one launch computes y (dec1_down_fused).  Work-group wg
// owns output rows rows * wg .. + rows - 1 (16 <= rows <= DF_ROWS, chosen so
// that the work-groups cover the CUs once) with 16 waves: wave w takes the
// 16-row half w % 2 of them for top-k slot w / 2 (if < k; output weighted by
// w_j) and the shared expert's K eighth w / 2, so every CU streams bf16
// shared rows while it looks up Q2_K codes.  A wave's shared bytes are
// requested before it computes, its routed blocks one ahead of use.  The
// sixteen wave sums of a row meet in LDS and are added in wave order.
constexpr int DF_ROWS = 32;
constexpr int DF_MAXK = 8;
constexpr int DF_THREADS = 1024;                 // 16 waves: one slot and one shared K eighth each
constexpr int DF_SHS = 2048 / 8 / 32;            // shared K steps per wave (sh_inter <= 2048)
constexpr int DF_ST = DF_MAXK * 2048 / 8 / DF_THREADS;   // staged 8-element chunks of h per thread
constexpr int DF_SX = (DF_MAXK * 8 * 16 + DF_THREADS - 1) / DF_THREADS;  // staged per-16 sums per thread
// Routed Q2_K blocks requested ahead of the one being computed.  Each wave
// keeps few loads in flight: with all of a wave's blocks requested up front
// the waves stall at issue until the loads drain, and the table lookups then
// run after the stream instead of under it.
constexpr int DF_PF = 1;

// Routed h of every slot (chunk partials added in chunk order) and shared h
// (K parts added in order): silu(g) * u as hi + lo bf16 terms, and the
// per-16 sums of routed h for the Q2_K min term.  One feature per thread, so
// that the few bytes spread over many waves (the launch is latency-bound);
// I % 256 == 0 and sh_inter % 512 == 0 keep whole waves on one side.
__global__ __launch_bounds__(256) void dec1_hform_kernel(DecPass p)
{
    const int q = blockIdx.x * 256 + threadIdx.x, lane = threadIdx.x & 63;
    const int I = p.I, nq_rt = p.k * I;
    // staged layer: the shared h was formed by stage 2's shared down units
    if (q >= nq_rt + (p.staged ? 0 : p.Ish)) return;              // uniform over each wave
    float g, uu;
    int slot = 0, f;
    if (q < nq_rt) {
        slot = q / I;
        f = q % I;
        const int64_t cstride = (int64_t)2 * p.k * I;
        const float *pg = p.part_rt + (int64_t)2 * slot * I + f;
        float gv[DN_MAXKC], uv[DN_MAXKC];
#pragma unroll
        for (int c = 0; c < DN_MAXKC; ++c) {
            const int64_t o = cstride * min(c, p.nkc - 1);
            gv[c] = pg[o];
            uv[c] = pg[o + I];
        }
        g = gv[0];
        uu = uv[0];
#pragma unroll
        for (int c = 1; c < DN_MAXKC; ++c)
            if (c < p.nkc) { g += gv[c]; uu += uv[c]; }
    } else {
        f = q - nq_rt;
        float gv[SH_KQ], uv[SH_KQ];
#pragma unroll
        for (int c = 0; c < SH_KQ; ++c) {
            gv[c] = p.part_sh[(int64_t)(2 * c) * p.Ish + f];
            uv[c] = p.part_sh[(int64_t)(2 * c + 1) * p.Ish + f];
        }
        g = gv[0];
        uu = uv[0];
#pragma unroll
        for (int c = 1; c < SH_KQ; ++c) { g += gv[c]; uu += uv[c]; }
    }
    const float h = g / (1.0f + expf(-g)) * uu;
    uint32_t hi, lo;
    split_bf16(h, hi, lo);
    if (q < nq_rt) {
        p.h_hi[(int64_t)slot * p.hstride + f] = (uint16_t)hi;
        p.h_lo[(int64_t)slot * p.hstride + f] = (uint16_t)lo;
        float hs = h;
        hs += __shfl_xor(hs, 1, 64);
        hs += __shfl_xor(hs, 2, 64);
        hs += __shfl_xor(hs, 4, 64);
        hs += __shfl_xor(hs, 8, 64);
        if ((lane & 15) == 0) p.X[((int64_t)slot * p.nbI + (f >> 8)) * 16 + ((f & 255) >> 4)] = hs;
    } else {
        p.sh_hi[f] = (uint16_t)hi;
        p.sh_lo[f] = (uint16_t)lo;
    }
}

// SHP: the staged layer, whose shared down is already done (O_sh parts, added
// to y in part order after the wave sums); otherwise each wave also takes a K
// eighth of the bf16 shared down.
template <bool SHP>
__global__ __launch_bounds__(DF_THREADS) void dec1_down_fused_kernel(DecPass p, int rows)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int kid[64];
    __shared__ float wsum[DF_THREADS / 64][16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4;
    const int nb = p.nbI, I = p.I, k = p.k, Ish = SHP ? 0 : p.Ish;
    uint16_t *tab = (uint16_t *)dsm;                               // [16 sc][256 bytes][4]
    uint16_t *hh = tab + 16 * 256 * 4;                             // [k][I] routed h hi
    uint16_t *hl = hh + k * I;                                     // [k][I] lo
    float *xm = (float *)(hl + k * I);                             // [k][nb][16]
    uint16_t *sh = (uint16_t *)(xm + k * nb * 16);                 // [Ish] shared h hi
    uint16_t *sl = sh + Ish;                                       // [Ish] lo
    if (tid < k) kid[tid] = expert_matrix(p, clamp_expert(p.topk_idx[tid], p.E));
    __syncthreads();                                               // expert ids
    // h (every slot), its per-16 sums and shared h: loaded into registers
    // before any weight byte is requested, so that storing them into LDS
    // waits for these loads only (the load counter retires in order)
    const int nch = k * I / 8, nxm = k * nb * 16, nsc = Ish / 8;
    u32x4 rhh[DF_ST], rhl[DF_ST], rsh, rsl;
    float rxm[DF_SX];
#pragma unroll
    for (int j = 0; j < DF_ST; ++j) {
        const int i = min(tid + DF_THREADS * j, nch - 1), slot = i / (I / 8), c = i % (I / 8);
        rhh[j] = *(const u32x4 *)(p.h_hi + (int64_t)slot * p.hstride + 8 * c);
        rhl[j] = *(const u32x4 *)(p.h_lo + (int64_t)slot * p.hstride + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < DF_SX; ++j) rxm[j] = p.X[min(tid + DF_THREADS * j, nxm - 1)];
    if (Ish > 0) {
        rsh = *(const u32x4 *)(p.sh_hi + 8 * min(tid, nsc - 1));
        rsl = *(const u32x4 *)(p.sh_lo + 8 * min(tid, nsc - 1));
    }
    const int hg = wave & 1, wp = wave >> 1;                       // wp: this wave's slot and shared K eighth
    // lanes past the work-group's rows (or past H) repeat its last row; their
    // sums are not stored
    const int row = min(rows * (int)blockIdx.x + min(16 * hg + fr, rows - 1), p.H - 1);
    // this wave's shared-down bytes up front, its routed blocks DF_PF ahead of
    // use (unconditional loads: a slot past k re-reads slot k - 1, blocks past
    // nb the last block, steps past the eighth its last step; none of those
    // are used)
    const int KQs = Ish / 8, nsh = KQs / 32, kq0 = wp * KQs;
    u32x4 Wsh[DF_SHS];
    if (Ish > 0) {
#pragma unroll
        for (int st = 0; st < DF_SHS; ++st)
            Wsh[st] = *(const u32x4 *)(p.sd + (int64_t)row * Ish + kq0 + 32 * min(st, nsh - 1) + 8 * fc);
    }
    u32x4 C[DN_MAXB];
    uint32_t Sc[DN_MAXB], Dd[DN_MAXB];
    const uint8_t *wrow = p.wd + (int64_t)kid[min(wp, k - 1)] * p.d_expert_bytes + (int64_t)row * p.d_row_bytes;
    auto load_block = [&](int b) {
        const uint8_t *blk = wrow + 84 * min(b, nb - 1);
        C[b] = *(const u32x4 *)(blk + 20 + 16 * fc);
        Sc[b] = *(const uint32_t *)(blk + 4 + 4 * fc);
        Dd[b] = *(const uint32_t *)blk;
    };
#pragma unroll
    for (int b = 0; b < DF_PF; ++b) load_block(b);
    // the code table, then the staged values (indices past the end rewrite
    // the last element with its own value)
    for (int i = tid; i < 16 * 256; i += DF_THREADS) {
        const int sc = i >> 8, byte = i & 255;
        uint32_t v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = f32_to_bf16_exact((float)(sc * ((byte >> (2 * t)) & 3)));
        *(uint2 *)&tab[4 * i] = uint2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
    }
#pragma unroll
    for (int j = 0; j < DF_ST; ++j) {
        const int i = min(tid + DF_THREADS * j, nch - 1);
        *(u32x4 *)&hh[8 * i] = rhh[j];
        *(u32x4 *)&hl[8 * i] = rhl[j];
    }
#pragma unroll
    for (int j = 0; j < DF_SX; ++j) xm[min(tid + DF_THREADS * j, nxm - 1)] = rxm[j];
    if (Ish > 0) {
        *(u32x4 *)&sh[8 * min(tid, nsc - 1)] = rsh;
        *(u32x4 *)&sl[8 * min(tid, nsc - 1)] = rsl;
    }
    __syncthreads();                                               // h, X, shared h, table staged

    float yv = 0.f;                                                // this lane's row (lanes fc == 0)
    if (Ish > 0) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < DF_SHS; ++st) {
            bf16x8 a = act_rows<true>(sh, sl, kq0 + 32 * min(st, nsh - 1) + 8 * fc, fr);
            if (st >= nsh) a = bf16x8{};
            P = mfma16x16x32(a, __builtin_bit_cast(bf16x8, Wsh[st]), P);
        }
        yv = P[0] + P[1];
    }
    if (wp < k) {                                                  // uniform over the wave
        const uint16_t *sa_row = ((fr & 1) ? hl : hh) + wp * I;    // A rows 0, 1: h hi, lo
        const float *sx = xm + wp * nb * 16;
        float acc = 0.f, accm = 0.f;
#pragma unroll
        for (int bl = 0; bl < DN_MAXB; ++bl) {
            if (bl + DF_PF < DN_MAXB) load_block(bl + DF_PF);
            const int b = min(bl, nb - 1);
            const uint32_t cw[4] = {C[bl].x, C[bl].y, C[bl].z, C[bl].w};
            const uint32_t scw = Sc[bl];
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mh = 0; mh < 2; ++mh) {
                bf16x8 a[4];
                u32x4 Bq[4];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const int m = 4 * mh + mm;
                    a[mm] = fr < 2 ? *(const bf16x8 *)&sa_row[256 * b + 64 * fc + 8 * m] : bf16x8{};
                    const int sc = (scw >> (8 * (m >> 1))) & 15;
                    const uint32_t word = cw[m >> 1];
                    const int by0 = (word >> (16 * (m & 1))) & 255, by1 = (word >> (16 * (m & 1) + 8)) & 255;
                    const uint2 t0 = *(const uint2 *)&tab[4 * (sc * 256 + by0)];
                    const uint2 t1 = *(const uint2 *)&tab[4 * (sc * 256 + by1)];
                    Bq[mm] = u32x4{t0.x, t0.y, t1.x, t1.y};
                }
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) P = mfma16x16x32(a[mm], __builtin_bit_cast(bf16x8, Bq[mm]), P);
            }
            const f32x4 xv = *(const f32x4 *)&sx[b * 16 + 4 * fc];
            float mt = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) mt += (float)((scw >> (8 * e + 4)) & 15) * xv[e];
            const float d = f16_bits_to_f32(Dd[bl] & 0xffffu), dmin = f16_bits_to_f32(Dd[bl] >> 16);
            acc += bl < nb ? d * (P[0] + P[1]) : 0.f;
            accm += bl < nb ? dmin * mt : 0.f;
        }
        accm += __shfl_xor(accm, 16, 64);
        accm += __shfl_xor(accm, 32, 64);
        yv += p.topk_w[wp] * (acc - accm);
    }
    if (fc == 0) wsum[wave][fr] = yv;
    __syncthreads();
    if (tid < rows && rows * (int)blockIdx.x + tid < p.H) {
        const int g2 = tid >> 4, r = tid & 15;
        float y = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < DF_THREADS / 128; ++w2) y += wsum[2 * w2 + g2][r];
        if constexpr (SHP) {
            if (p.Ish > 0) y += p.O_sh[rows * blockIdx.x + tid];      // the shared down's row
        }
        p.y[rows * blockIdx.x + tid] = y;
    }
}

// ============================================================== launchers
namespace {

// shared role: x (one or two bf16 terms) and the wave sums; routed role: the
// chunk's table.  One launch, so the larger.
size_t lds_gateup(int H, bool xf32)
{
    const size_t sh = (size_t)(xf32 ? 4 : 2) * H + 2 * 16 * GU_WAVES * sizeof(float);
    const size_t rt = (size_t)32 * DEC_LUT_KB * 256 * sizeof(float);
    return std::max(sh, rt);
}

size_t lds_down(int nbI, int k) { return 16 * 256 * 4 * 2 + (size_t)k * (2 * (size_t)nbI * 256 * 2 + (size_t)nbI * 32 * 2); }

// Resident work-groups per CU for a kernel at a dynamic LDS size; also lifts
// the kernel's dynamic LDS limit to that size.  Kept per device, with the LDS
// size it was computed for.
template <typename K>
int resident(K kernel, size_t lds, DevSlots &cache, int threads = D1_THREADS)
{
    const int slot = device_slot();
    const uint64_t c = cache.get(slot);
    if (c && (c >> 32) == lds) return (int)(c & 0xffffffffu);
    (void)hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1) n = 1;
    cache.set(slot, ((uint64_t)lds << 32) | (uint32_t)n);
    return n;
}

DevSlots occ_gu_bf16{}, occ_gu_f32{}, occ_dn{};

// Split G work-groups between two roles with n_a units of cost c_a and n_b
// units of cost c_b, minimising the larger per-work-group load.
void split_roles(int n_a, double c_a, int n_b, double c_b, int G, int &g_a, int &g_b)
{
    if (n_a == 0 || G < 2) { g_a = 0; g_b = std::max(1, std::min(n_b, G)); return; }
    if (n_b == 0) { g_a = std::min(n_a, G); g_b = 0; return; }
    double best = 1e300;
    g_a = 1;
    for (int a = 1; a < G; ++a) {
        const double la = ((n_a + a - 1) / a) * c_a, lb = ((n_b + (G - a) - 1) / (G - a)) * c_b;
        const double l = std::max(la, lb);
        if (l < best) { best = l; g_a = a; }
    }
    g_b = G - g_a;
    g_a = std::min(g_a, n_a);
    g_b = std::min(g_b, n_b);
}

// Time per byte of a routed unit relative to a bf16 shared-expert unit, as
// measured per work-group on the MI355X: a codebook tile is bound by its LDS
// table reads (one 4-byte read per 8 weights) and its rows' strided bytes, a
// Q2_K unit by its LDS table reads and VALU work.  The role split gives each
// role work in proportion to these costs.
constexpr double CB2_COST = 1.5;
constexpr double Q2K_COST = 2.5;

}  // namespace

bool dec_single_ok(int T, int H, int I, int Ish, int k, int gu_row_bytes, bool x_f32)
{
    return T == 1 && k <= 64 && H % 512 == 0 && H <= 256 * DEC_LUT_KB * DN_MAXKC && (Ish == 0 || Ish % DN_KPART == 0) &&
           I % 256 == 0 && I / 256 <= DN_MAXB && gu_row_bytes == 38 * (H / 256) && H / SH_KQ / 32 <= GU_WAVES * SH_MAXS &&
           lds_gateup(H, x_f32) <= LDS_MAX && lds_down(I / 256, k) <= LDS_MAX;
}

void dec_plan(DecPass &p)
{
    const int ncu = cu_count();
    const size_t lgu = lds_gateup(p.H, p.x_f32);
    const int occ_gu = p.x_f32 ? resident(dec1_gateup_kernel<true>, lgu, occ_gu_f32, GU_THREADS)
                               : resident(dec1_gateup_kernel<false>, lgu, occ_gu_bf16, GU_THREADS);
    const int occ_d = resident(dec1_down_kernel, lds_down(p.nbI, p.k), occ_dn);
    // routed gate/up: work-groups in whole multiples of the K chunk count
    const int n_sh = (p.Ish / 16) * SH_KQ, ntile = p.k * p.I / 128, G = occ_gu * ncu;
    int g_sh = 0, g_rt = 0;
    split_roles(n_sh, 16.0 * (p.H / SH_KQ) * 2 * 2, p.nkc * ntile, CB2_COST * 256.0 * DEC_LUT_KB * 38, G, g_sh, g_rt);
    const int R = std::max(1, std::min(ntile, (g_rt + p.nkc / 2) / p.nkc));
    p.gu_rt_wg = R * p.nkc;
    p.gu_sh_wg = n_sh ? std::max(1, std::min(n_sh, G - p.gu_rt_wg)) : 0;
    const int n_ot = (p.H + DN_ROWS - 1) / DN_ROWS;
    split_roles(n_ot * (p.Ish / DN_KPART), (double)DN_ROWS * DN_KPART * 2, p.k * n_ot,
                Q2K_COST * DN_ROWS * p.d_row_bytes, occ_d * ncu, p.dn_sh_wg, p.dn_rt_wg);
}

hipError_t launch_dec_gateup(const DecPass &p, hipStream_t s)
{
    const int grid = p.gu_sh_wg + p.gu_rt_wg;
    const size_t lds = lds_gateup(p.H, p.x_f32);
    if (p.x_f32) dec1_gateup_kernel<true><<<grid, GU_THREADS, lds, s>>>(p);
    else dec1_gateup_kernel<false><<<grid, GU_THREADS, lds, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_dec_down(const DecPass &p, hipStream_t s)
{
    const int grid = p.dn_sh_wg + p.dn_rt_wg;
    dec1_down_kernel<<<grid, D1_THREADS, lds_down(p.nbI, p.k), s>>>(p);
    return hipGetLastError();
}

hipError_t launch_dec_combine(const DecPass &p, hipStream_t s)
{
    dec1_combine_kernel<<<(p.H / 4 + 63) / 64, 64, 0, s>>>(p);
    return hipGetLastError();
}

bool dec_fused_ok(int k, int I, int Ish)
{
    return k <= DF_MAXK && I <= 256 * DN_MAXB && Ish <= 8 * 32 * DF_SHS && Ish % 256 == 0;
}

size_t lds_dn_fused(int k, int I, int nbI, int Ish)
{
    return 16 * 256 * 4 * 2 + (size_t)k * I * 2 * 2 + (size_t)k * nbI * 16 * 4 + (size_t)Ish * 2 * 2;
}

hipError_t launch_dec_hform(const DecPass &p, hipStream_t s)
{
    const int nq = p.k * p.I + (p.staged ? 0 : p.Ish);
    dec1_hform_kernel<<<(nq + 255) / 256, 256, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_dec_down_fused(const DecPass &p, hipStream_t s)
{
    const size_t lds = lds_dn_fused(p.k, p.I, p.nbI, p.staged ? 0 : p.Ish);
    static DevSlots attr[2];                                       // dynamic LDS limit set, per device
    const void *fn = p.staged ? (const void *)dec1_down_fused_kernel<true> : (const void *)dec1_down_fused_kernel<false>;
    const hipError_t e = lds_limit(fn, attr[p.staged ? 1 : 0], lds);
    if (e != hipSuccess) return e;
    // one work-group per CU where H allows: fewer rows per CU than a fixed
    // 32 when H / 32 work-groups would leave CUs idle
    const int ncu = cu_count();
    const int rows = std::min(DF_ROWS, std::max(16, (p.H + ncu - 1) / ncu));
    if (p.staged) dec1_down_fused_kernel<true><<<(p.H + rows - 1) / rows, DF_THREADS, lds, s>>>(p, rows);
    else dec1_down_fused_kernel<false><<<(p.H + rows - 1) / rows, DF_THREADS, lds, s>>>(p, rows);
    return hipGetLastError();
}

// ------------------------------------------------------------------ staged layer
namespace {

// x (one or two bf16 terms; a spare 8-value slot after it), the wave sums
size_t lds_stage1(int H, bool xf32) { return (size_t)(xf32 ? 4 : 2) * (H + 8) + 2 * 16 * GU_WAVES * sizeof(float); }
size_t lds_stage2() { return (size_t)32 * DEC_LUT_KB * 256 * sizeof(float); }

// experts per lane of the selection: 4 (E <= 256) or 16 (E <= 1024)
bool wide_select(const DecPass &p) { return p.route && p.E > 256; }

// stage 1 with each router item overlapping its wave's first shared rows:
// bf16 x, at most one item per wave, an item's H chunk in one batch of 8 steps
bool stage1_overlapped(const DecPass &p)
{
    return p.route && !p.x_f32 && p.E * p.rnc <= p.s1_wg * GU_WAVES && p.rhc <= 256 * 8;
}

DevSlots occ_s1[3], occ_s2[4];

}  // namespace

void dec_plan_staged(DecPass &p)
{
    const int ncu = cu_count();
    // stage 1: work-groups of 8 shared features (both halves of K each), and
    // router items spread over all of its waves
    const size_t l1 = lds_stage1(p.H, p.x_f32);
    const int occ1 = p.x_f32 ? resident(dec1_gateup_kernel<true, GU_STAGE1, 4>, l1, occ_s1[1], GU_THREADS)
                             : resident(dec1_gateup_kernel<false, GU_STAGE1, 4>, l1, occ_s1[0], GU_THREADS);
    int g1 = std::max(1, (p.Ish + 7) / 8);
    if (p.route) g1 = std::max(g1, std::min(ncu, (p.E * p.rnc + GU_WAVES - 1) / GU_WAVES));
    p.s1_wg = std::min(g1, occ1 * ncu);
    if (stage1_overlapped(p)) (void)resident(dec1_gateup_kernel<false, GU_STAGE1R, 4>, l1, occ_s1[2], GU_THREADS);
    // stage 2: routed gate/up units (one LDS table per work-group) on every
    // work-group, R per K chunk; the shared down rides in their prologue
    const size_t l2 = lds_stage2();
    const int wide = wide_select(p) ? 1 : 0;
    int occ2;
    if (p.x_f32) occ2 = wide ? resident(dec1_gateup_kernel<true, GU_STAGE2, 16>, l2, occ_s2[3], GU_THREADS)
                             : resident(dec1_gateup_kernel<true, GU_STAGE2, 4>, l2, occ_s2[2], GU_THREADS);
    else occ2 = wide ? resident(dec1_gateup_kernel<false, GU_STAGE2, 16>, l2, occ_s2[1], GU_THREADS)
                     : resident(dec1_gateup_kernel<false, GU_STAGE2, 4>, l2, occ_s2[0], GU_THREADS);
    const int ntile = p.k * p.I / 128;
    const int R = std::max(1, std::min(ntile, occ2 * ncu / p.nkc));
    p.s2_wg = R * p.nkc;
    p.staged = 1;
}

hipError_t launch_dec_stage1(const DecPass &p, hipStream_t s)
{
    const size_t lds = lds_stage1(p.H, p.x_f32);
    if (p.x_f32) dec1_gateup_kernel<true, GU_STAGE1, 4><<<p.s1_wg, GU_THREADS, lds, s>>>(p);
    else if (stage1_overlapped(p)) dec1_gateup_kernel<false, GU_STAGE1R, 4><<<p.s1_wg, GU_THREADS, lds, s>>>(p);
    else dec1_gateup_kernel<false, GU_STAGE1, 4><<<p.s1_wg, GU_THREADS, lds, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_dec_stage2(const DecPass &p, hipStream_t s)
{
    const size_t lds = lds_stage2();
    const int grid = p.s2_wg;
    const bool wide = wide_select(p);
    if (p.x_f32) {
        if (wide) dec1_gateup_kernel<true, GU_STAGE2, 16><<<grid, GU_THREADS, lds, s>>>(p);
        else dec1_gateup_kernel<true, GU_STAGE2, 4><<<grid, GU_THREADS, lds, s>>>(p);
    } else {
        if (wide) dec1_gateup_kernel<false, GU_STAGE2, 16><<<grid, GU_THREADS, lds, s>>>(p);
        else dec1_gateup_kernel<false, GU_STAGE2, 4><<<grid, GU_THREADS, lds, s>>>(p);
    }
    return hipGetLastError();
}

}  // namespace moe
