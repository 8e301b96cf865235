// Prefill expert FFN on gfx950: grouped GEMMs over the token rows routed to
// each expert, with the 2-bit (or 4-bit) routed weights dequantized in
// registers on their way into the matrix cores.
//
// Only the routed experts are quantized (gate/up in the 2-bit codebook
// format, down in Q2_K, Q4_K as the wide variant); the shared expert stays
// bf16 ("DwarfStar" README, section on model weights; deep-dive article,
// section 3.4.3).  Prefill is the compute-bound side of the layer, so the
// weights are expanded once per work-group straight into MFMA operands and
// never pass through LDS as bf16.
//
// Tiling.  A tile is up to 96 rows (positions) of one group (expert, or the
// shared expert as group E); a work-group of 8 waves owns one tile and one
// slice of output columns.  Every wave covers all rows of the tile and its own
// 64 GEMM columns (gate/up: 32 gate + the 32 matching up columns; down: 64
// output features), so each weight is dequantized by exactly one lane.  The
// activations of the tile are staged through LDS in half-blocks of 128 K,
// double-buffered; row fragments beyond the tile's valid rows are skipped.
//
// K order.  Within each 256-weight block of a packed format, MFMA step s
// (0..7) gives the lanes of column group fc (0..3) the 8-weight group
// 8*fc + s, so each lane walks 64 consecutive weights of its row across the
// block and reads its packed bytes once per block; the activations are read
// with the same permutation, which leaves every dot product unchanged.  The
// bf16 shared expert keeps the natural order (step s covers K 32s..32s+31),
// where the 4 lanes of a row read 64 contiguous bytes per step.
//
// Dequantization into bf16 operands (the weights are rounded to bf16, RNE):
//   CB2   w = d*s_j*C, C in {-3,-1,1,3}: a 4-value pool {+-d s_j, +-3 d s_j}
//         per lane and sub-block, and per-codeword byte selectors (a 256-entry
//         LDS table) pick each packed pair with one v_perm.
//   Q2_K  w = d*sc_j*q - dmin*m_j, q in 0..3: the same scheme with the pool of
//         the four levels and selectors indexed by the code byte.
//   Q4_K  16 levels: byte -> fp32 convert, one fma and a packed bf16 convert.
// Work-groups are mapped to tiles XCD by XCD, so all column slices of a tile
// (which share its activations) run on the same XCD and its L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "devcache.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int NP_THREADS = 512;
constexpr int NP_MF = NP_BM / 16;                  // row fragments per tile
static_assert(NP_MF == 6 && NP_BM_SH == 80, "the dispatch switches instantiate 1..6 (routed) and 1..5 (shared) row fragments");
constexpr int NP_COPIES = 8;                       // selector-table copies (bank spread)
constexpr int NP_TAB_CB2 = 256 * NP_COPIES * 16;   // bytes
constexpr int NP_TAB_Q2K = 256 * NP_COPIES * 8;

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

// bytes of {hi:lo} picked by the four selector bytes (0..3: lo, 4..7: hi)
__device__ __forceinline__ uint32_t vperm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float ubyte(uint32_t v, int i) { return (float)((v >> (8 * i)) & 0xffu); }

struct NpTile {
    int g, row0, nvalid, Ng, Kg, n0;
    int w;                            // index of the routed group's matrices in w0 / w1
    int part, k0, Kfull;              // shared expert: K part, its first K, full K
    bool sh;
};

// Work-group -> (tile, column slice).  Work-groups are dispatched to the 8
// XCDs round-robin (work-group f to XCD f % 8); a tile's S slices run on one
// XCD back to back.  PAIR: tiles 2m and 2m + 1 of the list (consecutive
// token tiles of one expert, mostly) go to the same XCD, so the second reads
// the expert's weight slices from that XCD's L2 (the grid then covers a
// multiple of 16 tiles); else tile tau goes to XCD tau % 8.  Returns false
// (uniformly) when the work-group has no work.
template <bool PAIR = false>
__device__ __forceinline__ bool np_tile(const FfnPass &p, int S, int wg_cols, int bm, int bm_sh, NpTile &t)
{
    const int f = blockIdx.x, q = f >> 3, j = q / S, x = f & 7;
    const int tau = PAIR ? ((j >> 1) * 8 + x) * 2 + (j & 1) : j * 8 + x, slice = q % S;
    if (tau >= p.sched[0]) return false;
    t.g = p.sched[1 + 2 * tau];
    const int m0 = p.sched[2 + 2 * tau];
    t.sh = t.g >= p.E;                              // shared expert, K part g - E
    const int ks = max(p.sh_parts, 1);
    t.part = t.sh ? t.g - p.E : 0;
    if (t.part >= ks) return false;                 // a part of the other pass
    t.Ng = t.sh ? p.Nsh : p.N;
    t.Kfull = t.sh ? p.Ksh : p.K;
    t.Kg = t.sh ? p.Ksh / ks : p.K;
    t.k0 = t.part * t.Kg;
    t.n0 = slice * wg_cols;
    if (t.n0 >= t.Ng) return false;
    const int Tk = p.T * p.k;
    int pb, pe;
    if (t.sh) { pb = Tk; pe = Tk + p.T; }
    else { pb = min(max(p.offsets[t.g], 0), Tk); pe = min(max(p.offsets[t.g + 1], pb), Tk); }
    t.row0 = pb + m0;
    t.nvalid = min(t.sh ? bm_sh : bm, pe - t.row0);
    t.w = t.sh ? 0 : p.slot ? max(p.slot[t.g], 0) : t.g;
    return t.nvalid > 0;
}

__device__ __forceinline__ int64_t np_act_row(const FfnPass &p, const NpTile &t, int i)
{
    const int pos = t.row0 + i;
    if (!p.act_by_token) return pos;
    if (t.sh) return pos - p.T * p.k;
    const int tok = p.perm[pos] / p.k;
    return min(max(tok, 0), p.T - 1);              // in bounds even for corrupt routing
}

// Selector tables.  CB2: entry idx holds, for each packed pair (C_2i, C_2i+1)
// of codeword idx, the byte selector into the pool {lo: bf16(ds) | bf16(3ds),
// hi: the same with the signs flipped}.  Q2_K: entry `byte` holds the two
// selectors of its four 2-bit codes into the pool {lo: v0 | v1, hi: v2 | v3}.
__device__ __forceinline__ uint32_t cb2_pos(int c)
{
    return (c < 0 ? 4u : 0u) + ((c == 3 || c == -3) ? 2u : 0u);
}

template <int FMT>
__device__ __forceinline__ void np_build_table(const FfnPass &p, uint32_t *tab)
{
    if constexpr (FMT == FMT_CB2) {
        for (int e = threadIdx.x; e < 256 * 4; e += NP_THREADS) {
            const int idx = e >> 2, i = e & 3;
            const uint32_t b0 = cb2_pos(p.codebook[8 * idx + 2 * i]), b1 = cb2_pos(p.codebook[8 * idx + 2 * i + 1]);
            const uint32_t sel = b0 | ((b0 + 1) << 8) | (b1 << 16) | ((b1 + 1) << 24);
#pragma unroll
            for (int c = 0; c < NP_COPIES; ++c) tab[(idx * NP_COPIES + c) * 4 + i] = sel;
        }
    } else if constexpr (FMT == FMT_CB2S) {
        // CB2S: the selectors of grid entry idx into the magnitude pool
        // {lo: bf16(ds) | bf16(3ds), hi: bf16(5ds) | bf16(7ds)}
        const uint8_t *grid = (const uint8_t *)p.codebook;
        for (int e = threadIdx.x; e < 256 * 4; e += NP_THREADS) {
            const int idx = e >> 2, i = e & 3;
            const uint32_t b0 = (uint32_t)(grid[8 * idx + 2 * i] - 1), b1 = (uint32_t)(grid[8 * idx + 2 * i + 1] - 1);
            const uint32_t sel = b0 | ((b0 + 1) << 8) | (b1 << 16) | ((b1 + 1) << 24);
#pragma unroll
            for (int c = 0; c < NP_COPIES; ++c) tab[(idx * NP_COPIES + c) * 4 + i] = sel;
        }
    } else if constexpr (FMT == FMT_Q2K) {
        for (int e = threadIdx.x; e < 256 * 2; e += NP_THREADS) {
            const int byte = e >> 1, i = e & 1;
            const uint32_t q0 = (byte >> (4 * i)) & 3, q1 = (byte >> (4 * i + 2)) & 3;
            const uint32_t sel = (2 * q0) | ((2 * q0 + 1) << 8) | ((2 * q1) << 16) | ((2 * q1 + 1) << 24);
#pragma unroll
            for (int c = 0; c < NP_COPIES; ++c) tab[(byte * NP_COPIES + c) * 2 + i] = sel;
        }
    }
}

// Raw weight bytes of one lane and one column fragment for one half-block
// (MFMA steps 4h..4h+3 of block b).
struct RawCB2 { uint32_t d, sc, ix; };               // d, scale byte pair, 4 indices
struct RawQ2K { uint32_t dd, scw, c0, c1; };         // d|dmin, 4 scale bytes, 16 codes
struct RawQ4K { uint32_t dd, s0, s1, s2; u32x4 c; }; // d|dmin, 12 scale bytes, 32 codes
struct RawQ5K { uint32_t dd, s0, s1, s2; u32x4 c; uint32_t hb; };  // + bit 4 of the 32 codes
struct RawQ6K { uint32_t dd, sc2; u32x4 c; uint2 hb; };            // d, 2 int8 scales, 32 low nibbles, high bits
struct RawBF16 { uint32_t unused; };                 // bf16 streams per MFMA step

template <int FMT> struct RawOf;
template <> struct RawOf<FMT_CB2> { using T = RawCB2; };
template <> struct RawOf<FMT_Q2K> { using T = RawQ2K; };
template <> struct RawOf<FMT_Q4K> { using T = RawQ4K; };
template <> struct RawOf<FMT_Q5K> { using T = RawQ5K; };
template <> struct RawOf<FMT_Q6K> { using T = RawQ6K; };

// the formats staged half a block at a time (one lane: 32 weights of its row)
template <int FMT> constexpr bool half_staged() { return FMT == FMT_Q4K || FMT == FMT_Q5K || FMT == FMT_Q6K; }
template <> struct RawOf<FMT_BF16> { using T = RawBF16; };

__device__ __forceinline__ uint32_t ld_u32_unaligned(const uint8_t *p)
{
    uint32_t v;
    __builtin_memcpy(&v, p, 4);
    return v;
}

// half-block hs = 2 b + h of the row
template <int FMT>
__device__ __forceinline__ void raw_load(const uint8_t *row, int hs, int fc, typename RawOf<FMT>::T &r)
{
    const int b = hs >> 1, h = hs & 1;
    if constexpr (FMT == FMT_CB2) {
        const uint8_t *blk = row + (int64_t)b * 38;
        r.d = ld_u16(blk);
        r.sc = ld_u16(blk + 2 + 2 * (fc >> 1));
        r.ix = ld_u32_unaligned(blk + 6 + 8 * fc + 4 * h);      // 2-byte aligned
    } else if constexpr (FMT == FMT_Q2K) {
        const uint8_t *blk = row + (int64_t)b * 84;
        r.dd = *(const uint32_t *)blk;
        r.scw = *(const uint32_t *)(blk + 4 + 4 * fc);
        const uint2 c = *(const uint2 *)(blk + 20 + 16 * fc + 8 * h);
        r.c0 = c.x;
        r.c1 = c.y;
    } else if constexpr (FMT == FMT_Q4K || FMT == FMT_Q5K) {
        const uint8_t *blk = row + (int64_t)b * (FMT == FMT_Q4K ? 144 : 176);
        r.dd = *(const uint32_t *)blk;
        r.s0 = *(const uint32_t *)(blk + 4);
        r.s1 = *(const uint32_t *)(blk + 8);
        r.s2 = *(const uint32_t *)(blk + 12);
        r.c = *(const u32x4 *)(blk + 16 + 32 * fc + 16 * h);
        if constexpr (FMT == FMT_Q5K) r.hb = *(const uint32_t *)(blk + 144 + 8 * fc + 4 * h);
    } else if constexpr (FMT == FMT_Q6K) {
        // 210-byte blocks start 2-byte aligned: every field is read unaligned
        const uint8_t *blk = row + (int64_t)b * 210;
        r.dd = ld_u16(blk);
        r.sc2 = ld_u16(blk + 2 + 4 * fc + 2 * h);
        __builtin_memcpy(&r.c, blk + 18 + 32 * fc + 16 * h, 16);
        __builtin_memcpy(&r.hb, blk + 146 + 16 * fc + 8 * h, 8);
    }
}

// Per-half-block dequantization state of one lane and fragment.
struct Pool { uint32_t lo[2], hi[2], mv[2]; float mul, off, mul1; };

// DEC (decode): exact integer codes -- CB2 {+-s, +-3s}, Q2_K {0, sc, 2sc, 3sc}
// and the sub-block min m as a separate operand -- whose block scales d
// (and dmin) are applied to each block's fp32 sums.
template <int FMT, bool DEC = false>
__device__ __forceinline__ void pool_prep(const typename RawOf<FMT>::T &r, int h, int fc, Pool &P)
{
    if constexpr (FMT == FMT_CB2) {
        // sub-block 2 fc + h: nibble h of scale byte 2 + fc
        const uint32_t s = (r.sc >> (8 * (fc & 1) + 4 * h)) & 15u;
        const float ds = DEC ? (float)s : f16_bits_to_f32(r.d) * (float)s;   // exact (11 x 4 bits)
        P.lo[0] = pk_bf16(ds, 3.0f * ds);
        P.hi[0] = P.lo[0] ^ 0x80008000u;
    } else if constexpr (FMT == FMT_Q2K) {
        // sub-blocks 4 fc + 2 h + u, u = 0, 1 (each two MFMA steps)
        const float d = f16_bits_to_f32(r.dd & 0xffffu), dmin = f16_bits_to_f32(r.dd >> 16);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t sm = (r.scw >> (8 * (2 * h + u))) & 0xffu;
            const float mul = d * (float)(sm & 15u), off = dmin * (float)(sm >> 4);
            P.lo[u] = pk_bf16(-off, mul - off);
            P.hi[u] = pk_bf16(2.0f * mul - off, 3.0f * mul - off);
        }
    } else if constexpr (FMT == FMT_Q6K) {
        // sub-blocks 4 fc + 2 h + u (u = 0: MFMA steps 0, 1; u = 1: steps 2, 3),
        // signed scales; no min term
        const float s0 = (float)(int8_t)(r.sc2 & 0xffu), s1 = (float)(int8_t)(r.sc2 >> 8);
        const float d = DEC ? 1.0f : f16_bits_to_f32(r.dd & 0xffffu);
        P.mul = d * s0;                             // exact (11 x 7 bits)
        P.mul1 = d * s1;
    } else if constexpr (FMT == FMT_Q4K || FMT == FMT_Q5K) {
        // sub-block 2 fc + h; 6-bit fields sc_0..7, m_0..7 in a 96-bit stream
        const int j = 2 * fc + h;
        const uint64_t lo64 = (uint64_t)r.s0 | ((uint64_t)r.s1 << 32);
        const uint64_t hi64 = (uint64_t)r.s1 | ((uint64_t)r.s2 << 32);
        const int bsc = 6 * j, bm = 6 * (8 + j);
        const uint32_t sc = (uint32_t)(bsc < 32 ? lo64 >> bsc : hi64 >> (bsc - 32)) & 63u;
        const uint32_t m = (uint32_t)(hi64 >> (bm - 32)) & 63u;
        if (DEC) {
            // exact integers: sc (codes enter as sc*q, split in two bf16 terms)
            // and the min operand m
            P.mul = (float)sc;
            P.off = (float)m;
            P.mv[0] = P.mv[1] = pk_bf16((float)m, (float)m);
        } else {
            P.mul = f16_bits_to_f32(r.dd & 0xffffu) * (float)sc;
            P.off = f16_bits_to_f32(r.dd >> 16) * (float)m;
        }
    }
}

// The 8 codes of MFMA step s4 (weights 8 s4 .. 8 s4 + 7 of the lane's half
// block) as exact floats, element 2i and 2i + 1 in v[i][0], v[i][1]; the
// multiplier that applies to them (Q6_K: its sub-block's).
template <int FMT>
__device__ __forceinline__ float step_codes(const typename RawOf<FMT>::T &r, const Pool &P, int s4, float v[4][2])
{
    const uint32_t cw = r.c[s4];
    const uint32_t cl = cw & 0x0f0f0f0fu, ch = (cw >> 4) & 0x0f0f0f0fu;
    if constexpr (FMT == FMT_Q4K) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i][0] = ubyte(cl, i); v[i][1] = ubyte(ch, i); }
        return P.mul;
    } else if constexpr (FMT == FMT_Q5K) {
        // bit 4 of weight 8 s4 + e is bit 8 s4 + e of the half-block's plane
        const uint32_t hb = r.hb >> (8 * s4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i][0] = ubyte(cl, i) + (float)(((hb >> (2 * i)) & 1u) << 4);
            v[i][1] = ubyte(ch, i) + (float)(((hb >> (2 * i + 1)) & 1u) << 4);
        }
        return P.mul;
    } else {
        // Q6_K: u = nibble | (two high bits << 4), q = u - 32; the high bits of
        // weight 8 s4 + e sit at bits 2 e of the half-block's 16-bit group s4
        const uint32_t hw = s4 < 2 ? r.hb.x : r.hb.y;
        const uint32_t hg = hw >> (16 * (s4 & 1));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i][0] = (float)((int)(((cl >> (8 * i)) & 15u) | (((hg >> (4 * i)) & 3u) << 4)) - 32);
            v[i][1] = (float)((int)(((ch >> (8 * i)) & 15u) | (((hg >> (4 * i + 2)) & 3u) << 4)) - 32);
        }
        return s4 < 2 ? P.mul : P.mul1;
    }
}

// Q4_K decode operands of MFMA step s4: sc * q (integers up to 63 * 15 = 945)
// as hi = bf16(sc * q) plus lo = sc * q - hi (an integer of magnitude <= 2),
// both exact, so the two MFMAs sum the exact products.
// Q5_K: sc * q up to 63 * 31 = 1953, Q6_K: |sc * q| up to 128 * 32 = 4096;
// the same split holds (the remainder of rounding an integer of at most 13
// significant bits to bf16 has at most 5, so it is exact in bf16).
template <int FMT>
__device__ __forceinline__ void bfrag_split_dec(const typename RawOf<FMT>::T &r, const Pool &P, int s4, uint32_t hi[4],
                                                uint32_t lo[4])
{
    float q[4][2];
    const float mul = step_codes<FMT>(r, P, s4, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float v0 = mul * q[i][0], v1 = mul * q[i][1];
        hi[i] = pk_bf16(v0, v1);
        lo[i] = pk_bf16(v0 - __uint_as_float(hi[i] << 16), v1 - __uint_as_float(hi[i] & 0xffff0000u));
    }
}

// B fragment (8 bf16 = 4 dwords) of MFMA step s4 of the half-block.
template <int FMT>
__device__ __forceinline__ void bfrag(const typename RawOf<FMT>::T &r, const Pool &P, int s4,
                                      const uint32_t *tab, int copy, uint32_t out[4])
{
    if constexpr (FMT == FMT_CB2) {
        const uint32_t idx = (r.ix >> (8 * s4)) & 0xffu;
        const u32x4 sel = *(const u32x4 *)&tab[(idx * NP_COPIES + copy) * 4];
        out[0] = vperm(P.hi[0], P.lo[0], sel.x);
        out[1] = vperm(P.hi[0], P.lo[0], sel.y);
        out[2] = vperm(P.hi[0], P.lo[0], sel.z);
        out[3] = vperm(P.hi[0], P.lo[0], sel.w);
    } else if constexpr (FMT == FMT_Q2K) {
        const uint32_t cw = s4 < 2 ? r.c0 : r.c1;
        const uint32_t b0 = (cw >> (16 * (s4 & 1))) & 0xffu, b1 = (cw >> (16 * (s4 & 1) + 8)) & 0xffu;
        const uint2 s0 = *(const uint2 *)&tab[(b0 * NP_COPIES + copy) * 2];
        const uint2 s1 = *(const uint2 *)&tab[(b1 * NP_COPIES + copy) * 2];
        const int u = s4 >> 1;
        out[0] = vperm(P.hi[u], P.lo[u], s0.x);
        out[1] = vperm(P.hi[u], P.lo[u], s0.y);
        out[2] = vperm(P.hi[u], P.lo[u], s1.x);
        out[3] = vperm(P.hi[u], P.lo[u], s1.y);
    } else if constexpr (FMT == FMT_Q4K) {
        const uint32_t cw = r.c[s4];
        const uint32_t lo = cw & 0x0f0f0f0fu, hi = (cw >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = pk_bf16(__builtin_fmaf(P.mul, ubyte(lo, i), -P.off), __builtin_fmaf(P.mul, ubyte(hi, i), -P.off));
    } else if constexpr (FMT == FMT_Q5K || FMT == FMT_Q6K) {
        // the exact fp32 value (Q6_K: the product of exact factors, no min
        // term), rounded to bf16
        float q[4][2];
        const float mul = step_codes<FMT>(r, P, s4, q);
        const float off = FMT == FMT_Q5K ? P.off : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = pk_bf16(__builtin_fmaf(mul, q[i][0], -off), __builtin_fmaf(mul, q[i][1], -off));
    }
}

__device__ __forceinline__ float np_silu_mul(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Activation stages: 2 LDS buffers of 96 rows x 128 bf16 (256 B per row,
// 16-B chunks XOR-swizzled by the row so that a column read of 16 rows hits
// all banks).  Logical chunk c of the stage of half-block h of block b holds
// K offsets 64 (c >> 2) + 32 h + 8 (c & 3) (packed formats) or 128 h + 8 c
// (bf16).
constexpr int NP_ABUF = NP_BM * 256;               // bytes per stage
constexpr int NP_NBUF = 2;

template <bool GATEUP, int NMF, bool DEC>
__device__ __forceinline__ void np_epilogue(const FfnPass &p, const NpTile &t, const f32x4 (&acc)[NMF][4])
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4;
    // D lane (fr, fc) holds rows 4 fc + v of column fr
    if (t.sh && p.sh_part_out) {
        // one K part of the shared expert: fp32 partial sums (gate/up: g and
        // u, SwiGLU after all parts are added)
        const int Tk = p.T * p.k;
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = mf * 16 + 4 * fc + v;
                if (i >= t.nvalid) continue;
                const int64_t tt = t.row0 + i - Tk;
#pragma unroll
                for (int nf = 0; nf < 4; ++nf) {
                    int n;
                    int64_t o;
                    if (GATEUP) {
                        n = t.n0 + wave * 32 + (nf & 1) * 16 + fr;
                        o = (((int64_t)t.part * 2 + (nf >> 1)) * p.T + tt) * t.Ng + n;
                    } else {
                        n = t.n0 + wave * 64 + nf * 16 + fr;
                        o = ((int64_t)t.part * p.T + tt) * t.Ng + n;
                    }
                    if (n < t.Ng) p.sh_part_out[o] = acc[mf][nf][v];
                }
            }
        return;
    }
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = mf * 16 + 4 * fc + v;
            if (i >= t.nvalid) continue;
            const int64_t pos = t.row0 + i;
            if (GATEUP) {
#pragma unroll
                for (int nf = 0; nf < 2; ++nf) {
                    const int n = t.n0 + wave * 32 + nf * 16 + fr;
                    if (n < t.Ng) {
                        const float hv = np_silu_mul(acc[mf][nf][v], acc[mf][nf + 2][v]);
                        if (DEC) ((float *)p.out)[pos * p.out_stride + n] = hv;
                        else ((uint16_t *)p.out)[pos * p.out_stride + n] = (uint16_t)(pk_bf16(hv, 0.f) & 0xffffu);
                    }
                }
            } else {
#pragma unroll
                for (int nf = 0; nf < 4; ++nf) {
                    const int n = t.n0 + wave * 64 + nf * 16 + fr;
                    if (n < t.Ng) ((float *)p.out)[pos * p.out_stride + n] = acc[mf][nf][v];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Routed CB2 / Q2_K body.  Weights stream from HBM as small scattered reads
// (each lane reads a few bytes of its own row), so they are prefetched a
// whole block ahead: the bytes of block b + 1 are requested at the start of
// block b, after that half-block's activation loads, and are only needed two
// half-blocks later.  Vector-memory loads complete in order, so the
// activation loads (one half-block ahead, staged through registers into the
// swizzled LDS layout) never force the weight loads issued after them.
struct BlkCB2 { uint32_t d, sc, i0, i1; };            // d, scale byte pair, 8 indices
struct BlkQ2K { uint32_t dd, scw; uint2 c0, c1; };    // d|dmin, 4 scale bytes, 2 x 16 codes
struct BlkCB2S { uint32_t d; u32x4 rec; };            // d, records of sub-blocks 2 fc and 2 fc + 1
template <int FMT> struct BlkOf;
template <> struct BlkOf<FMT_CB2> { using T = BlkCB2; };
template <> struct BlkOf<FMT_Q2K> { using T = BlkQ2K; };
template <> struct BlkOf<FMT_CB2S> { using T = BlkCB2S; };

// the part of block b that half h of the previous block requests (Q2_K
// splits its codes so that only half of them are in flight at a time)
template <int FMT>
__device__ __forceinline__ void blk_load(const uint8_t *row, int b, int h, int fc, typename BlkOf<FMT>::T &r)
{
    if constexpr (FMT == FMT_CB2) {
        if (h == 0) {
            const uint8_t *blk = row + (int64_t)b * 38;
            r.d = ld_u16(blk);
            r.sc = ld_u16(blk + 2 + 2 * (fc >> 1));
            r.i0 = ld_u32_unaligned(blk + 6 + 8 * fc);           // 2-byte aligned
            r.i1 = ld_u32_unaligned(blk + 10 + 8 * fc);
        }
    } else if constexpr (FMT == FMT_CB2S) {
        if (h == 0) {
            // rows are a multiple of 4 bytes long (an even number of 66-byte
            // blocks), so the 16 record bytes at 2 + 16 fc start 4-byte
            // aligned in odd blocks and 2 bytes past a dword in even ones:
            // there they come from five aligned dwords that end at the
            // record's last byte
            const uint8_t *blk = row + (int64_t)b * 66;
            r.d = ld_u16(blk);
            const uint8_t *rec = blk + 2 + 16 * fc;
            if (b & 1) {
                r.rec = *(const u32x4 *)rec;
            } else {
                const uint32_t *a4 = (const uint32_t *)(rec - 2);
                const u32x4 v = *(const u32x4 *)a4;
                const uint32_t w = a4[4];
                r.rec = u32x4{__builtin_amdgcn_alignbit(v.y, v.x, 16), __builtin_amdgcn_alignbit(v.z, v.y, 16),
                              __builtin_amdgcn_alignbit(v.w, v.z, 16), __builtin_amdgcn_alignbit(w, v.w, 16)};
            }
        }
    } else {
        const uint8_t *blk = row + (int64_t)b * 84;
        if (h == 0) {
            r.dd = *(const uint32_t *)blk;
            r.scw = *(const uint32_t *)(blk + 4 + 4 * fc);
            r.c0 = *(const uint2 *)(blk + 20 + 16 * fc);
        } else {
            r.c1 = *(const uint2 *)(blk + 28 + 16 * fc);
        }
    }
}

template <int FMT, bool DEC>
__device__ __forceinline__ void blk_pool(const typename BlkOf<FMT>::T &r, int h, int fc, Pool &P)
{
    if constexpr (FMT == FMT_CB2) {
        RawCB2 x{r.d, r.sc, 0u};
        pool_prep<FMT_CB2, DEC>(x, h, fc, P);
    } else if constexpr (FMT == FMT_CB2S) {
        // sub-block 2 fc + h: s in the top nibble of its record's sign word;
        // DEC keeps the block scale d out (applied to the block's sums)
        const uint32_t s = (h == 0 ? r.rec.y : r.rec.w) >> 28;
        const float ds = DEC ? (float)s : f16_bits_to_f32(r.d) * (float)s;   // exact (11 x 4 bits)
        P.lo[0] = pk_bf16(ds, 3.0f * ds);
        P.hi[0] = pk_bf16(5.0f * ds, 7.0f * ds);
    } else {
        RawQ2K x{r.dd, r.scw, 0u, 0u};
        pool_prep<FMT_Q2K, DEC>(x, h, fc, P);
    }
}

template <bool DEC>
__device__ __forceinline__ void q2k_pool(const BlkQ2K &r, int h, int u, Pool &P)
{
    const uint32_t sm = (r.scw >> (8 * (2 * h + u))) & 0xffu;
    if (DEC) {
        const float sc = (float)(sm & 15u), m = (float)(sm >> 4);
        P.lo[u] = pk_bf16(0.0f, sc);
        P.hi[u] = pk_bf16(2.0f * sc, 3.0f * sc);
        P.mv[u] = pk_bf16(m, m);
    } else {
        const float d = f16_bits_to_f32(r.dd & 0xffffu), dmin = f16_bits_to_f32(r.dd >> 16);
        const float mul = d * (float)(sm & 15u), off = dmin * (float)(sm >> 4);
        P.lo[u] = pk_bf16(-off, mul - off);
        P.hi[u] = pk_bf16(2.0f * mul - off, 3.0f * mul - off);
    }
}

template <int FMT>
__device__ __forceinline__ void blk_frag(const typename BlkOf<FMT>::T &r, const Pool &P, int h, int s4,
                                         const uint32_t *tab, int copy, uint32_t out[4])
{
    if constexpr (FMT == FMT_CB2) {
        RawCB2 x{r.d, r.sc, h == 0 ? r.i0 : r.i1};
        bfrag<FMT_CB2>(x, P, s4, tab, copy, out);
    } else if constexpr (FMT == FMT_CB2S) {
        // magnitudes through the selector table, then the group's signs: 7
        // stored flags and their parity as the eighth, XORed into the bf16
        // sign bits (element 2i in bit 15, 2i + 1 in bit 31 of dword i)
        const uint32_t iw = h == 0 ? r.rec.x : r.rec.z, sw = h == 0 ? r.rec.y : r.rec.w;
        const uint32_t idx = (iw >> (8 * s4)) & 0xffu;
        const uint32_t n7 = (sw >> (7 * s4)) & 0x7fu;
        const uint32_t neg = n7 | ((uint32_t)(__builtin_popcount(n7) & 1) << 7);
        const u32x4 sel = *(const u32x4 *)&tab[(idx * NP_COPIES + copy) * 4];
        const uint32_t sv[4] = {sel.x, sel.y, sel.z, sel.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t m = ((neg >> (2 * i)) & 1u) << 15 | ((neg >> (2 * i + 1)) & 1u) << 31;
            out[i] = vperm(P.hi[0], P.lo[0], sv[i]) ^ m;
        }
    } else {
        const uint2 c = h == 0 ? r.c0 : r.c1;
        RawQ2K x{r.dd, r.scw, c.x, c.y};
        bfrag<FMT_Q2K>(x, P, s4, tab, copy, out);
    }
}

// DEC: decode precision (exact weights, see pool_prep); TWO: fp32 activations
// entered as two bf16 terms (hi, lo), each its own MFMA.
template <int FMT, bool GATEUP, int NMF, bool DEC, bool TWO>
__device__ __forceinline__ void np_body_r(const FfnPass &p, const NpTile &t, uint8_t *As, const uint32_t *tab)
{
    // per-format weight staging: CB2/Q2_K whole blocks (two sets), Q4_K
    // half-blocks (two sets), bf16 one MFMA step at a time (a ring of four)
    constexpr bool BLK = FMT == FMT_CB2 || FMT == FMT_Q2K || FMT == FMT_CB2S;
    using Blk = typename BlkOf<BLK ? FMT : FMT_CB2>::T;
    // bf16 weights use the natural K order (MFMA step s of a block covers K
    // 32 s .. 32 s + 31, lane group fc its 8-wide slice), so the 4 lanes of a
    // row read 64 contiguous bytes per step; the packed formats use the
    // block-walking order (one small read per block)
    constexpr bool NAT = FMT == FMT_BF16;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4, copy = lane & (NP_COPIES - 1);
    const int nb = t.Kg >> 8;                        // even (checked on the host)
    const int nhs = 2 * nb;

    // ---- activation staging: 16-B chunk ci = tid + 512 j of a stage is row
    // ci >> 4, physical chunk ci & 15 (logical chunk (ci & 15) ^ (row & 15));
    // fp32 activations are split into hi and lo bf16 stages
    constexpr int NCH = (DEC ? NP_BM_DEC : NP_BM) * 16 / NP_THREADS;
    uint32_t aoffs[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int ci = tid + NP_THREADS * j, r = ci >> 4;
        const int c = (ci & 15) ^ (r & 15);
        aoffs[j] = (uint32_t)(np_act_row(p, t, min(r, t.nvalid - 1)) * p.act_stride) + t.k0 +
                   (NAT ? 8 * c : 64 * (c >> 2) + 8 * (c & 3));
    }
    u32x4 av[NCH], avl[TWO ? NCH : 1];
    auto a_load = [&](int hs) {
        const uint32_t koff = 256 * (hs >> 1) + (NAT ? 128 : 32) * (hs & 1);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if constexpr (TWO) {
                const f32x4 *src = (const f32x4 *)((const float *)p.act + (aoffs[j] + koff));
                const f32x4 v0 = src[0], v1 = src[1];
                const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = pk_bf16(v[2 * e], v[2 * e + 1]);
                    lo[e] = pk_bf16(v[2 * e] - __uint_as_float(hi[e] << 16),
                                    v[2 * e + 1] - __uint_as_float(hi[e] & 0xffff0000u));
                }
                av[j] = u32x4{hi[0], hi[1], hi[2], hi[3]};
                avl[j] = u32x4{lo[0], lo[1], lo[2], lo[3]};
            } else {
                av[j] = *(const u32x4 *)((const uint16_t *)p.act + (aoffs[j] + koff));
            }
        }
    };
    auto a_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            *(u32x4 *)(As + buf * NP_ABUF + (tid + NP_THREADS * j) * 16) = av[j];
            if constexpr (TWO) *(u32x4 *)(As + (NP_NBUF + buf) * NP_ABUF + (tid + NP_THREADS * j) * 16) = avl[j];
        }
    };
    int aoff[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) aoff[s4] = fr * 256 + (((NAT ? 4 * s4 + fc : 4 * fc + s4) ^ fr) << 4);

    // ---- weight rows of this lane's four column fragments (byte offsets
    // inside one expert's matrix, < 2^32, from per-tile bases)
    const uint8_t *wb0, *wb1;
    if (FMT == FMT_BF16) { wb0 = (const uint8_t *)p.s0; wb1 = (const uint8_t *)p.s1; }
    else {
        wb0 = p.w0 + (int64_t)t.w * p.w_expert_bytes;
        wb1 = GATEUP ? p.w1 + (int64_t)t.w * p.w_expert_bytes : wb0;
    }
    uint32_t wo[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
        int col;
        if (GATEUP) col = t.n0 + wave * 32 + (nf & 1) * 16 + fr;
        else col = t.n0 + wave * 64 + nf * 16 + fr;
        col = min(col, t.Ng - 1);
        wo[nf] = FMT == FMT_BF16 ? (uint32_t)col * (uint32_t)t.Kfull * 2u + 2u * t.k0 + 16u * fc
                                 : (uint32_t)col * (uint32_t)p.w_row_bytes;
    }
    auto wrow = [&](int nf) -> const uint8_t * { return (GATEUP && nf >= 2 ? wb1 : wb0) + wo[nf]; };

    // DEC with packed weights: each block's sums (P1: codes, P2: Q2_K min
    // operand) are scaled by the block's d (and dmin) into acc
    constexpr bool PBLK = DEC && FMT != FMT_BF16;
    constexpr bool HALF = half_staged<FMT>();
    using RawH = typename RawOf<HALF ? FMT : FMT_Q4K>::T;
    constexpr bool PMIN = DEC && (FMT == FMT_Q2K || FMT == FMT_Q4K || FMT == FMT_Q5K);
    constexpr bool Q4D = DEC && HALF;               // two exact B terms per step
    f32x4 acc[NMF][4], P1[PBLK ? NMF : 1][4], P2[PMIN ? NMF : 1][4];
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mf = 0; mf < (PBLK ? NMF : 1); ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) P1[mf][nf] = P2[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

    Blk blk[2][4];                                   // CB2/Q2_K: [block parity][fragment]
    RawH r4[2][4];                                   // Q4_K/Q5_K/Q6_K: [half parity][fragment]
    u32x4 bw[4][4];                                  // bf16: [step mod 4][fragment]
    const int nks = 8 * nb;
    auto bw_load = [&](int ks) {
        const int kc = min(ks, nks - 1);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) bw[ks & 3][nf] = *(const u32x4 *)(wrow(nf) + 512 * (kc >> 3) + 64 * (kc & 7));
    };
    a_load(0);
    if constexpr (BLK) {
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
            blk_load<FMT>(wrow(nf), 0, 0, fc, blk[0][nf]);
            blk_load<FMT>(wrow(nf), 0, 1, fc, blk[0][nf]);
        }
    } else if constexpr (HALF) {
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) raw_load<FMT>(wrow(nf), 0, fc, r4[0][nf]);
    } else {
        bw_load(0);
        bw_load(1);
        bw_load(2);
    }
    a_store(0);
    __syncthreads();

    for (int b = 0; b < nb; b += 2) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int bb = b + q;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int hs = 2 * bb + h;
                a_load(min(hs + 1, nhs - 1));
                // keep the weight loads behind this step's activation loads
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (BLK) {
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf) blk_load<FMT>(wrow(nf), min(bb + 1, nb - 1), h, fc, blk[q ^ 1][nf]);
                } else if constexpr (HALF) {
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf) raw_load<FMT>(wrow(nf), min(hs + 1, nhs - 1), fc, r4[h ^ 1][nf]);
                }
                Pool P[4];
                if constexpr (FMT == FMT_CB2 || FMT == FMT_CB2S) {
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf) blk_pool<FMT, DEC>(blk[q][nf], h, fc, P[nf]);
                } else if constexpr (HALF) {
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf) pool_prep<FMT, DEC>(r4[h][nf], h, fc, P[nf]);
                }
                const uint8_t *ab = As + h * NP_ABUF, *abl = As + (NP_NBUF + h) * NP_ABUF;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    if constexpr (FMT == FMT_Q2K) {
                        // the pool of sub-block 4 fc + 2 h + s4 / 2, built when first needed
                        if ((s4 & 1) == 0) {
#pragma unroll
                            for (int nf = 0; nf < 4; ++nf) q2k_pool<DEC>(blk[q][nf], h, s4 >> 1, P[nf]);
                        }
                    }
                    bf16x8 a[NMF], al[TWO ? NMF : 1];
#pragma unroll
                    for (int mf = 0; mf < NMF; ++mf) {
                        a[mf] = *(const bf16x8 *)(ab + aoff[s4] + mf * 4096);
                        if constexpr (TWO) al[mf] = *(const bf16x8 *)(abl + aoff[s4] + mf * 4096);
                    }
                    bf16x8 bq[4], bql[Q4D ? 4 : 1];
                    if constexpr (Q4D) {
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf) {
                            uint32_t oh[4], ol[4];
                            bfrag_split_dec<FMT>(r4[h][nf], P[nf], s4, oh, ol);
                            bq[nf] = __builtin_bit_cast(bf16x8, u32x4{oh[0], oh[1], oh[2], oh[3]});
                            bql[nf] = __builtin_bit_cast(bf16x8, u32x4{ol[0], ol[1], ol[2], ol[3]});
                        }
                    } else if constexpr (FMT == FMT_BF16) {
                        const int ks = 8 * bb + 4 * h + s4;
                        bw_load(ks + 3);                             // ring slot (s4 + 3) & 3
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf) bq[nf] = __builtin_bit_cast(bf16x8, bw[s4][nf]);
                    } else {
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf) {
                            uint32_t o[4];
                            if constexpr (BLK) blk_frag<FMT>(blk[q][nf], P[nf], h, s4, tab, copy, o);
                            else bfrag<HALF ? FMT : FMT_Q4K>(r4[h][nf], P[nf], s4, tab, copy, o);
                            bq[nf] = __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
                        }
                    }
#pragma unroll
                    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf) {
                            if constexpr (PBLK) {
                                P1[mf][nf] = mfma16x16x32(a[mf], bq[nf], P1[mf][nf]);
                                if constexpr (TWO) P1[mf][nf] = mfma16x16x32(al[mf], bq[nf], P1[mf][nf]);
                                if constexpr (Q4D) {
                                    P1[mf][nf] = mfma16x16x32(a[mf], bql[nf], P1[mf][nf]);
                                    if constexpr (TWO) P1[mf][nf] = mfma16x16x32(al[mf], bql[nf], P1[mf][nf]);
                                }
                                if constexpr (PMIN) {
                                    const uint32_t mv = P[nf].mv[s4 >> 1];
                                    const bf16x8 bm = __builtin_bit_cast(bf16x8, u32x4{mv, mv, mv, mv});
                                    P2[mf][nf] = mfma16x16x32(a[mf], bm, P2[mf][nf]);
                                    if constexpr (TWO) P2[mf][nf] = mfma16x16x32(al[mf], bm, P2[mf][nf]);
                                }
                            } else {
                                acc[mf][nf] = mfma16x16x32(a[mf], bq[nf], acc[mf][nf]);
                                if constexpr (TWO) acc[mf][nf] = mfma16x16x32(al[mf], bq[nf], acc[mf][nf]);
                            }
                        }
                }
                if constexpr (PBLK) {
                    if (h == 1) {
                        // block bb done: its sums times this lane's column scales
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf) {
                            float d, dmin = 0.f;
                            if constexpr (FMT == FMT_CB2 || FMT == FMT_CB2S) d = f16_bits_to_f32(blk[q][nf].d);
                            else if constexpr (FMT == FMT_Q6K) d = f16_bits_to_f32(r4[h][nf].dd & 0xffffu);
                            else if constexpr (HALF) {
                                d = f16_bits_to_f32(r4[h][nf].dd & 0xffffu);
                                dmin = f16_bits_to_f32(r4[h][nf].dd >> 16);
                            } else {
                                d = f16_bits_to_f32(blk[q][nf].dd & 0xffffu);
                                dmin = f16_bits_to_f32(blk[q][nf].dd >> 16);
                            }
#pragma unroll
                            for (int mf = 0; mf < NMF; ++mf) {
                                acc[mf][nf] += d * P1[mf][nf];
                                if constexpr (PMIN) acc[mf][nf] -= dmin * P2[mf][nf];
                                P1[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
                                if constexpr (PMIN) P2[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
                            }
                        }
                    }
                }
                a_store(h ^ 1);
                __syncthreads();
            }
        }
    }
    np_epilogue<GATEUP, NMF, DEC>(p, t, acc);
}

// ---------------------------------------------------------------------------
// Prefill down-projection body for routed tiles on v_mfma_f32_32x32x16_bf16
// (measured on the MI355X at almost twice the rate of the 16x16x32 shape).
// Same tiling as above (96-row tiles, 8 waves, 64 GEMM columns per wave) with
// 32-row fragments and two 32-column fragments per wave.  Lane l supplies
// column (or row, for A) l % 32 and K group kg = l / 32 of each MFMA step
// (K = 16).  K order inside a 256-weight block: step 8h + s (half h,
// s = 0..7) gives lane half kg the 8-weight group 16 kg + 8 h + s, so each
// lane walks 128 consecutive weights of its row per block; the activations
// are staged with the same permutation.  D element v of lane l is row
// 8 (v / 4) + 4 kg + v % 4, column l % 32.  Gate/up passes and the shared
// expert stay on the 16x16x32 bodies, which measured faster for them.
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// one lane's bytes of one Q2_K block or one Q4_K half-block
struct C32Q2K { uint32_t dd; uint2 sc; uint2 c[4]; };
struct C32Q4K { uint32_t dd, s0, s1, s2; u32x4 c[2]; };
template <int FMT> struct C32Of { using T = C32Q2K; };
template <> struct C32Of<FMT_Q4K> { using T = C32Q4K; };

// Q2_K: b is the block, h the half of this lane's 32 code bytes.  Q4_K: b is
// the half-block (h unused).
template <int FMT>
__device__ __forceinline__ void c32_load(const uint8_t *row, int b, int h, int kg, typename C32Of<FMT>::T &r)
{
    if constexpr (FMT == FMT_Q2K) {
        const uint8_t *blk = row + (int64_t)b * 84;
        if (h == 0) {
            r.dd = *(const uint32_t *)blk;
            r.sc = *(const uint2 *)(blk + 4 + 8 * kg);
            r.c[0] = *(const uint2 *)(blk + 20 + 32 * kg);
            r.c[1] = *(const uint2 *)(blk + 28 + 32 * kg);
        } else {
            r.c[2] = *(const uint2 *)(blk + 36 + 32 * kg);
            r.c[3] = *(const uint2 *)(blk + 44 + 32 * kg);
        }
    } else {
        const uint8_t *blk = row + (int64_t)(b >> 1) * 144;
        r.dd = *(const uint32_t *)blk;
        r.s0 = *(const uint32_t *)(blk + 4);
        r.s1 = *(const uint32_t *)(blk + 8);
        r.s2 = *(const uint32_t *)(blk + 12);
        r.c[0] = *(const u32x4 *)(blk + 16 + 64 * kg + 32 * (b & 1));
        r.c[1] = *(const u32x4 *)(blk + 32 + 64 * kg + 32 * (b & 1));
    }
}

template <int FMT, int NMF>
__device__ __forceinline__ void np_body32_down(const FfnPass &p, const NpTile &t, uint8_t *As, const uint32_t *tab)
{
    static_assert(FMT == FMT_Q2K || FMT == FMT_Q4K, "routed down formats");
    using Raw = typename C32Of<FMT>::T;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c32 = lane & 31, kg = lane >> 5, copy = lane & (NP_COPIES - 1);
    const int nb = t.Kg >> 8;                        // even (checked on the host)
    const int nhs = 2 * nb;

    // ---- activation staging: 16-byte chunks, swizzled as in the 16x16x32
    // body; chunk c of a row holds K 128 (c / 8) + 8 (c % 8) .. + 7 of the
    // half-block, so a lane half reads its 8 consecutive groups
    constexpr int NCH = NP_BM * 16 / NP_THREADS;
    uint32_t aoffs[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int ci = tid + NP_THREADS * j, r = ci >> 4;
        const int c = (ci & 15) ^ (r & 15);
        aoffs[j] = (uint32_t)(np_act_row(p, t, min(r, t.nvalid - 1)) * p.act_stride) + t.k0 + 128 * (c >> 3) + 8 * (c & 7);
    }
    u32x4 av[NCH];
    auto a_load = [&](int hs) {
        const uint32_t koff = 256 * (hs >> 1) + 64 * (hs & 1);
#pragma unroll
        for (int j = 0; j < NCH; ++j) av[j] = *(const u32x4 *)((const uint16_t *)p.act + (aoffs[j] + koff));
    };
    auto a_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) *(u32x4 *)(As + buf * NP_ABUF + (tid + NP_THREADS * j) * 16) = av[j];
    };
    int aoff[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) aoff[s8] = c32 * 256 + (((8 * kg + s8) ^ (c32 & 15)) << 4);

    // ---- weight rows of this lane's two column fragments
    const uint8_t *wb = p.w0 + (int64_t)t.w * p.w_expert_bytes;
    const uint8_t *wr[2];
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) {
        const int col = min(t.n0 + wave * 64 + cf * 32 + c32, t.Ng - 1);
        wr[cf] = wb + (int64_t)col * p.w_row_bytes;
    }

    f32x16 acc[NMF][2];
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int cf = 0; cf < 2; ++cf)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mf][cf][v] = 0.f;

    Raw blk[2][2];                                   // Q2_K: [block parity][fragment]; Q4_K: [half parity][fragment]
    a_load(0);
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) {
        c32_load<FMT>(wr[cf], 0, 0, kg, blk[0][cf]);
        if constexpr (FMT == FMT_Q2K) c32_load<FMT>(wr[cf], 0, 1, kg, blk[0][cf]);
    }
    a_store(0);
    __syncthreads();

    for (int b = 0; b < nb; b += 2) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int bb = b + q;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int hs = 2 * bb + h;
                a_load(min(hs + 1, nhs - 1));
                // keep the weight loads behind this step's activation loads
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int cf = 0; cf < 2; ++cf) {
                    if constexpr (FMT == FMT_Q2K) c32_load<FMT>(wr[cf], min(bb + 1, nb - 1), h, kg, blk[q ^ 1][cf]);
                    else c32_load<FMT>(wr[cf], min(hs + 1, nhs - 1), 0, kg, blk[h ^ 1][cf]);
                }
                // per-fragment dequantization state of this half: Q2_K four
                // sub-block pools, Q4_K two (mul, off) pairs
                uint32_t plo[2][4], phi[2][4];
                float pmul[2][2], poff[2][2];
#pragma unroll
                for (int cf = 0; cf < 2; ++cf) {
                    if constexpr (FMT == FMT_Q2K) {
                        const float d = f16_bits_to_f32(blk[q][cf].dd & 0xffffu), dmin = f16_bits_to_f32(blk[q][cf].dd >> 16);
                        const uint32_t sw = h ? blk[q][cf].sc.y : blk[q][cf].sc.x;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const uint32_t sm = (sw >> (8 * u)) & 0xffu;
                            const float mul = d * (float)(sm & 15u), off = dmin * (float)(sm >> 4);
                            plo[cf][u] = pk_bf16(-off, mul - off);
                            phi[cf][u] = pk_bf16(2.0f * mul - off, 3.0f * mul - off);
                        }
                    } else {
                        const Raw &r = blk[h][cf];
                        const uint64_t lo64 = (uint64_t)r.s0 | ((uint64_t)r.s1 << 32);
                        const uint64_t hi64 = (uint64_t)r.s1 | ((uint64_t)r.s2 << 32);
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int j = 4 * kg + 2 * h + u;
                            const int bsc = 6 * j, bm = 6 * (8 + j);
                            const uint32_t sc = (uint32_t)(bsc < 32 ? lo64 >> bsc : hi64 >> (bsc - 32)) & 63u;
                            const uint32_t m = (uint32_t)(hi64 >> (bm - 32)) & 63u;
                            pmul[cf][u] = f16_bits_to_f32(r.dd & 0xffffu) * (float)sc;
                            poff[cf][u] = f16_bits_to_f32(r.dd >> 16) * (float)m;
                        }
                    }
                }
                const uint8_t *ab = As + h * NP_ABUF;
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) {
                    bf16x8 a[NMF];
#pragma unroll
                    for (int mf = 0; mf < NMF; ++mf) a[mf] = *(const bf16x8 *)(ab + aoff[s8] + mf * 8192);
                    bf16x8 bq[2];
#pragma unroll
                    for (int cf = 0; cf < 2; ++cf) {
                        uint32_t o[4];
                        if constexpr (FMT == FMT_Q2K) {
                            // code bytes 16 h + 2 s8, +1 of this lane's 32; sub-block 4 h + s8 / 2
                            const uint2 cw2 = blk[q][cf].c[2 * h + (s8 >> 2)];
                            const uint32_t cw = (s8 & 2) ? cw2.y : cw2.x;
                            const uint32_t b0 = (cw >> (16 * (s8 & 1))) & 0xffu, b1 = (cw >> (16 * (s8 & 1) + 8)) & 0xffu;
                            const uint2 t0 = *(const uint2 *)&tab[(b0 * NP_COPIES + copy) * 2];
                            const uint2 t1 = *(const uint2 *)&tab[(b1 * NP_COPIES + copy) * 2];
                            const int u = s8 >> 1;
                            o[0] = vperm(phi[cf][u], plo[cf][u], t0.x);
                            o[1] = vperm(phi[cf][u], plo[cf][u], t0.y);
                            o[2] = vperm(phi[cf][u], plo[cf][u], t1.x);
                            o[3] = vperm(phi[cf][u], plo[cf][u], t1.y);
                        } else {
                            // code dword s8 of this half's eight; sub-block 2 h + s8 / 4
                            const uint32_t cw = blk[h][cf].c[s8 >> 2][s8 & 3];
                            const uint32_t lo = cw & 0x0f0f0f0fu, hi = (cw >> 4) & 0x0f0f0f0fu;
                            const int u = s8 >> 2;
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                o[i] = pk_bf16(__builtin_fmaf(pmul[cf][u], ubyte(lo, i), -poff[cf][u]),
                                               __builtin_fmaf(pmul[cf][u], ubyte(hi, i), -poff[cf][u]));
                        }
                        bq[cf] = __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
                    }
#pragma unroll
                    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
                        for (int cf = 0; cf < 2; ++cf) acc[mf][cf] = mfma32x32x16(a[mf], bq[cf], acc[mf][cf]);
                }
                a_store(h ^ 1);
                __syncthreads();
            }
        }
    }

    // ---- epilogue: fp32 rows of the down output
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = mf * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
            if (i >= t.nvalid) continue;
            const int64_t pos = t.row0 + i;
#pragma unroll
            for (int cf = 0; cf < 2; ++cf) {
                const int n = t.n0 + wave * 64 + cf * 32 + c32;
                if (n < t.Ng) ((float *)p.out)[pos * p.out_stride + n] = acc[mf][cf][v];
            }
        }
}

template <int FMT>
__device__ __forceinline__ void np_dispatch32_down(const FfnPass &p, const NpTile &t, uint8_t *As, const uint32_t *tab)
{
    const int nmf = (t.nvalid + 31) >> 5;
    if (nmf <= 1) np_body32_down<FMT, 1>(p, t, As, tab);
    else if (nmf == 2) np_body32_down<FMT, 2>(p, t, As, tab);
    else np_body32_down<FMT, 3>(p, t, As, tab);
}

// decode tiles are at most 32 rows (2 fragments), prefill tiles 96 (6)
template <int FMT, bool GATEUP, bool DEC, bool TWO, int MAXF>
__device__ __forceinline__ void np_dispatch(const FfnPass &p, const NpTile &t, uint8_t *As, const uint32_t *tab)
{
    const int nmf = (t.nvalid + 15) >> 4;
    if constexpr (MAXF <= 2) {
        if (nmf <= 1) np_body_r<FMT, GATEUP, 1, DEC, TWO>(p, t, As, tab);
        else np_body_r<FMT, GATEUP, 2, DEC, TWO>(p, t, As, tab);
    } else {
        switch (nmf) {
        case 1: np_body_r<FMT, GATEUP, 1, DEC, TWO>(p, t, As, tab); break;
        case 2: np_body_r<FMT, GATEUP, 2, DEC, TWO>(p, t, As, tab); break;
        case 3: np_body_r<FMT, GATEUP, 3, DEC, TWO>(p, t, As, tab); break;
        case 4: np_body_r<FMT, GATEUP, 4, DEC, TWO>(p, t, As, tab); break;
        case 5: np_body_r<FMT, GATEUP, 5, DEC, TWO>(p, t, As, tab); break;
        default:
            if constexpr (MAXF >= 6) np_body_r<FMT, GATEUP, 6, DEC, TWO>(p, t, As, tab);
            else np_body_r<FMT, GATEUP, 5, DEC, TWO>(p, t, As, tab);
            break;
        }
    }
}

template <int FMT> constexpr int np_tab_bytes()
{
    return FMT == FMT_CB2 || FMT == FMT_CB2S ? NP_TAB_CB2 : FMT == FMT_Q2K ? NP_TAB_Q2K : 0;
}
template <int FMT, bool TWO> constexpr int np_lds_bytes() { return (TWO ? 2 : 1) * NP_NBUF * NP_ABUF + np_tab_bytes<FMT>(); }

// prefill deals tile pairs to one XCD (np_tile's PAIR): measured 1-2% faster
// for CB2/Q2_K and Q4_K layers at 2048- and 8192-token prefills, 2.5% slower
// for CB2S gate/up
template <int FMT, bool DEC> constexpr bool np_paired() { return !DEC && FMT != FMT_CB2S; }

template <int FMT, bool GATEUP, bool DEC, bool TWO>
__global__ __launch_bounds__(NP_THREADS) void np_kernel(FfnPass p, int S)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t np_smem[];
    NpTile t;
    if (!np_tile<np_paired<FMT, DEC>()>(p, S, GATEUP ? 256 : 512, DEC ? NP_BM_DEC : NP_BM, DEC ? NP_BM_DEC : NP_BM_SH, t))
        return;
    uint8_t *As = np_smem;
    uint32_t *tab = (uint32_t *)(np_smem + (TWO ? 2 : 1) * NP_NBUF * NP_ABUF);
    if (t.sh) {
        // shared-expert tiles are at most 80 rows: the bf16 weight ring and
        // six row fragments would not fit the register budget together
        np_dispatch<FMT_BF16, GATEUP, DEC, TWO, DEC ? 2 : 5>(p, t, As, tab);
    } else if (p.skip_routed) {
        return;
    } else {
        np_build_table<FMT>(p, tab);
        __syncthreads();
        if constexpr (!DEC && !TWO && !GATEUP && (FMT == FMT_Q2K || FMT == FMT_Q4K))
            np_dispatch32_down<FMT>(p, t, As, tab);
        else
            np_dispatch<FMT, GATEUP, DEC, TWO, DEC ? 2 : 6>(p, t, As, tab);
    }
}

template <int FMT, bool GATEUP, bool DEC, bool TWO>
hipError_t np_launch(const FfnPass &p, hipStream_t s)
{
    constexpr int lds = np_lds_bytes<FMT, TWO>();
    static DevSlots attr{};                        // dynamic LDS limit set, per device
    const hipError_t e = lds_limit((const void *)np_kernel<FMT, GATEUP, DEC, TWO>, attr, lds);
    if (e != hipSuccess) return e;
    const int wg_cols = GATEUP ? 256 : 512;
    const int S = (std::max(p.N, p.Nsh) + wg_cols - 1) / wg_cols;
    // every tile the schedule can hold, the shared expert's K parts included
    // (both passes read one schedule built with the larger part count)
    const int ks = std::max(p.sched_parts, 1);
    const int tiles = DEC ? ffn_max_tiles(p.T, p.k, p.E, p.Nsh > 0, NP_BM_DEC, NP_BM_DEC, ks)
                          : ffn_max_tiles(p.T, p.k, p.E, p.Nsh > 0, NP_BM, NP_BM_SH, ks);
    const int64_t grid = np_paired<FMT, DEC>() ? (int64_t)((tiles + 15) / 16) * 16 * S : (int64_t)((tiles + 7) / 8) * 8 * S;
    np_kernel<FMT, GATEUP, DEC, TWO><<<dim3((unsigned)grid), NP_THREADS, lds, s>>>(p, S);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Batched decode of the routed tiles.  At decode sizes (a few tokens per
// expert) the grouped GEMM above is bound by how it reads weights: every lane
// owns one weight row and reads a few bytes of it per step, so each load
// instruction touches as many cache lines as rows.  Here a work-group stages
// its weight rows through LDS one block pair (512 K) at a time with
// lane-consecutive dword loads (a wave's load covers a few rows' contiguous
// bytes), two pairs in flight in registers while the pair before them is
// computed from LDS.  The arithmetic is the decode precision of the grouped
// GEMM: exact integer codes as bf16 MFMA operands, the fp32 sums of each
// block scaled by its d (and the Q2_K min term by dmin), fp32 activations as
// hi + lo bf16 terms.  The K order is the natural one (step s of a block
// covers K 32s..32s+31, lane group fc its 8-wide slice), so the activations
// are staged in plain row order, 16-byte pieces XOR-swizzled by the row.
//
// Tiles are BD_BM = 16 positions of one expert (one MFMA row fragment).
// gate/up (CB2): 4 waves, each 16 h-features x {gate, up}: 128 weight rows;
// a block's bytes start 2 bytes past a dword in odd blocks, so each block is
// staged as the 10-dword window from the dword at or below it.
// down (Q2_K): 8 waves, each 32 output features: 256 weight rows, 42 dwords
// per row and pair (84-byte blocks are dword aligned).
constexpr int BD_COPIES = 4;                       // selector-table copies

template <int FMT_> struct Bd {
    static constexpr int FMT = FMT_;
    static constexpr bool GATEUP = FMT != FMT_Q2K;             // CB2 / CB2S gate/up, Q2_K down
    static constexpr int WAVES = GATEUP ? 4 : 8;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS = 32 * WAVES;                       // weight rows per work-group
    static constexpr int COLS = GATEUP ? 16 * WAVES : 32 * WAVES; // GEMM output columns per work-group
    // dwords per row and block pair: CB2 two 10-dword block windows, CB2S the
    // 33 dwords of the pair and one pad dword (never read), Q2_K 42
    static constexpr int WDW = FMT == FMT_CB2 ? 20 : FMT == FMT_CB2S ? 34 : 42;
    static constexpr int PB = FMT == FMT_CB2 ? 76 : FMT == FMT_CB2S ? 132 : 168;   // bytes of a block pair in a row
    static constexpr int COPIES = FMT == FMT_CB2S ? 2 : BD_COPIES;                // lookup-table copies
    static constexpr int WLD = ROWS * WDW / THREADS;              // weight dwords one thread loads per pair
    static constexpr int WSLOT = ROWS * WDW * 4;                  // bytes of one weight stage
    static constexpr int APLANE = BD_BM * 1024;                   // 16 rows x 512 K bf16
    static constexpr int APT = BD_BM * 64 / THREADS;              // 8-K pieces one thread loads per pair
    static constexpr int TAB = 256 * COPIES * (GATEUP ? 16 : 8);
    // Q2_K min term: per slot, the 16-K sub-block sums of the staged rows as
    // MFMA A operands, [block][hi, lo][16 rows][16 bf16]
    static constexpr int XSLOT = GATEUP ? 0 : 2 * 2 * BD_BM * 32;
    static_assert(ROWS * WDW % THREADS == 0 && BD_BM * 64 % THREADS == 0, "whole loads per thread");
};

template <int FMT, bool TWO> constexpr int bd_lds_bytes()
{
    return 2 * Bd<FMT>::WSLOT + 2 * (TWO ? 2 : 1) * Bd<FMT>::APLANE + Bd<FMT>::TAB + 2 * Bd<FMT>::XSLOT;
}

// the selector tables of np_build_table, COPIES copies, built by THREADS threads
template <int FMT, int THREADS, int COPIES>
__device__ __forceinline__ void bd_build_table(const FfnPass &p, uint32_t *tab)
{
    if constexpr (FMT == FMT_CB2 || FMT == FMT_CB2S) {
        for (int e = threadIdx.x; e < 256 * 4; e += THREADS) {
            const int idx = e >> 2, i = e & 3;
            uint32_t b0, b1;
            if constexpr (FMT == FMT_CB2) {
                b0 = cb2_pos(p.codebook[8 * idx + 2 * i]);
                b1 = cb2_pos(p.codebook[8 * idx + 2 * i + 1]);
            } else {
                // grid magnitudes {1, 3, 5, 7} -> bytes 0, 2, 4, 6 of the pool
                const uint8_t *grid = (const uint8_t *)p.codebook;
                b0 = (uint32_t)(grid[8 * idx + 2 * i] - 1);
                b1 = (uint32_t)(grid[8 * idx + 2 * i + 1] - 1);
            }
            const uint32_t sel = b0 | ((b0 + 1) << 8) | (b1 << 16) | ((b1 + 1) << 24);
#pragma unroll
            for (int c = 0; c < COPIES; ++c) tab[(idx * COPIES + c) * 4 + i] = sel;
        }
    } else {
        for (int e = threadIdx.x; e < 256 * 2; e += THREADS) {
            const int byte = e >> 1, i = e & 1;
            const uint32_t q0 = (byte >> (4 * i)) & 3, q1 = (byte >> (4 * i + 2)) & 3;
            const uint32_t sel = (2 * q0) | ((2 * q0 + 1) << 8) | ((2 * q1) << 16) | ((2 * q1 + 1) << 24);
#pragma unroll
            for (int c = 0; c < COPIES; ++c) tab[(byte * COPIES + c) * 2 + i] = sel;
        }
    }
}

template <int FMT_, bool TWO>
__global__ __launch_bounds__(Bd<FMT_>::THREADS) void bd_kernel(FfnPass p, int S)
{
    using C = Bd<FMT_>;
    constexpr int FMT = C::FMT, THREADS = C::THREADS, NF = 2, COPIES = C::COPIES;
    constexpr bool GATEUP = C::GATEUP;
    extern __shared__ __attribute__((aligned(16))) uint8_t bd_smem[];
    NpTile t;
    if (!np_tile(p, S, C::COLS, BD_BM, NP_BM_DEC, t)) return;
    if (t.sh) return;                                        // the grouped GEMM takes the shared tiles
    uint8_t *Ws = bd_smem;                                   // [2][ROWS][WDW] dwords
    uint8_t *As = bd_smem + 2 * C::WSLOT;                    // [2][hi, lo][16][1024 B]
    uint32_t *tab = (uint32_t *)(As + 2 * (TWO ? 2 : 1) * C::APLANE);
    uint8_t *Xs = (uint8_t *)tab + C::TAB;                   // [2][XSLOT] (Q2_K)
    bd_build_table<FMT, THREADS, COPIES>(p, tab);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int fr = lane & 15, fc = lane >> 4, copy = lane & (COPIES - 1);
    const int npair = t.Kg >> 9;                             // >= 1 (K % 512 == 0, checked on the host)

    // ---- this thread's load slots: weight dwords (row, dword) and activation pieces (row, 8-K piece)
    const uint8_t *wb0 = p.w0 + (int64_t)t.w * p.w_expert_bytes;
    const uint8_t *wb1 = GATEUP ? p.w1 + (int64_t)t.w * p.w_expert_bytes : wb0;
    uint32_t woff[C::WLD];                                   // byte offset inside the expert's matrix
    const uint8_t *wsrc[C::WLD];
#pragma unroll
    for (int j = 0; j < C::WLD; ++j) {
        const int q = tid + THREADS * j, r = q / C::WDW, i = q - r * C::WDW;
        int col, off;
        const uint8_t *base;
        if (GATEUP) {
            col = t.n0 + (r & 63);
            base = r < 64 ? wb0 : wb1;
            if constexpr (FMT == FMT_CB2) off = i < 10 ? 4 * i : 36 + 4 * (i - 10);   // two 40-byte block windows
            else off = i < 33 ? 4 * i : 0;                   // CB2S: the pair, pad dword re-reads dword 0
        } else {
            col = t.n0 + r;
            base = wb0;
            off = 4 * i;
        }
        col = min(col, t.Ng - 1);
        wsrc[j] = base;
        woff[j] = (uint32_t)col * (uint32_t)p.w_row_bytes + (uint32_t)off;
    }
    constexpr int PB = C::PB;
    int64_t arow[C::APT];
    int akp[C::APT], ar[C::APT];
#pragma unroll
    for (int j = 0; j < C::APT; ++j) {
        const int q = tid + THREADS * j;
        ar[j] = q >> 6;
        akp[j] = q & 63;
        arow[j] = np_act_row(p, t, min(ar[j], t.nvalid - 1)) * p.act_stride + t.k0;
    }
    // ---- prefetch registers: two sets (two objects, never indexed at run time)
    struct Regs {
        uint32_t w[C::WLD];
        u32x4 a0[C::APT], a1[TWO ? C::APT : 1];
    };
    Regs R0, R1;
    auto load_pair = [&](int pr, Regs &R) {
#pragma unroll
        for (int j = 0; j < C::WLD; ++j) R.w[j] = *(const uint32_t *)(wsrc[j] + woff[j] + (uint32_t)(PB * pr));
#pragma unroll
        for (int j = 0; j < C::APT; ++j) {
            const int64_t e = arow[j] + 512 * pr + 8 * akp[j];
            if constexpr (TWO) {
                const u32x4 *src = (const u32x4 *)((const float *)p.act + e);
                R.a0[j] = src[0];
                R.a1[j] = src[1];
            } else {
                R.a0[j] = *(const u32x4 *)((const uint16_t *)p.act + e);
            }
        }
    };
    auto store_pair = [&](const Regs &R, int slot) {
        uint32_t *w = (uint32_t *)(Ws + slot * C::WSLOT);
#pragma unroll
        for (int j = 0; j < C::WLD; ++j) w[tid + THREADS * j] = R.w[j];
        uint8_t *a = As + slot * (TWO ? 2 : 1) * C::APLANE;
#pragma unroll
        for (int j = 0; j < C::APT; ++j) {
            const int o = ar[j] * 1024 + ((akp[j] ^ (ar[j] & 15)) << 4);
            if constexpr (TWO) {
                const u32x4 v0 = R.a0[j], v1 = R.a1[j];
                const float v[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z),
                                    __uint_as_float(v0.w), __uint_as_float(v1.x), __uint_as_float(v1.y),
                                    __uint_as_float(v1.z), __uint_as_float(v1.w)};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = pk_bf16(v[2 * e], v[2 * e + 1]);
                    lo[e] = pk_bf16(v[2 * e] - __uint_as_float(hi[e] << 16),
                                    v[2 * e + 1] - __uint_as_float(hi[e] & 0xffff0000u));
                }
                *(u32x4 *)(a + o) = u32x4{hi[0], hi[1], hi[2], hi[3]};
                *(u32x4 *)(a + C::APLANE + o) = u32x4{lo[0], lo[1], lo[2], lo[3]};
                if constexpr (FMT == FMT_Q2K) {
                    // sub-block sum over K 16 u .. 16 u + 15 of the pair (u = akp / 2):
                    // this piece's 8 values, then the neighbouring lane's (akp ^ 1)
                    float s8 = v[0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) s8 += v[e];
                    const float other = __shfl_xor(s8, 1);
                    if ((akp[j] & 1) == 0) {
                        const float xs = s8 + other;
                        const uint32_t xh = pk_bf16(xs, 0.f) & 0xffffu;
                        const uint32_t xl = pk_bf16(xs - __uint_as_float(xh << 16), 0.f) & 0xffffu;
                        const int u = akp[j] >> 1, blkx = u >> 4, jj = u & 15;
                        uint16_t *xp = (uint16_t *)(Xs + slot * C::XSLOT + blkx * 2 * BD_BM * 32);
                        xp[ar[j] * 16 + jj] = (uint16_t)xh;
                        xp[BD_BM * 16 + ar[j] * 16 + jj] = (uint16_t)xl;
                    }
                }
            } else {
                *(u32x4 *)(a + o) = R.a0[j];
            }
        }
    };

    f32x4 acc[NF], P1[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) acc[nf] = P1[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
    // LDS row of fragment nf of this lane: gate/up nf 0 = gate, 1 = up of feature
    // n0 + 16 wave + fr; down: feature n0 + 32 wave + 16 nf + fr
    int wrow[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) wrow[nf] = GATEUP ? nf * 64 + 16 * wave + fr : 32 * wave + 16 * nf + fr;
    // K order inside a block, as in the grouped GEMM: MFMA step s4 of half h
    // gives lane group fc the 8 weights 64 fc + 32 h + 8 s4 .. + 7, so a lane's
    // half-block is one sub-block (CB2) or two (Q2_K) and its pool is built once
    // per half; the activation pieces are read in the same order.
    auto compute_pair = [&](int slot) {
        const uint32_t *w = (const uint32_t *)(Ws + slot * C::WSLOT);
        const uint8_t *a = As + slot * (TWO ? 2 : 1) * C::APLANE;
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            // this lane's fields of block b2 for each fragment
            uint32_t d16[NF], f0[NF], f1[NF], f2[NF], f3[NF] = {}, f4[NF] = {}, f5[NF] = {};
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
                if constexpr (FMT == FMT_CB2S) {
                    // block b2 at byte 66 b2 of the pair; record j = 2 fc + h at byte 2 + 8 j:
                    // 4 grid indices, then the sign/scale word
                    const uint16_t *bp = (const uint16_t *)(w + wrow[nf] * C::WDW) + 33 * b2;
                    d16[nf] = bp[0];
                    f1[nf] = (uint32_t)bp[1 + 8 * fc] | ((uint32_t)bp[2 + 8 * fc] << 16);
                    f2[nf] = (uint32_t)bp[3 + 8 * fc] | ((uint32_t)bp[4 + 8 * fc] << 16);
                    f3[nf] = (uint32_t)bp[5 + 8 * fc] | ((uint32_t)bp[6 + 8 * fc] << 16);
                    f4[nf] = (uint32_t)bp[7 + 8 * fc] | ((uint32_t)bp[8 + 8 * fc] << 16);
                    f0[nf] = 0;
                } else if constexpr (FMT == FMT_CB2) {
                    // odd blocks start 2 bytes into their 10-dword window
                    const uint16_t *bp = (const uint16_t *)(w + wrow[nf] * C::WDW + 10 * b2) + b2;
                    d16[nf] = bp[0];
                    f0[nf] = bp[1 + (fc >> 1)];                              // scale byte pair
                    f1[nf] = (uint32_t)bp[3 + 4 * fc] | ((uint32_t)bp[4 + 4 * fc] << 16);   // indices, half 0
                    f2[nf] = (uint32_t)bp[5 + 4 * fc] | ((uint32_t)bp[6 + 4 * fc] << 16);   // indices, half 1
                } else {
                    const uint32_t *bp = w + wrow[nf] * C::WDW + 21 * b2;
                    d16[nf] = bp[0];                                         // d | dmin << 16
                    f0[nf] = bp[1 + fc];                                     // sc|m of sub-blocks 4 fc ..
                    f1[nf] = bp[5 + 4 * fc];                                 // codes, half 0
                    f2[nf] = bp[6 + 4 * fc];
                    f3[nf] = bp[7 + 4 * fc];                                 // codes, half 1
                    f4[nf] = bp[8 + 4 * fc];
                    // m of sub-blocks 8 fc .. 8 fc + 7 (lanes fc < 2) for the min term
                    f5[nf] = bp[1 + 2 * (fc & 1)];
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t plo[NF][2], phi[NF][2];
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    if constexpr (FMT == FMT_CB2S) {
                        // magnitudes {s, 3s, 5s, 7s} (exact); signs per weight below
                        const float sj = (float)((h ? f4[nf] : f2[nf]) >> 28);
                        plo[nf][0] = pk_bf16(sj, 3.0f * sj);
                        phi[nf][0] = pk_bf16(5.0f * sj, 7.0f * sj);
                    } else if constexpr (FMT == FMT_CB2) {
                        const float sj = (float)((f0[nf] >> (8 * (fc & 1) + 4 * h)) & 15u);
                        plo[nf][0] = pk_bf16(sj, 3.0f * sj);
                        phi[nf][0] = plo[nf][0] ^ 0x80008000u;
                    } else {
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const float sc = (float)((f0[nf] >> (8 * (2 * h + u))) & 15u);
                            plo[nf][u] = pk_bf16(0.0f, sc);
                            phi[nf][u] = pk_bf16(2.0f * sc, 3.0f * sc);
                        }
                    }
                }
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int o = (32 * b2 + 8 * fc + 4 * h + s4) ^ fr;
                    const bf16x8 ah = *(const bf16x8 *)(a + fr * 1024 + (o << 4));
                    bf16x8 al;
                    if constexpr (TWO) al = *(const bf16x8 *)(a + C::APLANE + fr * 1024 + (o << 4));
#pragma unroll
                    for (int nf = 0; nf < NF; ++nf) {
                        uint32_t ob[4];
                        if constexpr (FMT == FMT_CB2S) {
                            const uint32_t idx = ((h ? f3[nf] : f1[nf]) >> (8 * s4)) & 0xffu;
                            const u32x4 sel = *(const u32x4 *)&tab[(idx * COPIES + copy) * 4];
                            const uint32_t n7 = ((h ? f4[nf] : f2[nf]) >> (7 * s4)) & 0x7fu;
                            const uint32_t neg = n7 | ((uint32_t)(__builtin_popcount(n7) & 1) << 7);
                            const uint32_t sv[4] = {sel.x, sel.y, sel.z, sel.w};
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                ob[i] = vperm(phi[nf][0], plo[nf][0], sv[i]) ^
                                        (((neg >> (2 * i)) & 1u) << 15 | ((neg >> (2 * i + 1)) & 1u) << 31);
                        } else if constexpr (FMT == FMT_CB2) {
                            const uint32_t idx = ((h ? f2[nf] : f1[nf]) >> (8 * s4)) & 0xffu;
                            const u32x4 sel = *(const u32x4 *)&tab[(idx * COPIES + copy) * 4];
                            ob[0] = vperm(phi[nf][0], plo[nf][0], sel.x);
                            ob[1] = vperm(phi[nf][0], plo[nf][0], sel.y);
                            ob[2] = vperm(phi[nf][0], plo[nf][0], sel.z);
                            ob[3] = vperm(phi[nf][0], plo[nf][0], sel.w);
                        } else {
                            const uint32_t cw = h ? (s4 < 2 ? f3[nf] : f4[nf]) : (s4 < 2 ? f1[nf] : f2[nf]);
                            const uint32_t b0 = (cw >> (16 * (s4 & 1))) & 0xffu, b1 = (cw >> (16 * (s4 & 1) + 8)) & 0xffu;
                            const uint2 s0 = *(const uint2 *)&tab[(b0 * COPIES + copy) * 2];
                            const uint2 s1 = *(const uint2 *)&tab[(b1 * COPIES + copy) * 2];
                            const int u = s4 >> 1;
                            ob[0] = vperm(phi[nf][u], plo[nf][u], s0.x);
                            ob[1] = vperm(phi[nf][u], plo[nf][u], s0.y);
                            ob[2] = vperm(phi[nf][u], plo[nf][u], s1.x);
                            ob[3] = vperm(phi[nf][u], plo[nf][u], s1.y);
                        }
                        const bf16x8 bq = __builtin_bit_cast(bf16x8, u32x4{ob[0], ob[1], ob[2], ob[3]});
                        P1[nf] = mfma16x16x32(ah, bq, P1[nf]);
                        if constexpr (TWO) P1[nf] = mfma16x16x32(al, bq, P1[nf]);
                    }
                }
            }
            if constexpr (FMT != FMT_Q2K) {
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    acc[nf] += f16_bits_to_f32(d16[nf]) * P1[nf];
                    P1[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else {
                // the block's code sums times d; the min term: the 16 sub-block
                // sums of the activation rows (K 0..15; lanes fc >= 2 supply the
                // zero K 16..31) against the sub-blocks' m (exact integers),
                // times dmin
                const uint16_t *xp = (const uint16_t *)(Xs + slot * C::XSLOT + b2 * 2 * BD_BM * 32);
                u32x4 xh{0u, 0u, 0u, 0u}, xl{0u, 0u, 0u, 0u};
                if (fc < 2) {
                    xh = *(const u32x4 *)(xp + fr * 16 + 8 * fc);
                    xl = *(const u32x4 *)(xp + BD_BM * 16 + fr * 16 + 8 * fc);
                }
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    acc[nf] += f16_bits_to_f32(d16[nf] & 0xffffu) * P1[nf];
                    P1[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
                    // m of sub-blocks 8 fc .. 8 fc + 7: high nibbles of bytes 4 + 8 fc ..
                    // (dwords 1 + 2 fc and 2 + 2 fc; the second read here)
                    const uint32_t m0 = f5[nf];
                    const uint32_t m1 = w[wrow[nf] * C::WDW + 21 * b2 + 2 + 2 * (fc & 1)];
                    uint32_t mb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wv = e < 2 ? m0 : m1;
                        const int sh = 16 * (e & 1);
                        mb[e] = fc < 2 ? pk_bf16((float)((wv >> (sh + 4)) & 15u), (float)((wv >> (sh + 12)) & 15u)) : 0u;
                    }
                    const bf16x8 bm = __builtin_bit_cast(bf16x8, u32x4{mb[0], mb[1], mb[2], mb[3]});
                    f32x4 Pm = mfma16x16x32(__builtin_bit_cast(bf16x8, xh), bm, f32x4{0.f, 0.f, 0.f, 0.f});
                    Pm = mfma16x16x32(__builtin_bit_cast(bf16x8, xl), bm, Pm);
                    acc[nf] -= f16_bits_to_f32(d16[nf] >> 16) * Pm;
                }
            }
        }
    };

    // ---- pipeline: pairs p + 1 and p + 2 in flight while pair p is computed
    load_pair(0, R0);
    if (npair > 1) load_pair(1, R1);
    store_pair(R0, 0);
    if (npair > 2) load_pair(2, R0);
    __syncthreads();
    // pair pr sits in LDS slot pr % 2; `nx` holds pair pr + 1 (requested two
    // steps back) and takes pair pr + 3
    auto iter = [&](int pr, Regs &nx) {
        compute_pair(pr & 1);
        if (pr + 1 < npair) store_pair(nx, (pr + 1) & 1);
        if (pr + 3 < npair) load_pair(pr + 3, nx);
        __syncthreads();
    };
    for (int pr = 0; pr < npair; pr += 2) {
        iter(pr, R1);
        if (pr + 1 < npair) iter(pr + 1, R0);
    }

    // ---- epilogue: D lane (fr, fc) holds rows 4 fc + v of column fr
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int i = 4 * fc + v;
        if (i >= t.nvalid) continue;
        const int64_t pos = t.row0 + i;
        if (GATEUP) {
            const int n = t.n0 + 16 * wave + fr;
            if (n < t.Ng) ((float *)p.out)[pos * p.out_stride + n] = np_silu_mul(acc[0][v], acc[1][v]);
        } else {
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
                const int n = t.n0 + 32 * wave + 16 * nf + fr;
                if (n < t.Ng) ((float *)p.out)[pos * p.out_stride + n] = acc[nf][v];
            }
        }
    }
}

template <int FMT, bool TWO>
hipError_t bd_launch(const FfnPass &p, hipStream_t s)
{
    constexpr int lds = bd_lds_bytes<FMT, TWO>();
    static DevSlots attr{};
    const hipError_t e = lds_limit((const void *)bd_kernel<FMT, TWO>, attr, lds);
    if (e != hipSuccess) return e;
    const int S = (p.N + Bd<FMT>::COLS - 1) / Bd<FMT>::COLS;
    const int tiles = ffn_max_tiles(p.T, p.k, p.E, p.Nsh > 0, BD_BM, NP_BM_DEC, std::max(p.sched_parts, 1));
    const int64_t grid = (int64_t)((tiles + 7) / 8) * 8 * S;
    bd_kernel<FMT, TWO><<<dim3((unsigned)grid), Bd<FMT>::THREADS, lds, s>>>(p, S);
    return hipGetLastError();
}

}  // namespace

bool np_prefill_ok(const FfnPass &p)
{
    if (p.act_f32) return false;
    if (p.K % (2 * QK) || p.K < 2 * QK) return false;   // routed blocks run in pairs
    if (p.Nsh > 0 && (p.Ksh % (2 * QK) || p.Ksh < 2 * QK)) return false;
    return true;
}

hipError_t launch_np_prefill(const FfnPass &p, bool gateup, hipStream_t s)
{
    if (!np_prefill_ok(p) || p.out_f32 == gateup) return hipErrorInvalidValue;
    if (gateup) {
        switch (p.fmt) {
        case FMT_CB2: return np_launch<FMT_CB2, true, false, false>(p, s);
        case FMT_CB2S: return np_launch<FMT_CB2S, true, false, false>(p, s);
        case FMT_Q2K: return np_launch<FMT_Q2K, true, false, false>(p, s);
        case FMT_Q4K: return np_launch<FMT_Q4K, true, false, false>(p, s);
        case FMT_Q5K: return np_launch<FMT_Q5K, true, false, false>(p, s);
        }
    } else {
        switch (p.fmt) {
        case FMT_Q2K: return np_launch<FMT_Q2K, false, false, false>(p, s);
        case FMT_Q4K: return np_launch<FMT_Q4K, false, false, false>(p, s);
        case FMT_Q5K: return np_launch<FMT_Q5K, false, false, false>(p, s);
        case FMT_Q6K: return np_launch<FMT_Q6K, false, false, false>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

bool np_decode_ok(const FfnPass &p)
{
    if (p.K % (2 * QK) || p.K < 2 * QK) return false;
    if (p.Nsh > 0 && (p.Ksh % (2 * QK) || p.Ksh < 2 * QK)) return false;
    return p.out_f32 && (p.fmt == FMT_CB2 || p.fmt == FMT_Q2K || p.fmt == FMT_Q4K || p.fmt == FMT_Q5K ||
                         p.fmt == FMT_Q6K || p.fmt == FMT_CB2S);
}

// gate/up takes x (bf16, or fp32 as two bf16 terms); down takes the fp32 h
template <int FMT>
hipError_t np_decode_fmt(const FfnPass &p, bool gateup, hipStream_t s)
{
    if (gateup) {
        if constexpr (FMT == FMT_Q6K) return hipErrorInvalidValue;
        else {
            if (p.act_f32) return np_launch<FMT, true, true, true>(p, s);
            return np_launch<FMT, true, true, false>(p, s);
        }
    }
    if constexpr (FMT == FMT_CB2 || FMT == FMT_CB2S) return hipErrorInvalidValue;
    else {
        if (!p.act_f32) return hipErrorInvalidValue;
        return np_launch<FMT, false, true, true>(p, s);
    }
}

bool bd_ok(const FfnPass &up, const FfnPass &dn, int T)
{
    // CB2 or CB2S gate/up, Q2_K down, every K a multiple of 512, at most 64 tokens
    return (up.fmt == FMT_CB2 || up.fmt == FMT_CB2S) && dn.fmt == FMT_Q2K && up.K % 512 == 0 && dn.K % 512 == 0 && T <= 64 &&
           up.out_f32 && dn.act_f32 && !up.slot == !dn.slot;
}

hipError_t launch_bd(const FfnPass &p, bool gateup, hipStream_t s)
{
    if (gateup) {
        if (p.fmt == FMT_CB2S) return p.act_f32 ? bd_launch<FMT_CB2S, true>(p, s) : bd_launch<FMT_CB2S, false>(p, s);
        if (p.fmt != FMT_CB2) return hipErrorInvalidValue;
        return p.act_f32 ? bd_launch<FMT_CB2, true>(p, s) : bd_launch<FMT_CB2, false>(p, s);
    }
    if (!p.act_f32 || p.fmt != FMT_Q2K) return hipErrorInvalidValue;
    return bd_launch<FMT_Q2K, true>(p, s);
}

hipError_t launch_np_decode(const FfnPass &p, bool gateup, hipStream_t s)
{
    if (!np_decode_ok(p)) return hipErrorInvalidValue;
    switch (p.fmt) {
    case FMT_CB2: return np_decode_fmt<FMT_CB2>(p, gateup, s);
    case FMT_CB2S: return np_decode_fmt<FMT_CB2S>(p, gateup, s);
    case FMT_Q2K: return np_decode_fmt<FMT_Q2K>(p, gateup, s);
    case FMT_Q4K: return np_decode_fmt<FMT_Q4K>(p, gateup, s);
    case FMT_Q5K: return np_decode_fmt<FMT_Q5K>(p, gateup, s);
    case FMT_Q6K: return np_decode_fmt<FMT_Q6K>(p, gateup, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
