// Device-side building blocks shared by the gfx950 kernels.
//
// Block formats (256 weights per block, one row = ceil(K/256) blocks):
//   CB2  38 B  fp16 d | 8 x 4-bit s_j | 32 codebook indices (group of 8 each)
//   Q2_K 84 B  fp16 d | fp16 dmin | 16 x (sc | m<<4) | 64 B of 2-bit codes
//   Q4_K 144 B fp16 d | fp16 dmin | 12 B of 6-bit sc/m | 128 B of 4-bit codes
//   Q5_K 176 B as Q4_K | 32 B plane of the codes' fifth bit
//   Q6_K 210 B fp16 d | 16 int8 scales | 128 B low nibbles, 64 B high 2 bits of q+32
// Only the routed experts are quantized, gate/up in the 2-bit codebook format
// and down in Q2_K ("DwarfStar" README, section on model weights).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int QK = 256;          // weights per block
constexpr int KS = 128;          // K-step of the FFN kernels (half a block)
constexpr int LROW = KS + 8;     // LDS row stride in bf16 elements (16 B pad)

enum { FMT_CB2 = 1, FMT_Q2K = 2, FMT_Q4K = 3, FMT_BF16 = 4, FMT_Q5K = 5, FMT_Q6K = 6, FMT_CB2S = 7 };

constexpr int block_bytes(int fmt)
{
    return fmt == FMT_CB2 ? 38 : fmt == FMT_Q2K ? 84 : fmt == FMT_Q4K ? 144 : fmt == FMT_Q5K ? 176 : fmt == FMT_Q6K ? 210
         : fmt == FMT_CB2S ? 66 : 0;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// bf16 bits of a float that is exactly representable in bf16
__device__ __forceinline__ uint32_t f32_to_bf16_exact(float f) { return __float_as_uint(f) >> 16; }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) { return *(const uint16_t *)p; }

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------------------------------
// Dequantization of one "unit": 32 consecutive weights of one row starting at
// position k0 (a multiple of 32) inside block `blk`.  Output: 16 dwords of
// packed bf16 pairs (element 2i in the low half).
//
// EXACT = true: integer codes with the sub-block scale folded in (CB2: s_j*C,
//   Q2_K: sc_j*q, both |v| <= 45 and so exact in bf16); the block scale d is
//   applied by the caller after the MFMA.  For Q2_K the min term needs the two
//   sub-block mins m_j (returned in m2[0..1]) and dmin (returned in *dmin).
// EXACT = false: the dequantized fp32 value (exact), rounded to bf16 (RNE).
// ----------------------------------------------------------------------------
template <bool EXACT>
__device__ __forceinline__ void unit_cb2(const uint8_t *blk, int k0, const int8_t *cb,
                                         uint32_t out[16], float *d_out)
{
    const float d = f16_bits_to_f32(ld_u16(blk));
    const int j = k0 >> 5;
    const int s = (blk[2 + (j >> 1)] >> (4 * (j & 1))) & 15;
    const float step = d * (float)s;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int idx = blk[6 + 4 * j + g];
        const int8_t *c = cb + 8 * idx;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            uint32_t lo, hi;
            if (EXACT) {
                lo = f32_to_bf16_exact((float)(s * (int)c[i]));
                hi = f32_to_bf16_exact((float)(s * (int)c[i + 1]));
            } else {
                lo = f32_to_bf16_rne(step * (float)c[i]);
                hi = f32_to_bf16_rne(step * (float)c[i + 1]);
            }
            out[4 * g + i / 2] = lo | (hi << 16);
        }
    }
    *d_out = d;
}

template <bool EXACT>
__device__ __forceinline__ void unit_q2k(const uint8_t *blk, int k0, uint32_t out[16],
                                         float *d_out, float *dmin_out, int m2[2])
{
    const float d = f16_bits_to_f32(ld_u16(blk));
    const float dmin = f16_bits_to_f32(ld_u16(blk + 2));
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = (k0 >> 4) + jj;
        const int sm = blk[4 + j];
        const int sc = sm & 15, m = sm >> 4;
        m2[jj] = m;
        const float mul = d * (float)sc, off = dmin * (float)m;
#pragma unroll
        for (int bq = 0; bq < 4; ++bq) {             // 4 code bytes = 16 weights
            const int byte = blk[20 + 4 * j + bq];
#pragma unroll
            for (int t = 0; t < 4; t += 2) {
                const int q0 = (byte >> (2 * t)) & 3, q1 = (byte >> (2 * t + 2)) & 3;
                uint32_t lo, hi;
                if (EXACT) {
                    lo = f32_to_bf16_exact((float)(sc * q0));
                    hi = f32_to_bf16_exact((float)(sc * q1));
                } else {
                    lo = f32_to_bf16_rne(mul * (float)q0 - off);
                    hi = f32_to_bf16_rne(mul * (float)q1 - off);
                }
                out[8 * jj + 2 * bq + t / 2] = lo | (hi << 16);
            }
        }
    }
    *d_out = d;
    *dmin_out = dmin;
}

__device__ __forceinline__ int q4k_field(const uint8_t *blk, int n)
{
    const int bit = 6 * n;
    const int byte = 4 + (bit >> 3), sh = bit & 7;
    int v = blk[byte] >> sh;
    if (sh > 2) v |= blk[byte + 1] << (8 - sh);
    return v & 63;
}

// Q4_K: only the bf16-rounded path (sc*q needs up to 10 bits)
__device__ __forceinline__ void unit_q4k_bf16(const uint8_t *blk, int k0, uint32_t out[16])
{
    const float d = f16_bits_to_f32(ld_u16(blk));
    const float dmin = f16_bits_to_f32(ld_u16(blk + 2));
    const int j = k0 >> 5;
    const int sc = q4k_field(blk, j), m = q4k_field(blk, 8 + j);
    const float mul = d * (float)sc, off = dmin * (float)m;
#pragma unroll
    for (int b = 0; b < 16; ++b) {                   // 16 code bytes = 32 weights
        const int byte = blk[16 + 16 * j + b];
        const uint32_t lo = f32_to_bf16_rne(mul * (float)(byte & 15) - off);
        const uint32_t hi = f32_to_bf16_rne(mul * (float)(byte >> 4) - off);
        out[b] = lo | (hi << 16);
    }
}

}  // namespace moe
