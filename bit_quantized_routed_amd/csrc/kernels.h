// Host-side launchers of the gfx950 kernels (all asynchronous on stream s).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ FFN
// One grouped GEMM pass over the routed experts (groups 0..E-1) and the
// shared expert (group E).  Rows of group g are "positions": routed expert e
// owns positions offsets[e]..offsets[e+1]-1 (in perm order); the shared
// expert owns positions T*k .. T*k+T-1 (token t at T*k+t).
struct FfnPass {
    int T, k, E;
    const int32_t *offsets, *perm;
    int fmt;                          // routed format
    const uint8_t *w0, *w1;           // routed gate,up (gate/up pass) or down,null
    int64_t w_expert_bytes;           // bytes of one expert's matrix
    int64_t w_row_bytes;              // bytes of one packed row
    const uint16_t *s0, *s1;          // shared expert bf16 matrices (or null)
    const int8_t *codebook;           // CB2 codebook (device)
    int K, N;                         // routed: reduction length, output rows
    int Ksh, Nsh;                     // shared: reduction length, output rows (Nsh = 0: none)
    const void *act;                  // activations
    int act_f32;                      // 1: fp32 elements, 0: bf16
    int act_by_token;                 // 1: gate/up (row = token of the position), 0: down (row = position)
    int64_t act_stride;               // elements per activation row
    void *out;                        // output rows by position
    int out_f32;                      // 1: fp32 output, 0: bf16 (RNE)
    int64_t out_stride;               // elements per output row
    const int32_t *sched;             // [0] = tile count, then (group, m0) pairs
    // shared expert split over K (batched decode): tiles of group E + q take
    // K part q of sh_parts; with sh_part_out set they write fp32 partial sums
    // there (gate/up: [q][2][T][Nsh] g and u; down: [q][T][Nsh]) instead of out
    int sh_parts;                     // 0 or 1: one part
    float *sh_part_out;               // null: shared rows go to out like the others
    int sched_parts;                  // shared K parts the schedule was built with (>= sh_parts; 0 or 1: one);
                                      // the launch grid covers every tile of that schedule
    const int32_t *slot;              // null, or expert -> index of its matrices in w0/w1 (expert cache view)
    int skip_routed;                  // 1: the grouped GEMM runs the shared expert's tiles only (the
                                      // routed tiles go to the batched-decode kernels)
};

// tiles of BM rows per routed group and BMsh (<= 0: BM) for the shared group,
// each shared row tile repeated for KSsh K parts (group ids E .. E+KSsh-1)
int ffn_max_tiles(int T, int k, int E, int has_shared, int BM, int BMsh = 0, int KSsh = 1);
void launch_ffn_schedule(const int32_t *offsets, int T, int k, int E, int has_shared, int BM,
                         int32_t *sched, hipStream_t s, int BMsh = 0, int KSsh = 1);
// h of the shared rows from K-part partial sums: silu(sum g) * sum u
void launch_sh_finalize(const float *part, int KS, int T, int I, int Tk, uint16_t *h_bf16, float *h_f32, int hstride,
                        hipStream_t s);
// decode (exact codes, fp32 accumulation); returns hipSuccess or an error
hipError_t launch_ffn_decode(const FfnPass &p, bool gateup, hipStream_t s);
// prefill (bf16-rounded weights, bf16 MFMA)
hipError_t launch_ffn_prefill(const FfnPass &p, bool gateup, hipStream_t s);
// sh_parts > 0: the shared expert's output is the sum of sh_parts slices
// [q][T][H] at sh (fixed order); 0: no shared expert
void launch_combine(const float *O, const int32_t *inv, const float *topk_w, int T, int k, int H,
                    int sh_parts, const float *sh, float *y, hipStream_t s);
hipError_t launch_unpack(int fmt, const uint8_t *packed, int64_t rows, int K, const int8_t *codebook,
                         float *out, hipStream_t s);

constexpr int DEC_BM = 16, DEC_BN = 16;
constexpr int PRE_BM = 64, PRE_BN = 64;

// prefill grouped GEMMs with in-register dequantization (K multiples of 256,
// bf16 activations); tiles of NP_BM rows
constexpr int NP_BM = 96, NP_BM_SH = 80;
bool np_prefill_ok(const FfnPass &p);
hipError_t launch_np_prefill(const FfnPass &p, bool gateup, hipStream_t s);
// the same GEMMs at decode precision (exact weights, fp32 h), tiles of
// NP_BM_DEC rows, for batched decode (T > 1)
constexpr int NP_BM_DEC = 32;
bool np_decode_ok(const FfnPass &p);
hipError_t launch_np_decode(const FfnPass &p, bool gateup, hipStream_t s);

// Batched decode of the routed tiles (CB2 gate/up, Q2_K down; every K a
// multiple of 512): weights staged through LDS in block pairs with coalesced
// loads, BD_BM positions per tile.  The schedule must be built with BD_BM
// rows per routed tile and NP_BM_DEC per shared tile; the shared tiles are
// left to launch_np_decode with skip_routed set.
constexpr int BD_BM = 16;
bool bd_ok(const FfnPass &up, const FfnPass &dn, int T);
hipError_t launch_bd(const FfnPass &p, bool gateup, hipStream_t s);

}  // namespace moe
