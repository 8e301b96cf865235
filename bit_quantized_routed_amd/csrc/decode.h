// Launch interface of the single-token decode kernels (decode.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct DecPass {
    int T, k, E, H, I, Ish, nbI;
    const int32_t *topk_idx, *offsets, *inv;
    const float *topk_w;
    const uint8_t *wg, *wu, *wd;                 // routed CB2 gate, up; Q2_K down
    const int32_t *slot;                         // null, or expert -> index of its matrices (expert cache view)
    int64_t gu_expert_bytes, d_expert_bytes;
    int gu_row_bytes, d_row_bytes;
    const uint16_t *sg, *su, *sd;                // shared expert bf16 (Ish == 0: none)
    const int8_t *codebook;
    const void *x;
    int x_f32;
    int nkc;                                     // K chunks of the routed gate/up tables
    float *part_rt;                              // [nkc][k][2][I] routed gate/up partial sums by K chunk
    float *part_sh;                              // [DEC_SH_KQ][2][Ish] shared gate/up partial sums (K parts)
    uint16_t *h_hi, *h_lo;                       // [k][hstride] routed h as two bf16 terms (fused down)
    int hstride;
    float *X;                                    // [k][nbI][16] per-16 sums of h (Q2_K min term; fused down)
    uint16_t *sh_hi, *sh_lo;                     // [Ish] shared h as two bf16 terms (fused down)
    int fused;                                   // 1: h formed once, then one down launch writes y
    float *O;                                    // [k][H] by top-k slot
    float *O_sh;                                 // [Ish/512][H]
    float *y;                                    // [H]
    int gu_sh_wg, gu_rt_wg;                      // gate/up work-groups: shared, routed role
    int dn_sh_wg, dn_rt_wg;                      // down work-groups: shared, routed role
    // staged single-token layer (dec_stage1 / dec_stage2, then dec_hform and
    // dec_down_fused with the shared down already done)
    int s1_wg;                                   // stage 1 work-groups (every one takes shared gate/up units)
    int s2_wg;                                   // stage 2 work-groups (routed gate/up units; the shared
                                                 //    down in their prologue)
    int staged;                                  // 1: the shared down is done in stage 2 (O_sh parts),
                                                 //    so dec_hform forms routed h only and dec_down_fused
                                                 //    adds the O_sh parts to y
    // router inside the stages (the fused layer entry point): stage 1 writes the
    // partial logits, stage 2 selects from them
    int route;                                   // 1: stage 1 computes the logits, stage 2 selects
    const float *wr;                             // [E][H] fp32 router weights
    const float *bias;                           // [E] or null
    double *rpart;                               // [rnc][E] partial logits
    int rnc, rhc;                                // H chunks and chunk length of the partial logits
    int32_t *o_idx, *o_off, *o_perm, *o_inv;     // routing outputs written by stage 2
    float *o_w;
};
constexpr int DEC_SH_KQ = 8;                     // K parts of the single-token shared gate/up (part_sh)
constexpr int DEC_LUT_KB = 4;                    // 256-wide blocks per K chunk of a routed gate/up table
bool dec_single_ok(int T, int H, int I, int Ish, int k, int gu_row_bytes, bool x_f32);
void dec_plan(DecPass &p);                       // fills the work-group split
hipError_t launch_dec_gateup(const DecPass &p, hipStream_t s);
hipError_t launch_dec_down(const DecPass &p, hipStream_t s);
hipError_t launch_dec_combine(const DecPass &p, hipStream_t s);
// the fused down (k <= 8, I <= 2048, sh_inter <= 2048): h formed once, then
// y from every slot and the shared expert in one launch (no combine)
bool dec_fused_ok(int k, int I, int Ish);
hipError_t launch_dec_hform(const DecPass &p, hipStream_t s);
hipError_t launch_dec_down_fused(const DecPass &p, hipStream_t s);
// the staged single-token layer (p.staged = 1; dec_fused_ok shapes): stage 1
// (shared gate/up, and with p.route the router's partial logits), stage 2
// (routed gate/up -- with p.route selecting the experts first -- and the
// shared down), then dec_hform and dec_down_fused
void dec_plan_staged(DecPass &p);
hipError_t launch_dec_stage1(const DecPass &p, hipStream_t s);
hipError_t launch_dec_stage2(const DecPass &p, hipStream_t s);

}  // namespace moe
