// Launchers of the router kernels (csrc/route.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ router
void launch_route_logits(const void *x, bool xbf16, const float *wr, const float *bias, int T, int H, int E,
                         double *logits, hipStream_t s);
void launch_route_select_small(const double *logits, int T, int E, int k, int32_t *topk_idx, float *topk_w,
                               int32_t *offsets, int32_t *perm, int32_t *inv, hipStream_t s);
// logits: [route_logits_parts(T, H)][T][E] (partial sums for the fp64 MFMA
// kernel, which leaves the bias to the top-k kernel)
constexpr int ROUTE_KPARTS = 4;
int route_logits_parts(int T, int H);
void launch_route_topk(const double *logits, const float *bias, int T, int H, int E, int k, int32_t *topk_idx,
                       float *topk_w, hipStream_t s);
void launch_route_rank(const int32_t *topk_idx, int T, int E, int k, int32_t *rank, int32_t *tile_counts,
                       hipStream_t s);
void launch_route_scan(int T, int E, int k, int32_t *tile_counts, int32_t *offsets, hipStream_t s);
void launch_route_scatter(const int32_t *topk_idx, const int32_t *rank, const int32_t *tile_base,
                          const int32_t *offsets, int T, int E, int k, int32_t *perm, int32_t *inv,
                          hipStream_t s);

// small-T router (T <= 64, k <= 64, E <= 1024): partial logits, then one
// work-group selects and groups
int route_decode_chunks(int T, int H);
void launch_route_partial(const void *x, bool xbf16, const float *wr, int T, int H, int E, double *part,
                          hipStream_t s);
void launch_route_select(const double *part, const float *bias, int T, int H, int E, int k, int32_t *topk_idx,
                         float *topk_w, int32_t *offsets, int32_t *perm, int32_t *inv, hipStream_t s);

}  // namespace moe
