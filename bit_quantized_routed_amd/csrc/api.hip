// C ABI of the routed-MoE expert layer (see include/moe.h): host-side argument
// validation, workspace carving and the kernel launch sequences.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "cache.h"
#include "decode.h"
#include "devcache.h"
#include "kernels.h"
#include "route.h"
#include "probe.h"
#include "status.h"
#include "moe.h"
#include "moe_probe.h"

namespace moe {

namespace {
thread_local std::string g_err;
}

int set_error(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

}  // namespace moe

using namespace moe;

namespace {

int hip_fail(hipError_t e, const char *what)
{
    return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// Records the caller's events around launch number `prof->kernel`.
struct Prof {
    moe_profile *p;
    hipStream_t s;
    int n = 0;
    bool before(const char *name)
    {
        if (p && p->kernel == n) {
            p->name = name;
            if (hipEventRecord((hipEvent_t)p->ev_start, s) != hipSuccess) return false;
        }
        return true;
    }
    bool after()
    {
        if (p && p->kernel == n && hipEventRecord((hipEvent_t)p->ev_stop, s) != hipSuccess) return false;
        ++n;
        if (p) p->n_launches = n;
        return true;
    }
};

bool fmt_ok(int f)
{
    return f == MOE_FMT_CB2 || f == MOE_FMT_Q2K || f == MOE_FMT_Q4K || f == MOE_FMT_Q5K || f == MOE_FMT_Q6K ||
           f == MOE_FMT_CB2S;
}
int bbytes(int f)
{
    return f == MOE_FMT_CB2 ? 38 : f == MOE_FMT_Q2K ? 84 : f == MOE_FMT_Q4K ? 144 : f == MOE_FMT_Q5K ? 176
         : f == MOE_FMT_Q6K ? 210 : f == MOE_FMT_CB2S ? 66 : 0;
}
int nblocks(int K) { return (K + 255) / 256; }

int check_router(const moe_layer *L)
{
    if (!L) return set_error(MOE_ERR_INVALID_ARG, "layer is NULL");
    if (L->hidden < 8 || L->hidden % 8) return set_error(MOE_ERR_INVALID_ARG, "hidden=%d must be a positive multiple of 8", L->hidden);
    if (L->n_experts < 1 || L->n_experts > 1024) return set_error(MOE_ERR_INVALID_ARG, "n_experts=%d outside [1,1024]", L->n_experts);
    if (L->top_k < 1 || L->top_k > L->n_experts) return set_error(MOE_ERR_INVALID_ARG, "top_k=%d outside [1,n_experts]", L->top_k);
    if (!L->w_router) return set_error(MOE_ERR_INVALID_ARG, "w_router is NULL");
    return MOE_OK;
}

int check_layer(const moe_layer *L)
{
    int rc = check_router(L);
    if (rc) return rc;
    if (L->inter < 8 || L->inter % 8) return set_error(MOE_ERR_INVALID_ARG, "inter=%d must be a positive multiple of 8", L->inter);
    const int fg = L->fmt_gate_up, fd = L->fmt_down;
    if (fg != MOE_FMT_CB2 && fg != MOE_FMT_CB2S && fg != MOE_FMT_Q2K && fg != MOE_FMT_Q4K && fg != MOE_FMT_Q5K)
        return set_error(MOE_ERR_INVALID_ARG, "fmt_gate_up=%d must be CB2, CB2S, Q2K, Q4K or Q5K", fg);
    if (fd != MOE_FMT_Q2K && fd != MOE_FMT_Q4K && fd != MOE_FMT_Q5K && fd != MOE_FMT_Q6K)
        return set_error(MOE_ERR_INVALID_ARG, "fmt_down=%d must be Q2K, Q4K, Q5K or Q6K", fd);
    if (!L->w_gate || !L->w_up || !L->w_down) return set_error(MOE_ERR_INVALID_ARG, "routed expert weights are NULL");
    if ((fg == MOE_FMT_CB2 || fg == MOE_FMT_CB2S) && !L->codebook)
        return set_error(MOE_ERR_INVALID_ARG, "CB2 needs a codebook, CB2S its magnitude grid");
    for (const void *ptr : {L->w_gate, L->w_up, L->w_down, (const void *)L->codebook, L->sh_gate, L->sh_up,
                            L->sh_down, (const void *)L->w_router})
        if ((uintptr_t)ptr % 16) return set_error(MOE_ERR_INVALID_ARG, "layer pointer %p is not 16-byte aligned", ptr);
    if (L->sh_inter < 0) return set_error(MOE_ERR_INVALID_ARG, "sh_inter=%d < 0", L->sh_inter);
    if ((uintptr_t)L->expert_slot % 4) return set_error(MOE_ERR_INVALID_ARG, "expert_slot is not 4-byte aligned");
    if (L->flags & ~(MOE_LAYER_TOKENWISE_DECODE | MOE_LAYER_ONE_STREAM))
        return set_error(MOE_ERR_INVALID_ARG, "flags=%#x: unknown bits", L->flags);
    if (L->sh_inter > 0) {
        if (!L->sh_gate || !L->sh_up || !L->sh_down) return set_error(MOE_ERR_INVALID_ARG, "shared expert weights are NULL");
        if (L->sh_inter % 256 || L->hidden % 256)
            return set_error(MOE_ERR_INVALID_ARG, "shared expert needs sh_inter and hidden multiples of 256");
    }
    return MOE_OK;
}

struct RouteWs {
    double *logits;          // fused path: [NC][T][E] partial logits (chunk 0 ends as the logits)
    int32_t *rank, *tile_counts;
    size_t bytes;
};

bool route_fused(const moe_layer *L, int T) { return T <= 64 && L->top_k <= 64; }
bool route_small(const moe_layer *L, int T) { return T <= 64 && T * L->top_k <= 2048; }

RouteWs route_ws(const moe_layer *L, int T, char *base)
{
    RouteWs w{};
    size_t off = 0;
    const size_t E = L->n_experts, k = L->top_k;
    w.logits = (double *)(base + off);
    const size_t nc = route_fused(L, T) ? (size_t)route_decode_chunks(T, L->hidden)
                                        : (size_t)route_logits_parts(T, L->hidden);
    off = align_up(off + nc * (size_t)T * E * sizeof(double));
    if (!route_fused(L, T) && !route_small(L, T)) {
        w.rank = (int32_t *)(base + off);
        off = align_up(off + (size_t)T * k * sizeof(int32_t));
        w.tile_counts = (int32_t *)(base + off);
        off = align_up(off + (size_t)((T + 63) / 64) * E * sizeof(int32_t));
    }
    w.bytes = off;
    return w;
}

struct FfnWs {
    int32_t *sched;
    void *h;
    float *O;
    size_t bytes;
    int hstride;
    // single-token decode
    bool single;
    float *part_sh, *O_sh;
    float *sh_part;                   // batched decode: shared-expert K-part partial sums
    int ks_gu, ks_dn;                 // its K parts for gate/up and down (0: not split)
    float *part_rt;
    int nkc;
    uint16_t *h_hi, *h_lo, *sh_hi, *sh_lo;
    float *X;
};

// Decode batches of up to DEC_TOKENWISE_MAX tokens run the single-token
// kernels once per token (measured faster than the grouped GEMMs there, since
// almost every assignment is a distinct expert), so such a token's result does
// not depend on the batch it came in.  They apply for CB2/Q2K and the shapes
// the single-token kernels support.
constexpr int DEC_TOKENWISE_MAX = 4;
bool tokenwise_flag(const moe_layer *L) { return (L->flags & MOE_LAYER_TOKENWISE_DECODE) != 0; }
bool dec_single(const moe_layer *L, int T, bool prefill, bool x_f32)
{
    if (prefill || T < 1 || (T > DEC_TOKENWISE_MAX && !tokenwise_flag(L))) return false;
    if (L->fmt_gate_up != MOE_FMT_CB2 || L->fmt_down != MOE_FMT_Q2K) return false;
    return dec_single_ok(1, L->hidden, L->inter, L->sh_inter, L->top_k, nblocks(L->hidden) * 38, x_f32);
}

// Workspace carving.  `single` selects the single-token layout; the size a
// caller must provide (moe_workspace_bytes) is the larger of the layouts the
// call may take, since the choice also depends on the activation type.
FfnWs ffn_ws(const moe_layer *L, int T, bool prefill, bool single, char *base)
{
    FfnWs w{};
    const int has_sh = L->sh_inter > 0;
    const int BM = prefill ? PRE_BM : DEC_BM;
    const size_t rows = (size_t)T * L->top_k + (has_sh ? T : 0);
    w.hstride = std::max(L->inter, L->sh_inter);
    size_t off = 0;
    w.single = single;
    if (w.single) {
        const size_t k = L->top_k, H = L->hidden, Ish = L->sh_inter;
        w.part_sh = (float *)(base + off);
        off = align_up(off + DEC_SH_KQ * 2 * Ish * sizeof(float));
        w.nkc = (int)((H + 256 * DEC_LUT_KB - 1) / (256 * DEC_LUT_KB));
        w.part_rt = (float *)(base + off);
        off = align_up(off + (size_t)w.nkc * k * 2 * L->inter * sizeof(float));
        // h formed once for the fused down: routed (two bf16 terms, per-16 sums), shared
        const size_t nbI = nblocks(L->inter);
        w.h_hi = (uint16_t *)(base + off);
        off = align_up(off + k * w.hstride * 2);
        w.h_lo = (uint16_t *)(base + off);
        off = align_up(off + k * w.hstride * 2);
        w.X = (float *)(base + off);
        off = align_up(off + k * nbI * 16 * sizeof(float));
        w.sh_hi = (uint16_t *)(base + off);
        off = align_up(off + Ish * 2);
        w.sh_lo = (uint16_t *)(base + off);
        off = align_up(off + Ish * 2);
        w.O = (float *)(base + off);
        off = align_up(off + k * H * sizeof(float));
        w.O_sh = (float *)(base + off);
        off = align_up(off + (Ish / 512) * H * sizeof(float));
        w.bytes = off;
        return w;
    }
    // batched decode splits the shared expert over K in parts of 512
    if (!prefill && has_sh) {
        w.ks_gu = std::max(1, L->hidden / 512);
        w.ks_dn = std::max(1, L->sh_inter / 512);
    }
    int tiles = ffn_max_tiles(T, L->top_k, L->n_experts, has_sh, BM);
    if (!prefill) {
        tiles = std::max(tiles, ffn_max_tiles(T, L->top_k, L->n_experts, has_sh, NP_BM_DEC, NP_BM_DEC,
                                              std::max(w.ks_gu, w.ks_dn)));
        tiles = std::max(tiles, ffn_max_tiles(T, L->top_k, L->n_experts, has_sh, BD_BM, NP_BM_DEC,
                                              std::max(w.ks_gu, w.ks_dn)));
    }
    w.sched = (int32_t *)(base + off);
    off = align_up(off + (1 + 2 * (size_t)tiles) * sizeof(int32_t));
    w.sh_part = (float *)(base + off);
    off = align_up(off + std::max((size_t)w.ks_gu * 2 * T * L->sh_inter, (size_t)w.ks_dn * T * L->hidden) * sizeof(float));
    w.h = base + off;
    off = align_up(off + rows * w.hstride * (prefill ? 2 : 4));
    w.O = (float *)(base + off);
    off = align_up(off + rows * (size_t)L->hidden * sizeof(float));
    w.bytes = off;
    return w;
}

size_t ffn_ws_bytes(const moe_layer *L, int T, bool prefill)
{
    size_t b = ffn_ws(L, T, prefill, false, nullptr).bytes;
    for (int xf = 0; xf < 2; ++xf)
        if (dec_single(L, T, prefill, xf)) b = std::max(b, ffn_ws(L, 1, prefill, true, nullptr).bytes);
    return b;
}

// The staged single-token layer: stage 1 (shared gate/up, and with d.route
// the router's partial logits), stage 2 (routed gate/up -- with d.route after
// selecting the experts -- beside the shared down), routed h, routed down + y.
int launch_staged(const DecPass &d, Prof &pr)
{
    hipError_t e;
#define MOE_STAGE(name, call)                                                      \
    do {                                                                           \
        if (!pr.before(name)) return hip_fail(hipGetLastError(), "event record");  \
        e = call;                                                                  \
        if (e != hipSuccess) return hip_fail(e, name);                             \
        if (!pr.after()) return hip_fail(hipGetLastError(), "event record");       \
    } while (0)
    MOE_STAGE("dec_stage1", launch_dec_stage1(d, pr.s));
    MOE_STAGE("dec_stage2", launch_dec_stage2(d, pr.s));
    MOE_STAGE("dec_hform", launch_dec_hform(d, pr.s));
    MOE_STAGE("dec_down_fused", launch_dec_down_fused(d, pr.s));
#undef MOE_STAGE
    return MOE_OK;
}

// the single-token pass over one layer (everything but the activations, the
// routing and the output), for the decode path's token-wise kernels
DecPass single_pass(const moe_layer *L, const FfnWs &w, int act)
{
    DecPass d{};
    const int H = L->hidden, I = L->inter;
    d.T = 1; d.k = L->top_k; d.E = L->n_experts; d.H = H; d.I = I; d.Ish = L->sh_inter; d.nbI = nblocks(I);
    d.wg = (const uint8_t *)L->w_gate; d.wu = (const uint8_t *)L->w_up; d.wd = (const uint8_t *)L->w_down;
    d.slot = L->expert_slot;
    d.gu_row_bytes = nblocks(H) * 38;
    d.gu_expert_bytes = (int64_t)d.gu_row_bytes * I;
    d.d_row_bytes = nblocks(I) * 84;
    d.d_expert_bytes = (int64_t)d.d_row_bytes * H;
    d.sg = (const uint16_t *)L->sh_gate; d.su = (const uint16_t *)L->sh_up; d.sd = (const uint16_t *)L->sh_down;
    d.codebook = L->codebook;
    d.x_f32 = act == MOE_ACT_F32;
    d.nkc = w.nkc; d.part_rt = w.part_rt;
    d.h_hi = w.h_hi; d.h_lo = w.h_lo; d.hstride = w.hstride; d.X = w.X; d.sh_hi = w.sh_hi; d.sh_lo = w.sh_lo;
    d.fused = dec_fused_ok(d.k, I, d.Ish);
    d.part_sh = w.part_sh;
    d.O = w.O; d.O_sh = w.O_sh;
    return d;
}

// Batched decode with the LDS-staged routed kernels: the shared expert's
// chain (gate/up, finalize, down) does not depend on the routed one, so it runs
// on a second stream of the device, forked from and joined back into the
// caller's stream by two events (the combine waits for both chains; a caller
// capturing its stream into a graph captures the fork and the join with it).
// The stream (default priority, non-blocking) and events are created on the
// first such call on a device and kept until the process ends; enqueues that
// use them hold a mutex, so each call's join event is its own when host
// threads call concurrently.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool failed = false;
};
SideStream g_side[MAX_DEVICES];
std::mutex g_side_mu;

// this device's side stream (the mutex held), or null: no slot for the device,
// or creating it failed (the call then runs on the caller's stream alone)
SideStream *side_stream()
{
    const int slot = device_slot();
    if (slot < 0) return nullptr;
    SideStream &S = g_side[slot];
    if (S.failed) return nullptr;
    if (!S.s) {
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();                              // leave no sticky error behind
            S.failed = true;
            return nullptr;
        }
        S.s = st;
        S.fork = f;
        S.join = j;
    }
    return &S;
}

int ffn_common(const moe_layer *L, const void *x, int act, int T, const int32_t *topk_idx, const float *topk_w,
               const int32_t *offsets, const int32_t *perm, const int32_t *inv, float *y, void *ws,
               size_t ws_bytes, void *stream, moe_profile *prof, bool prefill, bool side_ok = false)
{
    int rc = check_layer(L);
    if (rc) return rc;
    if (T < 0) return set_error(MOE_ERR_INVALID_ARG, "T=%d < 0", T);
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16) return set_error(MOE_ERR_INVALID_ARG, "act=%d unknown", act);
    if (prof) prof->n_launches = 0;
    if (T == 0) return MOE_OK;
    if ((int64_t)T * L->top_k > (1 << 30)) return set_error(MOE_ERR_INVALID_ARG, "T*k too large");
    if (!x || !topk_idx || !topk_w || !offsets || !perm || !inv || !y) return set_error(MOE_ERR_INVALID_ARG, "NULL tensor argument");
    if (!ws) return set_error(MOE_ERR_INVALID_ARG, "workspace is NULL");
    if ((uintptr_t)x % 16 || (uintptr_t)y % 16 || (uintptr_t)ws % 16)
        return set_error(MOE_ERR_INVALID_ARG, "x, y and the workspace must be 16-byte aligned");
    // CB2/Q4K gate/up with Q2K/Q4K down run on every shape; the other format
    // pairs, and decode with anything but CB2 + Q2K, only on the grouped GEMMs
    // with in-register dequantization, which need every K a multiple of 512
    const bool gemm = L->hidden % 512 == 0 && L->inter % 512 == 0 && (L->sh_inter == 0 || L->sh_inter % 512 == 0);
    const bool base_fmts = (L->fmt_gate_up == MOE_FMT_CB2 || L->fmt_gate_up == MOE_FMT_Q4K) &&
                           (L->fmt_down == MOE_FMT_Q2K || L->fmt_down == MOE_FMT_Q4K);
    if (prefill) {
        if (act != MOE_ACT_BF16) return set_error(MOE_ERR_INVALID_ARG, "prefill needs bf16 activations");
        if (!base_fmts && !gemm)
            return set_error(MOE_ERR_UNSUPPORTED, "prefill with gate/up fmt %d, down fmt %d needs hidden, inter and "
                             "sh_inter multiples of 512", L->fmt_gate_up, L->fmt_down);
    } else {
        const bool cb2q2k = L->fmt_gate_up == MOE_FMT_CB2 && L->fmt_down == MOE_FMT_Q2K;
        if (tokenwise_flag(L) && !dec_single(L, T, false, act == MOE_ACT_F32))
            return set_error(MOE_ERR_UNSUPPORTED, "token-by-token decode needs a layer the single-token kernels take "
                             "(CB2 gate/up, Q2K down, H %% 512 == 0, H <= 8192, I %% 256 == 0, I <= 2048, "
                             "sh_inter %% 512 == 0)");
        if (!cb2q2k && !gemm)
            return set_error(MOE_ERR_UNSUPPORTED, "decode with gate/up fmt %d, down fmt %d needs hidden, inter and "
                             "sh_inter multiples of 512", L->fmt_gate_up, L->fmt_down);
    }
    // the grouped-GEMM kernels index activation rows with 32-bit element offsets
    const int64_t act_rows = (int64_t)T * L->top_k + (L->sh_inter > 0 ? T : 0);
    if ((int64_t)T * L->hidden >= ((int64_t)1 << 31) || act_rows * std::max(L->inter, L->sh_inter) >= ((int64_t)1 << 31))
        return set_error(MOE_ERR_UNSUPPORTED, "T=%d: activations beyond 2^31 elements per call", T);
    const size_t need = ffn_ws_bytes(L, T, prefill);
    if (ws_bytes < need) return set_error(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    const bool single = dec_single(L, T, prefill, act == MOE_ACT_F32);
    FfnWs w = ffn_ws(L, single ? 1 : T, prefill, single, (char *)ws);

    hipStream_t s = (hipStream_t)stream;
    Prof pr{prof, s};
    const int H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k, Ish = L->sh_inter;
    const int has_sh = Ish > 0;
    const int BM = prefill ? PRE_BM : DEC_BM;

    if (w.single) {
        DecPass d = single_pass(L, w, act);
        d.topk_idx = topk_idx; d.offsets = offsets; d.inv = inv; d.topk_w = topk_w;
        d.x = x; d.y = y;
        dec_plan(d);
        if (d.fused) dec_plan_staged(d);
        const size_t xrow = (size_t)H * (act == MOE_ACT_F32 ? 4 : 2);
        for (int t = 0; t < T; ++t) {                              // one token at a time, in order
            d.x = (const char *)x + t * xrow;
            d.topk_idx = topk_idx + (size_t)t * k;
            d.topk_w = topk_w + (size_t)t * k;
            d.y = y + (size_t)t * H;
            if (d.fused) {
                const int rc2 = launch_staged(d, pr);
                if (rc2) return rc2;
                continue;
            }
            if (!pr.before("dec_gateup")) return hip_fail(hipGetLastError(), "event record");
            hipError_t e = launch_dec_gateup(d, s);
            if (e != hipSuccess) return hip_fail(e, "dec_gateup launch");
            if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
            if (!pr.before("dec_down")) return hip_fail(hipGetLastError(), "event record");
            e = launch_dec_down(d, s);
            if (e != hipSuccess) return hip_fail(e, "dec_down launch");
            if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
            if (!pr.before("dec_combine")) return hip_fail(hipGetLastError(), "event record");
            e = launch_dec_combine(d, s);
            if (e != hipSuccess) return hip_fail(e, "dec_combine launch");
            if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
        }
        return MOE_OK;
    }

    FfnPass up{};
    up.T = T; up.k = k; up.E = E;
    up.offsets = offsets; up.perm = perm;
    up.fmt = L->fmt_gate_up;
    up.w0 = (const uint8_t *)L->w_gate; up.w1 = (const uint8_t *)L->w_up;
    up.w_row_bytes = (int64_t)nblocks(H) * bbytes(L->fmt_gate_up);
    up.w_expert_bytes = up.w_row_bytes * I;
    up.s0 = (const uint16_t *)L->sh_gate; up.s1 = (const uint16_t *)L->sh_up;
    up.codebook = L->codebook;
    up.K = H; up.N = I; up.Ksh = H; up.Nsh = has_sh ? Ish : 0;
    up.act = x; up.act_f32 = act == MOE_ACT_F32; up.act_by_token = 1; up.act_stride = H;
    up.out = w.h; up.out_f32 = prefill ? 0 : 1; up.out_stride = w.hstride;
    up.sched = w.sched;
    up.slot = L->expert_slot;

    FfnPass dn = up;
    dn.fmt = L->fmt_down;
    dn.w0 = (const uint8_t *)L->w_down; dn.w1 = nullptr;
    dn.w_row_bytes = (int64_t)nblocks(I) * bbytes(L->fmt_down);
    dn.w_expert_bytes = dn.w_row_bytes * H;
    dn.s0 = (const uint16_t *)L->sh_down; dn.s1 = nullptr;
    dn.K = I; dn.N = H; dn.Ksh = Ish; dn.Nsh = has_sh ? H : 0;
    dn.act = w.h; dn.act_f32 = prefill ? 0 : 1; dn.act_by_token = 0; dn.act_stride = w.hstride;
    dn.out = w.O; dn.out_f32 = 1; dn.out_stride = H;

    // prefill: in-register dequantization kernels when every K is a multiple of 256
    const bool np = prefill && np_prefill_ok(up) && np_prefill_ok(dn);
    const bool npd = !prefill && np_decode_ok(up) && np_decode_ok(dn);
    // batched decode of CB2/Q2_K layers: routed tiles on the LDS-staged
    // kernels, the shared expert's tiles on the grouped GEMM
    const bool bd = npd && bd_ok(up, dn, T);
    const int sched_bm = np ? NP_BM : bd ? BD_BM : npd ? NP_BM_DEC : BM;
    // batched decode: the shared expert's few rows are spread over K parts so
    // that its work-groups stream no more than a routed tile's
    const bool split = npd && has_sh && H % 512 == 0 && Ish % 512 == 0;
    if (split) {
        up.sh_parts = w.ks_gu; up.sh_part_out = w.sh_part;
        dn.sh_parts = w.ks_dn; dn.sh_part_out = w.sh_part;
        up.sched_parts = dn.sched_parts = std::max(w.ks_gu, w.ks_dn);
    }
    if (!pr.before("ffn_schedule")) return hip_fail(hipGetLastError(), "event record");
    launch_ffn_schedule(offsets, T, k, E, has_sh, sched_bm, w.sched, s, np ? NP_BM_SH : bd ? NP_BM_DEC : sched_bm,
                        split ? std::max(w.ks_gu, w.ks_dn) : 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "ffn_schedule launch");
    if (!pr.after()) return hip_fail(hipGetLastError(), "event record");

    const char *nm_up = prefill ? "ffn_prefill_gateup" : "ffn_decode_gateup";
    const char *nm_dn = prefill ? "ffn_prefill_down" : "ffn_decode_down";
    // the shared chain's stream: a second one, forked here, when the routed
    // tiles run on their own kernels (see SideStream)
    std::unique_lock<std::mutex> side_lock;
    SideStream *side = nullptr;
    if (bd && split && side_ok && !(L->flags & MOE_LAYER_ONE_STREAM)) {
        side_lock = std::unique_lock<std::mutex>(g_side_mu);
        side = side_stream();
        if (side) {
            if (hipEventRecord(side->fork, s) != hipSuccess) return hip_fail(hipGetLastError(), "fork record");
            if (hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess) return hip_fail(hipGetLastError(), "fork wait");
        }
    }
    const hipStream_t ss = side ? side->s : s;
    auto shared_up = [&]() -> int {
        pr.s = ss;
        if (!pr.before(nm_up)) return hip_fail(hipGetLastError(), "event record");
        e = np ? launch_np_prefill(up, true, ss) : npd ? launch_np_decode(up, true, ss)
               : prefill ? launch_ffn_prefill(up, true, ss) : launch_ffn_decode(up, true, ss);
        if (e != hipSuccess) return hip_fail(e, nm_up);
        if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
        if (split) {
            if (!pr.before("sh_finalize")) return hip_fail(hipGetLastError(), "event record");
            launch_sh_finalize(w.sh_part, w.ks_gu, T, Ish, T * k, nullptr, (float *)w.h, w.hstride, ss);
            e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(e, "sh_finalize launch");
            if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
        }
        pr.s = s;
        return MOE_OK;
    };
    auto shared_down = [&]() -> int {
        pr.s = ss;
        if (!pr.before(nm_dn)) return hip_fail(hipGetLastError(), "event record");
        e = np ? launch_np_prefill(dn, false, ss) : npd ? launch_np_decode(dn, false, ss)
               : prefill ? launch_ffn_prefill(dn, false, ss) : launch_ffn_decode(dn, false, ss);
        if (e != hipSuccess) return hip_fail(e, nm_dn);
        if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
        pr.s = s;
        return MOE_OK;
    };
    if (bd) {
        if (!pr.before("bd_gateup")) return hip_fail(hipGetLastError(), "event record");
        e = launch_bd(up, true, s);
        if (e != hipSuccess) return hip_fail(e, "bd_gateup");
        if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
        up.skip_routed = dn.skip_routed = 1;
    }
    if (!bd || has_sh) {
        rc = shared_up();
        if (rc) return rc;
    }
    if (side && has_sh) {
        // the shared down follows its gate/up on the side stream
        rc = shared_down();
        if (rc) return rc;
    }
    if (bd) {
        if (!pr.before("bd_down")) return hip_fail(hipGetLastError(), "event record");
        FfnPass dr = dn;
        dr.skip_routed = 0;
        e = launch_bd(dr, false, s);
        if (e != hipSuccess) return hip_fail(e, "bd_down");
        if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
    }
    if ((!bd || has_sh) && !side) {
        rc = shared_down();
        if (rc) return rc;
    }
    if (side) {
        if (hipEventRecord(side->join, side->s) != hipSuccess) return hip_fail(hipGetLastError(), "join record");
        if (hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return hip_fail(hipGetLastError(), "join wait");
    }

    if (!pr.before("combine")) return hip_fail(hipGetLastError(), "event record");
    launch_combine(w.O, inv, topk_w, T, k, H, has_sh ? (split ? w.ks_dn : 1) : 0,
                   split ? w.sh_part : w.O + (size_t)T * k * H, y, s);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    if (!pr.after()) return hip_fail(hipGetLastError(), "event record");
    return MOE_OK;
}

// moe_layer_decode's workspace: the router's, then the decode FFN's
size_t layer_ws_bytes(const moe_layer *L, int T) { return align_up(route_ws(L, T, nullptr).bytes) + ffn_ws_bytes(L, T, false); }

// the fused single-token layer applies (router in the stages) for one token of
// a CB2/Q2K layer of the single-token shapes with the fused down
bool layer_fused(const moe_layer *L, int T, int act)
{
    return T == 1 && route_fused(L, 1) && dec_single(L, 1, false, act == MOE_ACT_F32) &&
           dec_fused_ok(L->top_k, L->inter, L->sh_inter);
}

// ---------------------------------------------------------------- no-allocation decode
// The decode workspace of moe_expert_ffn_decode_noalloc: one fixed array per
// device, which the library holds until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address is looked up once per device (hipGetSymbolAddress with that device
// current) and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

DevSlots g_scratch_addr{};

// device address of this device's scratch array (looked up on the first call on
// the device), or nullptr with the error text set
void *scratch_address()
{
    const int slot = device_slot();
    if (const uint64_t a = g_scratch_addr.get(slot)) return (void *)(uintptr_t)a;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
        hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        return nullptr;
    }
    g_scratch_addr.set(slot, (uint64_t)(uintptr_t)ptr);
    return ptr;
}

}  // namespace

extern "C" {

const char *moe_status_str(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char *moe_last_error(void) { return g_err.c_str(); }

size_t q2_packed_bytes(int fmt, int64_t rows, int K)
{
    if (!fmt_ok(fmt) || rows < 0 || K < 1) return 0;
    return (size_t)rows * nblocks(K) * bbytes(fmt);
}

size_t moe_workspace_bytes(const moe_layer *L, int T, int path)
{
    if (T < 0) return 0;
    if (path == MOE_PATH_ROUTE) {
        if (check_router(L)) return 0;
        return route_ws(L, T, nullptr).bytes;
    }
    if (path != MOE_PATH_DECODE && path != MOE_PATH_PREFILL && path != MOE_PATH_LAYER_DECODE) return 0;
    if (check_layer(L)) return 0;
    if (path == MOE_PATH_LAYER_DECODE) return layer_ws_bytes(L, T);
    return ffn_ws_bytes(L, T, path == MOE_PATH_PREFILL);
}

int moe_route(const moe_layer *L, const void *x, int act, int T, const float *bias, int32_t *topk_idx,
              float *topk_w, int32_t *offsets, int32_t *perm, int32_t *inv, void *ws, size_t ws_bytes,
              void *stream, moe_profile *prof)
{
    int rc = check_router(L);
    if (rc) return rc;
    if (T < 0) return set_error(MOE_ERR_INVALID_ARG, "T=%d < 0", T);
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16) return set_error(MOE_ERR_INVALID_ARG, "act=%d unknown", act);
    if (prof) prof->n_launches = 0;
    if (T == 0) return MOE_OK;
    if ((int64_t)T * L->top_k > (1 << 30)) return set_error(MOE_ERR_INVALID_ARG, "T*k too large");
    if (!x || !topk_idx || !topk_w || !offsets || !perm || !inv) return set_error(MOE_ERR_INVALID_ARG, "NULL tensor argument");
    if (!ws) return set_error(MOE_ERR_INVALID_ARG, "workspace is NULL");
    // the logit kernels read x and W_r in 8- and 16-byte pieces
    if ((uintptr_t)x % 16 || (uintptr_t)L->w_router % 16 || (uintptr_t)ws % 16)
        return set_error(MOE_ERR_INVALID_ARG, "x, w_router and the workspace must be 16-byte aligned");
    RouteWs w = route_ws(L, T, (char *)ws);
    if (ws_bytes < w.bytes) return set_error(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.bytes);

    hipStream_t s = (hipStream_t)stream;
    Prof pr{prof, s};
    const int H = L->hidden, E = L->n_experts, k = L->top_k;
    hipError_t e;
#define MOE_LAUNCH(name, call)                                                     \
    do {                                                                           \
        if (!pr.before(name)) return hip_fail(hipGetLastError(), "event record");  \
        call;                                                                      \
        e = hipGetLastError();                                                     \
        if (e != hipSuccess) return hip_fail(e, name);                             \
        if (!pr.after()) return hip_fail(hipGetLastError(), "event record");       \
    } while (0)

    if (route_fused(L, T)) {
        MOE_LAUNCH("route_partial", launch_route_partial(x, act == MOE_ACT_BF16, L->w_router, T, H, E, w.logits, s));
        MOE_LAUNCH("route_select", launch_route_select(w.logits, bias, T, H, E, k, topk_idx, topk_w, offsets, perm,
                                                       inv, s));
        return MOE_OK;
    }
    MOE_LAUNCH("route_logits", launch_route_logits(x, act == MOE_ACT_BF16, L->w_router, bias, T, H, E, w.logits, s));
    if (route_small(L, T)) {
        MOE_LAUNCH("route_select_small", launch_route_select_small(w.logits, T, E, k, topk_idx, topk_w, offsets, perm, inv, s));
    } else {
        MOE_LAUNCH("route_topk", launch_route_topk(w.logits, bias, T, H, E, k, topk_idx, topk_w, s));
        MOE_LAUNCH("route_rank", launch_route_rank(topk_idx, T, E, k, w.rank, w.tile_counts, s));
        MOE_LAUNCH("route_scan", launch_route_scan(T, E, k, w.tile_counts, offsets, s));
        MOE_LAUNCH("route_scatter", launch_route_scatter(topk_idx, w.rank, w.tile_counts, offsets, T, E, k, perm, inv, s));
    }
#undef MOE_LAUNCH
    return MOE_OK;
}

int moe_expert_ffn_decode(const moe_layer *L, const void *x, int act, int T, const int32_t *topk_idx,
                          const float *topk_w, const int32_t *offsets, const int32_t *perm, const int32_t *inv,
                          float *y, void *ws, size_t ws_bytes, void *stream, moe_profile *prof)
{
    return ffn_common(L, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, ws, ws_bytes, stream, prof, false, true);
}

int moe_expert_ffn_decode_noalloc(const moe_layer *L, const void *x, int act, int T, const int32_t *topk_idx,
                                  const float *topk_w, const int32_t *offsets, const int32_t *perm,
                                  const int32_t *inv, float *y, void *stream, moe_profile *prof)
{
    int rc = check_layer(L);
    if (rc) return rc;
    if (T < 0) return set_error(MOE_ERR_INVALID_ARG, "T=%d < 0", T);
    if (prof) prof->n_launches = 0;
    if (T == 0) return MOE_OK;
    const size_t need = ffn_ws_bytes(L, T, false);
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return set_error(MOE_ERR_WORKSPACE, "decode of T=%d needs %zu workspace bytes, more than the %d of the "
                         "no-allocation scratch", T, need, MOE_NOALLOC_SCRATCH_BYTES);
    void *ws = scratch_address();
    if (!ws) return MOE_ERR_HIP;
    return ffn_common(L, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, ws, MOE_NOALLOC_SCRATCH_BYTES, stream,
                      prof, false);
}

int moe_layer_decode(const moe_layer *L, const void *x, int act, int T, const float *bias, int32_t *topk_idx,
                     float *topk_w, int32_t *offsets, int32_t *perm, int32_t *inv, float *y, void *ws,
                     size_t ws_bytes, void *stream, moe_profile *prof)
{
    int rc = check_layer(L);
    if (rc) return rc;
    if (L->expert_slot)
        return set_error(MOE_ERR_UNSUPPORTED, "moe_layer_decode takes a resident layer; with an expert cache view "
                         "call moe_route, moe_expert_cache_map, then moe_expert_ffn_decode");
    if (T < 0) return set_error(MOE_ERR_INVALID_ARG, "T=%d < 0", T);
    if (act != MOE_ACT_F32 && act != MOE_ACT_BF16) return set_error(MOE_ERR_INVALID_ARG, "act=%d unknown", act);
    if (prof) prof->n_launches = 0;
    if (T == 0) return MOE_OK;
    if (!x || !topk_idx || !topk_w || !offsets || !perm || !inv || !y) return set_error(MOE_ERR_INVALID_ARG, "NULL tensor argument");
    if (!ws) return set_error(MOE_ERR_INVALID_ARG, "workspace is NULL");
    if ((uintptr_t)x % 16 || (uintptr_t)y % 16 || (uintptr_t)ws % 16)
        return set_error(MOE_ERR_INVALID_ARG, "x, y and the workspace must be 16-byte aligned");
    if ((int64_t)T * L->top_k > (1 << 30)) return set_error(MOE_ERR_INVALID_ARG, "T*k too large");
    const size_t need = layer_ws_bytes(L, T);
    if (ws_bytes < need) return set_error(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    const size_t rbytes = align_up(route_ws(L, T, nullptr).bytes);
    char *fws = (char *)ws + rbytes;
    if (!layer_fused(L, T, act)) {
        // the router's launches, then the decode FFN's, on the two parts of the
        // workspace; the FFN's launches are numbered after the router's
        rc = moe_route(L, x, act, T, bias, topk_idx, topk_w, offsets, perm, inv, ws, rbytes, stream, prof);
        if (rc) return rc;
        moe_profile fp{}, *fpp = nullptr;
        const int nr = prof ? prof->n_launches : 0;
        if (prof) {
            fp = *prof;
            fp.kernel = prof->kernel - nr;
            fpp = &fp;
        }
        rc = ffn_common(L, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, fws, ws_bytes - rbytes, stream, fpp,
                        false, true);
        if (prof) {
            prof->n_launches = nr + fp.n_launches;
            if (fp.kernel >= 0 && fp.kernel < fp.n_launches) prof->name = fp.name;
        }
        return rc;
    }
    FfnWs w = ffn_ws(L, 1, false, true, fws);
    DecPass d = single_pass(L, w, act);
    d.x = x; d.y = y;
    d.topk_idx = topk_idx; d.topk_w = topk_w; d.offsets = offsets; d.inv = inv;
    d.route = 1;
    d.wr = L->w_router; d.bias = bias;
    d.rpart = route_ws(L, 1, (char *)ws).logits;
    d.rnc = route_decode_chunks(1, L->hidden);
    const int steps = (L->hidden + 255) / 256;
    d.rhc = ((steps + d.rnc - 1) / d.rnc) * 256;
    d.o_idx = topk_idx; d.o_w = topk_w; d.o_off = offsets; d.o_perm = perm; d.o_inv = inv;
    dec_plan(d);
    dec_plan_staged(d);
    Prof pr{prof, (hipStream_t)stream};
    return launch_staged(d, pr);
}

int moe_expert_ffn_prefill(const moe_layer *L, const void *x, int act, int T, const int32_t *topk_idx,
                           const float *topk_w, const int32_t *offsets, const int32_t *perm, const int32_t *inv,
                           float *y, void *ws, size_t ws_bytes, void *stream, moe_profile *prof)
{
    return ffn_common(L, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, ws, ws_bytes, stream, prof, true);
}

int q2_unpack(int fmt, const void *packed_dev, int64_t rows, int K, const int8_t *codebook_dev, float *out_dev,
              void *stream)
{
    if (!fmt_ok(fmt)) return set_error(MOE_ERR_INVALID_ARG, "fmt=%d unknown", fmt);
    if (rows < 0 || K < 1) return set_error(MOE_ERR_INVALID_ARG, "rows=%lld K=%d", (long long)rows, K);
    if (rows == 0) return MOE_OK;
    if (!packed_dev || !out_dev) return set_error(MOE_ERR_INVALID_ARG, "NULL tensor argument");
    if ((fmt == MOE_FMT_CB2 || fmt == MOE_FMT_CB2S) && !codebook_dev)
        return set_error(MOE_ERR_INVALID_ARG, "CB2 needs a codebook, CB2S its grid");
    if (rows * nblocks(K) * 8 > ((int64_t)1 << 40)) return set_error(MOE_ERR_INVALID_ARG, "too large");
    hipError_t e = launch_unpack(fmt, (const uint8_t *)packed_dev, rows, K, codebook_dev, out_dev, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "q2_unpack launch");
    return MOE_OK;
}

// ------------------------------------------------------------ expert streaming
namespace {

struct CacheLayout {
    int64_t gate_bytes, down_bytes;
    size_t o_sg, o_su, o_sd, o_slot_of, o_key_of, o_stamp, o_ctl, o_stats, bytes;
};

bool cache_layout(const moe_layer *L, int n_layers, int n_slots, CacheLayout &c)
{
    if (!L || check_layer(L) || n_slots < 1 || n_slots > CACHE_MAX_SLOTS || n_layers < 1 ||
        (int64_t)n_layers * L->n_experts >= ((int64_t)1 << 24))
        return false;
    c.gate_bytes = (int64_t)L->inter * nblocks(L->hidden) * bbytes(L->fmt_gate_up);
    c.down_bytes = (int64_t)L->hidden * nblocks(L->inter) * bbytes(L->fmt_down);
    if (c.gate_bytes % 16 || c.down_bytes % 16) return false;      // copied in 16-byte pieces (H, I % 8 == 0 give it)
    size_t off = 0;
    c.o_sg = off; off = align_up(off + (size_t)n_slots * c.gate_bytes);
    c.o_su = off; off = align_up(off + (size_t)n_slots * c.gate_bytes);
    c.o_sd = off; off = align_up(off + (size_t)n_slots * c.down_bytes);
    c.o_slot_of = off; off = align_up(off + (size_t)n_layers * L->n_experts * sizeof(int32_t));
    c.o_key_of = off; off = align_up(off + (size_t)n_slots * sizeof(int32_t));
    c.o_stamp = off; off = align_up(off + (size_t)n_slots * sizeof(uint32_t));
    c.o_ctl = off; off = align_up(off + (size_t)cache_ctl_len(L->n_experts) * sizeof(int32_t));
    c.o_stats = off; off = align_up(off + 4 * sizeof(uint64_t));
    c.bytes = off;
    return true;
}

// the device address of host memory the GPU may read (pinned, mapped)
int mapped(const void *host, const void **dev, const char *what)
{
    void *d = nullptr;
    const hipError_t e = hipHostGetDevicePointer(&d, const_cast<void *>(host), 0);
    if (e != hipSuccess || !d) {
        (void)hipGetLastError();
        return set_error(MOE_ERR_INVALID_ARG, "%s is not pinned host memory the GPU can read (%s)", what,
                         hipGetErrorString(e));
    }
    *dev = d;
    return MOE_OK;
}

// resolve `n` expert ids of layer `layer_id` and fetch the misses
int cache_load(moe_expert_cache *c, int layer_id, const moe_layer *H, const int32_t *ids, int n, void *stream)
{
    if (!c || !H || !ids) return set_error(MOE_ERR_INVALID_ARG, "NULL cache, layer or expert ids");
    int rc = check_layer(H);
    if (rc) return rc;
    if (H->hidden != c->hidden || H->inter != c->inter || H->n_experts != c->n_experts ||
        H->fmt_gate_up != c->fmt_gate_up || H->fmt_down != c->fmt_down)
        return set_error(MOE_ERR_INVALID_ARG, "the layer's shape or formats differ from the cache's");
    if (layer_id < 0 || layer_id >= c->n_layers)
        return set_error(MOE_ERR_INVALID_ARG, "layer_id=%d outside [0, %d)", layer_id, c->n_layers);
    if (n < 0) return set_error(MOE_ERR_INVALID_ARG, "%d expert ids", n);
    if (std::min(n, c->n_experts) > c->n_slots)
        return set_error(MOE_ERR_UNSUPPORTED, "a call may need %d experts, the cache has %d slots",
                         std::min(n, c->n_experts), c->n_slots);
    const void *hg, *hu, *hd;
    if ((rc = mapped(H->w_gate, &hg, "w_gate")) || (rc = mapped(H->w_up, &hu, "w_up")) ||
        (rc = mapped(H->w_down, &hd, "w_down")))
        return rc;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_cache_resolve(ids, n, c->n_experts, c->n_slots, layer_id * c->n_experts, c->slot_of,
                                        c->key_of, c->stamp, c->ctl, c->stats, 2 * c->gate_bytes + c->down_bytes, s);
    if (e != hipSuccess) return hip_fail(e, "cache resolve launch");
    e = launch_cache_fetch(c->ctl, (const uint8_t *)hg, (const uint8_t *)hu, (const uint8_t *)hd,
                           (uint8_t *)c->slots_gate, (uint8_t *)c->slots_up, (uint8_t *)c->slots_down,
                           c->gate_bytes, c->down_bytes, s);
    if (e != hipSuccess) return hip_fail(e, "cache fetch launch");
    return MOE_OK;
}

}  // namespace

size_t moe_expert_cache_bytes(const moe_layer *L, int n_layers, int n_slots)
{
    CacheLayout c;
    return cache_layout(L, n_layers, n_slots, c) ? c.bytes : 0;
}

int moe_expert_cache_init(moe_expert_cache *c, const moe_layer *L, int n_layers, int n_slots, void *dev,
                          size_t dev_bytes, void *stream)
{
    if (!c || !L) return set_error(MOE_ERR_INVALID_ARG, "NULL cache or layer");
    int rc = check_layer(L);
    if (rc) return rc;
    CacheLayout lay;
    if (!cache_layout(L, n_layers, n_slots, lay))
        return set_error(MOE_ERR_INVALID_ARG, "n_layers=%d n_slots=%d (1..%d slots, n_layers * n_experts < 2^24)",
                         n_layers, n_slots, CACHE_MAX_SLOTS);
    if (!dev || (uintptr_t)dev % ALIGN) return set_error(MOE_ERR_INVALID_ARG, "device memory NULL or not 256-byte aligned");
    if (dev_bytes < lay.bytes) return set_error(MOE_ERR_WORKSPACE, "cache memory %zu < %zu bytes", dev_bytes, lay.bytes);
    char *b = (char *)dev;
    moe_expert_cache x{};
    x.n_layers = n_layers; x.n_experts = L->n_experts; x.n_slots = n_slots;
    x.hidden = L->hidden; x.inter = L->inter; x.fmt_gate_up = L->fmt_gate_up; x.fmt_down = L->fmt_down;
    x.gate_bytes = lay.gate_bytes; x.down_bytes = lay.down_bytes;
    x.slots_gate = b + lay.o_sg; x.slots_up = b + lay.o_su; x.slots_down = b + lay.o_sd;
    x.slot_of = (int32_t *)(b + lay.o_slot_of);
    x.key_of = (int32_t *)(b + lay.o_key_of);
    x.stamp = (uint32_t *)(b + lay.o_stamp);
    x.ctl = (int32_t *)(b + lay.o_ctl);
    x.stats = (uint64_t *)(b + lay.o_stats);
    const hipError_t e = launch_cache_clear(x.slot_of, (int64_t)n_layers * L->n_experts, x.key_of, x.stamp, n_slots,
                                            x.ctl, cache_ctl_len(L->n_experts), x.stats, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "cache clear launch");
    *c = x;
    return MOE_OK;
}

int moe_expert_cache_map(moe_expert_cache *c, int layer_id, const moe_layer *host_layer, const int32_t *topk_idx,
                         int T, moe_layer *view, void *stream)
{
    if (!view) return set_error(MOE_ERR_INVALID_ARG, "NULL view");
    if (!host_layer) return set_error(MOE_ERR_INVALID_ARG, "NULL layer");
    if (T < 0 || (int64_t)T * host_layer->top_k > (1 << 30)) return set_error(MOE_ERR_INVALID_ARG, "T=%d", T);
    int rc = cache_load(c, layer_id, host_layer, topk_idx, T * host_layer->top_k, stream);
    if (rc) return rc;
    *view = *host_layer;
    view->w_gate = c->slots_gate;
    view->w_up = c->slots_up;
    view->w_down = c->slots_down;
    view->expert_slot = c->slot_of + (size_t)layer_id * c->n_experts;
    return MOE_OK;
}

int moe_expert_cache_prefetch(moe_expert_cache *c, int layer_id, const moe_layer *host_layer,
                              const int32_t *experts_dev, int n, void *stream)
{
    return cache_load(c, layer_id, host_layer, experts_dev, n, stream);
}

int moe_probe_stream_read(const void *buf, size_t bytes, int grid, int nontemporal, void *sink, void *stream)
{
    if (!buf || !sink) return set_error(MOE_ERR_INVALID_ARG, "NULL pointer");
    if (bytes == 0 || bytes % 16 || (uintptr_t)buf % 16 || (uintptr_t)sink % 16)
        return set_error(MOE_ERR_INVALID_ARG, "bytes=%zu and both pointers must be 16-byte multiples", bytes);
    if (grid < 1 || grid > 65536) return set_error(MOE_ERR_INVALID_ARG, "grid=%d outside [1, 65536]", grid);
    hipError_t e = launch_probe_stream(buf, bytes, grid, nontemporal, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moe_probe_stream_read launch");
    return MOE_OK;
}

int moe_probe_mfma_loop(int shape, int grid, int iters, float *sink, void *stream)
{
    if (!sink) return set_error(MOE_ERR_INVALID_ARG, "NULL pointer");
    if (shape != 0 && shape != 1) return set_error(MOE_ERR_INVALID_ARG, "shape=%d must be 0 or 1", shape);
    if (grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 24))
        return set_error(MOE_ERR_INVALID_ARG, "grid=%d or iters=%d out of range", grid, iters);
    hipError_t e = launch_probe_mfma(shape, grid, iters, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moe_probe_mfma_loop launch");
    return MOE_OK;
}

}  // extern "C"
