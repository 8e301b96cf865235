/*
 * moe.h -- C ABI of the routed-MoE expert layer with 2-bit routed experts,
 * for one AMD Instinct MI355X (gfx950).
 *
 * The layer (one MoE FFN of a DeepSeek-V3/V4-class model) is
 *
 *   y[t] = FFN_sh(x_t) + sum_{j<k} w[t,j] * FFN_{e(t,j)}(x_t),
 *   FFN_e(x) = W_down,e ( silu(W_gate,e x) * (W_up,e x) ),
 *
 * where only the routed experts are quantized: gate/up in a 2-bit codebook
 * format (CB2), down in Q2_K (or all three in Q4_K); the shared expert and the
 * router stay unquantized.  This split follows the pages: "DwarfStar" README
 * and the "ds4" README mirror, sections on model weights (only routed experts
 * quantized, up/gate IQ2_XXS, down Q2_K, everything else unchanged); deep-dive
 * article on DwarfStar, section 3.4.3 (quantization tree; router kept at high
 * precision).  The pages give no bit layout; the block layouts are defined
 * below and are this library's own.
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device memory owned by the caller.  The library
 *    allocates no device memory: scratch comes from the caller's workspace
 *    `ws`, sized with moe_workspace_bytes().  Host pointers are marked "host".
 *    The one object it creates is a second stream with two events per device
 *    for batched decode (see moe_expert_ffn_decode).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise or read device data back to the host.
 *  - Arguments are validated on the host before any HIP call; a bad argument
 *    returns a negative moe_status and launches nothing.  A failed launch
 *    returns MOE_ERR_HIP; moe_last_error() gives the detail for the calling
 *    thread.  No entry point aborts or throws.
 *  - T == 0 returns MOE_OK without launching.
 *  - Non-finite inputs are caller error: results are then unspecified but
 *    every access stays in bounds.
 *  - Calls on one stream run in order; calls on different streams that share
 *    a workspace or an output race.
 *  - Thread safety: every entry point may be called from several host threads
 *    at once (on one device or several).  The only state the library keeps
 *    between calls is (a) the last error text, per thread, (b) per-device
 *    caches of launch facts -- a kernel's raised dynamic-LDS limit, its
 *    resident work-groups per CU, the device's CU count and the device
 *    address of the no-allocation scratch array -- each computed on first use
 *    on a device, stored atomically and never changed afterwards except
 *    upwards (the LDS limit), so a racing caller at most repeats the query,
 *    (c) the contents of that scratch array (see
 *    moe_expert_ffn_decode_noalloc), and (d) per device, the second stream
 *    and two events of batched decode, created on the first call that uses
 *    them and kept until the process ends; a call enqueues its fork and join
 *    on them under a mutex (held only while it enqueues), so concurrent
 *    callers each join their own work.  No entry point allocates device
 *    memory; no other lock is held.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status */
enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, bad size, k > E, ...          */
    MOE_ERR_UNSUPPORTED = -2,   /* valid but not implemented (format / path)   */
    MOE_ERR_WORKSPACE = -3,     /* ws_bytes smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = -4            /* a HIP launch or runtime call failed         */
};

/* ------------------------------------------------------------ formats
 * A quantized matrix [rows][K] is stored row by row; each row holds
 * nb = ceil(K/256) blocks of 256 consecutive weights (a row whose K is not a
 * multiple of 256 is zero-padded).  Little-endian fields:
 *
 * MOE_FMT_CB2  38 B/block: [0:2) fp16 d | [2:6) eight 4-bit sub-block scales,
 *   s_j in bits 4*(j%2).. of byte 2+j/2 | [6:38) 32 one-byte codebook indices,
 *   one per group of 8 weights.  w[8g+i] = d * s_{g/4} * C[idx_g][i], with C
 *   a caller-supplied int8 codebook [256][8] of values in {-3,-1,1,3}.
 * MOE_FMT_CB2S 66 B/block (2.0625 bits per weight, the byte budget of the
 *   pages' IQ2_XXS, with a sign field): [0:2) fp16 d | eight 8-byte
 *   sub-block records at [2+8j, 10+8j): bytes 0..3 the grid indices of groups
 *   4j..4j+3; bytes 4..7 a little-endian word with, for group 4j+u, the
 *   negative flags of its weights 0..6 at bits 7u..7u+6, and s_j at bits
 *   28..31.  Weight 7's flag is the parity of the other seven (an even
 *   number of negatives per group).  w[8g+i] = d * s_{g/4} * (-1)^neg *
 *   G[idx_g][i], with G a caller-supplied uint8 grid [256][8] of magnitudes
 *   (the synthetic workloads use values in {1,3,5}; any up to 15 are exact).
 * MOE_FMT_Q2K  84 B/block: [0:2) fp16 d | [2:4) fp16 dmin | [4:20) byte j =
 *   sc_j | m_j<<4 for 16 sub-blocks of 16 | [20:84) 2-bit q_i in bits
 *   2*(i%4) of byte i/4.  w_i = d*sc_j*q_i - dmin*m_j, j = i/16.
 * MOE_FMT_Q4K 144 B/block: [0:2) d | [2:4) dmin | [4:16) sixteen 6-bit
 *   fields at bits 6n..6n+5 of one little-endian 96-bit stream (n<8: sc_n,
 *   n>=8: m_{n-8}) | [16:144) 4-bit q_i in bits 4*(i%2) of byte i/2.
 *   w_i = d*sc_j*q_i - dmin*m_j, j = i/32.
 * MOE_FMT_Q5K 176 B/block: Q4_K with 5-bit codes: [0:16) as Q4_K |
 *   [16:144) the low 4 bits of q_i in bits 4*(i%2) of byte 16+i/2 |
 *   [144:176) bit 4 of q_i in bit i%8 of byte 144+i/8.
 *   w_i = d*sc_j*q_i - dmin*m_j, j = i/32.
 * MOE_FMT_Q6K 210 B/block: [0:2) fp16 d | [2:18) sixteen int8 scales sc_j
 *   (16 sub-blocks of 16) | [18:146) the low 4 bits of u_i = q_i + 32 in
 *   bits 4*(i%2) of byte 18+i/2 | [146:210) the high 2 bits of u_i in bits
 *   2*(i%4) of byte 146+i/4.  w_i = d*sc_j*q_i, q_i in -32..31, j = i/16.
 *   (Q5_K and Q6_K are among the routed layouts the "ds4" README mirror lists
 *   for other models' files, section on model weights.)
 * MOE_FMT_BF16 plain row-major bf16 (the shared expert), no blocks.
 *
 * Every dequantized value is exact in fp32 (products need at most 24
 * significant bits; the min term is subtracted with one rounding). */
enum moe_format { MOE_FMT_CB2 = 1, MOE_FMT_Q2K = 2, MOE_FMT_Q4K = 3, MOE_FMT_BF16 = 4, MOE_FMT_Q5K = 5,
                  MOE_FMT_Q6K = 6, MOE_FMT_CB2S = 7 };

/* activation element type of x */
enum moe_act { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 };

/* workspace query paths */
enum moe_path { MOE_PATH_ROUTE = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2, MOE_PATH_LAYER_DECODE = 3 };

/* One MoE layer.  The struct itself lives in host memory; every pointer in
 * it is device memory.
 *   hidden (H), inter (I), n_experts (E), top_k (k): 1 <= k <= E <= 1024,
 *     H % 8 == 0, I % 8 == 0.
 *   fmt_gate_up: MOE_FMT_CB2, CB2S, Q2K, Q4K or Q5K; fmt_down: MOE_FMT_Q2K,
 *     Q4K, Q5K or Q6K.  (CB2 or Q4K gate/up with Q2K or Q4K down run on any shape; the
 *     other pairs need hidden, inter and sh_inter multiples of 512, else the
 *     FFN calls return MOE_ERR_UNSUPPORTED.)
 *   w_gate, w_up: [E][I rows][ceil(H/256) blocks]; w_down: [E][H rows][ceil(I/256)
 *     blocks]; experts stored back to back with no gaps.
 *   codebook: int8 [256][8] codebook for CB2, the uint8 [256][8] magnitude
 *     grid (passed through this pointer) for CB2S, else may be NULL.
 *   sh_inter: intermediate size of the bf16 shared expert, 0 if there is none
 *     (then sh_* are ignored); sh_gate, sh_up: [sh_inter][H] bf16; sh_down:
 *     [H][sh_inter] bf16; sh_inter % 256 == 0 and H % 256 == 0 when present.
 *   w_router: fp32 [E][H].
 *   flags: 0, or MOE_LAYER_TOKENWISE_DECODE: decode computes every token of a
 *     batch with the single-token kernels, one token after another, so each
 *     token's y is bit-identical to decoding it alone whatever batch it
 *     arrives in -- the property the pages' serving layer holds batched
 *     decode to ("Part 5: 服务层", section 6: a batched step returns exactly
 *     what running each session alone returns) -- at the single-token cost
 *     per token (about 60 us at H=7168, I=2048, k=8, against about 26 us per
 *     token for a 32-token batch on the grouped GEMMs).  Without it, batches
 *     of up to 4 tokens still run token by token and larger ones on the
 *     grouped GEMMs, which agree with the single-token result to about 1e-6
 *     relative, not bit for bit.  It needs a layer the single-token kernels
 *     take (CB2 gate/up, Q2K down; see moe_expert_ffn_decode), otherwise
 *     decode returns MOE_ERR_UNSUPPORTED.
 *     MOE_LAYER_ONE_STREAM (may be combined with the other): every launch of
 *     a call stays on the caller's stream; batched decode otherwise runs the
 *     shared expert's chain on a second stream beside the routed kernels (see
 *     moe_expert_ffn_decode).  For callers that arrange streams themselves
 *     or time each launch on one stream.  Results are the same bit for bit.
 *     Other bits: MOE_ERR_INVALID_ARG.
 *   expert_slot: NULL, or a device int32 [n_experts] map from expert to slot:
 *     the FFN calls then read expert e's routed weights at w_* + expert_slot[e]
 *     * (bytes of one expert's matrix) -- the layer view of an expert cache
 *     (moe_expert_cache_map fills one in; every expert the routing selects
 *     must map to a slot the weight arrays hold).  Nothing else changes:
 *     routing, tiles and sums are those of the resident layer, so y is
 *     bit-identical.  The router and moe_layer_decode's fused single-token
 *     path need the resident layout (moe_layer_decode returns
 *     MOE_ERR_UNSUPPORTED for a view).
 *   Every pointer must be 16-byte aligned (device allocations are); the
 *   kernels read weights and the codebook in 8- and 16-byte pieces. */
#define MOE_LAYER_TOKENWISE_DECODE 1
#define MOE_LAYER_ONE_STREAM 2
typedef struct moe_layer {
    int32_t hidden, inter, n_experts, top_k;
    int32_t fmt_gate_up, fmt_down;
    int32_t sh_inter, flags;
    const void *w_gate, *w_up, *w_down;
    const int8_t *codebook;
    const void *sh_gate, *sh_up, *sh_down;
    const float *w_router;
    const int32_t *expert_slot;
} moe_layer;

/* Optional per-kernel timing.  When `prof` is non-NULL and prof->kernel is
 * the 0-based index of one of the kernel launches a call makes, the library
 * records hipEvent_t prof->ev_start immediately before that launch and
 * prof->ev_stop immediately after it, on the stream the launch runs on (the
 * call's stream; the second stream for the shared expert's launches of
 * batched decode, whose interval then spans the routed kernels beside them
 * as well); it always stores
 * the number of launches the call made in prof->n_launches and the kernel's
 * name in prof->name.  Events are created and destroyed by the caller. */
typedef struct moe_profile {
    int32_t kernel;
    int32_t n_launches;
    void *ev_start, *ev_stop;
    const char *name;
} moe_profile;

/* ------------------------------------------------------------ routing
 * moe_route: router scores, top-k selection and grouping (device side).
 *   l[t,e] = sum_h x[t,h]*W_r[e,h] + bias[e]      (accumulated in fp64)
 *   topk_idx[t,0..k) = the k largest l[t,:], descending, ties to the lower e
 *   topk_w[t,j] = s_j / sum_j' s_j',  s = 1/(1+exp(-l))   (fp64, stored fp32)
 *   offsets[E+1]: exclusive prefix sum of per-expert assignment counts
 *   perm[T*k]: assignment ids a = t*k+j sorted by (expert, token)
 *   inv[T*k]: inv[a] = position of a in perm
 * The router is kept at full precision, as the pages do (deep-dive article,
 * section 3.4.3; section 9.2 on routing quality); the function (sigmoid,
 * top-k, renormalised weights) is the workload's definition.
 * x: [T][H] of type `act` (device).  bias: fp32 [E] or NULL.  All outputs are
 * device arrays of the sizes shown.  x, L->w_router and ws must be 16-byte
 * aligned (MOE_ERR_INVALID_ARG otherwise).  Launches: for T <= 64 and k <= 64 fp64
 * partial logits, then one work-group that selects and groups; otherwise
 * logits, then top-k, rank, scan and scatter. */
int moe_route(const moe_layer *L, const void *x, int act, int T, const float *bias,
              int32_t *topk_idx, float *topk_w, int32_t *offsets, int32_t *perm, int32_t *inv,
              void *ws, size_t ws_bytes, void *stream, moe_profile *prof);

/* ------------------------------------------------------------ expert FFN
 * Both compute y [T][H] fp32 (overwritten) = shared expert + routing-weighted
 * sum of the k routed expert FFNs (SwiGLU), from the routing that moe_route
 * produced.  Inputs as in moe_route; x, y and ws must be 16-byte aligned
 * (MOE_ERR_INVALID_ARG otherwise).  One call handles at most 2^31 - 1
 * activation elements per operand (T*H, and (T*k + T)*max(I, sh_inter)):
 * larger T returns MOE_ERR_UNSUPPORTED (split the batch).
 *
 * moe_expert_ffn_decode -- fp32-accurate path meant for small T (any T works):
 *   weights applied exactly (integer codes as exact bf16 MFMA operands, or,
 *   for the single-token gate/up, through fp32 tables of codeword . x
 *   products; fp32 block rescale), activations exact (bf16) or split into two
 *   bf16 terms (fp32), fp32 accumulation, intermediate h in fp32
 *   (single-token path: h held as two bf16 terms).  Relative L2 error against
 *   an exact evaluation is far below 1e-4.  Formats: every pair the layer
 *   struct allows; anything but CB2 gate/up with Q2K down needs hidden, inter
 *   and sh_inter multiples of 512 (MOE_ERR_UNSUPPORTED otherwise; Q4K/Q5K/Q6K
 *   codes enter as sc*q split exactly into two bf16 terms).  Launches: for
 *   T <= 4 (any T with MOE_LAYER_TOKENWISE_DECODE) with CB2 gate/up and Q2K
 *   down (and H % 512 == 0, H <= 8192, I % 256 == 0, I <= 2048,
 *   sh_inter % 512 == 0, k <= 64) per token, in order: for k <= 8 and
 *   sh_inter <= 2048 four launches -- the shared gate/up; the routed gate/up
 *   beside the shared down; routed h; the routed down, which adds the shared
 *   output and writes y -- else gate/up, down (SwiGLU as it forms h) and
 *   combine; so such a token's y does not depend on the other tokens of the
 *   call.  Otherwise schedule, gate/up+SwiGLU, down, combine; for CB2/CB2S
 *   gate/up with Q2K down, T <= 64, a shared expert and hidden, inter and
 *   sh_inter multiples of 512, the routed tiles' gate/up and down run on
 *   `stream` while the shared expert's gate/up, its K-part finalize and its
 *   down run on the library's second stream of the device, forked from
 *   `stream` after the schedule and joined back before the combine (events;
 *   a graph capture of `stream` captures both branches; the first such call
 *   on a device creates the stream, so make one call before capturing).  If
 *   the stream cannot be created, every launch stays on `stream`.  The results are
 *   those of one stream, bit for bit; moe_expert_ffn_decode_noalloc, and a
 *   layer with MOE_LAYER_ONE_STREAM, keep every launch on `stream`.
 * moe_expert_ffn_prefill -- bf16 MFMA path for any T: x must be bf16;
 *   dequantized weights rounded to bf16 (RNE) in LDS; fp32 accumulation;
 *   h rounded to bf16; down output and combine in fp32.  Relative L2 error
 *   below 5e-3.  Formats: every pair the layer struct allows (see there for
 *   the shapes each needs), BF16 shared.
 *   Launches: schedule, gate/up+SwiGLU, down, combine. */
int moe_expert_ffn_decode(const moe_layer *L, const void *x, int act, int T,
                          const int32_t *topk_idx, const float *topk_w, const int32_t *offsets,
                          const int32_t *perm, const int32_t *inv, float *y,
                          void *ws, size_t ws_bytes, void *stream, moe_profile *prof);
int moe_expert_ffn_prefill(const moe_layer *L, const void *x, int act, int T,
                           const int32_t *topk_idx, const float *topk_w, const int32_t *offsets,
                           const int32_t *perm, const int32_t *inv, float *y,
                           void *ws, size_t ws_bytes, void *stream, moe_profile *prof);

/* ------------------------------------------------------------ fused layer decode
 * moe_layer_decode (+): moe_route followed by moe_expert_ffn_decode in one
 * call, with the same arguments and outputs as the two (the routing outputs
 * are written too) and one workspace of moe_workspace_bytes(L, T,
 * MOE_PATH_LAYER_DECODE) bytes.  For one token of a layer the single-token
 * decode kernels take (CB2 gate/up, Q2K down, H % 512 == 0, H <= 8192,
 * I % 256 == 0, I <= 2048, sh_inter % 512 == 0, sh_inter <= 2048, k <= 8,
 * E <= 1024), the router runs inside the FFN's launches: the first launch
 * computes the fp64 partial logits beside the shared expert's gate/up, which
 * does not depend on the routing, and every work-group of the routed gate/up
 * launch selects the experts itself (the same arithmetic as moe_route, so
 * the routing and y are bit-identical to the two separate calls).  Four
 * launches instead of six: decode reads every weight once per token while
 * compute idles, so the shorter chain of dependent launches is what it buys
 * ("Part 5: 服务层", section 6).  Otherwise it runs moe_route and
 * moe_expert_ffn_decode.  Errors as in those two. */
int moe_layer_decode(const moe_layer *L, const void *x, int act, int T, const float *bias, int32_t *topk_idx,
                     float *topk_w, int32_t *offsets, int32_t *perm, int32_t *inv, float *y, void *ws,
                     size_t ws_bytes, void *stream, moe_profile *prof);

/* ------------------------------------------------------------ no-allocation decode
 * moe_expert_ffn_decode_noalloc: for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results (bit for bit) as
 * moe_expert_ffn_decode, without `ws`: the workspace is a fixed array inside
 * the library, MOE_NOALLOC_SCRATCH_BYTES (32 MiB) of device memory on each
 * device the library runs on, held until the process ends (enough for decode
 * batches of about 60 tokens at H=7168, I=2048, k=8; 17 MiB at T=32).
 * A call whose moe_workspace_bytes(L, T, MOE_PATH_DECODE) exceeds it returns
 * MOE_ERR_WORKSPACE and launches nothing.  The call allocates nothing (no
 * hipMalloc, no allocating library routine); on the first call on a device it
 * looks up the array's device address once.  Every call on one device shares
 * that device's array and leaves its contents behind: the decode kernels write
 * every workspace byte before they read it, so nothing needs clearing, but
 * calls that overlap in time on one device (different streams, or threads
 * whose calls are not ordered on one stream) race on it. */
#define MOE_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int moe_expert_ffn_decode_noalloc(const moe_layer *L, const void *x, int act, int T,
                                  const int32_t *topk_idx, const float *topk_w, const int32_t *offsets,
                                  const int32_t *perm, const int32_t *inv, float *y, void *stream,
                                  moe_profile *prof);

/* ------------------------------------------------------------ expert streaming
 * An HBM-resident cache of routed-expert slots for layers whose routed
 * weights live in pinned host memory: the non-routed weights (router, shared
 * expert, codebook) stay resident, each slot holds one whole expert (gate, up
 * and down), and a miss is copied from host memory into a slot by the GPU
 * itself, with no host round trip -- the MI355X form of the pages' streaming
 * mode, which keeps routed experts in a cache of dynamic expert slots and
 * loads them on a miss ("DwarfStar" README and the "ds4" README mirror,
 * section on running models larger than RAM).
 *
 * moe_expert_cache_bytes: device bytes a cache of n_slots slots for n_layers
 *   layers of L's geometry (hidden, inter, n_experts, formats) needs; 0 if
 *   invalid (1 <= n_slots <= 8192, 1 <= n_layers, n_layers * n_experts <
 *   2^24).
 * moe_expert_cache_init: carve the cache out of dev (dev_bytes >= the size
 *   above, 256-byte aligned; owned by the caller, which keeps it alive and
 *   must not touch it while the cache is in use) and clear it on `stream`
 *   (every slot empty).  Fills *c (host memory).
 * moe_expert_cache_map: for layer layer_id, make every expert that
 *   topk_idx [T][k] (device, from moe_route) selects resident, and fill *view
 *   with the layer view the FFN calls take: host_layer with w_gate, w_up,
 *   w_down set to the slot arrays and expert_slot to the layer's slot map.
 *   host_layer is the layer with its routed weights in pinned host memory
 *   (hipHostMalloc; device-accessible), its other pointers in device memory.
 *   On `stream`: one work-group resolves hits and misses and picks victims
 *   -- the least recently used slots not needed by this call, ties to the
 *   lower slot -- then a copy kernel pulls each miss's three matrices from
 *   host memory into its slot.  Needs n_slots >= min(n_experts, T * k) so
 *   that the whole call fits (MOE_ERR_UNSUPPORTED otherwise).
 * moe_expert_cache_prefetch: the same for the n expert ids in experts_dev
 *   (device int32; duplicates allowed), without a view: run it on another
 *   stream to load a layer's experts while the previous layer computes.
 *   Calls on one cache must not overlap in time (one stream, or ordered by
 *   events): they update its slot state.  Overlap loads with compute by
 *   giving consecutive layers their own caches (the pages reserve two full
 *   routed layers for overlapped streaming prefill, same section).
 * c->stats (device uint64 [4]): hits, misses, bytes copied and calls, summed
 *   since init. */
typedef struct moe_expert_cache {
    int32_t n_layers, n_experts, n_slots, hidden, inter, fmt_gate_up, fmt_down, reserved0;
    int64_t gate_bytes, down_bytes;           /* one expert's gate (= up) and down matrix */
    void *slots_gate, *slots_up, *slots_down; /* device [n_slots][bytes] */
    int32_t *slot_of;                         /* device [n_layers][n_experts], -1 = absent */
    int32_t *key_of;                          /* device [n_slots]: layer * n_experts + expert, or -1 */
    uint32_t *stamp;                          /* device [n_slots]: call counter at last use */
    int32_t *ctl;                             /* device: clock, fetch count, fetch list */
    uint64_t *stats;                          /* device [4] */
} moe_expert_cache;
size_t moe_expert_cache_bytes(const moe_layer *L, int n_layers, int n_slots);
int moe_expert_cache_init(moe_expert_cache *c, const moe_layer *L, int n_layers, int n_slots, void *dev,
                          size_t dev_bytes, void *stream);
int moe_expert_cache_map(moe_expert_cache *c, int layer_id, const moe_layer *host_layer, const int32_t *topk_idx,
                         int T, moe_layer *view, void *stream);
int moe_expert_cache_prefetch(moe_expert_cache *c, int layer_id, const moe_layer *host_layer,
                              const int32_t *experts_dev, int n, void *stream);

/* ------------------------------------------------------------ pack / unpack
 * q2_pack (host): quantize a row-major fp32 matrix w_host [rows][K] into
 * out_host (q2_packed_bytes(fmt, rows, K) bytes).  fmt: CB2 (needs
 * codebook_host int8 [256][8]), CB2S (needs the uint8 grid [256][8] there),
 * Q2K, Q4K, Q5K or Q6K.  Quantizer (fp32 arithmetic,
 * round-half-to-even everywhere, fp16 conversion RNE):
 *   Q2_K / Q4_K, per sub-block j (16 / 32 weights): lo = min(0, min w),
 *     hi = max w, scale_j = (hi-lo)/L, mn_j = -lo (L = 3 / 15); per block
 *     d = fp16(max scale_j / S), dmin = fp16(max mn_j / S) (S = 15 / 63);
 *     sc_j = rint(scale_j/d), m_j = rint(mn_j/dmin) clamped to [0,S] (0 if
 *     the divisor is 0); q_i = rint((w_i + dmin*m_j)/(d*sc_j)) clamped to
 *     [0,L] (0 if d*sc_j == 0).
 *   CB2, per sub-block j of 32: sigma_j = max|w|/3; d = fp16(max sigma_j/15);
 *     s_j = rint(sigma_j/d) clamped to [0,15]; per group of 8 with
 *     step = d*s_j > 0: t_i = rint(w_i/step*4096), idx = argmin over the
 *     codebook of the integer distance sum_i (t_i - 4096*C[idx][i])^2, lowest
 *     index on ties (0 when step == 0).
 *   CB2S: as CB2 with sigma_j = max|w|/5 and, per group with step > 0,
 *     magnitude targets a_i = rint(|w_i|/step*4096) and natural signs
 *     neg_i = (w_i < 0); entry c costs sum_i (a_i - 4096*G[c][i])^2 plus, if
 *     the count of negatives is odd, the cheapest single sign flip
 *     min_p 4*a_p*4096*G[c][p] (lowest p on ties); the lowest-cost entry
 *     (lowest index on ties) is chosen and its flip applied (index 0 and no
 *     flags when step == 0).
 *   Q5_K: as Q4_K with L = 31.
 *   Q6_K, per sub-block j of 16: scale_j = max|w|/31; d = fp16(max
 *     scale_j/127); sc_j = rint(scale_j/d) clamped to [0,127] (0 if d == 0);
 *     q_i = rint(w_i/(d*sc_j)) clamped to [-32,31] (0 if d*sc_j == 0).
 * Rows are spread over at most 16 host threads; the bytes do not depend on the thread
 * count.  Returns MOE_OK or MOE_ERR_INVALID_ARG (with moe_last_error() set). */
int q2_pack(int fmt, const float *w_host, int64_t rows, int K, const int8_t *codebook_host,
            void *out_host);

/* q2_unpack (device): dequantize packed_dev [rows][nb blocks] to out_dev fp32
 * [rows][K] (padding dropped), bit-exact with the definitions above.
 * codebook_dev: int8 [256][8] device array for CB2, the uint8 grid for CB2S,
 * else ignored. */
int q2_unpack(int fmt, const void *packed_dev, int64_t rows, int K, const int8_t *codebook_dev,
              float *out_dev, void *stream);

/* ------------------------------------------------------------ helpers */
/* bytes of a packed [rows][K] matrix; 0 for an unknown format */
size_t q2_packed_bytes(int fmt, int64_t rows, int K);
/* workspace bytes for a call of the given path (MOE_PATH_*) with T tokens;
 * 0 if L is invalid.  Sizes grow linearly with T. */
size_t moe_workspace_bytes(const moe_layer *L, int T, int path);
/* static text for a status code */
const char *moe_status_str(int status);
/* detail of the last error on the calling thread ("" if none) */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
