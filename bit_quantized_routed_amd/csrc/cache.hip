// Expert streaming: an HBM-resident cache of routed-expert slots whose misses
// the GPU copies in from pinned host memory.  The routed experts are what a
// model's size is made of, so they are the part kept in a cache of whole-expert
// slots while every other weight stays resident, and a miss loads the expert
// ("DwarfStar" README and the "ds4" README mirror, section on running models
// larger than RAM).  Here the cache is HBM and the backing store host memory;
// both the bookkeeping and the copies run on the device, so a layer call needs
// no host round trip between its routing and its FFN.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "cache.h"
#include "devcache.h"

namespace moe {

namespace {

constexpr int RES_THREADS = 1024;
constexpr int FETCH_THREADS = 256;

__global__ __launch_bounds__(256) void cache_clear_kernel(int32_t *slot_of, int64_t n_keys, int32_t *key_of,
                                                          uint32_t *stamp, int n_slots, int32_t *ctl, int ctl_len,
                                                          uint64_t *stats)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t j = i; j < n_keys; j += stride) slot_of[j] = -1;
    for (int64_t j = i; j < n_slots; j += stride) {
        key_of[j] = -1;
        stamp[j] = 0;
    }
    for (int64_t j = i; j < ctl_len; j += stride) ctl[j] = 0;
    if (i < 4) stats[i] = 0;
}

// One call's bookkeeping, in one work-group so that every decision is made in
// one place and in a fixed order:
//   1. mark the experts the call needs (bitmap in LDS);
//   2. a needed expert with a slot is a hit: its slot's stamp becomes this
//      call's clock; the others are misses, ranked by expert id;
//   3. if there are misses, every slot not used by this call is a candidate,
//      keyed (stamp, slot): the least recently used first, empty slots
//      (stamp 0) before any used one, the lower slot on ties; a bitonic sort
//      in LDS orders them and miss r takes candidate r;
//   4. a victim's old key (any layer) loses its slot; the miss gets it, and
//      the (slot, expert) pair goes to the fetch list.
// The host guarantees n_slots >= the number of distinct experts a call can
// need, so there are always enough candidates.
__global__ __launch_bounds__(RES_THREADS) void cache_resolve_kernel(const int32_t *ids, int n, int E, int n_slots,
                                                                    int P, int key_base, int32_t *slot_of,
                                                                    int32_t *key_of, uint32_t *stamp, int32_t *ctl,
                                                                    uint64_t *stats, int64_t expert_bytes)
{
    extern __shared__ __attribute__((aligned(16))) uint64_t skey[];      // [P] candidate keys
    __shared__ uint32_t needw[CACHE_MAX_EXPERTS / 32], missw[CACHE_MAX_EXPERTS / 32];
    __shared__ int n_hit;
    const int tid = threadIdx.x;
    const int nw = (E + 31) >> 5;
    if (tid < CACHE_MAX_EXPERTS / 32) needw[tid] = missw[tid] = 0;
    if (tid == 0) n_hit = 0;
    __syncthreads();
    for (int a = tid; a < n; a += RES_THREADS) {
        const int e = ids[a];
        if (e >= 0 && e < E) atomicOr(&needw[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    const uint32_t clock = (uint32_t)ctl[0] + 1u;
    int my_hits = 0;
    for (int e = tid; e < E; e += RES_THREADS) {
        if (!((needw[e >> 5] >> (e & 31)) & 1u)) continue;
        const int s = slot_of[key_base + e];
        if (s >= 0) {
            stamp[s] = clock;
            ++my_hits;
        } else {
            atomicOr(&missw[e >> 5], 1u << (e & 31));
        }
    }
    if (my_hits) atomicAdd(&n_hit, my_hits);
    __threadfence_block();
    __syncthreads();
    int m = 0;
    for (int w = 0; w < nw; ++w) m += __builtin_popcount(missw[w]);
    if (m > 0) {                                                       // uniform over the work-group
        for (int i = tid; i < P; i += RES_THREADS)
            skey[i] = (i < n_slots && stamp[i] != clock) ? ((uint64_t)stamp[i] << 32) | (uint32_t)i : ~0ull;
        __syncthreads();
        for (int k = 2; k <= P; k <<= 1)
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < P; i += RES_THREADS) {
                    const int ij = i ^ j;
                    if (ij > i) {
                        const uint64_t a = skey[i], b = skey[ij];
                        if ((a > b) == ((i & k) == 0)) {
                            skey[i] = b;
                            skey[ij] = a;
                        }
                    }
                }
                __syncthreads();
            }
        for (int e = tid; e < E; e += RES_THREADS) {
            const uint32_t bit = 1u << (e & 31);
            if (!(missw[e >> 5] & bit)) continue;
            int r = __builtin_popcount(missw[e >> 5] & (bit - 1u));
            for (int w = 0; w < (e >> 5); ++w) r += __builtin_popcount(missw[w]);
            if (skey[r] == ~0ull) {                                   // no candidate left (never, with
                ctl[CACHE_CTL_HEAD + 2 * r] = -1;                     // the host's slot check): the miss
                ctl[CACHE_CTL_HEAD + 2 * r + 1] = e;                  // stays unmapped, nothing is copied
                continue;
            }
            const int s = (int)(uint32_t)skey[r];
            const int old = key_of[s];
            if (old >= 0) slot_of[old] = -1;
            key_of[s] = key_base + e;
            slot_of[key_base + e] = s;
            stamp[s] = clock;
            ctl[CACHE_CTL_HEAD + 2 * r] = s;
            ctl[CACHE_CTL_HEAD + 2 * r + 1] = e;
        }
    }
    __threadfence_block();
    __syncthreads();
    if (tid == 0) {
        ctl[0] = (int32_t)clock;
        ctl[1] = m;
        stats[0] += (uint64_t)n_hit;
        stats[1] += (uint64_t)m;
        stats[2] += (uint64_t)m * (uint64_t)expert_bytes;
        stats[3] += 1;
    }
}

// Grid-stride copy of the fetch list in 16-byte pieces: piece i of the list
// is piece u = i % U of miss f = i / U (U pieces per expert: gate, up, down
// back to back), so consecutive lanes read consecutive bytes of one matrix.
__global__ __launch_bounds__(FETCH_THREADS) void cache_fetch_kernel(const int32_t *ctl, const uint8_t *hg,
                                                                    const uint8_t *hu, const uint8_t *hd,
                                                                    uint8_t *sg, uint8_t *su, uint8_t *sd,
                                                                    int64_t gate_bytes, int64_t down_bytes)
{
    const int nf = ctl[1];
    const int64_t ug = gate_bytes >> 4, ud = down_bytes >> 4, U = 2 * ug + ud;
    const int64_t total = (int64_t)nf * U;
    for (int64_t i = (int64_t)blockIdx.x * FETCH_THREADS + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * FETCH_THREADS) {
        const int f = (int)(i / U);
        int64_t u = i - (int64_t)f * U;
        const int64_t s = ctl[CACHE_CTL_HEAD + 2 * f], e = ctl[CACHE_CTL_HEAD + 2 * f + 1];
        if (s < 0) continue;
        const uint8_t *src;
        uint8_t *dst;
        if (u < ug) {
            src = hg + e * gate_bytes;
            dst = sg + s * gate_bytes;
        } else if (u < 2 * ug) {
            u -= ug;
            src = hu + e * gate_bytes;
            dst = su + s * gate_bytes;
        } else {
            u -= 2 * ug;
            src = hd + e * down_bytes;
            dst = sd + s * down_bytes;
        }
        ((uint4 *)dst)[u] = ((const uint4 *)src)[u];
    }
}

}  // namespace

hipError_t launch_cache_clear(int32_t *slot_of, int64_t n_keys, int32_t *key_of, uint32_t *stamp, int n_slots,
                              int32_t *ctl, int ctl_len, uint64_t *stats, hipStream_t s)
{
    const int64_t n = std::max<int64_t>(std::max<int64_t>(n_keys, n_slots), ctl_len);
    const int grid = (int)std::min<int64_t>((n + 255) / 256, 1024);
    cache_clear_kernel<<<grid, 256, 0, s>>>(slot_of, n_keys, key_of, stamp, n_slots, ctl, ctl_len, stats);
    return hipGetLastError();
}

hipError_t launch_cache_resolve(const int32_t *ids, int n, int E, int n_slots, int key_base, int32_t *slot_of,
                                int32_t *key_of, uint32_t *stamp, int32_t *ctl, uint64_t *stats,
                                int64_t expert_bytes, hipStream_t s)
{
    int P = 1;
    while (P < n_slots) P <<= 1;
    const int lds = P * (int)sizeof(uint64_t);
    static DevSlots attr{};
    const hipError_t e = lds_limit((const void *)cache_resolve_kernel, attr, lds);
    if (e != hipSuccess) return e;
    cache_resolve_kernel<<<1, RES_THREADS, lds, s>>>(ids, n, E, n_slots, P, key_base, slot_of, key_of, stamp, ctl,
                                                     stats, expert_bytes);
    return hipGetLastError();
}

hipError_t launch_cache_fetch(const int32_t *ctl, const uint8_t *hg, const uint8_t *hu, const uint8_t *hd,
                              uint8_t *sg, uint8_t *su, uint8_t *sd, int64_t gate_bytes, int64_t down_bytes,
                              hipStream_t s)
{
    // the miss count is only known on the device: a fixed grid strides over
    // whatever the list holds.  The host link, not the CUs, bounds the copy:
    // 64 work-groups keep 256 KB of reads in flight (enough for the link's
    // latency) and leave the other compute units to a layer running beside it
    const int grid = std::max(16, cu_count() / 4);
    cache_fetch_kernel<<<grid, FETCH_THREADS, 0, s>>>(ctl, hg, hu, hd, sg, su, sd, gate_bytes, down_bytes);
    return hipGetLastError();
}

}  // namespace moe
