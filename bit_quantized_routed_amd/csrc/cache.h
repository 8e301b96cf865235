// Launch interface of the expert-cache kernels (cache.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int CACHE_MAX_SLOTS = 8192;
constexpr int CACHE_MAX_EXPERTS = 1024;
// ctl: [0] call clock, [1] fetch count, [2..3] unused, then (slot, expert) pairs
constexpr int CACHE_CTL_HEAD = 4;
inline int cache_ctl_len(int n_experts) { return CACHE_CTL_HEAD + 2 * n_experts; }

// every slot empty, every key absent, counters zero
hipError_t launch_cache_clear(int32_t *slot_of, int64_t n_keys, int32_t *key_of, uint32_t *stamp, int n_slots,
                              int32_t *ctl, int ctl_len, uint64_t *stats, hipStream_t s);

// one work-group: hits, misses, victims and the fetch list of one call whose
// expert ids are ids[0..n) (keys key_base + expert)
hipError_t launch_cache_resolve(const int32_t *ids, int n, int E, int n_slots, int key_base, int32_t *slot_of,
                                int32_t *key_of, uint32_t *stamp, int32_t *ctl, uint64_t *stats,
                                int64_t expert_bytes, hipStream_t s);

// copy every listed miss's gate, up and down matrices from (device-mapped)
// host memory into its slot
hipError_t launch_cache_fetch(const int32_t *ctl, const uint8_t *hg, const uint8_t *hu, const uint8_t *hd,
                              uint8_t *sg, uint8_t *su, uint8_t *sd, int64_t gate_bytes, int64_t down_bytes,
                              hipStream_t s);

}  // namespace moe
