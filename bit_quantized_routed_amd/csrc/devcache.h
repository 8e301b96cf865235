// Per-device values of the host launch code: kernel attributes, occupancy and
// the compute-unit count depend on the device, so each is computed on first
// use on a device and kept in a slot of that device.  Slots are atomics that
// only ever move from "unset" to a value every thread would compute alike, so
// concurrent callers at most repeat the computation.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace moe {

constexpr int MAX_DEVICES = 64;

// slot of the calling thread's current device, or -1 (not cached) when the
// device index is outside the table
inline int device_slot()
{
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= MAX_DEVICES) return -1;
    return d;
}

// one set-once value per device (0 = unset)
struct DevSlots {
    std::atomic<uint64_t> v[MAX_DEVICES];
    uint64_t get(int slot) const { return slot < 0 ? 0 : v[slot].load(std::memory_order_acquire); }
    void set(int slot, uint64_t x)
    {
        if (slot >= 0) v[slot].store(x, std::memory_order_release);
    }
};

// compute units of the current device (256 if the query fails)
inline int cu_count()
{
    static DevSlots slots{};
    const int slot = device_slot();
    if (const uint64_t c = slots.get(slot)) return (int)c;
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    slots.set(slot, (uint64_t)n);
    return n;
}

// raises a kernel's dynamic LDS limit to at least `lds` bytes on the current
// device (the limit last set is remembered per device)
inline hipError_t lds_limit(const void *kernel, DevSlots &slots, size_t lds)
{
    const int slot = device_slot();
    if (slots.get(slot) >= lds) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess) slots.set(slot, lds);
    return e;
}

}  // namespace moe
