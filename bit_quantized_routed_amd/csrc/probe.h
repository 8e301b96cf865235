// Launchers of the machine-ceiling probes (moe_probe.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace moe {

hipError_t launch_probe_stream(const void *buf, size_t bytes, int grid, int nontemporal, void *sink, hipStream_t s);
hipError_t launch_probe_mfma(int shape, int grid, int iters, float *sink, hipStream_t s);

}  // namespace moe
