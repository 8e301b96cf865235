/*
 * moe_probe.h -- measurement helpers exported by the same library.
 *
 * The benchmark reports each kernel's rate both against the MI355X's published
 * peaks and against what this machine actually sustains, measured on the same
 * box: a streaming read of HBM and a bf16 MFMA loop.  These two kernels are
 * those measurements; they compute nothing of the layer.
 *
 * moe_probe_stream_read: `grid` work-groups of 512 threads read every byte of
 *   buf once (device, 16-byte aligned, bytes a positive multiple of 16) in
 *   16-byte loads, four per thread in flight (non-temporal loads when
 *   `nontemporal` is non-zero); each thread XORs what it read into
 *   sink[thread] (device, grid * 512 * 16 bytes) so no load can be dropped.
 *   Bytes read = `bytes`.
 * moe_probe_mfma_loop: `grid` work-groups of 256 threads; every wave runs
 *   `iters` rounds of 8 independent bf16 MFMAs -- shape 0:
 *   v_mfma_f32_16x16x32_bf16 (16384 flop each), shape 1:
 *   v_mfma_f32_32x32x16_bf16 (32768 flop each) -- and writes one float per
 *   thread to sink (device, grid * 256 floats).
 *   flop = grid * 4 * iters * 8 * (16384 or 32768).  Shape 1 gives the
 *   chip's MFMA ceiling.  Shape 0 reads about half of it: the compiler keeps
 *   that loop's accumulators in shifting registers and adds about 7 register
 *   moves per MFMA (SQ_INSTS_VALU / SQ_INSTS_MFMA), so it measures the loop,
 *   not the instruction, which runs at the full rate in the kernels.
 *
 * Both are asynchronous on `stream` (time them with events around the call)
 * and return MOE_OK, MOE_ERR_INVALID_ARG for bad sizes or pointers (nothing
 * launched) or MOE_ERR_HIP.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int moe_probe_stream_read(const void *buf, size_t bytes, int grid, int nontemporal, void *sink, void *stream);
int moe_probe_mfma_loop(int shape, int grid, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif
