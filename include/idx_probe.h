/*
 * idx_probe.h -- measured ceilings of the GPU the Indexer library runs on
 * (measurement support for the benchmark; not operations of the Indexer).
 * Each call launches one probe kernel on `stream`, waits for it and writes
 * the kernel's own duration (a HIP event pair attached to the launch) in
 * milliseconds.  Not thread-safe (one event pair per process).
 */
#ifndef IDX_PROBE_H
#define IDX_PROBE_H

#include "idx.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * idx_probe_stream_read -- read `bytes` of device memory at `buf` (16-byte
 * aligned, a multiple of 16) once with `grid` workgroups of 256 threads,
 * each reading one contiguous span in 16-byte loads.
 *   sink  device, [grid] uint32 (one folded word per workgroup)
 *   ms    host, the kernel's duration
 * Achieved bandwidth = bytes / ms.  IDX_EINVAL for bad arguments.
 */
idx_status idx_probe_stream_read(const void *buf, int64_t bytes, int grid, uint32_t *sink,
                                 float *ms, void *stream);

/*
 * idx_probe_mfma_fp4 -- `grid` workgroups of four waves, each wave issuing
 * `iters` x 4 back-to-back v_mfma_scale_f32_32x32x64_f8f6f4 on fp4 operands
 * in registers (four independent accumulators).
 *   sink   device, [grid * 256] fp32 (written only to keep the work live)
 *   flops  host, the dense fp4 flops issued (2 * 32 * 32 * 64 per MFMA)
 *   ms     host, the kernel's duration
 */
idx_status idx_probe_mfma_fp4(int grid, int iters, float *sink, double *flops, float *ms,
                              void *stream);

/*
 * idx_probe_bf16_convert -- the gfx950 conversion instruction that rounds
 * two fp32 values to bf16 (used by the query step inside the score launch)
 * against the software round-to-nearest-even of the other kernels, over
 * every finite fp32 bit pattern; waits for the result.
 *   count       device, one 8-byte aligned word (cleared, then counted into)
 *   mismatches  host, the number of finite inputs on which they differ
 * IDX_EINVAL for a null or misaligned pointer, IDX_EHIP when a HIP call
 * fails.
 */
idx_status idx_probe_bf16_convert(unsigned long long *count, unsigned long long *mismatches,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IDX_PROBE_H */
