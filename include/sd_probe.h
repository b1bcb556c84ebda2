/*
 * sd_probe.h -- measured ceilings of the GPU the step runs on.
 *
 * Not part of the draft-and-verify method: a streaming read and a loop of
 * back-to-back matrix-core instructions, so that the throughput of the
 * step's kernels can be reported as a fraction of what this GPU actually
 * reaches as well as of the vendor's peak figures.  Same conventions as
 * sd.h (device pointers owned by the caller, enqueued on `stream`, status
 * for host-side validation and launch errors only).
 */
#ifndef SD_PROBE_H
#define SD_PROBE_H

#include "sd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------
 * Measured ceilings (not part of the method; for the roofline figures).
 *
 * sd_probe_read  streams `bytes` (>= 16) of device memory at `src` (16-byte
 *   aligned) with plain 16-byte loads, 1,024 workgroups each reading
 *   contiguous 16 KiB blocks, and writes nothing (`sink`: a device word that is only written if the XOR of all
 *   words equals a fixed key).  HBM read rate = bytes / kernel time.
 * sd_probe_mfma  512 workgroups of 4 waves each run `iters` (1..2^24)
 *   rounds of 8 independent bf16 MFMA 32x32x16 on register operands;
 *   sd_probe_mfma_flops(iters) is the flop count of one launch (0 if
 *   iters < 1).  `sink`: a device float written only for one impossible sum.
 * Errors: NULL -> SD_ERR_NULL; bad sizes or alignment -> SD_ERR_SHAPE.
 * ------------------------------------------------------------------------ */
sd_status sd_probe_read(const void* src, size_t bytes, void* sink, void* stream);
int64_t sd_probe_mfma_flops(int32_t iters);
sd_status sd_probe_mfma(int32_t iters, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SD_PROBE_H */
