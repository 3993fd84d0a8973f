/*
 * moe_peaks.h -- C ABI of the chip-ceiling microbenchmarks for MI355X (gfx950).
 *
 * Not part of the MoE layer: these kernels measure what the matrix cores and
 * HBM sustain on this chip, so that the layer's kernels can be reported against
 * measured ceilings as well as the published peaks.  Each call queues one
 * kernel on `stream` (a hipStream_t; NULL is the default stream); the caller
 * times it (HIP events around the call) and owns every buffer.
 *
 * Errors: arguments are checked on the host before any launch (MOE_PEAKS_EINVAL
 * means nothing was queued); a failed launch returns MOE_PEAKS_EHIP.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_PEAKS_OK = 0, MOE_PEAKS_EINVAL = -1, MOE_PEAKS_EHIP = -4 };

/* Matrix-core rate on random operands.  `operands` (device, at least
 * moe_peaks_operand_bytes() bytes) holds random data: bf16 values for kind 0,
 * E4M3 codes for kind 1.  Each wavefront loads its own 32x32 operand
 * fragments from it once and runs `iters` (a multiple of 4) rounds of 8 independent MFMA chains
 * (kind 0: 32x32x16 bf16; kind 1: 32x32x64 E4M3 x E4M3 with unit E8M0 scales)
 * with the fragments rotating between chains, so that the matrix cores see
 * changing random bits as in a real GEMM.  `blocks` workgroups of 256 threads
 * (4 wavefronts); `out` (device, blocks*256 floats) receives each lane's
 * accumulator sum so that no work can be dropped.  FLOPs of one call:
 * moe_peaks_mfma_flops(kind, blocks, iters). */
size_t moe_peaks_operand_bytes(void);
double moe_peaks_mfma_flops(int kind, int blocks, int iters);
int moe_peaks_mfma(int kind, const void *operands, int blocks, int iters, float *out,
                   void *stream);

/* HBM read stream: every byte of `src` (device) read once by `blocks`
 * workgroups of 256 threads, block b streaming the contiguous b-th of `blocks`
 * equal chunks with 16-byte non-temporal loads, eight in flight per lane (the
 * fastest of the read patterns measured on the chip: grid-stride loops and
 * cached loads stream 10-20% slower).  `bytes` must be a multiple of
 * blocks * 4096 with chunks under 2 GiB, else MOE_PEAKS_EINVAL before any
 * launch.  `out` (device, blocks uint32) receives each block's XOR of what it
 * read.  Pick `bytes` well above the 256 MB Infinity Cache. */
int moe_peaks_read(const void *src, size_t bytes, int blocks, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PEAKS_H */
