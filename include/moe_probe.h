/*
 * moe_probe.h -- measured ceilings of the MI355X (gfx950) that the layer's
 * kernels are judged against, beside the chip's published peaks. These are
 * measurement probes, not part of the layer: libmoe_probe.so, separate from
 * libmoe.so.
 *
 * Each probe enqueues one kernel on `stream` (a hipStream_t, NULL = default)
 * and returns 0, or -1 for bad arguments (nothing launched), or a HIP error
 * code if the launch failed. The caller times the call (events on the same
 * stream) and owns every buffer. Each probe leaves a result the caller can
 * check exactly, so that a probe cannot be fast by skipping its work:
 *  - moe_probe_read: sink[0] += the sum, modulo 2^32, of every 32-bit word of
 *    buf (plain 16-byte vector loads into registers);
 *  - moe_probe_read_tiles: one pass without atomics: out[b] = the sum, modulo
 *    2^32, of the words of the b-th 32 KiB tile of buf (the last one may be
 *    partial), each workgroup issuing all its loads at once; the read of a
 *    buffer of tens of MB in one launch, the size of the layer's small kernels;
 *  - moe_probe_dma_read: the same sum, with buf streamed by direct-to-LDS loads
 *    (global_load_lds_dwordx4, the load of the expert GEMM's LDS ring) through
 *    a three-stage LDS ring, then read back from LDS;
 *  - moe_probe_copy: dst = src (16-byte loads and stores);
 *  - moe_probe_mfma: `waves` wavefronts each run `iters` rounds of 16
 *    independent 16x16x32 bf16 matrix-core products of all-ones operands and
 *    write sink[w] = the sum of its 16 accumulators' first elements
 *    (16 * 32 * iters, exact for iters <= 2^15); FLOP = waves * iters * 16 * 16384.
 * buf, src and dst are device pointers, 16-byte aligned; sizes as stated.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bytes a multiple of 16 */
int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
/* bytes a multiple of 16; out [ceil(bytes / 32768)] */
int moe_probe_read_tiles(const void* buf, size_t bytes, uint32_t* out, void* stream);
/* bytes a multiple of 32768 (one ring stage) */
int moe_probe_dma_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
/* bytes a multiple of 16; src and dst do not overlap */
int moe_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
/* waves a multiple of 4, 1 <= iters <= 32768; sink [waves] float */
int moe_probe_mfma(int32_t waves, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
