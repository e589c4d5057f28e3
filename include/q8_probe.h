/*
 * q8_probe.h -- measurement aids of the MI355X (gfx950) library, for benchmarks.
 *
 * Not part of the linears: they give the bounds a benchmark reports a kernel against on
 * the GPU it runs on.  A kernel that must read B bytes from HBM once cannot finish in one
 * launch faster than a plain streaming read of B bytes does, and no kernel finishes
 * faster than a launch that does nothing.  Errors as in q8_linear.h (typed status,
 * q8_last_error() holds the text); calls are enqueued on `stream` (a hipStream_t, NULL:
 * the default stream) and return without waiting.
 */
#ifndef Q8_PROBE_H
#define Q8_PROBE_H

#include "q8_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of launch shapes of q8_probe_stream_read (shapes 0 .. count-1). */
int32_t q8_probe_shape_count(void);

/* Words of sink that q8_probe_stream_read with this shape needs on the current device
 * (one uint32 per lane of the grid), or -1 for a shape out of range or a device error. */
int64_t q8_probe_sink_words(int32_t shape);

/*
 * Reads `bytes` bytes at src once, as 4 KB chunks of coalesced 16-byte non-temporal
 * loads spread over the whole GPU in the given launch shape (waves per block, chunks in
 * flight per wave, blocks per CU), and writes one xor of what each lane read to sink
 * (so that no load is dropped); nothing else is written.
 *   src  : device memory, 16-byte aligned, bytes a positive multiple of 4096
 *          (Q8_ERR_ALIGN / Q8_ERR_SHAPE otherwise; Q8_ERR_NULL for NULL)
 *   sink : device memory of at least q8_probe_sink_words(shape) uint32 (sink_words),
 *          4-byte aligned (Q8_ERR_WORKSPACE when smaller)
 */
q8_status q8_probe_stream_read(const void* src, int64_t bytes, int32_t shape, uint32_t* sink, int64_t sink_words,
                               void* stream);

/* Launches a kernel of `blocks` workgroups of 256 threads that does nothing (the cost of
 * a launch in a stream or graph).  blocks in [1, 2^31 - 1], else Q8_ERR_SHAPE. */
q8_status q8_probe_empty(int64_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8_PROBE_H */
