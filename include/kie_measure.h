/*
 * kie_measure.h -- plain memory-streaming kernels exported next to the decoder.
 *
 * Decode speed at batch 1 is the effective memory bandwidth divided by the bytes each token must
 * move (aikraft.ru «3000 токенов в секунду: как ускорить LLM на обычных GPU», §02; wink.run
 * 《GPU 算力越堆越高,生成 token 为什么还是慢》). These kernels measure the first factor on the
 * running GPU so that the decoder's achieved bandwidth can be set against what a plain stream
 * reaches, and they calibrate hardware byte counters (a copy of N bytes reads N and writes N).
 *
 * Both take device pointers (16-byte aligned), a size in bytes that is a multiple of 16, and a
 * hipStream_t (NULL = default stream). They enqueue one launch with one 512-thread workgroup per
 * compute unit, each streaming one contiguous slice, and return KIE_OK, KIE_ERR_INVALID_ARG or
 * KIE_ERR_HIP. Status codes are those of kie.h.
 */
#ifndef KIE_MEASURE_H
#define KIE_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "kie.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0..bytes) = src[0..bytes) (the buffers must not overlap). */
int32_t kie_stream_copy(void* dst, const void* src, size_t bytes, void* hip_stream);

/* Read src[0..bytes) once; sink_dev (device uint32 [1]) is written only in a practically
 * impossible case and exists to keep the loads. */
int32_t kie_stream_read(const void* src, size_t bytes, uint32_t* sink_dev, void* hip_stream);

/* Byte offset, inside the workspace of a context with this configuration, of the per-wave cycle
 * counters ([compute units][8 waves][16] uint64) that a build compiled with -DKIE_TRACE writes at
 * the end of each decode launch (zeros otherwise); -1 for an invalid configuration. */
int64_t kie_trace_offset(const kie_config* cfg);

/* Protocol stress for tests: with level > 0, every workgroup of the decode and prompt kernels
 * idles a pseudo-random 0 .. level-1 times ~3.4 us before each stage boundary, a different amount
 * per (workgroup, step, layer, boundary). Workgroups then reach each exchange out of their usual
 * order; tokens and logits must be bitwise the same as with level 0, which is the default and
 * adds no work. Applies to launches enqueued after the call. Returns KIE_OK, or
 * KIE_ERR_INVALID_ARG for a null context or a level above 64. */
kie_status kie_set_skew(kie_ctx* ctx, uint32_t level);

/* Time limit of every device-side wait of later launches, in microseconds (0 restores the
 * default of 2 s). A wait that exceeds it raises the timeout error (kie_sync then returns
 * KIE_ERR_TIMEOUT) and every workgroup leaves its waits and ends the launch. Tests set a tiny limit
 * together with kie_set_skew to exercise that path; waits are checked every 64 polls. Returns
 * KIE_OK, or KIE_ERR_INVALID_ARG for a null context or a limit above one hour. */
kie_status kie_set_wait_timeout(kie_ctx* ctx, uint64_t microseconds);

#ifdef __cplusplus
}
#endif
#endif /* KIE_MEASURE_H */
