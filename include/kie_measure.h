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

/* Exchange-latency probes, per chiplet (XCD). The pages place the decode step's synchronisation
 * cost in the GPU's chiplet topology: eight compute dies on four I/O dies, extra latency for an
 * access that crosses I/O dies, and a grid barrier of ~600 ns once every XCD polls a replica
 * behind its own I/O die (aikraft.ru «3000 токенов в секунду…», §05). These measure the decode
 * kernel's own exchange words (64-bit, value << 32 | tag, agent-scope relaxed atomics) on the
 * running GPU. Each enqueues one launch on hip_stream (NULL = default) with one workgroup per
 * compute unit, in dispatch order (workgroup w runs on XCD w mod 8 on the MI355X); every device
 * wait gives up after 200 ms and reports it. Times are s_memrealtime ticks of 10 ns. Return KIE_OK,
 * KIE_ERR_INVALID_ARG or KIE_ERR_HIP; all pointers are device pointers. */

/* Workgroups wg_a and wg_b bounce a counter `iters` times (1 .. 10^6) through flags_dev (>= 512
 * bytes, zeroed by the caller). out_dev [3]: elapsed ticks at wg_a (0 if a wait gave up), the XCD
 * of wg_a, the XCD of wg_b. One-way latency = ticks / (2 iters). */
kie_status kie_probe_pingpong(int32_t wg_a, int32_t wg_b, int32_t iters, uint64_t* flags_dev, uint64_t* out_dev,
                              void* hip_stream);

/* `rounds` all-gather hops of the decode kernel's shape: every workgroup publishes words_per_wg
 * words, to each of `replicas` copies (1, or 8: one per XCD), then polls all of them in its own
 * XCD's copy until every tag matches. ex_dev: 2 * replicas * compute_units * words_per_wg words,
 * zeroed by the caller; lat_dev [compute_units][rounds]: ticks from a workgroup's publication to
 * its gather being complete; xcc_dev [compute_units]: each workgroup's XCD; *fail_dev (zeroed by
 * the caller) becomes non-zero if a wait gave up. words_per_wg * replicas <= 512 and
 * compute_units * words_per_wg <= 8192. A cooperative launch: every workgroup is resident. */
kie_status kie_probe_allgather(int32_t words_per_wg, int32_t rounds, int32_t replicas, uint64_t* ex_dev,
                               uint32_t* lat_dev, uint32_t* xcc_dev, uint32_t* fail_dev, void* hip_stream);

/* Write-to-visible latency per page: workgroup writer_wg (not one of 8 .. 15) writes the first
 * word of page p (page_words words apart in buf_dev, zeroed by the caller) for p < npages; one
 * reader workgroup per XCD (workgroups 8 .. 15) polls it and records the ticks between the write
 * and its first sight of it, then acknowledges through acks_dev (>= 4096 bytes, zeroed; word 256
 * receives the writer's XCD); the writer waits for all eight before the next page. out_dev
 * [npages][8] by reader XCD (0xffffffff where a wait gave up; then *fail_dev is non-zero). Needs
 * >= 16 compute units. */
kie_status kie_probe_page_latency(int32_t npages, int32_t page_words, int32_t writer_wg, uint64_t* buf_dev,
                                  uint64_t* acks_dev, uint32_t* out_dev, uint32_t* fail_dev, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* KIE_MEASURE_H */
