/*
 * liboscar_kv measurement aid: a plain HBM read probe.
 *
 * Not part of the method.  Decode attention over a KV cache is bound by the
 * bandwidth at which the cache can be read from HBM (OScaR notes, "system
 * design": each decode step loads the whole KV cache; OSCAR summary page,
 * section 4: the INT2 gain comes from reading fewer bytes), so the decode
 * kernels are reported against the rate a kernel that does nothing but read
 * reaches on the same device, next to the datasheet peak.
 *
 * oscar_read_probe reads `bytes` bytes of `buf` once, with 16-byte loads:
 *  - chunk_ids == NULL: one sequential sweep over the whole buffer;
 *  - chunk_ids != NULL: chunks of `chunk_bytes` bytes, in the order of the
 *    device array chunk_ids[0 .. n_chunks), chunk c covering bytes
 *    [c * chunk_bytes, (c + 1) * chunk_bytes) (the access pattern of a paged
 *    cache whose pages sit in a shuffled pool).  Ids outside
 *    [0, bytes / chunk_bytes) are skipped.
 * The loaded words are folded into one uint32 per wave, written to
 * sink[0 .. 4 grid), so the loads cannot be elided; `grid` work-groups of
 * 256 threads (4 waves; 1 <= grid <= 2^20, 4 grid <= sink_words) do the work.
 * buf and sink are device pointers; buf 16-byte aligned, bytes and chunk_bytes
 * multiples of 1024.  Enqueued on `stream` (a hipStream_t).
 * Returns 0, or OSCAR_ERR_NULL / OSCAR_ERR_ARG / OSCAR_ERR_DEVICE / OSCAR_ERR_HIP
 * (oscar_kv.h).
 */
#ifndef OSCAR_PROBE_H
#define OSCAR_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oscar_read_probe(const void* buf, size_t bytes, const int32_t* chunk_ids, int32_t n_chunks,
                     int32_t chunk_bytes, uint32_t* sink, int32_t grid, int32_t sink_words,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_PROBE_H */
