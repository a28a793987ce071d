/*
 * pa_bench.h -- measurement helper exported by libpa (not part of the
 * decode path): a plain streaming read of a device buffer, used to state
 * the HBM read bandwidth a kernel on this GPU can reach for a given byte
 * count, beside the decode kernel's own figure.
 */
#ifndef PA_BENCH_H
#define PA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory `buf` (16-byte aligned, bytes % 16 == 0)
 * once, with 16-byte non-temporal loads spread over the whole GPU.  `sink` is a device
 * uint32 that is written only in the (practically impossible) case that the
 * XOR of everything read equals a fixed pattern; it keeps the loads alive.
 * `workgroups` = 0 picks one 256-thread workgroup per compute unit.  Enqueued on `stream`; returns
 * PA_ERR_INVALID_ARG for a null/misaligned pointer or bad size. */
pa_status pa_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BENCH_H */
