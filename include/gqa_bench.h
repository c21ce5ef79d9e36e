/*
 * gqa_bench.h -- measurement helper exported by libgqa.so for benchmarks.
 * Not part of the attention path (include/gqa.h declares that).
 */
#ifndef GQA_BENCH_H
#define GQA_BENCH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at `src` once with coalesced 16-byte loads (the plain
 * streaming read that bounds any HBM-bound kernel), so that a benchmark can
 * time the achievable read rate exactly as it times the decode kernels.
 * Stores nothing in practice: one 32-bit word at `sink` (device memory) is
 * written only if the data fold to one fixed value.  Requires bytes > 0 and
 * a multiple of 16, src and sink 16-byte aligned (device pointers); work is
 * enqueued on `stream` (a hipStream_t).  Returns a gqa_status_t value.
 */
int gqa_read_probe(const void *src, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_BENCH_H */
