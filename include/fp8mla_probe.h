/*
 * fp8mla_probe.h -- HBM ceiling probes of libfp8mla.so (benchmark-only).
 *
 * The pages judge the full-pool cast by the fraction of the device's memory
 * bandwidth it reaches ("The KV Cache Cast Bottleneck", Reasoning: the cast
 * runs at about 55% of the card's bandwidth).  These kernels measure, on the
 * device at hand, what its memory system delivers for the access mixes the
 * library's kernels use, so that every kernel's bandwidth can be stated
 * against a measured ceiling next to the specification's peak.  None of the
 * library's paths calls them; they compute nothing of the method.
 *
 * Conventions as in fp8mla.h: device pointers owned by the caller, a
 * hipStream_t in `stream`, enqueue only, host-side argument checks with the
 * same status codes, nothing allocated.
 */
#ifndef FP8MLA_PROBE_H
#define FP8MLA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Sequential read of `bytes` bytes of `src` (16-byte loads, non-temporal),
 * folded into a checksum; `sink` (uint32 [grid]) is written only if a
 * checksum equals a fixed constant.  grid workgroups of 256 lanes, each lane
 * keeping `unroll` (4, 8 or 16) loads in flight.  bytes > 0, a multiple of 16.
 */
int fp8mla_probe_read(const void* src, int64_t bytes, int32_t grid, int32_t unroll, uint32_t* sink,
                      void* stream);

/*
 * The cast's traffic mix without its arithmetic: src (`bytes` bytes) is
 * read once and every 16-byte chunk written twice into dst (2 * bytes
 * bytes; the 1 KB read by a wave lands as two copies in the matching 2 KB
 * of dst), non-temporal, each store covering a contiguous 1 KB span.  grid
 * and unroll as for the read probe; bytes > 0, a multiple of 1024.
 */
int fp8mla_probe_copy_1to2(const void* src, int64_t bytes, void* dst, int32_t grid, int32_t unroll,
                           void* stream);

/*
 * Sequential non-temporal writes of a constant pattern over `bytes` bytes of
 * dst (16-byte stores, each wave store a contiguous 1 KB span).  grid and
 * unroll as for the read probe; bytes > 0, a multiple of 16.
 */
int fp8mla_probe_write(void* dst, int64_t bytes, int32_t grid, int32_t unroll, void* stream);

/*
 * The decode's row gather without its arithmetic: the 576-byte rows
 * pool[indices[r]] (r < n, n a multiple of 16; slots clamped into the pool)
 * are copied global -> LDS by 16-byte copies in chunks of 16 rows, by grid
 * workgroups of 8 waves, each wave keeping `chunks_in_flight` (1 or 2)
 * chunks in flight.  With 2 a workgroup holds 151,552 bytes of LDS (one per
 * compute unit), the decode kernel's row budget.  sink (uint32 [grid * 8])
 * as for the read probe.
 */
int fp8mla_probe_gather_rows(const uint8_t* pool, int64_t num_slots, const int32_t* indices,
                             int64_t n, int32_t grid, int32_t chunks_in_flight, uint32_t* sink,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8MLA_PROBE_H */
