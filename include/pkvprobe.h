/*
 * pkvprobe.h -- the streaming-read probe of libpkvprobe.so (a measurement
 * built beside libpagedkv.so, not part of its ABI).
 *
 * pkvprobe_stream_read reads the K and V bytes of `num_units` units -- one
 * KV head's rows for 16 consecutive token slots of one block: 16 rows of
 * head_bytes (256) bytes, row_bytes apart, starting unit_off[u] bytes into
 * each plane -- with `workers` single-wave workgroups taking equal
 * contiguous shares and keeping `depth` (1..3) units of loads in flight, and
 * writes one XOR of the bytes per worker to sink[workers] (device uint32).
 * Every pointer is a device pointer; unit_off is int64 [num_units].  Units
 * must lie inside the planes (unchecked).  Returns 0, -1 for a NULL
 * pointer, -2 for unsupported sizes, -3 for a launch error.  Enqueues one
 * kernel on `stream`.
 */
#ifndef PKVPROBE_H
#define PKVPROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

__attribute__((visibility("default"))) int pkvprobe_stream_read(
    const void* k_plane, const void* v_plane, const int64_t* unit_off, int32_t num_units,
    int32_t row_bytes, int32_t head_bytes, int32_t tokens, int32_t workers, int32_t depth,
    uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKVPROBE_H */
