/* libkvq_probe: a measurement aid, not part of the decode path.
 *
 * Streams a device buffer through the vector memory pipeline with 16-byte
 * loads so that a benchmark can quote the HBM read rate this device actually
 * reaches next to the 8 TB/s data-sheet figure.  The rotated INT2 decode
 * kernel reads its packed cache the same way (16 B per lane), so the two
 * rates are comparable.
 */
#ifndef KVQ_PROBE_H
#define KVQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads bytes [0, n_bytes) of the device buffer `src` once, in 16-byte loads
 * spread over `n_workgroups` workgroups of 256 threads (grid-stride), and folds
 * every loaded word into one value per workgroup.  `sink` is a device buffer of
 * at least n_workgroups uint32 entries; a workgroup writes its entry only when
 * its folded value equals 0x9e3779b9, so the loads cannot be elided and the
 * kernel writes (almost) nothing.  `src` must be 16-byte aligned and n_bytes a
 * multiple of 16.  The launch is asynchronous on `stream` (a hipStream_t; NULL
 * = the null stream).  Returns 0, 1 for invalid arguments (nothing launched), or
 * 2 when the launch fails.  Buffers are owned by the caller. */
int kvq_probe_read_stream(const void* src, size_t n_bytes, uint32_t* sink, int32_t n_workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBE_H */
