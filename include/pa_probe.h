/*
 * pa_probe.h - streaming-read bandwidth probe on MI355X (gfx950).
 *
 * Measurement only, not part of the attention path. Decode is bound by HBM
 * reads ("Optimização da inferência" page, "O framework de operações:byte":
 * at a low ops:byte ratio the memory-bandwidth roof binds), so the decode
 * kernels are judged against the published 8.0 TB/s and against what a
 * kernel that does nothing but read can reach on the same chip. This probe
 * is that kernel: every byte of `buf` is read once with 128-bit
 * non-temporal loads (the decode kernels' K/V load form), with no other work.
 *
 * Each workgroup folds the 32-bit words it read into one XOR and stores it
 * in its own word of `sink` (one plain store per workgroup: no contended
 * atomics at the end of the pass). The launch uses
 *   n = min(ceil(bytes / PA_PROBE_CHUNK_BYTES), PA_PROBE_SINK_WORDS)
 * workgroups and writes sink[0 .. n); the XOR of those n words is the XOR
 * of all 32-bit words of buf[0 .. bytes), which lets a test check that every
 * word was read exactly once.
 *
 * Arguments: `buf` device memory, `bytes` > 0 and a multiple of 16, 16-byte
 * aligned; `sink` device memory for PA_PROBE_SINK_WORDS uint32 (4-byte
 * aligned); `stream` a hipStream_t as void* (NULL = the default stream).
 * Work is enqueued without synchronising; host-side validation before any
 * HIP call; returns a pa_status_t (PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_ALIGN,
 * PA_ERR_HIP).
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

#define PA_PROBE_CHUNK_BYTES 32768 /* bytes a workgroup reads per step (contiguous) */
#define PA_PROBE_SINK_WORDS 4096   /* most workgroups a launch uses: words of sink  */

#ifdef __cplusplus
extern "C" {
#endif

int pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}  // extern "C"
#endif

#endif /* PA_PROBE_H */
