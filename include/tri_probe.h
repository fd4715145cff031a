/*
 * tri_probe.h - attainable-bandwidth probes of the device the pass runs on (MI355X, gfx950).
 *
 * The pass is bound by HBM bandwidth ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 steps 2-5: every
 * cached key is read once to be scored; the kept rows are read and written once to be compacted).  Its kernels
 * are measured against the 8 TB/s peak of the part and against what two plain kernels reach on the same device:
 * a streaming read and a copy, both with 16-byte non-temporal accesses like the pass's own.
 *
 * Conventions as in tri.h: device pointers, asynchronous on `stream`, host-side validation before anything is
 * enqueued (nothing is enqueued on a non-OK status; tri_last_error() says why), the caller owns every buffer.
 */
#ifndef TRI_PROBE_H
#define TRI_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "tri.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes the probes' lengths must be a multiple of. */
#define TRI_PROBE_GRANULE 16384

/*
 * Read `bytes` bytes at src (16-byte aligned, bytes a positive multiple of TRI_PROBE_GRANULE).  sink: one
 * uint32 per workgroup of the probe (at most tri_probe_sink_words() words); it is written only if a
 * workgroup's combined data equals a fixed value that plain data does not produce, which keeps the loads alive.
 */
size_t tri_probe_sink_words(void);
tri_status tri_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Copy `bytes` bytes from src to dst (both 16-byte aligned, not overlapping; bytes as for tri_probe_read). */
tri_status tri_probe_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* TRI_PROBE_H */
