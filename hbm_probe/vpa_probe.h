/* vpa_probe.h -- HBM read-ceiling probe (libvpa_probe.so).
 *
 * Measurement only, not part of the argmax path: a persistent read-only
 * kernel that streams a device buffer once, so that the bandwidth the
 * statistics kernel reaches can be set beside what a plain read achieves on
 * the same GPU.  libvpa.so does not contain or call it.
 */
#ifndef VPA_PROBE_H
#define VPA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes one vpa_probe_read over `bytes` reads: `bytes` rounded down to whole
 * 4 KiB chunks (0 if bytes <= 0). */
int64_t vpa_probe_read_bytes(int64_t bytes);

/* uint32 words of the sink for `n_workgroups` workgroups (256 per
 * workgroup); 0 if n_workgroups < 1. */
int64_t vpa_probe_sink_words(int32_t n_workgroups);

/* Enqueue one read of the first vpa_probe_read_bytes(bytes) bytes of `buf`
 * on `stream` (a hipStream_t; NULL = the null stream), by n_workgroups
 * persistent workgroups of 256 threads.
 *  buf     device memory, 16-byte aligned; read only.
 *  sink    device uint32 [vpa_probe_sink_words(n_workgroups)], written: the
 *          XOR of all its words equals the XOR of every 32-bit word read.
 *  1 <= n_workgroups <= 2^20.
 * Returns 0 when enqueued, -1 for invalid arguments (nothing enqueued), or a
 * positive hipError_t code if the launch fails. */
int vpa_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t n_workgroups,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VPA_PROBE_H */
