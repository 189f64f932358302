/*
 * tq_probe.h — measurement helper of libtq, not part of the codec: a plain
 * read-and-reduce stream that measures how many bytes per second the GPU's
 * memory delivers to a kernel that only reads, the ceiling against which
 * the read-dominated scans (logits, decode attention) are judged beside
 * the datasheet peak.
 *
 * tq_probe_read: every 16-byte chunk of src [0, bytes) is loaded once (eight
 * loads in flight per thread, grid-stride over 4096 blocks of 256 threads)
 * and XOR-reduced; *sink (device uint32) is written only in the case that
 * the reduction hits a fixed pattern, so the loads cannot be dropped.
 *   src    device, 16-byte aligned; bytes a multiple of 16 (TQ_EINVAL else)
 *   sink   device uint32, may be written
 *   stream hipStream_t (NULL: the default stream); asynchronous
 */
#ifndef TQ_PROBE_H
#define TQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "tq.h"

#ifdef __cplusplus
extern "C" {
#endif

tq_status tq_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */
