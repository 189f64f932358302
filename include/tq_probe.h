/*
 * tq_probe.h — measurement helpers of libtq, not part of the codec's hot
 * path: a plain read-and-reduce stream that measures how many bytes per
 * second the GPU's memory delivers to a kernel that only reads, the ceiling
 * against which the read-dominated scans (logits, decode attention) are
 * compared with the datasheet peak; and the LDS-table formulation of the
 * logit scan, measured beside the matrix-core one.
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

/*
 * tq_logits_table: the logit scan of tq_logits with the codebook in LDS
 * instead of on the matrix cores, kept to measure the two formulations
 * against each other (the pages' method names no kernel design; both read
 * the same key records: "TurboQuantとは？…", section 第2段 for the estimator).
 * Every block builds, for a chunk of 4 query heads, nibble tables over the
 * key bit planes: for every 4 coordinates, the sums of the plane's
 * coefficients (2 beta_S q' for an odd subset S of the index bits, 2 p for
 * the sign plane) over each of the 16 bit patterns. A key's plane inner
 * products are then one table entry per nibble, summed by one lane per key.
 * A first kernel writes q' = R q and p = S q' of every head (fp32) to the
 * workspace. Same estimator and output as tq_logits; the fp32 sums run in
 * another order (equal within the logit tolerance, not bit for bit).
 *   workspace  device, >= tq_logits_table_workspace(...) bytes, 16-byte
 *              aligned, overwritten
 * Other arguments and errors as tq_logits; full key records (is_key = 1)
 * only (TQ_EINVAL otherwise).
 */
tq_status tq_logits_table(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch, int32_t n_kv_heads,
                          int32_t group, const uint8_t *kcodes, const uint16_t *kscalars, int64_t cap,
                          int64_t n_keys, float *logits, void *workspace, size_t ws_bytes, void *stream);
size_t tq_logits_table_workspace(int32_t batch, int32_t n_kv_heads, int32_t group, int32_t d);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */
