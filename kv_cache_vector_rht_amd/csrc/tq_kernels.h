// Kernel parameter blocks and launchers (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

struct EncodeParams {
  const void *x;
  int64_t x_seq_stride, x_tok_stride;   // elements
  int64_t n_tok, t0, cap;
  int64_t g0;                           // first slot group touched (64 or 32 slots)
  int64_t groups_per_seq;
  int64_t n_waves;                      // n_seq * groups_per_seq
  int xt;                               // 0 f32, 1 bf16, 2 f16
  const float *signs, *centroids, *thresholds;
  const uint16_t *sketch;
  void *codes;
  uint16_t *scalars;
};

template <int D>
hipError_t launch_encode_d(const EncodeParams &p, int w, bool key, hipStream_t st);

// Query preparation for one (batch, kv-head) group of `group` query heads:
// q' = R q, p = S q', the fixed-point MFMA operands for the key planes and
// the QJL plane, and per-head float constants (see tq_mfma.h).
struct QueryPrepParams {
  const void *q;                        // [batch][n_kv*group][D]
  int xt;
  int32_t batch, n_kv, group;
  int32_t kw;                           // key Lloyd-Max bits
  const float *signs, *centroids;
  const uint16_t *sketch;
  uint8_t *out;                         // [batch*n_kv][group_bytes]
  size_t group_bytes;
};

template <int D>
hipError_t launch_query_prep_d(const QueryPrepParams &p, hipStream_t st);

struct LogitsParams {
  const uint8_t *qprep;                 // prepared groups, group_bytes apart
  size_t group_bytes, frag_bytes;
  const uint8_t *kcodes;
  const uint16_t *kscalars;
  int64_t cap, n_keys;
  int32_t batch, n_kv, group;
  float *logits;                        // [batch][n_q][n_keys]
};

template <int D>
hipError_t launch_logits_d(const LogitsParams &p, int w, hipStream_t st);

struct DecodeParams {
  const uint8_t *qprep;
  size_t group_bytes, frag_bytes;
  const uint8_t *kcodes;
  const uint16_t *kscalars;
  const uint32_t *vcodes;
  const uint16_t *vscalars;
  const float *vcent, *vsigns;
  int64_t cap, max_ctx;
  const int32_t *ctx_lens;
  int32_t batch, n_kv, group;
  int32_t h0;                           // first head of this launch's head chunk (multiple of 8)
  int32_t n_hchunks;                    // ceil(group / 8)
  int32_t split;                        // tokens per context split (kDecodeSplit)
  int32_t n_splits;                     // blocks per (batch, kv-head) group
  float sm_scale;
  float *partials;                      // [batch*n_kv][blocks per group][group][D+2]
  void *out;
  int out_t;
};

template <int D>
hipError_t launch_decode_d(const DecodeParams &p, int kw, int vw, hipStream_t st);

// Tokens per split of the decode kernel (one pipeline stage), and the most
// blocks one (batch, kv-head) group is spread over.
constexpr int kDecodeSplit = 256;
constexpr int kDecodeMaxBlocks = 128;

}  // namespace tq
