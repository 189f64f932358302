// Kernel parameter blocks and launchers (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

struct EncodeParams {
  const void *x;
  int64_t x_seq_stride, x_tok_stride;   // elements
  int64_t n_tok, t0, cap;
  int64_t g0;                           // first 64-slot group touched
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

// Prepared queries: per query head, q' = R q (D floats) then p = S q' (D floats).
struct QueryPrepParams {
  const void *q;
  int xt;
  int64_t n_heads;                      // batch * n_q
  const float *signs;
  const uint16_t *sketch;
  float *out;                           // [n_heads][2][D]
};

template <int D>
hipError_t launch_query_prep_d(const QueryPrepParams &p, hipStream_t st);

struct LogitsParams {
  const float *qprep;                   // [batch][n_q][2][D]
  const uint8_t *kcodes;
  const uint16_t *kscalars;
  const float *centroids;
  int64_t cap, n_keys;
  int32_t batch, n_kv, group;
  float *logits;                        // [batch][n_q][n_keys]
};

template <int D>
hipError_t launch_logits_d(const LogitsParams &p, int w, hipStream_t st);

struct DecodeParams {
  const float *qprep;                   // [batch][n_q][2][D]
  const uint8_t *kcodes;
  const uint16_t *kscalars;
  const uint32_t *vcodes;
  const uint16_t *vscalars;
  const float *kcent, *vcent, *vsigns;
  int64_t cap, max_ctx;
  const int32_t *ctx_lens;
  int32_t batch, n_kv, group;
  int32_t split;                        // tokens per context split
  int32_t n_splits;
  float sm_scale;
  float *partials;                      // [batch*n_kv][n_splits][group][D+2]
  void *out;
  int out_t;
};

template <int D>
hipError_t launch_decode_d(const DecodeParams &p, int kw, int vw, hipStream_t st);

// LDS bytes of one decode-split block: queries, weights, value norms,
// codebooks, per-head softmax statistics.
inline size_t decode_split_smem(int d, int group, int split) {
  return (static_cast<size_t>(group) * 2 * d + static_cast<size_t>(group) * split + split + 32 +
          2 * static_cast<size_t>(group)) * sizeof(float);
}

}  // namespace tq
