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

// kind: 0 values, 1 keys, 2 MSE-only keys (key layout without the QJL part)
template <int D>
hipError_t launch_encode_d(const EncodeParams &p, int w, int kind, hipStream_t st);
// fp8 keys: codes[s][t][i] = e4m3fn(sat(x / scale)) for slots [t0, t0 + n_tok)
hipError_t launch_encode_fp8(const EncodeParams &p, int d, float scale, hipStream_t st);

// Logit scan and decode attention over the coded cache (one parameter block
// for both; the logit scan leaves the value fields unset).
struct ScanParams {
  // queries and the key codec (the scan kernels prepare the queries)
  const void *q;                        // [batch][n_kv*group][D]
  int xt;
  const float *ksigns, *kcent;
  const uint16_t *sketch;
  // caches, `cap` slots per sequence
  const uint8_t *kcodes;
  const uint16_t *kscalars;
  const uint32_t *vcodes;
  const uint16_t *vscalars;
  const float *vcent, *vsigns;
  int64_t cap;
  int64_t max_ctx;                      // logits: n_keys
  const int32_t *ctx_lens;              // decode: per batch row (null: max_ctx)
  int32_t batch, n_kv, group;
  int32_t h0;                           // first head of this launch's head chunk (multiple of 8)
  int32_t n_hchunks;                    // ceil(group / 8)
  int32_t nb;                           // blocks per (batch, kv-head) group
  // > 0: the head chunks of a group are interleaved into the grid's x
  // dimension (x = nb zin blocks, y = groups) instead of riding on z
  int32_t zin;
  float sm_scale;
  int32_t qjl;                          // 1: full estimator; 0 (logit scan only): its first (MSE) term
  float *partials;                      // decode: [batch*n_kv][nb][group][D+2]
  void *out;                            // decode: [batch][n_kv*group][D]
  int out_t;
  float *logits;                        // logits: [batch][n_kv*group][max_ctx]
  // decode with append (append = 1): the launch also encodes the new token of
  // every sequence, k_new / v_new [batch][n_kv][D] (dtype kv_t), into slot
  // ctx_lens[b] - 1 of the caches and attends over it; the partials then
  // hold nb + 1 splits per group, the last one that token's
  int32_t append;
  // query rows: head v of the launch's group of (b, kv-head) is row
  // (b chunk + v / qgroup) n_kv qgroup + kv-head qgroup + v % qgroup of q
  // (decode and logits: chunk 1, qgroup = group). Prefill (pos0 set): group
  // = chunk qgroup heads, the queries of chunk positions, and head v attends
  // to the tokens t <= pos0[b] + v / qgroup
  int32_t chunk, qgroup;
  const int32_t *pos0;
  // fp8 keys (key width kKeyFp8): logit = k_scale * q . e4m3(k)
  float k_scale;
  // prepared queries: one record of prepared_stride bytes per (group, head
  // chunk), written by the preparation kernel, read by the prepared scan
  const uint8_t *prepared;
  uint8_t *prepared_w;
  int kv_t;
  const void *k_new, *v_new;
  const float *kthr, *vthr;
  uint8_t *kcodes_w;
  uint16_t *kscal_w;
  uint32_t *vcodes_w;
  uint16_t *vscal_w;
};

template <int D>
hipError_t launch_logits_d(const ScanParams &p, int kw, hipStream_t st);
// the query preparation alone (into p.prepared_w), and the logit scan from it
template <int D>
hipError_t launch_prepare_d(const ScanParams &p, int kw, hipStream_t st);
template <int D>
hipError_t launch_logits_prepared_d(const ScanParams &p, int kw, hipStream_t st);
template <int D>
hipError_t launch_decode_d(const ScanParams &p, int kw, int vw, hipStream_t st);
template <int D>
hipError_t launch_append_decode_d(const ScanParams &p, int kw, int vw, hipStream_t st);
// Single-pass prefill attention: the query preparation of every 8 pairs into
// p.prepared_w (read back through p.prepared), one scan of the context per
// 64 (position, head) pairs, the merge.
template <int D>
hipError_t launch_prefill_d(const ScanParams &p, int kw, int vw, hipStream_t st);

// Tokens per split (one pipeline stage) of the logit scan and of decode
// attention, and the most blocks one (batch, kv-head) group is spread over.
constexpr int kLogitSplit = 256;
constexpr int kAttendSplit = 512;
constexpr int kDecodeMaxBlocks = 128;
// Key width selecting fp8 key records (d bytes of OCP e4m3fn per key, no
// scalars) in the decode kernels.
constexpr int kKeyFp8 = 8;
// Key width kKeyMse + w selects MSE-only key records (w index planes, one
// fp16 norm per token: no sign plane, no residual norm) in the scan and
// decode kernels; a plain w (1..4) the full records.
constexpr int kKeyMse = 16;
__host__ __device__ constexpr int key_lm(int kw) { return kw > kKeyMse ? kw - kKeyMse : kw; }
__host__ __device__ constexpr bool key_qjl(int kw) { return kw < kKeyMse && kw != kKeyFp8; }
__host__ __device__ constexpr int key_planes(int kw) { return key_lm(kw) + (key_qjl(kw) ? 1 : 0); }
// Bytes of the fp16 scalars stored per key token: {norm, residual norm} or {norm}.
__host__ __device__ constexpr int key_scalar_bytes(int kw) { return key_qjl(kw) ? 4 : 2; }
// Prefill: most query heads (chunk positions x heads per KV head) per call;
// (position, head) pairs per block of the single-pass prefill and its split.
constexpr int kPrefillMaxHeads = 1024;
constexpr int kPrefillBlockPairs = 64;
constexpr int kPrefillSplitTokens = 128;

// The logit scan with per-head nibble tables in LDS (measurement path):
// workspace bytes (q' and p of every head chunk) and the launches.
size_t table_workspace_bytes(int32_t batch, int32_t n_kv, int32_t group, int32_t d);
hipError_t launch_logits_table(const ScanParams &p, int d, int kw, float *qp, hipStream_t st);

// Row-wise top-k: columns per first-stage block, largest k.
constexpr int kTopkChunk = 4096;
constexpr int kTopkMaxK = 1024;
void topk_buffers(int64_t n_cols, int k, int64_t &stride_a, int64_t &stride_b);   // pairs per row
hipError_t launch_topk(const float *scores, int64_t n_rows, int64_t n_cols, int64_t ld, int k, float *top_scores,
                       int32_t *top_idx, uint64_t *cand, hipStream_t st);

}  // namespace tq
