/*
 * tq.h — C ABI of libtq, the TurboQuant KV-cache codec for AMD Instinct
 * MI355X (gfx950).
 *
 * The method (pages: "TurboQuant と RotorQuant を DGX Spark で試してみた",
 * section "PolarQuant + QJL の 2 段階圧縮"; "TurboQuantとは？仕組み・実測精度
 * ・2026年7月時点の実装状況", sections 第1段 and 第2段): a key or value vector
 * keeps its norm, its unit vector is rotated by a random-sign Walsh-Hadamard
 * transform and each coordinate is Lloyd-Max quantized with no per-block
 * scale; a key additionally keeps the 1-bit signs of a Gaussian (QJL)
 * projection of its quantization residual plus the residual norm, which makes
 * the inner-product estimate q.k unbiased. Attention reads the codes directly.
 *
 * Conventions shared by every call
 *   - All arrays are caller-allocated. "device" arrays live in GPU memory
 *     (hipMalloc / torch CUDA tensors), "host" arrays in CPU memory.
 *   - Device calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream). Results are valid after the stream synchronizes.
 *   - Calls keep no state between invocations and never allocate device
 *     memory; scratch space comes from the caller's `workspace`.
 *   - Arguments are validated on the host before anything is launched:
 *     TQ_EINVAL for a malformed argument (null pointer, negative size,
 *     workspace too small, inconsistent shapes), TQ_EUNSUPPORTED for a
 *     well-formed request this build does not implement (a head dimension
 *     other than 64 or 128, more than 4 Lloyd-Max bits, more than 65535
 *     (batch, kv-head) sequences in one logit or attention call, ...). A failed
 *     launch returns TQ_EHIP. tq_last_error() then describes the failure.
 *   - Data values are not inspected: NaN/Inf in inputs propagate, and a norm
 *     above 65504 is stored as fp16 infinity.
 *
 * Codes and scalars (the packed, scale-free cache)
 *   Let d be the head dimension, w the Lloyd-Max bits, L = 2^w.
 *   A sequence is one (layer, batch, kv-head) stream of tokens; a cache holds
 *   n_seq sequences of `cap` token slots each.
 *   Keys   codes   uint8  [n_seq][cap][(w+1)*d/8]  one record per token: w
 *                  index planes (plane p holds bit p of each index), then the
 *                  QJL sign plane; each plane is d/8 bytes, coordinate i at
 *                  byte i/8, bit i%8 (LSB first).
 *          scalars fp16   [n_seq][cap][2]  {norm, residual norm}
 *   MSE-only keys (the ablation without the QJL stage: codec is_key = 2)
 *          codes   uint8  [n_seq][cap][w*d/8]  the w index planes of a key
 *                  record, without the sign plane
 *          scalars fp16   [n_seq][cap]  {norm}
 *   Values codes   uint32 [n_seq][cap/32][w][d]  token-major: tokens are
 *                  grouped in blocks of 32; the word for (block B, plane p,
 *                  coordinate i) holds bit p of the index of token 32B+j at
 *                  bit j. `cap` must be a multiple of 32.
 *          scalars fp16   [n_seq][cap]  {norm}
 *   Index idx_i of coordinate i is the number of thresholds t_j <= y_i,
 *   taken with the codebook's symmetry: the sign of y_i gives the top index
 *   bit (y_i = +0 or -0 counts as positive) and |y_i| is compared with the
 *   upper half's thresholds. A positive y_i equal to a threshold therefore
 *   takes the upper cell and a negative one the lower cell (the cell further
 *   from zero); every encoding entry point (tq_encode_kv and the append of
 *   tq_append_decode_attend) follows this rule. The comparison itself is
 *   made on the rotated, unnormalised vector against the thresholds scaled
 *   by its norm, in fp32. A sign bit is 1 when its projection is >= 0.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,
  TQ_EUNSUPPORTED = -2,
  TQ_EHIP = -3
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/*
 * Codec parameters. They depend only on (d, bits, seed): no calibration data
 * ("TurboQuantとは？…", section キャリブレーション不要が効く場面).
 *   d           head dimension (a power of two)
 *   lm_bits     w, Lloyd-Max bits per coordinate: keys use b-1 of their b
 *               bits (the last bit is the QJL sign), values use all b
 *   is_key      1: keys (QJL sign plane + residual norm), 0: values,
 *               2: MSE-only keys (key records without the QJL part: every
 *               call that reads keys then computes the estimator's first
 *               term alone, logit = n sum_i q'_i c[idx_i])
 *   signs       device float [d], +1/-1: the rotation R = H diag(signs)/sqrt(d),
 *               H the Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i&j)
 *   centroids   device float [L], ascending and symmetric (c[L-1-k] = -c[k]),
 *               e.g. from tq_make_codebook
 *   thresholds  device float [L-1], t_j between c[j-1] and c[j], antisymmetric
 *               (t[L-2-k] = -t[k], middle one 0) as tq_make_codebook makes
 *               them: the kernels use the upper halves of both arrays (the
 *               sign of a rotated coordinate gives its top index bit)
 *   sketch      device fp16 bit patterns [d][d] (is_key = 1 only; ignored
 *               otherwise, may be NULL): the QJL projection S, row j = the
 *               j-th projection direction
 * The arrays are read, never written, and must stay alive while any call
 * that uses the codec is in flight.
 */
typedef struct {
  int32_t d;
  int32_t lm_bits;
  int32_t is_key;
  int32_t reserved;
  const float *signs;
  const float *centroids;
  const float *thresholds;
  const uint16_t *sketch;
} tq_codec;

/*
 * Lloyd-Max codebook for one coordinate of a uniformly random unit vector in
 * R^d, whose density is proportional to (1 - x^2)^((d-3)/2) on [-1, 1]; after
 * the random rotation every coordinate of a unit vector follows it, whatever
 * the data (stage 1 of the method: rotation, then per-coordinate Lloyd-Max;
 * "TurboQuantとは？…", section 第1段).
 *   d        >= 3 (any integer; the GPU calls need 64 or 128)
 *   lm_bits  1..8
 *   centroids   host float [2^lm_bits] out, ascending, exactly symmetric
 *   thresholds  host float [2^lm_bits - 1] out, midpoints (middle one 0)
 * Host only, synchronous, deterministic. TQ_EINVAL on bad arguments.
 */
tq_status tq_make_codebook(int32_t d, int32_t lm_bits, float *centroids, float *thresholds);

/*
 * Fractional rates: per-layer Lloyd-Max widths whose average gives `bits`
 * per channel (keys: including the QJL sign bit, so the Lloyd-Max average is
 * bits - 1; values: bits). The pages name 2.5- and 3.5-bit operating points
 * (quality-neutral at 3.5, slight loss at 2.5: "TurboQuantとは？…", section
 * 「精度劣化ゼロ」の出所と、マージ後に判明した実測値) and describe a serving
 * fork offering those two presets with the quantization parameters set per
 * layer in metadata ("TurboQuant と RotorQuant を DGX Spark で試してみた",
 * section DGX Spark 専用の vLLM フォーク). Here a rate is a mix of the two
 * neighbouring integer widths over the layers: with avg the Lloyd-Max
 * average, w = floor(avg) and n_hi = round((avg - w) * n_layers) layers take
 * w + 1, spread evenly over the depth (layer l when floor((l+1) n_hi / n)
 * > floor(l n_hi / n)); each layer's cache is then an ordinary cache of its
 * width. The achieved average is w + n_hi / n_layers.
 *   lm_bits  host int32 [n_layers] out
 * TQ_EINVAL for n_layers <= 0, a non-positive or non-finite rate or is_key
 * outside {0, 1}; TQ_EUNSUPPORTED when a width would leave 1..4. Host only.
 */
tq_status tq_rate_plan(double bits, int32_t n_layers, int32_t is_key, int32_t *lm_bits);

/* Bytes of one key record's codes, (w+1)*d/8; 0 if the arguments are invalid. */
size_t tq_key_record_bytes(int32_t d, int32_t lm_bits);
/* Bytes of one MSE-only key record's codes (is_key = 2), w*d/8; 0 if invalid. */
size_t tq_mse_key_record_bytes(int32_t d, int32_t lm_bits);
/* Bytes of one 32-token value block, 4*w*d; 0 if the arguments are invalid. */
size_t tq_value_block_bytes(int32_t d, int32_t lm_bits);

/*
 * Encode n_tok tokens of each of n_seq sequences into cache slots
 * [t0, t0 + n_tok) (steps: store the norm, rotate, Lloyd-Max quantize; keys
 * also take the residual, its norm and the QJL sign bits; pack). The two
 * stages are those of "TurboQuant と RotorQuant を DGX Spark で試してみた",
 * section "PolarQuant + QJL の 2 段階圧縮" (rotate and scalar-quantize, then
 * one bit per coordinate for the remaining error), with stage 1 as the
 * randomized Hadamard rotation and per-coordinate Lloyd-Max quantizer of
 * "TurboQuantとは？…", section 第1段, and stage 2 as the 1-bit sign of a
 * Gaussian random projection of the residual of its section 第2段; the
 * stored norms replace any per-block scale (section 第1段).
 *   x        device, dtype xt (TQ_F32 / TQ_BF16 / TQ_F16); element i of token
 *            t of sequence s at x[s*x_seq_stride + t*x_tok_stride + i]
 *            (strides in elements; rows are contiguous)
 *   codes    device, key or value layout above (uint32 words for values)
 *   scalars  device fp16 bit patterns, layout above
 *   cap      token slots per sequence in codes/scalars (values: multiple of 32)
 *   t0       first slot written; t0 + n_tok <= cap
 * Slots outside [t0, t0 + n_tok) are left untouched (value blocks that the
 * range only partly covers are merged bit by bit), so a decoding loop can
 * append one token per step. n_seq == 0 or n_tok == 0 is a no-op.
 */
tq_status tq_encode_kv(const tq_codec *codec, const void *x, tq_dtype xt, int64_t n_seq,
                       int64_t n_tok, int64_t x_seq_stride, int64_t x_tok_stride, void *codes,
                       uint16_t *scalars, int64_t cap, int64_t t0, void *stream);

/*
 * Estimated attention logits q.k for every query head against the first
 * n_keys keys of its KV head (the attention-logit computation the pages time:
 * "TurboQuantとは？…", section まとめ; "メモリの壁を砕く圧縮革命…", 検証結果):
 *   logit = n * ( sum_i q'_i c[idx_i]
 *                 + sqrt(pi/2)/d * gamma * sum_j p_j (2 sigma_j - 1) ),
 *   q' = R q, p = S q', n and gamma the stored fp16 norms.
 *   q        device [batch][n_kv_heads*group][d], dtype qt, 16-byte aligned
 *            (as are the codec's signs and sketch)
 *   query head h of batch b reads key sequence b*n_kv_heads + h/group
 *   kcodes, kscalars  key cache (layout above) with `cap` slots per
 *            sequence; cap a multiple of 32, both arrays 16-byte aligned,
 *            one sequence's codes below 4 GiB (else TQ_EUNSUPPORTED)
 *   logits   device float [batch][n_kv_heads*group][n_keys] out
 *   workspace  unused (tq_logits_workspace returns 0; may be NULL)
 * Every block prepares its queries (q', p and their fixed-point operands)
 * itself; no other state is read or written.
 */
tq_status tq_logits(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch,
                    int32_t n_kv_heads, int32_t group, const uint8_t *kcodes,
                    const uint16_t *kscalars, int64_t cap, int64_t n_keys, float *logits,
                    void *workspace, size_t ws_bytes, void *stream);
size_t tq_logits_workspace(int32_t batch, int32_t n_kv_heads, int32_t group, int32_t d);

/*
 * tq_logits in two calls, for callers that can run the query preparation
 * beside other work (e.g. on a second stream while the step's keys are
 * encoded): tq_prepare_queries does the preparation that every scan block
 * of tq_logits otherwise does itself (q' = R q, p = S q', their fixed-point
 * MFMA operands and per-head constants) once per (batch, kv-head, chunk of 8
 * heads) and stores it in `prepared`; tq_logits_prepared then scans the keys
 * with it and writes the same logits, bit for bit, as tq_logits.
 *   prepared  device, >= tq_prepared_queries_bytes(...) bytes, 16-byte
 *             aligned; an opaque record per (batch, kv-head, head chunk),
 *             valid for the codec and the queries it was prepared from
 * The other arguments and errors are those of tq_logits (the queries are
 * read by tq_prepare_queries only). tq_prepared_queries_bytes returns 0 for
 * invalid arguments.
 */
size_t tq_prepared_queries_bytes(int32_t batch, int32_t n_kv_heads, int32_t group, int32_t d,
                                 int32_t lm_bits);
tq_status tq_prepare_queries(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch,
                             int32_t n_kv_heads, int32_t group, void *prepared, size_t bytes,
                             void *stream);
tq_status tq_logits_prepared(const tq_codec *kc, const void *prepared, size_t bytes, int32_t batch,
                             int32_t n_kv_heads, int32_t group, const uint8_t *kcodes,
                             const uint16_t *kscalars, int64_t cap, int64_t n_keys, float *logits,
                             void *stream);

/*
 * The MSE-only estimator over full key records: the estimator's first term
 * alone,
 *   logit = n * sum_i q'_i c[idx_i],
 * from the same key records (their sign plane and residual norm are read
 * and left out), so that the bias can be measured on identical codes. It is
 * the biased estimate that the QJL bit corrects: the MSE-optimal codebook
 * shrinks inner products by about the per-coordinate distortion
 * ("TurboQuantとは？…", 第2段: the 1-bit residual removes the inner-product
 * bias). The MSE-only cache format, which also saves the sign plane's and
 * the residual norm's bytes, is the codec with is_key = 2 (any call that
 * reads keys). Arguments and errors as tq_logits (an is_key = 2 codec gives
 * the logits of tq_logits).
 */
tq_status tq_logits_mse(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch,
                        int32_t n_kv_heads, int32_t group, const uint8_t *kcodes,
                        const uint16_t *kscalars, int64_t cap, int64_t n_keys, float *logits,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * Fused decode attention over the coded cache: logits as tq_logits, exact
 * softmax of sm_scale*logit over tokens t < ctx_lens[b], and the weighted sum
 * of the decoded values n_t R_v^T c_v[idx_t] (accumulated in the rotated
 * domain, rotated back once per output row). This is the decode step the
 * pages measure: attention reads the keys and values of the past tokens
 * from the compressed cache ("TurboQuant と RotorQuant を DGX Spark で試して
 * みた", section TurboQuant とは: the KV cache holds the past tokens' keys
 * and values), with values quantized MSE-only to their own width (the k/v
 * widths of the presets in "TurboQuantとは？…", section 「精度劣化ゼロ」の
 * 出所と、マージ後に判明した実測値), and decode-heavy serving is where the
 * pages place the codec's cost (same section).
 *   q        device [batch][n_kv_heads*group][d], dtype qt, 16-byte aligned
 *            (as are the key codec's signs and sketch)
 *   kcodes, kscalars, vcodes, vscalars  key and value caches, `cap` slots
 *   ctx_lens device int32 [batch]; values are clamped to [0, max_ctx]; a
 *            row with no tokens gets zeros
 *   max_ctx  upper bound of ctx_lens (<= cap); sizes the context splits
 *   out      device [batch][n_kv_heads*group][d], dtype out_t (TQ_F32 or
 *            TQ_BF16, round to nearest even)
 *   workspace  device, >= tq_decode_attend_workspace(...) bytes, 256-byte
 *            aligned: the per-split partial softmax states {m, l, acc[d]}
 *            of every (batch, kv-head, block, head), overwritten by each call
 * Cache arrays must be 16-byte aligned and one sequence's key or value codes
 * below 4 GiB (else TQ_EUNSUPPORTED).
 */
tq_status tq_decode_attend(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt,
                           int32_t batch, int32_t n_kv_heads, int32_t group,
                           const uint8_t *kcodes, const uint16_t *kscalars,
                           const uint32_t *vcodes, const uint16_t *vscalars, int64_t cap,
                           const int32_t *ctx_lens, int64_t max_ctx, float sm_scale, void *out,
                           tq_dtype out_t, void *workspace, size_t ws_bytes, void *stream);
size_t tq_decode_attend_workspace(int32_t batch, int32_t n_kv_heads, int32_t group,
                                  int64_t max_ctx, int32_t d);

/*
 * tq_decode_attend without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the split partials go to a fixed scratch array
 * that the library holds in device memory, one copy per GPU, for the life of
 * the process. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up that
 * device's copy. The caller still provides q, the caches, ctx_lens and out.
 * Results are those of tq_decode_attend, bit for bit (the same kernels).
 * Calls that overlap on one GPU (several streams, or several host threads)
 * share the scratch and race: serialize them. Every call overwrites the
 * partials it uses, so nothing needs clearing between calls.
 *   Arguments, output and errors as tq_decode_attend; in addition
 *   TQ_EUNSUPPORTED when tq_decode_attend_workspace(batch, n_kv_heads, group,
 *   max_ctx, d) exceeds tq_decode_attend_noalloc_max_workspace() (16 MiB:
 *   e.g. up to 256 (batch, kv-head) groups of 32 query heads at d = 128).
 */
tq_status tq_decode_attend_noalloc(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt,
                                   int32_t batch, int32_t n_kv_heads, int32_t group,
                                   const uint8_t *kcodes, const uint16_t *kscalars,
                                   const uint32_t *vcodes, const uint16_t *vscalars, int64_t cap,
                                   const int32_t *ctx_lens, int64_t max_ctx, float sm_scale,
                                   void *out, tq_dtype out_t, void *stream);
size_t tq_decode_attend_noalloc_max_workspace(void);

/*
 * One decoding step in one launch: the new token's key and value of every
 * (batch, kv-head) sequence are encoded into the caches (as tq_encode_kv
 * would, into slot ctx_lens[b] - 1) and the query heads attend over the
 * whole context including that token (as tq_decode_attend). The pages count
 * the encoding against decode-heavy serving, whose throughput sits at the
 * low end of the measured range ("TurboQuantとは？…", section 「精度劣化ゼロ」
 * の出所と、マージ後に判明した実測値; "TurboQuant と RotorQuant を DGX Spark
 * で試してみた", section vLLM 本家 PR と llama.cpp の進捗): here the
 * encoding runs beside the context scan instead of in a launch of its own.
 *   k_new, v_new  device [batch][n_kv_heads][d], dtype kvt (TQ_F32 / TQ_BF16
 *                 / TQ_F16): the new token's key and value rows
 *   kcodes, kscalars, vcodes, vscalars  the caches (layouts above), written
 *                 at slot ctx_lens[b] - 1 only (value words of that slot's
 *                 32-token block change in the slot's bit only)
 *   ctx_lens      device int32 [batch]: context lengths INCLUDING the new
 *                 token, clamped to [0, max_ctx]; a row with 0 appends
 *                 nothing and gets zeros
 *   workspace     >= tq_append_decode_attend_workspace(...) bytes (one more
 *                 partial per group than tq_decode_attend)
 * The remaining arguments, the output and the errors are those of
 * tq_decode_attend; in addition k_new/v_new NULL or a bad kvt is TQ_EINVAL.
 * The new token's slot must not be read by other work in flight.
 */
tq_status tq_append_decode_attend(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt,
                                  const void *k_new, const void *v_new, tq_dtype kvt,
                                  int32_t batch, int32_t n_kv_heads, int32_t group,
                                  uint8_t *kcodes, uint16_t *kscalars, uint32_t *vcodes,
                                  uint16_t *vscalars, int64_t cap, const int32_t *ctx_lens,
                                  int64_t max_ctx, float sm_scale, void *out, tq_dtype out_t,
                                  void *workspace, size_t ws_bytes, void *stream);
size_t tq_append_decode_attend_workspace(int32_t batch, int32_t n_kv_heads, int32_t group,
                                         int64_t max_ctx, int32_t d);

/*
 * Causal attention of a prefill chunk over the coded cache: the pages put
 * long-prefill workloads at the high end of the measured throughput range,
 * decode-heavy ones at the low end ("TurboQuantとは？…", section 「精度劣化
 * ゼロ」の出所と、マージ後に判明した実測値). The chunk's own keys and values
 * must already be in the caches (tq_encode_kv at t0 = pos0[b]); query
 * position i of batch row b then attends to the tokens t <= pos0[b] + i
 * (logits as tq_logits, exact softmax, values decoded as in
 * tq_decode_attend).
 *   q       device [batch][chunk][n_kv_heads*group][d], dtype qt, 16-byte
 *           aligned; query head h of position i reads KV head h/group
 *   pos0    device int32 [batch]: cache position of each row's first chunk
 *           token; the context of position i, pos0[b] + i + 1, is clamped
 *           to [0, max_ctx] (so pos0[b] + chunk <= max_ctx <= cap)
 *   out     device [batch][chunk][n_kv_heads*group][d], dtype out_t
 *   workspace  >= tq_prefill_attend_workspace(...) bytes, 256-byte aligned
 * chunk*group <= 1024 (else TQ_EUNSUPPORTED); chunk == 0 is a no-op. The
 * other arguments and errors are those of tq_decode_attend. Every launch
 * covers 8 (position, head) pairs of a KV head and reads its context once.
 */
tq_status tq_prefill_attend(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt,
                            int32_t batch, int32_t chunk, int32_t n_kv_heads, int32_t group,
                            const uint8_t *kcodes, const uint16_t *kscalars, const uint32_t *vcodes,
                            const uint16_t *vscalars, int64_t cap, const int32_t *pos0,
                            int64_t max_ctx, float sm_scale, void *out, tq_dtype out_t,
                            void *workspace, size_t ws_bytes, void *stream);
size_t tq_prefill_attend_workspace(int32_t batch, int32_t chunk, int32_t n_kv_heads,
                                   int32_t group, int64_t max_ctx, int32_t d);

/*
 * The k8v4 cache shape: fp8 keys with 4-bit (any 1..4-bit) TurboQuant values,
 * the most conservative of the serving presets the pages list
 * ("TurboQuantとは？…", sections 「精度劣化ゼロ」の出所と、マージ後に判明した
 * 実測値 and vLLM：–kv-cache-dtypeの切り替えだけで利用可能), kept here as an
 * ablation of the key codec: keys store no rotation, no Lloyd-Max codes and
 * no QJL bits, only each coordinate as an OCP e4m3fn byte.
 *
 * tq_encode_fp8_keys: codes uint8 [n_seq][cap][d], byte i of slot t0 + t of
 * sequence s = e4m3fn(x_i / scale) for input row t of sequence s, the
 * quotient taken in fp32 (correctly rounded), rounded to nearest even; finite
 * quotients beyond +-448 saturate to +-448, NaN stays NaN (0x7f / 0xff).
 *   x, xt, strides, n_seq, n_tok, cap, t0  as tq_encode_kv; d a multiple of 8
 *   scale   positive finite per-tensor scale (1.0: a plain cast)
 *   codes   device, 8-byte aligned; slots outside [t0, t0 + n_tok) untouched
 *
 * tq_decode_attend_k8: tq_decode_attend with the key cache replaced by fp8
 * keys: logit = k_scale * sum_i q_i e4m3(k_i) (q as given, fp32-grade sums),
 * exact softmax of sm_scale * logit, values decoded as in tq_decode_attend.
 *   vc       the value codec (d from it); kcodes the fp8 key cache
 *            [batch*n_kv_heads][cap][d], 16-byte aligned; k_scale > 0
 *   workspace  >= tq_decode_attend_workspace(...) bytes, 256-byte aligned
 * Other arguments and errors as tq_decode_attend (q needs 16-byte alignment).
 */
tq_status tq_encode_fp8_keys(const void *x, tq_dtype xt, int32_t d, int64_t n_seq, int64_t n_tok,
                             int64_t x_seq_stride, int64_t x_tok_stride, float scale, uint8_t *codes,
                             int64_t cap, int64_t t0, void *stream);
tq_status tq_decode_attend_k8(const tq_codec *vc, const void *q, tq_dtype qt, int32_t batch,
                              int32_t n_kv_heads, int32_t group, const uint8_t *kcodes, float k_scale,
                              const uint32_t *vcodes, const uint16_t *vscalars, int64_t cap,
                              const int32_t *ctx_lens, int64_t max_ctx, float sm_scale, void *out,
                              tq_dtype out_t, void *workspace, size_t ws_bytes, void *stream);

/*
 * Row-wise top-k of a score matrix: the ranking step of inner-product search
 * over a coded database (the pages name vector-search indexes as a target of
 * the same codes and estimator: "メモリの壁を砕く圧縮革命、TurboQuant始動",
 * sections TurboQuantの全体像 and 仕組みをほどく). With the database encoded
 * as the keys of one KV head and up to 32 queries as its query heads,
 * tq_logits followed by tq_topk is the search scan.
 *   scores      device float [n_rows][ld], columns [0, n_cols) used
 *   top_scores  device float [n_rows][k] out: the k largest scores of each
 *               row, descending (ties: smaller column first)
 *   top_idx     device int32 [n_rows][k] out: their columns
 *   workspace   device, >= tq_topk_workspace(n_rows, n_cols, k) bytes,
 *               8-byte aligned: per-chunk candidates, overwritten
 * 0 <= k <= n_cols, k <= 1024, n_cols < 2^31; k == 0 or n_rows == 0 is a
 * no-op. Data values are not inspected: a NaN with the sign bit clear ranks
 * above +Inf, one with it set below -Inf; -0.0 ties with +0.0.
 */
tq_status tq_topk(const float *scores, int64_t n_rows, int64_t n_cols, int64_t ld, int32_t k,
                  float *top_scores, int32_t *top_idx, void *workspace, size_t ws_bytes,
                  void *stream);
size_t tq_topk_workspace(int64_t n_rows, int64_t n_cols, int32_t k);

/* Static description of a status code. */
const char *tq_status_string(tq_status s);
/* Message of the last failing call on this thread ("" if none). */
const char *tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
