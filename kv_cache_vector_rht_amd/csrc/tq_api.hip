// C ABI of libtq: argument validation, workspace layout and kernel dispatch.
// Every check runs on the host before any launch, so malformed calls fail
// with TQ_EINVAL / TQ_EUNSUPPORTED without touching the GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/tq.h"
#include "../../include/tq_probe.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
bool lloyd_max_positive_half(int d, int bits, std::vector<double> &c);
}

namespace {

thread_local char g_err[512] = "";

tq_status fail(tq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

tq_status ok() {
  g_err[0] = '\0';
  return TQ_OK;
}

tq_status hip_status(hipError_t e, const char *where) {
  if (e == hipSuccess) return ok();
  return fail(TQ_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int dtype_size(tq_dtype t) { return t == TQ_F32 ? 4 : 2; }

bool dtype_ok(tq_dtype t) { return t == TQ_F32 || t == TQ_BF16 || t == TQ_F16; }

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Codec checks shared by the device calls. `need_key` = 1 requires a key
// codec (full or MSE-only records), 0 a value codec, -1 any.
tq_status check_codec(const tq_codec *c, int need_key, const char *name) {
  if (!c) return fail(TQ_EINVAL, "%s: codec is NULL", name);
  if (!pow2(c->d) || c->d < 8) return fail(TQ_EINVAL, "%s: d=%d is not a power of two >= 8", name, c->d);
  if (c->d != 64 && c->d != 128) return fail(TQ_EUNSUPPORTED, "%s: d=%d (this build supports 64 and 128)", name, c->d);
  if (c->lm_bits < 1) return fail(TQ_EINVAL, "%s: lm_bits=%d", name, c->lm_bits);
  if (c->lm_bits > 4) return fail(TQ_EUNSUPPORTED, "%s: lm_bits=%d (this build supports 1..4)", name, c->lm_bits);
  if (c->is_key < 0 || c->is_key > 2) return fail(TQ_EINVAL, "%s: is_key=%d", name, c->is_key);
  if (need_key >= 0 && (c->is_key != 0) != (need_key != 0))
    return fail(TQ_EINVAL, "%s: expected a %s codec", name, need_key ? "key" : "value");
  if (!c->signs || !c->centroids || !c->thresholds) return fail(TQ_EINVAL, "%s: codec array is NULL", name);
  if (c->is_key == 1 && !c->sketch) return fail(TQ_EINVAL, "%s: key codec without a sketch", name);
  return TQ_OK;
}

// Key width for the scan kernels: w for full key records, kKeyMse + w for
// MSE-only ones; and the bytes of one key record's codes.
int key_width(const tq_codec *kc) { return kc->is_key == 2 ? tq::kKeyMse + kc->lm_bits : kc->lm_bits; }
int key_rec_bytes(const tq_codec *kc) { return tq::key_planes(key_width(kc)) * kc->d / 8; }

// Scan blocks per (batch, kv-head) group: each block walks every blocks-th
// split of `split` tokens. One block fills a CU's LDS, so aim for one block
// per CU (256), at most max_blocks per group (decode: the merge's bound
// kDecodeMaxBlocks) and never more than the context has splits.
int decode_blocks_per_group(int32_t batch, int32_t n_kv, int64_t max_ctx, int split,
                            int max_blocks = tq::kDecodeMaxBlocks) {
  const int64_t groups = std::max<int64_t>(1, static_cast<int64_t>(batch) * n_kv);
  const int64_t splits = std::max<int64_t>(1, (max_ctx + split - 1) / split);
  const int64_t want = std::min<int64_t>(max_blocks, std::max<int64_t>(1, (256 + groups - 1) / groups));
  return static_cast<int>(std::min<int64_t>(splits, want));
}

// The single-pass prefill: used when a KV head has more (position, head)
// pairs than one pass of the decode kernels holds (8). Blocks per group:
// about two per CU over the launch, at most one per split.
bool prefill_single_pass(int32_t chunk, int32_t group) { return static_cast<int64_t>(chunk) * group > 8; }

int prefill_blocks_per_group(int32_t batch, int32_t n_kv, int32_t pairs, int64_t max_ctx) {
  const int64_t groups = std::max<int64_t>(1, static_cast<int64_t>(batch) * n_kv) *
                         ((pairs + tq::kPrefillBlockPairs - 1) / tq::kPrefillBlockPairs);
  const int64_t splits = std::max<int64_t>(1, (max_ctx + tq::kPrefillSplitTokens - 1) / tq::kPrefillSplitTokens);
  const int64_t want = std::max<int64_t>(1, (512 + groups - 1) / groups);
  return static_cast<int>(std::min<int64_t>(std::min<int64_t>(splits, want), tq::kDecodeMaxBlocks));
}

// Bytes of the prepared query records of the single-pass prefill (one per 8
// pairs of every group, sized for the widest keys), after the partials.
size_t prefill_prepared_bytes(int32_t batch, int32_t n_kv, int32_t pairs, int32_t d) {
  return static_cast<size_t>(batch) * n_kv * ((pairs + 7) / 8) * static_cast<size_t>(tq::prepared_stride(d, 4));
}

// The scan kernels address one sequence's arrays with 32-bit offsets.
bool seq_offsets_fit(int64_t cap, int bytes_per_token) {
  return cap * static_cast<int64_t>(bytes_per_token) < (static_cast<int64_t>(1) << 32);
}

// The scan, merge and preparation launches put the (batch, kv-head)
// sequences on the grid's y dimension.
constexpr int64_t kMaxSequences = 65535;
bool sequences_fit(int32_t batch, int32_t n_kv_heads) {
  return static_cast<int64_t>(batch) * n_kv_heads <= kMaxSequences;
}

// The scan kernels stage the queries, signs and sketch with 16-byte loads.
bool staged_inputs_aligned(const tq_codec *kc, const void *q) {
  return reinterpret_cast<uintptr_t>(q) % 16 == 0 && reinterpret_cast<uintptr_t>(kc->signs) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(kc->sketch) % 16 == 0;
}

// Common part of the scan parameters (queries, key codec, key cache).
tq::ScanParams scan_params(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch, int32_t n_kv_heads,
                           int32_t group, const uint8_t *kcodes, const uint16_t *kscalars, int64_t cap,
                           int64_t max_ctx, int split) {
  tq::ScanParams sp{};
  sp.q = q;
  sp.xt = static_cast<int>(qt);
  sp.ksigns = kc->signs;
  sp.kcent = kc->centroids;
  sp.sketch = kc->sketch;
  sp.kcodes = kcodes;
  sp.kscalars = kscalars;
  sp.cap = cap;
  sp.max_ctx = max_ctx;
  sp.batch = batch;
  sp.n_kv = n_kv_heads;
  sp.group = group;
  sp.h0 = 0;
  sp.n_hchunks = (group + 7) / 8;
  // the logit scan merges nothing, so one group may spread over every CU
  sp.nb = decode_blocks_per_group(batch, n_kv_heads, max_ctx, split,
                                  split == tq::kLogitSplit ? 256 : tq::kDecodeMaxBlocks);
  sp.sm_scale = 1.0f;
  sp.qjl = 1;
  sp.chunk = 1;
  sp.qgroup = group;
  return sp;
}

// Shared argument checks and parameter block of the decode calls. mode 0:
// decode, 1: append + decode, 2: prefill (chunk query positions per batch
// row, ctx_lens holding their first positions), 3: decode over fp8 keys (no
// key codec: kc is ignored, d comes from the value codec).
tq_status decode_common(const char *fn, int mode, const tq_codec *kc, const tq_codec *vc, const void *q,
                        tq_dtype qt, int32_t batch, int32_t chunk, int32_t n_kv_heads, int32_t group,
                        const uint8_t *kcodes, const uint16_t *kscalars, const uint32_t *vcodes,
                        const uint16_t *vscalars, int64_t cap, const int32_t *ctx_lens, int64_t max_ctx,
                        float sm_scale, void *out, tq_dtype out_t, void *workspace, size_t ws_bytes,
                        tq::ScanParams &sp, bool &nothing) {
  nothing = false;
  const bool append = mode == 1;
  tq_status s = TQ_OK;
  if (mode == 3) {
    kc = vc;                                       // fp8 keys: no key codec (d from the value codec)
  } else {
    s = check_codec(kc, 1, fn);
    if (s != TQ_OK) return s;
  }
  s = check_codec(vc, 0, fn);
  if (s != TQ_OK) return s;
  if (kc->d != vc->d) return fail(TQ_EINVAL, "%s: key d=%d and value d=%d differ", fn, kc->d, vc->d);
  if (!dtype_ok(qt)) return fail(TQ_EINVAL, "%s: bad query dtype", fn);
  if (out_t != TQ_F32 && out_t != TQ_BF16) return fail(TQ_EUNSUPPORTED, "%s: output dtype must be f32 or bf16", fn);
  if (batch < 0 || n_kv_heads < 0 || group < 0 || cap < 0 || max_ctx < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (max_ctx > cap) return fail(TQ_EINVAL, "%s: max_ctx > cap", fn);
  if (cap % 32) return fail(TQ_EINVAL, "%s: cap must be a multiple of 32", fn);
  if (group > 32) return fail(TQ_EUNSUPPORTED, "%s: group=%d > 32", fn, group);
  if (!sequences_fit(batch, n_kv_heads))
    return fail(TQ_EUNSUPPORTED, "%s: batch*n_kv_heads above %lld", fn, static_cast<long long>(kMaxSequences));
  if (chunk < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (static_cast<int64_t>(chunk) * group > tq::kPrefillMaxHeads)
    return fail(TQ_EUNSUPPORTED, "%s: chunk*group=%lld > %d", fn, static_cast<long long>(chunk) * group,
                tq::kPrefillMaxHeads);
  const int key_rec = (mode == 3) ? kc->d : key_rec_bytes(kc);
  if (!seq_offsets_fit(cap, std::max(key_rec, vc->lm_bits * kc->d / 8)))
    return fail(TQ_EUNSUPPORTED, "%s: one sequence's codes exceed 4 GiB", fn);
  if (!std::isfinite(sm_scale)) return fail(TQ_EINVAL, "%s: sm_scale is not finite", fn);
  if (batch == 0 || n_kv_heads == 0 || group == 0 || chunk == 0) {
    nothing = true;
    return TQ_OK;
  }
  if (!q || !out || !ctx_lens || !workspace) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  if ((max_ctx > 0 || append) && (!kcodes || (mode != 3 && !kscalars) || !vcodes || !vscalars))
    return fail(TQ_EINVAL, "%s: NULL cache pointer", fn);
  const size_t need = mode == 1 ? tq_append_decode_attend_workspace(batch, n_kv_heads, group, max_ctx, kc->d)
                     : mode == 2 ? tq_prefill_attend_workspace(batch, chunk, n_kv_heads, group, max_ctx, kc->d)
                                 : tq_decode_attend_workspace(batch, n_kv_heads, group, max_ctx, kc->d);
  if (ws_bytes < need) return fail(TQ_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return fail(TQ_EINVAL, "%s: workspace not 256-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(kcodes) % 16 || reinterpret_cast<uintptr_t>(kscalars) % 16 ||
      reinterpret_cast<uintptr_t>(vcodes) % 16 || reinterpret_cast<uintptr_t>(vscalars) % 16)
    return fail(TQ_EINVAL, "%s: cache arrays must be 16-byte aligned", fn);
  if (mode == 3 ? reinterpret_cast<uintptr_t>(q) % 16 != 0 : !staged_inputs_aligned(kc, q))
    return fail(TQ_EINVAL, "%s: q, signs and sketch must be 16-byte aligned", fn);
  sp = scan_params(kc, q, qt, batch, n_kv_heads, chunk * group, kcodes, kscalars, cap, max_ctx, tq::kAttendSplit);
  sp.chunk = chunk;
  sp.qgroup = group;
  sp.vcodes = vcodes;
  sp.vscalars = vscalars;
  sp.vcent = vc->centroids;
  sp.vsigns = vc->signs;
  if (mode == 2) sp.pos0 = ctx_lens;
  else sp.ctx_lens = ctx_lens;
  sp.sm_scale = sm_scale;
  sp.partials = static_cast<float *>(workspace);
  sp.out = out;
  sp.out_t = static_cast<int>(out_t);
  return TQ_OK;
}

// Fixed device scratch of tq_decode_attend_noalloc: the split partials live
// in this file-scope array instead of a caller workspace. Every GPU the
// library runs on holds its own copy for the life of the process. Host code
// must use the address hipGetSymbolAddress returns for the current device
// (the array's name is a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device, with
// that device current); nullptr with the failure recorded otherwise.
void *device_scratch(const char *fn, tq_status &st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    st = fail(TQ_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    st = fail(TQ_EUNSUPPORTED, "%s: device %d beyond the %d the scratch table holds", fn, dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      st = fail(TQ_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  st = TQ_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char *tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_EINVAL: return "TQ_EINVAL: invalid argument";
    case TQ_EUNSUPPORTED: return "TQ_EUNSUPPORTED: not supported by this build";
    case TQ_EHIP: return "TQ_EHIP: HIP runtime error";
  }
  return "unknown tq_status";
}

const char *tq_last_error(void) { return g_err; }

tq_status tq_make_codebook(int32_t d, int32_t lm_bits, float *centroids, float *thresholds) {
  if (d < 3) return fail(TQ_EINVAL, "tq_make_codebook: d=%d < 3", d);
  if (lm_bits < 1 || lm_bits > 8) return fail(TQ_EINVAL, "tq_make_codebook: lm_bits=%d not in 1..8", lm_bits);
  if (!centroids || !thresholds) return fail(TQ_EINVAL, "tq_make_codebook: NULL output");
  std::vector<double> pos;
  if (!tq::lloyd_max_positive_half(d, lm_bits, pos))
    return fail(TQ_EINVAL, "tq_make_codebook: iteration did not settle (d=%d, bits=%d)", d, lm_bits);
  const int L = 1 << lm_bits;
  const int H = L / 2;
  std::vector<double> c(L);
  for (int k = 0; k < H; ++k) {
    c[H + k] = pos[k];
    c[H - 1 - k] = -pos[k];
  }
  for (int k = 0; k < L; ++k) centroids[k] = static_cast<float>(c[k]);
  for (int k = 0; k + 1 < L; ++k) thresholds[k] = static_cast<float>(0.5 * (c[k] + c[k + 1]));
  thresholds[H - 1] = 0.0f;
  return ok();
}

size_t tq_key_record_bytes(int32_t d, int32_t lm_bits) {
  if (!pow2(d) || d < 8 || lm_bits < 1 || lm_bits > 8) return 0;
  return static_cast<size_t>(lm_bits + 1) * d / 8;
}

size_t tq_mse_key_record_bytes(int32_t d, int32_t lm_bits) {
  if (!pow2(d) || d < 8 || lm_bits < 1 || lm_bits > 8) return 0;
  return static_cast<size_t>(lm_bits) * d / 8;
}

size_t tq_value_block_bytes(int32_t d, int32_t lm_bits) {
  if (!pow2(d) || d < 8 || lm_bits < 1 || lm_bits > 8) return 0;
  return static_cast<size_t>(4) * lm_bits * d;
}

tq_status tq_rate_plan(double bits, int32_t n_layers, int32_t is_key, int32_t *lm_bits) {
  const char *fn = "tq_rate_plan";
  if (!lm_bits) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  if (n_layers <= 0) return fail(TQ_EINVAL, "%s: n_layers=%d", fn, n_layers);
  if (is_key != 0 && is_key != 1) return fail(TQ_EINVAL, "%s: is_key=%d", fn, is_key);
  if (!std::isfinite(bits) || bits <= 0.0) return fail(TQ_EINVAL, "%s: bits is not a positive number", fn);
  // Lloyd-Max bits per coordinate on average: keys spend one bit on the QJL sign
  const double avg = bits - (is_key ? 1.0 : 0.0);
  const int w_lo = static_cast<int>(std::floor(avg));
  const int n_hi = static_cast<int>(std::floor((avg - w_lo) * n_layers + 0.5));
  // the widths used: w_lo on n_layers - n_hi layers, w_lo + 1 on n_hi
  const int used_lo = (n_hi < n_layers) ? w_lo : w_lo + 1, used_hi = (n_hi > 0) ? w_lo + 1 : w_lo;
  if (used_lo < 1 || used_hi > 4)
    return fail(TQ_EUNSUPPORTED, "%s: %.3f bits per channel needs Lloyd-Max widths outside 1..4", fn, bits);
  // layer l takes the wider codebook when the running count of wide layers,
  // floor(l * n_hi / n_layers), steps up at l + 1: the n_hi wide layers are
  // spread evenly over the depth
  for (int l = 0; l < n_layers; ++l) {
    const int64_t a = static_cast<int64_t>(l) * n_hi / n_layers, b = static_cast<int64_t>(l + 1) * n_hi / n_layers;
    lm_bits[l] = w_lo + ((b > a) ? 1 : 0);
  }
  return ok();
}

tq_status tq_encode_kv(const tq_codec *codec, const void *x, tq_dtype xt, int64_t n_seq, int64_t n_tok,
                       int64_t x_seq_stride, int64_t x_tok_stride, void *codes, uint16_t *scalars, int64_t cap,
                       int64_t t0, void *stream) {
  const char *fn = "tq_encode_kv";
  tq_status s = check_codec(codec, -1, fn);
  if (s != TQ_OK) return s;
  if (!dtype_ok(xt)) return fail(TQ_EINVAL, "%s: bad input dtype %d", fn, static_cast<int>(xt));
  if (n_seq < 0 || n_tok < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (cap < 0 || t0 < 0 || t0 + n_tok > cap) return fail(TQ_EINVAL, "%s: slots [t0, t0+n_tok) exceed cap", fn);
  if (!codec->is_key && cap % 32 != 0) return fail(TQ_EINVAL, "%s: value cache cap must be a multiple of 32", fn);
  if (n_seq == 0 || n_tok == 0) return ok();
  if (!x || !codes || !scalars) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  if (x_tok_stride < codec->d || (n_seq > 1 && x_seq_stride < 0))
    return fail(TQ_EINVAL, "%s: token stride must be >= d", fn);
  // one wave encodes 64 coordinates x 64 lanes: 64 tokens (d = 64) or 32 (d = 128)
  const int64_t tpw = codec->d == 128 ? 32 : 64;
  const int64_t g0 = t0 / tpw;
  const int64_t g1 = (t0 + n_tok - 1) / tpw;
  tq::EncodeParams p{};
  p.x = x;
  p.x_seq_stride = x_seq_stride;
  p.x_tok_stride = x_tok_stride;
  p.n_tok = n_tok;
  p.t0 = t0;
  p.cap = cap;
  p.g0 = g0;
  p.groups_per_seq = g1 - g0 + 1;
  p.n_waves = n_seq * p.groups_per_seq;
  p.signs = codec->signs;
  p.centroids = codec->centroids;
  p.thresholds = codec->thresholds;
  p.sketch = codec->sketch;
  p.codes = codes;
  p.scalars = scalars;
  p.xt = static_cast<int>(xt);
  const int es = dtype_size(xt);
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || (x_tok_stride * es) % 16 != 0 || (x_seq_stride * es) % 16 != 0)
    return fail(TQ_EUNSUPPORTED, "%s: input rows must start on 16-byte boundaries", fn);
  if (reinterpret_cast<uintptr_t>(codes) % 16 != 0 || reinterpret_cast<uintptr_t>(scalars) % 4 != 0)
    return fail(TQ_EINVAL, "%s: codes must be 16-byte and scalars 4-byte aligned", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = codec->d == 64 ? tq::launch_encode_d<64>(p, codec->lm_bits, codec->is_key, st)
                                : tq::launch_encode_d<128>(p, codec->lm_bits, codec->is_key, st);
  return hip_status(e, fn);
}

size_t tq_logits_workspace(int32_t batch, int32_t n_kv_heads, int32_t group, int32_t d) {
  (void)batch; (void)n_kv_heads; (void)group; (void)d;
  return 0;   // the scan prepares the queries in LDS
}

static tq_status logits_call(const char *fn, int qjl, const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch,
                             int32_t n_kv_heads, int32_t group, const uint8_t *kcodes, const uint16_t *kscalars,
                             int64_t cap, int64_t n_keys, float *logits, void *workspace, size_t ws_bytes,
                             void *stream) {
  (void)workspace; (void)ws_bytes;
  tq_status s = check_codec(kc, 1, fn);
  if (s != TQ_OK) return s;
  if (!dtype_ok(qt)) return fail(TQ_EINVAL, "%s: bad query dtype", fn);
  if (batch < 0 || n_kv_heads < 0 || group < 0 || n_keys < 0 || cap < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (n_keys > cap) return fail(TQ_EINVAL, "%s: n_keys > cap", fn);
  if (cap % 32) return fail(TQ_EINVAL, "%s: cap must be a multiple of 32", fn);
  if (group > 32) return fail(TQ_EUNSUPPORTED, "%s: group=%d > 32", fn, group);
  if (!sequences_fit(batch, n_kv_heads))
    return fail(TQ_EUNSUPPORTED, "%s: batch*n_kv_heads above %lld", fn, static_cast<long long>(kMaxSequences));
  if (!seq_offsets_fit(cap, key_rec_bytes(kc)))
    return fail(TQ_EUNSUPPORTED, "%s: one sequence's codes exceed 4 GiB", fn);
  if (batch == 0 || n_kv_heads == 0 || group == 0 || n_keys == 0) return ok();
  if (!q || !kcodes || !kscalars || !logits) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  if (reinterpret_cast<uintptr_t>(kcodes) % 16 || reinterpret_cast<uintptr_t>(kscalars) % 16)
    return fail(TQ_EINVAL, "%s: kcodes and kscalars must be 16-byte aligned", fn);
  if (!staged_inputs_aligned(kc, q)) return fail(TQ_EINVAL, "%s: q, signs and sketch must be 16-byte aligned", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  tq::ScanParams sp = scan_params(kc, q, qt, batch, n_kv_heads, group, kcodes, kscalars, cap, n_keys, tq::kLogitSplit);
  sp.logits = logits;
  sp.qjl = qjl;
  hipError_t e = kc->d == 64 ? tq::launch_logits_d<64>(sp, key_width(kc), st) : tq::launch_logits_d<128>(sp, key_width(kc), st);
  return hip_status(e, fn);
}

size_t tq_prepared_queries_bytes(int32_t batch, int32_t n_kv_heads, int32_t group, int32_t d, int32_t lm_bits) {
  if (batch < 0 || n_kv_heads < 0 || group < 0 || (d != 64 && d != 128) || lm_bits < 1 || lm_bits > 4) return 0;
  return align_up(static_cast<size_t>(batch) * n_kv_heads * ((group + 7) / 8) *
                  static_cast<size_t>(tq::prepared_stride(d, lm_bits)));
}

tq_status tq_prepare_queries(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch, int32_t n_kv_heads,
                             int32_t group, void *prepared, size_t bytes, void *stream) {
  const char *fn = "tq_prepare_queries";
  tq_status s = check_codec(kc, 1, fn);
  if (s != TQ_OK) return s;
  if (!dtype_ok(qt)) return fail(TQ_EINVAL, "%s: bad query dtype", fn);
  if (batch < 0 || n_kv_heads < 0 || group < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (group > 32) return fail(TQ_EUNSUPPORTED, "%s: group=%d > 32", fn, group);
  if (!sequences_fit(batch, n_kv_heads))
    return fail(TQ_EUNSUPPORTED, "%s: batch*n_kv_heads above %lld", fn, static_cast<long long>(kMaxSequences));
  if (batch == 0 || n_kv_heads == 0 || group == 0) return ok();
  if (!q || !prepared) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  const size_t need = tq_prepared_queries_bytes(batch, n_kv_heads, group, kc->d, kc->lm_bits);
  if (bytes < need) return fail(TQ_EINVAL, "%s: prepared buffer %zu < %zu bytes", fn, bytes, need);
  if (reinterpret_cast<uintptr_t>(prepared) % 16) return fail(TQ_EINVAL, "%s: prepared buffer not 16-byte aligned", fn);
  if (!staged_inputs_aligned(kc, q)) return fail(TQ_EINVAL, "%s: q, signs and sketch must be 16-byte aligned", fn);
  tq::ScanParams sp = scan_params(kc, q, qt, batch, n_kv_heads, group, nullptr, nullptr, 0, 0, tq::kLogitSplit);
  sp.prepared_w = static_cast<uint8_t *>(prepared);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = kc->d == 64 ? tq::launch_prepare_d<64>(sp, key_width(kc), st) : tq::launch_prepare_d<128>(sp, key_width(kc), st);
  return hip_status(e, fn);
}

tq_status tq_logits_prepared(const tq_codec *kc, const void *prepared, size_t bytes, int32_t batch,
                             int32_t n_kv_heads, int32_t group, const uint8_t *kcodes, const uint16_t *kscalars,
                             int64_t cap, int64_t n_keys, float *logits, void *stream) {
  const char *fn = "tq_logits_prepared";
  tq_status s = check_codec(kc, 1, fn);
  if (s != TQ_OK) return s;
  if (batch < 0 || n_kv_heads < 0 || group < 0 || n_keys < 0 || cap < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (n_keys > cap) return fail(TQ_EINVAL, "%s: n_keys > cap", fn);
  if (cap % 32) return fail(TQ_EINVAL, "%s: cap must be a multiple of 32", fn);
  if (group > 32) return fail(TQ_EUNSUPPORTED, "%s: group=%d > 32", fn, group);
  if (!sequences_fit(batch, n_kv_heads))
    return fail(TQ_EUNSUPPORTED, "%s: batch*n_kv_heads above %lld", fn, static_cast<long long>(kMaxSequences));
  if (!seq_offsets_fit(cap, key_rec_bytes(kc)))
    return fail(TQ_EUNSUPPORTED, "%s: one sequence's codes exceed 4 GiB", fn);
  if (batch == 0 || n_kv_heads == 0 || group == 0 || n_keys == 0) return ok();
  if (!prepared || !kcodes || !kscalars || !logits) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  const size_t need = tq_prepared_queries_bytes(batch, n_kv_heads, group, kc->d, kc->lm_bits);
  if (bytes < need) return fail(TQ_EINVAL, "%s: prepared buffer %zu < %zu bytes", fn, bytes, need);
  if (reinterpret_cast<uintptr_t>(prepared) % 16) return fail(TQ_EINVAL, "%s: prepared buffer not 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(kcodes) % 16 || reinterpret_cast<uintptr_t>(kscalars) % 16)
    return fail(TQ_EINVAL, "%s: kcodes and kscalars must be 16-byte aligned", fn);
  tq::ScanParams sp = scan_params(kc, nullptr, TQ_F32, batch, n_kv_heads, group, kcodes, kscalars, cap, n_keys,
                                  tq::kLogitSplit);
  sp.logits = logits;
  sp.prepared = static_cast<const uint8_t *>(prepared);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = kc->d == 64 ? tq::launch_logits_prepared_d<64>(sp, key_width(kc), st)
                             : tq::launch_logits_prepared_d<128>(sp, key_width(kc), st);
  return hip_status(e, fn);
}

tq_status tq_logits(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch, int32_t n_kv_heads,
                    int32_t group, const uint8_t *kcodes, const uint16_t *kscalars, int64_t cap, int64_t n_keys,
                    float *logits, void *workspace, size_t ws_bytes, void *stream) {
  return logits_call("tq_logits", 1, kc, q, qt, batch, n_kv_heads, group, kcodes, kscalars, cap, n_keys, logits,
                     workspace, ws_bytes, stream);
}

size_t tq_logits_table_workspace(int32_t batch, int32_t n_kv_heads, int32_t group, int32_t d) {
  if (batch < 0 || n_kv_heads < 0 || group < 0 || (d != 64 && d != 128)) return 0;
  return align_up(tq::table_workspace_bytes(batch, n_kv_heads, group, d));
}

tq_status tq_logits_table(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch, int32_t n_kv_heads,
                          int32_t group, const uint8_t *kcodes, const uint16_t *kscalars, int64_t cap,
                          int64_t n_keys, float *logits, void *workspace, size_t ws_bytes, void *stream) {
  const char *fn = "tq_logits_table";
  tq_status s = check_codec(kc, 1, fn);
  if (s != TQ_OK) return s;
  if (kc->is_key != 1) return fail(TQ_EINVAL, "%s: full key records (is_key = 1) only", fn);
  if (!dtype_ok(qt)) return fail(TQ_EINVAL, "%s: bad query dtype", fn);
  if (batch < 0 || n_kv_heads < 0 || group < 0 || n_keys < 0 || cap < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (n_keys > cap) return fail(TQ_EINVAL, "%s: n_keys > cap", fn);
  if (cap % 32) return fail(TQ_EINVAL, "%s: cap must be a multiple of 32", fn);
  if (group > 32) return fail(TQ_EUNSUPPORTED, "%s: group=%d > 32", fn, group);
  if (!sequences_fit(batch, n_kv_heads))
    return fail(TQ_EUNSUPPORTED, "%s: batch*n_kv_heads above %lld", fn, static_cast<long long>(kMaxSequences));
  if (!seq_offsets_fit(cap, key_rec_bytes(kc)))
    return fail(TQ_EUNSUPPORTED, "%s: one sequence's codes exceed 4 GiB", fn);
  if (batch == 0 || n_kv_heads == 0 || group == 0 || n_keys == 0) return ok();
  if (!q || !kcodes || !kscalars || !logits || !workspace) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  const size_t need = tq_logits_table_workspace(batch, n_kv_heads, group, kc->d);
  if (ws_bytes < need) return fail(TQ_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 || reinterpret_cast<uintptr_t>(kcodes) % 16 ||
      reinterpret_cast<uintptr_t>(kscalars) % 16)
    return fail(TQ_EINVAL, "%s: workspace and key cache must be 16-byte aligned", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  tq::ScanParams sp = scan_params(kc, q, qt, batch, n_kv_heads, group, kcodes, kscalars, cap, n_keys, tq::kLogitSplit);
  sp.logits = logits;
  hipError_t e = tq::launch_logits_table(sp, kc->d, kc->lm_bits, static_cast<float *>(workspace), st);
  return hip_status(e, fn);
}

tq_status tq_logits_mse(const tq_codec *kc, const void *q, tq_dtype qt, int32_t batch, int32_t n_kv_heads,
                        int32_t group, const uint8_t *kcodes, const uint16_t *kscalars, int64_t cap, int64_t n_keys,
                        float *logits, void *workspace, size_t ws_bytes, void *stream) {
  return logits_call("tq_logits_mse", 0, kc, q, qt, batch, n_kv_heads, group, kcodes, kscalars, cap, n_keys,
                     logits, workspace, ws_bytes, stream);
}

size_t tq_topk_workspace(int64_t n_rows, int64_t n_cols, int32_t k) {
  if (n_rows < 0 || n_cols < 0 || k < 0 || k > tq::kTopkMaxK) return 0;
  int64_t sa = 0, sb = 0;
  tq::topk_buffers(n_cols, k, sa, sb);
  return align_up(static_cast<size_t>(n_rows) * static_cast<size_t>(sa + sb) * sizeof(uint64_t));
}

tq_status tq_topk(const float *scores, int64_t n_rows, int64_t n_cols, int64_t ld, int32_t k, float *top_scores,
                  int32_t *top_idx, void *workspace, size_t ws_bytes, void *stream) {
  const char *fn = "tq_topk";
  if (n_rows < 0 || n_cols < 0 || k < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (ld < n_cols) return fail(TQ_EINVAL, "%s: ld=%lld < n_cols=%lld", fn, static_cast<long long>(ld),
                               static_cast<long long>(n_cols));
  if (k > n_cols) return fail(TQ_EINVAL, "%s: k=%d > n_cols=%lld", fn, k, static_cast<long long>(n_cols));
  if (k > tq::kTopkMaxK) return fail(TQ_EUNSUPPORTED, "%s: k=%d > %d", fn, k, tq::kTopkMaxK);
  if (n_cols > INT32_MAX) return fail(TQ_EUNSUPPORTED, "%s: n_cols above 2^31 - 1", fn);
  if (n_rows == 0 || k == 0) return ok();
  if (!scores || !top_scores || !top_idx || !workspace) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  if (reinterpret_cast<uintptr_t>(workspace) % 8) return fail(TQ_EINVAL, "%s: workspace must be 8-byte aligned", fn);
  const size_t need = tq_topk_workspace(n_rows, n_cols, k);
  if (ws_bytes < need) return fail(TQ_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  hipError_t e = tq::launch_topk(scores, n_rows, n_cols, ld, k, top_scores, top_idx,
                                 static_cast<uint64_t *>(workspace), static_cast<hipStream_t>(stream));
  return hip_status(e, fn);
}

size_t tq_decode_attend_workspace(int32_t batch, int32_t n_kv_heads, int32_t group, int64_t max_ctx, int32_t d) {
  if (batch < 0 || n_kv_heads < 0 || group <= 0 || max_ctx < 0 || d <= 0) return 0;
  const int nb = decode_blocks_per_group(batch, n_kv_heads, max_ctx, tq::kAttendSplit);
  return align_up(static_cast<size_t>(batch) * n_kv_heads * nb * group * (d + 2) * sizeof(float));
}

size_t tq_append_decode_attend_workspace(int32_t batch, int32_t n_kv_heads, int32_t group, int64_t max_ctx,
                                         int32_t d) {
  if (batch < 0 || n_kv_heads < 0 || group <= 0 || max_ctx < 0 || d <= 0) return 0;
  const int nb = decode_blocks_per_group(batch, n_kv_heads, max_ctx, tq::kAttendSplit) + 1;
  return align_up(static_cast<size_t>(batch) * n_kv_heads * nb * group * (d + 2) * sizeof(float));
}

tq_status tq_encode_fp8_keys(const void *x, tq_dtype xt, int32_t d, int64_t n_seq, int64_t n_tok,
                             int64_t x_seq_stride, int64_t x_tok_stride, float scale, uint8_t *codes, int64_t cap,
                             int64_t t0, void *stream) {
  const char *fn = "tq_encode_fp8_keys";
  if (!dtype_ok(xt)) return fail(TQ_EINVAL, "%s: bad input dtype", fn);
  if (d <= 0 || d % 8) return fail(TQ_EINVAL, "%s: d=%d must be a positive multiple of 8", fn, d);
  if (n_seq < 0 || n_tok < 0 || cap < 0 || t0 < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (t0 + n_tok > cap) return fail(TQ_EINVAL, "%s: t0 + n_tok > cap", fn);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(TQ_EINVAL, "%s: scale must be positive and finite", fn);
  if (n_seq == 0 || n_tok == 0) return ok();
  if (!x || !codes) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  if (x_tok_stride < d || x_seq_stride < 0) return fail(TQ_EINVAL, "%s: bad strides", fn);
  if (reinterpret_cast<uintptr_t>(codes) % 8) return fail(TQ_EINVAL, "%s: codes must be 8-byte aligned", fn);
  tq::EncodeParams ep{};
  ep.x = x;
  ep.x_seq_stride = x_seq_stride;
  ep.x_tok_stride = x_tok_stride;
  ep.n_tok = n_tok;
  ep.t0 = t0;
  ep.cap = cap;
  ep.n_waves = n_seq;
  ep.xt = static_cast<int>(xt);
  ep.codes = codes;
  return hip_status(tq::launch_encode_fp8(ep, d, scale, static_cast<hipStream_t>(stream)), fn);
}

tq_status tq_decode_attend_k8(const tq_codec *vc, const void *q, tq_dtype qt, int32_t batch, int32_t n_kv_heads,
                              int32_t group, const uint8_t *kcodes, float k_scale, const uint32_t *vcodes,
                              const uint16_t *vscalars, int64_t cap, const int32_t *ctx_lens, int64_t max_ctx,
                              float sm_scale, void *out, tq_dtype out_t, void *workspace, size_t ws_bytes,
                              void *stream) {
  const char *fn = "tq_decode_attend_k8";
  if (!vc) return fail(TQ_EINVAL, "%s: codec is NULL", fn);
  if (!(k_scale > 0.f) || !std::isfinite(k_scale)) return fail(TQ_EINVAL, "%s: k_scale must be positive and finite", fn);
  tq::ScanParams sp;
  bool nothing = false;
  tq_status s = decode_common(fn, 3, nullptr, vc, q, qt, batch, 1, n_kv_heads, group, kcodes, nullptr, vcodes,
                              vscalars, cap, ctx_lens, max_ctx, sm_scale, out, out_t, workspace, ws_bytes, sp, nothing);
  if (s != TQ_OK) return s;
  if (nothing) return ok();
  sp.k_scale = k_scale;
  sp.ksigns = nullptr;
  sp.kcent = nullptr;
  sp.sketch = nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = vc->d == 64 ? tq::launch_decode_d<64>(sp, tq::kKeyFp8, vc->lm_bits, st)
                             : tq::launch_decode_d<128>(sp, tq::kKeyFp8, vc->lm_bits, st);
  return hip_status(e, fn);
}

size_t tq_prefill_attend_workspace(int32_t batch, int32_t chunk, int32_t n_kv_heads, int32_t group,
                                   int64_t max_ctx, int32_t d) {
  if (batch < 0 || chunk < 0 || n_kv_heads < 0 || group <= 0 || max_ctx < 0 || d <= 0) return 0;
  const int64_t pairs = static_cast<int64_t>(chunk) * group;
  if (pairs > tq::kPrefillMaxHeads) return 0;
  if (!prefill_single_pass(chunk, group)) {
    const int nb = decode_blocks_per_group(batch, n_kv_heads, max_ctx, tq::kAttendSplit);
    return align_up(static_cast<size_t>(batch) * n_kv_heads * nb * pairs * (d + 2) * sizeof(float));
  }
  const int nb = prefill_blocks_per_group(batch, n_kv_heads, static_cast<int32_t>(pairs), max_ctx);
  return align_up(static_cast<size_t>(batch) * n_kv_heads * nb * pairs * (d + 2) * sizeof(float)) +
         align_up(prefill_prepared_bytes(batch, n_kv_heads, static_cast<int32_t>(pairs), d));
}

tq_status tq_prefill_attend(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt, int32_t batch,
                            int32_t chunk, int32_t n_kv_heads, int32_t group, const uint8_t *kcodes,
                            const uint16_t *kscalars, const uint32_t *vcodes, const uint16_t *vscalars, int64_t cap,
                            const int32_t *pos0, int64_t max_ctx, float sm_scale, void *out, tq_dtype out_t,
                            void *workspace, size_t ws_bytes, void *stream) {
  const char *fn = "tq_prefill_attend";
  tq::ScanParams sp;
  bool nothing = false;
  tq_status s = decode_common(fn, 2, kc, vc, q, qt, batch, chunk, n_kv_heads, group, kcodes, kscalars, vcodes,
                              vscalars, cap, pos0, max_ctx, sm_scale, out, out_t, workspace, ws_bytes, sp, nothing);
  if (s != TQ_OK) return s;
  if (nothing) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (prefill_single_pass(chunk, group)) {
    // one scan of the context per 64 pairs; the prepared query records
    // follow the partials in the workspace
    const int32_t pairs = chunk * group;
    sp.nb = prefill_blocks_per_group(batch, n_kv_heads, pairs, max_ctx);
    const size_t part = align_up(static_cast<size_t>(batch) * n_kv_heads * sp.nb * pairs * (kc->d + 2) * sizeof(float));
    uint8_t *prep = static_cast<uint8_t *>(workspace) + part;
    sp.prepared_w = prep;
    sp.prepared = prep;
    e = kc->d == 64 ? tq::launch_prefill_d<64>(sp, key_width(kc), vc->lm_bits, st)
                    : tq::launch_prefill_d<128>(sp, key_width(kc), vc->lm_bits, st);
  } else {
    e = kc->d == 64 ? tq::launch_decode_d<64>(sp, key_width(kc), vc->lm_bits, st)
                    : tq::launch_decode_d<128>(sp, key_width(kc), vc->lm_bits, st);
  }
  return hip_status(e, fn);
}

tq_status tq_append_decode_attend(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt,
                                  const void *k_new, const void *v_new, tq_dtype kvt, int32_t batch,
                                  int32_t n_kv_heads, int32_t group, uint8_t *kcodes, uint16_t *kscalars,
                                  uint32_t *vcodes, uint16_t *vscalars, int64_t cap, const int32_t *ctx_lens,
                                  int64_t max_ctx, float sm_scale, void *out, tq_dtype out_t, void *workspace,
                                  size_t ws_bytes, void *stream) {
  const char *fn = "tq_append_decode_attend";
  tq::ScanParams sp;
  bool nothing = false;
  tq_status s = decode_common(fn, 1, kc, vc, q, qt, batch, 1, n_kv_heads, group, kcodes, kscalars, vcodes,
                              vscalars, cap, ctx_lens, max_ctx, sm_scale, out, out_t, workspace, ws_bytes, sp, nothing);
  if (s != TQ_OK) return s;
  if (!dtype_ok(kvt)) return fail(TQ_EINVAL, "%s: bad k_new/v_new dtype", fn);
  if (nothing) return ok();
  if (!k_new || !v_new) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  sp.append = 1;
  sp.kv_t = static_cast<int>(kvt);
  sp.k_new = k_new;
  sp.v_new = v_new;
  sp.kthr = kc->thresholds;
  sp.vthr = vc->thresholds;
  sp.kcodes_w = kcodes;
  sp.kscal_w = kscalars;
  sp.vcodes_w = vcodes;
  sp.vscal_w = vscalars;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = kc->d == 64 ? tq::launch_append_decode_d<64>(sp, key_width(kc), vc->lm_bits, st)
                             : tq::launch_append_decode_d<128>(sp, key_width(kc), vc->lm_bits, st);
  return hip_status(e, fn);
}

tq_status tq_decode_attend(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt, int32_t batch,
                           int32_t n_kv_heads, int32_t group, const uint8_t *kcodes, const uint16_t *kscalars,
                           const uint32_t *vcodes, const uint16_t *vscalars, int64_t cap, const int32_t *ctx_lens,
                           int64_t max_ctx, float sm_scale, void *out, tq_dtype out_t, void *workspace,
                           size_t ws_bytes, void *stream) {
  const char *fn = "tq_decode_attend";
  tq::ScanParams sp;
  bool nothing = false;
  tq_status s = decode_common(fn, 0, kc, vc, q, qt, batch, 1, n_kv_heads, group, kcodes, kscalars, vcodes,
                              vscalars, cap, ctx_lens, max_ctx, sm_scale, out, out_t, workspace, ws_bytes, sp, nothing);
  if (s != TQ_OK) return s;
  if (nothing) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = kc->d == 64 ? tq::launch_decode_d<64>(sp, key_width(kc), vc->lm_bits, st)
                             : tq::launch_decode_d<128>(sp, key_width(kc), vc->lm_bits, st);
  return hip_status(e, fn);
}

size_t tq_decode_attend_noalloc_max_workspace(void) { return kScratchBytes; }

tq_status tq_decode_attend_noalloc(const tq_codec *kc, const tq_codec *vc, const void *q, tq_dtype qt, int32_t batch,
                                   int32_t n_kv_heads, int32_t group, const uint8_t *kcodes, const uint16_t *kscalars,
                                   const uint32_t *vcodes, const uint16_t *vscalars, int64_t cap,
                                   const int32_t *ctx_lens, int64_t max_ctx, float sm_scale, void *out,
                                   tq_dtype out_t, void *stream) {
  const char *fn = "tq_decode_attend_noalloc";
  // the partials this call needs, checked against the fixed scratch before
  // anything else touches the device (0 for arguments the checks below reject)
  const int32_t d = kc ? kc->d : 0;
  const size_t need = tq_decode_attend_workspace(batch, n_kv_heads, group, max_ctx, d);
  if (need > kScratchBytes)
    return fail(TQ_EUNSUPPORTED, "%s: the call needs %zu bytes of split partials, above the fixed %zu-byte scratch "
                                 "(use tq_decode_attend with a workspace)", fn, need, kScratchBytes);
  // the arguments are validated as tq_decode_attend's, against a stand-in
  // for the workspace (the scratch is aligned and large enough); the
  // scratch's device address is looked up only for a call that launches
  tq::ScanParams sp;
  bool nothing = false;
  tq_status s = decode_common(fn, 0, kc, vc, q, qt, batch, 1, n_kv_heads, group, kcodes, kscalars, vcodes, vscalars,
                              cap, ctx_lens, max_ctx, sm_scale, out, out_t, reinterpret_cast<void *>(kAlign),
                              kScratchBytes, sp, nothing);
  if (s != TQ_OK) return s;
  if (nothing) return ok();
  void *ws = device_scratch(fn, s);
  if (!ws) return s;
  sp.partials = static_cast<float *>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = kc->d == 64 ? tq::launch_decode_d<64>(sp, key_width(kc), vc->lm_bits, st)
                             : tq::launch_decode_d<128>(sp, key_width(kc), vc->lm_bits, st);
  return hip_status(e, fn);
}

}  // extern "C"
