// Logit scan and decode attention for head dimension 128.
#include "tq_decode.inc.h"

namespace tq {
template hipError_t launch_logits_d<128>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_logits_prepared_d<128>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_prepare_d<128>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_decode_d<128>(const ScanParams &p, int kw, int vw, hipStream_t st);
}  // namespace tq
