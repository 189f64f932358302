// Logit scan and decode attention for head dimension 64.
#include "tq_decode.inc.h"

namespace tq {
template hipError_t launch_logits_d<64>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_logits_prepared_d<64>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_prepare_d<64>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_decode_d<64>(const ScanParams &p, int kw, int vw, hipStream_t st);
}  // namespace tq
