// Logit scan, query preparation and decode attention over MSE-only key
// records (index planes and the norm only), head dimension 128.
#include "tq_decode.inc.h"

namespace tq {
template hipError_t launch_logits_msek_d<128>(const ScanParams &p, int kw, int mode, hipStream_t st);
template void launch_decode_msek_d<128, false>(const ScanParams &p, int kw, int vw, dim3 grid, hipStream_t st);
}  // namespace tq
