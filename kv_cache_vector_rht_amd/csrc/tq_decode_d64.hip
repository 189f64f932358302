// Logit scan and decode attention for head dimension 64.
#include "tq_decode.inc.h"

namespace tq {
// the kernels for MSE-only key records are instantiated in tq_msek_d64.hip
extern template hipError_t launch_logits_msek_d<64>(const ScanParams &p, int kw, int mode, hipStream_t st);
extern template void launch_decode_msek_d<64, false>(const ScanParams &p, int kw, int vw, dim3 grid, hipStream_t st);

template hipError_t launch_logits_d<64>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_logits_prepared_d<64>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_prepare_d<64>(const ScanParams &p, int kw, hipStream_t st);
template hipError_t launch_decode_d<64>(const ScanParams &p, int kw, int vw, hipStream_t st);
}  // namespace tq
