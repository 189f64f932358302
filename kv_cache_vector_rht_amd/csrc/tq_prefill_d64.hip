// Single-pass prefill attention, head dimension 64.
#include "tq_prefill.inc.h"

namespace tq {
// the preparation kernels are instantiated in tq_decode_d64.hip and tq_msek_d64.hip
extern template hipError_t launch_prepare_d<64>(const ScanParams &p, int kw, hipStream_t st);

template hipError_t launch_prefill_d<64>(const ScanParams &p, int kw, int vw, hipStream_t st);
}  // namespace tq
