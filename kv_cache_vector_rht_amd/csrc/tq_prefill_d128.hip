// Single-pass prefill attention, head dimension 128.
#include "tq_prefill.inc.h"

namespace tq {
// the preparation kernels are instantiated in tq_decode_d128.hip and tq_msek_d128.hip
extern template hipError_t launch_prepare_d<128>(const ScanParams &p, int kw, hipStream_t st);

template hipError_t launch_prefill_d<128>(const ScanParams &p, int kw, int vw, hipStream_t st);
}  // namespace tq
