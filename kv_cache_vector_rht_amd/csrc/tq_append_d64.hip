// Decode attention with the new token appended in the same launch, head
// dimension 64.
#include "tq_decode.inc.h"

namespace tq {
// the kernels for MSE-only key records are instantiated in tq_msek_append_d64.hip
extern template void launch_decode_msek_d<64, true>(const ScanParams &p, int kw, int vw, dim3 grid, hipStream_t st);

template hipError_t launch_append_decode_d<64>(const ScanParams &p, int kw, int vw, hipStream_t st);
}  // namespace tq
