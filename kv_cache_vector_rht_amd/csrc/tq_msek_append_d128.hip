// Decode attention with the new token appended in the same launch, over
// MSE-only key records, head dimension 128.
#include "tq_decode.inc.h"

namespace tq {
template void launch_decode_msek_d<128, true>(const ScanParams &p, int kw, int vw, dim3 grid, hipStream_t st);
}  // namespace tq
