// Decode attention with the new token appended in the same launch, head
// dimension 64.
#include "tq_decode.inc.h"

namespace tq {
template hipError_t launch_append_decode_d<64>(const ScanParams &p, int kw, int vw, hipStream_t st);
}  // namespace tq
