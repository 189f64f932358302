// Encode kernels instantiated for head dimension 64.
#include "tq_encode.inc.h"

namespace tq {
template hipError_t launch_encode_d<64>(const EncodeParams &p, int w, int kind, hipStream_t st);
}  // namespace tq
