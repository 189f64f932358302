// Encode kernels instantiated for head dimension 128.
#include "tq_encode.inc.h"

namespace tq {
template hipError_t launch_encode_d<128>(const EncodeParams &p, int w, int kind, hipStream_t st);
}  // namespace tq
