// Decode kernel instantiations for multi-token items (several query tokens of
// one request per work item): head size 128, fp8 cache.
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_MULTI_INST(, 128, PKV_FP8_E4M3)
}  // namespace pkv
