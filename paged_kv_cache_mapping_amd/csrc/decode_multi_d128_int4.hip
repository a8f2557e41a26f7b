// Decode kernel instantiations for multi-token items (several query tokens of
// one request per work item): head size 128, INT4 cache.
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_MULTI_INST(, 128, PKV_INT4)
}  // namespace pkv
