// Merge kernels of multi-token items (head size 128).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_MERGE_MULTI_INST(, 128)
}  // namespace pkv
