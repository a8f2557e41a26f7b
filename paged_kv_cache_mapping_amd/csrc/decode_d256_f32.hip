// Decode kernel instantiations: head size 256, fp32 cache, and the combine kernels of that size (one file per share so that
// the library builds in parallel).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_SPLIT_INST(, 256, PKV_F32)
PKV_DECODE_COMBINE_INST(, 256)
}  // namespace pkv
