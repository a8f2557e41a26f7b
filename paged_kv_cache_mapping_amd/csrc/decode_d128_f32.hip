// Decode kernel instantiations: head size 128, fp32 cache, and the combine kernels of that size (one file per share so that
// the library builds in parallel).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_SPLIT_INST(, 128, PKV_F32)
PKV_DECODE_COMBINE_INST(, 128)
}  // namespace pkv
