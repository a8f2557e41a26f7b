// Decode kernel instantiations: head size 128, bf16 cache (one file per share so that
// the library builds in parallel).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_SPLIT_INST(, 128, PKV_BF16)
PKV_DECODE_STREAM_INST(, 128, PKV_BF16)
}  // namespace pkv
