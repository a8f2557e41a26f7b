// Decode kernel instantiations: head size 128, fp8 cache (one file per share so that
// the library builds in parallel).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_SPLIT_INST(, 128, PKV_FP8_E4M3)
PKV_DECODE_STREAM_INST(, 128, PKV_FP8_E4M3)
}  // namespace pkv
