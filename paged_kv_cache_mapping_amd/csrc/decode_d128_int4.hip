// Decode kernel instantiations: head size 128, INT4 cache (matrix-core
// balanced kernels only; one file per share so that the library builds in
// parallel).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_STREAM_INST(, 128, PKV_INT4)
}  // namespace pkv
