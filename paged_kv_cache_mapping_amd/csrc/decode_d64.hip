// Decode kernel instantiations: head size 64 (one file per share so that
// the library builds in parallel).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_ALL_D(, 64)
}  // namespace pkv
