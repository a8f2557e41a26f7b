// Decode kernel instantiations: head sizes 8, 16 and 32 (one file per share so that
// the library builds in parallel).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_ALL_D(, 8)
PKV_DECODE_ALL_D(, 16)
PKV_DECODE_ALL_D(, 32)
}  // namespace pkv
