// Decode kernel instantiations: head size 128, INT4 cache, items over two
// adjacent KV heads (whole 128-byte lines per token).
#include "decode_kernels.h"

namespace pkv {
PKV_DECODE_PAIR_INST(, 128)
}  // namespace pkv
