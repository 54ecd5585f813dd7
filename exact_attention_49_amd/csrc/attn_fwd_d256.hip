// Kernel instantiations for head_dim = 256 (all dtypes and mask modes).
#include "attn_dispatch.h"

namespace xattn {
XATTN_DEFINE_LAUNCHER(256)
}  // namespace xattn
