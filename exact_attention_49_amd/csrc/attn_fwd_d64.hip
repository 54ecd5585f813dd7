// Kernel instantiations for head_dim = 64 (all dtypes and mask modes).
#include "attn_dispatch.h"

namespace xattn {
XATTN_DEFINE_LAUNCHER(64)
}  // namespace xattn
