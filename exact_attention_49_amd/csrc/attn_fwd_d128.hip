// Kernel instantiations for head_dim = 128 (all dtypes and mask modes).
#include "attn_dispatch.h"

namespace xattn {
XATTN_DEFINE_LAUNCHER(128)
}  // namespace xattn
