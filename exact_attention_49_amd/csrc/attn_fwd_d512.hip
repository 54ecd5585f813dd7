// Kernel instantiations for head_dim = 512 (all dtypes and mask modes).
#include "attn_dispatch.h"

namespace xattn {
XATTN_DEFINE_LAUNCHER(512)
}  // namespace xattn
