// Backward kernel instantiations for head_dim = 128 (all dtypes and mask modes).
#include "attn_bwd.h"

namespace xattn {
XATTN_DEFINE_BWD_LAUNCHER(128)
}  // namespace xattn
