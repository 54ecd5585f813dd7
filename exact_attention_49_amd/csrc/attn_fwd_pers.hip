// Persistent ping-pong kernel instantiations (head_dim = 128; all dtypes and mask modes).
#include "attn_fwd_persistent.h"

namespace xattn {

hipError_t launch_fwd_persistent(const FwdArgs& a, bool bf16, int mode, int grid,
                                 hipStream_t s) {
  constexpr unsigned NT = PingPongShape::NT;
  if (bf16) {
    if (mode == MASK_NONE) return launch_kernel(attn_fwd_pers_kernel<true, 128, MASK_NONE>, grid, NT, s, a);
    if (mode == MASK_CAUSAL) return launch_kernel(attn_fwd_pers_kernel<true, 128, MASK_CAUSAL>, grid, NT, s, a);
    return launch_kernel(attn_fwd_pers_kernel<true, 128, MASK_WINDOW>, grid, NT, s, a);
  }
  if (mode == MASK_NONE) return launch_kernel(attn_fwd_pers_kernel<false, 128, MASK_NONE>, grid, NT, s, a);
  if (mode == MASK_CAUSAL) return launch_kernel(attn_fwd_pers_kernel<false, 128, MASK_CAUSAL>, grid, NT, s, a);
  return launch_kernel(attn_fwd_pers_kernel<false, 128, MASK_WINDOW>, grid, NT, s, a);
}

}  // namespace xattn
