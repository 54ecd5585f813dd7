// FP8 forward kernel instantiations (head_dim 128; bf16 or fp16 output; all mask modes).
#include "attn_fwd_fp8.h"

namespace xattn {

hipError_t launch_fwd_fp8(const Fp8Args& a, bool out_bf16, int mode, int n_work,
                          hipStream_t s) {
  const dim3 grid(n_work), block(Fp8Shape::NT);
  if (out_bf16) {
    if (mode == MASK_NONE) hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, MASK_NONE>), grid, block, 0, s, a);
    else if (mode == MASK_CAUSAL) hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, MASK_CAUSAL>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, MASK_WINDOW>), grid, block, 0, s, a);
  } else {
    if (mode == MASK_NONE) hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, MASK_NONE>), grid, block, 0, s, a);
    else if (mode == MASK_CAUSAL) hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, MASK_CAUSAL>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, MASK_WINDOW>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace xattn
