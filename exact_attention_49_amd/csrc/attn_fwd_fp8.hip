// FP8 forward kernel instantiations (head dims 64/128/256; bf16 or fp16 output; all masks).
#include "attn_fwd_fp8.h"

namespace xattn {

template <int D>
static void launch_d(const Fp8Args& a, bool out_bf16, int mode, dim3 grid, hipStream_t s) {
  const dim3 block(Fp8Shape<D>::NT);
  if (out_bf16) {
    if (mode == MASK_NONE) hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, D, MASK_NONE>), grid, block, 0, s, a);
    else if (mode == MASK_CAUSAL) hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, D, MASK_CAUSAL>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, D, MASK_WINDOW>), grid, block, 0, s, a);
  } else {
    if (mode == MASK_NONE) hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, D, MASK_NONE>), grid, block, 0, s, a);
    else if (mode == MASK_CAUSAL) hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, D, MASK_CAUSAL>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, D, MASK_WINDOW>), grid, block, 0, s, a);
  }
}

hipError_t launch_fwd_fp8(const Fp8Args& a, int head_dim, bool out_bf16, int mode, int n_work,
                          hipStream_t s) {
  const dim3 grid(n_work);
  if (head_dim == 64) launch_d<64>(a, out_bf16, mode, grid, s);
  else if (head_dim == 128) launch_d<128>(a, out_bf16, mode, grid, s);
  else launch_d<256>(a, out_bf16, mode, grid, s);
  return hipGetLastError();
}

}  // namespace xattn
