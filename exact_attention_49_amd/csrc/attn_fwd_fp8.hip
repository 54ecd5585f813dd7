// FP8 forward kernel instantiations (head dims 64/128/256; bf16 or fp16 output; all masks).
#include "attn_fwd_fp8.h"

namespace xattn {

template <int D>
static hipError_t launch_d(const Fp8Args& a, bool out_bf16, int mode, unsigned grid,
                           hipStream_t s) {
  constexpr unsigned NT = Fp8Shape<D>::NT;
  if (out_bf16) {
    if (mode == MASK_NONE) return launch_kernel(attn_fwd_fp8_kernel<true, D, MASK_NONE>, grid, NT, s, a);
    if (mode == MASK_CAUSAL) return launch_kernel(attn_fwd_fp8_kernel<true, D, MASK_CAUSAL>, grid, NT, s, a);
    return launch_kernel(attn_fwd_fp8_kernel<true, D, MASK_WINDOW>, grid, NT, s, a);
  }
  if (mode == MASK_NONE) return launch_kernel(attn_fwd_fp8_kernel<false, D, MASK_NONE>, grid, NT, s, a);
  if (mode == MASK_CAUSAL) return launch_kernel(attn_fwd_fp8_kernel<false, D, MASK_CAUSAL>, grid, NT, s, a);
  return launch_kernel(attn_fwd_fp8_kernel<false, D, MASK_WINDOW>, grid, NT, s, a);
}

hipError_t launch_fwd_fp8(const Fp8Args& a, int head_dim, bool out_bf16, int mode, int n_work,
                          hipStream_t s) {
  if (head_dim == 64) return launch_d<64>(a, out_bf16, mode, (unsigned)n_work, s);
  if (head_dim == 128) return launch_d<128>(a, out_bf16, mode, (unsigned)n_work, s);
  return launch_d<256>(a, out_bf16, mode, (unsigned)n_work, s);
}

}  // namespace xattn
