// Split-KV merge for the exact-attention forward on gfx950.  Each split s of a row holds a
// normalised partial output O_s (fp32) and the natural-log LSE_s of the scores it saw; the
// row's result is the combination that the online softmax would have produced over all keys:
//     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// with splits that saw no key (LSE_s = -inf, whose O_s is never written) contributing
// nothing, and O = 0, LSE = -inf when no split saw a key.  A NaN partial (the rows of a packed
// sequence longer than max_seqlen) makes the row's O and LSE NaN.  This is the merge of
// partial softmax results that split-KV kernels use (page "flash_fwd_kernel.h" @c272619:
// split-KV work items, n_split_idx); the formula is the log-sum-exp identity written out.
#pragma once

#include "attn_common.h"

namespace xattn {

struct MergeArgs {
  const float* o_part;   // [num_splits][rows][D]
  const float* lse_part; // [num_splits][rows]
  uint16_t* o;           // [rows][D]
  float* lse;            // [rows] or null
  long rows;
  int num_splits;
};

// D / 4 threads per row, each owning 4 consecutive columns: a split's partial row is one
// contiguous 16-byte load per thread, and the rows of a workgroup follow one another.
template <int D> struct MergeShape {
  static constexpr int TPR = D / 4;        // threads per row
  static constexpr int RPB = 256 / TPR;    // rows per 256-thread workgroup
};

template <bool BF16, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int TPR = MergeShape<D>::TPR, RPB = MergeShape<D>::RPB;
  constexpr float LOG2E = 1.44269504088896340736f;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= a.rows) return;
  const int c = (threadIdx.x % TPR) * 4;
  const float* lp = a.lse_part + row;
  float m = -INFINITY;  // the largest LSE_s, or NaN if any is NaN (fmaxf would drop a NaN)
  for (int s = 0; s < a.num_splits; ++s) {
    const float x = lp[(long)s * a.rows];
    m = (x > m || x != x) ? x : m;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float total = 0.f;
  if (m != -INFINITY) {
    const float* op = a.o_part + row * D + c;
    const long stride = a.rows * D;
    // an empty split's O was never written: it is loaded (in bounds, for loads without
    // branches between them) but not used
#pragma unroll 4
    for (int s = 0; s < a.num_splits; ++s) {
      const float x = lp[(long)s * a.rows];
      const f32x4 o = *(const f32x4*)(op + s * stride);
      const bool seen = x != -INFINITY;
      const float ws = seen ? fast_exp2((x - m) * LOG2E) : 0.f;
      total += ws;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = seen ? fmaf(ws, o[i], acc[i]) : acc[i];
    }
  }
  const float inv = total > 0.f ? 1.0f / total : 0.f;
  const uint32_t lo = Elt<BF16>::pack2(acc[0] * inv, acc[1] * inv);
  const uint32_t hi = Elt<BF16>::pack2(acc[2] * inv, acc[3] * inv);
  *(uint2*)(a.o + row * D + c) = make_uint2(lo, hi);
  if (a.lse != nullptr && c == 0) {
    constexpr float LN2 = 0.693147180559945309f;
    a.lse[row] = !(total <= 0.f) ? m + fast_log2(total) * LN2 : -INFINITY;  // NaN stays NaN
  }
}

}  // namespace xattn
