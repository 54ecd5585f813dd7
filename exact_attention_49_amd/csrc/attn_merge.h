// Split-KV merge for the exact-attention forward on gfx950.  Each split s of a row holds a
// normalised partial output O_s (fp32) and the natural-log LSE_s of the scores it saw; the
// row's result is the combination that the online softmax would have produced over all keys:
//     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// with splits that saw no key (LSE_s = -inf) contributing nothing, and O = 0, LSE = -inf when
// no split saw a key.  A NaN partial (the rows of a packed sequence longer than max_seqlen)
// makes the row's O and LSE NaN.  This is the merge of partial softmax results that split-KV
// kernels use (page "flash_fwd_kernel.h" @c272619: split-KV work items, n_split_idx); the
// formula is the log-sum-exp identity written out.  One wave per row; each lane owns PER >= 2 columns.
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

template <bool BF16, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int PER = D >= 128 ? D / 64 : 2;  // columns per lane (pairs, for 32-bit stores)
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const bool owns = lane * PER < D;
  float m = -INFINITY;  // the largest LSE_s, or NaN if any is NaN (fmaxf would drop a NaN)
  for (int s = 0; s < a.num_splits; ++s) {
    const float x = a.lse_part[(long)s * a.rows + row];
    m = (x > m || x != x) ? x : m;
  }
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float total = 0.f;
  if (m != -INFINITY) {
    constexpr float LOG2E = 1.44269504088896340736f;
    for (int s = 0; s < a.num_splits; ++s) {
      const long r = (long)s * a.rows + row;
      const float ws = fast_exp2((a.lse_part[r] - m) * LOG2E);  // 0 for an empty split
      total += ws;
      if (owns) {
        const float* src = a.o_part + r * D + lane * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(ws, src[i], acc[i]);
      }
    }
  }
  const float inv = total > 0.f ? 1.0f / total : 0.f;
  if (owns) {
    uint16_t* dst = a.o + row * D + lane * PER;
#pragma unroll
    for (int i = 0; i < PER; i += 2)
      *(uint32_t*)(dst + i) = Elt<BF16>::pack2(acc[i] * inv, acc[i + 1] * inv);
  }
  if (a.lse != nullptr && lane == 0) {
    constexpr float LN2 = 0.693147180559945309f;
    a.lse[row] = !(total <= 0.f) ? m + fast_log2(total) * LN2 : -INFINITY;  // NaN stays NaN
  }
}

}  // namespace xattn
