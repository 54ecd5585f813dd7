// Kernel selection and launch for the exact-attention forward: one tile shape per head dim for
// grids that fill the chip several times over ("big") and one with fewer rows per workgroup
// for small grids.  Shapes were chosen by measurement on MI355X.
#pragma once

#include <type_traits>

#include "attn_fwd_kernel.h"
#include "attn_fwd_pingpong.h"
#include "attn_fwd_wide.h"
#include "attn_merge.h"

namespace xattn {

// Shape tags: the ping-pong kernel, the wide-head-dim kernel, or the generic kernel with a
// Tile shape.
struct UsePingPong {
  static constexpr int BR = PingPongShape::BR;
};
struct UseWide {
  static constexpr int BR = WideShape::BR;
};
template <class T> struct UseGeneric {
  static constexpr int BR = T::BR;
};

template <int D> struct TileCfg;
template <> struct TileCfg<64> {
  // at d = 64 the softmax outweighs the MFMA work, and independent waves interleave it better
  // than the two-group ping-pong.  Direct global -> LDS loads leave no staging registers, so
  // the kernel fits 128 VGPRs and four waves per SIMD (measured on MI355X, 16 packed sequences
  // of H = 32, d = 64: 359 -> 320 us against register staging at three waves per SIMD; three
  // stages at three waves: 338 us; 8-wave workgroups: 334-340 us)
  using Big = UseGeneric<Tile<4, 64, 2, 4, true>>;
  using Small = Big;
};
template <> struct TileCfg<128> {
  using Big = UsePingPong;
  // LDS-DMA loads: the same occupancy as register staging (2 waves per SIMD) with the global
  // loads off the VALU and the staging registers gone (measured on MI355X: split-KV B1 H2
  // N16384 causal 290 -> 252 us; B1 H4 N4096 causal 108 -> 89 us)
  using Small = UseGeneric<Tile<4, 64, 2, 2, true>>;
};
template <> struct TileCfg<256> {
  using Big = UseWide;
  using Small = Big;
};
template <> struct TileCfg<512> {
  using Big = UseWide;
  using Small = Big;
};

// Workgroups the big shape must yield before it is preferred.  Unmasked: one per CU on 256
// CUs (measured on MI355X at d = 128: from 256 workgroups up the ping-pong kernel is 4-7%
// faster than the generic one; with 128 it is up to 7% slower on some shapes).  Masked q-tiles
// differ in cost, and with about one 256-row tile per CU the heaviest tiles set the time: at
// 256 causal (B1 H8 N8192) or windowed tiles the generic kernel's 128-row tiles balance better
// (196 vs 219 us causal, 59 vs 61 us window 1024), while from 384 causal tiles up the
// ping-pong kernel is again 2-12% faster.
constexpr long BIG_TILE_MIN_WORK = 256;
constexpr long BIG_TILE_MIN_WORK_MASKED = 384;
inline long big_tile_min_work(int mode) {
  return mode == MASK_NONE ? BIG_TILE_MIN_WORK : BIG_TILE_MIN_WORK_MASKED;
}

template <bool BF16, int D, int MODE, class S, bool SPLIT> struct Launch;
template <bool BF16, int D, int MODE> struct Launch<BF16, D, MODE, UsePingPong, false> {
  static hipError_t go(const FwdArgs& a, int n_work, hipStream_t s) {
    return launch_kernel(attn_fwd_pp_kernel<BF16, D, MODE>, n_work, PingPongShape::NT, s, a);
  }
};
template <bool BF16, int D, int MODE, bool SPLIT> struct Launch<BF16, D, MODE, UseWide, SPLIT> {
  static hipError_t go(const FwdArgs& a, int n_work, hipStream_t s) {
    return launch_kernel(attn_fwd_wide_kernel<BF16, D, MODE, SPLIT>, n_work, WideShape::NT, s,
                         a);
  }
};
template <bool BF16, int D, int MODE, class T, bool SPLIT>
struct Launch<BF16, D, MODE, UseGeneric<T>, SPLIT> {
  static hipError_t go(const FwdArgs& a, int n_work, hipStream_t s) {
    return launch_kernel(attn_fwd_kernel<BF16, D, MODE, T, SPLIT>, n_work, T::NT, s, a);
  }
};

template <int D, class S, bool SPLIT = false>
hipError_t launch_shape(const FwdArgs& a, bool bf16, int mode, int n_work, hipStream_t s) {
  if (bf16) {
    if (mode == MASK_NONE) return Launch<true, D, MASK_NONE, S, SPLIT>::go(a, n_work, s);
    if (mode == MASK_CAUSAL) return Launch<true, D, MASK_CAUSAL, S, SPLIT>::go(a, n_work, s);
    return Launch<true, D, MASK_WINDOW, S, SPLIT>::go(a, n_work, s);
  }
  if (mode == MASK_NONE) return Launch<false, D, MASK_NONE, S, SPLIT>::go(a, n_work, s);
  if (mode == MASK_CAUSAL) return Launch<false, D, MASK_CAUSAL, S, SPLIT>::go(a, n_work, s);
  return Launch<false, D, MASK_WINDOW, S, SPLIT>::go(a, n_work, s);
}

// Split-KV runs on the small shape of a head dim (the one for grids too small to fill the
// chip); the merge runs 1024 / D rows per 256-thread workgroup.
template <int D>
hipError_t launch_merge_shape(const MergeArgs& m, bool bf16, hipStream_t s) {
  constexpr int RPB = MergeShape<D>::RPB;
  const long blocks = (m.rows + RPB - 1) / RPB;
  if (bf16) return launch_kernel(attn_merge_kernel<true, D>, (unsigned)blocks, 256, s, m);
  return launch_kernel(attn_merge_kernel<false, D>, (unsigned)blocks, 256, s, m);
}

// Host launchers for one head dim (explicitly specialised per head dim in its own translation
// unit).  launch_fwd: `big` selects the shape; the caller sizes the grid with that shape's BR.
// launch_fwd_split: the split-KV sweep on the small shape (grid = work items x splits).
// launch_merge: the split-KV merge.
template <int D>
hipError_t launch_fwd(const FwdArgs& a, bool bf16, int mode, bool big, int n_work,
                      hipStream_t stream);
template <int D>
hipError_t launch_fwd_split(const FwdArgs& a, bool bf16, int mode, int n_work,
                            hipStream_t stream);
template <int D>
hipError_t launch_merge(const MergeArgs& m, bool bf16, hipStream_t stream);
// The persistent ping-pong kernel (head dim 128) over `grid` workgroups (attn_fwd_pers.hip).
hipError_t launch_fwd_persistent(const FwdArgs& a, bool bf16, int mode, int grid,
                                 hipStream_t stream);

#define XATTN_DEFINE_LAUNCHER(D)                                                            \
  template <>                                                                               \
  hipError_t launch_fwd<D>(const FwdArgs& a, bool bf16, int mode, bool big, int n_work,     \
                           hipStream_t stream) {                                            \
    if (big || std::is_same<TileCfg<D>::Big, TileCfg<D>::Small>::value)                     \
      return launch_shape<D, TileCfg<D>::Big>(a, bf16, mode, n_work, stream);               \
    return launch_shape<D, TileCfg<D>::Small>(a, bf16, mode, n_work, stream);               \
  }                                                                                         \
  template <>                                                                               \
  hipError_t launch_fwd_split<D>(const FwdArgs& a, bool bf16, int mode, int n_work,         \
                                 hipStream_t stream) {                                      \
    return launch_shape<D, TileCfg<D>::Small, true>(a, bf16, mode, n_work, stream);         \
  }                                                                                         \
  template <>                                                                               \
  hipError_t launch_merge<D>(const MergeArgs& m, bool bf16, hipStream_t stream) {           \
    return launch_merge_shape<D>(m, bf16, stream);                                          \
  }

}  // namespace xattn
