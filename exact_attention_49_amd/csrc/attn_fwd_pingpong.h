// Ping-pong exact-attention forward kernel for gfx950 (head dim 128; the shape also compiles
// for 64, where the generic kernel is faster).
//
// A workgroup is 8 waves of 32 query rows (256 rows of one (batch|sequence, head)); the waves
// are split into two groups of four, A (waves 0-3) and B (waves 4-7), so that each SIMD runs
// one wave of each.  Per K/V tile a wave does three steps: S = K Q^T (MFMA), the online softmax
// (VALU + transcendental) and O += V^T P^T (MFMA).  Grouped as
//     MFMA block j:  O += V_j^T P_j^T  and  S_{j+1} = K_{j+1} Q^T
//     VALU block j:  softmax of S_j -> P_j
// group B runs half a tile behind group A: while A's waves issue their MFMA block, B's waves
// run their softmax on the same SIMDs, and the other way round.  Two workgroup barriers per
// tile keep the two groups in step.  This is the producer/consumer overlap of the Hopper
// kernels on page "flash_fwd_kernel.h" (@26a6e0a, the MMA warpgroups working while others do
// softmax) realised with wave64 barriers instead of warpgroup specialisation.
//
// K and V tiles (64 keys) are loaded by group B, straight from global memory into LDS
// (buffer_load ... lds: lane l writes LDS base + 16 l, so the XOR swizzle is applied by choosing
// which 16-byte chunk each lane fetches).  The load instructions are spread thinly over B's
// softmax step: a wave that issues several of them back to back stalls until the address unit
// has taken the others.  They target the buffer nobody reads in that half-phase and have two
// half-phases to arrive.  Buffers are double-buffered per matrix.  Rows past the end of the
// sequence fetch the last valid row instead (finite data; those keys are masked to -inf, so
// they contribute exactly 0).
//
// Half-phase schedule (h counts barriers; U_u = {V_u, K_{u+1}} lives in buffer u & 1):
//   h = 2j   : A softmax(j)              | B  O += V_{j-1} P_{j-1}, S_j = K_j Q^T
//   h = 2j+1 : A  O += V_j P_j, S_{j+1}  | B softmax(j), and B issues the loads of U_{j+1}
//   B waits for its loads of U_j at the end of h = 2j; the barrier then publishes them.
//
// Dense causal grids may be folded (FwdArgs::fold): a workgroup then runs q-tile tiles - 1 - m
// and then q-tile m of its head, one after the other, so that every workgroup of a head does
// the same work and they all stream the head's K/V in step.
//
// Grouped K/V heads may be packed (FwdArgs::pack > 1): a q-tile then holds `pack` query heads
// of one K/V head (the kBlockH packing of page "flash_fwd_kernel.h" @c272619) and BR / pack
// positions of each, wave w computing 32 positions of head w / (8 / pack), so that all eight
// waves use every K/V tile the workgroup loads.  The work decoding treats each packed group of
// query heads as one head of BR / pack rows per q-tile.
//
// After a q-tile's last barrier the four tile buffers are free: each wave stages its 32 output
// rows in 8 KiB of them and stores whole rows (store_rows_staged); a folded pair's second
// tile starts with one more barrier, once every wave has read its rows back.
#pragma once

#include <type_traits>

#include "attn_common.h"

namespace xattn {

struct PingPongShape {
  static constexpr int NW = 8, NT = 512, BR = 256, BC = 64;
};

// Folded causal grid: workgroup -> (batch, head) and the q-tile pair (tiles - 1 - m, m), whose
// two tiles together see tiles + 1 key tiles, so every workgroup of a head does the same work.
// Same grouped order as decode_slot, over pairs.  `light` is m, or -1 when the pair is the
// middle tile of an odd count.
__device__ __forceinline__ void decode_work_fold(const FwdArgs& a, Work& w, int& light) {
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int per = a.tiles_per_head, per2 = (per + 1) / 2;
  const int nbh = gridDim.x / per2;
  const int G = min((nbh + 7) / 8, max(a.kv_group, (32 + per2 - 1) / per2));
  const int g = wid / (G * per2);
  const int r = wid - g * G * per2;
  const int gsize = min(G, nbh - g * G);
  const int m = r / gsize;
  const int bh = g * G + (r - m * gsize);
  w.tile = per - 1 - m;
  light = (per - 1 - m != m) ? m : -1;
  w.split = 0;
  w.seqlen = a.seqlen;
  w.row0 = (long)bh * a.seqlen;
  w.c0 = 0;
  const int b = bh / a.heads_q, h = bh - b * a.heads_q;
  w.kv_row0 = ((long)b * (a.heads_q / a.kv_group) + h / a.kv_group) * a.seqlen;
}

template <bool BF16, int D, int MODE, int PF = 3>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_pp_kernel(FwdArgs a) {
  constexpr int BR = PingPongShape::BR, BC = PingPongShape::BC;
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int TILEB = BC * D * 2;             // bytes per K (or V) tile
  constexpr int LOADERS = 4;                    // group B's waves issue the tile loads
  constexpr int LI = BC * CH / (LOADERS * 64);  // load instructions per matrix per loader wave
  static_assert(BC * CH % (LOADERS * 64) == 0, "tile must split evenly over the loader waves");
  static_assert(D == 64 || D == 128, "ping-pong shape is for head dims 64 and 128");

  __shared__ __attribute__((aligned(1024))) char k_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const bool grp_a = wave < 4;

  // packed heads: the decoding sees groups of `pack` query heads as heads of P rows per q-tile
  const int P = BR / a.pack;                             // positions per q-tile
  const int wpp = 8 / a.pack;                            // waves per head of the q-tile
  const long hstride = a.cu_seqlens != nullptr ? (long)a.total_tokens : (long)a.seqlen;
  FwdArgs ap = a;
  ap.heads_q = a.heads_q / a.pack;
  ap.kv_group = a.kv_group / a.pack;
  Work w0;
  int light = -1;
  if (MODE == MASK_CAUSAL && a.fold) {
    decode_work_fold(ap, w0, light);
  } else if (const Decoded dc = decode_work<BR, MODE>(ap, w0, P); dc != Decoded::Run) {
    if (dc == Decoded::Malformed) {  // NaN rows of every query head of the group
      w0.row0 = (long)a.pack * (w0.row0 - w0.c0) + w0.c0;
      for (int j = 0; j < a.pack; ++j, w0.row0 += hstride) fill_malformed_fwd<D>(a, w0);
    }
    return;
  }
  w0.row0 = (long)a.pack * (w0.row0 - w0.c0) + w0.c0;  // the group's first query head
  auto run_tile = [&](const Work& w) XATTN_INLINE {
    const int seqlen = w.seqlen;
    int wl, wr;
    mode_windows<MODE>(a, wl, wr);

    const int q0 = w.tile * P;
    const int qw0 = q0 + (wave % wpp) * 32;              // first position of this wave
    const long wrow0 = w.row0 + (long)(wave / wpp) * hstride;  // its head's row 0
    const int q_last = min(q0 + P, seqlen) - 1;          // last valid position of the tile
    int k_lo = 0, k_hi = seqlen - 1;                     // keys any valid row can see
    if (wl >= 0) k_lo = max(0, q0 - wl);
    if (wr >= 0) k_hi = min(seqlen - 1, q_last + wr);
    const int t_lo = k_lo / BC;
    const int n = k_hi / BC - t_lo + 1;                  // K/V tiles to sweep (>= 1)

    const bool wave_active = qw0 < seqlen;
    const int qw_last = min(qw0 + 32, seqlen) - 1;
    int kw_lo = 0, kw_hi = seqlen - 1;                   // keys this wave's rows can see
    if (wl >= 0) kw_lo = max(0, qw0 - wl);
    if (wr >= 0) kw_hi = min(seqlen - 1, qw_last + wr);

    const uint16_t* __restrict__ kp = a.k + w.kv_row0 * D;
    const uint16_t* __restrict__ vp = a.v + w.kv_row0 * D;
    const int qrow = qw0 + l32;

    i32x4 qf[D / 16];
    load_q_nowait<D>(a.q + wrow0 * D, qrow, seqlen, hh, qf);  // waited for after the prologue loads
    const LaneOffsets<D> lo = lane_offsets<D>(lane);

    f32x16 oacc[D / 32];
  #pragma unroll
    for (int db = 0; db < D / 32; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;
    f32x16 sacc[BC / 32];  // S^T of the tile between its MFMA block and its softmax
    i32x4 pf[BC / 16];     // P of the tile between its softmax and its MFMA block

    // ---- direct global -> LDS tile loads (group B only) ------------------------------------
    // Loader wave lw, instruction i fills LDS 16-byte slots (i * LOADERS + lw) * 64 + lane.  Slot
    // p holds row p / CH, chunk (p % CH) ^ swizzle(row); since LOADERS * 64 / CH rows is a whole
    // number of swizzle periods, instruction i reads the bytes of instruction 0 shifted by
    // i * 4096, so one per-lane offset serves all of them (the shift goes to the scalar offset).
    const int lw = __builtin_amdgcn_readfirstlane(wave & 3);  // loader index within group B
    static_assert((LOADERS * 64 / CH) % 16 == 0, "loader rows must cover whole swizzle periods");
    const int lrow = (lw * 64 + lane) / CH;  // row of this lane's slot in instruction 0
    const int lch = (lw * 64 + lane) % CH;
    const int voff_k = lrow * D * 2 + ((lch ^ swz_k<D>(lrow)) << 4);
    const int voff_v = lrow * D * 2 + ((lch ^ swz_v<D>(lrow)) << 4);
    const i32x4 rsrc_k = make_rsrc(kp, (unsigned)seqlen * D * 2);
    const i32x4 rsrc_v = make_rsrc(vp, (unsigned)seqlen * D * 2);
    constexpr int ISTEP = LOADERS * 64 * 16;  // bytes per load instruction (all loader waves)
    // instruction II of the load of K (is_k) or V tile r into the LDS buffer at `dst`
    auto load_one = [&](auto k_tile, int r, unsigned dst, auto ii) XATTN_INLINE {
      constexpr bool is_k = decltype(k_tile)::value;
      constexpr int II = decltype(ii)::value;
      const int kbase = (t_lo + r) * BC;
      const unsigned lds = dst + lw * 1024;
      if (kbase + BC <= seqlen) {
        buffer_load_lds16_at<II * ISTEP, II * ISTEP>(is_k ? rsrc_k : rsrc_v, is_k ? voff_k : voff_v,
                                                     kbase * D * 2, lds);
      } else {  // last tile: rows past the end re-read the sequence's last row (finite data)
        const int row = lrow + II * (LOADERS * 64 / CH);
        const int crow = min(row, seqlen - 1 - kbase);
        const int sw = is_k ? swz_k<D>(row) : swz_v<D>(row);
        buffer_load_lds16_at<II * ISTEP, 0>(is_k ? rsrc_k : rsrc_v,
                                            crow * D * 2 + ((lch ^ sw) << 4), kbase * D * 2, lds);
      }
    };
    // instruction II of the load of a tile that lies wholly inside the sequence
    auto load_full = [&](auto k_tile, int r, unsigned dst, auto ii) XATTN_INLINE {
      constexpr bool is_k = decltype(k_tile)::value;
      constexpr int II = decltype(ii)::value;
      buffer_load_lds16_at<II * ISTEP, II * ISTEP>(is_k ? rsrc_k : rsrc_v, is_k ? voff_k : voff_v,
                                                   (t_lo + r) * BC * D * 2, dst + lw * 1024);
    };
    auto load_all = [&](auto k_tile, int r, unsigned dst) XATTN_INLINE {
      static_for<LI>([&](auto ii) XATTN_INLINE { load_one(k_tile, r, dst, ii); });
    };
    const std::true_type K_TILE;
    const std::false_type V_TILE;
    const unsigned k_lds0a = lds_address(k_lds0), k_lds1a = lds_address(k_lds1);
    const unsigned v_lds0a = lds_address(v_lds0), v_lds1a = lds_address(v_lds1);

    // ---- the three per-tile steps of a wave (r = tile index relative to t_lo) ---------------
    auto sees = [&](int r) XATTN_INLINE {
      const int k0 = (t_lo + r) * BC;
      return wave_active && k0 <= kw_hi && k0 + BC - 1 >= kw_lo;
    };
    auto step_scores = [&](int r, const char* kt) XATTN_INLINE {
      if (sees(r)) mma_scores<BF16, D, BC, PF>(kt, lo, qf, sacc);
    };
    // softmax of tile r; group B also issues the loads of U_{r+1} = {V_{r+1}, K_{r+2}}, one
    // instruction every SL exponentials (all at once when the tile is not visible to the wave)
    constexpr int NLD = 2 * LI, SL = (BC / 2) / NLD;
    // (the d = 128 sliding-window variant runs out of registers with the second softmax copy)
    constexpr bool SPREAD_LOADS = !(MODE == MASK_WINDOW && D > 64);
    static_assert((BC / 2) % NLD == 0, "loads must spread evenly over the softmax");
    auto step_softmax = [&](int r, bool ld_v, bool ld_k, unsigned vdst, unsigned kdst) XATTN_INLINE {
      // spread the loads only in the common case (both tiles wanted and whole); otherwise issue
      // them up front
      const bool spread = SPREAD_LOADS && ld_v && ld_k && (t_lo + r + 3) * BC <= seqlen;
      if (!spread) {
        if (ld_v) load_all(V_TILE, r + 1, vdst);
        if (ld_k) load_all(K_TILE, r + 2, kdst);
      }
      if (!sees(r)) {
        if (spread) {
          load_all(V_TILE, r + 1, vdst);
          load_all(K_TILE, r + 2, kdst);
        }
        return;
      }
      const int k0 = (t_lo + r) * BC;
      const bool need_mask = (k0 + BC > seqlen) || (wr >= 0 && k0 + BC - 1 > qw0 + wr) ||
                             (wl >= 0 && k0 < qw0 + 31 - wl);
      if (need_mask) mask_scores<BC>(sacc, k0, qrow, seqlen, wl, wr, hh);
      bool moved;
      float alpha;
      if (spread) {  // one load instruction every SL exponentials: V first, then K
        alpha = softmax_tile<BF16, BC>(sacc, pf, c2, m_run, l_run, moved, [&](int i) XATTN_INLINE {
          at_step<NLD, SL>(i, [&](auto l) XATTN_INLINE {
            constexpr int L = decltype(l)::value;
            sched_fence();  // keep the loads where they are placed
            if constexpr (L < LI)
              load_full(V_TILE, r + 1, vdst, std::integral_constant<int, L>{});
            else
              load_full(K_TILE, r + 2, kdst, std::integral_constant<int, L - LI>{});
            sched_fence();
          });
        });
      } else {
        alpha = softmax_tile<BF16, BC>(sacc, pf, c2, m_run, l_run, moved);
      }
      if (__builtin_amdgcn_ballot_w64(moved) != 0) scale_o<D>(oacc, alpha);  // wave-uniform
    };
    // an MFMA block: O += V_{rp}^T P_{rp}^T (when pv) and S_{rs} = K_{rs} Q^T (when sc),
    // interleaved when the wave needs both
    auto step_mfma = [&](bool pv, int rp, const char* vt, bool sc, int rs,
                         const char* kt) XATTN_INLINE {
      const bool dp = pv && sees(rp), ds = sc && sees(rs);
      if (dp && ds) {
        mma_pv_scores<BF16, D, BC, PF>(vt, pf, oacc, kt, qf, sacc, lo);
      } else {
        if (dp) mma_pv<BF16, D, BC, PF>(vt, lo, pf, oacc);
        if (ds) mma_scores<BF16, D, BC, PF>(kt, lo, qf, sacc);
      }
    };

    // ---- prologue: K_0 (buffer 1), V_0 and K_1 (buffer 0) ---------------------------------
    if (!grp_a) {
      load_all(K_TILE, 0, k_lds1a);
      load_all(V_TILE, 0, v_lds0a);
      if (n > 1) load_all(K_TILE, 1, k_lds0a);
    }
    q_arrived<D>(qf);
    if (!grp_a) wait_vmem();
    block_barrier();
    if (grp_a) step_scores(0, k_lds1);

    // ---- main loop: two half-phases per tile, buffer parity P = j & 1 known at compile time ----
    auto iteration = [&](int j, auto parity) XATTN_INLINE {
      constexpr int P = decltype(parity)::value;
      char* const kP = P ? k_lds1 : k_lds0;  // holds K_{j+1}
      char* const kQ = P ? k_lds0 : k_lds1;  // holds K_j, then receives K_{j+2}
      char* const vP = P ? v_lds1 : v_lds0;  // holds V_j
      char* const vQ = P ? v_lds0 : v_lds1;  // holds V_{j-1}, then receives V_{j+1}
      const unsigned kQa = P ? k_lds0a : k_lds1a;
      const unsigned vQa = P ? v_lds0a : v_lds1a;
      // half-phase 2j
      if (grp_a) {
        if (j < n) step_softmax(j, false, false, 0, 0);
      } else {
        __builtin_amdgcn_s_setprio(2);  // MFMA block: win issue over the partner's softmax
        step_mfma(j >= 1, j - 1, vQ, j < n, j, kQ);
        __builtin_amdgcn_s_setprio(0);
      }
      if (j >= 1) wait_vmem();  // group B's loads of U_j (issued at half-phase 2j-1)
      block_barrier();
      // half-phase 2j+1
      if (grp_a) {
        __builtin_amdgcn_s_setprio(2);
        if (j < n) step_mfma(true, j, vP, j + 1 < n, j + 1, kP);
        __builtin_amdgcn_s_setprio(0);
      } else {
        if (j < n) step_softmax(j, j + 1 < n, j + 2 < n, vQa, kQa);
      }
      block_barrier();
    };
    for (int j = 0; j <= n; j += 2) {
      iteration(j, std::integral_constant<int, 0>{});
      if (j + 1 <= n) iteration(j + 1, std::integral_constant<int, 1>{});
    }

    // all waves are past the sweep's last barrier and no tile load is in flight: the four
    // tile buffers are free, 8 KiB (32 rows of 2D bytes at d = 128) per wave
    static_assert(8 * 32 * D * 2 <= 4 * TILEB, "the output rows fit the tile buffers");
    char* const region = (wave >> 1) == 0   ? k_lds0
                         : (wave >> 1) == 1 ? k_lds1
                         : (wave >> 1) == 2 ? v_lds0
                                            : v_lds1;
    if (wave_active)
      store_rows_staged<BF16, D>(a, wrow0, qrow, seqlen, oacc, m_run, l_run,
                                 region + (wave & 1) * (TILEB / 2));
  };
  run_tile(w0);
  if (light >= 0) {  // the pair's second tile, once every wave has read its staged rows back
    block_barrier();
    Work w1 = w0;
    w1.tile = light;
    run_tile(w1);
  }
}

}  // namespace xattn
