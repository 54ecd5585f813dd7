// Generic exact-attention forward kernel for gfx950: NW waves, each owning 32 query rows of one
// (batch|sequence, head) for the whole K/V sweep.  K/V tiles of BC keys reach LDS either staged
// global -> registers -> LDS with 16-byte accesses (STAGES = 2: the next tile's global loads are
// in flight while the current tile is consumed), or with DMA straight from global memory into
// LDS (buffer_load ... lds), STAGES - 1 tiles ahead; one barrier per tile.  Only tiles that
// cross a mask edge or the end of the sequence evaluate the mask, and a wave skips tiles its
// rows cannot see.  The math per tile is in attn_common.h.
#pragma once

#include "attn_common.h"

namespace xattn {

// Tile shape: NW waves of 32 query rows, BC keys per K/V tile, STAGES LDS buffers, at least
// WPE waves per SIMD (which caps the registers per wave at 512 / WPE), and DMA for direct
// global -> LDS tile loads instead of staging through registers.
template <int NW_, int BC_, int STAGES_, int WPE_, bool DMA_ = false>
struct Tile {
  static constexpr int NW = NW_, BC = BC_, STAGES = STAGES_, WPE = WPE_;
  static constexpr bool DMA = DMA_;
  static constexpr int BR = NW * 32;  // query rows per workgroup
  static constexpr int NT = NW * 64;  // threads per workgroup
};

// SPLIT: split-KV mode (the workgroup sweeps its split's share of the key tiles and writes
// fp32 partial results; see FwdArgs).
template <bool BF16, int D, int MODE, class C, bool SPLIT = false>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE)))
void attn_fwd_kernel(FwdArgs a) {
  constexpr int BC = C::BC, STAGES = C::STAGES;
  constexpr int NT = C::NT, BR = C::BR;
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int ROWB = D * 2;          // bytes per row
  constexpr int TILEB = BC * ROWB;     // bytes per K (or V) tile
  constexpr int LPT = BC * CH / NT;    // 16-byte chunks per thread per matrix per tile
  static_assert(BC * CH % NT == 0, "tile must split evenly over the threads");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * 2 * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  Work w;
  if (const Decoded dc = decode_work<BR, MODE, SPLIT>(a, w); dc != Decoded::Run) {
    if (dc == Decoded::Malformed) fill_malformed_fwd<D, SPLIT>(a, w);
    return;
  }
  const int seqlen = w.seqlen;
  int wl, wr;
  mode_windows<MODE>(a, wl, wr);

  const int q0 = w.tile * BR;
  const int qw0 = q0 + wave * 32;                      // first row of this wave
  const int q_last = min(q0 + BR, seqlen) - 1;         // last valid row of the workgroup
  int k_lo = 0, k_hi = seqlen - 1;                     // keys any valid row can see
  if (wl >= 0) k_lo = max(0, q0 - wl);
  if (wr >= 0) k_hi = min(seqlen - 1, q_last + wr);
  int t_lo = k_lo / BC, n_tiles = k_hi / BC - t_lo + 1;
  if constexpr (SPLIT) split_tiles(a, w.split, t_lo, n_tiles);
  const int t_hi = t_lo + n_tiles - 1;

  const bool wave_active = qw0 < seqlen;
  const int qw_last = min(qw0 + 32, seqlen) - 1;
  int kw_lo = 0, kw_hi = seqlen - 1;                   // keys this wave's rows can see
  if (wl >= 0) kw_lo = max(0, qw0 - wl);
  if (wr >= 0) kw_hi = min(seqlen - 1, qw_last + wr);

  const uint16_t* __restrict__ kp = a.k + w.kv_row0 * D;
  const uint16_t* __restrict__ vp = a.v + w.kv_row0 * D;
  const int qrow = qw0 + l32;

  i32x4 qf[D / 16];
  load_q_nowait<D>(a.q + w.row0 * D, qrow, seqlen, hh, qf);  // waited for after the first tile loads
  const LaneOffsets<D> lo = lane_offsets<D>(lane);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;

  // ---- global -> registers -> LDS staging of one K/V tile -------------------------------
  i32x4 stage_k[LPT], stage_v[LPT];
  auto gload = [&](int t) {
    const int kbase = t * BC;
    if (kbase + BC <= seqlen) {  // whole tile inside the sequence
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const int id = tid + u * NT;
        const int r = id / CH, c = id % CH;
        stage_k[u] = ((const i32x4*)(kp + (long)(kbase + r) * D))[c];
        stage_v[u] = ((const i32x4*)(vp + (long)(kbase + r) * D))[c];
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int id = tid + u * NT;
      const int r = id / CH, c = id % CH;
      const int key = kbase + r;
      if (key < seqlen) {
        stage_k[u] = ((const i32x4*)(kp + (long)key * D))[c];
        stage_v[u] = ((const i32x4*)(vp + (long)key * D))[c];
      } else {  // past the end of the sequence: zeros keep P V finite (P is 0 there)
        stage_k[u] = (i32x4){0, 0, 0, 0};
        stage_v[u] = (i32x4){0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int s) {
    char* kt = smem + s * 2 * TILEB;
    char* vt = kt + TILEB;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int id = tid + u * NT;
      const int r = id / CH, c = id % CH;
      *(i32x4*)(kt + r * ROWB + ((c ^ swz_k<D>(r)) << 4)) = stage_k[u];
      *(i32x4*)(vt + r * ROWB + ((c ^ swz_v<D>(r)) << 4)) = stage_v[u];
    }
  };

  // ---- one K/V tile: S^T, mask, online softmax, O^T update --------------------------------
  // (s: the LDS stage, an int or, for the unrolled two-stage sweep, a compile-time constant)
  auto consume = [&](int t, auto s) {
    const int k0 = t * BC;
    if (!wave_active || k0 > kw_hi || k0 + BC - 1 < kw_lo) return;  // nothing visible
    const char* kt = smem + s * 2 * TILEB;
    const char* vt = kt + TILEB;
    const bool need_mask = (k0 + BC > seqlen) || (wr >= 0 && k0 + BC - 1 > qw0 + wr) ||
                           (wl >= 0 && k0 < qw0 + 31 - wl);
    f32x16 sacc[BC / 32];
    auto scores = [&]() XATTN_INLINE {
      __builtin_amdgcn_s_setprio(1);  // MFMA runs win issue over the other waves' VALU work
      mma_scores<BF16, D, BC>(kt, lo, qf, sacc);
      __builtin_amdgcn_s_setprio(0);
      if (need_mask) mask_scores<BC>(sacc, k0, qrow, seqlen, wl, wr, hh);
    };
    scores();
    // the first V operands, read now so that their latency overlaps the softmax (no room for
    // them in the d = 64 kernel's 128 registers)
    constexpr bool HEAD = D >= 128;
    PvHead<D> vhead;
    if constexpr (HEAD) vhead = pv_head<D>(vt, lo);
    i32x4 pf[BC / 16];
    // the weights against the running reference when no row needs it moved (the common
    // case); otherwise the full online-softmax step: on S as it is while some row has seen no
    // key yet (softmax_tile_fast then leaves it untouched), else on S recomputed from the K
    // tile, still in LDS
    if (!softmax_tile_fast<BF16, BC>(sacc, pf, c2, m_run, l_run)) {
      if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0) scores();
      bool moved;
      const float alpha = softmax_tile<BF16, BC>(sacc, pf, c2, m_run, l_run, moved);
      if (__builtin_amdgcn_ballot_w64(moved) != 0) scale_o<D>(oacc, alpha);  // wave-uniform
    }
    __builtin_amdgcn_s_setprio(1);
    mma_pv<BF16, D, BC>(vt, lo, pf, oacc, NoHook(), HEAD ? &vhead : nullptr);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- C::DMA: direct global -> LDS loads, STAGES - 1 tiles in flight --------------------
  // Instruction i of wave w fills the 16-byte LDS slots (i * NW + w) * 64 + lane of a tile:
  // slot p holds row p / CH, chunk (p % CH) ^ swizzle(row).  One instruction round covers
  // NW * 64 / CH rows, a whole number of swizzle periods, so instruction i reads the bytes of
  // instruction 0 shifted by i rounds and one per-lane offset serves all of them.
  constexpr int NW = C::NW;
  constexpr int RROWS = NW * 64 / CH;  // rows per instruction round
  static_assert(!C::DMA || RROWS % 16 == 0, "rounds must cover whole swizzle periods");
  const int drow = (wave * 64 + lane) / CH, dch = (wave * 64 + lane) % CH;
  const int dvoff_k = drow * ROWB + ((dch ^ swz_k<D>(drow)) << 4);
  const int dvoff_v = drow * ROWB + ((dch ^ swz_v<D>(drow)) << 4);
  const i32x4 rsrc_k = make_rsrc(kp, (unsigned)seqlen * ROWB);
  const i32x4 rsrc_v = make_rsrc(vp, (unsigned)seqlen * ROWB);
  const unsigned smem_a = lds_address(smem);
  auto dma_tile = [&](int t, int s) XATTN_INLINE {
    const int kbase = t * BC;
    const unsigned kdst = smem_a + s * 2 * TILEB + wave * 1024, vdst = kdst + TILEB;
    if (kbase + BC <= seqlen) {
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        buffer_load_lds16_at<I * NW * 1024, I * RROWS * ROWB>(rsrc_k, dvoff_k, kbase * ROWB, kdst);
        buffer_load_lds16_at<I * NW * 1024, I * RROWS * ROWB>(rsrc_v, dvoff_v, kbase * ROWB, vdst);
      });
    } else {  // last tile: rows past the end re-read the sequence's last row (finite data)
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        const int row = drow + I * RROWS;
        const int crow = min(row, seqlen - 1 - kbase);
        buffer_load_lds16_at<I * NW * 1024, 0>(
            rsrc_k, crow * ROWB + ((dch ^ swz_k<D>(row)) << 4), kbase * ROWB, kdst);
        buffer_load_lds16_at<I * NW * 1024, 0>(
            rsrc_v, crow * ROWB + ((dch ^ swz_v<D>(row)) << 4), kbase * ROWB, vdst);
      });
    }
  };
  // wait for the loads of all but the newest tile (when `newer`, a later tile's 2 * LPT load
  // instructions may stay outstanding)
  auto wait_older = [&](bool newer) XATTN_INLINE {
    if (newer)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPT) : "memory");
    else
      wait_vmem();
  };

  // ---- the sweep over K/V tiles ---------------------------------------------------------
  if constexpr (C::DMA) {
    static_assert(STAGES == 2 || STAGES == 3, "direct loads keep one or two tiles in flight");
    constexpr int LEAD = STAGES - 1;
    if (n_tiles > 0) dma_tile(t_lo, 0);
    if (LEAD == 2 && n_tiles > 1) dma_tile(t_lo + 1, 1);
    q_arrived<D>(qf);
    wait_older(LEAD == 2 && n_tiles > 1);
    block_barrier();
    if constexpr (STAGES == 2) {
      sweep_two_stages(t_lo, t_hi, [&](int t, auto stage) XATTN_INLINE {
        constexpr int S = decltype(stage)::value;
        if (t + 1 <= t_hi) dma_tile(t + 1, 1 - S);  // stage 1 - S held tile t - 1
        consume(t, stage);
        if (t + 1 <= t_hi) wait_older(false);
        block_barrier();
      });
    } else {
      int s = 0;
      for (int t = t_lo; t <= t_hi; ++t) {
        // stage (s + LEAD) % STAGES held tile t - 1, free since the last barrier
        const int sl = s + LEAD < STAGES ? s + LEAD : s + LEAD - STAGES;
        if (t + LEAD <= t_hi) dma_tile(t + LEAD, sl);
        consume(t, s);
        if (t + 1 <= t_hi) wait_older(LEAD == 2 && t + 2 <= t_hi);
        block_barrier();
        s = s + 1 < STAGES ? s + 1 : 0;
      }
    }
  } else if constexpr (STAGES == 2) {
    if (n_tiles > 0) gload(t_lo);
    q_arrived<D>(qf);
    if (n_tiles > 0) lstore(0);
    __syncthreads();
    for (int t = t_lo; t <= t_hi; ++t) {
      const int s = (t - t_lo) & 1;
      if (t < t_hi) gload(t + 1);
      consume(t, s);
      if (t < t_hi) lstore(s ^ 1);
      __syncthreads();
    }
  } else {
    q_arrived<D>(qf);
    for (int t = t_lo; t <= t_hi; ++t) {
      if (t > t_lo) __syncthreads();
      gload(t);
      lstore(0);
      __syncthreads();
      consume(t, 0);
    }
  }

  if (!wave_active) return;
  if constexpr (SPLIT) {
    store_rows_partial<D>(a, w.split, w.row0, qrow, seqlen, hh, oacc, m_run, l_run);
  } else {
    // every wave is past the sweep's last barrier and no tile load is in flight: the tile
    // buffers are free, 32 rows of 2D bytes per wave
    static_assert(BR * ROWB <= STAGES * 2 * TILEB, "the output rows fit the tile buffers");
    store_rows_staged<BF16, D>(a, w.row0, qrow, seqlen, oacc, m_run, l_run,
                               smem + __builtin_amdgcn_readfirstlane(wave) * 32 * ROWB);
  }
}

}  // namespace xattn
