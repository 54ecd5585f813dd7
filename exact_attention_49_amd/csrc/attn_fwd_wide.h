// Exact-attention forward kernel for gfx950 and large head dims (256, 512).
//
// At d = 512 the output accumulator of 32 query rows is 256 fp32 values per lane, and Q is 128
// more, so a wave needs the whole register file of its SIMD (one wave per SIMD).  The output
// accumulators O^T live in the 256 accumulation registers (AGPRs): the O^T += V^T P^T MFMAs are
// issued through a small inline-assembly wrapper with AGPR operands, and the compiler selects
// every other MFMA (the scores S^T = K Q^T) in VGPR form (compile flag of this unit), so Q, S,
// P and the operand buffers fit in the 256 VGPRs without copies.  The compiler cannot see the
// MFMAs inside the assembly, so the few places where VALU code touches O (the rare rescale and
// the epilogue) are preceded by explicit wait states.
//
// A workgroup is 4 waves, 128 query rows of one (batch|sequence, head) and 32-key K/V tiles,
// double-buffered in LDS and loaded by all four waves straight from global memory
// (buffer_load ... lds): the loads of tile t+1 are issued before tile t is consumed and waited
// for after it, with one barrier per tile.  The math per tile is in attn_common.h.
#pragma once

#include <type_traits>

#include "attn_common.h"

namespace xattn {

struct WideShape {
  static constexpr int NW = 4, NT = 256, BR = 128, BC = 32;
};

// LDS operand reads run PFW - 1 MFMAs ahead of their use: with one wave per SIMD nothing else
// covers the LDS latency (measured on MI355X at d = 512: depth 5 is about 1% faster than 3)
constexpr int PFW = 5;

// acc += a * b with acc in AGPRs (v_mfma_f32_32x32x16).  The s_nop covers an operand written
// by a VALU instruction just before; an MFMA that reads its own previous result as the
// accumulator needs no wait.
template <bool BF16>
__device__ __forceinline__ void mfma_agpr(f32x16& acc, i32x4 a, i32x4 b) {
  if constexpr (BF16)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last MFMA that wrote an AGPR accumulator and VALU access to it.
template <int N>
__device__ __forceinline__ void agpr_settle(f32x16 (&o)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(o[i]));
}

// O *= alpha one 32-column block at a time (AGPR -> VGPR -> AGPR), so that only one block is
// held in VGPRs.
template <int N>
__device__ __forceinline__ void scale_o_agpr(f32x16 (&o)[N], float alpha) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    f32x16 t = o[i];
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] *= alpha;
    asm volatile("" : "+v"(t));
    o[i] = t;
    asm volatile("" : "+a"(o[i]));
  }
}

// O^T += V^T P^T with O^T in AGPRs; operand reads prefetched PF - 1 steps ahead.
template <bool BF16, int D, int BC, int PF = 3>
__device__ __forceinline__ void mma_pv_agpr(const char* vt, const LaneOffsets<D>& lo,
                                            i32x4 (&pf)[BC / 16], f32x16 (&o)[D / 32]) {
  constexpr int ROWB = D * 2, DB = D / 32, N = (BC / 16) * DB;
  // P was just written by VALU instructions: order them before the MFMAs with wait states
  asm volatile("s_nop 4" : "+v"(pf[0]), "+v"(pf[BC / 16 - 1]));
  auto read = [&](int i) {
    const char* p = vt + lo.vofs(i % DB, i / DB);
    const i32x2 a = __builtin_bit_cast(i32x2, lds_read_tr(p));
    const i32x2 b = __builtin_bit_cast(i32x2, lds_read_tr(p + 8 * ROWB));
    return (i32x4){a[0], a[1], b[0], b[1]};
  };
  i32x4 buf[PF];
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) buf[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + PF - 1 < N) buf[(i + PF - 1) % PF] = read(i + PF - 1);
    sched_fence();
    mfma_agpr<BF16>(o[i % DB], buf[i % PF], pf[i / DB]);
    sched_fence();
  }
}

// SPLIT: split-KV mode (the workgroup sweeps its split's share of the key tiles and writes
// fp32 partial results; see FwdArgs).
template <bool BF16, int D, int MODE, bool SPLIT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void attn_fwd_wide_kernel(FwdArgs a) {
  constexpr int BR = WideShape::BR, BC = WideShape::BC, NT = WideShape::NT;
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;            // bytes per K (or V) tile
  constexpr int LI = BC * CH / NT;            // load instructions per matrix per wave
  constexpr int R = NT / CH;                  // rows covered by one load instruction (all waves)
  constexpr int NKO = R >= 16 ? 1 : 16 / R;   // distinct per-lane K load offsets (swizzle period)
  constexpr int NVO = R >= 4 ? 1 : 4 / R;     // distinct per-lane V load offsets
  static_assert(D == 256 || D == 512, "wide shape is for head dims 256 and 512");
  static_assert(BC * CH % NT == 0 && LI % NKO == 0 && LI % NVO == 0, "tile split");

  __shared__ __attribute__((aligned(1024))) char k_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int qw0 = q0 + wave * 32;
  const int q_last = min(q0 + BR, seqlen) - 1;
  int k_lo = 0, k_hi = seqlen - 1;
  if (wl >= 0) k_lo = max(0, q0 - wl);
  if (wr >= 0) k_hi = min(seqlen - 1, q_last + wr);
  int t_lo = k_lo / BC;
  int n = k_hi / BC - t_lo + 1;
  if constexpr (SPLIT) split_tiles(a, w.split, t_lo, n);

  const bool wave_active = qw0 < seqlen;
  const int qw_last = min(qw0 + 32, seqlen) - 1;
  int kw_lo = 0, kw_hi = seqlen - 1;
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

  // ---- tile loads: instruction i of wave w fills 16-byte LDS slots (i * 4 + w) * 64 + lane ----
  int koff[NKO], voff[NVO];
#pragma unroll
  for (int i = 0; i < NKO; ++i) {
    const int p = (i * 4 + wave) * 64 + lane;
    koff[i] = (p / CH) * ROWB + (((p % CH) ^ swz_k<D>(p / CH)) << 4);
  }
#pragma unroll
  for (int i = 0; i < NVO; ++i) {
    const int p = (i * 4 + wave) * 64 + lane;
    voff[i] = (p / CH) * ROWB + (((p % CH) ^ swz_v<D>(p / CH)) << 4);
  }
  const i32x4 rsrc_k = make_rsrc(kp, (unsigned)seqlen * ROWB);
  const i32x4 rsrc_v = make_rsrc(vp, (unsigned)seqlen * ROWB);
  auto load_tile = [&](int t, unsigned kdst, unsigned vdst) {
    const int kbase = t * BC;
    if (kbase + BC <= seqlen) {
#pragma unroll
      for (int i = 0; i < LI; ++i) {
        const int dst = (i * 4 + wave) * 1024;
        buffer_load_lds16(rsrc_k, koff[i % NKO], kbase * ROWB + (i / NKO) * NKO * R * ROWB,
                          kdst + dst);
        buffer_load_lds16(rsrc_v, voff[i % NVO], kbase * ROWB + (i / NVO) * NVO * R * ROWB,
                          vdst + dst);
      }
    } else {  // last tile: rows past the end re-read the sequence's last row (finite data)
#pragma unroll
      for (int i = 0; i < LI; ++i) {
        const int p = (i * 4 + wave) * 64 + lane;
        const int row = p / CH, c = p % CH;
        const int crow = min(row, seqlen - 1 - kbase);
        const int dst = (i * 4 + wave) * 1024;
        buffer_load_lds16(rsrc_k, crow * ROWB + ((c ^ swz_k<D>(row)) << 4), kbase * ROWB,
                          kdst + dst);
        buffer_load_lds16(rsrc_v, crow * ROWB + ((c ^ swz_v<D>(row)) << 4), kbase * ROWB,
                          vdst + dst);
      }
    }
  };

  // instruction II of the K (or V) load of a tile that lies wholly inside the sequence
  const unsigned wave_lds = wave * 1024;
  auto load_full = [&](auto k_tile, int t, unsigned dst, auto ii) XATTN_INLINE {
    constexpr int II = decltype(ii)::value;
    if constexpr (decltype(k_tile)::value)
      buffer_load_lds16_at<II * 4 * 1024, (II / NKO) * NKO * R * ROWB>(
          rsrc_k, koff[II % NKO], t * BC * ROWB, dst + wave_lds);
    else
      buffer_load_lds16_at<II * 4 * 1024, (II / NVO) * NVO * R * ROWB>(
          rsrc_v, voff[II % NVO], t * BC * ROWB, dst + wave_lds);
  };

  // One K/V tile: S^T, mask, online softmax, O^T update.  With ld, the loads of tile t + 1
  // (into kdst / vdst) are slipped between the score MFMAs, one instruction every SH of them;
  // a partial next tile or a tile this wave does not see gets them all up front.
  constexpr int NS = (D / 16) * (BC / 32), SH = NS / (2 * LI);
  static_assert(NS % (2 * LI) == 0, "loads must spread evenly over the score MFMAs");
  auto consume = [&](int t, const char* kt, const char* vt, bool ld, unsigned kdst,
                     unsigned vdst) XATTN_INLINE {
    const int k0 = t * BC;
    const bool vis = wave_active && k0 <= kw_hi && k0 + BC - 1 >= kw_lo;
    const bool spread = ld && vis && (t + 2) * BC <= seqlen;
    if (ld && !spread) load_tile(t + 1, kdst, vdst);
    if (!vis) return;  // nothing visible
    f32x16 sacc[BC / 32];
    if (spread) {
      mma_scores<BF16, D, BC, PFW>(kt, lo, qf, sacc, [&](auto i) XATTN_INLINE {
        constexpr int I = decltype(i)::value;
        if constexpr (I % SH == 0) {
          constexpr int L = I / SH;  // K instructions first, then V
          sched_fence();
          if constexpr (L < LI)
            load_full(std::true_type{}, t + 1, kdst, std::integral_constant<int, L>{});
          else
            load_full(std::false_type{}, t + 1, vdst, std::integral_constant<int, L - LI>{});
          sched_fence();
        }
      });
    } else {
      mma_scores<BF16, D, BC, PFW>(kt, lo, qf, sacc);
    }
    const bool need_mask = (k0 + BC > seqlen) || (wr >= 0 && k0 + BC - 1 > qw0 + wr) ||
                           (wl >= 0 && k0 < qw0 + 31 - wl);
    if (need_mask) mask_scores<BC>(sacc, k0, qrow, seqlen, wl, wr, hh);
    i32x4 pf[BC / 16];
    // the weights against the running reference when no row needs it moved (the common
    // case); otherwise the full online-softmax step: on S as it is while some row has seen no
    // key yet, else on S recomputed from the K tile, still in LDS
    if (!softmax_tile_fast<BF16, BC>(sacc, pf, c2, m_run, l_run)) {
      if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0) {
        mma_scores<BF16, D, BC, PFW>(kt, lo, qf, sacc);
        if (need_mask) mask_scores<BC>(sacc, k0, qrow, seqlen, wl, wr, hh);
      }
      bool moved;
      const float alpha = softmax_tile<BF16, BC>(sacc, pf, c2, m_run, l_run, moved);
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {  // wave-uniform, rare
        agpr_settle(oacc);
        scale_o_agpr(oacc, alpha);
      }
    }
    mma_pv_agpr<BF16, D, BC, PFW>(vt, lo, pf, oacc);
  };

  // ---- sweep: tiles alternate between the two buffers (parity known at compile time) -------
  const int t_hi = t_lo + n - 1;
  const unsigned k0a = lds_address(k_lds0), k1a = lds_address(k_lds1);
  const unsigned v0a = lds_address(v_lds0), v1a = lds_address(v_lds1);
  if (n > 0) load_tile(t_lo, k0a, v0a);
  q_arrived<D>(qf);
  wait_vmem();
  block_barrier();
  for (int t = t_lo; t <= t_hi; t += 2) {
    consume(t, k_lds0, v_lds0, t + 1 <= t_hi, k1a, v1a);
    wait_vmem();
    block_barrier();
    if (t + 1 > t_hi) break;
    consume(t + 1, k_lds1, v_lds1, t + 2 <= t_hi, k0a, v0a);
    wait_vmem();
    block_barrier();
  }

  // all waves are past the last barrier: the tile buffers are free, one per wave
  agpr_settle(oacc);
  char* const region = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
  static_assert(TILEB == 32 * ROWB, "a tile buffer holds one wave's 32 output rows");
  if (!wave_active) return;
  if constexpr (SPLIT)
    store_rows_partial<D>(a, w.split, w.row0, qrow, seqlen, hh, oacc, m_run, l_run);
  else
    store_rows_staged<BF16, D>(a, w.row0, qrow, seqlen, oacc, m_run, l_run, region);
}

}  // namespace xattn
