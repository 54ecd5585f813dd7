// gfx950 exact-attention backward: dQ, dK and dV from Q, K, V, O, the forward's LSE and dO.
//
// What is computed (page "mainloop_bwd_sm90_tma_gmma_ws.hpp", the backward `mma`): with
// S = scale * Q K^T under the forward's mask and P recomputed from S and the stored LSE,
//   P_ij = exp(S_ij - LSE_i),  dP = dO V^T,  dS = P * (dP - dPsum_i),
//   dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K,
// where dPsum_i = sum_j P_ij dP_ij = dO_i . O_i (the pages take it as an input; this library
// forms it from dO and O).  With grouped K/V heads the dK and dV of a key/value head sum the
// contributions of every query head of its group.
//
// Two kernels, both deterministic (no atomics):
//  * attn_bwd_dq_kernel: one workgroup per q-tile, as the forward.  Each wave keeps its 32
//    query rows of Q and dO in registers and sweeps the visible K/V tiles:
//    S^T = K Q^T and dP^T = V dO^T (lane = query, as in the forward), dS^T from them, and
//    dQ^T += K^T dS^T (the forward's O^T += V^T P^T with K in V's place).  It also writes
//    dPsum for its rows, which the second kernel reads.
//  * attn_bwd_dkdv_kernel: one workgroup per tile of 128 keys of one key/value head, two
//    waves per 32 keys, sweeping the visible q-tiles of every query head of the group.  The
//    "dV wave" keeps the keys' K rows in registers and forms S = Q K^T (lane = key), P and
//    dV^T += dO^T P; it hands P to the "dK wave" through LDS.  The dK wave keeps the V rows
//    and, one q-tile behind, forms dP = dO V^T, dS and dK^T += Q^T dS.  The same building
//    blocks as the forward, with the roles of queries and keys exchanged: the mask is the
//    forward's with the window bounds swapped (key j sees query i iff
//    j - window_right <= i <= j + window_left).
// Both kernels load their tiles straight from global memory into LDS (buffer_load ... lds).
// An operand read both row-wise (MFMA A operand) and transposed (ds_read_b64_tr_b16) is
// stored once, with the swizzle that serves both reads (swz_rt).  The dQ kernel double-buffers
// K and V; the dK/dV kernel keeps three stages of Q, dO and the rows' LSE (log2 units, which
// the dQ kernel writes beside dPsum) and dPsum, so that each tile's loads are in flight for a
// step and a half.
#pragma once

#include "attn_common.h"

namespace xattn {

struct BwdArgs {
  FwdArgs f;               // q, k, v, o (read), lse (read, natural log), sizes, mask, heads
  const uint16_t* dout;    // dO, laid out as q
  uint16_t* dq;            // laid out as q
  uint16_t* dk;            // laid out as k
  uint16_t* dv;            // laid out as v
  float* dpsum;            // [rows of q]: written by the dQ kernel, read by the dK/dV kernel
  float* lse2;             // [rows of q]: the LSE in log2 units, written and read likewise
  float scale;             // softmax scale (dQ and dK are multiplied by it)
  int ktiles_per_head;     // key-tile slots per key/value head (dK/dV kernel); the q-tile
                           // slots of the dQ kernel are f.tiles_per_head
};

struct BwdShape {
  // dQ kernel: DQ_NW waves of 32 query rows share each K/V tile of BC keys, DQ_WPE waves per
  // SIMD
  static constexpr int DQ_NW = 8, DQ_NT = 64 * DQ_NW, DQ_WPE = 2;
  static constexpr int BR = 32 * DQ_NW;  // query rows per workgroup
  static constexpr int BC = 64;          // keys per K/V tile
  // dK/dV kernel: NW waves, two per block of 32 keys (one accumulates dV, the other dK), WPE
  // waves per SIMD, Q/dO tiles of BQ rows
  static constexpr int NW = 8, NT = 64 * NW, WPE = 2;
  static constexpr int BK = 32 * (NW / 2);  // keys per workgroup
  static constexpr int BQ = 64;          // query rows per Q/dO tile
};

// Sum of the eight products of two packed 16-bit vectors, in fp32.
template <bool BF16>
__device__ __forceinline__ float dot8(i32x4 x, i32x4 y) {
  float acc = 0.f;
  if constexpr (BF16) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, x), b = __builtin_bit_cast(bf16x8, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)a[i], (float)b[i], acc);
  } else {
    const f16x8 a = __builtin_bit_cast(f16x8, x), b = __builtin_bit_cast(f16x8, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)a[i], (float)b[i], acc);
  }
  return acc;
}

// Packs score-layout fp32 values (two 32-row blocks of 16 registers per 64) to the 16-bit
// B operand of a transposed-accumulator product, as the forward packs P.
template <bool BF16, int BN>
__device__ __forceinline__ void pack_operand(const f32x16 (&s)[BN / 32], i32x4 (&pf)[BN / 16]) {
#pragma unroll
  for (int kc = 0; kc < BN / 16; ++kc) {
    const int kb = kc >> 1, o8 = (kc & 1) * 8;
    pf[kc] = (i32x4){(int)Elt<BF16>::pack2(s[kb][o8 + 0], s[kb][o8 + 1]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 2], s[kb][o8 + 3]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 4], s[kb][o8 + 5]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 6], s[kb][o8 + 7])};
  }
}

constexpr float kBwdLog2e = 1.44269504088896340736f;

// The forward's natural-log LSE in base-2 units; +inf for a row with no visible key (and for
// rows past the end), so that exp2(s * c2 - lse2) is 0 there.
__device__ __forceinline__ float lse_to_log2(float lse) {
  return lse > -INFINITY ? lse * kBwdLog2e : INFINITY;
}

// ---------------------------------------------------------------------------------------------
// dQ (and dPsum)
// ---------------------------------------------------------------------------------------------

template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(BwdShape::DQ_NT)
__attribute__((amdgpu_waves_per_eu(BwdShape::DQ_WPE)))
void attn_bwd_dq_kernel(BwdArgs ba) {
  const FwdArgs& a = ba.f;
  constexpr int BR = BwdShape::BR, BC = BwdShape::BC, NT = BwdShape::DQ_NT;
  constexpr int CH = D / 8, ROWB = D * 2, TILEB = BC * ROWB, LPT = BC * CH / NT;
  constexpr int STAGEB = 2 * TILEB;  // K, V (shared swizzle: K is read both ways)
  static_assert(BC * CH % NT == 0, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  Work w;
  if (const Decoded dc = decode_work<BR, MODE>(a, w); dc != Decoded::Run) {
    if (dc == Decoded::Malformed)  // dQ rows of the sequence: NaN
      fill_nan_rows(ba.dq, w.row0 + w.bad_lo, w.row0 + w.bad_hi, D / 8);
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
  const int t_lo = k_lo / BC, t_hi = k_hi / BC;

  const bool wave_active = qw0 < seqlen;
  const int qw_last = min(qw0 + 32, seqlen) - 1;
  int kw_lo = 0, kw_hi = seqlen - 1;
  if (wl >= 0) kw_lo = max(0, qw0 - wl);
  if (wr >= 0) kw_hi = min(seqlen - 1, qw_last + wr);

  const uint16_t* __restrict__ kp = a.k + w.kv_row0 * D;
  const uint16_t* __restrict__ vp = a.v + w.kv_row0 * D;
  const int qrow = qw0 + l32;
  const long grow = w.row0 + qrow;  // global row of the lane's query

  i32x4 qf[D / 16], dof[D / 16];
  load_q<D>(a.q + w.row0 * D, qrow, seqlen, hh, qf);
  load_q<D>(ba.dout + w.row0 * D, qrow, seqlen, hh, dof);
  float dps;
  {
    i32x4 of[D / 16];
    load_q<D>(a.o + w.row0 * D, qrow, seqlen, hh, of);
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) part += dot8<BF16>(dof[c], of[c]);
    dps = halves_sum(part);
  }
  const float lse2 = qrow < seqlen ? lse_to_log2(a.lse[grow]) : INFINITY;
  if (hh == 0 && qrow < seqlen) {
    ba.dpsum[grow] = dps;
    ba.lse2[grow] = lse2;
  }
  const LaneOffsets<D> lo = lane_offsets<D, true>(lane);
  const float c2 = a.scale_log2;

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  // K/V tiles go straight from global memory into LDS (buffer_load ... lds), with the swizzle
  // that serves both the row reads and K's transpose reads.  Instruction i of wave w fills the 16-byte LDS slots
  // (i * NW + w) * 64 + lane of a tile (row p / CH, chunk position p % CH): the lane fetches
  // the chunk that position holds.  One instruction round covers RROWS rows, a whole number of
  // swizzle periods, so instruction i reads instruction 0's bytes shifted by i rounds.
  constexpr int NW = BwdShape::DQ_NW;
  constexpr int RROWS = NW * 64 / CH;
  static_assert(RROWS % 16 == 0, "rounds must cover whole swizzle periods");
  const int drow = (wave * 64 + lane) / CH, dch = (wave * 64 + lane) % CH;
  const int doff = drow * ROWB + ((dch ^ swz_rt<D>(drow)) << 4);
  const i32x4 rsrc_k = make_rsrc(kp, (unsigned)seqlen * ROWB);
  const i32x4 rsrc_v = make_rsrc(vp, (unsigned)seqlen * ROWB);
  const unsigned smem_a = lds_address(smem);
  auto dma_tile = [&](int t, int s) XATTN_INLINE {
    const int kbase = t * BC;
    const unsigned kd = smem_a + s * STAGEB + wave * 1024, vd = kd + TILEB;
    if (kbase + BC <= seqlen) {
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        constexpr int L = I * NW * 1024, G = I * RROWS * ROWB;
        buffer_load_lds16_at<L, G>(rsrc_k, doff, kbase * ROWB, kd);
        buffer_load_lds16_at<L, G>(rsrc_v, doff, kbase * ROWB, vd);
      });
    } else {  // last tile: rows past the end re-read the sequence's last row (masked keys)
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        constexpr int L = I * NW * 1024;
        const int row = drow + I * RROWS;
        const int off = min(row, seqlen - 1 - kbase) * ROWB + ((dch ^ swz_rt<D>(row)) << 4);
        buffer_load_lds16_at<L, 0>(rsrc_k, off, kbase * ROWB, kd);
        buffer_load_lds16_at<L, 0>(rsrc_v, off, kbase * ROWB, vd);
      });
    }
  };

  auto consume = [&](int t, auto s) {  // s: the stage, a compile-time constant
    const int k0 = t * BC;
    if (!wave_active || k0 > kw_hi || k0 + BC - 1 < kw_lo) return;
    const char* kn = smem + s * STAGEB;  // read row-wise (S) and transposed (dQ)
    const char* vn = kn + TILEB;
    f32x16 sacc[BC / 32], dpacc[BC / 32];
    __builtin_amdgcn_s_setprio(1);  // MFMA runs win issue over the partner wave's VALU work
    mma_scores_two<BF16, D, BC>(kn, qf, sacc, vn, dof, dpacc, lo);  // S and dP
    __builtin_amdgcn_s_setprio(0);
    const bool need_mask = (k0 + BC > seqlen) || (wr >= 0 && k0 + BC - 1 > qw0 + wr) ||
                           (wl >= 0 && k0 < qw0 + 31 - wl);
    if (need_mask) mask_scores<BC>(sacc, k0, qrow, seqlen, wl, wr, hh);
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[kb][r], c2, -lse2));
        sacc[kb][r] = p * (dpacc[kb][r] - dps);  // dS^T
      }
    i32x4 dsf[BC / 16];
    pack_operand<BF16, BC>(sacc, dsf);
    __builtin_amdgcn_s_setprio(1);
    mma_pv<BF16, D, BC, 3, true>(kn, lo, dsf, dqacc);
    __builtin_amdgcn_s_setprio(0);
  };

  dma_tile(t_lo, 0);
  wait_vmem();
  block_barrier();
  sweep_two_stages(t_lo, t_hi, [&](int t, auto stage) XATTN_INLINE {
    constexpr int S = decltype(stage)::value;
    if (t < t_hi) dma_tile(t + 1, 1 - S);  // held tile t - 1, free since the last barrier
    consume(t, stage);
    if (t < t_hi) wait_vmem();
    block_barrier();
  });

  // every wave is past the sweep's last barrier and no tile load is in flight: the tile
  // buffers hold each wave's 32 rows of dQ for whole-row stores
  static_assert(BR * ROWB <= 2 * STAGEB, "the dQ rows fit the tile buffers");
  if (wave_active) {
    const int row_w = qrow - l32;  // the wave's first row
    store_block_staged<BF16, D>(ba.dq + (w.row0 + row_w) * D, seqlen - row_w, dqacc, ba.scale,
                                smem + __builtin_amdgcn_readfirstlane(wave) * 32 * ROWB);
  }
}

// ---------------------------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------------------------

struct KeyWork {
  int tile;       // key-tile index within the sequence
  int seqlen;
  long kv_row0;   // row of the sequence's token 0 in the k/v row space
  long q_row0;    // the same in the q row space, for the group's first query head
  long q_stride;  // rows between consecutive query heads
  int bad_lo, bad_hi;  // Decoded::Malformed only: the sequence rows to fill with NaN
};

// Map this workgroup to (key tile, key/value head, batch | sequence).  Key tiles run in
// ascending order: under a causal mask the first ones are seen by the most queries.  Packed
// sequences longer than max_seqlen decode as Malformed (see Decoded).
template <int BK>
__device__ __forceinline__ Decoded decode_key_work(const BwdArgs& ba, KeyWork& w) {
  const FwdArgs& a = ba.f;
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int per = ba.ktiles_per_head;
  const int g = a.kv_group;
  if (a.cu_seqlens == nullptr) {
    const int bh = wid / per;  // (batch, key/value head)
    w.tile = wid - bh * per;
    w.seqlen = a.seqlen;
    w.kv_row0 = (long)bh * a.seqlen;
    w.q_row0 = (long)bh * g * a.seqlen;  // query head (b, kvh * g) = row block b*Hq + kvh*g
    w.q_stride = a.seqlen;
    return Decoded::Run;
  }
  const int h = wid / per;
  const int slot = wid - h * per;
  int c0, len, t, nt;
  const Decoded d = find_seq_tile(a, slot, BK, c0, len, t, nt);
  if (d == Decoded::Skip) return d;
  w.tile = t;
  w.seqlen = len;
  w.kv_row0 = (long)h * a.total_tokens + c0;
  w.q_row0 = (long)h * g * a.total_tokens + c0;
  w.q_stride = a.total_tokens;
  if (d == Decoded::Malformed) malformed_rows(t, nt, BK, len, w.bad_lo, w.bad_hi);
  return d;
}

template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(BwdShape::NT) __attribute__((amdgpu_waves_per_eu(BwdShape::WPE)))
void attn_bwd_dkdv_kernel(BwdArgs ba) {
  const FwdArgs& a = ba.f;
  constexpr int BK = BwdShape::BK, BQ = BwdShape::BQ, NT = BwdShape::NT;
  constexpr int CH = D / 8, ROWB = D * 2, TILEB = BQ * ROWB, LPT = BQ * CH / NT;
  // per stage: Q and dO (the shared swizzle: each is read both ways), then the rows' LSE (log2
  // units) and dPsum; three stages, so that a tile's loads have a step and a half to arrive
  constexpr int STAGEB = 2 * TILEB + 2 * BQ * 4;
  constexpr int NSTAGE = 3;
  // P handed from each dV wave to its dK wave: per lane BQ / 2 fp32 scores as fp16
  constexpr int NPW = BQ / 16;  // 16-byte words per lane
  constexpr int PBUFB = (BwdShape::NW / 2) * NPW * 64 * 16;
  static_assert(BQ * CH % NT == 0 && BQ <= NT, "tile must split evenly over the threads");
  static_assert(BK == 32 * (BwdShape::NW / 2), "each key block has one dV and one dK wave");

  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGEB + PBUFB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  // Waves 0..NW/2-1 ("dV waves") and NW/2..NW-1 ("dK waves") take the same blocks of 32 keys;
  // waves w and w + NW/2 share a SIMD, so each SIMD runs one of each and overlaps the MFMAs of
  // one with the VALU work of the other.  For q-tile t the dV wave forms S, P and
  // dV^T += dO^T P, and hands P (as fp16) to its dK wave through LDS.  The dK wave works one
  // tile behind: dP = dO V^T, dS = P (dP - dPsum) and dK^T += Q^T dS for tile t - 1, whose
  // staged rows stay in LDS until the second barrier of step t.
  const int pair = wave & (BwdShape::NW / 2 - 1);
  const bool dk_wave = wave >= BwdShape::NW / 2;
  i32x4* pbuf = (i32x4*)(smem + NSTAGE * STAGEB) + pair * NPW * 64 + lane;  // word c at [c * 64]

  KeyWork w;
  if (const Decoded dc = decode_key_work<BK>(ba, w); dc != Decoded::Run) {
    if (dc == Decoded::Malformed) {  // dK and dV rows of the sequence: NaN
      fill_nan_rows(ba.dk, w.kv_row0 + w.bad_lo, w.kv_row0 + w.bad_hi, D / 8);
      fill_nan_rows(ba.dv, w.kv_row0 + w.bad_lo, w.kv_row0 + w.bad_hi, D / 8);
    }
    return;
  }
  const int seqlen = w.seqlen;
  int wl, wr;
  mode_windows<MODE>(a, wl, wr);

  const int k0 = w.tile * BK;
  const int kw0 = k0 + pair * 32;
  const int k_last = min(k0 + BK, seqlen) - 1;
  int q_lo = 0, q_hi = seqlen - 1;  // queries that see any key of the workgroup
  if (wr >= 0) q_lo = max(0, k0 - wr);
  if (wl >= 0) q_hi = min(seqlen - 1, k_last + wl);
  const int qt_lo = q_lo / BQ, nq = q_hi / BQ - qt_lo + 1;
  const int n_it = a.kv_group * nq;  // (query head of the group, q-tile) pairs

  const bool wave_active = kw0 < seqlen;
  const int kw_last = min(kw0 + 32, seqlen) - 1;
  int qw_lo = 0, qw_hi = seqlen - 1;  // queries that see any key of this pair of waves
  if (wr >= 0) qw_lo = max(0, kw0 - wr);
  if (wl >= 0) qw_hi = min(seqlen - 1, kw_last + wl);

  const int krow = kw0 + l32;
  // K (dV waves) or V (dK waves) rows of the lane's key
  i32x4 kvf[D / 16];
  load_q<D>((dk_wave ? a.v : a.k) + w.kv_row0 * D, krow, seqlen, hh, kvf);
  const LaneOffsets<D> lo = lane_offsets<D, true>(lane);
  const float c2 = a.scale_log2;

  f32x16 acc[D / 32];  // dV^T (dV waves) or dK^T / scale (dK waves)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  auto tile_base = [&](int it) {
    const int j = it / nq;
    return (qt_lo + it - j * nq) * BQ;
  };
  // Tile it (query head j of the group, rows qbase ..) straight from global memory into LDS
  // stage st: Q and dO with 16-byte loads (instruction i of wave w fills the 16-byte slots
  // (i * NW + w) * 64 + lane: row p / CH, chunk position p % CH, which holds chunk
  // (p % CH) ^ swz_rt(row)), and one 4-byte load each for the rows' LSE (wave 0) and dPsum
  // (wave 1).  Rows past the end of the sequence re-read its last row: their scores are masked.
  constexpr int NW = BwdShape::NW;
  constexpr int RROWS = NW * 64 / CH;  // rows per instruction round, whole swizzle periods
  static_assert(RROWS % 16 == 0 && BQ == 64, "tile split");
  const int drow = (wave * 64 + lane) / CH, dch = (wave * 64 + lane) % CH;
  const int doff = drow * ROWB + ((dch ^ swz_rt<D>(drow)) << 4);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const unsigned smem_a = lds_address(smem);
  auto dma_tile = [&](int it, int st) XATTN_INLINE {
    const int j = it / nq;
    const int qbase = (qt_lo + it - j * nq) * BQ;
    const long hrow = w.q_row0 + j * w.q_stride;  // row of token 0 of query head j
    const i32x4 rsrc_q = make_rsrc(a.q + hrow * D, (unsigned)seqlen * ROWB);
    const i32x4 rsrc_d = make_rsrc(ba.dout + hrow * D, (unsigned)seqlen * ROWB);
    const unsigned qd = smem_a + st * STAGEB + wave * 1024, dd = qd + TILEB;
    if (qbase + BQ <= seqlen) {
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        constexpr int L = I * NW * 1024, G = I * RROWS * ROWB;
        buffer_load_lds16_at<L, G>(rsrc_q, doff, qbase * ROWB, qd);
        buffer_load_lds16_at<L, G>(rsrc_d, doff, qbase * ROWB, dd);
      });
    } else {
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        constexpr int L = I * NW * 1024;
        const int row = drow + I * RROWS;
        const int off = min(row, seqlen - 1 - qbase) * ROWB + ((dch ^ swz_rt<D>(row)) << 4);
        buffer_load_lds16_at<L, 0>(rsrc_q, off, qbase * ROWB, qd);
        buffer_load_lds16_at<L, 0>(rsrc_d, off, qbase * ROWB, dd);
      });
    }
    if (wave_s < 2) {  // wave 0: the rows' LSE (log2 units), wave 1: their dPsum
      const float* src = (wave_s == 0 ? ba.lse2 : ba.dpsum) + hrow;
      const i32x4 rsrc_s = make_rsrc(src, (unsigned)seqlen * 4);
      const int row = min(qbase + lane, seqlen - 1);
      buffer_load_lds4(rsrc_s, row * 4, 0, smem_a + st * STAGEB + 2 * TILEB + wave_s * BQ * 4);
    }
  };
  // wait for the loads of all but the newest tile (when `newer`, the 2 LPT + 1 or 2 LPT load
  // instructions of a later tile may stay outstanding)
  auto wait_older = [&](bool newer) XATTN_INLINE {
    if (!newer)
      wait_vmem();
    else if (wave_s < 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPT + 1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPT) : "memory");
  };
  // whether the pair's keys see any query of the tile at qbase
  auto tile_active = [&](int qbase) {
    return wave_active && qbase <= qw_hi && qbase + BQ - 1 >= qw_lo;
  };

  // dV wave, tile it (stage s): S = Q K^T (lane = key), P, dV^T += dO^T P; P as fp16 into ph.
  // key krow sees query i iff krow - wr <= i <= krow + wl: the forward's test with the window
  // bounds exchanged.
  i32x4 ph[NPW];
  auto consume_dv = [&](int qbase, auto s) {  // s: the stage, an int or a constant
    const char* qn = smem + s * STAGEB;
    const char* dn = qn + TILEB;
    const float* ls = (const float*)(dn + TILEB);
    f32x16 sacc[BQ / 32];
    __builtin_amdgcn_s_setprio(1);  // MFMA runs win issue over the partner wave's VALU work
    mma_scores<BF16, D, BQ>(qn, lo, kvf, sacc);
    __builtin_amdgcn_s_setprio(0);
    const bool need_mask = (qbase + BQ > seqlen) || (wr >= 0 && qbase < kw0 + 31 - wr) ||
                           (wl >= 0 && qbase + BQ - 1 > kw0 + wl);
    if (need_mask) mask_scores<BQ>(sacc, qbase, krow, seqlen, wr, wl, hh);
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // register 4 g4 + i of block qb holds query 32 qb + 8 g4 + 4 hh + i
        const f32x4 l2 = *(const f32x4*)(ls + 32 * qb + 8 * g4 + 4 * hh);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sacc[qb][4 * g4 + i] = fast_exp2(fmaf(sacc[qb][4 * g4 + i], c2, -l2[i]));
      }
    i32x4 pf[BQ / 16];
    pack_operand<BF16, BQ>(sacc, pf);
    if constexpr (BF16)
      pack_operand<false, BQ>(sacc, ph);
    else
#pragma unroll
      for (int c = 0; c < NPW; ++c) ph[c] = pf[c];
    __builtin_amdgcn_s_setprio(1);
    mma_pv<BF16, D, BQ, 3, true>(dn, lo, pf, acc);
    __builtin_amdgcn_s_setprio(0);
  };

  // dK wave, tile it (stage s, P of the tile in pbuf): dP = dO V^T, dS, dK^T += Q^T dS.
  auto consume_dk = [&](auto s) {
    const char* qn = smem + s * STAGEB;
    const char* dn = qn + TILEB;
    const float* ls = (const float*)(dn + TILEB);
    f32x16 dpacc[BQ / 32];
    __builtin_amdgcn_s_setprio(1);
    mma_scores<BF16, D, BQ>(dn, lo, kvf, dpacc);
    __builtin_amdgcn_s_setprio(0);
    i32x4 pw[NPW];
#pragma unroll
    for (int c = 0; c < NPW; ++c) pw[c] = pbuf[c * 64];
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 dd = *(const f32x4*)(ls + BQ + 32 * qb + 8 * g4 + 4 * hh);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g4 + i;
          // element r of block qb sits in word 2 qb + r / 8, 32-bit lane (r % 8) / 2, half r % 2.
          // (The element is copied out first: clang's __builtin_bit_cast of a vector element
          // expression reads the vector's first element.)
          const int wd = pw[2 * qb + (r >> 3)][(r & 7) >> 1];
          const f16x2 h2 = __builtin_bit_cast(f16x2, wd);
          const float p = (float)h2[r & 1];
          dpacc[qb][r] = p * (dpacc[qb][r] - dd[i]);  // dS
        }
      }
    i32x4 dsf[BQ / 16];
    pack_operand<BF16, BQ>(dpacc, dsf);
    __builtin_amdgcn_s_setprio(1);
    mma_pv<BF16, D, BQ, 3, true>(qn, lo, dsf, acc);
    __builtin_amdgcn_s_setprio(0);
  };

  // Tile it lives in stage it % 3.  Step it: the dV waves consume tile it, the dK waves tile
  // it - 1; after the first barrier stage (it + 2) % 3 = (it - 1) % 3 is free and receives tile
  // it + 2; before the second, tile it + 1 (loaded during step it - 1) must have arrived.
  dma_tile(0, 0);
  if (n_it > 1) dma_tile(1, 1);
  wait_older(n_it > 1);
  block_barrier();
  // (unrolled by three, so that the stages, and with them the LDS operand addresses, are
  // compile-time constants)
  auto step = [&](int it, auto stage) XATTN_INLINE {
    constexpr int S = decltype(stage)::value;  // it % 3
    using SP = std::integral_constant<int, (S + 2) % 3>;  // (it - 1) % 3
    const bool act = tile_active(tile_base(it));
    if (!dk_wave) {
      if (act) consume_dv(tile_base(it), stage);
    } else if (it >= 1 && tile_active(tile_base(it - 1))) {
      consume_dk(SP{});
    }
    block_barrier();  // the dK waves are done with stage SP and with the P of tile it - 1
    if (it + 2 < n_it) dma_tile(it + 2, SP::value);
    if (!dk_wave && act)
#pragma unroll
      for (int c = 0; c < NPW; ++c) pbuf[c * 64] = ph[c];
    if (it + 1 < n_it) wait_older(it + 2 < n_it);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the P words are in LDS
    block_barrier();
  };
  for (int it = 0; it < n_it; it += 3) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < n_it) step(it + 1, std::integral_constant<int, 1>{});
    if (it + 2 < n_it) step(it + 2, std::integral_constant<int, 2>{});
  }
  if (dk_wave && tile_active(tile_base(n_it - 1))) consume_dk((n_it - 1) % 3);

  // Past the sweep's last barrier no load is in flight and only the dK waves' last step reads
  // an LDS stage, (n_it - 1) % 3: the other two stages hold each wave's 32 rows of dK or dV
  // (dV waves in one, dK waves in the other) for whole-row stores, with no further barrier.
  static_assert((BwdShape::NW / 2) * 32 * ROWB <= STAGEB, "half the waves' rows fit a stage");
  if (wave_active) {
    const int row_w = krow - l32;  // the wave's first key row
    const int stage = (n_it + (dk_wave ? 1 : 0)) % NSTAGE;
    char* const region = smem + stage * STAGEB + __builtin_amdgcn_readfirstlane(pair) * 32 * ROWB;
    if (dk_wave)
      store_block_staged<BF16, D>(ba.dk + (w.kv_row0 + row_w) * D, seqlen - row_w, acc,
                                  ba.scale, region);
    else
      store_block_staged<BF16, D>(ba.dv + (w.kv_row0 + row_w) * D, seqlen - row_w, acc, 1.0f,
                                  region);
  }
}

// Host launchers for one head dim (explicitly specialised per head dim in its own translation
// unit): the dQ kernel over n_q workgroups, then the dK/dV kernel over n_k, on one stream.
template <int D>
hipError_t launch_bwd(const BwdArgs& a, bool bf16, int mode, int n_q, int n_k,
                      hipStream_t stream);

template <bool BF16, int D, int MODE>
hipError_t launch_bwd_mode(const BwdArgs& a, int n_q, int n_k, hipStream_t s) {
  const hipError_t e = launch_kernel(attn_bwd_dq_kernel<BF16, D, MODE>, n_q, BwdShape::DQ_NT, s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(attn_bwd_dkdv_kernel<BF16, D, MODE>, n_k, BwdShape::NT, s, a);
}

#define XATTN_DEFINE_BWD_LAUNCHER(D)                                                         \
  template <>                                                                                \
  hipError_t launch_bwd<D>(const BwdArgs& a, bool bf16, int mode, int n_q, int n_k,          \
                           hipStream_t s) {                                                  \
    if (bf16) {                                                                              \
      if (mode == MASK_NONE) return launch_bwd_mode<true, D, MASK_NONE>(a, n_q, n_k, s);     \
      if (mode == MASK_CAUSAL) return launch_bwd_mode<true, D, MASK_CAUSAL>(a, n_q, n_k, s); \
      return launch_bwd_mode<true, D, MASK_WINDOW>(a, n_q, n_k, s);                          \
    }                                                                                        \
    if (mode == MASK_NONE) return launch_bwd_mode<false, D, MASK_NONE>(a, n_q, n_k, s);      \
    if (mode == MASK_CAUSAL) return launch_bwd_mode<false, D, MASK_CAUSAL>(a, n_q, n_k, s);  \
    return launch_bwd_mode<false, D, MASK_WINDOW>(a, n_q, n_k, s);                           \
  }

}  // namespace xattn
