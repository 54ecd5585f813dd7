// FP8 (E4M3) exact-attention forward for gfx950, head_dim 64/128/256: Q, K, V are 8-bit floats with
// one fp32 descale per tensor; O is written in bf16 or fp16 with the natural-log LSE.
//
// What is computed: plain attention of the dequantized tensors (code * descale).  As on the
// pages, the Q and K descales fold into the softmax scale and the V descale is applied to the
// output (page "flash_fwd_kernel.h" @c272619, `compute_attn_ws_fp8`; page "flash_fwd_kernel.h"
// @26a6e0a: a missing scale pointer means 1), and P is exponentiated with an offset of 8 in the
// exponent (`Max_offset`), so that its largest values use the upper part of the E4M3 range
// (P in (0, 256]) before it is rounded to E4M3 for the P V product.
//
// MFMA: v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3), 32 bytes of A and of B per lane.  The
// products pair A and B bytes by the same (lane half, byte) -> k rule, so loading both
// operands of S^T = K Q^T as 32 contiguous bytes of a row needs no knowledge of that rule.
// For O^T += V^T P^T the two operands are built differently (P from registers, V^T with
// ds_read_b64_tr_b8), so both are laid out by one explicit key order: byte b of lane half hh
// is key 32 (b / 16) + 16 hh + b % 16 of the 64-key tile.
//  * So that the S^T accumulators come out in that order, K rows sit in LDS in a permuted slot
//    order: slot i of a 32-key block holds key perm(i) = 16 ((i >> 2) & 1) + 4 (i >> 3) + i % 4.
//    Lane l reads slot l % 32 as its A row, and accumulator register r of lane half hh then
//    holds key 32 kb + 16 hh + r.
//  * ds_read_b64_tr_b8 (measured on gfx950): a group of 16 lanes reads an 8-row x 16-byte block
//    (lane i gives row i / 2, bytes 8 (i % 2) .. + 7) and lane i receives column i of the block,
//    rows 0..7 as bytes 0..7.  Four such reads give a lane the 32 keys of its P bytes for one
//    column d of V.
// K and V tiles are stored with D-byte rows and the 16-byte chunk index XORed with a function
// of the row, so that neither the K row reads (16 lanes, 16 consecutive slots, one chunk) nor
// the V transpose reads (32 lanes: two 16-lane groups reading adjacent chunks of the same 8
// rows) hit a bank twice.  With 64 four-byte banks, D = 64 / 128 / 256 puts 4 / 2 / 1 rows in
// one 256-byte bank line, so the keys are:
//     K:  (slot / 4) % 4,       (slot / 2) % 8,       slot % 16
//     V:  2 ((row / 4) % 2),    2 ((row / 2) % 4),    2 (row % 8)
// (rows r and r + 8 share the V key in all three cases).
// The tiles go straight from global memory into LDS (buffer_load ... lds), double-buffered:
// each lane fetches the row and chunk that its LDS slot holds under the permutation and
// swizzle, and the next tile's loads are in flight while the current one is consumed.
#pragma once

#include "attn_common.h"

namespace xattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Fp8Args {
  FwdArgs f;                 // q, k, v hold E4M3 codes; o is bf16 / fp16
  const float* descale_q;    // null = 1
  const float* descale_k;
  const float* descale_v;
};

// Tile shape per head dim: NW waves of 32 query rows share each K/V tile of BC keys; at least
// two waves per SIMD.  At d = 256 the registers only allow two waves per SIMD with eight waves
// in a workgroup, which measured 1.5x faster than four waves at one per SIMD.  With the tiles
// loaded straight into LDS (no staging registers) the kernels use 114-121 VGPRs at d = 64,
// 159-166 at d = 128 (three waves per SIMD) and 248-255 at d = 256, without spills.
template <int D> struct Fp8Shape {
  static constexpr int NW = D == 256 ? 8 : 4, NT = 64 * NW, BR = 32 * NW, BC = 64, WPE = 2;
};
constexpr int fp8_block_rows(int head_dim) { return head_dim == 256 ? 256 : 128; }

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 (E4M3) for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four fp32 values -> four E4M3 bytes (round to nearest even) in one dword.
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D> __device__ __forceinline__ int swz8k(int slot) {
  return D == 64 ? (slot >> 2) & 3 : D == 128 ? (slot >> 1) & 7 : slot & 15;
}
template <int D> __device__ __forceinline__ int swz8v(int row) {
  return D == 64 ? ((row >> 2) & 1) << 1 : D == 128 ? ((row >> 1) & 3) << 1 : (row & 7) << 1;
}

// LDS slot of key kk (0..31) of a 32-key block: the inverse of perm above.
__device__ __forceinline__ int key_slot(int kk) {
  return 8 * ((kk >> 2) & 3) + 4 * (kk >> 4) + (kk & 3);
}
// Key held by LDS slot s (0..31) of a 32-key block (the inverse of key_slot).
__device__ __forceinline__ int slot_key(int s) {
  return 16 * ((s >> 2) & 1) + 4 * (s >> 3) + (s & 3);
}

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(Fp8Shape<D>::NT)
__attribute__((amdgpu_waves_per_eu(Fp8Shape<D>::WPE)))
void attn_fwd_fp8_kernel(Fp8Args fa) {
  static_assert(D == 64 || D == 128 || D == 256, "FP8 head dims");
  static_assert(fp8_block_rows(D) == Fp8Shape<D>::BR, "host and kernel tile rows");
  const FwdArgs& a = fa.f;
  constexpr int BC = Fp8Shape<D>::BC, NT = Fp8Shape<D>::NT, BR = Fp8Shape<D>::BR;
  constexpr int CH = D / 16;            // 16-byte chunks per row
  constexpr int TILEB = BC * D;         // bytes per K (or V) tile
  constexpr int LPT = BC * CH / NT;     // chunks per thread per matrix per tile
  static_assert(BC * CH % NT == 0 && BC == 64, "tile shape");

  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  Work w;
  if (const Decoded dc = decode_work<BR, MODE>(a, w); dc != Decoded::Run) {
    if (dc == Decoded::Malformed) fill_malformed_fwd<D>(a, w);
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

  const uint8_t* __restrict__ kp = (const uint8_t*)a.k + w.kv_row0 * D;
  const uint8_t* __restrict__ vp = (const uint8_t*)a.v + w.kv_row0 * D;
  const int qrow = qw0 + l32;

  // Q^T operand: lane's query row, bytes 64 c + 32 hh .. + 31 of d-chunk c
  i32x8 qf[D / 64];
  {
    const uint8_t* src = (const uint8_t*)a.q + (w.row0 + qrow) * D;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      i32x4 lo4 = {0, 0, 0, 0}, hi4 = {0, 0, 0, 0};
      if (qrow < seqlen) {
        lo4 = *(const i32x4*)(src + 64 * c + 32 * hh);
        hi4 = *(const i32x4*)(src + 64 * c + 32 * hh + 16);
      }
      qf[c] = (i32x8){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    }
  }
  const float dsq = fa.descale_q ? *fa.descale_q : 1.f;
  const float dsk = fa.descale_k ? *fa.descale_k : 1.f;
  const float dsv = fa.descale_v ? *fa.descale_v : 1.f;
  const float c2 = a.scale_log2 * dsq * dsk;
  constexpr float OFFSET = 8.0f;  // P = 2^(s - m + 8) in (0, 2^(8 + SLACK)]
  // The reference max m moves only when a row's tile max exceeds it by more than SLACK (log2
  // units), which spares most O rescales; P then stays at most 2^8.8 = 445.7, inside E4M3's
  // largest finite value (448 = 2^8.807).
  constexpr float SLACK = 0.8f;
  static_assert(OFFSET + SLACK < 8.807f, "P must stay below E4M3's largest finite value");

  // per-lane LDS byte offsets: K row reads (slot l32, chunks 4c + 2hh and + 1, swizzled) and
  // V transpose reads (row 16 hh + i16 / 2, bytes 32 db + 16 (g & 1) + 8 (i16 & 1))
  int kofs[D / 64][2];
#pragma unroll
  for (int c = 0; c < D / 64; ++c)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      kofs[c][h2] = l32 * D + (((4 * c + 2 * hh + h2) ^ swz8k<D>(l32)) << 4);
  // (the V key of a row repeats every 8 rows, so the reads of rows + 8, + 32, + 40 are the
  // first one's address plus a constant)
  const int g = lane >> 4, i16 = lane & 15;
  const int vrow = 16 * hh + (i16 >> 1);
  int vofs[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int col = 32 * db + 16 * (g & 1) + 8 * (i16 & 1);
    vofs[db] = vrow * D + (((col >> 4) ^ swz8v<D>(vrow)) << 4) + (col & 15);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // K/V tiles go straight from global memory into LDS (buffer_load ... lds).  Instruction i of
  // wave w fills the 16-byte LDS slots (i * NW + w) * 64 + lane: slot p sits at tile row
  // p / CH, chunk position p % CH, so the lane fetches the global row and chunk that position
  // holds (K: the key of that slot and the swizzled chunk; V: the swizzled chunk).  One
  // instruction round covers RROWS rows, a whole number of key-permutation (32) and swizzle
  // periods, so instruction i reads instruction 0's bytes shifted by i rounds.
  constexpr int NW = Fp8Shape<D>::NW;
  constexpr int RROWS = NW * 64 / CH;
  static_assert(RROWS % 32 == 0, "rounds must cover whole permutation and swizzle periods");
  const int dpos = (wave * 64 + lane) / CH, dcp = (wave * 64 + lane) % CH;
  const int dkrow = (dpos & ~31) + slot_key(dpos & 31);
  const int dkch = dcp ^ swz8k<D>(dpos), dvch = dcp ^ swz8v<D>(dpos);
  const i32x4 rsrc_k = make_rsrc(kp, (unsigned)seqlen * D);
  const i32x4 rsrc_v = make_rsrc(vp, (unsigned)seqlen * D);
  const unsigned smem_a = lds_address(smem);
  auto dma_tile = [&](int t, int s) XATTN_INLINE {
    const int kbase = t * BC;
    const unsigned kdst = smem_a + s * 2 * TILEB + wave * 1024, vdst = kdst + TILEB;
    if (kbase + BC <= seqlen) {
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        buffer_load_lds16_at<I * NW * 1024, I * RROWS * D>(rsrc_k, dkrow * D + (dkch << 4),
                                                           kbase * D, kdst);
        buffer_load_lds16_at<I * NW * 1024, I * RROWS * D>(rsrc_v, dpos * D + (dvch << 4),
                                                           kbase * D, vdst);
      });
    } else {  // last tile: rows past the end re-read the sequence's last row (finite data)
      static_for<LPT>([&](auto ic) XATTN_INLINE {
        constexpr int I = decltype(ic)::value;
        const int kr = min(dkrow + I * RROWS, seqlen - 1 - kbase);
        const int vr = min(dpos + I * RROWS, seqlen - 1 - kbase);
        buffer_load_lds16_at<I * NW * 1024, 0>(rsrc_k, kr * D + (dkch << 4), kbase * D, kdst);
        buffer_load_lds16_at<I * NW * 1024, 0>(rsrc_v, vr * D + (dvch << 4), kbase * D, vdst);
      });
    }
  };

  auto consume = [&](int t, auto s) {  // s: the stage, a compile-time constant
    const int k0 = t * BC;
    if (!wave_active || k0 > kw_hi || k0 + BC - 1 < kw_lo) return;
    const char* kt = smem + s * 2 * TILEB;
    const char* vt = kt + TILEB;
    // S^T = K Q^T: register r of block kb, lane half hh holds key k0 + 32 kb + 16 hh + r
    f32x16 sacc[BC / 32];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        const char* base = kt + kb * 32 * D;
        const i32x4 x0 = *(const i32x4*)(base + kofs[c][0]);
        const i32x4 x1 = *(const i32x4*)(base + kofs[c][1]);
        const i32x8 av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        sacc[kb] = mfma_fp8(av, qf[c], sacc[kb]);
      }
    }
    // mask: key offset 32 kb + 16 hh + r against the row's visible range
    const bool need_mask = (k0 + BC > seqlen) || (wr >= 0 && k0 + BC - 1 > qw0 + wr) ||
                           (wl >= 0 && k0 < qw0 + 31 - wl);
    if (need_mask) {
      const int base = k0 + 16 * hh;
      int lo = wl >= 0 ? qrow - wl - base : -(1 << 30);
      int hi = seqlen - 1 - base;
      if (wr >= 0) hi = min(hi, qrow + wr - base);
      if (lo > hi) lo = hi = -(1 << 30);
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + r;
          if (min(max(c, lo), hi) != c) sacc[kb][r] = -INFINITY;
        }
    }
    // softmax with a lazily moved reference max and the exponent offset; the row max runs in
    // four independent chains
    float pm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pm[r % 4] = fmaxf(pm[r % 4], sacc[kb][r]);
    const float mx = halves_max(fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]))) * c2;
    const bool moved = mx > m_run + SLACK;  // false while both are -inf
    const float m_new = moved ? mx : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new - OFFSET;
    const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(sacc[kb][r], c2, -m_use));
        sacc[kb][r] = e;
        ps += e;
      }
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {  // wave-uniform
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      l_run *= alpha;
    }
    l_run += ps;
    m_run = m_new;
    // P^T operand: bytes 16 kb + r <- register r of block kb (key 32 kb + 16 hh + r)
    i32x8 pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kb = j >> 2, r0 = 4 * (j & 3);
      pf[j] = pack4_fp8(sacc[kb][r0], sacc[kb][r0 + 1], sacc[kb][r0 + 2], sacc[kb][r0 + 3]);
    }
    // O^T += V^T P^T: column d = 32 db + l32, keys in the same byte order via four
    // transpose reads (rows 16 hh + 0..7, + 8..15, + 32..39, + 40..47)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const i32x2 r0 = lds_read_tr8(vt + vofs[db]);
      const i32x2 r1 = lds_read_tr8(vt + vofs[db] + 8 * D);
      const i32x2 r2 = lds_read_tr8(vt + vofs[db] + 32 * D);
      const i32x2 r3 = lds_read_tr8(vt + vofs[db] + 40 * D);
      const i32x8 av = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
      oacc[db] = mfma_fp8(av, pf, oacc[db]);
    }
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

  if (!wave_active) return;
  // epilogue: O = O * descale_v / l, LSE = (m - 8 + log2 l) ln 2
  constexpr float LN2 = 0.693147180559945309f;
  const float lt = halves_sum(l_run);
  const float inv = lt > 0.f ? dsv / lt : 0.f;
  if constexpr ((BR / 32) * 32 * D * 2 <= (int)sizeof(smem)) {
    // every wave is past the sweep's last barrier and no tile load is in flight: the tile
    // buffers hold each wave's 32 rows of 16-bit output for whole-row stores
    const int row_w = qrow - (__lane_id() & 31);  // the wave's first row
    store_block_staged<BF16, D>(a.o + (w.row0 + row_w) * D, seqlen - row_w, oacc, inv,
                                smem + __builtin_amdgcn_readfirstlane(wave) * 32 * D * 2);
  } else if (qrow < seqlen) {
    uint16_t* dst = a.o + (w.row0 + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16& x = oacc[db];
        const i32x2 val = {(int)Elt<BF16>::pack2(x[4 * g4 + 0] * inv, x[4 * g4 + 1] * inv),
                           (int)Elt<BF16>::pack2(x[4 * g4 + 2] * inv, x[4 * g4 + 3] * inv)};
        *(i32x2*)(dst + db * 32 + 8 * g4 + 4 * hh) = val;
      }
  }
  if (a.lse != nullptr && hh == 0 && qrow < seqlen)
    a.lse[w.row0 + qrow] = lt > 0.f ? (m_run - OFFSET + fast_log2(lt)) * LN2 : -INFINITY;
}

// Host launcher (defined in attn_fwd_fp8.hip): out_bf16 selects the output type.
hipError_t launch_fwd_fp8(const Fp8Args& a, int head_dim, bool out_bf16, int mode, int n_work,
                          hipStream_t stream);

}  // namespace xattn
