// Exact attention forward (FlashAttention-2 style) for gfx950 / MI355X.
//
// What is computed.  For every query row i of a (batch, head) or (sequence, head):
//   S_ij = scale * q_i . k_j   (keys j visible under the causal / sliding-window mask),
//   O_i  = sum_j softmax_j(S_ij) v_j,  LSE_i = log sum_j exp(S_ij)  (natural log),
// by the streaming recurrence of page "flash_attn_mma_tiling_qk.cu" (its KV loop and the
// "Rescale O" block): per K/V tile keep a running row max m and row sum l,
//   m_new = max(m, rowmax(S_tile)),  P = exp(S_tile - m_new),  alpha = exp(m - m_new),
//   l = alpha * l + rowsum(P),  O = alpha * O + P V_tile,
// and divide O by l at the end.  Masks follow page "mainloop_bwd_sm90_tma_gmma_ws.hpp"
// (`mma`: causal masking iterations and the Is_local branch) with seqlen_q == seqlen_k:
// key j is visible to query i iff j <= i + window_right (causal: window_right = 0) and
// j >= i - window_left (a bound of -1 is unbounded).  A row with no visible key stores
// O = 0, LSE = -inf (page "flash_fwd_kernel.h" @26a6e0a, consumer loop, store_zero).
//
// How it maps to CDNA4.
//   * One workgroup = NW wave64s and BR = NW * QB * 32 query rows of one (batch|sequence,
//     head).  Each wave owns QB blocks of 32 query rows for the whole K/V sweep.
//   * Both contractions run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulators.
//     The score tile is computed transposed, S^T = K Q^T (the swap-AB idea of page
//     "mainloop_bwd_sm90_tma_gmma_ws.hpp", SdP_swapAB), so the accumulator of lane l holds
//     query (l % 32) against 16 keys: the row max / row sum are in-lane plus one exchange
//     between the two 32-lane halves (v_permlane32_swap).
//   * The output is accumulated transposed too, O^T += V^T P^T.  The S^T accumulator
//     registers, converted to 16-bit, are exactly the B operand (P^T) of that MFMA, so P
//     never leaves registers; the matching V^T A operand is read from row-major V in LDS
//     with ds_read_b64_tr_b16.  Each lane ends up holding its own query's O row, so the
//     rescale by alpha and the final 1/l are in-lane.
//   * Q stays in VGPRs for the whole sweep.  K and V tiles (BC keys) go global -> LDS with
//     16-byte loads, double-buffered (the next tile's loads are in flight while the current
//     tile is consumed; one barrier per tile).  The LDS layout XORs the 16-byte chunk index
//     with a function of the row so that both the K operand reads (32 rows, one chunk) and
//     the V transpose reads (8 rows, 64 bytes each) are bank-conflict free.
//   * Only tiles that cross a mask edge or the end of the sequence evaluate the mask; a
//     wave skips tiles its rows cannot see (causal diagonal, window edge).
//   * Workgroup ids are remapped so that each XCD (8 on MI355X, dispatched round-robin)
//     runs a contiguous range of work, i.e. the q-tiles of the same heads share that XCD's
//     L2; causal and windowed work is ordered heaviest q-tile first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum MaskMode { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_WINDOW = 2 };

// Kernel arguments (plain data; pointers are device addresses).
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                 // may be null
  const int32_t* cu_seqlens;  // null for a dense batch
  int seqlen;                 // dense: N
  int num_seqs;               // packed: number of sequences
  int total_tokens;           // packed: rows per head
  int tiles_per_head;         // dense: ceil(N / BR); packed: q-tile slots per head
  float scale_log2;           // softmax_scale * log2(e): scores are exponentiated base 2
  int window_left;            // -1 = unbounded (MASK_WINDOW only)
  int window_right;           // -1 = unbounded (MASK_WINDOW only; causal folded in as 0)
};

// Tile shape per head dim: QB 32-row query blocks per wave, NW waves, BC keys per K/V tile,
// STAGES LDS buffers.  Registers: O^T takes QB*D/2 fp32 per lane, Q takes QB*D/4.
template <int D> struct TileCfg;
template <> struct TileCfg<64>  { static constexpr int QB = 2, NW = 4, BC = 64, STAGES = 2; };
template <> struct TileCfg<128> { static constexpr int QB = 2, NW = 4, BC = 64, STAGES = 2; };
template <> struct TileCfg<256> { static constexpr int QB = 1, NW = 4, BC = 32, STAGES = 2; };
template <> struct TileCfg<512> { static constexpr int QB = 1, NW = 4, BC = 32, STAGES = 1; };

template <int D> constexpr int block_rows() { return TileCfg<D>::NW * TileCfg<D>::QB * 32; }

// ---------------------------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------------------------

template <bool BF16> struct Elt;
template <> struct Elt<true> {
  static __device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> packed pair, round to nearest even.
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    bf16x2 r = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
};
template <> struct Elt<false> {
  static __device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f16x2 r = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
};

// Reduce a value across the two 32-lane halves of the wave; both halves get the result.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Workgroup i is dispatched to XCD i % 8.  Renumber so that XCD x runs the contiguous work
// range [x * n / 8, (x + 1) * n / 8) (a bijection for any n).
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  constexpr int NX = 8;
  const int xcd = bid % NX, local = bid / NX;
  const int per = nwg / NX, rem = nwg % NX;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// LDS swizzles: XOR masks on the 16-byte chunk index of a row.
//  K is read as the MFMA A operand: 32 consecutive rows, same chunk -> spread rows over all
//  16 chunk positions of a 256-byte bank window.
//  V is read by ds_read_b64_tr_b16: 8 consecutive rows x 64 bytes -> move each group of 4
//  rows to a different 64-byte quarter of the bank window.
template <int D> __device__ __forceinline__ int swz_k(int r) {
  return D >= 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ int swz_v(int r) {
  return D >= 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// ---------------------------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------------------------

template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(TileCfg<D>::NW * 64)
void attn_fwd_kernel(FwdArgs a) {
  using C = TileCfg<D>;
  constexpr int QB = C::QB, NW = C::NW, BC = C::BC, STAGES = C::STAGES;
  constexpr int NT = NW * 64;          // threads per workgroup
  constexpr int BR = NW * QB * 32;     // query rows per workgroup
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int DC = D / 16;           // K steps of the S^T MFMA
  constexpr int DB = D / 32;           // 32-wide column blocks of O^T
  constexpr int KB = BC / 32;          // 32-key blocks per tile
  constexpr int KC = BC / 16;          // 16-key K steps of the O^T MFMA
  constexpr int ROWB = D * 2;          // bytes per row
  constexpr int TILEB = BC * ROWB;     // bytes per K (or V) tile
  constexpr int LPT = BC * CH / NT;    // 16-byte chunks per thread per matrix per tile
  static_assert(BC * CH % NT == 0, "tile must split evenly over the threads");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  using E = Elt<BF16>;

  __shared__ __attribute__((aligned(16))) char smem[STAGES * 2 * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- which (rows, head, sequence) this workgroup owns --------------------------------
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  int tile, seqlen;
  long row0;  // index of this sequence's token 0 in the [*, D] row space of q/k/v/o and lse
  if (a.cu_seqlens == nullptr) {
    const int per = a.tiles_per_head;
    const int bh = wid / per, t = wid - bh * per;
    tile = (MODE != MASK_NONE) ? per - 1 - t : t;
    seqlen = a.seqlen;
    row0 = (long)bh * seqlen;
  } else {
    const int per = a.tiles_per_head;
    const int h = wid / per;
    const int slot = wid - h * per;
    int found = -1, acc = 0, start = 0, len = 0, t = 0;
    int c_prev = min(max(a.cu_seqlens[0], 0), a.total_tokens);
    for (int s = 0; s < a.num_seqs; ++s) {
      const int c_next = min(max(a.cu_seqlens[s + 1], c_prev), a.total_tokens);
      const int nt = (c_next - c_prev + BR - 1) / BR;
      if (slot < acc + nt) {
        found = s; start = c_prev; len = c_next - c_prev; t = slot - acc;
        if (MODE != MASK_NONE) t = nt - 1 - t;
        break;
      }
      acc += nt;
      c_prev = c_next;
    }
    if (found < 0) return;  // unused slot (the grid is an upper bound)
    tile = t;
    seqlen = len;
    row0 = (long)h * a.total_tokens + start;
  }

  int wl = a.window_left, wr = a.window_right;
  if (MODE == MASK_NONE) { wl = -1; wr = -1; }
  if (MODE == MASK_CAUSAL) { wl = -1; wr = 0; }

  const int q0 = tile * BR;
  const int qw0 = q0 + wave * QB * 32;                 // first row of this wave
  const int q_last = min(q0 + BR, seqlen) - 1;         // last valid row of the workgroup
  int k_lo = 0, k_hi = seqlen - 1;                     // keys any valid row can see
  if (wl >= 0) k_lo = max(0, q0 - wl);
  if (wr >= 0) k_hi = min(seqlen - 1, q_last + wr);
  const int t_lo = k_lo / BC, t_hi = k_hi / BC;

  const bool wave_active = qw0 < seqlen;
  const int qw_last = min(qw0 + QB * 32, seqlen) - 1;
  int kw_lo = 0, kw_hi = seqlen - 1;                   // keys this wave's rows can see
  if (wl >= 0) kw_lo = max(0, qw0 - wl);
  if (wr >= 0) kw_hi = min(seqlen - 1, qw_last + wr);

  const uint16_t* __restrict__ qp = a.q + row0 * D;
  const uint16_t* __restrict__ kp = a.k + row0 * D;
  const uint16_t* __restrict__ vp = a.v + row0 * D;

  // ---- Q^T operand fragments: lane holds query (qw0 + 32 qb + l32), d = 16c + 8hh .. +7 ----
  i32x4 qf[QB][DC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
    const i32x4* src = (const i32x4*)(qp + (long)row * D);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      qf[qb][c] = (row < seqlen) ? src[2 * c + hh] : (i32x4){0, 0, 0, 0};
    }
  }

  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; }

  // ---- global -> registers -> LDS staging of one K/V tile -------------------------------
  i32x4 stage_k[LPT], stage_v[LPT];
  auto gload = [&](int t) {
    const int kbase = t * BC;
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
    char* kb_ = smem + s * 2 * TILEB;
    char* vb_ = kb_ + TILEB;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int id = tid + u * NT;
      const int r = id / CH, c = id % CH;
      *(i32x4*)(kb_ + r * ROWB + ((c ^ swz_k<D>(r)) << 4)) = stage_k[u];
      *(i32x4*)(vb_ + r * ROWB + ((c ^ swz_v<D>(r)) << 4)) = stage_v[u];
    }
  };

  const float c2 = a.scale_log2;

  // ---- one K/V tile: S^T, mask, online softmax, O^T update --------------------------------
  auto consume = [&](int t, int s) {
    const int k0 = t * BC;
    if (!wave_active || k0 > kw_hi || k0 + BC - 1 < kw_lo) return;  // nothing visible
    const char* kb_ = smem + s * 2 * TILEB;
    const char* vb_ = kb_ + TILEB;

    f32x16 sacc[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.f;

    // S^T[key, query] = sum_d K[key, d] Q[query, d]
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = kb * 32 + l32;
        const int ch = 2 * c + hh;
        const i32x4 kf = *(const i32x4*)(kb_ + row * ROWB + ((ch ^ swz_k<D>(row)) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = E::mfma(kf, qf[qb][c], sacc[kb][qb]);
      }
    }

    // mask: only tiles that reach past the sequence end or cross a mask edge
    const bool need_mask = (k0 + BC > seqlen) ||
                           (wr >= 0 && k0 + BC - 1 > qw0 + wr) ||
                           (wl >= 0 && k0 < qw0 + QB * 32 - 1 - wl);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qrow = qw0 + qb * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = key < seqlen && (wr < 0 || key <= qrow + wr) &&
                             (wl < 0 || key >= qrow - wl);
            if (!vis) sacc[kb][qb][r] = -INFINITY;
          }
        }
    }

    // online softmax (base 2), P packed to 16-bit as the B operand of O^T += V^T P^T
    i32x4 pf[KC][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run[qb], mx * c2);
      // a row with nothing visible so far keeps m = -inf; subtract 0 so exp2 gives 0, not NaN
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[qb] - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(sacc[kb][qb][r], c2, -m_use));
          sacc[kb][qb][r] = e;
          rs += e;
        }
      l_run[qb] = fmaf(l_run[qb], alpha, rs);  // per-lane partial; halves summed at the end
      m_run[qb] = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int kb = kc >> 1, o8 = (kc & 1) * 8;
        pf[kc][qb] = (i32x4){(int)E::pack2(sacc[kb][qb][o8 + 0], sacc[kb][qb][o8 + 1]),
                             (int)E::pack2(sacc[kb][qb][o8 + 2], sacc[kb][qb][o8 + 3]),
                             (int)E::pack2(sacc[kb][qb][o8 + 4], sacc[kb][qb][o8 + 5]),
                             (int)E::pack2(sacc[kb][qb][o8 + 6], sacc[kb][qb][o8 + 7])};
      }
    }

    // O^T[d, query] += sum_key V[key, d] P[query, key].  The A operand (V^T) for lane l is
    // column d = 32 db + l % 32, keys 16 kc + 4 hh + {0..3} and 16 kc + 8 + 4 hh + {0..3}:
    // the same key slots the S^T accumulator gave P.  Two transpose reads fetch them.
    const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 16 * kc + 4 * (g >> 1) + (i16 >> 2);
        const int col = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
        const int off0 = row * ROWB + (((col >> 3) ^ swz_v<D>(row)) << 4) + ((col & 7) << 1);
        const int off1 = (row + 8) * ROWB + (((col >> 3) ^ swz_v<D>(row + 8)) << 4) +
                         ((col & 7) << 1);
        const i16x4 lo = lds_read_tr(vb_ + off0);
        const i16x4 hi = lds_read_tr(vb_ + off1);
        const i32x2 lo2 = __builtin_bit_cast(i32x2, lo), hi2 = __builtin_bit_cast(i32x2, hi);
        const i32x4 vf = (i32x4){lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma(vf, pf[kc][qb], oacc[qb][db]);
      }
    }
  };

  // ---- the sweep over K/V tiles ---------------------------------------------------------
  if constexpr (STAGES == 2) {
    gload(t_lo);
    lstore(0);
    __syncthreads();
    for (int t = t_lo; t <= t_hi; ++t) {
      const int s = (t - t_lo) & 1;
      if (t < t_hi) gload(t + 1);
      consume(t, s);
      if (t < t_hi) lstore(s ^ 1);
      __syncthreads();
    }
  } else {
    for (int t = t_lo; t <= t_hi; ++t) {
      if (t > t_lo) __syncthreads();
      gload(t);
      lstore(0);
      __syncthreads();
      consume(t, 0);
    }
  }

  // ---- epilogue: O = O / l, LSE = (m + log2 l) ln 2 -------------------------------------
  constexpr float LN2 = 0.693147180559945309f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const int qrow = qw0 + qb * 32 + l32;
    if (!wave_active || qrow >= seqlen) continue;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    uint16_t* dst = a.o + (row0 + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16& x = oacc[qb][db];
        const i32x2 val = {(int)E::pack2(x[4 * g4 + 0] * inv, x[4 * g4 + 1] * inv),
                           (int)E::pack2(x[4 * g4 + 2] * inv, x[4 * g4 + 3] * inv)};
        *(i32x2*)(dst + db * 32 + 8 * g4 + 4 * hh) = val;
      }
    if (a.lse != nullptr && hh == 0)
      a.lse[row0 + qrow] = lt > 0.f ? (m_run[qb] + fast_log2(lt)) * LN2 : -INFINITY;
  }
}

// Host launcher for one head dim (explicitly instantiated per head dim).
template <int D>
hipError_t launch_fwd(const FwdArgs& a, bool bf16, int mode, int n_work, hipStream_t stream);

#define XATTN_LAUNCH_CASE(BF, D, MODE)                                                      \
  hipLaunchKernelGGL((attn_fwd_kernel<BF, D, MODE>), dim3(n_work),                          \
                     dim3(TileCfg<D>::NW * 64), 0, stream, a)

#define XATTN_DEFINE_LAUNCHER(D)                                                            \
  template <>                                                                               \
  hipError_t launch_fwd<D>(const FwdArgs& a, bool bf16, int mode, int n_work,               \
                           hipStream_t stream) {                                            \
    if (bf16) {                                                                             \
      if (mode == MASK_NONE) XATTN_LAUNCH_CASE(true, D, MASK_NONE);                         \
      else if (mode == MASK_CAUSAL) XATTN_LAUNCH_CASE(true, D, MASK_CAUSAL);                \
      else XATTN_LAUNCH_CASE(true, D, MASK_WINDOW);                                         \
    } else {                                                                                \
      if (mode == MASK_NONE) XATTN_LAUNCH_CASE(false, D, MASK_NONE);                        \
      else if (mode == MASK_CAUSAL) XATTN_LAUNCH_CASE(false, D, MASK_CAUSAL);               \
      else XATTN_LAUNCH_CASE(false, D, MASK_WINDOW);                                        \
    }                                                                                       \
    return hipGetLastError();                                                               \
  }

}  // namespace xattn
