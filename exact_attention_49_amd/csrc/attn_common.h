// Shared pieces of the gfx950 exact-attention kernels (the forward kernels use all of it; the
// backward and FP8 kernels reuse the argument block, the wrappers, work decoding and the
// 16-bit operand steps): argument block, MFMA and conversion wrappers, cross-lane reductions,
// LDS layout (swizzles), work decoding and the per-tile steps (S^T = K Q^T, mask, online
// softmax, O^T += V^T P^T, epilogue).
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
// Register layout (v_mfma_f32_32x32x16, wave64).  The score tile is computed transposed,
// S^T = K Q^T (the swap-AB idea of page "mainloop_bwd_sm90_tma_gmma_ws.hpp", SdP_swapAB):
// lane l of a wave owning 32 query rows holds query (l % 32), and accumulator register r of
// 32-key block kb holds key 32 kb + 8 (r / 4) + 4 (l / 32) + r % 4.  Row max / row sum are
// therefore in-lane plus one exchange between the two 32-lane halves.  The output is
// accumulated transposed too, O^T += V^T P^T: the S^T registers converted to 16-bit are the
// B operand (P^T) as they stand, so P never leaves registers; the matching V^T A operand is
// read from row-major V in LDS with ds_read_b64_tr_b16.  Register r of 32-wide column block db
// of O^T holds d = 32 db + 8 (r / 4) + 4 (l / 32) + r % 4 of the lane's own query.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace xattn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
  // grouped-query attention: q/o have heads_q heads, k/v heads_q / kv_group; query head h
  // reads key/value head h / kv_group (kv_group = 1: one K/V head per query head; page
  // "mainloop_bwd_sm90_tma_gmma_ws.hpp", qhead_per_khead division)
  int heads_q;
  int kv_group;
  // split-KV mode only: the key tiles of each q-tile are shared out among num_splits work
  // items, which write normalised fp32 partial outputs and their LSE instead of o / lse
  int num_splits;             // 1 outside split-KV mode
  long split_rows;            // rows of one split's partial arrays (= rows of o)
  float* o_part;              // [num_splits][split_rows][D]
  float* lse_part;            // [num_splits][split_rows], natural log
  // dense causal ping-pong launches only: the grid covers pairs of q-tiles (m, tiles - 1 - m)
  int fold;
  // persistent launches: work slots of the sweep (the grid is smaller and loops over them)
  int n_slots;
  // ping-pong launches: query heads of one K/V head packed into one q-tile (1: none); a q-tile
  // then holds BR / pack positions of each of them
  int pack;
  // packed batches: the caller's bound on every sequence length (the grid is sized from it)
  int max_seqlen;
};

// The running max is only moved when a tile's row max exceeds it by more than this (in log2
// units), so the O rescale is skipped on almost every tile.  The weights exp2(s - m) then stay
// below 2^8, harmless in fp32 and in the 16-bit P operand, and the result is unchanged: O and
// l are both taken relative to the same reference m, and LSE = m + log2(l).
constexpr float RESCALE_SLACK = 8.0f;
constexpr float RESCALE_LIMIT = 256.0f;  // 2^RESCALE_SLACK: the largest weight exp2(s - m)

// Host: launch a kernel that takes one argument block, and return this launch's own status.
// hipLaunchKernel reports the launch itself; hipGetLastError after a triple-chevron launch
// would also return (and clear) an earlier error left by the caller's own HIP calls.
template <class A>
inline hipError_t launch_kernel(void (*kernel)(A), unsigned grid, unsigned block, hipStream_t s,
                                const A& arg) {
  void* args[] = {const_cast<A*>(&arg)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), args,
                         0, s);
}

// ---------------------------------------------------------------------------------------------
// Instruction wrappers
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

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Workgroup-wide barrier without a memory fence: the compiler may not move memory operations
// across it, and no wait on outstanding global loads is implied (those are waited for
// explicitly where the data is needed).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer resource for raw 32-bit-offset loads from `base` (gfx9 family: no stride, dword data
// format word); `bytes` bounds the range.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long p = (unsigned long long)base;
  // the descriptor must live in scalar registers: the values are uniform by construction
  return (i32x4){__builtin_amdgcn_readfirstlane((int)(unsigned)p),
                 __builtin_amdgcn_readfirstlane((int)((unsigned)(p >> 32) & 0xffffu)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 16 bytes per lane from buffer `rsrc` at voff + soff straight into LDS at lds + 16 * lane
// (buffer_load ... lds).  Issued as inline assembly so that the compiler's wait-count tracking
// does not treat later LDS reads as dependent on it; completion is waited for explicitly with
// wait_vmem() followed by a workgroup barrier.  The LDS address goes through M0, whose previous
// value is restored.
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, int voff, int soff,
                                                  unsigned lds_addr) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)lds_addr);
  int saved;  // M0 is reserved by the compiler: restore whatever it held
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}

// As above, with compile-time byte offsets added in scalar registers inside the instruction
// sequence: LDS address lds_base + LDS_IMM, global offset voff + soff + G_IMM.  Keeps the
// per-instruction constants out of live scalar registers.
template <int LDS_IMM, int G_IMM>
__device__ __forceinline__ void buffer_load_lds16_at(i32x4 rsrc, int voff, int soff,
                                                     unsigned lds_base) {
  int saved, so;
  // the descriptor is uniform by construction; say so, so that it stays in scalar registers
  const i32x4 rs = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_add_u32 m0, %2, %6\n\ts_add_u32 %1, %5, %7\n\t"
      "buffer_load_dwordx4 %3, %4, %1 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved), "=&s"(so)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds_base)), "v"(voff), "s"(rs),
        "s"(__builtin_amdgcn_readfirstlane(soff)), "n"(LDS_IMM), "n"(G_IMM)
      : "memory", "scc");
}

// 4 bytes per lane from buffer `rsrc` at voff + soff straight into LDS at lds_base + 4 * lane
// (buffer_load_dword ... lds); completion as for buffer_load_lds16.
__device__ __forceinline__ void buffer_load_lds4(i32x4 rsrc, int voff, int soff,
                                                 unsigned lds_base) {
  int saved;
  const i32x4 rs = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds_base)), "v"(voff), "s"(rs),
        "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(unsigned long long)((__attribute__((address_space(3))) const char*)p);
}

__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, int voff, int soff,
                                                  const char* lds) {
  buffer_load_lds16(rsrc, voff, soff, lds_address(lds));
}

// Wait until this wave's outstanding vector-memory loads (including loads into LDS) are done.
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

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
// One swizzle for a tile read both ways (32-row ds_read_b128 and 8-row ds_read_b64_tr_b16),
// measured free of bank conflicts for both on gfx950: a bijection on 16 consecutive rows (two
// rows per 256-byte bank line at d = 64) whose top two bits take each value twice over any 8
// aligned rows, so every 64-byte quarter of the bank line is hit twice by a transpose read.
template <int D> __device__ __forceinline__ int swz_rt(int r) {
  static_assert(D == 64 || D == 128, "shared swizzle for head dims 64 and 128");
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// ---------------------------------------------------------------------------------------------
// Work decoding
// ---------------------------------------------------------------------------------------------

struct Work {
  int tile;    // q-tile index within the sequence
  int seqlen;  // rows (= keys) of the sequence
  long row0;   // index of the sequence's token 0 in the [*, D] row space of q/o and lse
  long kv_row0;  // the same for k/v (differs from row0 with grouped K/V heads)
  int split;   // split-KV: which share of the q-tile's key tiles (0 otherwise)
  int bad_lo, bad_hi;  // Decoded::Malformed only: the sequence rows to fill with NaN
  int c0;      // the sequence's first token (0 for a dense batch)
};

// What a workgroup's slot decodes to: nothing (a slot past the last tile), a tile to compute,
// or a tile of a packed sequence longer than the caller's max_seqlen.  Such a sequence is never
// computed or read (the grid and the kernels' 32-bit offsets are sized from max_seqlen): its
// tiles are counted as if it had max_seqlen rows, so the grid still covers them, and their
// workgroups fill every output row of the sequence with NaN instead, the last counted tile
// taking the rows past max_seqlen as well.
enum class Decoded { Skip, Run, Malformed };

// Rows of a malformed sequence of `len` rows that counted tile t of nt (tiles of `rows`)
// fills with NaN.
__device__ __forceinline__ void malformed_rows(int t, int nt, int rows, int len, int& lo,
                                               int& hi) {
  lo = t * rows;
  hi = (t == nt - 1) ? len : min(len, (t + 1) * rows);
}

// Walk the sequences of a packed batch to the one holding q-tile slot `slot` (tiles of
// `rows` rows).  Sets the sequence's first token c0, its length len, the tile index t and the
// sequence's tile count nt (counted with at most max_seqlen rows).  Returns Skip for a slot
// past the last tile, Malformed for a sequence longer than max_seqlen.  Entries of cu_seqlens
// are clamped so that malformed prefix sums cannot address outside [0, total_tokens).
__device__ __forceinline__ Decoded find_seq_tile(const FwdArgs& a, int slot, int rows, int& c0,
                                                 int& len, int& t, int& nt) {
  int acc = 0;
  int c_prev = min(max(a.cu_seqlens[0], 0), a.total_tokens);
  for (int s = 0; s < a.num_seqs; ++s) {
    const int c_next = min(max(a.cu_seqlens[s + 1], c_prev), a.total_tokens);
    const int l = c_next - c_prev;
    const int n = (min(l, a.max_seqlen) + rows - 1) / rows;
    if (slot < acc + n) {
      c0 = c_prev;
      len = l;
      t = slot - acc;
      nt = n;
      return l > a.max_seqlen ? Decoded::Malformed : Decoded::Run;
    }
    acc += n;
    c_prev = c_next;
  }
  return Decoded::Skip;
}

// Fill rows [r0, r1) of a row-major array of `words` 16-byte words per row with all-ones bits
// (a NaN in fp32, fp16 and bf16), with every thread of the workgroup.
__device__ __forceinline__ void fill_nan_rows(void* base, long r0, long r1, int words) {
  i32x4* p = (i32x4*)base + r0 * words;
  const long n = (r1 - r0) * words;
  for (long i = threadIdx.x; i < n; i += blockDim.x) p[i] = (i32x4){-1, -1, -1, -1};
}
__device__ __forceinline__ void fill_nan_f32(float* base, long r0, long r1) {
  for (long i = r0 + threadIdx.x; i < r1; i += blockDim.x) base[i] = __uint_as_float(~0u);
}

// The forward's outputs for a malformed sequence's tile: O (or the split's fp32 partial O)
// and LSE rows set to NaN.
template <int D, bool SPLIT = false>
__device__ __forceinline__ void fill_malformed_fwd(const FwdArgs& a, const Work& w) {
  if constexpr (SPLIT) {
    const long r = (long)w.split * a.split_rows + w.row0;
    fill_nan_rows(a.o_part, r + w.bad_lo, r + w.bad_hi, D / 4);
    fill_nan_f32(a.lse_part, r + w.bad_lo, r + w.bad_hi);
  } else {
    fill_nan_rows(a.o, w.row0 + w.bad_lo, w.row0 + w.bad_hi, D / 8);
    if (a.lse != nullptr) fill_nan_f32(a.lse, w.row0 + w.bad_lo, w.row0 + w.bad_hi);
  }
}

// Map work slot `wid` of a sweep of `nslots` slots to (q-tile, head, batch | sequence).
// Dense batches: heads of all batch entries in order with the q-tiles of a head consecutive;
// masked modes, whose later q-tiles see more keys, instead run each group of heads tile-major,
// heaviest first.  Packed batches: the q-tile slots of a head walk the sequences in order;
// slots past the last tile are unused (Skip).
// (`rows`: rows per q-tile, BR unless the caller packs several heads into a tile.)
template <int BR, int MODE>
__device__ __forceinline__ Decoded decode_slot(const FwdArgs& a, int wid, int nslots, Work& w,
                                               int rows = BR) {
  const int per = a.tiles_per_head;
  if (a.cu_seqlens == nullptr) {
    int bh, t;
    if constexpr (MODE != MASK_NONE) {
      // Masked q-tiles differ in cost (a causal tile m sees m + 1 key tiles).  The (batch,
      // head) pairs are cut into groups of G, inside which the order is tile-major, heaviest
      // first.  G is chosen so that a group holds at least 32 q-tiles (one per CU of an XCD)
      // but no more pairs than an XCD's share of the slots: with a few tiles per head, a
      // head-by-head order would start some heads' heaviest tiles last and leave an XCD on a
      // long tail; with many, one head's tiles already fill the XCD, and all of them stream
      // the same K/V through its L2 together.  With grouped K/V heads a group also holds at
      // least the query heads of one K/V head, so that their tiles run side by side on the
      // same K/V instead of one head after another (B2 Hq32 Hkv8 N8192 causal: 1035 -> 1000 us).
      const int nbh = nslots / per;
      const int G = min((nbh + 7) / 8, max(a.kv_group, (32 + per - 1) / per));
      const int g = wid / (G * per);
      const int r = wid - g * G * per;
      const int gsize = min(G, nbh - g * G);  // the last group may be smaller
      t = r / gsize;
      bh = g * G + (r - t * gsize);
    } else {
      bh = wid / per;
      t = wid - bh * per;
    }
    w.tile = (MODE != MASK_NONE) ? per - 1 - t : t;
    w.seqlen = a.seqlen;
    w.row0 = (long)bh * a.seqlen;
    // (batch, query head) -> (batch, K/V head); query heads of a group are neighbours, so
    // they run on the same XCD and share its L2 copy of the K/V head
    const int b = bh / a.heads_q, h = bh - b * a.heads_q;
    w.kv_row0 = ((long)b * (a.heads_q / a.kv_group) + h / a.kv_group) * a.seqlen;
    w.c0 = 0;
    return Decoded::Run;
  }
  const int h = wid / per;
  const int slot = wid - h * per;
  int c0, len, t, nt;
  const Decoded d = find_seq_tile(a, slot, rows, c0, len, t, nt);
  if (d == Decoded::Skip) return d;
  w.tile = (MODE != MASK_NONE) ? nt - 1 - t : t;
  w.seqlen = len;
  w.row0 = (long)h * a.total_tokens + c0;
  w.kv_row0 = (long)(h / a.kv_group) * a.total_tokens + c0;
  w.c0 = c0;
  if (d == Decoded::Malformed) malformed_rows(t, nt, rows, len, w.bad_lo, w.bad_hi);
  return d;
}

// Map this workgroup of a plain grid (one work slot per workgroup) to its slot and, in
// split-KV mode, a split (the splits of one q-tile are neighbours: they share its Q rows).
// The grid is XCD-remapped, so that an XCD runs a contiguous range of the work list: whole
// heads, whose K/V its L2 then holds, or neighbouring q-tiles, which share most of a window's
// K/V.  A dense causal split-KV grid over at most SPLIT_SPREAD_HEADS (batch, head) pairs is
// not: its heads are long and each fills several XCDs, and a contiguous range of a causal
// head's heaviest-first list would give one XCD all of its heaviest q-tiles (B1 H2 N16384: one
// XCD with 1.7x the mean work).  Workgroup i then runs item i, on XCD i % 8, so every XCD
// takes every eighth item of that list.
// (Measured on MI355X with 2 and 4 splits: B1 H3 N16384 d = 128 331 -> 270 us dealt out one
// by one; at 4 pairs, B1 H4 N8192, no gain at d = 128 and 97 -> 108 us at d = 64.)
constexpr int SPLIT_SPREAD_HEADS = 3;
template <int BR, int MODE, bool SPLIT = false>
__device__ __forceinline__ Decoded decode_work(const FwdArgs& a, Work& w, int rows = BR) {
  int wid = blockIdx.x;
  w.split = 0;
  int nslots = gridDim.x;
  if constexpr (SPLIT) nslots /= a.num_splits;
  if (!(SPLIT && MODE == MASK_CAUSAL && a.cu_seqlens == nullptr &&
        nslots <= SPLIT_SPREAD_HEADS * a.tiles_per_head))
    wid = xcd_remap(wid, gridDim.x);
  if constexpr (SPLIT) {
    w.split = wid % a.num_splits;
    wid /= a.num_splits;
  }
  return decode_slot<BR, MODE>(a, wid, nslots, w, rows);
}

// Persistent grids: workgroup w runs on XCD w % 8.  The work slots are split into 8 contiguous
// ranges, one per XCD (as xcd_remap splits a plain grid), and the workgroups of an XCD take
// its range in rounds, one slot each, alternating direction from round to round.  Slots are
// ordered heaviest first (decode_slot), so a workgroup's heavy slot of one round is paired with
// a light one in the next, and all of an XCD's workgroups work on neighbouring slots (the
// same heads, whose K/V stream through the XCD's L2) at the same time.
struct Persist {
  int base, count;  // this XCD's slot range
  int gx, l;        // workgroups on this XCD and this workgroup's index among them
};
__device__ __forceinline__ Persist persist_init(int nslots) {
  constexpr int NX = 8;
  const int w = blockIdx.x, P = gridDim.x;
  const int x = w % NX;
  const int per = nslots / NX, rem = nslots % NX;
  return {x * per + min(x, rem), per + (x < rem ? 1 : 0), P / NX + (x < P % NX ? 1 : 0), w / NX};
}
// The slot of this workgroup's k-th item, or -1 past its last (rounds are in order, so once a
// round is past the range every later one is too).
__device__ __forceinline__ int persist_slot(const Persist& p, int k) {
  const int local = k * p.gx + ((k & 1) ? p.gx - 1 - p.l : p.l);
  return local < p.count ? p.base + local : -1;
}

// Split-KV: restrict the key-tile range [t_lo, t_lo + n) of a q-tile to the share of split
// `split` (contiguous, as equal as integer division allows; possibly empty).  32-bit
// arithmetic suffices (n * num_splits < 2^31 for any sequence the buffer loads can address).
__device__ __forceinline__ void split_tiles(const FwdArgs& a, int split, int& t_lo, int& n) {
  const unsigned a0 = (unsigned)n * (unsigned)split / (unsigned)a.num_splits;
  const unsigned a1 = (unsigned)n * (unsigned)(split + 1) / (unsigned)a.num_splits;
  t_lo += (int)a0;
  n = (int)(a1 - a0);
}

// Effective window bounds of a mask mode (-1 = unbounded).
template <int MODE>
__device__ __forceinline__ void mode_windows(const FwdArgs& a, int& wl, int& wr) {
  wl = a.window_left;
  wr = a.window_right;
  if (MODE == MASK_NONE) { wl = -1; wr = -1; }
  if (MODE == MASK_CAUSAL) { wl = -1; wr = 0; }
}

// ---------------------------------------------------------------------------------------------
// Per-wave steps on one 32-row query block
// ---------------------------------------------------------------------------------------------

// Q^T operand fragments: lane holds query `row`, d = 16 c + 8 hh .. + 7 (zeros past the end).
// load_q_nowait issues the loads only (their data is waited for where it is first used).
template <int D>
__device__ __forceinline__ void load_q_nowait(const uint16_t* qp, int row, int seqlen, int hh,
                                              i32x4 (&qf)[D / 16]) {
  const i32x4* src = (const i32x4*)(qp + (long)row * D);
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = (row < seqlen) ? src[2 * c + hh] : (i32x4){0, 0, 0, 0};
}
// q_arrived marks the fragments as used here, so that the compiler places the wait for their
// loads at this point and not at their first use inside the K/V sweep (where it would also
// wait for tile loads still in flight: the compiler does not see the loads into LDS).  Kernels
// issue their Q loads, then their first tile loads, then call it, so that the two latencies
// overlap.
template <int D>
__device__ __forceinline__ void q_arrived(const i32x4 (&qf)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" ::"v"(qf[c]));
}
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* qp, int row, int seqlen, int hh,
                                       i32x4 (&qf)[D / 16]) {
  load_q_nowait<D>(qp, row, seqlen, hh, qf);
  q_arrived<D>(qf);
}

// Per-lane LDS byte offsets of the MFMA operand reads.  The swizzle key of every row a lane
// reads is the same (it depends only on row bits fixed by the lane), and it only permutes the
// low four (K) or the bits 2-3 (V) of the 16-byte chunk index.  So an operand address is tile
// base + one of a few lane offsets + a compile-time constant (key block, key chunk, and the
// 256-byte group of the d-chunk), which the compiler folds into the immediate offset.
template <int D>
struct LaneOffsets {
  static constexpr int NK = D / 16 < 8 ? D / 16 : 8;  // distinct K offsets (d-chunks mod 8)
  static constexpr int NV = D / 32 < 4 ? D / 32 : 4;  // distinct V offsets (column blocks mod 4)
  int k[NK];  // K read of d-chunk c: row l32, 16-byte chunk (2c + hh) swizzled
  int v[NV];  // first V transpose read of column block db (add 8 rows for the second)
  int v8[NV];  // shared swizzle only: the second transpose read (8 rows further), whose rows
               // have a different swizzle than the first's
  // byte offset (within a tile) of the K operand of d-chunk c and 32-key block kb
  __device__ __forceinline__ int kofs(int c, int kb) const {
    return k[c % NK] + (c / NK) * 256 + kb * 32 * D * 2;
  }
  // byte offset of the first V transpose read of column block db and 16-key chunk kc
  __device__ __forceinline__ int vofs(int db, int kc) const {
    return v[db % NV] + (db / NV) * 256 + 16 * kc * D * 2;
  }
  __device__ __forceinline__ int vofs8(int db, int kc) const {
    return v8[db % NV] + (db / NV) * 256 + 16 * kc * D * 2;
  }
};

// RT: the tiles use the shared swizzle swz_rt for both read patterns.
template <int D, bool RT = false>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int lane) {
  constexpr int ROWB = D * 2;
  const int l32 = lane & 31, hh = lane >> 5, g = lane >> 4, i16 = lane & 15;
  auto sk = [](int r) {
    if constexpr (RT) return swz_rt<D>(r); else return swz_k<D>(r);
  };
  auto sv = [](int r) {
    if constexpr (RT) return swz_rt<D>(r); else return swz_v<D>(r);
  };
  LaneOffsets<D> o;
#pragma unroll
  for (int c = 0; c < LaneOffsets<D>::NK; ++c)
    o.k[c] = l32 * ROWB + (((2 * c + hh) ^ sk(l32)) << 4);
  const int vrow = 4 * (g >> 1) + (i16 >> 2);
#pragma unroll
  for (int db = 0; db < LaneOffsets<D>::NV; ++db) {
    const int col = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
    o.v[db] = vrow * ROWB + (((col >> 3) ^ sv(vrow)) << 4) + ((col & 7) << 1);
    if constexpr (RT)
      o.v8[db] = (vrow + 8) * ROWB + (((col >> 3) ^ sv(vrow + 8)) << 4) + ((col & 7) << 1);
  }
  return o;
}

// Lambdas that must be inlined (the kernels rely on every array staying in registers).
#define XATTN_INLINE __attribute__((always_inline))

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A sweep over tiles t_lo..t_hi that alternates between two LDS stages, tile t_lo in stage 0:
// step(t, std::integral_constant<int, S>{}) for each tile, unrolled by two so that the stage,
// and with it every LDS operand address of the step, is a compile-time constant (immediate
// offsets instead of address arithmetic per read).
template <class Step>
__device__ __forceinline__ void sweep_two_stages(int t_lo, int t_hi, Step&& step) {
  for (int t = t_lo; t <= t_hi; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 <= t_hi) step(t + 1, std::integral_constant<int, 1>{});
  }
}

// Keeps the compiler from moving instructions across this point, so that operand reads stay
// ahead of the MFMAs that consume them.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// S^T[key, query] = sum_d K[key, d] Q[query, d] for the BC keys of an LDS K tile.  Steps go
// d-chunk by d-chunk, alternating the 32-key blocks (independent accumulators); the K operand
// of step i + PF - 1 is read before the MFMA of step i.  hook(i) runs at the start of step i
// (used to slip other instructions, such as tile loads, between the MFMAs).
struct NoHook {
  template <class I> __device__ __forceinline__ void operator()(I) const {}
};

// Calls f(std::integral_constant<int, k>{}) for the k in [0, N) with i == k * STRIDE, if any.
// Meant for an i that is a constant after loop unrolling: the tests then fold away.
template <int N, int STRIDE, class F>
__device__ __forceinline__ void at_step(int i, F&& f) {
  static_for<N>([&](auto kc) XATTN_INLINE {
    if (i == decltype(kc)::value * STRIDE) f(kc);
  });
}

template <bool BF16, int D, int BC, int PF = 3, class Hook = NoHook>
__device__ __forceinline__ void mma_scores(const char* kt, const LaneOffsets<D>& lo,
                                           const i32x4 (&qf)[D / 16], f32x16 (&s)[BC / 32],
                                           const Hook& hook = Hook()) {
  constexpr int KB = BC / 32, N = (D / 16) * KB;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
  auto read = [&](int i) XATTN_INLINE {
    return *(const i32x4*)(kt + lo.kofs(i / KB, i % KB));
  };
  i32x4 buf[PF];
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) buf[i] = read(i);
  static_for<N>([&](auto ic) XATTN_INLINE {
    constexpr int i = decltype(ic)::value;
    hook(ic);
    if constexpr (i + PF - 1 < N) buf[(i + PF - 1) % PF] = read(i + PF - 1);
    sched_fence();
    s[i % KB] = Elt<BF16>::mfma(buf[i % PF], qf[i / KB], s[i % KB]);
    sched_fence();
  });
}

// Set invisible scores to -inf: key k0 + (tile position) against query qrow.  Register r of
// block kb holds tile offset c = 32 kb + 8 (r / 4) + 4 hh + r % 4; the lane's visible offsets
// form one range [lo, hi] (the key bounds of the row, clipped to the sequence).  Each edge of
// the range is applied only when it falls inside the tile for some lane of the wave, as three
// VALU operations per score: t = hi - c (or c - lo) is negative exactly for the masked scores,
// its sign spread over the word (t >> 31) selects the bits of -inf (a bitfield insert), and no
// lane mask registers are needed.
template <int BC>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[BC / 32], int k0, int qrow, int seqlen,
                                            int wl, int wr, int hh) {
  constexpr int CMAX = BC - 5;  // the largest offset a lane holds: 32 (BC / 32 - 1) + 24 + 3
  constexpr unsigned NEG_INF = 0xff800000u;
  const int base = k0 + 4 * hh;
  int hi = seqlen - 1 - base;
  if (wr >= 0) hi = min(hi, qrow + wr - base);
  const int lo = wl >= 0 ? qrow - wl - base : 0;  // offsets are >= 0: lo <= 0 clips nothing
  auto edge = [&](auto right) XATTN_INLINE {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
        const int t = decltype(right)::value ? hi - c : c - lo;
        const unsigned m = (unsigned)(t >> 31);  // all ones where masked
        s[kb][r] = __uint_as_float((m & NEG_INF) | (~m & __float_as_uint(s[kb][r])));
      }
  };
  if (__builtin_amdgcn_ballot_w64(hi < CMAX) != 0) edge(std::true_type{});
  if (__builtin_amdgcn_ballot_w64(lo > 0) != 0) edge(std::false_type{});
}

// Online softmax of one tile (base 2) with a lazily moved reference max.  Turns the scores
// into P packed to 16-bit (the B operand of O^T += V^T P^T), updates m and the lane's partial
// l, and returns the factor O must be multiplied by (1 unless the reference max moved).
// `moved` tells whether any row of the lane moved it.  hook(i) runs before the exponential of
// the lane's i-th score (used to spread other instructions, such as tile loads, over the step).
template <bool BF16, int BC, class Hook = NoHook>
__device__ __forceinline__ float softmax_tile(f32x16 (&s)[BC / 32], i32x4 (&pf)[BC / 16],
                                              float c2, float& m_run, float& l_run,
                                              bool& moved, const Hook& hook = Hook()) {
  // Row max and row sum over the lane's BC / 2 scores use NP independent partial chains: the
  // serial chain of dependent max / add instructions is what bounds this step otherwise.
  constexpr int NP = 4;
  float pm[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) pm[k] = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) pm[r % NP] = fmaxf(pm[r % NP], s[kb][r]);
  float mx = fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]));
  mx = halves_max(mx) * c2;                          // this tile's row max, log2 units
  const bool move = mx > m_run + RESCALE_SLACK;      // false while both are -inf
  const float m_new = move ? mx : m_run;
  // a row with nothing visible so far keeps m = -inf; subtract 0 so exp2 gives 0, not NaN
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = move ? fast_exp2(m_run - m_use) : 1.f;
  float ps[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) ps[k] = 0.f;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      hook(kb * 16 + r);  // a constant once the loops are unrolled
      const float e = fast_exp2(fmaf(s[kb][r], c2, -m_use));
      s[kb][r] = e;
      ps[r % NP] += e;
    }
  const float rs = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  l_run = fmaf(l_run, alpha, rs);  // per-lane partial; the two halves are summed at the end
  m_run = m_new;
  moved = move;
#pragma unroll
  for (int kc = 0; kc < BC / 16; ++kc) {
    const int kb = kc >> 1, o8 = (kc & 1) * 8;
    pf[kc] = (i32x4){(int)Elt<BF16>::pack2(s[kb][o8 + 0], s[kb][o8 + 1]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 2], s[kb][o8 + 3]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 4], s[kb][o8 + 5]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 6], s[kb][o8 + 7])};
  }
  return alpha;
}

// The common case of softmax_tile, without the tile's row max: the exponentials against the
// running reference m_run, their row sum and P.  Any reference gives the same O and LSE (O and
// l are both taken relative to it); it only has to keep every weight exp2(s - m) in range.
// So the exponentials are taken first and the lane sums checked after: a lane's BC / 2
// weights sum to at most FAST_SUM_LIMIT = (BC / 2) * RESCALE_LIMIT, which bounds each of them
// by 2^13 at BC = 64, far inside fp16's range (the narrowest P operand).  Returns true with
// l_run and pf updated when every lane's sum is within the limit, and false when some lane's
// is not (or is not finite), with s overwritten and l_run, pf untouched; the caller then
// recomputes S and runs softmax_tile.  A failed sum means some weight exceeded
// RESCALE_LIMIT, so softmax_tile moves the reference and the next tiles pass again.  While some
// row of the wave has seen no key (m_run = -inf, its first visible tile) it returns false at
// once, with s untouched.  The weights, sums and P are those softmax_tile computes whenever it
// keeps the reference, in the same order.
template <bool BF16, int BC>
__device__ __forceinline__ bool softmax_tile_fast(f32x16 (&s)[BC / 32], i32x4 (&pf)[BC / 16],
                                                  float c2, float m_run, float& l_run) {
  constexpr float FAST_SUM_LIMIT = (BC / 2) * RESCALE_LIMIT;
  static_assert(FAST_SUM_LIMIT <= 16384.0f, "weights must stay within fp16's range");
  if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0) return false;  // s untouched
  constexpr int NP = 4;
  float ps[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) ps[k] = 0.f;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(s[kb][r], c2, -m_run));
      s[kb][r] = e;
      ps[r % NP] += e;
    }
  const float rs = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  if (__builtin_amdgcn_ballot_w64(!(rs <= FAST_SUM_LIMIT)) != 0) return false;
  l_run += rs;
#pragma unroll
  for (int kc = 0; kc < BC / 16; ++kc) {
    const int kb = kc >> 1, o8 = (kc & 1) * 8;
    pf[kc] = (i32x4){(int)Elt<BF16>::pack2(s[kb][o8 + 0], s[kb][o8 + 1]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 2], s[kb][o8 + 3]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 4], s[kb][o8 + 5]),
                     (int)Elt<BF16>::pack2(s[kb][o8 + 6], s[kb][o8 + 7])};
  }
  return true;
}

template <int D>
__device__ __forceinline__ void scale_o(f32x16 (&o)[D / 32], float alpha) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
}

// O^T[d, query] += sum_key V[key, d] P[query, key] for the BC keys of an LDS V tile.  The A
// operand (V^T) for lane l is column d = 32 db + l % 32, keys 16 kc + 4 hh + {0..3} and
// 16 kc + 8 + 4 hh + {0..3}: the key slots the S^T accumulator gave P.  Two transpose reads
// fetch them.  Steps alternate the column blocks (independent accumulators); the operand of
// step i + PF - 1 is read before the MFMA of step i; hook(i) runs at the start of step i.
// RT: the tile uses the shared swizzle (lane_offsets<D, true>), whose second 8-row read has
// its own offset.
// The A operand of P V step i (both transpose reads).
template <int D, bool RT = false>
__device__ __forceinline__ i32x4 pv_operand(const char* vt, const LaneOffsets<D>& lo, int i) {
  constexpr int ROWB = D * 2, DB = D / 32;
  const char* p = vt + lo.vofs(i % DB, i / DB);
  const char* p8 = RT ? vt + lo.vofs8(i % DB, i / DB) : p + 8 * ROWB;
  const i32x2 a = __builtin_bit_cast(i32x2, lds_read_tr(p));
  const i32x2 b = __builtin_bit_cast(i32x2, lds_read_tr(p8));
  return (i32x4){a[0], a[1], b[0], b[1]};
}
// The operands of the first PF - 1 steps of mma_pv, read ahead of it (before a softmax that
// ends in a branch, which would otherwise expose their LDS latency).
template <int D, int PF = 3, bool RT = false> struct PvHead {
  i32x4 buf[PF - 1];
};
template <int D, int PF = 3, bool RT = false>
__device__ __forceinline__ PvHead<D, PF, RT> pv_head(const char* vt, const LaneOffsets<D>& lo) {
  PvHead<D, PF, RT> h;
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) h.buf[i] = pv_operand<D, RT>(vt, lo, i);
  return h;
}

template <bool BF16, int D, int BC, int PF = 3, bool RT = false, class Hook = NoHook>
__device__ __forceinline__ void mma_pv(const char* vt, const LaneOffsets<D>& lo,
                                       const i32x4 (&pf)[BC / 16], f32x16 (&o)[D / 32],
                                       const Hook& hook = Hook(),
                                       const PvHead<D, PF, RT>* head = nullptr) {
  constexpr int DB = D / 32, N = (BC / 16) * DB;
  auto read = [&](int i) XATTN_INLINE { return pv_operand<D, RT>(vt, lo, i); };
  i32x4 buf[PF];
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) buf[i] = head ? head->buf[i] : read(i);
  static_for<N>([&](auto ic) XATTN_INLINE {
    constexpr int i = decltype(ic)::value;
    hook(ic);
    if constexpr (i + PF - 1 < N) buf[(i + PF - 1) % PF] = read(i + PF - 1);
    sched_fence();
    o[i % DB] = Elt<BF16>::mfma(buf[i % PF], pf[i / DB], o[i % DB]);
    sched_fence();
  });
}

// Two independent score products of one tile as one interleaved sequence: step i of
// s0 = T0 B0^T, then step i of s1 = T1 B1^T (T0, T1 tiles in LDS read like K, B0, B1 operands
// in registers), so that the two streams' operand reads alternate.  Each accumulator receives
// its MFMAs in the same order as in two mma_scores calls (bit-identical results).
template <bool BF16, int D, int BC, int PF = 3>
__device__ __forceinline__ void mma_scores_two(const char* t0, const i32x4 (&b0)[D / 16],
                                               f32x16 (&s0)[BC / 32], const char* t1,
                                               const i32x4 (&b1)[D / 16], f32x16 (&s1)[BC / 32],
                                               const LaneOffsets<D>& lo) {
  constexpr int KB = BC / 32, N = (D / 16) * KB;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[kb][r] = 0.f;
      s1[kb][r] = 0.f;
    }
  auto read = [&](const char* t, int i) XATTN_INLINE {
    return *(const i32x4*)(t + lo.kofs(i / KB, i % KB));
  };
  i32x4 buf0[PF], buf1[PF];
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) {
    buf0[i] = read(t0, i);
    buf1[i] = read(t1, i);
  }
  static_for<N>([&](auto ic) XATTN_INLINE {
    constexpr int i = decltype(ic)::value;
    if constexpr (i + PF - 1 < N) buf0[(i + PF - 1) % PF] = read(t0, i + PF - 1);
    sched_fence();
    s0[i % KB] = Elt<BF16>::mfma(buf0[i % PF], b0[i / KB], s0[i % KB]);
    sched_fence();
    if constexpr (i + PF - 1 < N) buf1[(i + PF - 1) % PF] = read(t1, i + PF - 1);
    sched_fence();
    s1[i % KB] = Elt<BF16>::mfma(buf1[i % PF], b1[i / KB], s1[i % KB]);
    sched_fence();
  });
}

// mma_pv of one tile and mma_scores of the next as one interleaved sequence: P V step i, then
// S step i, so that the transposed V reads and the K reads alternate (and the two operand
// streams share the prefetch window).  Each accumulator receives its MFMAs in the same order
// as in the two separate calls (bit-identical results).
template <bool BF16, int D, int BC, int PF = 3>
__device__ __forceinline__ void mma_pv_scores(const char* vt, const i32x4 (&pf)[BC / 16],
                                              f32x16 (&o)[D / 32], const char* kt,
                                              const i32x4 (&qf)[D / 16], f32x16 (&s)[BC / 32],
                                              const LaneOffsets<D>& lo) {
  constexpr int DB = D / 32, KB = BC / 32, N = (BC / 16) * DB;
  static_assert(N == (D / 16) * KB, "equal step counts");
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
  auto vread = [&](int i) XATTN_INLINE { return pv_operand<D, false>(vt, lo, i); };
  auto kread = [&](int i) XATTN_INLINE {
    return *(const i32x4*)(kt + lo.kofs(i / KB, i % KB));
  };
  i32x4 vbuf[PF], kbuf[PF];
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) {
    vbuf[i] = vread(i);
    kbuf[i] = kread(i);
  }
  static_for<N>([&](auto ic) XATTN_INLINE {
    constexpr int i = decltype(ic)::value;
    if constexpr (i + PF - 1 < N) vbuf[(i + PF - 1) % PF] = vread(i + PF - 1);
    sched_fence();
    o[i % DB] = Elt<BF16>::mfma(vbuf[i % PF], pf[i / DB], o[i % DB]);
    sched_fence();
    if constexpr (i + PF - 1 < N) kbuf[(i + PF - 1) % PF] = kread(i + PF - 1);
    sched_fence();
    s[i % KB] = Elt<BF16>::mfma(kbuf[i % PF], qf[i / KB], s[i % KB]);
    sched_fence();
  });
}

// Epilogue for one 32-row block: O = O / l (16-bit, round to nearest even) and
// LSE = (m + log2 l) ln 2.  All lanes must call it (cross-half sum); rows past the end of the
// sequence are not stored.
template <bool BF16, int D>
__device__ __forceinline__ void store_rows(const FwdArgs& a, long row0, int qrow, int seqlen,
                                           int hh, const f32x16 (&o)[D / 32], float m_run,
                                           float l_run) {
  constexpr float LN2 = 0.693147180559945309f;
  const float lt = halves_sum(l_run);
  if (qrow >= seqlen) return;
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  uint16_t* dst = a.o + (row0 + qrow) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x16& x = o[db];
      const i32x2 val = {(int)Elt<BF16>::pack2(x[4 * g4 + 0] * inv, x[4 * g4 + 1] * inv),
                         (int)Elt<BF16>::pack2(x[4 * g4 + 2] * inv, x[4 * g4 + 3] * inv)};
      *(i32x2*)(dst + db * 32 + 8 * g4 + 4 * hh) = val;
    }
  if (a.lse != nullptr && hh == 0)
    a.lse[row0 + qrow] = lt > 0.f ? (m_run + fast_log2(lt)) * LN2 : -INFINITY;
}

// One wave's 32 rows of a transposed accumulator (register r of column block db holds
// d = 32 db + 8 (r / 4) + 4 hh + r % 4 of the lane's row), times the lane's `mul` and rounded
// to 16 bits, written through the wave's LDS region (32 rows x 2D bytes) so that every global
// store writes whole rows with 16-byte accesses: row r goes to dst + r D for r < nrows.
// The two 8-byte halves of a 16-byte chunk of a row sit in lanes l and l + 32; one
// v_permlane32_swap per dword gathers chunk 4 db + 2 gp in the low lane and chunk
// 4 db + 2 gp + 1 in the high one, so each lane writes whole chunks (ds_write_b128).  Chunk c
// of row r sits at chunk position c ^ g(r), with g(r) = r for 32 or more chunks per row,
// r mod 16 for 16 and r mod 8 for 8, so that any 8 consecutive rows put one chunk into 8
// different 16-byte slots of a 128-byte bank window: the SQ_LDS_BANK_CONFLICT counter shows a
// 16-byte write served 8 lanes at a time over 128 bytes (at 8 chunks per row, the K tile's
// two-rows-per-window swizzle costs 2-way conflicts here), and the read-back, a whole row per
// 8 or 16 lanes, is free of conflicts for any g.  Called by all lanes of the wave; the region
// must not be in use by any other wave.
template <int CH>
__device__ __forceinline__ int staged_chunk(int c, int r) {
  if constexpr (CH == 8) return c ^ (r & 7);
  else if constexpr (CH == 16) return c ^ (r & 15);
  else return c ^ r;
}
template <bool BF16, int D>
__device__ __forceinline__ void store_block_staged(uint16_t* dst, int nrows,
                                                   const f32x16 (&acc)[D / 32], float mul,
                                                   char* region) {
  constexpr int ROWB = D * 2, CH = D / 8, RPI = 64 / CH;  // rows per 64-lane read
  static_assert(CH >= 8 && CH <= 64 && 64 % CH == 0, "one row spans 8 to 64 chunks");
  // the lane index, recomputed here rather than kept live through a kernel's main loop
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int l32 = lane & 31, hh = lane >> 5;
  char* const wrow = region + l32 * ROWB;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const f32x16& x = acc[db];
      const int r0 = 8 * gp;  // registers r0..r0+3: 4 columns of chunk 4 db + 2 gp; r0+4..: of the next
      const uint32_t x0 = Elt<BF16>::pack2(x[r0 + 0] * mul, x[r0 + 1] * mul);
      const uint32_t x1 = Elt<BF16>::pack2(x[r0 + 2] * mul, x[r0 + 3] * mul);
      const uint32_t y0 = Elt<BF16>::pack2(x[r0 + 4] * mul, x[r0 + 5] * mul);
      const uint32_t y1 = Elt<BF16>::pack2(x[r0 + 6] * mul, x[r0 + 7] * mul);
      // low lanes keep x and take the high lanes' x; high lanes take the low lanes' y
      const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
      const i32x4 val = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
      const int c = 4 * db + 2 * gp + hh;
      *(i32x4*)(wrow + (staged_chunk<CH>(c, l32) << 4)) = val;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  const int rsub = lane / CH, c = lane % CH;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + rsub;
    const i32x4 v = *(const i32x4*)(region + r * ROWB + (staged_chunk<CH>(c, r) << 4));
    if (r < nrows) *(i32x4*)(dst + (long)r * D + c * 8) = v;
  }
}

// Epilogue for one wave's 32 rows: O = O / l through store_block_staged and
// LSE = (m + log2 l) ln 2.  Rows past the end of the sequence are not stored.  Called by all
// lanes of the wave; the region must not be in use by any other wave.
template <bool BF16, int D>
__device__ __forceinline__ void store_rows_staged(const FwdArgs& a, long row0, int qrow, int seqlen,
                                                  const f32x16 (&o)[D / 32], float m_run,
                                                  float l_run, char* region) {
  constexpr float LN2 = 0.693147180559945309f;
  const float lt = halves_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const int qw0 = qrow - (__lane_id() & 31);  // the wave's first row
  store_block_staged<BF16, D>(a.o + (row0 + qw0) * D, seqlen - qw0, o, inv, region);
  if (a.lse != nullptr && (__lane_id() >> 5) == 0 && qrow < seqlen)
    a.lse[row0 + qrow] = lt > 0.f ? (m_run + fast_log2(lt)) * LN2 : -INFINITY;
}

// Split-KV epilogue for one 32-row block: the normalised fp32 partial O = O / l and its
// natural-log LSE go to split `split` of the partial arrays.  A row with nothing visible in
// this split gets LSE = -inf and no O (the merge reads no O behind an LSE of -inf).  All lanes
// must call it; rows past the end of the sequence are not stored.
template <int D>
__device__ __forceinline__ void store_rows_partial(const FwdArgs& a, int split, long row0,
                                                   int qrow, int seqlen, int hh,
                                                   const f32x16 (&o)[D / 32], float m_run,
                                                   float l_run) {
  constexpr float LN2 = 0.693147180559945309f;
  const float lt = halves_sum(l_run);
  if (qrow >= seqlen) return;
  const long row = (long)split * a.split_rows + row0 + qrow;
  if (hh == 0) a.lse_part[row] = lt > 0.f ? (m_run + fast_log2(lt)) * LN2 : -INFINITY;
  if (!(lt > 0.f)) return;
  const float inv = 1.0f / lt;
  float* dst = a.o_part + row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x16& x = o[db];
      const f32x4 val = {x[4 * g4 + 0] * inv, x[4 * g4 + 1] * inv, x[4 * g4 + 2] * inv,
                         x[4 * g4 + 3] * inv};
      *(f32x4*)(dst + db * 32 + 8 * g4 + 4 * hh) = val;
    }
}

}  // namespace xattn
