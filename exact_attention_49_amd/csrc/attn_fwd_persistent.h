// Persistent variant of the ping-pong exact-attention forward kernel for gfx950 (head dim 128),
// behind attn_fwd_persistent / attn_fwd_varlen_persistent.
//
// The per-tile work is the ping-pong kernel's (attn_fwd_pingpong.h): 8 waves of 32 rows in two
// groups, A and B, half a tile apart, each group's MFMA block beside the other's softmax, K/V
// tiles loaded by group B straight into double-buffered LDS.  What differs is the schedule.
// The grid has one workgroup per compute unit (the shape fills a CU), and each workgroup takes
// a static list of q-tiles (Persist: its XCD's work slots in rounds, alternating direction, so
// that heavy and light causal tiles pair up; the persistent tile scheduler of page
// "flash_fwd_kernel.h" @26a6e0a, get_initial_work / get_next_work, here a list fixed at the
// start).  Wave 0 decodes the list into an LDS table once.  The key tiles of the workgroup's
// q-tiles are then swept as one stream of steps g = 0, 1, ...: the pipeline never drains
// between q-tiles.  At the last key tile of a q-tile a wave loads the next q-tile's Q rows
// into its Q registers during its softmax (they are free once its last S = K Q^T is formed),
// stores its O rows and LSE after its last O += V^T P^T, resets O, m, l and goes on with the
// next q-tile's first S in the same MFMA block; the tile loads run on across q-tiles, so the
// next q-tile's first K/V tiles are already in LDS.  Grouped K/V heads are packed as in the
// grid-launched kernel (FwdArgs::pack).
//
// Half-phase schedule (h counts barriers; U_g = {V_g, K_{g+1}} lives in buffer g & 1; steps g
// run over the key tiles of all of the workgroup's q-tiles in order):
//   h = 2g   : A softmax(g)              | B  O += V_{g-1} P_{g-1}, S_g = K_g Q^T
//   h = 2g+1 : A  O += V_g P_g, S_{g+1}  | B softmax(g), and B issues the loads of U_{g+1}
//   B waits for its loads of U_g at the end of h = 2g; the barrier then publishes them.
#pragma once

#include <type_traits>

#include "attn_common.h"
#include "attn_fwd_pingpong.h"

namespace xattn {

// One q-tile of a persistent workgroup's list, as its sweep sees it.
struct PPItem {
  int g0;      // step of the q-tile's first key tile in the workgroup's sweep
  int n;       // key tiles it sweeps (>= 1)
  int t_lo;    // its first key tile
  int seqlen;  // rows (= keys) of its sequence
  int q0;      // its first query row
  long row0;   // its sequence's token 0 in the row space of q / o / lse
  long kv_row0;  // the same in the row space of k / v
};

// A q-tile as one wave of the sweep sees it: which of its steps the wave's rows see, and which
// of those need the mask (a tile crossing the window's left edge, the causal / right edge or
// the sequence's end).
struct PPWave {
  int end;             // one past the q-tile's last step
  int vis_lo, vis_hi;  // steps some row of the wave sees (vis_lo > vis_hi: none)
  int mask_lo;         // steps below this need the left-edge mask
  int mask_hi;         // steps from this one on need the right-edge mask
  int kofs;            // the first key of step g's tile is g * BC + kofs
  int qw0;             // the wave's first query row in the sequence
  int seqlen;          // rows (= keys) of the sequence
  i32x4 rk, rv;        // buffer resources of the sequence's K and V rows (the tile loads)
};

__device__ __forceinline__ int floor_div(int x, int y) {  // y > 0
  return x >= 0 ? x / y : -((-x + y - 1) / y);
}

// Items (q-tiles) a persistent workgroup can hold in its LDS table; the host sizes the grid so
// that no workgroup has more.
constexpr int PP_MAX_ITEMS = 256;

// The workgroup's item table in LDS, built once at the start (pp_build_table): its q-tiles in
// sweep order, each as 12 ints (three 16-byte words: g0, n, t_lo, seqlen | q0, row0 lo, row0 hi,
// kv_row0 lo | kv_row0 hi, -, -, -), and the slots that hold a packed sequence longer than
// max_seqlen (4 ints: row0 lo, row0 hi, first and end row to fill with NaN).
struct PPTable {
  i32x4 item[PP_MAX_ITEMS * 3];
  i32x4 bad[PP_MAX_ITEMS];
  int count, total, nbad;
};

__device__ __forceinline__ PPItem pp_read_item(const PPTable& t, int k) {
  const i32x4 e0 = t.item[3 * k], e1 = t.item[3 * k + 1], e2 = t.item[3 * k + 2];
  auto u = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  PPItem it;
  it.g0 = u(e0[0]);
  it.n = u(e0[1]);
  it.t_lo = u(e0[2]);
  it.seqlen = u(e0[3]);
  it.q0 = u(e1[0]);
  it.row0 = (long)(((unsigned long)(unsigned)u(e1[2]) << 32) | (unsigned)u(e1[1]));
  it.kv_row0 = (long)(((unsigned long)(unsigned)u(e2[0]) << 32) | (unsigned)u(e1[3]));
  return it;
}

// Wave 0 decodes the workgroup's slots, one per lane, 64 at a time (decode_slot), and writes the
// q-tiles to compute, in order, with the step g0 of each one's first key tile (a prefix sum of
// the key-tile counts), and the malformed slots.  The caller publishes it with a barrier.
template <int MODE>
__device__ __forceinline__ void pp_build_table(const FwdArgs& a, const Persist& ps,
                                               PPTable& t, int lane) {
  constexpr int BR = PingPongShape::BR, BC = PingPongShape::BC;
  int wl, wr;
  mode_windows<MODE>(a, wl, wr);
  int base = 0, nbad = 0, g_acc = 0;
  for (int c = 0;; ++c) {
    const int slot = persist_slot(ps, c * 64 + lane);
    if (__builtin_amdgcn_ballot_w64(slot >= 0) == 0) break;
    Work w;
    w.split = 0;
    // with packing, a slot is one group of `pack` query heads of a K/V head ("pseudo-head") and
    // P positions of each
    FwdArgs ap = a;
    ap.heads_q = a.heads_q / a.pack;
    ap.kv_group = a.kv_group / a.pack;
    const int P = BR / a.pack;
    const Decoded d = slot >= 0 ? decode_slot<BR, MODE>(ap, slot, a.n_slots, w, P)
                                : Decoded::Skip;
    w.row0 = (long)a.pack * (w.row0 - w.c0) + w.c0;  // the group's first query head
    const bool run = d == Decoded::Run, bad = d == Decoded::Malformed;
    int n = 0, t_lo = 0;
    if (run) {
      const int q0 = w.tile * P;
      const int q_last = min(q0 + P, w.seqlen) - 1;  // last valid position of the tile
      int k_lo = 0, k_hi = w.seqlen - 1;              // keys any valid row can see
      if (wl >= 0) k_lo = max(0, q0 - wl);
      if (wr >= 0) k_hi = min(w.seqlen - 1, q_last + wr);
      t_lo = k_lo / BC;
      n = k_hi / BC - t_lo + 1;
    }
    // exclusive prefix sum of n over the lanes (n = 0 where no q-tile)
    int incl = n;
#pragma unroll
    for (int d2 = 1; d2 < 64; d2 *= 2) {
      const int up = __shfl_up(incl, d2, 64);
      if (lane >= d2) incl += up;
    }
    const unsigned long mrun = __builtin_amdgcn_ballot_w64(run);
    const unsigned long mbad = __builtin_amdgcn_ballot_w64(bad);
    const unsigned long below = (1ul << lane) - 1;
    if (run) {
      const int k = base + __builtin_popcountl(mrun & below);
      if (k < PP_MAX_ITEMS) {
        t.item[3 * k] = (i32x4){g_acc + incl - n, n, t_lo, w.seqlen};
        t.item[3 * k + 1] = (i32x4){w.tile * P, (int)(unsigned)w.row0,
                                    (int)(unsigned)((unsigned long)w.row0 >> 32),
                                    (int)(unsigned)w.kv_row0};
        t.item[3 * k + 2] = (i32x4){(int)(unsigned)((unsigned long)w.kv_row0 >> 32), 0, 0, 0};
      }
    }
    if (bad) {
      const int k = nbad + __builtin_popcountl(mbad & below);
      if (k < PP_MAX_ITEMS)
        t.bad[k] = (i32x4){(int)(unsigned)w.row0, (int)(unsigned)((unsigned long)w.row0 >> 32),
                           w.bad_lo, w.bad_hi};
    }
    base += __builtin_popcountl(mrun);
    nbad += __builtin_popcountl(mbad);
    g_acc += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) {
    t.count = min(base, PP_MAX_ITEMS);
    t.total = g_acc;
    t.nbad = min(nbad, PP_MAX_ITEMS);
  }
}

template <bool BF16, int D, int MODE, int PF = 3>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_pers_kernel(FwdArgs a) {
  constexpr int BR = PingPongShape::BR, BC = PingPongShape::BC;
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int TILEB = BC * D * 2;             // bytes per K (or V) tile
  constexpr int LOADERS = 4;                    // group B's waves issue the tile loads
  constexpr int LI = BC * CH / (LOADERS * 64);  // load instructions per matrix per loader wave
  static_assert(BC * CH % (LOADERS * 64) == 0, "tile must split evenly over the loader waves");
  static_assert(D == 128, "the persistent ping-pong kernel is built for head dim 128");
  (void)BR;

  __shared__ __attribute__((aligned(1024))) char k_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const bool grp_a = wave < 4;
  int wl, wr;
  mode_windows<MODE>(a, wl, wr);
  // Packed grouped heads (FwdArgs::pack > 1): a q-tile holds `pack` query heads of one K/V
  // head (the kBlockH packing of page "flash_fwd_kernel.h" @c272619) and BR / pack positions
  // of each; wave w computes 32 positions of head w / wpp, so every wave uses the same K/V
  // tiles.  hstride: rows between consecutive query heads.
  const int wpp = 8 / a.pack;  // waves per head of the q-tile
  const long hstride = a.cu_seqlens != nullptr ? (long)a.total_tokens : (long)a.seqlen;

  // ---- the workgroup's q-tiles and the length of its sweep ------------------------------
  __shared__ PPTable tab;
  if (wave == 0) pp_build_table<MODE>(a, persist_init(a.n_slots), tab, lane);
  block_barrier();
  const int n_items = __builtin_amdgcn_readfirstlane(tab.count);
  const int total = __builtin_amdgcn_readfirstlane(tab.total);  // steps of the whole sweep
  {  // rows of packed sequences longer than max_seqlen: NaN (all waves share the work)
    const int nbad = __builtin_amdgcn_readfirstlane(tab.nbad);
    for (int i = 0; i < nbad; ++i) {
      const i32x4 e = tab.bad[i];
      Work w;
      w.row0 = (long)(((unsigned long)(unsigned)__builtin_amdgcn_readfirstlane(e[1]) << 32) |
                      (unsigned)__builtin_amdgcn_readfirstlane(e[0]));
      w.bad_lo = __builtin_amdgcn_readfirstlane(e[2]);
      w.bad_hi = __builtin_amdgcn_readfirstlane(e[3]);
      for (int j = 0; j < a.pack; ++j) {  // every query head of the packed group
        fill_malformed_fwd<D>(a, w);
        w.row0 += hstride;
      }
    }
  }
  if (n_items == 0) return;
  // The q-tile state is updated only outside the group branches, at the start of each step,
  // so that it stays scalar: wcur is this wave's view of the q-tile of step g - 1 (group B's
  // oldest tile in use, table entry k_cur) and wnxt of the one after it; every step either
  // wave group touches lies in one of the two (or, for the loads, possibly further on: looked
  // up in the table).  wv is the wave index
  // as a scalar (the group branches themselves stay as they are).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto kv_rsrc = [&](const PPItem& it, bool is_k) XATTN_INLINE {
    return make_rsrc((is_k ? a.k : a.v) + it.kv_row0 * D, (unsigned)it.seqlen * D * 2);
  };
  auto wave_view = [&](const PPItem& it) XATTN_INLINE {
    PPWave v;
    v.end = it.g0 + it.n;
    v.kofs = (it.t_lo - it.g0) * BC;
    v.seqlen = it.seqlen;
    v.rk = kv_rsrc(it, true);
    v.rv = kv_rsrc(it, false);
    const int qw0 = it.q0 + (wv % wpp) * 32;
    v.qw0 = qw0;
    if (qw0 >= it.seqlen) {  // no row of this wave in the q-tile
      v.vis_lo = v.end;
      v.vis_hi = v.end - 1;
      v.mask_lo = v.mask_hi = 0;
      return v;
    }
    const int qw_last = min(qw0 + 32, it.seqlen) - 1;
    const int kw_lo = wl >= 0 ? max(0, qw0 - wl) : 0;
    const int kw_hi = wr >= 0 ? min(it.seqlen - 1, qw_last + wr) : it.seqlen - 1;
    v.vis_lo = max(it.g0, kw_lo / BC + it.g0 - it.t_lo);
    v.vis_hi = min(v.end - 1, kw_hi / BC + it.g0 - it.t_lo);
    // step g (first key k0 = g BC + kofs) needs the mask iff k0 + BC > seqlen, or (wr >= 0)
    // k0 + BC - 1 > qw0 + wr, or (wl >= 0) k0 < qw0 + 31 - wl
    int r_edge = it.seqlen - BC + 1;  // the smallest k0 that crosses a right edge
    if (wr >= 0) r_edge = min(r_edge, qw0 + wr - BC + 2);
    v.mask_hi = floor_div(r_edge - v.kofs + BC - 1, BC);
    v.mask_lo = wl >= 0 ? floor_div(qw0 + 31 - wl - v.kofs + BC - 1, BC) : -(1 << 30);
    return v;
  };
  int k_cur = 0;
  const PPItem first = pp_read_item(tab, 0);
  PPWave wcur = wave_view(first);
  PPWave wnxt = n_items > 1 ? wave_view(pp_read_item(tab, 1)) : wcur;
  // does some row of this wave see the key tile of step g (g in wcur or wnxt)
  auto sees = [&](int g) XATTN_INLINE {
    return (g >= wcur.vis_lo && g <= wcur.vis_hi) || (g >= wnxt.vis_lo && g <= wnxt.vis_hi);
  };
  // the same for any step g < total: group A's S of step g + 1 (at half-phase 2g + 1) lies past
  // wnxt when wnxt has a single key tile (looked up in the table)
  auto sees_any = [&](int g) XATTN_INLINE {
    if (g < wnxt.end || k_cur + 1 >= n_items) return sees(g);
    int kk = k_cur + 2;
    PPItem t = pp_read_item(tab, kk);
    while (g >= t.g0 + t.n) t = pp_read_item(tab, ++kk);
    const PPWave v = wave_view(t);
    return g >= v.vis_lo && g <= v.vis_hi;
  };
  auto needs_mask = [&](int g) XATTN_INLINE {
    const bool c = g < wcur.end;
    return g < (c ? wcur.mask_lo : wnxt.mask_lo) || g >= (c ? wcur.mask_hi : wnxt.mask_hi);
  };

  const LaneOffsets<D> lo = lane_offsets<D>(lane);
  i32x4 qf[D / 16];
  // the rows of this wave's head, and its first position in a q-tile
  const long hrow = (long)(wv / wpp) * hstride;
  const int wpos = (wv % wpp) * 32;
  load_q<D>(a.q + (first.row0 + hrow) * D, first.q0 + wpos + l32, first.seqlen, hh, qf);

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
  constexpr int ISTEP = LOADERS * 64 * 16;  // bytes per load instruction (all loader waves)
  // Where one K or V tile comes from: the q-tile's K/V rows and the tile's first key.
  struct TileSrc {
    i32x4 rsrc;
    int kbase, seqlen;
    bool full;  // wholly inside the sequence
  };
  auto tile_src = [&](const PPItem& it, int g, bool is_k) XATTN_INLINE {
    TileSrc t;
    t.rsrc = kv_rsrc(it, is_k);
    t.kbase = (it.t_lo + g - it.g0) * BC;
    t.seqlen = it.seqlen;
    t.full = t.kbase + BC <= it.seqlen;
    return t;
  };
  // instruction II of the load of a K (is_k) or V tile into the LDS buffer at `dst`
  auto load_one = [&](auto k_tile, const TileSrc& t, unsigned dst, auto ii) XATTN_INLINE {
    constexpr bool is_k = decltype(k_tile)::value;
    constexpr int II = decltype(ii)::value;
    const unsigned lds = dst + lw * 1024;
    if (t.full) {
      buffer_load_lds16_at<II * ISTEP, II * ISTEP>(t.rsrc, is_k ? voff_k : voff_v,
                                                   t.kbase * D * 2, lds);
    } else {  // last tile: rows past the end re-read the sequence's last row (finite data)
      const int row = lrow + II * (LOADERS * 64 / CH);
      const int crow = min(row, t.seqlen - 1 - t.kbase);
      const int sw = is_k ? swz_k<D>(row) : swz_v<D>(row);
      buffer_load_lds16_at<II * ISTEP, 0>(t.rsrc, crow * D * 2 + ((lch ^ sw) << 4),
                                          t.kbase * D * 2, lds);
    }
  };
  // instruction II of the load of a tile that lies wholly inside the sequence
  auto load_full = [&](auto k_tile, const TileSrc& t, unsigned dst, auto ii) XATTN_INLINE {
    constexpr bool is_k = decltype(k_tile)::value;
    constexpr int II = decltype(ii)::value;
    buffer_load_lds16_at<II * ISTEP, II * ISTEP>(t.rsrc, is_k ? voff_k : voff_v,
                                                 t.kbase * D * 2, dst + lw * 1024);
  };
  auto load_all = [&](auto k_tile, const TileSrc& t, unsigned dst) XATTN_INLINE {
    static_for<LI>([&](auto ii) XATTN_INLINE { load_one(k_tile, t, dst, ii); });
  };
  const std::true_type K_TILE;
  const std::false_type V_TILE;
  const unsigned k_lds0a = lds_address(k_lds0), k_lds1a = lds_address(k_lds1);
  const unsigned v_lds0a = lds_address(v_lds0), v_lds1a = lds_address(v_lds1);
  // The source of key tile g of the sweep (g < total): in wcur or wnxt, or further on (only
  // after a q-tile with a single key tile; looked up in the table).
  auto src_of = [&](int g, bool is_k) XATTN_INLINE {
    if (g < wcur.end || g < wnxt.end || k_cur + 1 >= n_items) {
      const PPWave& v = g < wcur.end ? wcur : wnxt;
      const int kbase = g * BC + v.kofs;
      return TileSrc{is_k ? v.rk : v.rv, kbase, v.seqlen, kbase + BC <= v.seqlen};
    }
    int kk = k_cur + 2;
    PPItem t = pp_read_item(tab, kk);
    while (g >= t.g0 + t.n) t = pp_read_item(tab, ++kk);
    return tile_src(t, g, is_k);
  };

  // ---- the per-tile steps of a wave (g = step of the sweep) --------------------------------
  // the MFMA block: O += V_gpv P_gpv (gpv < 0: none) and, after the last key tile of a
  // q-tile, its epilogue (store, then reset O, m, l); then S_gs = K_gs Q^T (gs = gpv + 1, if it
  // is a step of the sweep; a next q-tile's Q rows are in qf by then)
  auto mfma_block = [&](int gpv, const char* vt, const char* kt) XATTN_INLINE {
    __builtin_amdgcn_s_setprio(2);  // MFMA block: win issue over the partner's softmax
    if (gpv >= 0) {
      if (sees(gpv)) mma_pv<BF16, D, BC, PF>(vt, lo, pf, oacc);
      const bool in_c = gpv < wcur.end;
      if (gpv == (in_c ? wcur.end : wnxt.end) - 1) {  // the q-tile is done: store it, reset
        const PPItem it = pp_read_item(tab, in_c ? k_cur : k_cur + 1);
        const int qw0 = it.q0 + wpos;
        if (qw0 < it.seqlen)
          store_rows<BF16, D>(a, it.row0 + hrow, qw0 + l32, it.seqlen, hh, oacc, m_run, l_run);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
        m_run = -INFINITY;
        l_run = 0.f;
      }
    }
    const int gs = gpv + 1;
    if (gs < total && sees_any(gs)) mma_scores<BF16, D, BC, PF>(kt, lo, qf, sacc);
    __builtin_amdgcn_s_setprio(0);
  };
  // softmax of step g.  At a q-tile's last key tile, the loads of the next q-tile's Q rows
  // into qf start (this wave's last S of the q-tile is formed; they are waited for at the next
  // S).  Group B also issues the loads of U_{g+1} = {V_{g+1}, K_{g+2}}, one instruction every SL
  // exponentials (all at once when the tile is not visible to the wave, or at a q-tile
  // boundary or a sequence's end).
  constexpr int NLD = 2 * LI, SL = (BC / 2) / NLD;
  static_assert((BC / 2) % NLD == 0, "loads must spread evenly over the softmax");
  // (the sliding-window variant runs out of registers with the second softmax copy)
  constexpr bool SPREAD_LOADS = MODE != MASK_WINDOW;
  auto step_softmax = [&](int g, bool loads, unsigned vdst, unsigned kdst) XATTN_INLINE {
    const bool in_c = g < wcur.end;
    const int it_end = in_c ? wcur.end : wnxt.end;
    if (g == it_end - 1 && g + 1 < total) {
      const PPItem nx = pp_read_item(tab, k_cur + (in_c ? 1 : 2));
      load_q_nowait<D>(a.q + (nx.row0 + hrow) * D, nx.q0 + wpos + l32, nx.seqlen, hh, qf);
    }
    const bool vis = sees(g);
    bool spread = false;
    int kb_v = 0;  // first key of V_{g+1} when both loaded tiles are the same q-tile's
    i32x4 rv, rk;
    if (loads && g + 1 < total) {
      if (g + 2 < it_end) {  // the common case: V_{g+1} and K_{g+2} are g's q-tile's
        const PPWave& v = in_c ? wcur : wnxt;
        kb_v = g * BC + v.kofs + BC;
        rv = v.rv;
        rk = v.rk;
        const bool full = kb_v + 2 * BC <= v.seqlen;
        spread = SPREAD_LOADS && full && vis;
        if (!spread) {
          load_all(V_TILE, TileSrc{rv, kb_v, v.seqlen, kb_v + BC <= v.seqlen}, vdst);
          load_all(K_TILE, TileSrc{rk, kb_v + BC, v.seqlen, full}, kdst);
        }
      } else {  // at a q-tile boundary of the load stream
        load_all(V_TILE, src_of(g + 1, false), vdst);
        if (g + 2 < total) load_all(K_TILE, src_of(g + 2, true), kdst);
      }
    }
    if (!vis) return;
    if (needs_mask(g)) {
      const PPWave& v = in_c ? wcur : wnxt;
      mask_scores<BC>(sacc, g * BC + v.kofs, v.qw0 + l32, v.seqlen, wl, wr, hh);
    }
    bool moved;
    float alpha;
    if (spread) {  // one load instruction every SL exponentials: V first, then K
      alpha = softmax_tile<BF16, BC>(sacc, pf, c2, m_run, l_run, moved, [&](int i) XATTN_INLINE {
        at_step<NLD, SL>(i, [&](auto l) XATTN_INLINE {
          constexpr int L = decltype(l)::value;
          sched_fence();  // keep the loads where they are placed
          if constexpr (L < LI)
            load_full(V_TILE, TileSrc{rv, kb_v, 0, true}, vdst, std::integral_constant<int, L>{});
          else
            load_full(K_TILE, TileSrc{rk, kb_v + BC, 0, true}, kdst,
                      std::integral_constant<int, L - LI>{});
          sched_fence();
        });
      });
    } else {
      alpha = softmax_tile<BF16, BC>(sacc, pf, c2, m_run, l_run, moved);
    }
    if (__builtin_amdgcn_ballot_w64(moved) != 0) scale_o<D>(oacc, alpha);  // wave-uniform
  };

  // ---- prologue: K_0 (buffer 1), V_0 and K_1 (buffer 0) ---------------------------------
  if (!grp_a) {
    load_all(K_TILE, src_of(0, true), k_lds1a);
    load_all(V_TILE, src_of(0, false), v_lds0a);
    if (total > 1) load_all(K_TILE, src_of(1, true), k_lds0a);
    wait_vmem();
  }
  block_barrier();
  if (grp_a) mfma_block(-1, v_lds1, k_lds1);  // S_0 only

  // ---- main loop: two half-phases per step, buffer parity P = g & 1 known at compile time ----
  auto iteration = [&](int g, auto parity) XATTN_INLINE {
    constexpr int P = decltype(parity)::value;
    char* const kP = P ? k_lds1 : k_lds0;  // holds K_{g+1}
    char* const kQ = P ? k_lds0 : k_lds1;  // holds K_g, then receives K_{g+2}
    char* const vP = P ? v_lds1 : v_lds0;  // holds V_g
    char* const vQ = P ? v_lds0 : v_lds1;  // holds V_{g-1}, then receives V_{g+1}
    const unsigned kQa = P ? k_lds0a : k_lds1a;
    const unsigned vQa = P ? v_lds0a : v_lds1a;
    // move on once wcur is behind group B (its last tile was B's O += V P of step g - 2)
    if (g - 1 >= wcur.end && k_cur + 1 < n_items) {
      ++k_cur;
      wcur = wnxt;
      if (k_cur + 1 < n_items) wnxt = wave_view(pp_read_item(tab, k_cur + 1));
    }
    // half-phase 2g
    if (grp_a) {
      if (g < total) step_softmax(g, false, 0, 0);
    } else {
      mfma_block(g - 1, vQ, kQ);
    }
    // group B's loads of U_g (issued at half-phase 2g-1); group A's loads of a next q-tile's
    // Q rows are waited for where they are used
    if (!grp_a && g >= 1) wait_vmem();
    block_barrier();
    // half-phase 2g+1
    if (grp_a) {
      if (g < total) mfma_block(g, vP, kP);
    } else {
      if (g < total) step_softmax(g, true, vQa, kQa);
    }
    block_barrier();
  };
  for (int g = 0; g <= total; g += 2) {
    iteration(g, std::integral_constant<int, 0>{});
    if (g + 1 <= total) iteration(g + 1, std::integral_constant<int, 1>{});
  }
}

}  // namespace xattn
