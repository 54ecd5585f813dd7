// C ABI of the exact-attention forward library: argument validation, kernel selection and
// launch.  Declared in include/exact_attn.h.  Validation runs entirely on the host and before
// any HIP call, so a rejected call touches neither the device nor the stream.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "exact_attn.h"
#include "attn_bwd.h"
#include "attn_fwd_fp8.h"
#include "attn_dispatch.h"
#include "attn_fwd_persistent.h"

namespace xattn {
template <> hipError_t launch_fwd<64>(const FwdArgs&, bool, int, bool, int, hipStream_t);
template <> hipError_t launch_fwd<128>(const FwdArgs&, bool, int, bool, int, hipStream_t);
template <> hipError_t launch_fwd<256>(const FwdArgs&, bool, int, bool, int, hipStream_t);
template <> hipError_t launch_fwd<512>(const FwdArgs&, bool, int, bool, int, hipStream_t);
template <> hipError_t launch_fwd_split<64>(const FwdArgs&, bool, int, int, hipStream_t);
template <> hipError_t launch_fwd_split<128>(const FwdArgs&, bool, int, int, hipStream_t);
template <> hipError_t launch_fwd_split<256>(const FwdArgs&, bool, int, int, hipStream_t);
template <> hipError_t launch_fwd_split<512>(const FwdArgs&, bool, int, int, hipStream_t);
template <> hipError_t launch_merge<64>(const MergeArgs&, bool, hipStream_t);
template <> hipError_t launch_merge<128>(const MergeArgs&, bool, hipStream_t);
template <> hipError_t launch_merge<256>(const MergeArgs&, bool, hipStream_t);
template <> hipError_t launch_merge<512>(const MergeArgs&, bool, hipStream_t);
template <> hipError_t launch_bwd<64>(const BwdArgs&, bool, int, int, int, hipStream_t);
template <> hipError_t launch_bwd<128>(const BwdArgs&, bool, int, int, int, hipStream_t);
}  // namespace xattn

// Scratch memory of attn_fwd_splitkv_noalloc: the split partial outputs and their LSE, in a
// device array of fixed size that the library owns (one copy per GPU, held until the process
// ends).  In host code `scratch` only names the symbol: its device address on each GPU comes
// from hipGetSymbolAddress (scratch_address below) and is the only form passed to kernels.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

// Query rows per workgroup of the big / small tile shape of a head dim.
int block_rows(int d, bool big) {
  switch (d) {
    case 64: return big ? xattn::TileCfg<64>::Big::BR : xattn::TileCfg<64>::Small::BR;
    case 128: return big ? xattn::TileCfg<128>::Big::BR : xattn::TileCfg<128>::Small::BR;
    case 256: return big ? xattn::TileCfg<256>::Big::BR : xattn::TileCfg<256>::Small::BR;
    default: return big ? xattn::TileCfg<512>::Big::BR : xattn::TileCfg<512>::Small::BR;
  }
}

// Common checks of the element pointers, dtype, head dim, scale and mask arguments.
int check_common(const void* q, const void* k, const void* v, void* o, const float* lse,
                 int head_dim, int dtype, float scale, int causal, int wl, int wr) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (wl < -1 || wr < -1) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return ATTN_ERR_MISALIGNED;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

// Fold causal into the window bounds and drop bounds that cannot clip anything (which also
// keeps i + window inside int range).  Returns the kernel's mask mode.
int mask_mode(int causal, int max_len, int* wl, int* wr) {
  if (*wl >= max_len) *wl = -1;
  if (*wr >= max_len) *wr = -1;
  if (causal) *wr = 0;  // j <= i and j <= i + wr (wr >= 0) is j <= i
  if (*wl < 0 && *wr < 0) return xattn::MASK_NONE;
  if (*wl < 0 && *wr == 0) return xattn::MASK_CAUSAL;
  return xattn::MASK_WINDOW;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip_error = (int)e;
  return ATTN_ERR_HIP;
}

long varlen_slots(int rows, int num_seqs, int max_seqlen, int total_tokens);
constexpr int kMaxDevices = 64;
// Compute units assumed when the runtime cannot say (MI355X has 256).
constexpr int kDefaultCUs = 256;

// Compute units of HIP device `dev` (the current device for dev < 0), cached per device; the
// default count if the runtime cannot tell.  Host-side query only.
int device_cus(int dev = -1) {
  static std::atomic<int> cache[kMaxDevices];
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return kDefaultCUs;
  if (dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = kDefaultCUs;
    cache[dev].store(cus, std::memory_order_relaxed);
    v = cus;
  }
  return v;
}

// The device a launch on `stream` runs on (the current device for the null stream), or -1.
int stream_device(void* stream) {
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev)
                              : hipGetDevice(&dev);
  return e == hipSuccess ? dev : -1;
}

// Grouped K/V heads on the ping-pong shape: the query heads of a K/V head share each K/V tile
// in one q-tile (`pack` of them, the largest power of two dividing the group, at most 8: one
// wave of 32 positions per head at least), which then holds 256 / pack positions of each.
// Rewrites the tile count per (packed) head and the work count n_work.
int pack_heads(xattn::FwdArgs& b, long& n_work) {
  int pack = 1;
  while (pack < 8 && b.kv_group % (2 * pack) == 0) pack *= 2;
  if (pack == 1) return ATTN_OK;
  const int rows = xattn::PingPongShape::BR / pack;
  const long groups = b.heads_q / pack;  // packed groups of query heads
  long per;
  if (b.cu_seqlens == nullptr) {
    const long batch = n_work / ((long)b.heads_q * b.tiles_per_head);
    per = (b.seqlen + rows - 1) / rows;
    n_work = batch * groups * per;
  } else {
    per = varlen_slots(rows, b.num_seqs, b.max_seqlen, b.total_tokens);
    n_work = groups * per;
  }
  if (per > std::numeric_limits<int>::max() || n_work > std::numeric_limits<int>::max())
    return ATTN_ERR_TOO_LARGE;
  b.tiles_per_head = (int)per;
  b.pack = pack;
  return ATTN_OK;
}

int launch(int head_dim, const xattn::FwdArgs& a, int dtype, int mode, bool big, long n_work,
           void* stream) {
  if (n_work <= 0) return ATTN_OK;
  if (n_work > std::numeric_limits<int>::max()) return ATTN_ERR_TOO_LARGE;
  const bool bf16 = dtype == ATTN_DTYPE_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  xattn::FwdArgs b = a;
  long grid = n_work;
  if (big && head_dim == 128) {
    if (const int st = pack_heads(b, n_work); st != ATTN_OK) return st;
    grid = n_work;
    // Dense causal grids fold the q-tiles of a head into pairs of equal total work (t, T-1-t)
    // when the pairs fill their last round of one workgroup per CU at least to 95%: halving
    // the workgroup count then costs no balance and saves a Q load and a prologue per pair.
    if (mode == xattn::MASK_CAUSAL && b.cu_seqlens == nullptr) {
      const long heads = n_work / b.tiles_per_head;  // (batch, packed head) pairs
      const long pairs = heads * ((b.tiles_per_head + 1) / 2);
      const long cus = device_cus(stream_device(stream));
      const long rounds = (pairs + cus - 1) / cus;
      if (pairs * 20 >= rounds * cus * 19) {
        b.fold = 1;
        grid = pairs;
      }
    }
  }
  switch (head_dim) {
    case 64: return hip_status(xattn::launch_fwd<64>(b, bf16, mode, big, (int)grid, s));
    case 128: return hip_status(xattn::launch_fwd<128>(b, bf16, mode, big, (int)grid, s));
    case 256: return hip_status(xattn::launch_fwd<256>(b, bf16, mode, big, (int)grid, s));
    default: return hip_status(xattn::launch_fwd<512>(b, bf16, mode, big, (int)grid, s));
  }
}

// The persistent ping-pong kernel (head dim 128, 256-row q-tiles): one workgroup per compute
// unit, each sweeping its list of the n_work q-tile slots.
int launch_persistent(const xattn::FwdArgs& a, int dtype, int mode, long n_work, void* stream) {
  if (n_work <= 0) return ATTN_OK;
  xattn::FwdArgs b = a;
  if (const int st = pack_heads(b, n_work); st != ATTN_OK) return st;
  if (n_work > std::numeric_limits<int>::max()) return ATTN_ERR_TOO_LARGE;
  b.fold = 0;
  b.n_slots = (int)n_work;
  const long cus = device_cus(stream_device(stream));
  long grid = n_work < cus ? n_work : cus;
  // each workgroup's list must fit its LDS item table: the slots split into 8 XCD ranges of at
  // most ceil(n_work / 8), shared by the XCD's workgroups
  const long per_xcd = (n_work + 7) / 8;
  const long wg_per_xcd = (per_xcd + xattn::PP_MAX_ITEMS - 1) / xattn::PP_MAX_ITEMS;
  if (grid < 8 * wg_per_xcd) grid = 8 * wg_per_xcd;
  return hip_status(xattn::launch_fwd_persistent(b, dtype == ATTN_DTYPE_BF16, mode, (int)grid,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

// Split-KV: the split sweep (grid = n_work x num_splits) and then the merge.
int launch_split(int head_dim, const xattn::FwdArgs& a, const xattn::MergeArgs& m, int dtype,
                 int mode, long n_work, void* stream) {
  const long grid = n_work * a.num_splits;
  if (n_work <= 0) return ATTN_OK;
  if (grid > std::numeric_limits<int>::max() || (m.rows + 1) / 2 > 0x7fffffffL)  // merge grid
    return ATTN_ERR_TOO_LARGE;
  const bool bf16 = dtype == ATTN_DTYPE_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  switch (head_dim) {
    case 64: e = xattn::launch_fwd_split<64>(a, bf16, mode, (int)grid, s); break;
    case 128: e = xattn::launch_fwd_split<128>(a, bf16, mode, (int)grid, s); break;
    case 256: e = xattn::launch_fwd_split<256>(a, bf16, mode, (int)grid, s); break;
    default: e = xattn::launch_fwd_split<512>(a, bf16, mode, (int)grid, s); break;
  }
  if (e != hipSuccess) return hip_status(e);
  switch (head_dim) {
    case 64: return hip_status(xattn::launch_merge<64>(m, bf16, s));
    case 128: return hip_status(xattn::launch_merge<128>(m, bf16, s));
    case 256: return hip_status(xattn::launch_merge<256>(m, bf16, s));
    default: return hip_status(xattn::launch_merge<512>(m, bf16, s));
  }
}

constexpr float kLog2e = 1.44269504088896340736f;
constexpr long kMaxRows = 1L << 40;  // rows * head_dim stays far inside int64
// The kernels address one sequence's K/V rows with 32-bit byte offsets (buffer loads).
constexpr long kMaxSeqBytes = (1L << 31) - 1;
constexpr int kMaxSplits = 64;
// Workgroups of the small shape resident per CU at once: four at d = 64, two at d = 128
// (register-bound), one for the wide head dims (LDS-bound).  (Measured on MI355X, B1 H2 N16384
// d64 causal: 4 splits 168 us, 3 splits 171 us.)
int resident_per_cu(int d) { return d == 64 ? 4 : d == 128 ? 2 : 1; }
// Keys per K/V tile of the small shape.
int small_tile_keys(int d) { return d >= 256 ? xattn::WideShape::BC : 64; }

// A validated launch: the kernel arguments and the grid for one tile shape.
struct Plan {
  int status = ATTN_OK;
  bool empty = false;    // nothing to compute (a zero size): return OK without launching
  xattn::FwdArgs a{};
  int mode = 0;
  bool big = false;
  long n_work = 0;       // workgroups of one sweep (one split)
  long rows = 0;         // rows of o
  int max_len = 0;       // longest sequence
};

// shape: 1 = choose (big if the grid is large enough), 0 = small shape, 2 = big shape.
Plan plan_dense(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                int heads, int heads_kv, int seqlen, int head_dim, int dtype,
                float softmax_scale, int causal, int window_left, int window_right, int shape) {
  Plan p;
  if (batch < 0 || heads < 0 || seqlen < 0) { p.status = ATTN_ERR_INVALID_ARG; return p; }
  if (heads > 0 && (heads_kv < 1 || heads % heads_kv != 0)) {
    p.status = ATTN_ERR_INVALID_ARG;
    return p;
  }
  p.rows = (long)batch * heads * seqlen;
  if (p.rows == 0) {  // empty problem: still reject malformed non-size arguments
    if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16)
      p.status = ATTN_ERR_UNSUPPORTED_DTYPE;
    else if (!supported_head_dim(head_dim))
      p.status = ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    p.empty = true;
    return p;
  }
  p.status = check_common(q, k, v, o, lse, head_dim, dtype, softmax_scale, causal, window_left,
                          window_right);
  if (p.status != ATTN_OK) return p;
  if (p.rows > kMaxRows || (long)seqlen * head_dim * 2 > kMaxSeqBytes) {
    p.status = ATTN_ERR_TOO_LARGE;
    return p;
  }
  int wl = window_left, wr = window_right;
  p.mode = mask_mode(causal, seqlen, &wl, &wr);
  const int br_big = block_rows(head_dim, true);
  const long big_tiles = (long)batch * heads * ((seqlen + br_big - 1) / br_big);
  p.big = shape == 2 || (shape == 1 && big_tiles >= xattn::big_tile_min_work(p.mode));
  const int br = block_rows(head_dim, p.big);
  xattn::FwdArgs& a = p.a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.cu_seqlens = nullptr;
  a.seqlen = seqlen;
  a.tiles_per_head = (seqlen + br - 1) / br;
  a.scale_log2 = softmax_scale * kLog2e;
  a.window_left = wl;
  a.window_right = wr;
  a.heads_q = heads;
  a.kv_group = heads / heads_kv;
  a.num_splits = 1;
  a.pack = 1;
  a.max_seqlen = seqlen;
  p.n_work = (long)batch * heads * a.tiles_per_head;
  p.max_len = seqlen;
  return p;
}

Plan plan_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                 const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                 int heads, int heads_kv, int head_dim, int dtype, float softmax_scale,
                 int causal, int window_left, int window_right, int shape) {
  Plan p;
  if (num_seqs < 0 || total_tokens < 0 || heads < 0 || max_seqlen < 0) {
    p.status = ATTN_ERR_INVALID_ARG;
    return p;
  }
  if (heads > 0 && (heads_kv < 1 || heads % heads_kv != 0)) {
    p.status = ATTN_ERR_INVALID_ARG;
    return p;
  }
  if (num_seqs == 0 || total_tokens == 0 || heads == 0) {
    if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16)
      p.status = ATTN_ERR_UNSUPPORTED_DTYPE;
    else if (!supported_head_dim(head_dim))
      p.status = ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    p.empty = true;
    return p;
  }
  p.status = check_common(q, k, v, o, lse, head_dim, dtype, softmax_scale, causal, window_left,
                          window_right);
  if (p.status != ATTN_OK) return p;
  if (!cu_seqlens) { p.status = ATTN_ERR_INVALID_ARG; return p; }
  if (!aligned(cu_seqlens, 4)) { p.status = ATTN_ERR_MISALIGNED; return p; }
  if (max_seqlen < 1 || max_seqlen > total_tokens) { p.status = ATTN_ERR_INVALID_ARG; return p; }
  p.rows = (long)heads * total_tokens;
  if (p.rows > kMaxRows || (long)max_seqlen * head_dim * 2 > kMaxSeqBytes) {
    p.status = ATTN_ERR_TOO_LARGE;
    return p;
  }
  int wl = window_left, wr = window_right;
  p.mode = mask_mode(causal, max_seqlen, &wl, &wr);
  const int br_big = block_rows(head_dim, true);
  const long big_tiles = (long)heads * (((long)total_tokens + br_big - 1) / br_big);
  p.big = shape == 2 || (shape == 1 && big_tiles >= xattn::big_tile_min_work(p.mode));
  const int br = block_rows(head_dim, p.big);
  // q-tile slots per head: an upper bound on sum_s ceil(len_s / br) that needs no lengths
  const long by_total = ((long)total_tokens + br - 1) / br + num_seqs;
  const long by_max = (long)num_seqs * ((max_seqlen + br - 1) / br);
  const long slots = by_total < by_max ? by_total : by_max;
  if (slots > std::numeric_limits<int>::max()) { p.status = ATTN_ERR_TOO_LARGE; return p; }
  xattn::FwdArgs& a = p.a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.seqlen = 0;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.tiles_per_head = (int)slots;
  a.scale_log2 = softmax_scale * kLog2e;
  a.window_left = wl;
  a.window_right = wr;
  a.heads_q = heads;
  a.kv_group = heads / heads_kv;
  a.num_splits = 1;
  a.pack = 1;
  a.max_seqlen = max_seqlen;
  p.n_work = (long)heads * slots;
  p.max_len = max_seqlen;
  return p;
}

// Split count for num_splits = 0: enough work items to give every CU its resident share of
// small-shape workgroups, keeping at least eight K/V tiles per split (shorter splits cost more
// in merge traffic and per-workgroup set-up than they gain); 1 when the plain grid already
// fills the chip.  `spread`: a dense causal grid of at most SPLIT_SPREAD_HEADS (batch, head)
// pairs, whose items are dealt out to the XCDs one by one (decode_work) and range from one key
// tile to all of them; with the heaviest items at twice the mean, one item per slot would leave
// the chip on a tail of them, and twice the items balance it, as long as a split of the longest
// range keeps 16 key tiles (its items average half of that).  Chosen by measurement on MI355X
// over dense and causal shapes (d = 128 causal, 4 splits against 2: B1 H2 N16384 251 -> 194 us,
// B1 H1 N32768 366 -> 320 us; with more heads, B1 H8 N4096, 2 splits stay best: 77 vs 82 us;
// B1 H1 N8192, 16 splits against 8: 69 vs 64 us).
int auto_splits(long n_work, int max_len, int head_dim, bool spread) {
  const long target = (long)device_cus() * resident_per_cu(head_dim);
  const int tiles = (max_len + small_tile_keys(head_dim) - 1) / small_tile_keys(head_dim);
  auto count = [&](long items, int min_tiles) -> long {
    if (n_work <= 0 || n_work >= items) return 1;
    const long s = (items + n_work - 1) / n_work;
    return s < tiles / min_tiles ? s : tiles / min_tiles;
  };
  long s = count(target, 8);
  if (spread) s = std::max(s, count(2 * target, 16));
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace bytes for num_splits partial outputs of `rows` rows of head_dim fp32 plus their LSE.
size_t workspace_bytes_for(long rows, int head_dim, int num_splits) {
  if (num_splits <= 1) return 0;
  return align256((size_t)num_splits * rows * head_dim * 4) +
         align256((size_t)num_splits * rows * 4);
}

// Run a plan as split-KV with the given split count (> 1) in the caller's workspace.
int run_split(Plan& p, int head_dim, int dtype, int num_splits, void* workspace,
              size_t workspace_size, void* stream) {
  const size_t need = workspace_bytes_for(p.rows, head_dim, num_splits);
  if (!workspace || !aligned(workspace, 256) || workspace_size < need)
    return ATTN_ERR_INVALID_ARG;
  char* ws = static_cast<char*>(workspace);
  p.a.num_splits = num_splits;
  p.a.split_rows = p.rows;
  p.a.o_part = reinterpret_cast<float*>(ws);
  p.a.lse_part =
      reinterpret_cast<float*>(ws + align256((size_t)num_splits * p.rows * head_dim * 4));
  xattn::MergeArgs m{};
  m.o_part = p.a.o_part;
  m.lse_part = p.a.lse_part;
  m.o = p.a.o;
  m.lse = p.a.lse;
  m.rows = p.rows;
  m.num_splits = num_splits;
  return launch_split(head_dim, p.a, m, dtype, p.mode, p.n_work, stream);
}

// ---- allocation-free split-KV --------------------------------------------------------------

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the GPU that runs `stream` (the current device for the null
// stream), looked up once per device with that device current and cached.
int scratch_address(void* stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev)
                        : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e != hipSuccess) return hip_status(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_status(e);
    if (e2 != hipSuccess) return hip_status(e2);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

// ---- backward ---------------------------------------------------------------------------

bool bwd_head_dim(int d) { return d == 64 || d == 128; }

// Tile slots per head of `rows`-row tiles for a packed batch: an upper bound on
// sum_s ceil(len_s / rows) that needs no lengths.
long varlen_slots(int rows, int num_seqs, int max_seqlen, int total_tokens) {
  const long by_total = ((long)total_tokens + rows - 1) / rows + num_seqs;
  const long by_max = (long)num_seqs * ((max_seqlen + rows - 1) / rows);
  return by_total < by_max ? by_total : by_max;
}

// dPsum, then the LSE in log2 units: one fp32 per query row each, 256-byte aligned arrays.
size_t bwd_workspace_bytes(long rows) { return rows > 0 ? 2 * align256((size_t)rows * 4) : 0; }

// The gradient-side arguments of a backward call (the forward-side ones went through a Plan).
int check_bwd_pointers(const float* lse, const void* dout, void* dq, void* dk, void* dv) {
  if (!lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

// Launch both backward kernels for a validated plan: q_slots q-tiles per query head (dQ
// kernel) and k_slots key tiles per key/value head (dK/dV kernel), over heads_q query heads
// and heads_q / kv_group key/value heads.
int run_bwd(const Plan& p, int head_dim, int dtype, long q_slots, long k_slots, long heads_q,
            long outer, const void* dout, void* dq, void* dk, void* dv, float scale,
            void* workspace, size_t workspace_size, void* stream) {
  if (!workspace || !aligned(workspace, 256) || workspace_size < bwd_workspace_bytes(p.rows))
    return ATTN_ERR_INVALID_ARG;
  const long n_q = outer * heads_q * q_slots;
  const long n_k = outer * (heads_q / p.a.kv_group) * k_slots;
  constexpr long kIntMax = std::numeric_limits<int>::max();
  if (q_slots > kIntMax || k_slots > kIntMax || n_q > kIntMax || n_k > kIntMax)
    return ATTN_ERR_TOO_LARGE;
  xattn::BwdArgs b{};
  b.f = p.a;
  b.f.tiles_per_head = (int)q_slots;
  b.ktiles_per_head = (int)k_slots;
  b.dout = static_cast<const uint16_t*>(dout);
  b.dq = static_cast<uint16_t*>(dq);
  b.dk = static_cast<uint16_t*>(dk);
  b.dv = static_cast<uint16_t*>(dv);
  b.dpsum = static_cast<float*>(workspace);
  b.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)p.rows * 4));
  b.scale = scale;
  const bool bf16 = dtype == ATTN_DTYPE_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (head_dim == 64)
    return hip_status(xattn::launch_bwd<64>(b, bf16, p.mode, (int)n_q, (int)n_k, s));
  return hip_status(xattn::launch_bwd<128>(b, bf16, p.mode, (int)n_q, (int)n_k, s));
}

// ---- FP8 forward -------------------------------------------------------------------------

bool fp8_head_dim(int d) { return d == 64 || d == 128 || d == 256; }

int run_fp8(Plan& p, int head_dim, long slots, long heads, long outer, const float* dq,
            const float* dk, const float* dv, int out_dtype, void* stream) {
  if ((dq && !aligned(dq, 4)) || (dk && !aligned(dk, 4)) || (dv && !aligned(dv, 4)))
    return ATTN_ERR_MISALIGNED;
  const long n_work = outer * heads * slots;
  if (slots > std::numeric_limits<int>::max() || n_work > std::numeric_limits<int>::max())
    return ATTN_ERR_TOO_LARGE;
  xattn::Fp8Args f{};
  f.f = p.a;
  f.f.tiles_per_head = (int)slots;
  f.descale_q = dq;
  f.descale_k = dk;
  f.descale_v = dv;
  return hip_status(xattn::launch_fwd_fp8(f, head_dim, out_dtype == ATTN_DTYPE_BF16, p.mode,
                                          (int)n_work, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
             int heads, int seqlen, int head_dim, int dtype, float softmax_scale, int causal,
             int window_left, int window_right, void* stream) {
  Plan p = plan_dense(q, k, v, o, lse, batch, heads, heads, seqlen, head_dim, dtype,
                      softmax_scale, causal, window_left, window_right, 1);
  if (p.status != ATTN_OK || p.empty) return p.status;
  return launch(head_dim, p.a, dtype, p.mode, p.big, p.n_work, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                    int heads, int head_dim, int dtype, float softmax_scale, int causal,
                    int window_left, int window_right, void* stream) {
  Plan p = plan_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total_tokens, heads,
                       heads, head_dim, dtype, softmax_scale, causal, window_left, window_right,
                       1);
  if (p.status != ATTN_OK || p.empty) return p.status;
  return launch(head_dim, p.a, dtype, p.mode, p.big, p.n_work, stream);
}

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                 int heads_q, int heads_kv, int seqlen, int head_dim, int dtype,
                 float softmax_scale, int causal, int window_left, int window_right,
                 void* stream) {
  Plan p = plan_dense(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen, head_dim, dtype,
                      softmax_scale, causal, window_left, window_right, 1);
  if (p.status != ATTN_OK || p.empty) return p.status;
  return launch(head_dim, p.a, dtype, p.mode, p.big, p.n_work, stream);
}

int attn_fwd_varlen_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                        int total_tokens, int heads_q, int heads_kv, int head_dim, int dtype,
                        float softmax_scale, int causal, int window_left, int window_right,
                        void* stream) {
  Plan p = plan_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total_tokens,
                       heads_q, heads_kv, head_dim, dtype, softmax_scale, causal, window_left,
                       window_right, 1);
  if (p.status != ATTN_OK || p.empty) return p.status;
  return launch(head_dim, p.a, dtype, p.mode, p.big, p.n_work, stream);
}

int attn_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse,
                        int batch, int heads_q, int heads_kv, int seqlen, int head_dim,
                        int dtype, float softmax_scale, int causal, int window_left,
                        int window_right, void* stream) {
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  Plan p = plan_dense(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen, head_dim, dtype,
                      softmax_scale, causal, window_left, window_right, 2);
  if (p.status != ATTN_OK || p.empty) return p.status;
  return launch_persistent(p.a, dtype, p.mode, p.n_work, stream);
}

int attn_fwd_varlen_persistent(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                               int total_tokens, int heads_q, int heads_kv, int head_dim,
                               int dtype, float softmax_scale, int causal, int window_left,
                               int window_right, void* stream) {
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  Plan p = plan_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total_tokens,
                       heads_q, heads_kv, head_dim, dtype, softmax_scale, causal, window_left,
                       window_right, 2);
  if (p.status != ATTN_OK || p.empty) return p.status;
  return launch_persistent(p.a, dtype, p.mode, p.n_work, stream);
}

// Whether a dense split-KV call deals its items out to the XCDs one by one (decode_work): a
// causal mask without a left window, over at most SPLIT_SPREAD_HEADS (batch, head) pairs.
bool split_spread(int batch, int heads, int seqlen, int causal, int window_left) {
  return causal && (window_left < 0 || window_left >= seqlen) &&
         (long)batch * heads <= xattn::SPLIT_SPREAD_HEADS;
}

int attn_fwd_splitkv_num_splits(int batch, int heads, int seqlen, int head_dim, int causal,
                                int window_left) {
  if (batch <= 0 || heads <= 0 || seqlen <= 0 || !supported_head_dim(head_dim)) return 1;
  const int br = block_rows(head_dim, false);
  const long n_work = (long)batch * heads * ((seqlen + br - 1) / br);
  return auto_splits(n_work, seqlen, head_dim,
                     split_spread(batch, heads, seqlen, causal, window_left));
}

size_t attn_fwd_splitkv_workspace_size(int batch, int heads, int seqlen, int head_dim,
                                       int num_splits, int causal, int window_left) {
  if (batch <= 0 || heads <= 0 || seqlen <= 0 || !supported_head_dim(head_dim) ||
      num_splits < 0 || num_splits > kMaxSplits)
    return 0;
  const int s = num_splits ? num_splits
                           : attn_fwd_splitkv_num_splits(batch, heads, seqlen, head_dim, causal,
                                                         window_left);
  return workspace_bytes_for((long)batch * heads * seqlen, head_dim, s);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads, int heads_kv, int seqlen, int head_dim, int dtype,
                     float softmax_scale, int causal, int window_left, int window_right,
                     int num_splits, void* workspace, size_t workspace_size, void* stream) {
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
  Plan p = plan_dense(q, k, v, o, lse, batch, heads, heads_kv, seqlen, head_dim, dtype,
                      softmax_scale, causal, window_left, window_right, 0);
  if (p.status != ATTN_OK || p.empty) return p.status;
  const int s = num_splits ? num_splits
                           : attn_fwd_splitkv_num_splits(batch, heads, seqlen, head_dim, causal,
                                                         window_left);
  if (s == 1)
    return attn_fwd_gqa(q, k, v, o, lse, batch, heads, heads_kv, seqlen, head_dim, dtype,
                        softmax_scale, causal, window_left, window_right, stream);
  return run_split(p, head_dim, dtype, s, workspace, workspace_size, stream);
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int batch, int heads, int heads_kv, int seqlen, int head_dim,
                             int dtype, float softmax_scale, int causal, int window_left,
                             int window_right, int num_splits, void* stream) {
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
  Plan p = plan_dense(q, k, v, o, lse, batch, heads, heads_kv, seqlen, head_dim, dtype,
                      softmax_scale, causal, window_left, window_right, 0);
  if (p.status != ATTN_OK || p.empty) return p.status;
  int s = num_splits;
  if (s == 0) {  // the library's choice, lowered to the largest count whose partials fit
    s = attn_fwd_splitkv_num_splits(batch, heads, seqlen, head_dim, causal, window_left);
    while (s > 1 && workspace_bytes_for(p.rows, head_dim, s) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
      --s;
  }
  if (s == 1)  // the plain kernels need no scratch
    return attn_fwd_gqa(q, k, v, o, lse, batch, heads, heads_kv, seqlen, head_dim, dtype,
                        softmax_scale, causal, window_left, window_right, stream);
  if (workspace_bytes_for(p.rows, head_dim, s) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return ATTN_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int st = scratch_address(stream, &ws);
  if (st != ATTN_OK) return st;
  return run_split(p, head_dim, dtype, s, ws, ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

int attn_fwd_varlen_splitkv_num_splits(int num_seqs, int max_seqlen, int total_tokens,
                                       int heads, int head_dim) {
  if (num_seqs <= 0 || max_seqlen <= 0 || total_tokens <= 0 || heads <= 0 ||
      !supported_head_dim(head_dim))
    return 1;
  const int br = block_rows(head_dim, false);
  const long by_total = ((long)total_tokens + br - 1) / br + num_seqs;
  const long by_max = (long)num_seqs * ((max_seqlen + br - 1) / br);
  return auto_splits((long)heads * (by_total < by_max ? by_total : by_max), max_seqlen,
                     head_dim, false);
}

size_t attn_fwd_varlen_splitkv_workspace_size(int num_seqs, int max_seqlen, int total_tokens,
                                              int heads, int head_dim, int num_splits) {
  if (num_seqs <= 0 || max_seqlen <= 0 || total_tokens <= 0 || heads <= 0 ||
      !supported_head_dim(head_dim) || num_splits < 0 || num_splits > kMaxSplits)
    return 0;
  const int s = num_splits ? num_splits
                           : attn_fwd_varlen_splitkv_num_splits(num_seqs, max_seqlen,
                                                                total_tokens, heads, head_dim);
  return workspace_bytes_for((long)heads * total_tokens, head_dim, s);
}

int attn_fwd_varlen_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                            int total_tokens, int heads, int heads_kv, int head_dim,
                            int dtype, float softmax_scale, int causal, int window_left,
                            int window_right, int num_splits, void* workspace,
                            size_t workspace_size, void* stream) {
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
  Plan p = plan_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total_tokens, heads,
                       heads_kv, head_dim, dtype, softmax_scale, causal, window_left,
                       window_right, 0);
  if (p.status != ATTN_OK || p.empty) return p.status;
  const int s = num_splits ? num_splits : auto_splits(p.n_work, p.max_len, head_dim, false);
  if (s == 1)
    return attn_fwd_varlen_gqa(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen,
                               total_tokens, heads, heads_kv, head_dim, dtype, softmax_scale,
                               causal, window_left, window_right, stream);
  return run_split(p, head_dim, dtype, s, workspace, workspace_size, stream);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 const float* descale_q, const float* descale_k, const float* descale_v,
                 int batch, int heads_q, int heads_kv, int seqlen, int head_dim, int out_dtype,
                 float softmax_scale, int causal, int window_left, int window_right,
                 void* stream) {
  if (!fp8_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  Plan p = plan_dense(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen, head_dim, out_dtype,
                      softmax_scale, causal, window_left, window_right, 0);
  if (p.status != ATTN_OK || p.empty) return p.status;
  const int br = xattn::fp8_block_rows(head_dim);
  const long slots = ((long)seqlen + br - 1) / br;
  return run_fp8(p, head_dim, slots, heads_q, batch, descale_q, descale_k, descale_v, out_dtype,
                 stream);
}

int attn_fwd_varlen_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                        const float* descale_q, const float* descale_k,
                        const float* descale_v, const int32_t* cu_seqlens, int num_seqs,
                        int max_seqlen, int total_tokens, int heads_q, int heads_kv,
                        int head_dim, int out_dtype, float softmax_scale, int causal,
                        int window_left, int window_right, void* stream) {
  if (!fp8_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  Plan p = plan_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total_tokens,
                       heads_q, heads_kv, head_dim, out_dtype, softmax_scale, causal,
                       window_left, window_right, 0);
  if (p.status != ATTN_OK || p.empty) return p.status;
  return run_fp8(p, head_dim,
                 varlen_slots(xattn::fp8_block_rows(head_dim), num_seqs, max_seqlen,
                              total_tokens), heads_q,
                 1, descale_q, descale_k, descale_v, out_dtype, stream);
}

size_t attn_bwd_workspace_size(int batch, int heads_q, int seqlen) {
  if (batch <= 0 || heads_q <= 0 || seqlen <= 0) return 0;
  return bwd_workspace_bytes((long)batch * heads_q * seqlen);
}

size_t attn_bwd_varlen_workspace_size(int total_tokens, int heads_q) {
  if (total_tokens <= 0 || heads_q <= 0) return 0;
  return bwd_workspace_bytes((long)heads_q * total_tokens);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int batch, int heads_q,
             int heads_kv, int seqlen, int head_dim, int dtype, float softmax_scale, int causal,
             int window_left, int window_right, void* workspace, size_t workspace_size,
             void* stream) {
  if (!bwd_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  Plan p = plan_dense(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), batch, heads_q,
                      heads_kv, seqlen, head_dim, dtype, softmax_scale, causal, window_left,
                      window_right, 0);
  if (p.status != ATTN_OK || p.empty) return p.status;
  const int st = check_bwd_pointers(lse, dout, dq, dk, dv);
  if (st != ATTN_OK) return st;
  const long q_slots = ((long)seqlen + xattn::BwdShape::BR - 1) / xattn::BwdShape::BR;
  const long k_slots = ((long)seqlen + xattn::BwdShape::BK - 1) / xattn::BwdShape::BK;
  return run_bwd(p, head_dim, dtype, q_slots, k_slots, heads_q, batch, dout, dq, dk, dv,
                 softmax_scale, workspace, workspace_size, stream);
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                    int heads_q, int heads_kv, int head_dim, int dtype, float softmax_scale,
                    int causal, int window_left, int window_right, void* workspace,
                    size_t workspace_size, void* stream) {
  if (!bwd_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  Plan p = plan_varlen(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), cu_seqlens,
                       num_seqs, max_seqlen, total_tokens, heads_q, heads_kv, head_dim, dtype,
                       softmax_scale, causal, window_left, window_right, 0);
  if (p.status != ATTN_OK || p.empty) return p.status;
  const int st = check_bwd_pointers(lse, dout, dq, dk, dv);
  if (st != ATTN_OK) return st;
  return run_bwd(p, head_dim, dtype,
                 varlen_slots(xattn::BwdShape::BR, num_seqs, max_seqlen, total_tokens),
                 varlen_slots(xattn::BwdShape::BK, num_seqs, max_seqlen, total_tokens), heads_q,
                 1, dout, dq, dk, dv, softmax_scale, workspace, workspace_size, stream);
}

int attn_device_info(int device, int* num_cus, int* clock_khz) {
  if (!num_cus || !clock_khz) return ATTN_ERR_INVALID_ARG;
  int cus = 0, clk = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, device);
  if (e != hipSuccess) return hip_status(e);
  *num_cus = cus;
  *clock_khz = clk;
  return ATTN_OK;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED_HEAD_DIM:
      return "ATTN_ERR_UNSUPPORTED_HEAD_DIM: head_dim must be 64, 128, 256 or 512 (backward: "
             "64 or 128; FP8: 64, 128 or 256)";
    case ATTN_ERR_UNSUPPORTED_DTYPE:
      return "ATTN_ERR_UNSUPPORTED_DTYPE: dtype must be ATTN_DTYPE_FP16 or ATTN_DTYPE_BF16";
    case ATTN_ERR_MISALIGNED:
      return "ATTN_ERR_MISALIGNED: q/k/v/o need 16-byte, lse/cu_seqlens 4-byte alignment";
    case ATTN_ERR_TOO_LARGE: return "ATTN_ERR_TOO_LARGE: problem exceeds index limits";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error at launch";
    case ATTN_ERR_SCRATCH_LIMIT:
      return "ATTN_ERR_SCRATCH_LIMIT: the split partials exceed the 64 MiB static scratch of "
             "attn_fwd_splitkv_noalloc (use attn_fwd_splitkv with a workspace, or fewer splits)";
    default: return "unknown status";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
