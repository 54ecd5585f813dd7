// C ABI of the exact-attention forward library: argument validation, kernel selection and
// launch.  Declared in include/exact_attn.h.  Validation runs entirely on the host and before
// any HIP call, so a rejected call touches neither the device nor the stream.
#include <cmath>
#include <cstdint>
#include <limits>

#include "exact_attn.h"
#include "attn_dispatch.h"

namespace xattn {
template <> hipError_t launch_fwd<64>(const FwdArgs&, bool, int, bool, int, hipStream_t);
template <> hipError_t launch_fwd<128>(const FwdArgs&, bool, int, bool, int, hipStream_t);
template <> hipError_t launch_fwd<256>(const FwdArgs&, bool, int, bool, int, hipStream_t);
template <> hipError_t launch_fwd<512>(const FwdArgs&, bool, int, bool, int, hipStream_t);
}  // namespace xattn

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

int launch(int head_dim, const xattn::FwdArgs& a, int dtype, int mode, bool big, long n_work,
           void* stream) {
  if (n_work <= 0) return ATTN_OK;
  if (n_work > std::numeric_limits<int>::max()) return ATTN_ERR_TOO_LARGE;
  const bool bf16 = dtype == ATTN_DTYPE_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  switch (head_dim) {
    case 64: e = xattn::launch_fwd<64>(a, bf16, mode, big, (int)n_work, s); break;
    case 128: e = xattn::launch_fwd<128>(a, bf16, mode, big, (int)n_work, s); break;
    case 256: e = xattn::launch_fwd<256>(a, bf16, mode, big, (int)n_work, s); break;
    default: e = xattn::launch_fwd<512>(a, bf16, mode, big, (int)n_work, s); break;
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

constexpr float kLog2e = 1.44269504088896340736f;
constexpr long kMaxRows = 1L << 40;  // rows * head_dim stays far inside int64
// The kernels address one sequence's K/V rows with 32-bit byte offsets (buffer loads).
constexpr long kMaxSeqBytes = (1L << 31) - 1;

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
             int heads, int seqlen, int head_dim, int dtype, float softmax_scale, int causal,
             int window_left, int window_right, void* stream) {
  if (batch < 0 || heads < 0 || seqlen < 0) return ATTN_ERR_INVALID_ARG;
  const long rows = (long)batch * heads * seqlen;
  if (rows == 0) {  // empty problem: still reject malformed non-size arguments
    if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    return ATTN_OK;
  }
  int st = check_common(q, k, v, o, lse, head_dim, dtype, softmax_scale, causal, window_left,
                        window_right);
  if (st != ATTN_OK) return st;
  if (rows > kMaxRows) return ATTN_ERR_TOO_LARGE;
  if ((long)seqlen * head_dim * 2 > kMaxSeqBytes) return ATTN_ERR_TOO_LARGE;
  int wl = window_left, wr = window_right;
  const int mode = mask_mode(causal, seqlen, &wl, &wr);
  const bool big = (long)batch * heads * ((seqlen + block_rows(head_dim, true) - 1) /
                                          block_rows(head_dim, true)) >= xattn::BIG_TILE_MIN_WORK;
  const int br = block_rows(head_dim, big);
  xattn::FwdArgs a{};
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
  const long n_work = (long)batch * heads * a.tiles_per_head;
  return launch(head_dim, a, dtype, mode, big, n_work, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                    int heads, int head_dim, int dtype, float softmax_scale, int causal,
                    int window_left, int window_right, void* stream) {
  if (num_seqs < 0 || total_tokens < 0 || heads < 0 || max_seqlen < 0)
    return ATTN_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_tokens == 0 || heads == 0) {
    if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    return ATTN_OK;
  }
  int st = check_common(q, k, v, o, lse, head_dim, dtype, softmax_scale, causal, window_left,
                        window_right);
  if (st != ATTN_OK) return st;
  if (!cu_seqlens) return ATTN_ERR_INVALID_ARG;
  if (!aligned(cu_seqlens, 4)) return ATTN_ERR_MISALIGNED;
  if (max_seqlen < 1 || max_seqlen > total_tokens) return ATTN_ERR_INVALID_ARG;
  if ((long)heads * total_tokens > kMaxRows) return ATTN_ERR_TOO_LARGE;
  if ((long)max_seqlen * head_dim * 2 > kMaxSeqBytes) return ATTN_ERR_TOO_LARGE;
  int wl = window_left, wr = window_right;
  const int mode = mask_mode(causal, max_seqlen, &wl, &wr);
  const int br_big = block_rows(head_dim, true);
  const bool big = (long)heads * (((long)total_tokens + br_big - 1) / br_big) >=
                   xattn::BIG_TILE_MIN_WORK;
  const int br = block_rows(head_dim, big);
  // q-tile slots per head: an upper bound on sum_s ceil(len_s / br) that needs no lengths
  const long by_total = ((long)total_tokens + br - 1) / br + num_seqs;
  const long by_max = (long)num_seqs * ((max_seqlen + br - 1) / br);
  const long slots = by_total < by_max ? by_total : by_max;
  if (slots > std::numeric_limits<int>::max()) return ATTN_ERR_TOO_LARGE;
  xattn::FwdArgs a{};
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
  return launch(head_dim, a, dtype, mode, big, (long)heads * slots, stream);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED_HEAD_DIM:
      return "ATTN_ERR_UNSUPPORTED_HEAD_DIM: head_dim must be 64, 128, 256 or 512";
    case ATTN_ERR_UNSUPPORTED_DTYPE:
      return "ATTN_ERR_UNSUPPORTED_DTYPE: dtype must be ATTN_DTYPE_FP16 or ATTN_DTYPE_BF16";
    case ATTN_ERR_MISALIGNED:
      return "ATTN_ERR_MISALIGNED: q/k/v/o need 16-byte, lse/cu_seqlens 4-byte alignment";
    case ATTN_ERR_TOO_LARGE: return "ATTN_ERR_TOO_LARGE: problem exceeds index limits";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error at launch";
    default: return "unknown status";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
