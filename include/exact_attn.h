/*
 * exact_attn.h - C ABI of the MI355X (gfx950) exact-attention library (forward, and the
 * backward at the end of this file).
 *
 * The library computes the FlashAttention-2 forward pass (page "flash_attn_mma_tiling_qk.cu",
 * header comment and kernel: each block takes a tile of Q rows, streams every K/V tile of the
 * sequence, keeps a running row max and row sum, rescales the O accumulator and normalises O at
 * the end).  The result is the plain softmax(scale * Q K^T + mask) V, plus the per-row
 * log-sum-exp of the scaled, masked scores.
 *
 * Conventions shared by both entry points
 *   - q, k, v, o hold fp16 or bf16 values, contiguous, head_dim fastest.  They are DEVICE
 *     pointers owned by the caller and must be 16-byte aligned.  o must not alias q, k or v.
 *   - lse, if not NULL, is a DEVICE fp32 array owned by the caller (4-byte aligned).  It
 *     receives the NATURAL-log log-sum-exp of each row; a row that sees no key gets -inf and
 *     O = 0 (page "flash_fwd_kernel.h" @26a6e0a, consumer loop: empty tiles store zeros).
 *   - softmax_scale multiplies Q K^T; it must be finite and > 0 (usually 1/sqrt(head_dim)).
 *   - Masks (page "mainloop_bwd_sm90_tma_gmma_ws.hpp", `mma`: causal masking iterations and the
 *     Is_local branch; here seqlen_q == seqlen_k): key j is visible to query i iff
 *         (causal == 0 || j <= i)
 *      && (window_left  < 0 || j >= i - window_left)
 *      && (window_right < 0 || j <= i + window_right).
 *     causal must be 0 or 1; window_left/window_right are >= 0, or -1 for unbounded.
 *     causal = 1 is the window mask with window_right = 0.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls are asynchronous: they only
 *     enqueue kernels.  The library allocates no memory and keeps no state except the
 *     calling thread's last HIP error code, so concurrent calls from several threads are
 *     safe.
 *   - Errors are returned, never thrown or printed; nothing is launched when the arguments
 *     fail validation.  Arguments are validated on the host; of the device arrays, cu_seqlens
 *     entries are clamped into [0, total_tokens] and a sequence longer than max_seqlen gets
 *     NaN rows (see attn_fwd_varlen).
 *   - ATTN_ERR_HIP is the status of the kernel launch itself (hipLaunchKernel); an error left
 *     on the thread by the caller's earlier HIP calls is neither returned nor cleared.
 *   - Supported head_dim: 64, 128, 256, 512.  Supported dtype: ATTN_DTYPE_FP16,
 *     ATTN_DTYPE_BF16.  Any sequence length is accepted (no tile-multiple requirement) up to
 *     seqlen * head_dim * 2 < 2^31 bytes per (sequence, head) (ATTN_ERR_TOO_LARGE beyond).
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
enum {
  ATTN_DTYPE_FP16 = 0,
  ATTN_DTYPE_BF16 = 1
};

/* Status codes returned by every entry point. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,          /* null pointer, bad size, scale or mask argument      */
  ATTN_ERR_UNSUPPORTED_HEAD_DIM = 2, /* head_dim not supported by the call (see each call)  */
  ATTN_ERR_UNSUPPORTED_DTYPE = 3,    /* dtype not fp16 / bf16                               */
  ATTN_ERR_MISALIGNED = 4,           /* q/k/v/o not 16-byte or lse/cu_seqlens not 4-byte    */
  ATTN_ERR_TOO_LARGE = 5,            /* a size would overflow the kernel's index arithmetic */
  ATTN_ERR_HIP = 6,                  /* the HIP runtime reported an error at launch         */
  ATTN_ERR_SCRATCH_LIMIT = 7         /* attn_fwd_splitkv_noalloc: partials exceed its scratch */
};

/*
 * attn_fwd - dense batch.
 *   q, k, v, o : [batch, heads, seqlen, head_dim]
 *   lse        : [batch, heads, seqlen] fp32, or NULL
 * batch, heads, seqlen >= 0 (a zero size is a no-op that returns ATTN_OK).
 * Defined by page "flash_attn_mma_tiling_qk.cu" (problem statement: Q, K, V, O are
 * [B, H, N, d]) with the masks and LSE described above.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int batch, int heads, int seqlen, int head_dim, int dtype,
             float softmax_scale, int causal, int window_left, int window_right,
             void* stream);

/*
 * attn_fwd_varlen - packed batch of variable-length sequences (self-attention).
 *   q, k, v, o : [heads, total_tokens, head_dim]
 *   lse        : [heads, total_tokens] fp32, or NULL
 *   cu_seqlens : DEVICE int32 array of num_seqs + 1 prefix sums; cu_seqlens[0] = 0,
 *                nondecreasing, cu_seqlens[num_seqs] = total_tokens.  Sequence s owns tokens
 *                [cu_seqlens[s], cu_seqlens[s+1]) and attends only within itself (page
 *                "mainloop_bwd_sm90_tma_gmma_ws.hpp", get_seqlen_q/k: a sequence's length is
 *                the difference of consecutive cu_seqlens entries).  Zero-length sequences
 *                are allowed.
 *   max_seqlen : host upper bound on every sequence length (>= 1 when total_tokens > 0); it
 *                only sizes the launch, so no device-to-host copy is needed.  A sequence
 *                longer than max_seqlen is an error the host cannot see: it is not computed
 *                and none of its K/V rows are read; instead every row of it in o and lse
 *                (every call that takes max_seqlen: dq/dk/dv in the backward, the partial
 *                and merged rows in split-KV) is filled with NaN, and the other sequences are
 *                computed as usual.
 * num_seqs, total_tokens >= 0 (zero is a no-op).  Masks apply per sequence, as above.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                    int heads, int head_dim, int dtype, float softmax_scale,
                    int causal, int window_left, int window_right, void* stream);

/*
 * Grouped-query variants (GQA; MQA when heads_kv = 1): q, o and lse have heads_q heads, k and
 * v have heads_kv heads, heads_kv >= 1 divides heads_q, and query head h attends with key /
 * value head h / (heads_q / heads_kv) (page "mainloop_bwd_sm90_tma_gmma_ws.hpp", the
 * qhead_per_khead division: a query head's key/value head is its index divided by the number
 * of query heads per key/value head).
 *   attn_fwd_gqa        : q, o [batch, heads_q, seqlen, head_dim];
 *                         k, v [batch, heads_kv, seqlen, head_dim]; lse [batch, heads_q, seqlen]
 *   attn_fwd_varlen_gqa : q, o [heads_q, total_tokens, head_dim];
 *                         k, v [heads_kv, total_tokens, head_dim]; lse [heads_q, total_tokens]
 * A heads_kv that is < 1 or does not divide heads_q gives ATTN_ERR_INVALID_ARG.  Everything
 * else is as for attn_fwd / attn_fwd_varlen, which are the heads_kv = heads_q case.
 */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 int batch, int heads_q, int heads_kv, int seqlen, int head_dim, int dtype,
                 float softmax_scale, int causal, int window_left, int window_right,
                 void* stream);

int attn_fwd_varlen_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                        int total_tokens, int heads_q, int heads_kv, int head_dim, int dtype,
                        float softmax_scale, int causal, int window_left, int window_right,
                        void* stream);

/*
 * Persistent-schedule variants of attn_fwd_gqa / attn_fwd_varlen_gqa for head_dim 128 (any
 * other head dim gives ATTN_ERR_UNSUPPORTED_HEAD_DIM).  The grid holds one workgroup per
 * compute unit; each takes a fixed list of 256-row q-tiles and sweeps their key tiles as one
 * continuous pipeline (the persistent tile scheduler of page "flash_fwd_kernel.h" @26a6e0a,
 * get_initial_work / get_next_work, with the list fixed at launch).  Arguments, layouts,
 * results and errors are those of attn_fwd_gqa / attn_fwd_varlen_gqa; outputs agree with
 * theirs up to rounding (the same arithmetic per q-tile, in a different tile order).  The
 * default entry points use the hardware's own dispatch of one workgroup per q-tile, which
 * balances uneven tiles as well or better on MI355X; these are for callers that want the
 * fixed schedule (a bounded number of resident workgroups).
 */
int attn_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse,
                        int batch, int heads_q, int heads_kv, int seqlen, int head_dim,
                        int dtype, float softmax_scale, int causal, int window_left,
                        int window_right, void* stream);

int attn_fwd_varlen_persistent(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                               int total_tokens, int heads_q, int heads_kv, int head_dim,
                               int dtype, float softmax_scale, int causal, int window_left,
                               int window_right, void* stream);

/*
 * Split-KV variants, for problems whose plain grid cannot fill the GPU (few heads and q-tiles
 * over long sequences).  The key tiles that every q-tile sees are shared out among num_splits
 * work items; each writes a normalised fp32 partial output O_s and the natural-log LSE_s of
 * the scores it saw into a caller-provided workspace, and a second kernel merges them:
 *     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * The result is the same function as attn_fwd / attn_fwd_varlen, up to rounding (page
 * "flash_fwd_kernel.h" @c272619: split-KV work items, n_split_idx; the merge is the
 * log-sum-exp identity written out).
 *   num_splits     : 1..64, or 0 to let the library choose (see
 *                    attn_fwd_splitkv_num_splits).  A count of 1 (chosen
 *                    or given) runs the plain kernels and leaves the workspace untouched (it
 *                    may then be NULL).
 *   workspace      : DEVICE memory owned by the caller, 256-byte aligned, of at least
 *                    workspace_size bytes, and workspace_size must be at least what the
 *                    matching *_workspace_size function returns for the same arguments;
 *                    otherwise ATTN_ERR_INVALID_ARG.  Its contents on entry do not
 *                    matter and on exit are unspecified; two calls in flight at once must not
 *                    share a workspace.
 *   heads, heads_kv: query heads and key/value heads, as heads_q and heads_kv of the
 *                    grouped-query variants (heads_kv = heads is plain multi-head attention).
 * All other arguments, layouts and errors are those of attn_fwd_gqa / attn_fwd_varlen_gqa.
 * The workspace depends on the query heads only.
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads, int heads_kv, int seqlen, int head_dim, int dtype,
                     float softmax_scale, int causal, int window_left, int window_right,
                     int num_splits, void* workspace, size_t workspace_size, void* stream);

int attn_fwd_varlen_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                            int total_tokens, int heads, int heads_kv, int head_dim,
                            int dtype, float softmax_scale, int causal, int window_left,
                            int window_right, int num_splits, void* workspace,
                            size_t workspace_size, void* stream);

/*
 * attn_fwd_splitkv_noalloc - attn_fwd_splitkv for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It takes
 * no workspace: the split partials live in a device array of ATTN_NOALLOC_SCRATCH_BYTES that
 * the library owns, one per GPU, held until the process ends.  The call itself makes no
 * hipMalloc, hipFree or other allocating call; the caller passes inputs and outputs.
 *   - Arguments, layouts, num_splits and results are those of attn_fwd_splitkv; outputs are
 *     bitwise equal to attn_fwd_splitkv's for the same split count.  num_splits = 0 takes
 *     the count attn_fwd_splitkv would choose, lowered to the largest whose partials fit the
 *     scratch (down to 1, the plain kernels).
 *   - ATTN_ERR_SCRATCH_LIMIT when a given num_splits needs partials (num_splits x rows x
 *     (head_dim + 1) x 4 bytes, each part 256-byte aligned; attn_fwd_splitkv_workspace_size
 *     gives the figure) beyond ATTN_NOALLOC_SCRATCH_BYTES.  Nothing is launched then.  With
 *     one split (chosen or given) the plain kernels run and the scratch is not touched.
 *   - The scratch belongs to the GPU that runs `stream` (the current device for the null
 *     stream); its address is looked up on the first call there.  Every call on one GPU uses
 *     the same scratch: two calls in flight on that GPU at once (different streams, or host
 *     threads) race on it and give wrong results.  Calls ordered on one stream are safe.
 *     Nothing in the scratch needs clearing: each call writes every entry it reads.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int batch, int heads, int heads_kv, int seqlen, int head_dim,
                             int dtype, float softmax_scale, int causal, int window_left,
                             int window_right, int num_splits, void* stream);

/* Workspace bytes the split-KV calls need for these sizes (heads = query heads) and
 * num_splits (0 = the count the library would choose; for attn_fwd_splitkv that count also
 * depends on the call's causal and window_left, which are read for num_splits = 0 only).  0
 * when no workspace is needed (one split) or the arguments are invalid.  Host-only: no device
 * is touched. */
size_t attn_fwd_splitkv_workspace_size(int batch, int heads, int seqlen, int head_dim,
                                       int num_splits, int causal, int window_left);
size_t attn_fwd_varlen_splitkv_workspace_size(int num_seqs, int max_seqlen, int total_tokens,
                                              int heads, int head_dim, int num_splits);

/* The split count num_splits = 0 selects (1 = no split): enough work items to give every CU
 * its resident share of workgroups, with at least eight key tiles per split and at most 64
 * splits.  For attn_fwd_splitkv, a causal call without a left window (window_left < 0 or
 * >= seqlen) over at most 3 (batch, head) pairs takes twice as many items: its q-tiles range
 * from one key tile to all of them, and the library deals them out to the XCDs one by one.
 * Host-only. */
int attn_fwd_splitkv_num_splits(int batch, int heads, int seqlen, int head_dim, int causal,
                                int window_left);
int attn_fwd_varlen_splitkv_num_splits(int num_seqs, int max_seqlen, int total_tokens,
                                       int heads, int head_dim);

/*
 * FP8 forward: q, k, v hold 8-bit E4M3 codes (the OCP format: 4 exponent bits with bias 7, 3
 * mantissa bits, largest finite value 448), one byte per element, in the layouts of
 * attn_fwd_gqa / attn_fwd_varlen_gqa.  Each tensor stands for code * descale, with one fp32
 * descale per tensor given as a DEVICE pointer (NULL = 1, 4-byte aligned otherwise).  The
 * result is attention of the dequantized tensors: the Q and K descales fold into the softmax
 * scale and the V descale multiplies the output (page "flash_fwd_kernel.h" @c272619,
 * `compute_attn_ws_fp8`: descale_q, descale_k, descale_v; page "flash_fwd_kernel.h" @26a6e0a:
 * a missing scale pointer means 1).  P is rounded to E4M3 for the P V product, exponentiated
 * with the pages' offset of 8 (`Max_offset`) so that it spans (0, 256].
 *   o         : bf16 or fp16 output (out_dtype = ATTN_DTYPE_BF16 / ATTN_DTYPE_FP16), laid out
 *               as q with 2-byte elements; lse as in the forward (may be NULL).
 *   head_dim  : 64, 128 or 256 (ATTN_ERR_UNSUPPORTED_HEAD_DIM otherwise).
 * Everything else (masks, heads, errors, stream) is as for attn_fwd_gqa / attn_fwd_varlen_gqa.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 const float* descale_q, const float* descale_k, const float* descale_v,
                 int batch, int heads_q, int heads_kv, int seqlen, int head_dim, int out_dtype,
                 float softmax_scale, int causal, int window_left, int window_right,
                 void* stream);

int attn_fwd_varlen_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                        const float* descale_q, const float* descale_k,
                        const float* descale_v, const int32_t* cu_seqlens, int num_seqs,
                        int max_seqlen, int total_tokens, int heads_q, int heads_kv,
                        int head_dim, int out_dtype, float softmax_scale, int causal,
                        int window_left, int window_right, void* stream);

/*
 * Backward pass: the gradients dQ, dK, dV of a loss L given dO = dL/dO, for the forward that
 * the same arguments describe (page "mainloop_bwd_sm90_tma_gmma_ws.hpp", the backward `mma`:
 * P is recomputed from the scores and the stored LSE, dP = dO V^T,
 * dS = P * (dP - dPsum) with dPsum_i = dO_i . O_i, dV = P^T dO, dK = scale * dS^T Q and
 * dQ = scale * dS K).  With grouped heads the dK, dV of a key/value head are summed over the
 * query heads of its group.
 *   q, k, v, heads, mask, scale : as for attn_fwd_gqa / attn_fwd_varlen_gqa (heads_kv =
 *                   heads_q for plain multi-head attention).
 *   o, lse        : the forward's output and its natural-log LSE for these inputs (lse is
 *                   required here; layouts as in the forward).
 *   dout          : dO, laid out as o.  dq is laid out as q; dk and dv as k and v.  All
 *                   16-byte aligned DEVICE arrays owned by the caller; dq, dk, dv are fully
 *                   overwritten and must not alias any input.
 *   workspace     : DEVICE memory owned by the caller, 256-byte aligned, of at least
 *                   attn_bwd_workspace_size / attn_bwd_varlen_workspace_size bytes (two fp32
 *                   per query row: dPsum and the LSE in log2 units, each array padded to 256
 *                   bytes); otherwise ATTN_ERR_INVALID_ARG.  Its contents on entry do not
 *                   matter; two calls in flight at once must not share it.
 *   head_dim      : 64 or 128 (ATTN_ERR_UNSUPPORTED_HEAD_DIM otherwise).
 * Two kernels run on `stream`, deterministically (no atomics).  Other errors as for the
 * forward.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int batch, int heads_q,
             int heads_kv, int seqlen, int head_dim, int dtype, float softmax_scale, int causal,
             int window_left, int window_right, void* workspace, size_t workspace_size,
             void* stream);

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                    int heads_q, int heads_kv, int head_dim, int dtype, float softmax_scale,
                    int causal, int window_left, int window_right, void* workspace,
                    size_t workspace_size, void* stream);

/* Workspace bytes of a backward call (0 for an empty problem).  Host-only. */
size_t attn_bwd_workspace_size(int batch, int heads_q, int seqlen);
size_t attn_bwd_varlen_workspace_size(int total_tokens, int heads_q);

/* Compute units and peak engine clock (kHz) of HIP device `device`, as the HIP runtime
 * reports them (host-only query, for sizing and reporting; the kernels do not depend on it).
 * ATTN_ERR_INVALID_ARG on null pointers, ATTN_ERR_HIP if the runtime query fails. */
int attn_device_info(int device, int* num_cus, int* clock_khz);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(int status);

/* The hipError_t of the last ATTN_ERR_HIP returned on this thread (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
