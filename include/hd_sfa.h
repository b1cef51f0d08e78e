/*
 * hd_sfa.h -- C ABI of the MI355X (gfx950) Stream-Factorized Attention library.
 *
 * Hidden Decoding expands every token into n streams, each drawn from its own
 * embedding table, and runs the unchanged backbone over the resulting length-nL
 * sequence.  Most attention layers read only their own stream; a few mixing
 * layers use the base model's full causal pattern over the whole sequence; the
 * KV of every stream is kept so later tokens read it as context.  Sources:
 * "Hidden Decoding at Scale" review (romaanj.github.io), section Method; the
 * arXiv 2607.08186 abstract; the Tencent/Sequential-Hidden-Decoding README,
 * section Key Idea.
 *
 * Conventions shared by every entry point
 *   - Expanded position of (token t, stream s) is p = t*n + s (token-major,
 *     stream 0 first).  Table s feeds stream s.
 *   - All tensors are dense, row-major, contiguous, and live in device memory
 *     unless a parameter says otherwise.  bf16 values are passed as their
 *     16-bit patterns (uint16_t).  Pointers to bf16 data must be 16-byte
 *     aligned.
 *   - Query head h reads KV head h / (Hq / Hkv).
 *   - Every call is asynchronous on `stream` (NULL = the null stream), keeps
 *     no state between calls, never synchronises, and allocates nothing: the
 *     caller owns every buffer and the stream.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns a non-zero hd_status and touches no memory.  Data
 *     that only the device can check (token ids, decode token counts and page
 *     ids) is reported through a device flag.  No C++ exception crosses this
 *     interface.
 *   - A call whose total work is zero (B, L or S equal to 0) returns HD_OK
 *     without launching.
 */
#ifndef HD_SFA_H
#define HD_SFA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hd_status {
    HD_OK = 0,
    HD_ERR_NULL = 1,         /* a required pointer is NULL                       */
    HD_ERR_SHAPE = 2,        /* a size is negative/zero where it must not be,
                                Hq is not a multiple of Hkv, a pointer is
                                misaligned, or a softmax scale is not finite
                                and positive                                      */
    HD_ERR_UNSUPPORTED = 3,  /* head_dim other than 64/128, or a size beyond the
                                library's 32-bit index range                     */
    HD_ERR_CAPACITY = 4,     /* KV cache too small for the appended entries      */
    HD_ERR_LAUNCH = 5,       /* the HIP runtime refused a launch                 */
    HD_ERR_WORKSPACE = 6,    /* workspace NULL, smaller than required or misaligned */
    HD_ERR_SCRATCH = 7       /* the call needs more than the library's static
                                scratch (sfa_decode_step_noalloc) holds          */
} hd_status;

/* Static, NUL-terminated description of a status code; never NULL. */
const char* hd_status_string(int status);

/* Version of this interface (incremented on any signature change). */
int hd_abi_version(void);

/*
 * hd_expand -- embedding expansion and interleave.
 * Review, section Method (every token becomes n streams, each stream with an
 * embedding table of its own, laid out as one sequence of length nL); README,
 * section Key Idea, items 1 and 2.
 *
 *   out[b, t*n + s, :] = tables[s, ids[b, t], :]   for b < B, t < L, s < n
 *
 *   ids      int32 [B, L]           token ids
 *   tables   bf16  [n, V, H]        n stacked independent tables
 *   out      bf16  [B, n*L, H]      written in full
 *   err_flag int32 scalar or NULL   if not NULL and some id lies outside
 *                                   [0, V), *err_flag is set to 1 (it is never
 *                                   cleared: the caller zeroes it first); the n
 *                                   rows of such a token are written as zeros
 * Pure copy: the result is bit-identical to the gather.  H must be a multiple
 * of 8; B*L*n (output rows) must stay below 2^31 (HD_ERR_UNSUPPORTED).
 */
hd_status hd_expand(const int32_t* ids, int64_t B, int64_t L,
                    const uint16_t* tables, int32_t n, int64_t V, int64_t H,
                    uint16_t* out, int32_t* err_flag, hipStream_t stream);

/*
 * hd_final_stream_rows -- the rows the next-token loss reads.  Review, section
 * Method: the next-token loss is taken only where each token's last stream
 * sits; the earlier n-1 streams carry no loss and serve as latent states.
 *
 *   out[b, t, :] = x[b, t*n + n-1, :]   for b < B, t < L
 *
 *   x      bf16 [B, n*L, H]   hidden states of the expanded sequence
 *   out    bf16 [B, L, H]     must not overlap x
 * Pure copy (bit-identical).  H must be a multiple of 8, x and out 16-byte
 * aligned (HD_ERR_SHAPE otherwise); B*L*H/8 must stay below 2^32
 * (HD_ERR_UNSUPPORTED).
 */
hd_status hd_final_stream_rows(const uint16_t* x, int64_t B, int32_t n, int64_t L,
                               int64_t H, uint16_t* out, hipStream_t stream);

/*
 * hd_cyclic_replicate -- Cyclic Replication Initialization.  Review, section
 * Method: the expansion factor grows 1 -> 2 -> 4 -> 8, and when it grows the
 * new embedding tables are copies of the existing ones.
 *
 *   out[s] = tables[s mod n_old]   for s < n_new
 *
 *   tables bf16 [n_old, V, H]
 *   out    bf16 [n_new, V, H]; either out == tables (growth in place: the
 *          allocation holds n_new tables, the first n_old are left as they
 *          are and only tables n_old .. n_new-1 are written) or a buffer that
 *          does not overlap tables (HD_ERR_SHAPE on partial overlap)
 * Pure copy (bit-identical).  H must be a multiple of 8, pointers 16-byte
 * aligned; V*H/8 below 2^32 and n_new <= 65535 (HD_ERR_UNSUPPORTED).
 */
hd_status hd_cyclic_replicate(const uint16_t* tables, int32_t n_old, int64_t V, int64_t H,
                              uint16_t* out, int32_t n_new, hipStream_t stream);

/*
 * sfa_stream_attn -- within-stream causal attention over the expanded
 * sequence (prefill).  Review, section Method: the majority of layers keep each
 * stream to itself, at a cost of order n*L^2.
 *
 *   O[b, p(t,s), h] = sum over t' <= t of
 *       softmax_t'( scale * q[b,p(t,s),h] . k[b,p(t',s),g] ) v[b,p(t',s),g]
 *
 *   q, out   bf16 [B, n*L, Hq, D]
 *   k, v     bf16 [B, n*L, Hkv, D]
 *   D        64 or 128; Hq a multiple of Hkv
 *   softmax_scale  finite and > 0 (HD_ERR_SHAPE otherwise), as for every
 *            attention entry point of this library
 * Scores, softmax statistics and the output accumulator are fp32; the two
 * contractions run on bf16 matrix cores; out is rounded to nearest even.
 * Work skipped: only token tiles of the query's own stream that are not in
 * its future are visited, so the cost grows linearly in n.
 * The prefill entry points run a persistent grid of one workgroup per compute
 * unit; the environment variable HD_SFA_PREFILL_WORKGROUPS (a count from 1 to
 * 65536, read at every call) sets another grid size, a testing and tuning
 * control that never changes a result bit.
 */
hd_status sfa_stream_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          uint16_t* out, int64_t B, int32_t n, int64_t L,
                          int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                          hipStream_t stream);

/*
 * sfa_mix_attn -- mixing attention, full causal pattern over the interleaved
 * length-nL order (prefill).  Review, section Method: a few layers let the
 * streams see each other with the base model's (full) pattern, so they read
 * the retained KV of the intermediate streams.
 *
 *   O[b, i, h] = sum over j <= i of softmax_j(scale * q[b,i,h] . k[b,j,g]) v[b,j,g]
 *
 * Same arguments, layouts, precision and errors as sfa_stream_attn.
 */
hd_status sfa_mix_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       uint16_t* out, int64_t B, int32_t n, int64_t L,
                       int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                       hipStream_t stream);

/*
 * sfa_mix_attn_window -- mixing attention with the sliding-window pattern
 * (prefill).  Review, section Method: the mixing layers keep whatever pattern
 * the base model used, sliding-window or full (the 80B model has 23
 * sliding-window mixing layers of 49).  The pages give no window size; here
 * the window W is counted in positions of the interleaved length-nL order
 * (a base-model window of w tokens is W = n*w):
 *
 *   O[b, i, h] = sum over i - W < j <= i of softmax_j(scale * q[b,i,h] . k[b,j,g]) v[b,j,g]
 *
 *   window   W >= 1; W >= nL gives exactly sfa_mix_attn
 *
 * Same arguments, layouts, precision and errors as sfa_stream_attn, plus
 * HD_ERR_SHAPE for window < 1.
 */
hd_status sfa_mix_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* out, int64_t B, int32_t n, int64_t L,
                              int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                              int64_t window, hipStream_t stream);

/*
 * sfa_attn_fwd -- a prefill layer's forward with its log-sum-exp (training).
 * Review, sections Method and Results: the model trains on the expanded
 * sequence, and the backward pass needs each query row's softmax statistics.
 * Same output as sfa_stream_attn (mode 0) or sfa_mix_attn (mode 1), plus
 *
 *   lse[b, h, i] = log( sum over visible j of exp(scale * q[b,i,h] . k[b,j,g]) )
 *
 *   lse   fp32 [B, Hq, n*L] (natural log), 4-byte aligned, or NULL (then the
 *         call is exactly the plain forward)
 *   mode  0 within-stream, 1 mixing (HD_ERR_SHAPE otherwise)
 * Other arguments, layouts and errors as sfa_stream_attn.
 */
hd_status sfa_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       uint16_t* out, float* lse, int64_t B, int32_t n, int64_t L,
                       int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                       int32_t mode, hipStream_t stream);

/*
 * sfa_attn_split_workspace_size -- bytes of device workspace sfa_attn_split
 * needs for these sizes (0 if no work item of the layer has two key tiles,
 * or for arguments sfa_attn_split would reject).
 */
size_t sfa_attn_split_workspace_size(int64_t B, int32_t n, int64_t L, int32_t Hq,
                                     int32_t Hkv, int32_t D, int32_t mode);

/*
 * sfa_attn_split -- sfa_attn_fwd for launches too small to fill the GPU.
 * The attention is causal, so the work items of a layer (64-query tiles x
 * packed query heads) end at different key tiles; when there are no more
 * items than compute units (a base model at n = 1 and batch 1, say), the
 * longest item sets the time.  Here each item with two or more key tiles is
 * taken as two units, its first and its second half of the key tiles, by
 * different workgroups; each unit writes its partial softmax state (running
 * max m, sum l, unnormalised O) to the workspace and the second one to finish
 * merges the two (l and O rescaled to the larger m) and writes the output
 * and lse.  It is the usual split of a softmax over key blocks; the
 * operation is the one sfa_attn_fwd defines (review, section Method: the two
 * visibility rules).  With more items than compute units the call is
 * sfa_attn_fwd itself and the workspace is not touched.
 *
 *   workspace  device memory of at least sfa_attn_split_workspace_size()
 *              bytes, 16-byte aligned, owned by the caller, zero-filled
 *              before its first use; every call leaves its counters at zero
 *              again (HD_ERR_WORKSPACE if NULL, short or misaligned when the
 *              split is taken)
 * Results: within the forward's tolerance of sfa_attn_fwd, not bitwise (the
 * merge adds the two halves' sums in another order); the same bits on every
 * call, whichever half merges.  Calls that overlap on one workspace race.
 * Other arguments, layouts and errors as sfa_attn_fwd (lse may be NULL).
 */
hd_status sfa_attn_split(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         uint16_t* out, float* lse, int64_t B, int32_t n, int64_t L,
                         int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                         int32_t mode, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * sfa_attn_bwd_workspace_size -- bytes of device workspace sfa_attn_bwd needs
 * (one fp32 per query row and head).  Returns 0 for invalid sizes.
 */
size_t sfa_attn_bwd_workspace_size(int64_t B, int32_t n, int64_t L, int32_t Hq);

/*
 * sfa_attn_bwd -- gradients of a prefill layer (within-stream or mixing)
 * with respect to q, k and v.  With P the masked softmax of scale * Q K^T
 * (the same visibility as the forward, rebuilt from lse) and dO the upstream
 * gradient:
 *
 *   dP = dO V^T,   delta_i = sum_j P_ij dP_ij,   dS = P * (dP - delta)
 *   dq = scale * dS K,   dk = scale * dS^T Q,   dv = P^T dO
 *
 * (delta equals dO_i . O_i for the exact O; it is summed from P and dP so
 * that the bf16 rounding of the forward's output does not enter.)
 *
 * dk and dv of KV head g sum the contributions of its Hq/Hkv query heads.
 *
 *   q, dout        bf16 [B, n*L, Hq, D]
 *   k, v           bf16 [B, n*L, Hkv, D]
 *   lse            fp32 [B, Hq, n*L] from sfa_attn_fwd with the same arguments
 *   dq             bf16 [B, n*L, Hq, D]   written in full
 *   dk, dv         bf16 [B, n*L, Hkv, D]  written in full
 *   workspace      device memory of at least sfa_attn_bwd_workspace_size
 *                  bytes (HD_ERR_WORKSPACE otherwise), owned by the caller,
 *                  overwritten
 *   mode           0 within-stream, 1 mixing
 * Products on bf16 matrix cores with fp32 accumulation; P and dS enter them
 * as a pair of bf16 halves (hi + lo, about 2^-17 relative), the outputs are
 * rounded to nearest even.  No atomics: the result is bitwise reproducible.  All pointers 16-byte aligned, D 64 or 128,
 * Hq a multiple of Hkv.
 */
hd_status sfa_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* dout, const float* lse,
                       uint16_t* dq, uint16_t* dk, uint16_t* dv, int64_t B, int32_t n,
                       int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                       int32_t mode, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * sfa_attn_fwd_window -- the training forward of a sliding-window mixing
 * layer: the output of sfa_mix_attn_window plus each row's log-sum-exp over
 * its window (review, section Method: 23 of the 80B model's 49 layers mix
 * streams with a sliding window, and the model trains on the expanded
 * sequence).
 *
 *   lse      fp32 [B, Hq, n*L] (natural log over i - window < j <= i),
 *            4-byte aligned, or NULL (then the call is sfa_mix_attn_window)
 *   window   >= 1 (HD_ERR_SHAPE otherwise); window >= n*L gives exactly
 *            sfa_attn_fwd in mode 1
 * Other arguments, layouts and errors as sfa_mix_attn_window.
 */
hd_status sfa_attn_fwd_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* out, float* lse, int64_t B, int32_t n, int64_t L,
                              int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                              int64_t window, hipStream_t stream);

/*
 * sfa_attn_bwd_window -- gradients of a sliding-window mixing layer: the
 * formulas of sfa_attn_bwd with P the softmax over the window
 * i - window < j <= i (rebuilt from the lse of sfa_attn_fwd_window with the
 * same window).
 *
 *   window   >= 1 (HD_ERR_SHAPE otherwise); window >= n*L gives exactly
 *            sfa_attn_bwd in mode 1
 * Other arguments (no mode), the workspace size, layouts, precision and
 * errors as sfa_attn_bwd.
 */
hd_status sfa_attn_bwd_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const uint16_t* dout, const float* lse,
                              uint16_t* dq, uint16_t* dk, uint16_t* dv, int64_t B, int32_t n,
                              int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                              int64_t window, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * sfa_decode_workspace_size -- bytes of device workspace sfa_decode_step
 * needs for these sizes (fp32 split partials).  Returns 0 for invalid sizes.
 */
size_t sfa_decode_workspace_size(int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                                 int32_t D, int64_t max_tokens);

/*
 * sfa_decode_step -- one decode step of Hidden Decoding for S sequences.
 * Review, sections Method and Limitations: every stream's KV is retained, so
 * the cache holds n entries per token and decode reads all of them; the
 * review's Notes: small-batch decode is bandwidth-bound.
 *
 * 1. Append: for each sequence q with T = tokens_before[q],
 *      k_cache[q, T*n + s] = k_new[q, s],  v_cache likewise   (s < n)
 *    (idempotent: calling twice with the same inputs writes the same bytes).
 * 2. Attention of the n new queries (T, s) of every sequence:
 *      mode 0 (within-stream): keys t'*n + s for t' <= T
 *      mode 1 (mixing):        every entry j <= T*n + s
 *
 *   q_new          bf16 [S, n, Hq, D]
 *   k_new, v_new   bf16 [S, n, Hkv, D]
 *   k_cache, v_cache bf16 [S, C_max, Hkv, D], entry order p = t*n + s
 *   tokens_before  int32 [S], device memory, 0 <= T <= max_tokens
 *                  (values outside that range are clamped into it on the
 *                  device, so no access leaves the cache, and reported
 *                  through err_flag)
 *   max_tokens     host-side bound on tokens_before, sizes the grid
 *   C_max          must be >= (max_tokens + 1) * n, else HD_ERR_CAPACITY
 *   workspace      device scratch of at least sfa_decode_workspace_size()
 *                  bytes, else HD_ERR_WORKSPACE; contents need no init
 *   out            bf16 [S, n, Hq, D]
 *   err_flag       int32 scalar in device memory, or NULL: if not NULL and
 *                  some tokens_before value lies outside [0, max_tokens],
 *                  *err_flag is set to 1 (never cleared: the caller zeroes
 *                  it first).  Such a sequence is computed with the clamped
 *                  count, so its rows are defined but not what the caller
 *                  meant; the flag is how the caller learns of it.
 * Requires n * Hq / Hkv <= 64 query rows per KV head.
 */
hd_status sfa_decode_step(const uint16_t* q_new, const uint16_t* k_new,
                          const uint16_t* v_new, uint16_t* k_cache,
                          uint16_t* v_cache, const int32_t* tokens_before,
                          int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                          int32_t D, int64_t C_max, int64_t max_tokens,
                          int32_t mode, float softmax_scale, void* workspace,
                          size_t workspace_bytes, uint16_t* out, int32_t* err_flag,
                          hipStream_t stream);

/*
 * sfa_decode_step_noalloc -- sfa_decode_step for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments (without
 * workspace and workspace_bytes), results bit for bit those of
 * sfa_decode_step, same errors, plus:
 *
 *   - the split partials live in a static array of 16 MiB per device, part
 *     of the library's code object (held by every GPU the library runs on
 *     until the process ends).  Its device address is looked up once per
 *     device, on the first call there.  The call itself allocates nothing.
 *   - a call whose partials need more than 16 MiB returns HD_ERR_SCRATCH and
 *     launches nothing.  Partials take S*Hkv*(n*Hq/Hkv)*splits*(D+2)*4 bytes
 *     when a view is split (a view is split only while there are fewer than
 *     512 (sequence, KV head) views), none otherwise.  Use sfa_decode_step
 *     with a workspace for such sizes.
 *   - every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (different streams, or host threads) race and must be
 *     serialised by the caller.  Nothing in the array needs to start at
 *     zero: each call writes every partial it reads.
 */
hd_status sfa_decode_step_noalloc(const uint16_t* q_new, const uint16_t* k_new,
                                  const uint16_t* v_new, uint16_t* k_cache,
                                  uint16_t* v_cache, const int32_t* tokens_before,
                                  int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                                  int32_t D, int64_t C_max, int64_t max_tokens,
                                  int32_t mode, float softmax_scale, uint16_t* out,
                                  int32_t* err_flag, hipStream_t stream);

/*
 * sfa_decode_step_paged -- sfa_decode_step over a paged cache (the retained
 * KV of many sequences of different lengths held in fixed-size pages, as a
 * serving engine keeps it; review, section Limitations: the enlarged per-
 * stream cache is what decode pays for).  Entry e of sequence q (e = t*n + s)
 * lives in page page_table[q, e / page_size], slot e % page_size.
 *
 *   k_pages, v_pages  bf16 [num_pages, page_size, Hkv, D] pools
 *   page_table        int32 [S, max_pages_per_seq], device memory; ids outside
 *                     [0, num_pages) are clamped into it on the device (no
 *                     access leaves the pool) and, for the pages the step
 *                     reads or writes, reported through err_flag
 *   page_size         a power of two (HD_ERR_SHAPE otherwise); the pool may
 *                     hold at most 2^32 rows (num_pages*page_size,
 *                     HD_ERR_UNSUPPORTED beyond)
 *   max_tokens        as sfa_decode_step; (max_tokens+1)*n must fit in
 *                     max_pages_per_seq*page_size entries (HD_ERR_CAPACITY)
 *   mode              0 within-stream, 1 mixing
 *   window            0 for the full pattern, or the sliding window of a
 *                     mixing layer (as sfa_decode_step_window; HD_ERR_SHAPE
 *                     with mode 0)
 * The append writes the new rows into their pages; the attention reads every
 * live row through the table.  The result equals sfa_decode_step (or
 * sfa_decode_step_window) on the same rows laid out contiguously, bit for
 * bit.  Workspace size as sfa_decode_workspace_size(S, n, Hq, Hkv, D,
 * max_tokens).  err_flag as sfa_decode_step, also set for an out-of-range
 * page id.
 */
hd_status sfa_decode_step_paged(const uint16_t* q_new, const uint16_t* k_new,
                                const uint16_t* v_new, uint16_t* k_pages, uint16_t* v_pages,
                                const int32_t* page_table, const int32_t* tokens_before,
                                int64_t S, int32_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t page_size, int64_t num_pages, int32_t max_pages_per_seq,
                                int64_t max_tokens, int32_t mode, int64_t window,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                uint16_t* out, int32_t* err_flag, hipStream_t stream);

/*
 * sfa_decode_step_window -- sfa_decode_step for a sliding-window mixing layer
 * (review, section Method: mixing layers follow the base model's pattern,
 * sliding-window or full).  After the same append, the new query (T, s) at
 * p = T*n + s attends to the entries j with p - window < j <= p (window in
 * interleaved positions, as sfa_mix_attn_window), so only the last
 * window + n - 1 entries of each sequence are read.
 *
 *   window   >= 1 (HD_ERR_SHAPE otherwise); window >= (T+1)*n gives exactly
 *            the mixing mode of sfa_decode_step
 * Every other argument, the workspace size and the errors as sfa_decode_step.
 */
hd_status sfa_decode_step_window(const uint16_t* q_new, const uint16_t* k_new,
                                 const uint16_t* v_new, uint16_t* k_cache,
                                 uint16_t* v_cache, const int32_t* tokens_before,
                                 int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                                 int32_t D, int64_t C_max, int64_t max_tokens,
                                 int64_t window, float softmax_scale, void* workspace,
                                 size_t workspace_bytes, uint16_t* out, int32_t* err_flag,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HD_SFA_H */
