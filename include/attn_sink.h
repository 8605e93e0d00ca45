/*
 * attn_sink.h -- C ABI of libattn_sink.so: attention with a learnable per-head
 * sink logit on AMD MI355X (gfx950).
 *
 * What is computed.  For query head h (KV head h / (Hq/Hkv)), query row i and
 * its visible key set V_i:
 *     s_ij  = softmax_scale * <q_i, k_j>
 *     Z_i   = exp(sink[h]) + sum_{j in V_i} exp(s_ij)
 *     O_i   = sum_{j in V_i} exp(s_ij) * v_j / Z_i
 *     LSE_i = ln Z_i
 * The sink is one learnable value per head (a tensor of shape (nheads,)),
 * added as an extra logit before the softmax; it takes part in the denominator
 * only and has no value row.  Its gradient is returned by the backward pass.
 *   -- flash-attention PR #1819 "feat: Implement Sink Attention", Description;
 *      sglang PR #8825 "feat: openai oss attention sink support with
 *      trtllm-gen backend", Summary of Changes (an additional per-head value in
 *      the softmax denominator, None when the layer has no sink, passed to
 *      both the decode and the extend path).
 * The sink is in the units of the scaled scores (it is not multiplied by
 * softmax_scale).  sink == NULL means "no sink", identical to -inf.
 *
 * Visibility.  Causal masking is bottom-right aligned: query row i of Sq sits
 * at absolute position p = Sk - Sq + i and sees keys j <= p.  An optional
 * first/last window (W1, W2) = (window_first, window_last) further keeps only
 * keys with j < W1 or j > p - W2: the first W1 tokens and the last W2 tokens
 * up to and including the current one.  For the newest token of a sequence
 * of length L this is the whole prefix when L <= W1 + W2, and otherwise
 * tokens [0, W1) followed by [L - W2, L).
 *   -- sglang PR #12504 "To implement attention-sink", Motivation (first
 *      window 1024, last window 7168), Modifications and the bot's Code
 *      Review (page table = first-window slice followed by last-window slice,
 *      only when the sequence is longer than 1024 + 7168; kernel length
 *      becomes 1024 + 7168), and the maintainer's request to keep the last
 *      7168 tokens of each sequence.
 * Passing window_first = window_last = -1 disables the window.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major
 *     tensors, 16-byte aligned.  Shapes are given with each function.
 *   - The caller allocates and owns every buffer, including workspaces.  The
 *     library never synchronises: work is enqueued on `hip_stream` (a
 *     hipStream_t; NULL = the default stream).  It allocates no device memory
 *     at run time.  Its state: a thread-local error message; per device, the
 *     number of paged-decode workgroups resident at once and of chunked-prefill
 *     workgroups resident per XCD (queried from HIP on the first call that
 *     needs them, then reused); and, for
 *     attn_sink_fwd_decode_paged_noalloc only, a fixed device array per device
 *     (below).
 *   - Outputs are overwritten (never accumulated into) and must not alias
 *     inputs.  Inputs are never written.
 *   - Every argument is validated on the host BEFORE any HIP call.  On error
 *     nothing is enqueued, a status below is returned and
 *     attn_sink_last_error() describes the problem.
 *   - Values that live on the device (seqlens_k, block_table entries) are
 *     preconditions and are not validated: 0 <= block_table entries used <
 *     num_pages and 1 <= seqlens_k[b] <= max_pages_per_seq * page_size.
 *   - dtype: ATTN_SINK_BF16 (q/k/v/o/dO/dQ/dK/dV in bfloat16, all
 *     accumulation in fp32) or ATTN_SINK_F32 (fp32 everywhere; forward
 *     prefill only).  sink, lse and dsink are always fp32.
 */
#ifndef ATTN_SINK_H
#define ATTN_SINK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_SINK_ABI_VERSION 1

typedef enum {
  ATTN_SINK_OK = 0,
  ATTN_SINK_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misalignment     */
  ATTN_SINK_ERR_UNSUPPORTED = 2, /* valid but not implemented (D, dtype ...) */
  ATTN_SINK_ERR_WORKSPACE = 3,   /* workspace missing or too small           */
  ATTN_SINK_ERR_HIP = 4          /* a HIP launch error (message has details) */
} attn_sink_status;

typedef enum { ATTN_SINK_BF16 = 0, ATTN_SINK_F32 = 1 } attn_sink_dtype;

/* Version of this ABI (ATTN_SINK_ABI_VERSION of the built library). */
int attn_sink_abi_version(void);

/* Message of the last failing call on this thread ("" if none). The pointer
 * stays valid until the next call on this thread. */
const char* attn_sink_last_error(void);

/*
 * Forward prefill / extend with Sq queries against Sk keys per sequence.
 *   q     [B, Sq, Hq, D]         (dtype)
 *   k, v  [B, Sk, Hkv, D]        (dtype)
 *   sink  [Hq] fp32, or NULL for no sink
 *   o     [B, Sq, Hq, D]         (dtype)            -- output
 *   lse   [B, Hq, Sq] fp32 natural log, sink included, or NULL -- output
 * Requirements: B, Sq, Hq, Hkv >= 1; Sk >= 0; Hq % Hkv == 0; D in {64, 128};
 * softmax_scale finite and > 0; a window needs causal = 1, window_first >= 0
 * and window_last >= 1.  A row that sees no key gets O = 0 and LSE = sink
 * (or -inf without a sink).  Size limits (ATTN_SINK_ERR_UNSUPPORTED past
 * them): B <= 65535, B*Sq*Hq and B*Sk*Hkv < 2^31, and for bf16 one batch's K
 * (or V) slice Sk*Hkv*D*2 bytes <= 4 GiB - 1.
 */
int attn_sink_fwd_prefill(const void* q, const void* k, const void* v, const float* sink,
                          void* o, float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                          float softmax_scale, int causal, int window_first, int window_last,
                          int dtype, void* hip_stream);

/*
 * Chunked prefill (extend) against a paged KV cache.  Sequence b's nq_b new
 * query tokens are rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q; they are
 * the last nq_b of its L_b = seqlens_k[b] tokens, whose K/V (theirs included)
 * are already in the cache.  Row i of sequence b sits at position
 * L_b - nq_b + i and sees key j iff j <= that position and, with a window,
 * j < window_first or j > position - window_last (flash-attention PR #1819,
 * Description: the variable-length functions take the sink; sglang PR #8825,
 * Summary of Changes: so does the extend path).
 *   q            [total_q, Hq, D] bf16, packed
 *   k_cache,
 *   v_cache      [num_pages, page_size, Hkv, D] bf16
 *   block_table  [B, max_pages_per_seq] int32, as for the paged decode
 *   cu_seqlens_q [B+1] int32 device: 0 = cu[0] <= cu[1] <= ... <= cu[B] = total_q
 *   seqlens_k    [B] int32 device, L_b (at most max_pages_per_seq * page_size)
 *   sink         [Hq] fp32 or NULL
 *   o            [total_q, Hq, D] bf16                -- output
 *   lse          [Hq, total_q] fp32 or NULL           -- output
 *   max_seqlen_q host-side upper bound of every nq_b
 * Rows placed before the context (position < 0, when nq_b > L_b) see no key:
 * O = 0 and LSE = sink (or -inf).  Requirements: D in {64, 128}; page_size a
 * power of two in [1, 256]; Hq % Hkv == 0; bf16.  The device arrays are not
 * checked: cu_seqlens_q and seqlens_k must hold the stated ranges.
 */
int attn_sink_fwd_extend_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* cu_seqlens_q,
                               const int32_t* seqlens_k, const float* sink, void* o, float* lse,
                               int B, int total_q, int max_seqlen_q, int Hq, int Hkv, int D,
                               int page_size, int max_pages_per_seq, int num_pages,
                               float softmax_scale, int window_first, int window_last, int dtype,
                               void* hip_stream);

/*
 * Attention over KV index lists (chunked prefill against a paged cache).  As
 * in attn_sink_fwd_extend_paged, sequence b's nq_b new queries are rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and sit at positions
 * L_b - nq_b + i of its L_b = seqlens_k[b] cached tokens.  The rows of each
 * block of block_q consecutive queries of a sequence share one list of token
 * positions (an indexer's selection: the SGLang DSA write-up, sections layer0
 * and Other Layers, finds the selections of 128 adjacent queries largely
 * shared); row i attends to the tokens of list kv_index[cu_blocks[b] +
 * i / block_q] at or before its position, plus the sink.
 *   kv_index   [num_blocks, topk] int32 device: token positions; entries < 0
 *              or >= L_b are empty; a list names each token at most once
 *   cu_blocks  [B+1] int32 device: sequence b's lists are rows cu_blocks[b] ..
 *              cu_blocks[b] + ceil(nq_b / block_q) - 1
 *   other arguments as in attn_sink_fwd_extend_paged (lse [Hq, total_q]).
 * A row whose list holds no visible token gets O = 0 and LSE = sink (or
 * -inf).  Requirements (ATTN_SINK_ERR_UNSUPPORTED otherwise): bf16; D in {64,
 * 128}; Hq / Hkv a multiple of 4; block_q a positive multiple of 64;
 * 1 <= topk <= 2048; page_size a power of two in [1, 256].  The device arrays
 * are not checked: they must hold the stated ranges.
 */
int attn_sink_fwd_index_paged(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* cu_seqlens_q,
                              const int32_t* seqlens_k, const int32_t* kv_index,
                              const int32_t* cu_blocks, const float* sink, void* o, float* lse,
                              int B, int total_q, int max_seqlen_q, int Hq, int Hkv, int D,
                              int page_size, int max_pages_per_seq, int num_pages, int block_q,
                              int topk, float softmax_scale, int dtype, void* hip_stream);

/*
 * Attention over per-query KV index lists (an indexer's top-k selection per
 * query token: the SGLang DSA write-up, sections layer0 and Other Layers).
 * Packed query rows as in attn_sink_fwd_extend_paged (row i of sequence b at
 * position L_b - nq_b + i of its L_b = seqlens_k[b] cached tokens); packed row
 * r attends to the tokens of kv_index row r that lie in [0, L_b) and at or
 * before its position, plus the sink.
 *   kv_index   [total_q, topk] int32 device: token positions; entries < 0 or
 *              >= L_b are empty; a list names each token at most once
 *   o          [total_q, Hq, D] bf16; lse [Hq, total_q] fp32 or NULL -- outputs
 *   workspace  at least attn_sink_index_rows_workspace_bytes() bytes
 * Each row reads its own listed K/V rows (the decode path's cost per row, not
 * the shared-tile cost of attn_sink_fwd_index_paged).  A row whose list holds
 * no visible token gets O = 0 and LSE = sink (or -inf).  Requirements: bf16;
 * D in {64, 128}; Hq % Hkv == 0; topk >= 1; page_size a power of two in
 * [1, 256].  The device arrays are not checked: they must hold the stated
 * ranges.
 */
int attn_sink_fwd_index_rows_paged(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* cu_seqlens_q,
                                   const int32_t* seqlens_k, const int32_t* kv_index,
                                   const float* sink, void* o, float* lse, int B, int total_q,
                                   int Hq, int Hkv, int D, int page_size, int max_pages_per_seq,
                                   int num_pages, int topk, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, int dtype, void* hip_stream);

/* Workspace needed by attn_sink_fwd_index_rows_paged (0 on invalid arguments). */
size_t attn_sink_index_rows_workspace_bytes(int total_q, int Hq, int Hkv, int D, int topk);

/*
 * Variable-length (packed) forward.  Sequence b's queries are rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and its keys rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v; it is the prefill problem
 * on those rows alone (flash-attention PR #1819, Description: the
 * variable-length functions take the sink).  With nq_b queries and nk_b keys,
 * causal masking is bottom-right inside the sequence: row i sits at position
 * nk_b - nq_b + i and sees key j iff j <= that position and, with a window,
 * j < window_first or j > position - window_last.
 *   q            [total_q, Hq, D] bf16, packed (q and o may be NULL iff total_q == 0)
 *   k, v         [total_k, Hkv, D] bf16, packed (NULL allowed iff total_k == 0)
 *   cu_seqlens_q [B+1] int32 device: 0 = cu[0] <= ... <= cu[B] = total_q
 *   cu_seqlens_k [B+1] int32 device: 0 = cu[0] <= ... <= cu[B] = total_k
 *   sink         [Hq] fp32 or NULL
 *   o            [total_q, Hq, D] bf16                -- output
 *   lse          [Hq, total_q] fp32 or NULL           -- output
 *   max_seqlen_q host-side upper bound of every nq_b
 * A row that sees no key gets O = 0 and LSE = sink (or -inf).  Requirements:
 * D in {64, 128}; Hq % Hkv == 0; bf16; the window needs causal = 1.  Size
 * limits: total_q*Hq and total_k*Hkv < 2^31.  The device arrays are not
 * checked: they must hold the stated ranges.
 */
int attn_sink_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, const float* sink, void* o, float* lse,
                         int B, int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv,
                         int D, float softmax_scale, int causal, int window_first,
                         int window_last, int dtype, void* hip_stream);

/*
 * Forward paged decode: one new query token per sequence, whose K/V is already
 * stored in the cache and counted in seqlens_k.
 *   q            [B, Hq, D] bf16
 *   k_cache,
 *   v_cache      [num_pages, page_size, Hkv, D] bf16
 *   block_table  [B, max_pages_per_seq] int32: token t of sequence b lives in
 *                page block_table[b, t / page_size] at offset t % page_size
 *                (slot = page * page_size + t % page_size). Entries past the
 *                sequence's last selected page are never read.
 *   seqlens_k    [B] int32 device, context length L_b including the new token
 *   sink         [Hq] fp32 or NULL
 *   o            [B, Hq, D] bf16                   -- output
 *   lse          [B, Hq] fp32 or NULL              -- output
 *   num_splits   split-K parts per sequence; 0 picks the split itself: for
 *                large work (at most 256 sequences) equal token ranges of the
 *                whole batch, one per workgroup the device holds at once, else
 *                fixed-length chunks.  The result does not depend on it beyond
 *                fp32 rounding order.
 *   workspace    device scratch of at least attn_sink_decode_workspace_bytes()
 *                bytes for the same arguments; contents need no initialisation.
 * Requirements: D in {64, 128}; page_size a power of two in [1, 256];
 * Hq % Hkv == 0; max_pages_per_seq >= 1; num_pages >= 1.  Size limits
 * (ATTN_SINK_ERR_UNSUPPORTED past them): B and the number of splits <= 65535,
 * num_pages*page_size and max_pages_per_seq*page_size < 2^31.
 * With a window only the selected tokens are read from the cache.
 */
int attn_sink_fwd_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seqlens_k,
                               const float* sink, void* o, float* lse, int B, int Hq, int Hkv,
                               int D, int page_size, int max_pages_per_seq, int num_pages,
                               float softmax_scale, int window_first, int window_last,
                               int num_splits, void* workspace, size_t workspace_bytes,
                               int dtype, void* hip_stream);

/* Workspace needed by attn_sink_fwd_decode_paged with the same arguments
 * (0 on invalid arguments). */
size_t attn_sink_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int page_size,
                                        int max_pages_per_seq, int window_first,
                                        int window_last, int num_splits);

/*
 * attn_sink_fwd_decode_paged without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments, results and errors are
 * those of attn_sink_fwd_decode_paged; the split partials go to a device array
 * that the library holds, one per device (allocated when the library's code
 * is loaded on that device, held until the process ends), of
 * ATTN_SINK_DECODE_SCRATCH_BYTES bytes.  A call whose
 * attn_sink_decode_workspace_bytes() exceeds that returns
 * ATTN_SINK_ERR_UNSUPPORTED before any HIP call.  The first call on a device
 * looks the array's device address up (hipGetSymbolAddress, with that device
 * current); no call allocates or frees memory.  Every call on one device
 * shares that device's array: calls that overlap on one device (on different
 * streams, or from several threads) race and give wrong results; calls
 * ordered on one stream do not.
 */
#define ATTN_SINK_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int attn_sink_fwd_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seqlens_k,
                                       const float* sink, void* o, float* lse, int B, int Hq,
                                       int Hkv, int D, int page_size, int max_pages_per_seq,
                                       int num_pages, float softmax_scale, int window_first,
                                       int window_last, int num_splits, int dtype,
                                       void* hip_stream);

/*
 * Backward of the forward prefill (bf16).  Gradients of sum(dO * O):
 *   q, k, v, o, dout   as in the forward (o is the forward's output)
 *   lse    [B, Hq, Sq] fp32 from the forward (sink included)
 *   sink   [Hq] fp32 or NULL
 *   dq     [B, Sq, Hq, D], dk, dv [B, Sk, Hkv, D] (dtype) -- outputs
 *   dsink  [Hq] fp32, required iff sink != NULL      -- output
 * dSink_h = -sum_{b,i} exp(sink_h - LSE_i) * <dO_i, O_i>, reduced in fp32 in
 * a fixed order.
 * workspace: at least attn_sink_bwd_workspace_bytes() bytes.
 * Size limits (ATTN_SINK_ERR_UNSUPPORTED past them): B and ceil(Sk/128)
 * <= 65535, B*Sq*Hq and B*Sk*Hkv < 2^31, one batch's K/V slice
 * (Sk*Hkv*D*2 bytes) and Q/dO slice (Sq*Hq*D*2 bytes) <= 4 GiB - 1.
 */
int attn_sink_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, const float* sink, void* dq, void* dk, void* dv,
                  float* dsink, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                  float softmax_scale, int causal, int window_first, int window_last,
                  void* workspace, size_t workspace_bytes, int dtype, void* hip_stream);

/* Workspace needed by attn_sink_bwd (0 on invalid arguments). */
size_t attn_sink_bwd_workspace_bytes(int B, int Sq, int Sk, int Hq, int Hkv, int D);

/*
 * Backward of the variable-length forward (bf16): gradients of sum(dO * O)
 * for attn_sink_fwd_varlen with the same sequences, mask and scale
 * (flash-attention PR #1819, Description: the variable-length functions take
 * the sink and the backward returns its gradient).
 *   q, o, dout     [total_q, Hq, D]; k, v [total_k, Hkv, D]
 *   lse            [Hq, total_q] fp32 from the forward (sink included)
 *   cu_seqlens_q,
 *   cu_seqlens_k   [B+1] int32 device, as in the forward
 *   dq             [total_q, Hq, D], dk, dv [total_k, Hkv, D] bf16 -- outputs;
 *                  keys no query sees get dk = dv = 0
 *   dsink          [Hq] fp32, required iff sink != NULL: the sum over all
 *                  sequences' rows, reduced in fp32 in a fixed order -- output
 *   max_seqlen_q,
 *   max_seqlen_k   host-side upper bounds of every sequence's nq_b and nk_b
 * workspace: at least attn_sink_bwd_varlen_workspace_bytes() bytes.
 * Size limits (ATTN_SINK_ERR_UNSUPPORTED past them): B and
 * ceil(max_seqlen_k/128) <= 65535, total_q*Hq and total_k*Hkv < 2^31, one
 * sequence's K/V slice (max_seqlen_k*Hkv*D*2 bytes) and Q/dO slice
 * (max_seqlen_q*Hq*D*2 bytes) <= 4 GiB - 1.  The device arrays are not
 * checked: they must hold the stated ranges.
 */
int attn_sink_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, const float* sink,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq,
                         void* dk, void* dv, float* dsink, int B, int total_q, int total_k,
                         int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int D,
                         float softmax_scale, int causal, int window_first, int window_last,
                         void* workspace, size_t workspace_bytes, int dtype, void* hip_stream);

/* Workspace needed by attn_sink_bwd_varlen (0 on invalid arguments). */
size_t attn_sink_bwd_varlen_workspace_bytes(int B, int total_q, int max_seqlen_q, int Hq);

/*
 * Test / debug exports that run the same device index map as the decode
 * kernel.  Selection of sequence b: if a window is given and L_b > W1 + W2,
 * logical index u maps to token u for u < W1 and to L_b - W2 + (u - W1)
 * otherwise; without a window (or L_b <= W1 + W2) token = u.
 *
 * select_slots: slots [B, max_sel] int64 -- slot of the u-th selected token,
 *               -1 past the sequence's selection; counts [B] int32 = number
 *               of selected tokens (may exceed max_sel; only max_sel written).
 */
int attn_sink_decode_select_slots(const int32_t* block_table, const int32_t* seqlens_k, int B,
                                  int max_pages_per_seq, int page_size, int window_first,
                                  int window_last, int64_t* slots, int32_t* counts, int max_sel,
                                  void* hip_stream);

/* gather_kv: k_out, v_out [B, max_sel, Hkv, D] (dtype) -- rows of the selected
 * slots in selection order; rows past the selection are zero-filled. */
int attn_sink_gather_kv(const void* k_cache, const void* v_cache, const int32_t* block_table,
                        const int32_t* seqlens_k, int B, int Hkv, int D, int page_size,
                        int max_pages_per_seq, int window_first, int window_last, void* k_out,
                        void* v_out, int max_sel, int dtype, void* hip_stream);

/*
 * Device-side preconditions.  The values that live on the device -- seqlens_k
 * (decode: in [1, max_pages_per_seq * page_size]; extend and index lists: in
 * [0, that]), the block-table entries a call reads (in [0, num_pages)) and the
 * cumulative offsets cu_seqlens_q / cu_seqlens_k (0 = cu[0] <= ... <= cu[B] =
 * the total, no length above its stated maximum) -- are not checked by the
 * release library.  The debug build, libattn_sink_debug.so (the same sources
 * compiled with ATTN_SINK_DEVICE_CHECKS), checks them on the device ahead of
 * each paged or packed launch and ORs the violations into an error word; its
 * kernels then return without reading through the bad values (their outputs
 * are left unwritten).
 */
#define ATTN_SINK_CHECK_SEQLEN 1u     /* a sequence length out of range          */
#define ATTN_SINK_CHECK_PAGE 2u       /* a block-table entry read out of range   */
#define ATTN_SINK_CHECK_CU_SEQLENS 4u /* cumulative offsets not well formed      */

/* Debug build: waits for `hip_stream`, then stores in *flags the violations
 * recorded so far (ATTN_SINK_CHECK_* bits) and clears them when `clear` != 0.
 * This call synchronises.  The release library returns ATTN_SINK_ERR_UNSUPPORTED
 * and stores 0. */
int attn_sink_device_check_flags(unsigned* flags, int clear, void* hip_stream);

/* The same checks on HOST arrays (any build, no HIP call): block_table [B,
 * max_pages_per_seq], seqlens_k [B], cu_seqlens_q [B+1] or NULL (with total_q
 * and max_seqlen_q).  decode != 0 checks what the paged decode reads (lengths
 * >= 1, the pages of the selected tokens only); decode == 0 what the extend
 * and index-list paths read (lengths >= 0, every page of [0, L)).  *flags
 * receives the ATTN_SINK_CHECK_* bits of every violation. */
int attn_sink_check_paged_inputs(const int32_t* block_table, const int32_t* seqlens_k,
                                 const int32_t* cu_seqlens_q, int B, int total_q,
                                 int max_seqlen_q, int max_pages_per_seq, int page_size,
                                 int num_pages, int window_first, int window_last, int decode,
                                 unsigned* flags);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SINK_H */
