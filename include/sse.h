/*
 * sse.h -- C ABI of the MI355X (gfx950) Sparse State Expansion library.
 *
 * The operation is the SSE linear-attention layer of the web page "Scaling
 * Linear Attention with Sparse State Expansion: 中文研读笔记" (study notes on
 * arXiv 2507.16577v2).  Per token t and head h:
 *
 *   e_t     = softmax over N partitions of router_logits[t,h,:]   (§2.3, eq. 9)
 *   T_t     = the topk partitions with the largest logits           (§2.3, eq. 10)
 *             (descending; equal logits -> lower index first)
 *   kappa_t = softmax over the c rows of key_logits[t,h,:]          (§2.3, eq. 11)
 *   alpha_t = exp(log_alpha[t,h,:]), one decay per state row        (§2.1, eq. 6)
 *   S^i     = diag(alpha_t) S^i + e^i kappa_t^T v_t   for i in T_t   (§2.3, eq. 12)
 *   S^i     unchanged (no decay, no write)            for i not in T_t
 *   S^sh    = diag(alpha_t) S^sh + kappa_t^T v_t   (always-active shared
 *             partition, weight 1, same q/k/alpha; §2.5)
 *   o_t     = sum_{i in T_t} e^i q_t S^i + q_t S^sh    (read after the write;
 *             §2.3 eqs. 13-14, §2.6 gated sum back to the token)
 *
 * e is not renormalised over T_t (§2.3).  No query scale is applied.
 *
 * Conventions for every entry point
 *   - Device pointers unless stated otherwise; buffers are dense, row-major,
 *     in the layouts given.  The caller owns every buffer; the library never
 *     allocates or frees memory and never synchronises the stream (debug
 *     mode, below, does).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All
 *     work is enqueued on it asynchronously.
 *   - `dtype` selects the storage type of the five token inputs:
 *     SSE_F32 (float) or SSE_BF16 (bfloat16, 2-byte bit patterns).  States,
 *     outputs and all accumulation are fp32.
 *   - Supported sizes: c, d in {32, 64, 128}; 1 <= topk <= N <= 64,
 *     topk <= 8; 1 <= H <= 256.
 *   - Argument checks run on the host before any launch.  They return
 *     SSE_ERR_INVALID_ARG (null pointer, negative or inconsistent size),
 *     SSE_ERR_UNSUPPORTED (size outside the supported set) or
 *     SSE_ERR_WORKSPACE (workspace too small); nothing is launched then.
 *     A failed launch returns SSE_ERR_HIP.  No C++ exception crosses this
 *     interface.
 *   - Preconditions the library does not check (documented, not detected):
 *     cu_seqlens is non-decreasing with cu_seqlens[0] == 0 and
 *     cu_seqlens[num_seqs] == total_tokens; every length <= max_seqlen;
 *     inputs are finite; log_alpha <= 0 and, for bf16 inputs, the sum of
 *     log_alpha over any 64 consecutive records of one partition stays above
 *     -80 (the chunked factorisation multiplies by exp of minus the in-chunk
 *     sum in fp32; fp32 inputs are computed in fp64, where the sum over any 16
 *     consecutive records only has to stay above -700).
 *     The token inputs (q, key_logits, v, log_alpha, router_logits), the
 *     states, o, the gradients and the workspace start at 16-byte-aligned
 *     addresses (device allocators give 256): their rows are read and
 *     written in 16-byte pieces.
 */
#ifndef SSE_H
#define SSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSE_OK = 0,
    SSE_ERR_INVALID_ARG = 1,
    SSE_ERR_UNSUPPORTED = 2,
    SSE_ERR_WORKSPACE = 3,
    SSE_ERR_HIP = 4
} sse_status;

typedef enum { SSE_F32 = 0, SSE_BF16 = 1 } sse_dtype;

/* Parallel schedules of the forward (§2.6): varlen gathers each partition's
 * records into its own segment (one chunked pass over about k L records);
 * masked runs every partition over every token of the sequence with the
 * tokens outside its sets masked (no decay, no write, no read). */
typedef enum { SSE_SCHEDULE_VARLEN = 0, SSE_SCHEDULE_MASKED = 1 } sse_schedule;

/* Static, human-readable name of a status code (never NULL). */
const char *sse_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int sse_version(void);

/*
 * Bytes of device workspace sse_forward needs for these sizes (0 if the
 * sizes are invalid).  The workspace holds the router choice, the grouping
 * arrays and the segment bookkeeping; it may be reused across calls on the
 * same stream.
 */
size_t sse_forward_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                   int c, int d, int N, int topk);

/*
 * Varlen forward (prefill) over packed sequences.
 * Defined by §2.3 eqs. (9)-(14) with the shared partition of §2.5, computed
 * with the varlen grouping of §2.6: the records of each (sequence, head,
 * partition) are gathered in time order and run through a chunked gated
 * linear attention whose per-partition clock only advances on the
 * partition's own records (identity transition elsewhere, §2.6).
 *
 *   q, key_logits, log_alpha  [total_tokens, H, c]   (dtype)
 *   v                         [total_tokens, H, d]   (dtype)
 *   router_logits             [total_tokens, H, N]   (dtype)
 *   cu_seqlens                [num_seqs + 1] int32, device; sequence s is
 *                             tokens [cu_seqlens[s], cu_seqlens[s+1]); states
 *                             restart at every sequence start
 *   max_seqlen                upper bound of every sequence length (host int)
 *   initial_states            [num_seqs, H, N+1, c, d] fp32 or NULL (zeros);
 *                             partition index N is the shared partition
 *   o                         [total_tokens, H, d] fp32 (written)
 *   final_states              [num_seqs, H, N+1, c, d] fp32 (written; a
 *                             partition that no token selects keeps its
 *                             initial state bit for bit)
 *   topk_idx, topk_w          [total_tokens, H, topk] int32 / fp32, or NULL:
 *                             the chosen partitions (descending logits) and
 *                             their router probabilities
 *   seg_offsets               [num_seqs*H*N + 1] int32 or NULL: the grouping
 *                             this call ran (§2.6 varlen regrouping; the
 *                             layout of sse_group_by_partition): segment
 *                             g = (s*H + h)*N + i holds records
 *                             [seg_offsets[g], seg_offsets[g+1])
 *   seg_tok, seg_slot         [total_tokens*H*topk] int32 or NULL: token and
 *                             top-k rank of every record, in the order the
 *                             chunk kernels walk them (copied from the
 *                             forward's own segment records)
 *   workspace                 device buffer of workspace_bytes >=
 *                             sse_forward_workspace_bytes(...)
 * o may not alias any input.  Each routed read (e-gated) is stored into a
 * workspace slot [total_tokens, H, topk, d]; the shared-partition pass then
 * writes o = shared read + the topk slots of the token.  No atomics: o is the
 * same, bit for bit, on every run.
 */
int sse_forward(const void *q, const void *key_logits, const void *v, const void *log_alpha,
                const void *router_logits, int dtype, const int32_t *cu_seqlens, int num_seqs,
                int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                const float *initial_states, float *o, float *final_states, int32_t *topk_idx,
                float *topk_w, int32_t *seg_offsets, int32_t *seg_tok, int32_t *seg_slot,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * General forward: sse_forward plus the options the page describes beside
 * the default layer.  Each optional pointer may be NULL (the default):
 *   q_shared, key_logits_shared  [total_tokens, H, c] (dtype): the shared
 *             partition's own query and key logits (§2.5: it has rank-64
 *             LoRA projections of its own Q and K; the projected rows are
 *             passed here).  NULL -> q / key_logits.
 *   read_router_logits [total_tokens, H, N] (dtype): logits of the read set
 *             (§2.3: the read and write sets may differ, the same by
 *             default).  The read set is the read_topk largest read logits
 *             (same order and tie rule), read weights their softmax over N;
 *             the write set and its weights come from router_logits.  A
 *             partition read but not written at a token is read from its
 *             unchanged state.  Supported on the masked schedule only
 *             (SSE_ERR_UNSUPPORTED with varlen).  1 <= read_topk <= N, <= 8.
 *   schedule  SSE_SCHEDULE_VARLEN or SSE_SCHEDULE_MASKED (same results up
 *             to rounding order).  seg_* outputs must be NULL with masked.
 *   read_topk_idx [total_tokens, H, read_topk] int32 or NULL: the read set
 *             (only with read_router_logits).
 * o = sum over the read set of e_r q S + q_shared S_shared.  The workspace
 * is sse_forward_ex_workspace_bytes(..., read_topk or 0).
 */
size_t sse_forward_ex_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                      int c, int d, int N, int topk, int read_topk);
int sse_forward_ex(const void *q, const void *key_logits, const void *v, const void *log_alpha,
                   const void *router_logits, int dtype, const int32_t *cu_seqlens, int num_seqs,
                   int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                   const void *q_shared, const void *key_logits_shared,
                   const void *read_router_logits, int read_topk, int schedule,
                   const float *initial_states, float *o, float *final_states,
                   int32_t *topk_idx, float *topk_w, int32_t *read_topk_idx,
                   int32_t *seg_offsets, int32_t *seg_tok, int32_t *seg_slot, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * sse_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, with the workspace taken from a static
 * device array of the library (sse_forward_noalloc_max_bytes() bytes, 64 MiB,
 * one copy per device, held until the process ends) instead of a caller
 * buffer.  The caller still owns every input and output.  Sizes whose
 * workspace (sse_forward_workspace_bytes) exceeds that limit return
 * SSE_ERR_WORKSPACE before any HIP call.  No memory is allocated or freed;
 * the first call on a device looks up that device's array address
 * (SSE_ERR_HIP if the lookup fails).  Every call on one device shares that
 * array: calls that overlap in time on one device (concurrent streams or
 * host threads) race and must be serialised by the caller.  Nothing in the
 * array needs to start at zero (every pass writes what it later reads).
 * No grouping debug outputs.
 */
size_t sse_forward_noalloc_max_bytes(void);
int sse_forward_noalloc(const void *q, const void *key_logits, const void *v,
                        const void *log_alpha, const void *router_logits, int dtype,
                        const int32_t *cu_seqlens, int num_seqs, int max_seqlen,
                        int64_t total_tokens, int H, int c, int d, int N, int topk,
                        const float *initial_states, float *o, float *final_states,
                        int32_t *topk_idx, float *topk_w, void *stream);

/*
 * One decode step (§2.6: decoding recurs only on the selected states).
 * B independent sequences, one new token each, for every head.
 *   q, key_logits, log_alpha  [B, H, c]   (dtype)
 *   v                         [B, H, d]   (dtype)
 *   router_logits             [B, H, N]   (dtype)
 *   states                    [B, H, N+1, c, d] fp32, updated in place; the
 *                             N - topk unselected routed states of every
 *                             (b, h) are neither read nor written
 *   o                         [B, H, d] fp32 (written)
 *   topk_idx                  [B, H, topk] int32 or NULL
 * Needs no workspace.  Deterministic: the same inputs give the same bits.
 */
int sse_decode_step(const void *q, const void *key_logits, const void *v, const void *log_alpha,
                    const void *router_logits, int dtype, int B, int H, int c, int d, int N,
                    int topk, float *states, float *o, int32_t *topk_idx, void *stream);

/*
 * General decode step: sse_decode_step with the options of sse_forward_ex
 * (§2.5 the shared partition's own query and key; §2.3 a read set chosen
 * apart from the write set).  Each optional pointer may be NULL:
 *   q_shared, key_logits_shared [B, H, c] (dtype): NULL -> q / key_logits
 *   read_router_logits          [B, H, N] (dtype): the read set is its
 *             read_topk largest entries (descending, equal logits -> lower
 *             index), read weights their softmax over N; NULL -> the write
 *             set and weights (read_topk is then ignored)
 *   read_topk_idx               [B, H, read_topk] int32 or NULL
 * The write set's states are updated (eq. 12); each read partition is read
 * after the writes (a partition read but not written keeps its state and is
 * not stored); o = sum over the read set of e_r q S + q_shared S_shared.
 * States that are neither written nor read are not touched.  No workspace;
 * deterministic.  1 <= read_topk <= N, <= 8 when read_router_logits is set.
 */
int sse_decode_step_ex(const void *q, const void *key_logits, const void *v,
                       const void *log_alpha, const void *router_logits, int dtype, int B, int H,
                       int c, int d, int N, int topk, const void *q_shared,
                       const void *key_logits_shared, const void *read_router_logits,
                       int read_topk, float *states, float *o, int32_t *topk_idx,
                       int32_t *read_topk_idx, void *stream);

/*
 * Stage entry point: the router alone (§2.3 eqs. 9-10) for `rows` rows of
 * N logits (rows = tokens x heads).
 *   router_logits [rows, N] (dtype) -> topk_idx [rows, topk] int32,
 *   topk_w [rows, topk] fp32 (router probability of each chosen partition).
 * Deterministic.  The forward pass selects with the same per-row routine
 * (same top-k order and weights) inside its fused routing kernel.
 */
int sse_router_topk(const void *router_logits, int dtype, int64_t rows, int N, int topk,
                    int32_t *topk_idx, float *topk_w, void *stream);

/* Bytes of workspace sse_group_by_partition needs (0 if sizes are invalid). */
size_t sse_group_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H, int N,
                                 int topk);

/*
 * Stage entry point: the varlen grouping of §2.6.  Records (token, slot) of
 * every (sequence s, head h, partition i) segment, segment id
 * g = (s*H + h)*N + i, are laid out in id order, time order inside a
 * segment (a stable counting sort).
 *   topk_idx    [total_tokens, H, topk] int32 (partition of each choice)
 *   topk_w      [total_tokens, H, topk] fp32 or NULL
 *   seg_offsets [num_seqs*H*N + 1] int32: segment g is
 *               records [seg_offsets[g], seg_offsets[g+1])
 *   seg_tok     [total_tokens*H*topk] int32: global token index of a record
 *   seg_slot    [total_tokens*H*topk] int32 or NULL: the record's rank j in
 *               its token's top-k list
 *   seg_w       [total_tokens*H*topk] fp32 or NULL (requires topk_w): the
 *               record's router probability
 * Deterministic.  The forward pass groups with its own kernels (ballot
 * ranks fused into its routing kernel, then the same scan); its result is
 * observable through the seg_offsets / seg_tok / seg_slot outputs of
 * sse_forward and has this same layout and order.
 */
int sse_group_by_partition(const int32_t *topk_idx, const float *topk_w,
                           const int32_t *cu_seqlens, int num_seqs, int max_seqlen,
                           int64_t total_tokens, int H, int N, int topk, int32_t *seg_offsets,
                           int32_t *seg_tok, int32_t *seg_slot, float *seg_w, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Backward of sse_forward (the default layer: varlen grouping, shared
 * partition with the routed q/k, read set = write set).  Gradients of the
 * scalar L = <d_o, o> + <d_final_states, final_states> with respect to the
 * five token inputs and the initial states, through both gates (§2.3: the
 * same router probability e gates the write and the read, so the router
 * logits get a continuous gradient through e = softmax(router_logits); the
 * discrete top-k choice itself carries none) and the key softmax.  The
 * routing and grouping are recomputed from the inputs (the same top-k
 * choice as the forward).  Over the same (sequence, head, partition)
 * segments, in chunks of 32 records: a forward sweep stores every chunk's
 * starting state and a reverse sweep every chunk's state gradient in the
 * workspace, then all chunks' gradients are computed in parallel from them.
 * Accumulation in fp32.  With fp32 inputs every product runs on fp32 MFMA;
 * with bf16 inputs on bf16 MFMA, each fp32 operand in two bf16 terms (about
 * 2^-16 relative; the bf16 inputs themselves are exact).  The chunked
 * factorisation needs the sum of log_alpha over any 32 consecutive records
 * of one partition to stay above -80, for either input type.
 *   inputs as sse_forward; initial_states [num_seqs, H, N+1, c, d] or NULL
 *   d_o                   [total_tokens, H, d] fp32
 *   d_final_states        [num_seqs, H, N+1, c, d] fp32 or NULL (zeros)
 *   dq, dkey_logits, dlog_alpha [total_tokens, H, c] fp32 (written)
 *   dv                    [total_tokens, H, d] fp32 (written)
 *   drouter_logits        [total_tokens, H, N] fp32 (written)
 *   dinitial_states       [num_seqs, H, N+1, c, d] fp32 or NULL
 *   workspace >= sse_backward_workspace_bytes(...) (chunk states and state
 *   gradients, per-record gradient slots: about 8 c d (k+1) / 32 +
 *   4 (k+1)(3c + d) bytes per (token, head) plus the forward's grouping
 *   arrays).
 * Deterministic: per-record gradients go to slots summed in a fixed order.
 */
size_t sse_backward_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                    int c, int d, int N, int topk);
int sse_backward(const void *q, const void *key_logits, const void *v, const void *log_alpha,
                 const void *router_logits, int dtype, const int32_t *cu_seqlens, int num_seqs,
                 int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                 const float *initial_states, const float *d_o, const float *d_final_states,
                 float *dq, float *dkey_logits, float *dv, float *dlog_alpha,
                 float *drouter_logits, float *dinitial_states, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * Row-sparse top-k key variant (§2.2, eqs. (7)-(8)): one state per head,
 * no partitions.  Per token t and head h:
 *   kappa_t = softmax over the row_topk largest key logits (descending,
 *             equal logits -> lower row first); zero on the other rows
 *   S       = Lambda~_t S + kappa_t^T v_t,  o_t = q_t S (read after write)
 * where Lambda~_t = diag(alpha_t) on the selected rows and, with
 * identity_unselected != 0, the identity on the other rows (their memory is
 * neither written nor decayed: the no-forgetting form, which needs the
 * identity transition); with identity_unselected = 0 every row decays.
 *   q, key_logits, log_alpha  [total_tokens, H, c]; v [total_tokens, H, d]
 *   initial_states            [num_seqs, H, c, d] fp32 or NULL (zeros)
 *   o                         [total_tokens, H, d] fp32 (written)
 *   final_states              [num_seqs, H, c, d] fp32 (written)
 *   1 <= row_topk <= c; workspace >= sse_rowsparse_workspace_bytes(...).
 * Same conventions, checks and preconditions as sse_forward (the decay
 * bound applies to the masked log decay).  Deterministic.
 */
size_t sse_rowsparse_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                     int c, int d);
int sse_rowsparse_forward(const void *q, const void *key_logits, const void *v,
                          const void *log_alpha, int dtype, const int32_t *cu_seqlens,
                          int num_seqs, int max_seqlen, int64_t total_tokens, int H, int c, int d,
                          int row_topk, int identity_unselected, const float *initial_states,
                          float *o, float *final_states, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Stage tracing (profiling aid, not part of the method).  While enabled,
 * every sse_forward records HIP events on its stream around its five
 * stages: 0 = routing + per-block counts (+ key-softmax normalisers for fp32
 * inputs), 1 = states of the pieces of long shared chains (+ the key-softmax
 * normalisers for bf16 inputs), 2 = grouping scan and scatter,
 * 3 = routed partitions (store their e-gated reads into the workspace
 * slots), 4 = shared partition (writes o = shared read + slots).  When the
 * routed segments are cut into pieces (bf16 inputs, fewer (sequence, head,
 * partition) segments than 256), the grouping runs first and the states of
 * the routed pieces run with the shared pieces: stage 1 then holds both and
 * stage 2 is empty.
 * Events of the last 256 calls are kept.  Tracing assumes
 * one device per process.  The first sse_trace_enable(1) creates the HIP
 * events it records into (256 x 6 events, kept until the process ends):
 * the one place where the library itself acquires a runtime resource.
 *   sse_trace_enable(1) creates the events (first time) and starts a fresh
 *   record; sse_trace_enable(0) stops recording.
 *   sse_trace_read waits for the recorded calls to finish, writes the summed
 *   milliseconds of stages 0..n_stages-1 into ms_per_stage, the number of
 *   calls summed into *calls, and starts a fresh record.
 */
#define SSE_TRACE_STAGES 5
int sse_trace_enable(int enable);
int sse_trace_read(float *ms_per_stage, int n_stages, int64_t *calls);

/*
 * Debug mode (a development aid, not part of the method).  It is off unless
 * the environment variable SSE_DEBUG_CHECKS holds anything but "0" when the
 * library is first used, or sse_debug_checks(1) switches it on.  While it is
 * on:
 *   - every entry point that takes cu_seqlens (sse_forward, sse_forward_ex,
 *     sse_forward_noalloc, sse_backward, sse_rowsparse_forward,
 *     sse_group_by_partition) checks, before any launch, the precondition
 *     the kernels rely on: cu_seqlens[0] == 0, cu_seqlens never decreases,
 *     cu_seqlens[num_seqs] == total_tokens, and no sequence is longer than
 *     max_seqlen.  A violation returns SSE_ERR_INVALID_ARG and launches
 *     nothing.  The check copies cu_seqlens to the host, which synchronises
 *     the stream.
 *   - every entry point synchronises its stream before returning, so a
 *     kernel that failed is reported (SSE_ERR_HIP) by the call that
 *     launched it.
 * The synchronisations make debug mode unusable under HIP graph capture.
 * sse_debug_checks(0) or (1) sets the mode, and any other value only
 * queries it.  Returns the mode in effect (0 or 1).  Results are the same
 * bits in either mode.
 */
int sse_debug_checks(int mode);

#ifdef __cplusplus
}
#endif

#endif /* SSE_H */
