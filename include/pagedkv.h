/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV-cache attention library
 * (libpagedkv.so).
 *
 * The operations are those the tiny-vLLM pages name for the attention part of
 * an inference engine: a KV cache kept in fixed-size pages ("blocks") that a
 * per-sequence block table maps from logical to physical blocks, attention
 * with grouped-query heads, a FlashAttention-style online softmax, decode (one
 * new query token per sequence) and causal prefill (a whole prompt).
 *   - paper-digest page "Tiny-vLLM: a high-performance LLM inference engine in
 *     C++ and CUDA", section "Core Mechanics" (KV cache, online softmax,
 *     PagedAttention, GQA, causal mask);
 *   - tiny-vllm README (Korean translation), feature list and table of
 *     contents ("Prefill vs decode", "Why KV cache exists", "Attention",
 *     "GQA", "Softmax", "Causal mask", "Online softmax", "Paged Attention",
 *     "Paged KV cache", "Paged Attention CUDA kernel");
 *   - nano-vLLM guide announcement, ch. 3 "KV Cache", ch. 4 "PagedAttention",
 *     ch. 6 "Prefill vs Decode".
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or keeps them.  `stream` is a
 *     hipStream_t passed as void* (NULL = the default stream).
 *   - Work is enqueued asynchronously on `stream`; the return value reports
 *     argument validation and the launch itself (hipGetLastError), not the
 *     completion of the kernels.
 *   - bf16 means IEEE bfloat16 bit patterns (uint16).  Indices are int32.
 *   - Pool layout (both K and V, one pool per layer):
 *         cache[num_blocks][Hkv][block_size][D]
 *     so one (block, KV head) is block_size*D*2 bytes contiguous and one
 *     token's D-vector is a 2*D = 128-byte row at D = 64.
 *   - Query head h reads KV head h / (Hq / Hkv).
 *   - context_lens[b] is the number of valid tokens of sequence b AFTER this
 *     step's append.  Logical token j of sequence b is row j % block_size of
 *     physical block block_tables[b * max_blocks_per_seq + j / block_size].
 *   - Table entries past ceil(context_lens[b] / block_size) and pool rows past
 *     the context are never read.  Physical ids outside [0, num_blocks) and
 *     contexts longer than max_blocks_per_seq * block_size are data errors:
 *     the kernels never touch memory outside the pools for them, but the
 *     result for that sequence is then undefined.
 *   - Return: PKV_OK, or a negative status; pagedkv_last_error() gives text.
 *     Validation happens on the host before any HIP call, so invalid
 *     arguments never reach the device.  B == 0 (or no new tokens) returns
 *     PKV_OK without launching anything.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the C ABI are the only ones the shared library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#define PKV_OK 0
#define PKV_ERR_INVALID_ARG (-1) /* null pointer, negative or inconsistent size */
#define PKV_ERR_UNSUPPORTED (-2) /* shape this library does not implement        */
#define PKV_ERR_WORKSPACE (-3)   /* workspace missing or too small              */
#define PKV_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed  */

#define PKV_OUT_BF16 0 /* output written as bf16, round to nearest even */
#define PKV_OUT_F32 1  /* output written as fp32                         */

/* partition_size values for paged_attention_decode besides a positive size */
#define PKV_PARTITION_NONE 0  /* one wavefront per (sequence, KV head)        */
#define PKV_PARTITION_AUTO (-1) /* split sized to the batch and the GPU      */
#define PKV_PARTITION_PLANNED (-2) /* PKV_PARTITION_AUTO from a stored plan      */

/* pagedkv_last_error -- text describing the last non-OK status returned on
 * the calling thread (thread-local; "" before any failure).
 *
 * Defined by: paper-digest page, section "Evidence" -- the community's
 * criticism that the CUDA engine ignores the status codes its runtime calls
 * return, which makes failures hard to debug.  Here every entry point
 * returns a status (PKV_OK or a negative PKV_ERR_*), HIP errors included,
 * and leaves the reason in this string.  The pointer stays valid until the
 * next failing call on the same thread; the caller must not free it.
 */
PKV_API const char *pagedkv_last_error(void);

/* pagedkv_check_tables -- validate block tables and lengths held in HOST
 * memory: the data errors the kernels do not check in release builds.
 *
 * Defined by: paper-digest page, section "Evidence" (errors that go
 * unchecked are hard to debug).  With PAGEDKV_DEBUG=1 in the environment,
 * every kernel entry point copies its tables and lengths to the host (on its
 * stream, waiting for the copy; not while the stream is being captured into
 * a graph) and runs this check before launching; a failure returns
 * PKV_ERR_INVALID_ARG and launches nothing.
 *
 * block_tables  [B][max_blocks_per_seq], context_lens [B] (host pointers).
 * cu_lens       [B+1] prefix sums of new tokens (kind PKV_CHECK_APPEND; NULL
 *               = one per sequence, T == B) or of query tokens (kind
 *               PKV_CHECK_PREFILL); ignored when NULL for PKV_CHECK_READ.
 * T             total new or query tokens (cu_lens[B]).
 * Checks: 0 <= context_lens[b] <= max_blocks_per_seq * block_size; every
 * table entry a context uses (ceil(len / block_size) of them) in
 * [0, num_blocks); prefix sums start at 0, never decrease and end at T; an
 * append's length is at least its new tokens; a prompt's cached tokens are
 * at least its query tokens.  Returns PKV_OK or PKV_ERR_INVALID_ARG naming
 * the first offending sequence in pagedkv_last_error().  Host code only.
 */
#define PKV_CHECK_READ 0    /* decode: lengths and the table entries they use */
#define PKV_CHECK_APPEND 1  /* kv_append: also new-token counts             */
#define PKV_CHECK_PREFILL 2 /* prefill: also query-token counts             */
PKV_API int pagedkv_check_tables(const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *cu_lens, int32_t B, int32_t T,
                         int32_t max_blocks_per_seq, int32_t num_blocks,
                         int32_t block_size, int32_t kind);

/* kv_append -- store the new tokens' K and V rows into the paged pools.
 *
 * Defined by: README table of contents "Why KV cache exists" / "Paged KV
 * cache" and guide ch. 3 (each token's K and V are written once and looked
 * up afterwards) and ch. 4 (pages of the cache addressed through a table).
 *
 * k_cache, v_cache  [num_blocks][Hkv][block_size][D] bf16, written in place.
 * k_new, v_new      [T_new][Hkv][D] bf16, packed by sequence.
 * block_tables      [B][max_blocks_per_seq] int32.
 * context_lens      [B] int32, lengths AFTER the append.
 * cu_new_lens       [B+1] int32 prefix sums of new tokens per sequence, or
 *                   NULL for exactly one new token per sequence (T_new == B).
 * New token t of sequence b (n_b new tokens) goes to logical position
 * context_lens[b] - n_b + t.  The copy is bit-exact.  Rows whose slot falls
 * outside the table or pool are not written.  Requires D % 8 == 0.
 */
PKV_API int kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
              const int32_t *block_tables, const int32_t *context_lens,
              const int32_t *cu_new_lens, int32_t B, int32_t T_new, int32_t Hkv,
              int32_t D, int32_t block_size, int32_t max_blocks_per_seq,
              int32_t num_blocks, void *stream);

/* kv_copy_blocks -- copy whole pool blocks (every KV head and row of K and
 * of V): block dst_blocks[i] receives block src_blocks[i], for the copies on
 * write a scheduler step lists (guide ch. 7: shared prefix blocks are copied
 * before one of their sequences writes into them).
 *
 * src_blocks, dst_blocks  [n_pairs] int32 device arrays; pairs whose ids lie
 *                   outside [0, num_blocks) are skipped.  A destination must
 *                   not also be a source or another pair's destination.
 * k_cache, v_cache  pools as for kv_append, written in place.  Bit-exact.
 * D % 8 == 0; pools 16-byte aligned.  n_pairs == 0 is a no-op.
 */
PKV_API int kv_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_blocks,
                   const int32_t *dst_blocks, int32_t n_pairs, int32_t Hkv, int32_t D,
                   int32_t block_size, int32_t num_blocks, void *stream);

/* kv_append_rope -- the rotary position embedding (RoPE) of the new tokens'
 * keys, and optionally of their queries, fused with kv_append.
 *
 * Defined by: README feature list and table of contents "RoPE" (the model's
 * positional encoding), with kv_append's slot rule above.  The pages name
 * RoPE without a formula; this library takes the rotary embedding of the
 * model they run, in the layout of its Safetensors checkpoint: for i < D/2
 * the pair (x[i], x[i + D/2]) of a q or k row is turned by the angle of the
 * token's absolute position pos (kv_append's rule),
 *     y[i]       = x[i] * rope_cos[pos][i] - x[i + D/2] * rope_sin[pos][i]
 *     y[i + D/2] = x[i + D/2] * rope_cos[pos][i] + x[i] * rope_sin[pos][i],
 * each product and the difference rounded to fp32 (no fused multiply-add),
 * the result rounded to bf16 (nearest even).  V rows are copied unchanged.
 *
 * q                 [T_new][Hq][D] bf16, rotated in place; NULL leaves the
 *                   queries alone (Hq is then ignored).
 * k_new, v_new      [T_new][Hkv][D] bf16; the pools receive rotated K and
 *                   unchanged V at kv_append's slots.
 * rope_cos, rope_sin  [max_position][D/2] fp32, the caller's angle tables
 *                   (e.g. cos and sin of pos * inv_freq[i]; any frequency
 *                   scheme); read-only.
 * k_cache, v_cache, block_tables, context_lens, cu_new_lens, B, T_new, Hkv,
 * block_size, max_blocks_per_seq, num_blocks as for kv_append.
 * A token whose position lies outside [0, max_position) is left alone (no
 * rotation of its q rows, no store of its K/V rows).  Rows whose slot falls
 * outside the table or pool are not stored (their q rows are still rotated).
 * This library implements D == 64 (PKV_ERR_UNSUPPORTED otherwise); pools, rows
 * and tables must be 16-byte aligned.
 */
PKV_API int kv_append_rope(void *k_cache, void *v_cache, void *q, const void *k_new,
                   const void *v_new, const float *rope_cos, const float *rope_sin,
                   int32_t max_position, const int32_t *block_tables,
                   const int32_t *context_lens, const int32_t *cu_new_lens, int32_t B,
                   int32_t T_new, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                   int32_t max_blocks_per_seq, int32_t num_blocks, void *stream);

/* ---- Host control plane: block allocator and continuous-batching scheduler.
 *
 * Defined by: guide ch. 4 "PagedAttention" (KV pages handed out on demand by
 * a block allocator, against up-front reservations whose fragmentation wastes
 * 60-80% of the memory) and ch. 5 "The Scheduler" (continuous batching:
 * requests join and leave the running batch at every step); digest "Core
 * Mechanics" (continuous batching).  Host code only: no HIP call, no device
 * memory.  A scheduler object is not thread safe.
 *
 * Policy (the pages print none): every step schedules the running sequences
 * oldest first (one token each once decoding, the next prompt chunk while in
 * prefill), then waiting requests in arrival order while the batch
 * (max_batch rows), the token budget (max_step_tokens) and the free blocks
 * allow; prompts beyond the budget are processed in chunks over several
 * steps.  When a running sequence needs a block and none is free, the most
 * recently arrived running sequence not yet in this step's batch gives up
 * its blocks and waits again (it recomputes its tokens when readmitted); a
 * step that preempted admits no waiting request.
 * static_batching != 0 instead admits up to max_batch requests only when the
 * running set is empty (the comparison the guide draws).
 */
typedef struct pkv_scheduler pkv_scheduler;

/* Number of int64 counters pkv_sched_stats writes:
 *   0 steps            1 tokens scheduled        2 prefill tokens (incl. recomputed)
 *   3 decode tokens    4 preemptions             5 requests finished
 *   6 free blocks now  7 running now             8 waiting now
 *   9  sum over steps of the cached tokens of the running sequences
 *   10 sum over steps of the slots in their blocks (paged allocation)
 *   11 sum over steps of prompt + max_new - 1 per running sequence (a static
 *      reservation of each request's own maximum)
 *   12 sum over steps of max_blocks_per_seq * block_size per running sequence
 *      (a static reservation of the longest sequence allowed)
 *   13 sum over steps of the batch rows
 *   14 block copies on write                15 prompt tokens taken from a
 *                                              shared prefix instead of computed */
#define PKV_SCHED_STATS 16

/* New scheduler over physical blocks 0..num_blocks-1 (all free); NULL for a
 * non-positive argument or out of host memory. */
PKV_API pkv_scheduler *pkv_sched_create(int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t max_batch,
                                int32_t max_step_tokens, int32_t static_batching);
PKV_API void pkv_sched_destroy(pkv_scheduler *s);

/* Queue request `id` (unique among unfinished requests) with prompt_len prompt
 * tokens that will sample max_new_tokens tokens.  PKV_ERR_UNSUPPORTED if its
 * longest cached length (prompt_len + max_new_tokens - 1) needs more blocks
 * than a table row or the pool holds. */
PKV_API int pkv_sched_add_request(pkv_scheduler *s, int64_t id, int32_t prompt_len,
                          int32_t max_new_tokens);

/* As pkv_sched_add_request, for a request whose first prefix_len prompt tokens
 * (a positive multiple of block_size, below prompt_len) are those of the live
 * sequence prefix_owner (guide ch. 7 "Prefix Caching").  When admitted while
 * that sequence holds them computed, the request shares their blocks (each
 * block's count of tables goes up) and computes only the rest; otherwise it
 * computes everything.  The caller guarantees the tokens are the same. */
PKV_API int pkv_sched_add_request_prefix(pkv_scheduler *s, int64_t id, int32_t prompt_len,
                                 int32_t max_new_tokens, int64_t prefix_owner,
                                 int32_t prefix_len);

/* Start sequence child_id from the running sequence parent_id, which must be
 * decoding (every token but its latest sample cached): the child has the same
 * history and shares every block of it, its latest sample is its own, and it
 * samples extra_tokens more tokens (several samples of one prompt).  The first
 * store of either into their shared partly filled block copies that block
 * first (pkv_sched_copies). */
PKV_API int pkv_sched_fork(pkv_scheduler *s, int64_t parent_id, int64_t child_id,
                   int32_t extra_tokens);

/* Block copies the last step needs before its appends (copy on write):
 * returns their count and writes up to max_pairs (source, destination) block
 * ids, to be executed with kv_copy_blocks before the step's kv_append. */
PKV_API int32_t pkv_sched_copies(const pkv_scheduler *s, int32_t *src_blocks,
                         int32_t *dst_blocks, int32_t max_pairs);

/* Plan one engine step and advance the sequences as if it ran.  Returns the
 * batch size B >= 0 (or a negative status) and fills host arrays of at least
 * max_batch rows: seq_ids[B]; q_lens[B], the tokens of each sequence this step
 * stores and attends with (1 when decoding); context_lens[B], its cached
 * tokens after this step's append; cu_q_lens[B+1], prefix sums of q_lens;
 * block_tables[B][max_blocks_per_seq], its physical blocks in logical order,
 * -1 past the last.  These are the arguments kv_append (cu_new_lens =
 * cu_q_lens) and paged_attention_prefill_causal take; a batch of decoding
 * sequences alone fits paged_attention_decode.  Blocks of finished or
 * preempted sequences are reused from the next step on (or, for preempted
 * ones, later in the same step by other sequences), so steps must execute in
 * order on one stream. */
PKV_API int pkv_sched_step(pkv_scheduler *s, int64_t *seq_ids, int32_t *q_lens,
                   int32_t *context_lens, int32_t *cu_q_lens, int32_t *block_tables);

/* Requests that finished (which == 0) or were preempted (which == 1) in the
 * last step: returns their count and writes up to max_ids of them. */
PKV_API int32_t pkv_sched_events(const pkv_scheduler *s, int32_t which, int64_t *ids,
                         int32_t max_ids);

/* Counters (PKV_SCHED_STATS int64 values, see above) into out. */
PKV_API int pkv_sched_stats(const pkv_scheduler *s, int64_t *out);

/* paged_attention_decode_workspace_size -- bytes of device workspace that
 * paged_attention_decode (and _decode_append, _decode_plan) needs for these
 * arguments, 0 when the call splits nothing.
 *
 * Defined by: the split-context form of decode attention -- partial results
 * (o_p, m_p, l_p) of a sequence's key ranges kept until they are merged by
 * log-sum-exp, the online-softmax identity of README table of contents
 * "Online softmax" applied to partitions.  The pages give no interface; the
 * caller owns and sizes every device buffer (the library allocates nothing),
 * so the size of the scratch the split needs is a query.
 *
 * B, Hq, D, max_context_len, partition_size as for paged_attention_decode.
 * This library implements one GQA group (Hq == 4 * Hkv) and one block size
 * (16), so the KV head count is Hq / 4 and the block size 16.  Pure function
 * of its arguments; makes no HIP call.  Returns 0 (and sets
 * pagedkv_last_error) for arguments decode would reject.
 */
PKV_API size_t paged_attention_decode_workspace_size(int32_t B, int32_t Hq, int32_t D,
                                             int32_t max_context_len,
                                             int32_t partition_size);

/* paged_attention_decode -- one query token per sequence attends to all
 * context_lens[b] cached tokens of its sequence.
 *
 * Defined by: README table of contents "Attention", "GQA", "Softmax",
 * "Online softmax", "Paged Attention" and guide ch. 6 (decode reads the whole
 * cache for one new token and is memory bound):
 *     out[b][h] = sum_j softmax_j(scale * q[b][h] . k_j) v_j,
 *     j over the sequence's tokens, k_j/v_j gathered through the block table.
 *
 * out           [B][Hq][D], bf16 or fp32 per out_dtype.
 * q             [B][Hq][D] bf16.
 * k_cache/v_cache, block_tables, context_lens as for kv_append.
 * max_context_len  host-side upper bound of context_lens (sizes the grid;
 *               larger lengths on the device are clamped to it).
 * scale         multiplies q.k before the softmax (e.g. 1/sqrt(D)); finite.
 * partition_size  PKV_PARTITION_NONE: each (sequence, KV head) in one
 *               wavefront.  A positive multiple of block_size: each sequence
 *               is split at multiples of that many tokens, partitions run in
 *               parallel and the wavefront that finishes a sequence's last
 *               partition merges them by log-sum-exp (no second kernel).
 *               PKV_PARTITION_AUTO: each (sequence, KV head) is cut into
 *               pieces of equal length, no longer than a bound chosen from
 *               the batch's total length so that there is about one piece
 *               per wavefront of the grid (2048 wavefronts, or 512 plus one
 *               per (sequence, KV head) when there are more than 1536 of
 *               them), and pieces are merged the same way.
 *               PKV_PARTITION_PLANNED: the same split, read from a plan that
 *               paged_attention_decode_plan stored in this workspace (see
 *               there); a plan made for other B, Hkv, max_blocks_per_seq,
 *               num_blocks or max_context_len is ignored and the split is
 *               computed as for PKV_PARTITION_AUTO.
 * workspace     device scratch of at least
 *               paged_attention_decode_workspace_size(...) bytes (may be NULL
 *               when that is 0).  It must be zero-filled before its first use;
 *               its first 4 MiB hold per-stream split counters (one per
 *               128-byte line, so concurrent atomics on different streams
 *               do not share a line) that every call leaves at zero again, so one zero-fill serves all later
 *               calls, whatever their shapes.  Calls that share a workspace
 *               must not run concurrently (they would race on it).  Splits
 *               handle up to 32768 (sequence, KV head) streams and up to
 *               2^21 - 1 partial records (B * Hkv * partitions per sequence
 *               for a fixed partition_size, one per wavefront of the grid
 *               for PKV_PARTITION_AUTO);
 *               beyond either limit the call returns PKV_ERR_UNSUPPORTED.
 * This library implements D == 64, block_size == 16 and Hq == 4 * Hkv
 * (PKV_ERR_UNSUPPORTED otherwise).  Empty contexts give zero rows.
 */
PKV_API int paged_attention_decode(void *out, int32_t out_dtype, const void *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t max_context_len, float scale,
                           int32_t partition_size, void *workspace,
                           size_t workspace_bytes, void *stream);

/* paged_attention_decode_noalloc -- paged_attention_decode without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and partition modes as paged_attention_decode
 * except PKV_PARTITION_PLANNED (rejected: the plan lives in a caller
 * workspace).  The split's counters and partial records live in a static
 * device array of 16 MiB (PKV_NOALLOC_SCRATCH_BYTES) that each GPU holds
 * until the process ends; a call whose split needs more
 * (paged_attention_decode_workspace_size beyond it) returns
 * PKV_ERR_UNSUPPORTED.  The call allocates nothing: no hipMalloc, hipFree
 * or allocating library routine.  Its first call on a device zeroes the
 * counters with a fill kernel on `stream`; every call leaves them at zero
 * again.  All calls on one GPU share that GPU's array, so calls that
 * overlap on one GPU (different streams, threads or processes' contexts
 * excepted) race on it and must be ordered by the caller.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
PKV_API int paged_attention_decode_noalloc(void *out, int32_t out_dtype, const void *q,
                                   const void *k_cache, const void *v_cache,
                                   const int32_t *block_tables,
                                   const int32_t *context_lens, int32_t B, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t num_blocks,
                                   int32_t max_context_len, float scale,
                                   int32_t partition_size, void *stream);

/* paged_attention_decode_plan -- store the plan of the automatic split for
 * these lengths and tables in the workspace, for later calls of
 * paged_attention_decode / _decode_append with PKV_PARTITION_PLANNED.
 *
 * Defined by: the calls it serves (the split is a scheduling of the same
 * attention; guide ch. 6: every layer of a decode step reads the same block
 * tables and lengths).
 *
 * The plan is what the automatic split computes before its first key load:
 * its piece bound, the prefix of per-sequence piece counts, and for each
 * wavefront of its grid the piece it attends over and the block ids of that
 * piece's first 64 blocks.  Every layer of a decode step shares block_tables and
 * context_lens, so one plan per step serves all of them and each call starts
 * loading keys at once.  A plan describes the contents of block_tables and
 * context_lens at the time of this call: after they change (the next step),
 * plan again; a call with a plan whose contents are stale gives wrong
 * results (it stays inside the pools and the workspace).
 * Arguments as for paged_attention_decode; the workspace must hold
 * paged_attention_decode_workspace_size(..., PKV_PARTITION_PLANNED) bytes and
 * be the one the planned calls pass.  Calls sharing a workspace must not run
 * concurrently.
 */
PKV_API int paged_attention_decode_plan(const int32_t *block_tables,
                                const int32_t *context_lens, int32_t B, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t num_blocks,
                                int32_t max_context_len, void *workspace,
                                size_t workspace_bytes, void *stream);

/* paged_attention_decode_append -- one decode step of a layer: store one new
 * token per sequence in the pools (kv_append with cu_new_lens = NULL), then
 * attend (paged_attention_decode), with the same results as those two calls.
 *
 * Defined by: the two calls it combines (README table of contents "Why KV
 * cache exists", "Paged KV cache", "Paged Attention"; guide ch. 3, ch. 6: a
 * decode step caches the new token's K/V and reads the whole cache).
 *
 * k_new/v_new   [B][Hkv][D] bf16: the new token of each sequence, which is
 *               the last of its context_lens[b] tokens.
 * Other arguments as for paged_attention_decode; k_cache/v_cache are written.
 * With PKV_PARTITION_AUTO this is one kernel launch: the wavefront that reads
 * a sequence's last block writes the new rows and uses them directly.  Other
 * partition sizes run the append and the decode kernels in turn.  Rows are
 * stored exactly where kv_append stores them (none for context_lens[b] < 1 or
 * a slot outside the table or pool); the decode is clamped to
 * max_context_len as in paged_attention_decode.  k_new/v_new must be 16-byte
 * aligned and must not overlap the pools.
 */
PKV_API int paged_attention_decode_append(void *out, int32_t out_dtype, const void *q,
                                  void *k_cache, void *v_cache,
                                  const void *k_new, const void *v_new,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t block_size, int32_t max_blocks_per_seq,
                                  int32_t num_blocks, int32_t max_context_len, float scale,
                                  int32_t partition_size, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* paged_attention_prefill_causal -- every prompt token attends to the cached
 * tokens up to and including its own position.
 *
 * Defined by: README table of contents "Prefill vs decode", "Attention",
 * "GQA", "Causal mask", "Online softmax", "Paged Attention" and guide ch. 6
 * (prefill processes the whole prompt and is compute bound).  Query t of
 * sequence b sits at position pos = context_lens[b] - q_len_b + t and sees
 * keys 0..pos; the K/V of the prompt must already be in the pools (kv_append).
 *
 * out           [T_q][Hq][D], bf16 or fp32 per out_dtype.
 * q             [T_q][Hq][D] bf16, packed by sequence.
 * cu_q_lens     [B+1] int32 prefix sums of query tokens per sequence.
 * max_q_len     host-side upper bound of the per-sequence query counts
 *               (values above T_q are taken as T_q).  Only the first
 *               max_q_len rows of each sequence are computed and written:
 *               rows past them in a longer sequence keep what out held.
 * Other arguments as for decode.  This library implements D == 64,
 * block_size == 16 and Hq == 4 * Hkv.  Workgroups of 256 threads: one per
 * 32-row query tile, sequence and KV head; a sequence of at most 4 query
 * rows (a decoding sequence of a mixed batch, a few draft tokens) is one
 * workgroup per KV head whose 4 wavefronts split its context.  The grid has
 * ceil(min(max_q_len, T_q) / 32) ranks per sequence, or, for at most 256
 * sequences where at most a third of those would hold a query tile, only
 * B + T_q / 32 units per KV head (the tiles of a rank found on the device);
 * a grid beyond one launch (2^32 - 1 work-items) returns
 * PKV_ERR_UNSUPPORTED.
 */
PKV_API int paged_attention_prefill_causal(void *out, int32_t out_dtype, const void *q,
                                   const void *k_cache, const void *v_cache,
                                   const int32_t *block_tables,
                                   const int32_t *context_lens,
                                   const int32_t *cu_q_lens, int32_t B, int32_t T_q,
                                   int32_t Hq, int32_t Hkv, int32_t D,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, int32_t max_q_len, float scale,
                                   void *stream);

/* ---- Measurement.
 *
 * pagedkv_stream_blocks -- read, and do nothing else with, the K and V bytes
 * of whole (block, KV head) chunks of both pools for a list of physical block
 * ids: the floor a decode call reading the same blocks is measured against.
 *
 * Defined by: guide ch. 6 "Prefill vs Decode" (decode is memory bound: it
 * reads the whole cache once per new token) and ch. 11 "Benchmarks" (state
 * how close a kernel comes to its bound).  Not part of the attention path.
 *
 * block_ids     [n_ids] int32 device array (e.g. every table entry the
 *               batch's contexts use, in order); ids outside [0, num_blocks)
 *               read block 0.
 * k_cache, v_cache  pools as for kv_append; read only.  Every KV head of each
 *               listed block is read: n_ids * Hkv * block_size * D * 2 bytes
 *               from each pool.
 * sink          device buffer of at least PKV_STREAM_SINK_BYTES; receives
 *               one folded word per lane (meaningless; it keeps the reads).
 * This library reads 2 KB chunks: D == 64 and block_size == 16.  The grid is
 * 2048 wavefronts, each streaming an equal contiguous share of the chunks.
 */
#define PKV_STREAM_SINK_BYTES (2048u * 64u * 4u)
PKV_API int pagedkv_stream_blocks(const void *k_cache, const void *v_cache,
                          const int32_t *block_ids, int32_t n_ids, int32_t Hkv,
                          int32_t D, int32_t block_size, int32_t num_blocks, void *sink,
                          size_t sink_bytes, void *stream);

/* pagedkv_mfma_probe -- run bf16 matrix-core products and nothing else: the
 * issue rate that the prefill kernel's flops are measured against, taken on
 * this GPU at its running clock.
 *
 * Defined by: guide ch. 6 "Prefill vs Decode" (prefill is compute bound) and
 * ch. 11 "Benchmarks" (state how close a kernel comes to its bound).  Not
 * part of the attention path.
 *
 * 2048 wavefronts each run 4 independent chains of
 * v_mfma_f32_32x32x16_bf16 (32,768 flops a product) `iters` times on
 * operands held in registers: 2048 * 4 * iters * 32768 flops per launch.
 * iters         1 .. PKV_MFMA_PROBE_MAX_ITERS.
 * sink          device buffer of at least PKV_STREAM_SINK_BYTES, 16-byte
 *               aligned; lane l of wavefront w writes float w * 64 + l, whose
 *               value is exactly 4 * iters (every operand element is 2^-4).
 * Errors: PKV_ERR_INVALID_ARG for iters out of range or a null or misaligned
 * sink, PKV_ERR_WORKSPACE for a short sink.
 */
#define PKV_MFMA_PROBE_MAX_ITERS (1 << 18)
PKV_API int pagedkv_mfma_probe(int32_t iters, void *sink, size_t sink_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
