/*
 * kvc.h — C ABI of the paged-KV ragged attention library (libkvc.so, gfx950).
 *
 * One call runs one continuously-batched attention step for one layer: the
 * rows of several sequences are concatenated without a batch dimension, each
 * sequence's new K/V rows are appended to a paged cache, and every new row
 * attends over its sequence's cached keys plus the new keys up to itself.
 * Decode rows (one new token) and chunked-prefill rows (several new tokens)
 * mix freely in one call.
 *
 * Where the operations are defined (the four pages on KV caches and
 * continuous batching):
 *   - attention with a boolean causal mask and row-wise softmax, Q/K/V of
 *     different lengths: news.myit.tw/news/j9529p (translated "continuous
 *     batching from first principles" article), section "Attention";
 *   - KV cache, per-token cache size 2*L*H*A values: same article, "KV cache";
 *   - chunked prefill, cached K/V prepended and the mask shifted by the cached
 *     length: same article, "Chunked prefill";
 *   - ragged batching with a block-diagonal mask and mixed prefill/decode:
 *     same article, "Continuous batching";
 *   - paged cache, block table mapping logical blocks to physical blocks,
 *     just-in-time block allocation: clvsit.github.io AWS SageMaker page,
 *     section "PagedAttention 批处理"; klklkl10086.github.io kv_cache post,
 *     section "Paged Attention";
 *   - sharing blocks by editing block tables (a common prefix written once):
 *     the kv_cache post, "Paged Attention"; e2hang/Notes "KV Cache与Continuous
 *     Batching", section on prefix caching;
 *   - GQA/MQA, num_kv_heads = num_q_heads / ratio: e2hang/Notes, "MQA与GQA";
 *   - decode attention softmax(q K^T / sqrt(d)) V after appending the new
 *     token's K/V: the kv_cache post, "Batch Decode".
 *
 * Conventions shared by every entry point
 *   Memory    All device pointers are caller-owned device memory (e.g. from
 *             PyTorch), contiguous, 16-byte aligned.  The library never
 *             allocates device memory; scratch space is the caller's
 *             `workspace`.  The allocator below hands out block ids only.
 *   bf16      Every K/V/q/out element is bf16 (raw 16-bit storage).
 *   Layouts   q, out      [total_q][num_q_heads][head_dim]
 *             k_new,v_new [total_q][num_kv_heads][head_dim]
 *             k_cache,v_cache (the pools) [num_blocks][num_kv_heads][block_size][head_dim]
 *             block_table int32 [num_seqs][max_blocks_per_seq]
 *             cu_seqlens_q int32 [num_seqs+1], cu[0]=0, cu[num_seqs]=total_q,
 *                         non-decreasing; rows of sequence s are cu[s]..cu[s+1]-1
 *             context_lens int32 [num_seqs]: tokens of sequence s cached
 *                         BEFORE the call.
 *   Positions Token position p of sequence s lives in physical block
 *             block_table[s][p / block_size], slot p % block_size.
 *   Heads     Query head h reads kv head h / (num_q_heads / num_kv_heads).
 *   Streams   `stream` is a hipStream_t (NULL = the null stream).  Device
 *             work is enqueued asynchronously, in stream order.  When a step
 *             has prefill chunks and enough decode rows to fill the GPU
 *             (judged from the host sizes: the decode's work items, kv heads
 *             and head chunks against the compute units; otherwise the
 *             prefill simply runs first on `stream`),
 *             kvc_paged_attention_varlen runs the prefill kernel on an
 *             internal side stream that belongs to `stream` (one per caller
 *             stream and device, created on first use, default priority),
 *             forked from `stream` after the append and joined back before
 *             the call returns, so it overlaps the decode kernels; to the
 *             caller the step is still one ordered piece of `stream`: work
 *             the caller enqueues on `stream` afterwards (a copy of `out`, the
 *             next step reusing the workspace) starts after the whole step.
 *             If the join cannot be enqueued, the call waits on the host for
 *             the side stream before returning the error.  KVC_SERIAL=1
 *             keeps every kernel on `stream`.
 *   Errors    Every entry point returns a kvc_status.  Arguments are checked
 *             before anything is enqueued, so a call that returns an error
 *             has had no effect.  Values inside device arrays (table entries,
 *             lengths) are not read by the host; the kernels never touch
 *             memory outside the pools for a bad entry (they skip it and set a
 *             flag in the workspace, see kvc_workspace_flags), and the outputs
 *             of the affected rows are then unspecified.  With the environment
 *             variable KVC_DEBUG=1 the host also copies the lengths and the
 *             table back (synchronously) and rejects bad values with
 *             KVC_ERR_INVALID_ARG before launching.
 *   Supported head_dim in {16, 64, 128, 256}; block_size in {4, 16};
 *             num_q_heads % num_kv_heads == 0 with ratio G = 1, 2 or any
 *             multiple of 4 (MHA, GQA, MQA).  Others return
 *             KVC_ERR_UNSUPPORTED.
 *   Threads   Entry points are reentrant, and calls on different streams
 *             from different host threads do not wait for each other: only
 *             two threads calling on the same stream share its side stream's
 *             event pair (under a mutex), and per-kernel timing, while on,
 *             takes a lock.  An allocator or scheduler object is not
 *             thread-safe (one owner at a time).
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVC_OK = 0,
    KVC_ERR_INVALID_ARG = -1, /* null pointer, bad size, double free, ...   */
    KVC_ERR_OOM = -2,         /* allocator has too few free blocks          */
    KVC_ERR_UNSUPPORTED = -3, /* head_dim / block_size / head ratio         */
    KVC_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    KVC_ERR_HIP = -5          /* a HIP runtime call failed (launch, query)  */
} kvc_status;

/* Static description of a status code.  Never NULL. */
const char* kvc_status_string(int status);
/* Detail of the last failing call on this thread ("" if none).  Valid until
 * the next call on the same thread. */
const char* kvc_last_error(void);

/* ------------------------------------------------------------------------
 * Host block allocator (free list + reference counts).  Host memory only.
 * Physical blocks are fixed-size pages of the pool; a block table row lists a
 * sequence's physical blocks in logical order.  A block shared by several
 * tables (a common prefix) carries one reference per table and returns to the
 * free list when the last reference is dropped.
 * ---------------------------------------------------------------------- */
typedef struct kvc_allocator kvc_allocator;

/* Create an allocator over blocks 0..num_blocks-1, all free.
 * num_blocks >= 1, block_size >= 1.  *out receives the handle. */
int kvc_allocator_create(int32_t num_blocks, int32_t block_size, kvc_allocator** out);
/* Destroy (NULL is a no-op). */
void kvc_allocator_destroy(kvc_allocator* a);

/* Take n free blocks (refcount 1 each) into out_ids[0..n-1].  All or
 * nothing: with fewer than n free blocks it returns KVC_ERR_OOM and changes
 * nothing.  n == 0 is a no-op. */
int kvc_alloc_blocks(kvc_allocator* a, int32_t n, int32_t* out_ids);
/* Add one reference to each listed block (each must be allocated). */
int kvc_share_blocks(kvc_allocator* a, const int32_t* ids, int32_t n);
/* Drop one reference from each listed block; a block whose count reaches 0
 * returns to the free list.  A free or out-of-range id (or an id listed more
 * times than it has references) returns KVC_ERR_INVALID_ARG with no effect. */
int kvc_free_blocks(kvc_allocator* a, const int32_t* ids, int32_t n);
int32_t kvc_num_free_blocks(const kvc_allocator* a);
int32_t kvc_num_blocks(const kvc_allocator* a);
/* Tokens per block the allocator was created with (-1 for NULL). */
int32_t kvc_allocator_block_size(const kvc_allocator* a);
/* Reference count of a block (0 = free), or -1 for an out-of-range id. */
int32_t kvc_block_refcount(const kvc_allocator* a, int32_t id);

/* Just-in-time growth of one sequence's table row (the page's rule: a new
 * physical block only when the current one is full).  `row` holds *held valid
 * ids; blocks are taken until the row covers new_len tokens, i.e.
 * ceil(new_len / block_size) ids.  All or nothing (KVC_ERR_OOM leaves the row
 * and the allocator unchanged); KVC_ERR_INVALID_ARG if the row would need more
 * than max_blocks entries. */
int kvc_extend_table(kvc_allocator* a, int32_t* row, int32_t max_blocks,
                     int32_t* held, int64_t new_len);
/* The same growth for every row of a step's table at once: row s of `table`
 * ([num_seqs][max_blocks] int32, host) holds held[s] valid ids and is grown to
 * cover new_lens[s] tokens; held[s] is updated.  All or nothing for the whole
 * batch: on any error (KVC_ERR_INVALID_ARG for a bad size or a row too short,
 * KVC_ERR_OOM when the free blocks do not cover all rows) no row and no
 * block changes.  For callers that grow every running sequence per step,
 * one call instead of one per sequence. */
int kvc_extend_tables(kvc_allocator* a, int32_t* table, int32_t max_blocks, int32_t* held,
                      const int64_t* new_lens, int32_t num_seqs);

/* Copy-on-write of one block before a write into it (a shared block must
 * not change under its other sharers; sharing by table edits, klklkl10086
 * kv_cache post, sections "Paged Attention" and "连续内存分配").  If `id` has
 * one reference, *out_id = id and *copied = 0.  Otherwise a fresh block is
 * taken (refcount 1), one reference to `id` is dropped, *out_id is the new
 * block and *copied = 1: the caller copies the contents (kvc_copy_blocks)
 * before writing.  KVC_ERR_OOM (no free block) or KVC_ERR_INVALID_ARG (free
 * or out-of-range id) leave everything unchanged. */
int kvc_cow_block(kvc_allocator* a, int32_t id, int32_t* out_id, int32_t* copied);

/* Fork a sequence (a shared prefix or a beam): the child's table row takes the
 * parent's first ceil(len / block_size) blocks.  Full blocks are shared (one
 * more reference each); a partially filled last block (len % block_size != 0),
 * which the child will append into, is copied on write: the child gets a
 * fresh block and (copy_src[0], copy_dst[0]) = (parent's block, new block),
 * *n_copies = 1, for kvc_copy_blocks (else *n_copies = 0).  *child_held =
 * ceil(len / block_size).  All or nothing: KVC_ERR_OOM / KVC_ERR_INVALID_ARG
 * (row longer than max_blocks, a free or out-of-range parent id) change
 * nothing. */
int kvc_fork_table(kvc_allocator* a, const int32_t* parent_row, int64_t len,
                   int32_t* child_row, int32_t max_blocks, int32_t* child_held,
                   int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies);

/* ------------------------------------------------------------------------
 * Host continuous-batching scheduler (news.myit.tw continuous-batching
 * article, sections "Continuous batching" and "Chunked prefill"; blocks just
 * in time, clvsit.github.io "PagedAttention 批处理").  Host memory only, not
 * thread-safe.  Each step: one decode row per generating sequence (oldest
 * first), then the next chunks of prompts in progress, then first-come
 * first-served admissions, all within token_budget rows and max_seqs
 * sequences.  On admission a request reserves the blocks of its whole life
 * (ceil((prompt_len + max_new_tokens - 1) / block_size)); blocks are taken
 * from the allocator when rows need them and returned when the request
 * finishes, so an admitted request never runs out of blocks.  A prompt's last
 * chunk produces its first token, each decode row the next one; a request
 * finishes when it has produced max_new_tokens.
 * ---------------------------------------------------------------------- */
typedef struct kvc_scheduler kvc_scheduler;

/* Create over an allocator (not owned; it must outlive the scheduler).
 * token_budget >= 1 rows per step, max_seqs >= 1 sequences per step,
 * max_blocks_per_seq >= 1 = the width of the block-table rows it writes. */
int kvc_scheduler_create(kvc_allocator* alloc, int32_t token_budget, int32_t max_seqs,
                         int32_t max_blocks_per_seq, kvc_scheduler** out);
/* Destroy; blocks still held by running requests return to the allocator. */
void kvc_scheduler_destroy(kvc_scheduler* s);
/* Queue a request.  prompt_len, max_new_tokens >= 1; KVC_ERR_INVALID_ARG if
 * it could never fit a table row or the pool.  request_id is the caller's tag,
 * handed back by step and complete; requests are tracked by admission order,
 * so ids need not be unique. */
int kvc_scheduler_add(kvc_scheduler* s, int64_t request_id, int32_t prompt_len,
                      int32_t max_new_tokens);
/* Plan the next step into host arrays with capacity max_seqs (+1 for
 * cu_seqlens_q; block_table max_seqs * max_blocks_per_seq, entries past a
 * row's held blocks are -1): the rows of sequence k are
 * cu_seqlens_q[k] .. cu_seqlens_q[k+1]-1, cached before the step
 * context_lens[k], request request_ids[k].  *num_seqs = 0 when nothing can
 * run.  The table already covers the new rows.  A planned step must be
 * completed before the next one is planned. */
int kvc_scheduler_step(kvc_scheduler* s, int32_t* cu_seqlens_q, int32_t* context_lens,
                       int32_t* block_table, int64_t* request_ids, int32_t* num_seqs,
                       int32_t* total_q, int32_t* max_q_len, int32_t* max_context_len);
/* Mark the planned step as executed: the sequences advance, finished requests
 * (ids in finished_ids, capacity max_seqs, count *n_finished) free their blocks. */
int kvc_scheduler_complete(kvc_scheduler* s, int64_t* finished_ids, int32_t* n_finished);
int32_t kvc_scheduler_num_waiting(const kvc_scheduler* s);
int32_t kvc_scheduler_num_running(const kvc_scheduler* s);

/* Bytes of the two pools (K and V): 2 * num_blocks * block_size *
 * num_kv_heads * head_dim * elem_bytes.  Per token and layer this is the
 * 2*H*A values of the cache-size formula.  Returns -1 on a negative input. */
int64_t kvc_cache_bytes(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                        int32_t head_dim, int32_t elem_bytes);

/* ------------------------------------------------------------------------
 * Device operations.
 * ---------------------------------------------------------------------- */

/* Append: for every sequence s and new row i < q_len_s, copy
 * k_new[cu[s]+i][g][:] and v_new[cu[s]+i][g][:] (all kv heads g) into the
 * pool slot of position context_lens[s] + i.  A pure bit copy; nothing else in
 * the pools changes.  The table must already cover context_lens[s] + q_len_s
 * tokens.  num_blocks = pool length (bounds every block id). */
int kvc_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* cu_seqlens_q, const int32_t* context_lens,
                  int32_t num_seqs, int32_t total_q, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, void* stream);

/* Gather: rebuild each sequence's contiguous cache,
 * k_out[cu_seq_lens[s] + p][g][:] = k_cache[table[s][p / bs]][g][p % bs][:]
 * for p < seq_lens[s] (same for V).  Bit copy.  seq_lens int32 [num_seqs],
 * cu_seq_lens int64 [num_seqs+1] (its prefix sums), total_tokens =
 * cu_seq_lens[num_seqs]; k_out, v_out [total_tokens][num_kv_heads][head_dim]. */
int kvc_gather_kv(const void* k_cache, const void* v_cache, int64_t num_blocks,
                  const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* seq_lens, const int64_t* cu_seq_lens, int64_t total_tokens,
                  void* k_out, void* v_out, int32_t num_seqs, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, void* stream);

/* Block copy for copy-on-write: block dst_ids[i] := block src_ids[i] in both
 * pools (all kv heads and slots), i < n.  src_ids, dst_ids: device int32
 * arrays.  A pair with an id outside [0, num_blocks) is skipped (KVC_DEBUG=1
 * checks on the host and rejects it).  The destinations must be distinct and
 * must not be among the sources (the copies run concurrently).  Bit copy. */
int kvc_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks, const int32_t* src_ids,
                    const int32_t* dst_ids, int32_t n, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, void* stream);

/* Workspace bytes kvc_paged_attention_varlen needs for a step with these
 * bounds (max_context_len >= every context_lens[s], max_q_len >= every
 * q_len_s).  0 for invalid or unsupported arguments. */
size_t kvc_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                          int32_t max_context_len, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size);

/* One ragged paged-attention step.
 *   1. If k_new and v_new are non-NULL, append them exactly as kvc_append_kv
 *      (NULL for both means "already appended").
 *   2. For every sequence s, new row i < q_len_s and query head h:
 *        keys j = 0 .. context_lens[s] + i (inclusive; the causal mask shifted
 *        by the cached length), z_j = scale * q[cu[s]+i][h] . K_s[j][h/G],
 *        out[cu[s]+i][h][:] = sum_j softmax(z)_j * V_s[j][h/G][:]   (bf16).
 *      Rows with q_len_s == 1 take the split-K decode path, rows of longer
 *      chunks the MFMA prefill path; both compute the same function.
 * max_q_len / max_context_len are host-side upper bounds (no device readback);
 * they size the work lists, so they must not be exceeded.  total_q must equal
 * cu_seqlens_q[num_seqs]; together with num_seqs and max_q_len it also picks
 * the launches: when total_q > (num_seqs - 1) * max_q_len + 1 no row can be a
 * decode row, and the decode and merge launches are skipped.  scale must be
 * finite.  workspace: device memory of at least
 * kvc_workspace_size(num_seqs, total_q, max_q_len, max_context_len, ...) bytes,
 * 256-byte aligned, owned by the caller; it may be reused across calls that
 * do not overlap in time.  The result does not depend on the physical block
 * ids, on which other sequences share the call, or on the stream's history. */
int kvc_paged_attention_varlen(void* out, const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, int64_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* cu_seqlens_q, const int32_t* context_lens,
                               int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                               int32_t max_context_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream);

/* No-allocation variant, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, meaning and result as
 * kvc_paged_attention_varlen, without the workspace: the step's scratch is a
 * static device array of KVC_NOALLOC_SCRATCH_BYTES that each GPU holds from
 * the library's load until the process ends.  A step that needs more
 * (kvc_workspace_size above the limit) returns KVC_ERR_WORKSPACE before
 * anything is enqueued.  The call allocates nothing (no hipMalloc, no
 * stream or event creation) and runs every kernel on `stream`, so its prefill
 * does not overlap its decode.  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (two streams, two threads)
 * race, so callers serialise them.  The kernels' flags (see
 * kvc_workspace_flags) go to the static array and are not reported. */
#define KVC_NOALLOC_SCRATCH_BYTES (128u << 20)
int kvc_paged_attention_varlen_noalloc(void* out, const void* q, const void* k_new,
                                       const void* v_new, void* k_cache, void* v_cache,
                                       int64_t num_blocks, const int32_t* block_table,
                                       int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t total_q, int32_t max_q_len,
                                       int32_t max_context_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, float scale, void* stream);

/* Flags the kernels of the last call that used `workspace` raised (0 = none):
 *   1 a position beyond max_blocks_per_seq, 2 a block id outside
 *   [0, num_blocks), 4 more work than the host bounds allowed (lengths above
 *   max_context_len / max_q_len), 8 cu_seqlens_q inconsistent with total_q.
 * Synchronises `stream` and copies one int back. */
int kvc_workspace_flags(const void* workspace, void* stream, int32_t* flags);

/* ------------------------------------------------------------------------
 * The baseline that ragged continuous batching replaces: one decode step of
 * a left-padded batch (news.myit.tw continuous-batching article, section
 * "Continuous batching": the sequences of a static batch are padded on the
 * left to one length and a padding mask hides the pad positions) over a
 * contiguous cache that reserves n_max positions per sequence (klklkl10086
 * kv_cache post, section "连续内存分配").  For comparison with the paged
 * ragged step; it reads every position, pads included.
 *   k_cache, v_cache: [batch * n_max / block_size][num_kv_heads][block_size]
 *            [head_dim] bf16 (the pool's page format): sequence b owns pages
 *            b * n_max / block_size .. (b + 1) * n_max / block_size - 1, its
 *            position p in page p / block_size, slot p % block_size.
 *   pad_lens: device int32 [batch]; sequence b's tokens sit at positions
 *            pad_lens[b] .. n_max - 1 (values are clamped to [0, n_max - 1]).
 *            Pad positions may hold anything: they get weight exactly 0.
 *   q, out:  [batch][num_q_heads][head_dim]; k_new, v_new [batch][num_kv_heads]
 *            [head_dim] are first appended at position n_max - 1 (NULL for
 *            both: already in the cache).
 * Row b of out is attention over keys pad_lens[b] .. n_max - 1 of sequence b,
 * the same function kvc_paged_attention_varlen computes for a sequence of
 * n_max - 1 - pad_lens[b] cached tokens.  head_dim 128, block_size 4 or 16,
 * n_max a multiple of block_size (at most 2^24); otherwise
 * KVC_ERR_UNSUPPORTED / KVC_ERR_INVALID_ARG, before anything is enqueued.
 * workspace: kvc_padded_workspace_size(...) bytes, 256-byte aligned, caller
 * owned (0 = arguments not supported). */
size_t kvc_padded_workspace_size(int32_t batch, int32_t n_max, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size);
int kvc_padded_decode_attention(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* pad_lens,
                                int32_t batch, int32_t n_max, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                float scale, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Optional per-kernel timing (instrumentation; off by default).
 * kvc_profile_begin(n) makes the next n calls of kvc_paged_attention_varlen
 * record a HIP event just before and just after each of its kernels, on the
 * stream that kernel runs on (host-side hipEventCreate only; no device
 * memory).  kvc_profile_end waits for those events, writes into
 * ms_sum[KVC_PROF_PHASES] the summed start-to-end milliseconds of each kernel
 * over the recorded calls (0 for a kernel a call did not need), writes the
 * number of recorded calls, and turns timing off.  One profiling client at a
 * time.
 * ---------------------------------------------------------------------- */
enum {
    KVC_PROF_PLAN = 0,    /* work-list planning + append (one launch) */
    KVC_PROF_APPEND = 1,  /* reserved: the append shares the plan launch */
    KVC_PROF_PREFILL = 2, /* MFMA prefill-chunk kernel               */
    KVC_PROF_DECODE = 3,  /* split-K decode partials                 */
    KVC_PROF_MERGE = 4,   /* log-sum-exp merge of decode partials    */
    KVC_PROF_PHASES = 5
};
int kvc_profile_begin(int32_t max_calls);
int kvc_profile_end(double* ms_sum, int32_t* calls);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
