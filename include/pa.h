/*
 * pa.h -- C ABI of libpa: the PagedAttention hot path on MI355X (gfx950).
 *
 * Pages cited (titles as published; sections as numbered on each page):
 *   [P1] "12. 推理加速(二): nano-vllm — 1200 行手写 vLLM": §12.6 (Attention layer:
 *        paged KV cache -- the store kernel and the two FlashAttention calls),
 *        §12.7 (ModelRunner: KV-cache allocation, prepare_prefill/decode,
 *        CUDA-graph padding).
 *   [P2] kyonqi, "nano-vllm 05" (ModelRunner): prepare_prefill, prepare_decode,
 *        prepare_block_tables, run_model.
 *   [P4] "vLLM 深度解读", §3 (PagedAttention CUDA kernel sketch).
 *   [P5] "Nano-vLLM 源码解读 - 3. PagedAttention": §3 (two-step mapping),
 *        §4 (slot_mapping protocol; prefill and decode paths), §5 (block size).
 *
 * Common conventions
 *   - bf16 tensors are passed as untyped pointers to IEEE bfloat16 data.
 *   - A KV cache is ONE layer's pool, [num_blocks, block_size, num_kv_heads,
 *     head_dim], contiguous (the per-layer view of the engine's pool, [P1
 *     §12.7]). A "slot" is a row index into it viewed as
 *     [num_blocks * block_size, num_kv_heads * head_dim].
 *   - Pointers named as device pointers must point to device memory (or
 *     memory the device can read); host pointers to host memory. The caller
 *     owns every buffer. The library never allocates or frees memory; its only
 *     global state is a per-thread error message (and, for
 *     pa_decode_noalloc, one device array per GPU that the library holds).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Every
 *     device entry point only enqueues work on it and returns; nothing
 *     synchronises.
 *   - Return value: PA_OK (0) or a negative PA_ERR_* code; pa_last_error()
 *     then describes the problem. Host-side checks never read device memory;
 *     device-resident preconditions (slots, table entries, lengths) are the
 *     caller's to keep and are listed per function.
 *   - Supported shapes: head_dim 64 or 128; block_size a power of two in
 *     [16, 1024] (256 is the pages' size and the tuned one); num_q_heads a
 *     multiple of num_kv_heads with group size G = num_q_heads / num_kv_heads
 *     in 1 .. 16. Others return PA_ERR_UNSUPPORTED.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_OK 0
#define PA_ERR_INVALID_ARG (-1) /* null pointer, bad size/stride/alignment  */
#define PA_ERR_UNSUPPORTED (-2) /* shape outside the compiled set           */
#define PA_ERR_WORKSPACE (-3)   /* workspace missing or too small           */
#define PA_ERR_HIP (-4)         /* the HIP runtime reported a launch error  */

/* Geometry of one layer's cache. */
typedef struct pa_desc {
  int32_t num_q_heads;  /* H_q                                               */
  int32_t num_kv_heads; /* H_kv; q-head h reads kv-head h / (H_q / H_kv)     */
  int32_t head_dim;     /* d: 64 or 128                                      */
  int32_t block_size;   /* B: tokens per physical block; 256 in [P5 §5]      */
  int64_t num_blocks;   /* N: physical blocks in the pool                    */
} pa_desc;

/*
 * pa_store_kv -- scatter new tokens' K and V into the paged cache.
 * [P1 §12.6] store kernel; slot protocol [P5 §4].
 *
 * For every i < n_tokens with s = slot_mapping[i] != -1, copies the
 * H_kv*d bf16 values of k[i] into k_cache row s and those of v[i] into
 * v_cache row s, bit for bit. s == -1 is a padding entry and is skipped
 * (the graph-replay padding of [P1 §12.7]). Rows not named are untouched.
 *
 *   k, v          device, bf16 [n_tokens, H_kv, d]; the last two dims are
 *                 contiguous (head stride d) and token i starts at element
 *                 i * k_row_stride (resp. v_row_stride). The strides let k/v
 *                 be views of a fused qkv projection output.
 *   k_row_stride, v_row_stride   elements, >= H_kv*d.
 *   k_cache, v_cache  device, bf16 [N, B, H_kv, d], contiguous.
 *   slot_mapping  device, int32 [n_tokens]; each entry -1 or in [0, N*B);
 *                 entries other than -1 must be distinct (otherwise the
 *                 surviving value is unspecified).
 *   n_tokens      >= 0; 0 is a successful no-op.
 * Alignment: any; a 16-byte path is used when pointers and strides allow.
 */
int pa_store_kv(const void* k, int64_t k_row_stride, const void* v, int64_t v_row_stride,
                void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t n_tokens,
                const pa_desc* desc, void* stream);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs for
 * this batch geometry. Layout: a fixed 256 KiB header of arrival counters
 * (one per sequence and kv-head; the single-launch decode counts there which
 * pieces of a split sequence are done, so the last one merges them), then
 * the split-K partial results (one row per range of the grid and sequence).
 * Batches of more than 65,536 (sequence, kv-head) pairs, and explicit
 * partition lengths (pa_decode_partitioned), use the partitioned grid
 * instead: the same header (left untouched), partials per partition, and a
 * longest-first dispatch order. 0 on invalid arguments, and for a
 * partitioned grid that needs no workspace. The result depends only on the
 * arguments.
 */
size_t pa_decode_workspace_size(const pa_desc* desc, int32_t num_seqs, int32_t max_context_len);

/*
 * pa_decode -- paged decode attention, one query per sequence.
 * [P1 §12.6] decode branch (flash_attn_with_kvcache over the block table),
 * [P4 §3] kernel sketch (block-table read, online softmax), GQA grouping.
 *
 * For each sequence b and q-head h, with g = h / (H_q / H_kv) and
 * n = context_lens[b]:
 *   out[b,h,:] = sum_t softmax_t(scale * q[b,h,:] . K_t) * V_t,   t < n,
 * where K_t, V_t are the kv-head-g rows of token t, found at slot
 * block_tables[b][t / B] * B + t % B ([P5 §3]). n includes the token just
 * stored, so pa_store_kv runs first on the same stream. n == 0 marks a
 * padding row: its output is all zeros and nothing is read for it.
 * Accumulation is fp32; out is rounded to bf16 (nearest, ties to even).
 *
 *   q             device, bf16 [num_seqs, H_q, d], contiguous.
 *   k_cache, v_cache  device, bf16 [N, B, H_kv, d].
 *   block_tables  device, int32 [num_seqs, max_blocks_per_seq] row-major;
 *                 entries for blocks 0 .. ceil(n/B)-1 must be in [0, N); the
 *                 rest are padding (-1 by convention, [P2 prepare_block_tables])
 *                 and are never read.
 *   context_lens  device, int32 [num_seqs]; 0 <= n <= max_context_len and
 *                 ceil(n/B) <= max_blocks_per_seq.
 *   max_context_len  host upper bound of context_lens (sizes the grid);
 *                 at most 2^30.
 *   scale         softmax scale, e.g. 1/sqrt(d); must be positive and finite
 *                 (PA_ERR_INVALID_ARG otherwise): the kernels take the
 *                 maximum of the unscaled scores and scale it, which is the
 *                 maximum of the scaled scores only for a positive scale.
 *   out           device, bf16 [num_seqs, H_q, d]; must not alias inputs.
 *   workspace     device, >= pa_decode_workspace_size(...) bytes, 16-byte
 *                 aligned; may be NULL when that size is 0. Its first 256 KiB
 *                 (the counter header) must be zero before the first call
 *                 that uses it (hipMemset, torch.zeros); every call leaves
 *                 them zero again, so zeroing once per allocation is enough,
 *                 whatever the shapes of later calls. The rest needs no
 *                 initial value. Overlapping calls must not share it. (With
 *                 PA_DEBUG set, a call checks the header and returns
 *                 PA_ERR_WORKSPACE if it is not zero.)
 */
int pa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
              float scale, void* out, void* workspace, size_t workspace_bytes,
              const pa_desc* desc, void* stream);

/*
 * pa_decode_partitioned -- pa_decode with an explicit split-K partition of
 * partition_blocks * 256 tokens per work item, whatever block_size is (whole
 * blocks at block_size 256; 0 = the library's choice, which is what pa_decode
 * uses: estimated on the host from max_context_len, and chosen on the
 * device from the actual lengths, down to a quarter of that estimate, when
 * the dispatch order is computed). A partition longer than
 * ceil(max_context_len / 256) units is cut to that length (it already holds
 * every sequence whole). The result is the same attention for any partition
 * size up to rounding. This runs the partitioned grid (an ordering kernel,
 * the split kernel, a merge kernel). Workspace: pa_decode_workspace_size_ex
 * (the same cut applies; the same header rule as pa_decode).
 */
int pa_decode_partitioned(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_context_len, float scale, void* out, void* workspace,
                          size_t workspace_bytes, int32_t partition_blocks,
                          const pa_desc* desc, void* stream);
size_t pa_decode_workspace_size_ex(const pa_desc* desc, int32_t num_seqs,
                                   int32_t max_context_len, int32_t partition_blocks);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc. Same arguments, result and kernels as pa_decode,
 * minus the workspace: the call uses the library's own device array of
 * PA_NOALLOC_SCRATCH_BYTES (64 MiB; each GPU the library runs on holds one
 * until the process ends) and allocates nothing. A batch whose
 * pa_decode_workspace_size exceeds that returns PA_ERR_WORKSPACE before
 * anything is launched. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race and
 * must not be made. The array starts zeroed (the counter header's required
 * state) and every call leaves its header zero.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                      float scale, void* out, const pa_desc* desc, void* stream);

/*
 * pa_decode_step -- one decode step in one pass: pa_store_kv of each
 * sequence's newest token followed by pa_decode, fused ([P1 §12.6] Attention
 * forward stores K/V, then runs decode attention; [P1 §12.7] runs the
 * per-layer step as a replayed CUDA graph with slot -1 / length 0 padding).
 *
 * For every sequence b with n = context_lens[b] > 0: the newest token
 * (position n-1) is k_new[b], v_new[b]; they are written to cache row
 * slot_mapping[b] (skipped if -1 or out of range) and attended to from the
 * inputs directly, so no kernel of the call reads that row back. Tokens
 * 0 .. n-2 are read from the cache through block_tables. The output is the
 * pa_decode output of the stored cache (up to fp32 summation order). Rows
 * with n == 0 get zeros and store nothing.
 *
 *   q, block_tables, context_lens, max_context_len, scale, out, workspace:
 *                 as pa_decode (same workspace size and preconditions).
 *   k_new, v_new  device, bf16 [num_seqs, H_kv, d], row strides in elements
 *                 (multiples of 8, >= H_kv*d), 16-byte aligned.
 *   k_cache, v_cache  device, written (one row per sequence) and read.
 *   slot_mapping  device, int32 [num_seqs].
 */
int pa_decode_step(const void* q, const void* k_new, int64_t k_row_stride, const void* v_new,
                   int64_t v_row_stride, void* k_cache, void* v_cache,
                   const int32_t* slot_mapping, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                   int32_t max_context_len, float scale, void* out, void* workspace,
                   size_t workspace_bytes, const pa_desc* desc, void* stream);

/*
 * pa_prefill_varlen -- causal attention of a packed batch of new tokens over
 * paged K/V. [P1 §12.6] prefill branch with prefix cache
 * (flash_attn_varlen_func with a block table; the cu_seqlens notes).
 *
 * Sequence b owns queries cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (q_len of
 * them) and k_len = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys, read through
 * block_tables[b] (cached prefix and the new tokens alike, so pa_store_kv of
 * the new tokens runs first). Query i is the token at position
 * k_len - q_len + i and attends to keys 0 .. k_len - q_len + i. q-head h
 * reads kv-head h / (H_q / H_kv). fp32 accumulation, bf16 output.
 *
 *   q             device, bf16 [total_q, H_q, d], contiguous
 *                 (total_q = cu_seqlens_q[num_seqs]).
 *   cu_seqlens_q, cu_seqlens_k  device, int32 [num_seqs + 1], nondecreasing,
 *                 starting at 0, with 0 <= q_len <= k_len per sequence.
 *   max_seqlen_q, max_seqlen_k  host upper bounds of q_len and k_len.
 *   block_tables  device, int32 [num_seqs, max_blocks_per_seq]; entries for
 *                 blocks 0 .. ceil(k_len/B)-1 in [0, N).
 *   scale         as pa_decode: positive and finite (PA_ERR_INVALID_ARG
 *                 otherwise).
 *   out           device, bf16 [total_q, H_q, d].
 */
int pa_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, float scale,
                      void* out, const pa_desc* desc, void* stream);

/*
 * pa_mixed_varlen -- one varlen step that mixes decode rows and prefill rows
 * (decode sequences first, then new or chunked prompts: the mixed batch of a
 * token-budget scheduler; "对照 Nano-vLLM 实现：读懂 vLLM 调度" §2, and the
 * chunk that starts mid-block of "Nano-vLLM 源码解读 - 3. PagedAttention" §4).
 *
 * Same inputs and result as pa_prefill_varlen over all num_seqs sequences,
 * with one extra precondition: the first num_decode_rows sequences have
 * q_len = 1 (cu_seqlens_q[b] = b for b <= num_decode_rows). Those rows run
 * through the split-K decode kernels (k_len from cu_seqlens_k), the rest
 * through the prefill kernel, one launch each on `stream`.
 *
 *   num_decode_rows  0 <= num_decode_rows <= num_seqs.
 *   workspace     device, >= pa_mixed_workspace_size(desc, num_decode_rows,
 *                 max_seqlen_k) bytes (may be NULL when that is 0); the
 *                 decode rows' workspace, under pa_decode's header rule.
 */
size_t pa_mixed_workspace_size(const pa_desc* desc, int32_t num_decode_rows,
                               int32_t max_seqlen_k);
int pa_mixed_varlen(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                    int32_t num_decode_rows, int32_t max_seqlen_q, int32_t max_seqlen_k,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, float scale,
                    void* out, void* workspace, size_t workspace_bytes, const pa_desc* desc,
                    void* stream);

/*
 * pa_build_metadata -- host-side step metadata ([P5 §4]; [P2]
 * prepare_prefill / prepare_decode). Runs on the CPU, reads host memory only.
 *
 * Sequence b computes positions starts[b] .. ends[b]-1 this step (decode:
 * starts = len-1, ends = len). Writes, in batch order:
 *   slot_mapping[...]  the slot of every computed position (two-step map),
 *   cu_seqlens_q[b+1] = cu_seqlens_q[b] + (ends[b] - starts[b]),
 *   cu_seqlens_k[b+1] = cu_seqlens_k[b] + ends[b]   (cached keys count).
 *
 *   block_tables  host, int32 [num_seqs, max_blocks_per_seq].
 *   starts, ends  host, int32 [num_seqs], 0 <= starts <= ends,
 *                 ceil(ends/B) <= max_blocks_per_seq, table entries for
 *                 blocks touched >= 0 (checked: PA_ERR_INVALID_ARG).
 *   slot_mapping  host, int32 [slot_capacity] (>= total new tokens).
 *   cu_seqlens_q, cu_seqlens_k  host, int32 [num_seqs + 1]; either may be NULL.
 * Returns the number of slots written (>= 0) or a PA_ERR_* code.
 */
int64_t pa_build_metadata(const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* starts, const int32_t* ends, int32_t num_seqs,
                          int32_t block_size, int32_t* slot_mapping, int64_t slot_capacity,
                          int32_t* cu_seqlens_q, int32_t* cu_seqlens_k);

/*
 * Block manager -- host-side allocator of the physical blocks, with a
 * chained-hash prefix cache ([P1 §12.8] BlockManager; the worked trace of
 * "对照 Nano-vLLM 实现：读懂 vLLM 调度" §1.2). It produces the block tables
 * (and, through pa_build_metadata, the slots) that the kernels consume.
 * Host memory only; not thread-safe (one caller at a time per manager).
 *
 * State: per block a reference count, the prefix hash of its contents and
 * those token ids; a FIFO of free blocks (taken from the front, returned to
 * the back); an index from prefix hash to block. A full block's hash is
 * xxh64 (seed 0) of the previous block's hash as 8 little-endian bytes (none
 * for block 0) followed by its token ids as int64 little endian. Freeing keeps
 * a block's hash and index entry; handing the block out again drops them.
 * A sequence is held by the caller: its token ids (int64), its block table
 * and how many of its tokens are cached.
 *
 * Return values: >= 0 as documented, or a negative PA_ERR_* code.
 */
typedef struct pa_block_manager pa_block_manager;

/* num_blocks >= 1, block_size >= 1; NULL on bad arguments. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* xxh64 of (prefix as 8 LE bytes if has_prefix) + token_ids[0..n) as int64 LE. */
uint64_t pa_bm_chained_hash(const int64_t* token_ids, int32_t n, uint64_t prefix,
                            int32_t has_prefix);

/* Writes to *num_cached_blocks the leading blocks of the prompt (all but its
 * last block) found in the index with identical tokens; returns 1 if the free
 * FIFO can hold the blocks that are not cached-and-in-use, else 0. */
int32_t pa_bm_can_allocate(pa_block_manager* bm, const int64_t* token_ids, int32_t num_tokens,
                           int32_t* num_cached_blocks);

/* Fill block_table (capacity >= ceil(num_tokens / block_size)): the first
 * num_cached_blocks from the index (shared: count + 1; freed: revived), the
 * rest from the free FIFO. Returns the number of blocks; the caller's cached
 * token count becomes num_cached_blocks * block_size. */
int32_t pa_bm_allocate(pa_block_manager* bm, const int64_t* token_ids, int32_t num_tokens,
                       int32_t num_cached_blocks, int32_t* block_table, int32_t capacity);

/* Drop one reference to each block, last to first; blocks reaching zero go
 * to the back of the free FIFO. */
int32_t pa_bm_deallocate(pa_block_manager* bm, const int32_t* block_table, int32_t n_blocks);

/* 1 if a sequence of seq_len tokens (its newest included) can grow: it needs
 * a free block exactly when seq_len % block_size == 1. */
int32_t pa_bm_can_append(const pa_block_manager* bm, int32_t seq_len);

/* Append a block from the free FIFO when seq_len % block_size == 1; returns
 * the new number of blocks. */
int32_t pa_bm_may_append(pa_block_manager* bm, int32_t seq_len, int32_t* block_table,
                         int32_t n_blocks, int32_t capacity);

/* After a step computed num_scheduled_tokens tokens past num_cached_tokens:
 * hash and index the blocks that became full. Returns how many. */
int32_t pa_bm_hash_blocks(pa_block_manager* bm, const int64_t* token_ids, int32_t num_tokens,
                          const int32_t* block_table, int32_t n_blocks,
                          int32_t num_cached_tokens, int32_t num_scheduled_tokens);

/* Inspection. */
int32_t pa_bm_num_free(const pa_block_manager* bm);
int32_t pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int32_t capacity);
int32_t pa_bm_block_state(const pa_block_manager* bm, int32_t block_id, int32_t* ref_count,
                          uint64_t* hash, int32_t* hashed);
int32_t pa_bm_lookup(const pa_block_manager* bm, uint64_t hash);
int32_t pa_bm_index_entries(const pa_block_manager* bm, uint64_t* hashes, int32_t* block_ids,
                            int32_t capacity);

/* Message for the last nonzero status returned on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version, "major.minor.patch". */
const char* pa_version(void);

/*
 * pa_set_debug -- debug mode on (nonzero) or off (0); returns the previous
 * setting. The initial setting is on when the environment variable PA_DEBUG
 * is set to anything but "0" at the first call that consults it.
 *
 * In debug mode every device entry point, after its host checks, checks the
 * device-resident preconditions its kernels rely on, and returns
 * PA_ERR_INVALID_ARG (pa_last_error() names the first violation found)
 * before launching anything else:
 *   - slot_mapping: every slot in [-1, num_blocks * block_size), no slot
 *     twice ("Nano-vLLM 源码解读 - 3. PagedAttention", §4, -1 = skip);
 *   - lengths: 0 <= n <= the host bound (max_context_len / max_seqlen_k)
 *     and ceil(n / block_size) <= max_blocks_per_seq;
 *   - block tables: the entries of blocks 0 .. ceil(n / block_size) - 1 in
 *     [0, num_blocks) (later entries are padding and never read);
 *   - cu_seqlens_q/k: non-decreasing from 0, k_len >= q_len, q_len <=
 *     max_seqlen_q, k_len <= max_seqlen_k; q_len == 1 for the decode rows of
 *     pa_mixed_varlen.
 * The checks run on the call's stream and the call waits for them (a
 * device-to-host copy and a stream synchronisation), so debug mode is for
 * testing: it cannot be used under graph capture, and debug calls that
 * overlap on one device share one violation record. Outside debug mode a
 * broken entry is only kept from causing an out-of-bounds access.
 */
int pa_set_debug(int on);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
