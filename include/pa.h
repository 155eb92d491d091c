/*
 * pa.h -- C ABI of libpa: paged KV-cache attention for AMD MI355X (gfx950).
 *
 * The method (PagedAttention) keeps each sequence's keys and values in
 * fixed-size blocks (16 tokens by default) scattered through one pool, and
 * reaches them through a per-sequence block table; attention reads the blocks
 * as if they were one contiguous sequence ("Inside vLLM: How PagedAttention
 * Changes Python LLM Inference at the Systems Level", section "PagedAttention:
 * What the OS Figured Out Decades Ago"; "vLLM PagedAttention: Reducing KV
 * Cache Memory Waste", section "How PagedAttention Works").  Sequences that
 * branch from one prompt share its blocks by reference count; a shared block
 * is copied only when a branch writes into it ("Inside vLLM ...", section
 * "Copy-on-Write Makes Beam Search Cheap").
 *
 * Conventions for every call
 *   - Every call returns pa_status; nothing throws or aborts across the ABI.
 *     On failure pa_last_error() describes the cause (thread-local string,
 *     valid until this thread's next pa_* call).
 *   - Device calls take DEVICE pointers owned by the caller, enqueue their
 *     kernels on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) and return after the launch without synchronising.  Arguments
 *     are checked on the host before anything is launched; a rejected call
 *     launches nothing.
 *   - The library never allocates device memory.
 *   - dtype: K, V, Q and outputs share one 16-bit storage type; arithmetic is
 *     fp32 (MFMA fp32 accumulate); outputs are rounded to nearest even.
 *   - Supported: head_dim 64 or 128, block_size 16, fp16 or bf16,
 *     num_q_heads a multiple of num_kv_heads.  Anything else: PA_ENOTSUP.
 *   - Pointers to 16-bit data must be 16-byte aligned.
 *
 * KV cache storage (one pair of tensors per layer, caller-allocated):
 *   k_cache  [num_blocks][num_kv_heads][head_dim / 32][block_size][32]
 *   v_cache  [num_blocks][num_kv_heads][block_size / 4][head_dim][4]
 * Token t of a sequence lives in block block_table[t / block_size], slot
 * t % block_size; its storage address ("slot") is block * block_size + slot.
 * Element d of a key sits in 32-dim chunk d / 32 at position d % 32 of its
 * slot's 64-byte row; element d of a value in slot s sits at [s / 4][d][s % 4]
 * (groups of four slots, dim-major within a group).  One (block, kv head)
 * tile is contiguous in both tensors (4 KiB at D = 128).  The layouts serve
 * the matrix-core operands of the attention kernels: one load of the K
 * operand for a 32-dim step reads a whole contiguous 1 KiB chunk (16 keys x
 * 32 dims), and a P.V operand (four consecutive keys of one dim) is one
 * 8-byte piece of V.  A single new token's values then fill a quarter of each
 * 32-byte sector they touch (D / 4 sectors per head) instead of 2 bytes of
 * each of D sectors, which keeps the memory's read-modify-write of partly
 * written sectors small when decode tokens are written.
 *
 * Device data (block ids, slots, context lengths) is checked inside the
 * kernels: an out-of-range slot or pair is skipped by the write and copy
 * kernels, and a sequence with an out-of-range block id or context length
 * gets NaN output rows.  No call reads or writes outside the buffers it is
 * given when the sizes passed to it are right.
 *
 * Cache slots past a sequence's length may hold anything, NaN included; they
 * never reach a result.  Inf or NaN in a key or value a sequence does hold
 * reaches the rows that attend to it, as in the definition; in chunked
 * prefill an inf or NaN value can also reach some of the (at most 95) rows
 * just before the first row that attends to it, those computed with its
 * 64-key tile in the same 32-row group (their weight for it is 0, and
 * 0 * inf is NaN in the matrix product).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,   /* bad argument (null pointer, negative size, bad id)   */
  PA_ENOMEM = 2,   /* block pool exhausted (pool calls only)                */
  PA_EHIP = 3,     /* a HIP runtime call or kernel launch failed            */
  PA_ENOTSUP = 4   /* valid but unsupported shape / dtype / alignment      */
} pa_status;

typedef enum { PA_FP16 = 0, PA_BF16 = 1 } pa_dtype;

/* Thread-local description of the last failure on this thread ("" if none). */
const char* pa_last_error(void);
/* Library version string, e.g. "libpa 0.1 gfx950". */
const char* pa_version(void);

/* ------------------------------------------------------------------------
 * Slot-mapped KV write.  New tokens' keys and values are appended to their
 * sequence's blocks as they are generated ("Inside vLLM ...", section
 * "PagedAttention: What the OS Figured Out Decades Ago").
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim], token i starting at
 *                 element i * src_token_stride (heads contiguous after it);
 *                 src_token_stride >= num_kv_heads*head_dim, multiple of 8.
 *   k_cache, v_cache   the caches above, num_blocks blocks each.
 *   slot_mapping  [num_tokens] int64, device: storage slot of token i, or a
 *                 negative value to skip the token.  Slots must be distinct
 *                 (two tokens writing one slot race).
 * Bit-exact copy: the cache holds exactly the bits of k and v afterwards.
 * num_tokens == 0 launches nothing and returns PA_OK.
 * ---------------------------------------------------------------------- */
pa_status pa_write_kv(const void* k, const void* v, int64_t src_token_stride,
                      void* k_cache, void* v_cache, int64_t num_blocks,
                      const int64_t* slot_mapping, int32_t num_tokens,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Whole-block copies for copy-on-write ("Inside vLLM ...", section
 * "Copy-on-Write Makes Beam Search Cheap").
 *   pairs   [num_pairs][2] int32, device: (src, dst) physical block ids.
 * Copies K and V of every KV head of src to dst, bit-exact.  Pairs run
 * concurrently: a dst must not be the src or dst of another pair.
 * ---------------------------------------------------------------------- */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks,
                         const int32_t* pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Swapping blocks between the device cache and host memory: under memory
 * pressure a sequence's blocks can move to CPU memory and come back later,
 * at host-link cost ("Inside vLLM ...", section "Python LLM Inference
 * Optimization with vLLM: Parameters That Actually Matter").
 *   host_k, host_v  pinned host memory (hipHostMalloc, e.g. a torch tensor
 *                   made with pin_memory=True) of num_host_blocks blocks in
 *                   the caches' layout; the kernel reads or writes it
 *                   directly over the host link.  Anything else is PA_EINVAL.
 *   pairs           [num_pairs][2] int32, device: (src, dst) block ids,
 *                   PA_SWAP_OUT (device -> host): (device, host);
 *                   PA_SWAP_IN  (host -> device): (host, device).
 * Copies K and V of every KV head, bit-exact, in one launch; ids out of
 * range skip the pair.  Pairs run concurrently: a dst must not be the src or
 * dst of another pair.  Stream-ordered like every device call: enqueue a
 * swap-out before anything that reuses the released device blocks.
 * ---------------------------------------------------------------------- */
#define PA_SWAP_OUT 0
#define PA_SWAP_IN 1
pa_status pa_swap_blocks(void* k_cache, void* v_cache, int64_t num_blocks,
                         void* host_k, void* host_v, int64_t num_host_blocks,
                         const int32_t* pairs, int32_t num_pairs, int32_t direction,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Paged decode attention: one query token per sequence attends to all
 * context_lens[s] keys of its sequence (the newest token's K/V must already be
 * written), read through the sequence's block table as if its blocks were
 * contiguous ("Inside vLLM ...", section "PagedAttention: What the OS Figured
 * Out Decades Ago").  This step is bound by memory bandwidth ("PagedAttention
 * in vLLM: A Throughput Settings Guide", section "Continuous Batching Keeps
 * the GPU Busy").  Query head h reads KV head h / (num_q_heads /
 * num_kv_heads) (grouped-query attention; the pages do not treat it).
 *
 *   out, q          [num_seqs][num_q_heads][head_dim], contiguous.
 *   num_blocks      blocks in each cache; must be >= 1 when num_seqs > 0
 *                   (PA_EINVAL otherwise).
 *   block_tables    [num_seqs][bt_stride] int32, device.
 *   context_lens    [num_seqs] int32, device; 0 gives a zero row; a length
 *                   above max_context_len or bt_stride*block_size gives NaN.
 *   max_context_len host-side upper bound of context_lens (sizes the grid).
 *   scale           softmax scale (usually 1/sqrt(head_dim)).
 *   partition_size  long contexts are cut into partitions of at most this
 *                   many tokens (ceil(L / partition_size) partitions of
 *                   nearly equal size) whose states are merged by
 *                   log-sum-exp.  A small batch gives each partition its own
 *                   workgroup and merges in a second kernel, through the
 *                   workspace; a batch that already gives >= 1024 (sequence,
 *                   KV head) work items, with head groups of at most 8 query
 *                   heads and max_context_len <= 4096, merges on chip in a
 *                   single pass.  0 = library default
 *                   (pa_default_partition_size: no split when num_seqs *
 *                   num_kv_heads already gives >= 1024 work items, else just
 *                   enough split to reach that many).  Multiple of 16,
 *                   <= 4096.
 *                   The result for a sequence depends only on its own data
 *                   and on the partition size, never on the rest of the batch
 *                   (both merges compute the same bits).
 *   workspace       device scratch of at least pa_decode_workspace_size()
 *                   bytes for the same arguments (may be NULL if that size is
 *                   0; the single pass leaves it untouched); contents need not
 *                   be initialised.
 * Launch limits (PA_ENOTSUP beyond them): num_seqs <= 65535, and each grid's
 * work-item count below 2^32 (partitions x num_seqs x head groups of up to 16
 * query heads x 64 x waves for the partition kernel, num_seqs x num_q_heads x
 * 64 for the merge kernel).
 * ---------------------------------------------------------------------- */
int32_t   pa_default_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_context_len);
pa_status pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_size,
                                   int32_t num_kv_heads, size_t* bytes);
/* How pa_decode would run for these sizes, without launching anything:
 *   partition_out  the partition size it uses (partition_size, or the library
 *                  default when 0), in tokens;
 *   merge_out      PA_MERGE_NONE (one partition per sequence),
 *                  PA_MERGE_ON_CHIP (partition states merged in LDS, one
 *                  kernel) or PA_MERGE_TWO_PASS (partition kernel, then the
 *                  log-sum-exp merge kernel through the workspace);
 *   waves_out      waves that interleave the blocks of one partition (4 or 8).
 * The choice never changes results (both merges give the same bits); it is
 * reported for callers that size work or check which kernels run.  Any output
 * pointer may be NULL.  Errors as pa_decode's size checks. */
#define PA_MERGE_NONE 0
#define PA_MERGE_ON_CHIP 1
#define PA_MERGE_TWO_PASS 2
pa_status pa_decode_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                         int32_t* partition_out, int32_t* merge_out, int32_t* waves_out);
pa_status pa_decode(void* out, const void* q,
                    const void* k_cache, const void* v_cache, int64_t num_blocks,
                    const int32_t* block_tables, int32_t bt_stride,
                    const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_context_len, float scale,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode without allocation, for callers that cannot allocate device
 * memory or pass one in: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results (bit for bit)
 * and errors as pa_decode, without the workspace: when the partitions are
 * merged in two passes their states go to a static scratch array of
 * PA_DECODE_STATIC_SCRATCH_BYTES that the library holds on each device it
 * runs on until the process ends.  A call that would need more returns
 * PA_ENOTSUP before launching anything; the single pass, and calls with one
 * partition per sequence, need none.  The scratch of the current device is
 * used, so `stream` must belong to it.  Every call on one device shares that
 * scratch: calls that may overlap on one device (other streams, other
 * threads) race and must be serialised by the caller.  The call allocates
 * nothing; its first use on a device looks the scratch's address up once.
 * ---------------------------------------------------------------------- */
#define PA_DECODE_STATIC_SCRATCH_BYTES (16u << 20)
pa_status pa_decode_static(void* out, const void* q,
                           const void* k_cache, const void* v_cache, int64_t num_blocks,
                           const int32_t* block_tables, int32_t bt_stride,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_context_len, float scale,
                           int32_t partition_size, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Chunked prefill: the scheduler serves decode first and fills the rest of
 * the step's token budget with prefill chunks ("PagedAttention in vLLM: A
 * Throughput Settings Guide", section "Tuning Batching, Prefill, and Cache").
 * Chunk c continues its own sequence: its n_c query rows are the sequence's
 * newest tokens, already written to the cache, so row j (0-based) sits at
 * position seq_lens[c] - n_c + j and attends keys 0 .. seq_lens[c] - n_c + j.
 *
 *   out, q        [total_rows][num_q_heads][head_dim] packed; chunk c owns
 *                 rows q_start_loc[c] .. q_start_loc[c+1]-1.
 *   num_blocks    blocks in each cache; must be >= 1 when there is a chunk
 *                 with rows (PA_EINVAL otherwise).
 *   q_start_loc   [num_chunks+1] int32, device, non-decreasing, from 0.
 *   seq_lens      [num_chunks] int32, device: keys of chunk c's sequence
 *                 after the chunk, >= n_c.
 *   block_tables  [num_chunks][bt_stride] int32, device.
 *   max_q_len     host bound on n_c (sizes the grid).  A chunk with more
 *                 rows gets NaN in every row the grid covers (at least its
 *                 first max_q_len rows); rows beyond those are not written.
 *   max_seq_len   host bound on seq_lens (a longer sequence gets NaN rows).
 * Launch limits (PA_ENOTSUP beyond them): num_chunks <= 65535 and
 * ceil(max_q_len / 64) * 512 < 2^32 (about 5.4e8 rows).
 * ---------------------------------------------------------------------- */
pa_status pa_prefill_chunk(void* out, const void* q,
                           const void* k_cache, const void* v_cache, int64_t num_blocks,
                           const int32_t* block_tables, int32_t bt_stride,
                           const int32_t* q_start_loc, const int32_t* seq_lens,
                           int32_t num_chunks, int32_t max_q_len, int32_t max_seq_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, float scale, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Host-side block pool: refcounted blocks, per-sequence block tables and
 * copy-on-write ("Inside vLLM ...", sections "PagedAttention: What the OS
 * Figured Out Decades Ago", "Copy-on-Write Makes Beam Search Cheap" and
 * "Python LLM Inference Optimization with vLLM: Parameters That Actually
 * Matter", where the allocator is the pool's page-frame table).
 * The pool is library-owned, not thread-safe (one owner thread), and holds
 * only ids: the caller moves the data with pa_copy_blocks / pa_write_kv.
 *
 * Allocation order: the free list is a LIFO stack whose initial order is a
 * Fisher-Yates shuffle of [0, num_blocks) driven by SplitMix64(seed)
 * (seed 0: identity order); the first block handed out is order[0]; a freed
 * block goes on top and is handed out next.  Sequence ids count up from 1.
 * ---------------------------------------------------------------------- */
typedef struct pa_pool pa_pool;

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, uint64_t seed,
                         pa_pool** out);

/* Prefix caching ("Inside vLLM ...", section "PagedAttention in a Python RAG
 * Application" and its question on how prefix caching works; "PagedAttention
 * in vLLM: A Throughput Settings Guide", section "Tuning Batching, Prefill,
 * and Cache"): the content of each full block is keyed, and a request whose
 * leading whole blocks match content already computed reuses those physical
 * blocks instead of recomputing them.
 *   - A block's content is its token ids and everything before them: its key
 *     is (the content of the block before it, its token ids), compared
 *     exactly (the hash only indexes the table).
 *   - A block is registered when its last slot is appended through
 *     pa_seq_append_tokens, if the block before it is registered (or it is
 *     the sequence's first block).  Tokens appended by pa_seq_append have no
 *     ids, so their blocks are never registered.
 *   - When a registered block's references drop to zero it is not freed: it
 *     goes to the tail of an LRU list of cached blocks (pa_pool_num_cached).
 *     A later match takes it back; allocation uses the free stack first and
 *     only then evicts the head of that list, which forgets its content.
 * Without PA_POOL_PREFIX_CACHING the pool behaves exactly as pa_pool_create's
 * (and pa_seq_append_tokens never reuses). */
#define PA_POOL_PREFIX_CACHING 1u
/* flags: 0 or PA_POOL_PREFIX_CACHING; other bits give PA_EINVAL.
 * num_host_blocks: size of the host swap space (0: no swapping). */
pa_status pa_pool_create_ex(int32_t num_blocks, int32_t block_size, uint64_t seed,
                            uint32_t flags, int32_t num_host_blocks, pa_pool** out);
/* Cached blocks (no references, content kept); -1 if pool is NULL. */
int32_t   pa_pool_num_cached(const pa_pool* pool);
/* Free host swap blocks; -1 if pool is NULL. */
int32_t   pa_pool_num_free_host(const pa_pool* pool);
void      pa_pool_destroy(pa_pool* pool);                 /* NULL-safe */
int32_t   pa_pool_num_free(const pa_pool* pool);          /* -1 if pool is NULL */
int32_t   pa_pool_num_blocks(const pa_pool* pool);        /* -1 if pool is NULL */
int32_t   pa_block_refcount(const pa_pool* pool, int32_t block); /* -1 if out of range */

/* New empty sequence (0 tokens, 0 blocks). */
pa_status pa_seq_create(pa_pool* pool, int64_t* seq_id);
/* New sequence sharing every block of `parent` (each gains a reference). */
pa_status pa_seq_fork(pa_pool* pool, int64_t parent, int64_t* child);
/* Append n_tokens tokens.  Writes their storage slots to slot_mapping_out
 * [n_tokens] (host, caller-owned).  A copy-on-write copy happens exactly when
 * a token goes into a partly filled last block whose refcount is above one:
 * the sequence gets a fresh block and (old, new) is written to cow_pairs_out
 * [cow_cap][2] (host); at most one pair per call, so cow_cap >= 1 suffices.
 * All-or-nothing: if the free blocks cannot cover the new blocks plus the
 * copy, returns PA_ENOMEM and changes nothing. */
pa_status pa_seq_append(pa_pool* pool, int64_t seq, int32_t n_tokens,
                        int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                        int32_t cow_cap, int32_t* n_cow);
/* pa_seq_fork / pa_seq_free for n sequences in one call, in order
 * (children_out[n], host).  They stop at the first failure (PA_EINVAL,
 * unknown or swapped-out sequence) with the earlier ones applied; *n_done
 * counts those. */
pa_status pa_seq_fork_many(pa_pool* pool, const int64_t* parents, int32_t n,
                           int64_t* children_out, int32_t* n_done);
pa_status pa_seq_free_many(pa_pool* pool, const int64_t* seqs, int32_t n, int32_t* n_done);
/* pa_seq_append for n sequences in one call, in order: seqs[i] gets
 * n_tokens[i] tokens.  Slots are written back to back into slot_mapping_out
 * (sum of n_tokens entries), copy-on-write pairs into cow_pairs_out
 * [cow_cap][2] in the order they happen (at most one per sequence).  Each
 * sequence's append is all-or-nothing as in pa_seq_append; the call stops at
 * the first sequence that fails, leaving the earlier ones applied, and
 * *n_done counts the sequences applied.  Saves a call per sequence in a
 * decode or beam-search step. */
pa_status pa_seq_append_many(pa_pool* pool, const int64_t* seqs, const int32_t* n_tokens,
                             int32_t n, int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                             int32_t cow_cap, int32_t* n_cow, int32_t* n_done);
/* pa_seq_append with the tokens' ids (token_ids[n_tokens], host).  With
 * prefix caching, when the sequence ends on a block boundary, the longest run
 * of leading whole blocks of the new tokens (at most max_hit_tokens tokens)
 * whose content is cached is reused: those blocks join the table (one more
 * reference each), their tokens get slot -1 (their K/V is already stored;
 * pa_write_kv skips them) and *n_hit counts them.  The rest is appended as by
 * pa_seq_append.  Callers that must compute the last token pass
 * max_hit_tokens = n_tokens - 1.  All-or-nothing over the free stack plus the
 * cached blocks, less the cached blocks this call reuses. */
pa_status pa_seq_append_tokens(pa_pool* pool, int64_t seq, const int32_t* token_ids,
                               int32_t n_tokens, int32_t max_hit_tokens,
                               int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                               int32_t cow_cap, int32_t* n_cow, int32_t* n_hit);
/* Drop one reference from every block of seq, in table order; blocks that
 * reach zero go back on the free stack in that order (registered blocks, with
 * prefix caching, to the tail of the cached list instead). */
pa_status pa_seq_free(pa_pool* pool, int64_t seq);
/* Swapping a whole sequence (see pa_swap_blocks).  Host swap blocks come
 * from a LIFO stack whose initial order is the identity (host block 0 first).
 * pa_seq_swap_out: for each block in table order takes a host block, writes
 * (device, host) to pairs_out [cap][2] (host) and drops the device block's
 * reference (a shared block stays with its other holders; one reaching zero
 * is released as by pa_seq_free).  The sequence then holds no device blocks
 * (an empty table, its token count kept) and cannot append or fork until
 * swapped in.  pa_seq_swap_in: takes a device block per host block (free
 * stack, then eviction of cached blocks), writes (host, device), returns the
 * host blocks to their stack in table order; the new blocks are not
 * registered for prefix caching.  Both are all-or-nothing (PA_ENOMEM) and
 * need cap >= the sequence's block count (else PA_EINVAL, nothing changed).
 * pa_seq_free of a swapped-out sequence returns its host blocks. */
pa_status pa_seq_swap_out(pa_pool* pool, int64_t seq, int32_t* pairs_out, int32_t cap,
                          int32_t* n_pairs);
pa_status pa_seq_swap_in(pa_pool* pool, int64_t seq, int32_t* pairs_out, int32_t cap,
                         int32_t* n_pairs);
/* Block table of one sequence: up to cap ids into out (host). */
pa_status pa_seq_block_table(const pa_pool* pool, int64_t seq, int32_t* out, int32_t cap,
                             int32_t* n_blocks, int32_t* n_tokens);
/* Block tables of n sequences as rows of a [n][stride] int32 host array,
 * unused entries set to pad; context lengths into ctx_out[n] (may be NULL).
 * PA_EINVAL if a table is longer than stride. */
pa_status pa_seq_block_tables(const pa_pool* pool, const int64_t* seq_ids, int32_t n,
                              int32_t* out, int32_t stride, int32_t pad, int32_t* ctx_out);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
