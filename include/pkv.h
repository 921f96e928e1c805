/*
 * pkv.h - C ABI of libpkv: paged KV-cache attention (decode and multi-token
 * extend) and its block operations for AMD Instinct MI355X (gfx950).
 *
 * The cache of one attention layer is split into fixed-size physical blocks,
 * each holding the keys (one array) or values (a second array) of
 * `block_size` consecutive tokens of one sequence; a per-sequence block table
 * maps logical block j (token positions j*block_size .. j*block_size +
 * block_size - 1) to a physical block anywhere in the pool ("PagedAttention
 * Explained: Virtual Memory for the KV Cache", section "How PagedAttention
 * works", steps 1-3).  The operations on such a cache:
 *
 *   pkv_paged_kv_write     store new tokens' K/V rows in their slots
 *   pkv_paged_attn_decode  attention of one query token per sequence,
 *                          gathering K/V through the block table (step 5)
 *   pkv_paged_attn_extend  the same for several new tokens per sequence
 *                          (prefill, chunked extend), causal
 *   pkv_paged_block_copy   copy whole blocks, the copy step of copy-on-write
 *                          ("Sharing blocks between sequences")
 *   pkv_paged_block_move   copy blocks between a device pool and a pool in
 *                          pinned host memory (swapping, "Preemption and
 *                          scheduling")
 * and, on the host, a block manager (pkv_bm_*) that hands out the slots,
 * tables, copy-on-write pairs and swap pairs these operations consume.
 *
 * Conventions shared by every device entry point
 * ----------------------------------------------
 * Memory.   Every buffer argument is a device pointer to memory the caller
 *           allocated (hipMalloc or a framework allocator) and keeps alive
 *           until the work on `stream` has finished; pkv_paged_block_move
 *           also takes pinned host memory.  The library never allocates,
 *           frees or synchronises; it launches kernels on `stream` (a
 *           hipStream_t passed as void*; NULL is the default stream) and
 *           returns before they run.
 * Layouts.  All arrays are dense and row-major.
 *           cache:  [num_blocks, block_size, kv_heads, head_dim] of `dtype`;
 *                   the row of slot `s` (token offset s % block_size of
 *                   physical block s / block_size) starts at element
 *                   s * kv_heads * head_dim.
 *           q, out: [num_seqs, q_heads, head_dim] of the cache dtype for
 *                   decode; [num_tokens, q_heads, head_dim] for extend.
 *           bf16 is IEEE binary32's upper 16 bits (bfloat16).
 *           Cache, q, k, v, out and workspace pointers must be 16-byte
 *           aligned.
 * Errors.   Arguments are checked on the host before anything is launched;
 *           on any failure nothing is launched and a non-zero pkv_status is
 *           returned, with a message from pkv_last_error().  PKV_ERR_HIP
 *           reports a launch error from the HIP runtime.  Faults while the
 *           kernels run surface at the caller's next synchronisation.
 * Device-side safety.  Values read from device memory (slots, table entries,
 *           copy pairs) cannot be checked on the host.  Kernels never touch
 *           memory outside the pool for an id outside it: such a slot or copy
 *           pair is skipped, decode leaves the positions of such a table
 *           entry's block out of the sequence (the same in every split), and
 *           extend stops the sequence at it.  That is a guard, not a
 *           contract: callers must pass valid ids.
 * Threads.  The library keeps no state between calls apart from the
 *           thread-local last-error message, so calls from several host
 *           threads are safe; ordering between them is the streams'.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                     */
  PKV_ERR_SHAPE = 2,       /* a size is negative, zero or inconsistent       */
  PKV_ERR_DTYPE = 3,       /* unknown dtype code                             */
  PKV_ERR_UNSUPPORTED = 4, /* well-formed, but no kernel is built for it     */
  PKV_ERR_WORKSPACE = 5,   /* split decode needs a (larger) workspace        */
  PKV_ERR_HIP = 6,         /* the HIP runtime rejected a launch              */
  PKV_ERR_ALIGN = 7,       /* a pointer is not 16-byte aligned               */
  PKV_ERR_NO_BLOCKS = 8,   /* block manager: the pool has too few free blocks */
  PKV_ERR_KEY = 9          /* block manager: unknown or duplicate sequence id */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Shape of one layer's paged cache (K and V have the same shape). */
typedef struct {
  int32_t num_blocks; /* physical blocks in the pool, >= 1                  */
  int32_t block_size; /* token slots per block                              */
  int32_t kv_heads;   /* key/value heads per token                          */
  int32_t head_dim;   /* elements per head                                  */
  int32_t dtype;      /* pkv_dtype of the cache, q, k, v and out            */
} pkv_cache_desc;

/*
 * Slot write.  For every token i < num_tokens with 0 <= slot_mapping[i] <
 * num_blocks*block_size, copies k[i] and v[i] (each [kv_heads, head_dim])
 * into the row of slot slot_mapping[i] of k_cache and v_cache, bit for bit.
 * Negative slots are padding and write nothing.  Two tokens naming the same
 * slot in one call leave that slot holding one of them (unspecified which).
 * The cache grows by one such row per new token and layer ("PagedAttention
 * Explained", "The problem: the KV cache is big and unpredictable"); the
 * slot is physical_block * block_size + offset (same page, "How
 * PagedAttention works", steps 2-4).
 *   k, v          device, [num_tokens, kv_heads, head_dim], cache dtype
 *   slot_mapping  device, int64 [num_tokens]
 *   k_cache, v_cache  device, written in place
 * Supported: f32 or bf16 with head_dim * element size a multiple of 16
 * bytes.  num_tokens == 0 is a no-op (pointers may then be NULL).
 */
pkv_status pkv_paged_kv_write(const void* k, const void* v,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              void* k_cache, void* v_cache,
                              const pkv_cache_desc* cache, void* stream);

/*
 * Decode attention over a paged cache.  For each sequence s with length
 * L = seq_lens[s] and each query head h, with G = q_heads / kv_heads and
 * kv head g = h / G:
 *     out[s,h,:] = sum_{t<L} softmax_t(scale * q[s,h,:] . K_s[t,g,:]) V_s[t,g,:]
 * where K_s[t] is the row at offset t % block_size of physical block
 * block_table[s, t / block_size], and likewise V_s ("PagedAttention
 * Explained", "How PagedAttention works", steps 2, 3 and 5; the pages print
 * no formula, and this is standard scaled-dot-product attention of one
 * query token).  L == 0 gives a zero row.  Arithmetic is fp32 (bf16 inputs
 * are widened exactly; the output is rounded to nearest even for bf16).
 *   q            device, [num_seqs, q_heads, head_dim]
 *   k_cache, v_cache  device, read only
 *   block_table  device, int32 [num_seqs, table_width], readable in full;
 *                entries at or past ceil(L / block_size) never address the
 *                pool (entry 0 of every row is read to find shared
 *                blocks, whatever L is; any value is allowed there when
 *                L == 0).  Sequences may share
 *                physical blocks ("Sharing blocks between sequences"): when
 *                consecutive sequences (16 / G of them for bf16 caches) hold
 *                the same leading blocks, those blocks are read once for all
 *                of them.  An entry outside [0, num_blocks) is invalid input;
 *                the kernels never read outside the pool for it, and the
 *                positions of that block are left out of the sequence's
 *                attention (in every split; other sequences are unaffected).
 *   seq_lens     device, int32 [num_seqs]
 *   max_seq_len  host-side bound on every seq_lens[s] (sizes the grid without
 *                reading device memory); a sequence is cut to
 *                min(seq_lens[s], max_seq_len, table_width * block_size)
 *   scale        softmax scale, typically 1/sqrt(head_dim)
 *   out          device, [num_seqs, q_heads, head_dim], written
 *   part_tokens  partition length in tokens (rounded up to a multiple of
 *                16, at most 8192), or 0 for 16.  The call's work -- every
 *                sequence's positions, sequence after sequence -- is cut
 *                into partitions of this length (a sequence's last one may be
 *                shorter), and the partitions into pkv_decode_runs() equal
 *                runs, one workgroup per run and group of up to four kv
 *                heads; a run carries its softmax state across the
 *                partitions of one sequence and may span several sequences.
 *                pkv_decode_partition_tokens() reports the length used.
 *   workspace    device scratch of at least pkv_decode_workspace_size()
 *                bytes when the call has more than one run; may be NULL when
 *                that size is 0.  Contents need no initialisation and are
 *                left undefined.  It holds the plan of the call and, for each
 *                sequence more than one run contributes to, each run's max,
 *                sum and unnormalised output (fp32), merged by a second
 *                kernel in run order.
 * The result does not depend on where the blocks sit in the pool; it can
 * differ in the last bits between batches that split a sequence's work
 * differently (other lengths, other sharing), within the fp32 accumulation.
 * Supported: f32 with head_dim 64, bf16 with head_dim 128; block_size 16 or
 * 32; G in {1, 2, 4, 8}; num_seqs up to about 11000-14000, by G (PKV_ERR_UNSUPPORTED
 * beyond).
 */
pkv_status pkv_paged_attn_decode(const void* q, const void* k_cache,
                                 const void* v_cache,
                                 const pkv_cache_desc* cache,
                                 const int32_t* block_table,
                                 int32_t table_width, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t q_heads,
                                 int32_t max_seq_len, float scale, void* out,
                                 int32_t part_tokens, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Decode attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and result as
 * pkv_paged_attn_decode, with the split workspace taken from a device array
 * of the library (pkv_decode_noalloc_max_workspace() bytes, 64 MiB) instead
 * of caller memory.  Each GPU holds its own array from the first call on it
 * until the process ends.  Calls needing more than that (see
 * pkv_decode_workspace_size) return PKV_ERR_WORKSPACE before any HIP call.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (several streams or threads at once) race and may corrupt each other's
 * results.  Nothing in the array needs clearing between calls.
 */
pkv_status pkv_paged_attn_decode_noalloc(const void* q, const void* k_cache,
                                         const void* v_cache,
                                         const pkv_cache_desc* cache,
                                         const int32_t* block_table,
                                         int32_t table_width,
                                         const int32_t* seq_lens,
                                         int32_t num_seqs, int32_t q_heads,
                                         int32_t max_seq_len, float scale,
                                         void* out, int32_t part_tokens,
                                         void* stream);

/* Bytes of the array pkv_paged_attn_decode_noalloc uses per GPU. */
size_t pkv_decode_noalloc_max_workspace(void);

/*
 * Attention of several new tokens per sequence over a paged cache: a prefill
 * (nothing cached yet), or a chunk of new tokens on top of a cached context.
 * The new tokens' K/V rows must already be in the cache (pkv_paged_kv_write).
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1; with
 * n = query_start[s+1] - query_start[s] and L = seq_lens[s] (new tokens
 * included), query j sits at position p = L - n + j and, for each query head
 * h with kv head g = h / G,
 *     out[row,h,:] = sum_{t<=p} softmax_t(scale * q[row,h,:] . K_s[t,g,:]) V_s[t,g,:]
 * (causal: each new token sees the context and the new tokens up to itself;
 * "PagedAttention Explained", "How PagedAttention works", step 5, and
 * "Preemption and scheduling" for the prefill pass that recomputes a
 * sequence).  A query with p < 0 gets a zero row.  Keys stop at
 * table_width * block_size and at the first table entry outside the pool.
 * Arithmetic: bf16 products summed in fp32 for the logits, softmax in fp32,
 * the weights rounded to bf16 for the weighted sum of V (fp32 accumulation),
 * the output rounded to nearest even bf16.
 *   q, out       device, [num_tokens, q_heads, head_dim]
 *   block_table  device, int32 [num_seqs, table_width]
 *   seq_lens     device, int32 [num_seqs]
 *   query_start  device, int32 [num_seqs + 1], non-decreasing, from 0 to
 *                num_tokens; rows outside [0, num_tokens) are never read or
 *                written whatever it holds
 *   max_query_len host-side bound on every n (sizes the grid); query rows
 *                j >= max_query_len of a sequence are not written
 *   max_seq_len  host-side bound on every seq_lens[s] (sizes the split);
 *                a sequence is cut to min(seq_lens[s], max_seq_len,
 *                table_width * block_size) keys
 *   scale        softmax scale, positive and finite (PKV_ERR_SHAPE otherwise)
 *   part_tokens  split-K partition length in keys (rounded up to a multiple
 *                of 64), or 0 to let the library choose: it splits only when
 *                the batch has too few (sequence, kv head, query tile) units
 *                to fill the device and the keys are long;
 *                pkv_extend_partition_tokens() reports the choice
 *   workspace    device scratch of at least pkv_extend_workspace_size()
 *                bytes when the call splits; may be NULL when that size is
 *                0.  Contents need no initialisation and are left undefined.
 *                It holds each partition's max, sum and normalised output
 *                (all fp32) per query row and head, merged by a second
 *                kernel in a fixed order; rows whose query tile reads no
 *                key past the first partition are stored directly.
 * Supported: bf16 caches with head_dim 128, block_size 16 or 32, G in
 * {1, 2, 4, 8}; anything else returns PKV_ERR_UNSUPPORTED.
 */
pkv_status pkv_paged_attn_extend(const void* q, const void* k_cache,
                                 const void* v_cache,
                                 const pkv_cache_desc* cache,
                                 const int32_t* block_table,
                                 int32_t table_width, const int32_t* seq_lens,
                                 const int32_t* query_start, int32_t num_seqs,
                                 int32_t num_tokens, int32_t q_heads,
                                 int32_t max_query_len, int32_t max_seq_len,
                                 float scale, void* out, int32_t part_tokens,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Partition length (keys) pkv_paged_attn_extend uses for these arguments;
 * the call is split when it is below max_seq_len.  Returns 0 on invalid
 * arguments (see pkv_last_error()).
 */
int32_t pkv_extend_partition_tokens(const pkv_cache_desc* cache,
                                    int32_t num_seqs, int32_t num_tokens,
                                    int32_t q_heads, int32_t max_query_len,
                                    int32_t max_seq_len, int32_t part_tokens);

/*
 * Workspace bytes pkv_paged_attn_extend needs for these arguments (0 when it
 * does not split).  Returns 0 on invalid arguments as well.
 */
size_t pkv_extend_workspace_size(const pkv_cache_desc* cache, int32_t num_seqs,
                                 int32_t num_tokens, int32_t q_heads,
                                 int32_t max_query_len, int32_t max_seq_len,
                                 int32_t part_tokens);

/*
 * Partition length (tokens) pkv_paged_attn_decode uses for these arguments.
 * Returns 0 on invalid arguments (see pkv_last_error()).
 */
int32_t pkv_decode_partition_tokens(const pkv_cache_desc* cache,
                                    int32_t num_seqs, int32_t q_heads,
                                    int32_t max_seq_len, int32_t part_tokens);

/*
 * Runs pkv_paged_attn_decode cuts the work of these arguments into (1: one
 * kernel, no workspace).  Returns 0 on invalid arguments.
 */
int32_t pkv_decode_runs(const pkv_cache_desc* cache, int32_t num_seqs, int32_t q_heads,
                        int32_t max_seq_len, int32_t part_tokens);

/*
 * Workspace bytes pkv_paged_attn_decode needs for these arguments (0 when it
 * has one run).  Returns 0 on invalid arguments as well; check
 * pkv_last_error() when in doubt.
 */
size_t pkv_decode_workspace_size(const pkv_cache_desc* cache, int32_t num_seqs,
                                 int32_t q_heads, int32_t max_seq_len,
                                 int32_t part_tokens);

/*
 * Block copy.  For each pair i < num_pairs, (src, dst) = (pairs[2i],
 * pairs[2i+1]), the whole block dst of k_cache and of v_cache becomes a bit
 * copy of block src: the copy taken before a sequence writes into a block
 * that other sequences still share, after which the writer's table points
 * at dst ("PagedAttention Explained", "Sharing blocks between sequences").
 * Within one call the dst ids must be distinct and no dst may equal a src;
 * pairs with an id outside [0, num_blocks) are skipped.
 *   pairs        device, int64 [num_pairs, 2]
 *   k_cache, v_cache  device, written in place
 * num_pairs == 0 is a no-op.
 */
pkv_status pkv_paged_block_copy(const int64_t* pairs, int32_t num_pairs,
                                void* k_cache, void* v_cache,
                                const pkv_cache_desc* cache, void* stream);

/* ------------------------------------------------------------------------
 * Host block manager (host memory only; no device work, no stream).
 *
 * Owns the bookkeeping of one pool: which physical blocks are free, each
 * block's reference count and filled slots, and each sequence's block table
 * and length.  It implements the pages' allocation rules:
 *   - a sequence of L tokens holds ceil(L / block_size) blocks, all full but
 *     the last ("PagedAttention Explained", "How PagedAttention works",
 *     steps 1-2; "What does PagedAttention change in LLM KV allocation?",
 *     "Calculate unused block space");
 *   - a new block is taken only when the sequence's last block is full,
 *     nothing is reserved ahead (same page, step 4), and blocks return to
 *     the pool when no sequence references them any more;
 *   - sequences may share blocks (fork); a sequence about to write into a
 *     block with reference count > 1 first gets a copy, reported as a
 *     (src, dst) pair for pkv_paged_block_copy, and its table then points at
 *     the copy; the last holder writes in place ("Sharing blocks between
 *     sequences").
 * Every call validates its arguments and either succeeds completely or
 * changes nothing.  A manager is not thread-safe; use one per thread or
 * lock around it.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* Counters of one pool (the measurements "What does PagedAttention change in
 * LLM KV allocation?", "Sharing requires more than allocation", asks for). */
typedef struct {
  int64_t allocated_blocks; /* blocks with reference count > 0               */
  int64_t allocated_slots;  /* allocated_blocks * block_size                 */
  int64_t used_slots;       /* token positions stored, a shared block once   */
  int64_t free_blocks;
  int64_t sequences;        /* live sequences                                */
  int64_t logical_tokens;   /* sum of live sequence lengths                  */
  int64_t copies;           /* copy-on-write pairs handed out so far         */
  int64_t preemptions;      /* sequences released by pkv_bm_preempt so far   */
  int64_t cached_blocks;    /* full blocks findable by the prefix cache      */
  int64_t reused_blocks;    /* blocks pkv_bm_add_cached has reused so far    */
  int64_t host_blocks_used; /* swap space holding swapped-out blocks         */
  int64_t swapped_sequences;
  int64_t swap_outs;        /* pkv_bm_swap_out calls so far                  */
  int64_t unused_slots;     /* allocated_slots - used_slots: slots reserved
                               but holding no token ("What does PagedAttention
                               change in LLM KV allocation?", "Calculate
                               unused block space")                        */
  double waste_fraction;    /* unused_slots / allocated_slots (0 if none)    */
} pkv_bm_stats;

/* Create a manager for num_blocks blocks of block_size slots.  free_order
 * (host, num_blocks entries, a permutation of 0..num_blocks-1) sets the
 * order in which free blocks are handed out; NULL means ascending ids.
 * Released blocks go to the back of the free list. */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* free_order, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Start an empty sequence under a new id. */
pkv_status pkv_bm_add(pkv_block_manager* bm, int64_t seq);

/* Start `child` as a copy of `parent` that shares all of its blocks
 * (reference counts + 1); used for parallel samples, beams and shared
 * prompt prefixes ("Sharing blocks between sequences"). */
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Store n new tokens of `seq`.  slots (host, n entries) receives each new
 * token's slot (physical_block * block_size + offset) for
 * pkv_paged_kv_write; copies (host, copies_cap x 2) receives the (src, dst)
 * block copies the writes need, in order, and *n_copies their number (at
 * most one per call).  Fails with PKV_ERR_NO_BLOCKS, changing nothing, when
 * the pool cannot supply the blocks the call needs. */
pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int32_t n,
                         int64_t* slots, int64_t* copies, int32_t copies_cap,
                         int32_t* n_copies);

/* Prefix cache.  Requests with identical prefixes can reuse the same
 * physical blocks, but a paged layout does not find them by itself ("What
 * does PagedAttention change in LLM KV allocation?", "Sharing requires more
 * than allocation").  Here a full block is findable under the whole token
 * prefix it completes while some sequence holds it; lookups use a 64-bit
 * hash chain over the token ids and confirm every hit against the block's
 * stored token ids and its predecessor's hash.
 *
 * pkv_bm_add_cached starts `seq` for a request of n token ids, reusing the
 * longest run of findable full blocks from its start (reference counts + 1);
 * *reused_tokens receives their token count (a multiple of block_size).
 * The rest of the request is for the caller to store with
 * pkv_bm_append_tokens, which works like pkv_bm_append and registers the
 * blocks that become full.  A sequence that gets pkv_bm_append (no token ids)
 * stops registering blocks.  The first block registered under a prefix keeps
 * the entry; it is dropped when the block returns to the pool. */
pkv_status pkv_bm_add_cached(pkv_block_manager* bm, int64_t seq,
                             const int32_t* tokens, int32_t n,
                             int32_t* reused_tokens);
pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, int64_t seq,
                                const int32_t* tokens, int32_t n,
                                int64_t* slots, int64_t* copies,
                                int32_t copies_cap, int32_t* n_copies);

/* Blocks pkv_bm_append(seq, n) would take from the pool (new blocks plus a
 * copy-on-write copy if the last block is shared and not full). */
pkv_status pkv_bm_blocks_needed(const pkv_block_manager* bm, int64_t seq,
                                int32_t n, int32_t* blocks);

/* Release a finished sequence; blocks nobody references return to the pool
 * (for a swapped-out sequence, its host blocks return to the swap space). */
pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq);

/* Release a sequence the scheduler preempts (its cache is dropped, to be
 * recomputed or restored later; "PagedAttention Explained", "Preemption and
 * scheduling"); counted in pkv_bm_stats.preemptions. */
pkv_status pkv_bm_preempt(pkv_block_manager* bm, int64_t seq);

/* Preemption by swapping ("PagedAttention Explained", "Preemption and
 * scheduling").  pkv_bm_set_swap_space gives the manager host_blocks blocks
 * of host swap space (once).  pkv_bm_swap_out moves `seq` out: every block
 * of its table, in order, goes to its own free host block, the (device,
 * host) pairs are written to pairs (host, cap x 2) for pkv_paged_block_move
 * and *n receives their number; the sequence's device references are
 * dropped (blocks other sequences share stay for them).  pkv_bm_swap_in
 * brings it back into fresh device blocks and writes the (host, device)
 * pairs.  A swapped sequence cannot grow or be forked; sharing and prefix
 * registration do not survive a swap.  Both fail with PKV_ERR_NO_BLOCKS,
 * changing nothing, when the target pool is short, and with PKV_ERR_SHAPE
 * when cap is below the sequence's block count. */
pkv_status pkv_bm_set_swap_space(pkv_block_manager* bm, int32_t host_blocks);
pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq, int64_t* pairs,
                           int32_t cap, int32_t* n);
pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq, int64_t* pairs,
                          int32_t cap, int32_t* n);

/* Length (tokens) of a sequence. */
pkv_status pkv_bm_length(const pkv_block_manager* bm, int64_t seq, int32_t* len);

/* Block tables of n sequences as int32 [n, width] in host memory, entries
 * past each sequence's blocks set to -1; PKV_ERR_SHAPE if a sequence holds
 * more than width blocks. */
pkv_status pkv_bm_table(const pkv_block_manager* bm, const int64_t* seqs,
                        int32_t n, int32_t width, int32_t* table);

pkv_status pkv_bm_get_stats(const pkv_block_manager* bm, pkv_bm_stats* out);

/* Capacity of a pool for a list of request lengths taken in order:
 * *paged = how many leading requests fit when each takes ceil(len /
 * block_size) blocks; *contiguous = how many fit when each reserves
 * reserve_len token slots up front (the scheme paged blocks replace,
 * "PagedAttention Explained", table "Contiguous allocation vs
 * PagedAttention").  Lengths above reserve_len are an error. */
pkv_status pkv_capacity(int64_t num_blocks, int32_t block_size,
                        const int32_t* lens, int32_t n, int32_t reserve_len,
                        int32_t* paged, int32_t* contiguous);

/*
 * Block move between two pools of the same block shape and dtype (num_blocks
 * may differ): for each pair i, block pairs[2i+1] of (dst_k, dst_v) becomes
 * a bit copy of block pairs[2i] of (src_k, src_v).  Either pool may live in
 * pinned host memory (hipHostMalloc, or a torch tensor with pin_memory):
 * this moves a preempted sequence's blocks to host memory and back
 * ("PagedAttention Explained", "Preemption and scheduling"; the pairs come
 * from pkv_bm_swap_out / pkv_bm_swap_in).  `pairs` may be device or pinned
 * host memory.  Each pointer is checked with the HIP runtime first: pinned
 * host memory is reached through its device mapping, and pageable host
 * memory is refused with PKV_ERR_UNSUPPORTED (no launch).  Pairs naming a
 * block outside its pool are skipped.  Within one call the destination ids
 * must be distinct, and when source and destination are the same pool no
 * destination may also be a source (as for pkv_paged_block_copy).
 */
pkv_status pkv_paged_block_move(const int64_t* pairs, int32_t num_pairs,
                                const void* src_k, const void* src_v,
                                const pkv_cache_desc* src, void* dst_k,
                                void* dst_v, const pkv_cache_desc* dst,
                                void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string, e.g. "pkv 0.1.0 gfx950". */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
