/*
 * pa.h -- C ABI of the paged key/value cache and decode-attention library
 * for AMD MI355X (gfx950).
 *
 * What the library computes (sources, by page title and section):
 *
 *  - "vLLM PagedAttention and continuous batching" (netleverage.com),
 *    section "PagedAttention: fixed blocks, non-contiguous physical memory":
 *    a sequence's keys and values live in fixed-size blocks of B token slots;
 *    a per-sequence block table maps logical block j to a physical block; a
 *    block engine slices one contiguous device allocation into physical
 *    blocks; a new physical block is taken only when the previous one is full.
 *  - same article, section "Sharing with reference counts and
 *    copy-on-write": each physical block carries a reference count; a write
 *    into a block with count > 1 takes a new block, copies that block and
 *    drops the old count; a block at count 0 is released; the policies are
 *    fork, append and free; the kernel sees only physical block ids.
 *  - same article, section "The kernel page, and what the 2023 runs
 *    measured": a single-query decode kernel with separate key and value
 *    caches and a compile-time block size.
 *  - "Serving Language Models Within a Memory Budget" (auturnal.com),
 *    section 6 and eq. (4): dense scaled-dot-product attention evaluated
 *    block by block with a running maximum and normaliser; the same rescale
 *    merges partial results.
 *  - "PagedAttention and Online Inference" (auturnal.com), section 1:
 *    grouped-query attention has fewer key/value heads than query heads.
 *    Query head h reads key/value head floor(h / G), G = Hq / Hkv.
 *
 * Beyond the decode step (each declared below with its source):
 *  - beam selection as forks and frees (pa_seq_reorder);
 *  - preemption by swapping a group of sequences to a host pool and back
 *    (pa_move_blocks, pa_swap_blocks);
 *  - several causal queries per sequence, for chunked prefill and
 *    speculative verification (pa_multi_query_attention);
 *  - decode that reads a prefix shared by parallel samples or beams once
 *    per group (pa_prefix_groups, pa_decode_attention_grouped).
 *
 * Conventions for every call:
 *  - Return value: PA_OK (0) or a negative pa_status.  No call aborts or
 *    throws across the ABI.  After a failure, pa_last_error() returns a
 *    message for the calling thread (valid until that thread's next call).
 *  - "host" pointers are CPU memory; "device" pointers are GPU memory on
 *    the device that is current for the calling thread.  The caller owns
 *    every buffer it passes; the library never frees caller memory.
 *  - Device operations are asynchronous on the given HIP stream (0 = the
 *    null stream) and return after enqueueing.  Launch failures return
 *    PA_ERR_HIP with the HIP error string in pa_last_error().
 *  - The host block manager is synchronous and not thread-safe: serialise
 *    calls that use the same pool.
 *  - Storage type: Q, K, V and the attention output share one 16-bit type
 *    (pa_dtype).  Arithmetic is fp32; the output is rounded to nearest even.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same declaration as the HIP runtime's own; repeating it is legal. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* a null pointer, bad size, bad id, misalignment */
  PA_ERR_OUT_OF_BLOCKS = -2, /* the free list is empty; manager state unchanged */
  PA_ERR_UNSUPPORTED = -3,   /* a shape with no compiled kernel (see below)   */
  PA_ERR_HIP = -4            /* a HIP runtime call or launch failed            */
} pa_status;

typedef enum { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

typedef struct pa_pool pa_pool; /* opaque, host-owned */

typedef struct {
  int64_t allocs;          /* blocks taken from the free list            */
  int64_t cows;            /* copy-on-write block copies requested       */
  int64_t releases;        /* blocks returned to the free list           */
  int32_t live_blocks;     /* blocks with refcount > 0 now               */
  int32_t live_high_water; /* largest live_blocks seen                   */
  int32_t free_blocks;     /* blocks on the free list now                */
  int32_t num_blocks;      /* P                                          */
} pa_pool_stats;

/* ---------------------------------------------------------------------
 * Pool ("block engine")
 * ------------------------------------------------------------------- */

/* Bytes of device memory a pool of P blocks needs:
 *   L * 2 * P * Hkv * B * d * 2
 * (key/value cache bytes of eq. (1) of the memory-budget page with P*B
 * retained slots).  Returns 0 if any argument is not positive or the
 * product overflows. */
size_t pa_pool_bytes(int L, int Hkv, int d, int B, int P, pa_dtype dtype);

/* Create a pool over caller-provided device memory: the "block engine" of
 * "vLLM PagedAttention and continuous batching", section "PagedAttention:
 * fixed blocks, non-contiguous physical memory" (one contiguous allocation
 * sliced into physical blocks of B token slots; separate key and value
 * caches, section "The kernel page").
 *   dev_base  : device, 256-byte aligned, at least pa_pool_bytes(...) bytes.
 *               Layout, layer-major with separate key and value slabs:
 *                 K of layer l at dev_base + (2l)   * slab
 *                 V of layer l at dev_base + (2l+1) * slab
 *                 slab = P * Hkv * B * d * 2 bytes, each slab [P][Hkv][B][d].
 *   free_order: host [P], a permutation of 0..P-1 that seeds the FIFO free
 *               list (allocation takes the head, release appends at the
 *               tail), or NULL for 0..P-1.
 * The pool does not touch dev_base (no kernel runs here) and never frees it.
 * Errors: INVALID_ARG for non-positive sizes, a size product that
 * overflows, misaligned or short memory, or a free_order that is not a
 * permutation. */
pa_status pa_alloc_pool(pa_pool** out, int L, int Hkv, int d, int B, int P,
                        pa_dtype dtype, void* dev_base, size_t dev_bytes,
                        const int32_t* free_order);
void pa_free_pool(pa_pool* pool); /* host metadata only; NULL is a no-op */

/* Device addresses of layer `layer`'s key and value slabs (the layout
 * above).  INVALID_ARG for a NULL pool or output, or a layer outside
 * [0, L). */
pa_status pa_pool_layer_ptrs(const pa_pool* pool, int layer, void** k_slab,
                             void** v_slab);

/* ---------------------------------------------------------------------
 * Host block manager (bit-exact, synchronous, not thread-safe)
 * Block tables are host int32 arrays of `maxb` entries; entry j is the
 * physical block of logical block j (tokens jB..jB+B-1).  A sequence of n
 * tokens uses entries 0..ceil(n/B)-1; the rest are ignored.
 * Source: "vLLM PagedAttention and continuous batching", sections
 * "PagedAttention: fixed blocks, non-contiguous physical memory" (the block
 * table with its fill count; a new block only when the last one is full)
 * and "Sharing with reference counts and copy-on-write" (reference counts;
 * the fork, append and free policies; release at count 0).  The free list
 * is first in, first out -- the pages leave the order open; this one keeps
 * a released address out of reuse for as long as possible.
 * ------------------------------------------------------------------- */

/* Pop the head of the free list; the block gets refcount 1 (a new physical
 * block for a sequence, section "PagedAttention: fixed blocks").
 * OUT_OF_BLOCKS when the list is empty (nothing changes). */
pa_status pa_block_alloc(pa_pool* pool, int32_t* blk);
/* One more reference to a live block: the fork policy of section "Sharing
 * with reference counts and copy-on-write" (INVALID_ARG if free or out of
 * range). */
pa_status pa_block_incref(pa_pool* pool, int32_t blk);
/* Drop one reference; at 0 the block goes to the tail of the free list (the
 * free policy of the same section).  INVALID_ARG for a block that is
 * already free (double free) or out of range. */
pa_status pa_block_decref(pa_pool* pool, int32_t blk);
/* Current refcount, or -1 if blk is out of range. */
int32_t pa_block_refcount(const pa_pool* pool, int32_t blk);
int32_t pa_num_free_blocks(const pa_pool* pool);
/* Copy the free list, head first, into host out[cap]; *count = its length. */
pa_status pa_free_list(const pa_pool* pool, int32_t* out, int32_t cap,
                       int32_t* count);
pa_status pa_pool_get_stats(const pa_pool* pool, pa_pool_stats* stats);

/* Append one token to a sequence holding n_before tokens (its new token
 * goes to position n_before) -- the append policy with copy-on-write of
 * "vLLM PagedAttention and continuous batching", sections "PagedAttention:
 * fixed blocks" and "Sharing with reference counts and copy-on-write":
 *   - n_before % B == 0: take a new block for logical block n_before / B;
 *   - else if the block holding position n_before has refcount > 1
 *     (copy-on-write): take a new block, report (*cow_src, *cow_dst) =
 *     (old, new), drop one reference to old, point the table at new;
 *   - slot = phys * B + n_before % B.
 * The caller must copy cow_src to cow_dst (pa_copy_blocks) before writing
 * the token (pa_write_kv).  *cow_src = *cow_dst = -1 when no copy is needed.
 * On OUT_OF_BLOCKS nothing changes.  INVALID_ARG if n_before / B >= maxb or
 * the table maps a free block. */
pa_status pa_append_slot(pa_pool* pool, int32_t* table, int32_t maxb,
                         int32_t n_before, int64_t* slot, int32_t* cow_src,
                         int32_t* cow_dst);

/* `count` successive appends to one sequence (prefill: "vLLM PagedAttention
 * and continuous batching", section "How it works", writes the prompt's
 * keys and values; each append follows pa_append_slot).  slots: host
 * [count] or NULL; cow_pairs: host [count][2] or NULL; *n_pairs = copies
 * requested; *n_done = appends completed.  On failure the first *n_done
 * appends stay applied and the failing one changed nothing. */
pa_status pa_append_tokens(pa_pool* pool, int32_t* table, int32_t maxb,
                           int32_t n_before, int32_t count, int64_t* slots,
                           int32_t* cow_pairs, int32_t* n_pairs,
                           int32_t* n_done);

/* One decode step for S sequences (section "How it works": decode adds one
 * token per sequence per iteration; each append follows pa_append_slot),
 * processed in batch order (the first
 * writer into a shared block copies; the one that finds refcount 1 writes
 * in place).  tables: host [S][maxb] (edited in place); n_before: host [S];
 * slots: host [S]; cow_pairs: host [S][2]; *n_pairs, *n_done as above. */
pa_status pa_append_batch(pa_pool* pool, int32_t* tables, int32_t maxb,
                          const int32_t* n_before, int32_t S, int64_t* slots,
                          int32_t* cow_pairs, int32_t* n_pairs,
                          int32_t* n_done);

/* Fork (section "Sharing with reference counts and copy-on-write": parallel
 * samples and beams map the parent's blocks with one more reference each):
 * child_table[0..nb-1] = parent_table[0..nb-1] and one more reference
 * to each of those blocks, nb = ceil(n_tokens / B).  Nothing changes on
 * error. */
pa_status pa_seq_fork(pa_pool* pool, const int32_t* parent_table,
                      int32_t n_tokens, int32_t* child_table, int32_t maxb);

/* Free (same section: a finished or dropped sequence releases its
 * references; blocks at count 0 return to the free list): one reference
 * fewer for each of the sequence's ceil(n_tokens/B) blocks.  INVALID_ARG (and nothing changes) if a block would drop below
 * zero. */
pa_status pa_seq_free(pa_pool* pool, const int32_t* table, int32_t n_tokens);

/* Beam selection ("vLLM PagedAttention and continuous batching", section
 * "Sharing with reference counts and copy-on-write": candidates that leave
 * the beam drop their references, blocks at zero are released, survivors
 * keep sharing what they share).  New sequence i continues old sequence
 * parents[i]: it maps the first ceil(lens[parents[i]] / B) blocks of that
 * table with one more reference each (a fork, i = 0 .. S_new-1 in order);
 * then every old table is freed (old sequences 0 .. S_old-1 in order, each
 * table's entries in order, a block reaching zero going to the free list's
 * tail).  The copy-on-write of shared last blocks happens at the next
 * append.
 *   tables: host [S_old][maxb]; lens: host [S_old]; parents: host [S_new],
 *   each in [0, S_old); out_tables: host [S_new][maxb], must not overlap
 *   tables (entries past the mapped ones are set to -1); out_lens: host
 *   [S_new].  S_old = 0 or S_new = 0 are allowed.
 * INVALID_ARG (and nothing changes) for a parent out of range, a table entry
 * outside the pool, or a block with fewer references than the old tables
 * hold. */
pa_status pa_seq_reorder(pa_pool* pool, const int32_t* tables, const int32_t* lens,
                         int32_t S_old, int32_t maxb, const int32_t* parents,
                         int32_t S_new, int32_t* out_tables, int32_t* out_lens);

/* Swap a group of sequences between two pools of the same shape (L, Hkv,
 * d, B, dtype), e.g. from the device pool to a host pool and back:
 * preemption by swapping ("vLLM PagedAttention and continuous batching",
 * section "Preemption when blocks run out": all blocks of a sequence or
 * none; sequences that share blocks, such as the beams of one search, move
 * together; the host side has its own block allocator, no larger than the
 * device pool).  Host manager only; pa_swap_blocks moves the bytes.
 *   For each distinct block the group's tables name in `from` (in order of
 *   first appearance: sequence 0's entries, then sequence 1's, ...) one block
 *   of `to` is allocated and given as many references as the group holds;
 *   pairs[i] = (old block, new block).  Then the group's references in
 *   `from` are dropped (sequence by sequence, entry by entry, as by
 *   pa_seq_free), which releases every moved block.  Finally the tables are
 *   rewritten in place to name the blocks of `to`.
 *   tables: host [S][maxb]; lens: host [S]; pairs: host [cap][2];
 *   *n_pairs = blocks moved.
 * All or nothing: INVALID_ARG if a block is also mapped outside the group
 * (its refcount exceeds the group's references), if the shapes differ or cap
 * is too small; OUT_OF_BLOCKS if `to` has fewer free blocks than needed. */
pa_status pa_move_blocks(pa_pool* from, pa_pool* to, int32_t* tables,
                         const int32_t* lens, int32_t S, int32_t maxb,
                         int32_t* pairs, int32_t cap, int32_t* n_pairs);

/* Groups for pa_decode_attention_grouped, from the block tables.  The
 * batch is cut into runs of consecutive sequences: a run of two or more
 * sequences whose first block is the same physical block shares the number
 * of leading table entries all its members agree on, times B, capped at
 * (shortest member's length - 1) so that every member keeps the position
 * this step writes for its own pass, and rounded down to a multiple of 16;
 * every other run shares nothing (length 0), and neighbouring runs that
 * share nothing are joined.  Host arrays: tables [S][maxb]; lens [S]
 * (context lengths including this step's token); written: group_start
 * [S+1] (run g is sequences group_start[g] .. group_start[g+1]-1,
 * group_start[n_groups] = S), group_len [S] (shared length of each run),
 * seq_group [S] (the run of each sequence); *n_groups = runs, *max_group =
 * the largest run that shares, *max_shared = the largest shared length,
 * *max_suffix = the largest number of positions a sequence holds outside
 * its run's shared prefix (lens[s] - group_len[seq_group[s]]; the
 * max_suffix argument of pa_decode_attention_grouped).
 * No state changes.  INVALID_ARG for a NULL output or a length that does not
 * fit the table. */
pa_status pa_prefix_groups(const pa_pool* pool, const int32_t* tables,
                           const int32_t* lens, int32_t S, int32_t maxb,
                           int32_t* group_start, int32_t* group_len,
                           int32_t* seq_group, int32_t* n_groups,
                           int32_t* max_group, int32_t* max_shared,
                           int32_t* max_suffix);

/* Debug validator of a decode step's device inputs, on the host.  The
 * kernels trust table entries, lengths and slots for their results (they
 * only clamp them to stay in bounds), so a caller in debug mode checks them
 * here first, against the manager's state.  Checks, sequence by sequence:
 * lens[s] >= 0 and ceil(lens[s] / B) <= maxb; every mapped entry
 * tables[s][j], j < ceil(lens[s] / B), is a block of the pool that is not
 * free; no block is mapped by these tables more often than its reference
 * count ("vLLM PagedAttention and continuous batching", section "Sharing
 * with reference counts and copy-on-write": the counts are the number of
 * mappings); and, when slots (host int64 [S]) is given, slots[s] < 0 or it
 * is the slot of position lens[s]-1 in a block of reference count 1 (the
 * step's write goes to a private block: any copy-on-write has happened).
 * Returns INVALID_ARG with the first violation in pa_last_error() and its
 * sequence in *bad_seq (may be NULL; -1 when the arguments themselves are
 * bad).  No state changes. */
pa_status pa_validate_step(const pa_pool* pool, const int32_t* tables,
                           int32_t maxb, const int32_t* lens, int32_t S,
                           const int64_t* slots, int32_t* bad_seq);

/* ---------------------------------------------------------------------
 * Device operations ("fused block operations" of the reading guide
 * "Efficient Memory Management for Large Language Model Serving with
 * PagedAttention", section "Main concepts to understand")
 * ------------------------------------------------------------------- */

/* reshape_and_cache ("vLLM PagedAttention and continuous batching", section
 * "How it works": each step writes its token's key and value into the
 * cache; the reading guide's "fused block operations"): token s's key and
 * value, k[s] and v[s] (device,
 * [S][Hkv][d], 16-byte aligned, pool dtype), go to slot slot_mapping[s]
 * (device int64 [S]) of layer `layer`: block slot / B, offset slot % B, for
 * every key/value head.  A negative slot skips the token; a slot >= P*B is
 * ignored as well (never written).  Bitwise copy, no type change.
 * Slots of one call must be distinct. */
pa_status pa_write_kv(pa_pool* pool, int layer, const void* k, const void* v,
                      const int64_t* slot_mapping, int S, hipStream_t stream);

/* copy_blocks ("vLLM PagedAttention and continuous batching", section
 * "Sharing with reference counts and copy-on-write": a write into a shared
 * block copies that one block first; pa_append_slot emits the pairs): for
 * each pair (src, dst) in pairs (device int32 [N][2]) copy
 * the whole physical block -- every layer, keys and values, all B slots and
 * Hkv heads -- from src to dst.  Pairs with an id outside [0, P) or src ==
 * dst are skipped.  Destinations must be distinct and must not appear as a
 * source in the same call. */
pa_status pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int N,
                         hipStream_t stream);

/* swap_blocks: the bytes of pa_move_blocks.  For each pair (src block of
 * `from`, dst block of `to`) in pairs (device int32 [N][2]) copy the whole
 * block -- every layer, keys and values -- from one pool's memory to the
 * other's.  Each pool's memory is device memory or pinned host memory
 * allocated with hipHostMalloc (mapped into the device's address space); the
 * copy is one kernel launch in which the GPU reads or writes host memory
 * directly over the host link, so a small block costs no transfer of its
 * own.  Pools must have the same shape; pairs with an id outside either
 * pool are skipped.  INVALID_ARG if a pool's memory is neither device memory
 * nor mapped pinned host memory.  Asynchronous on `stream`: host memory is
 * complete once the stream has been synchronised. */
pa_status pa_swap_blocks(pa_pool* from, pa_pool* to, const int32_t* pairs, int N,
                         hipStream_t stream);

/* Workspace for pa_decode_attention calls with up to S sequences, Hq query
 * heads and max_ctx context: split-K partial results (fp32 running maximum,
 * normaliser and weighted value sum per query head and context partition:
 * the state of eq. (4) of "Serving Language Models Within a Memory Budget",
 * merged by its rescale).
 * The size never decreases with S or max_ctx, so one workspace sized for the
 * largest call serves every smaller one.  Returns 0 for max_ctx == 0 or
 * invalid arguments. */
size_t pa_decode_workspace_bytes(const pa_pool* pool, int S, int Hq,
                                 int max_ctx);

/* Zero a workspace.  Optional: every partial a call reads was written by the
 * same call. */
pa_status pa_decode_workspace_init(void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* Decode-step paged attention for layer `layer` ("vLLM PagedAttention and
 * continuous batching", sections "PagedAttention: fixed blocks,
 * non-contiguous physical memory" and "The kernel page": one query token per
 * sequence reads its blocks through the block table, with the attention
 * formula unchanged; "Serving Language Models Within a Memory Budget",
 * section 6 and eq. (4): evaluated block by block with a running maximum and
 * normaliser, and context partitions merged by the same rescale; "PagedAttention
 * and Online Inference", section 1: GQA).  For each sequence s and query
 * head h,
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . K[t]) V[t]
 * over context positions t = 0..context_lens[s]-1, where K[t], V[t] are key
 * and value head floor(h / (Hq/Hkv)) of slot t % B of physical block
 * block_tables[s][t / B].
 *   out, q        : device [S][Hq][d], pool dtype, 16-byte aligned.
 *   block_tables  : device int32 [S][maxb].
 *   context_lens  : device int32 [S], each in [0, max_ctx]; 0 gives zeros.
 *   max_ctx       : host; an upper bound of context_lens (sizes the grid);
 *                   must be <= maxb * B.
 *   workspace     : device, 256-byte aligned, >= pa_decode_workspace_bytes(
 *                   pool, S, Hq, max_ctx) bytes; may be NULL when that size
 *                   is 0.  Calls that overlap in time need separate
 *                   workspaces.
 * Supported: d = 128, B in {8, 16, 32, 64, 128}, Hq / Hkv in {1, 2, 4, 8}; other shapes
 * return UNSUPPORTED.  Device-side values are trusted for results but
 * clamped for memory safety: a table entry outside [0, P) reads block
 * min(max(entry, 0), P-1) and a length above max_ctx is cut to max_ctx.
 * Context positions are read only through entries 0..ceil(len/B)-1 of a
 * table; slots past a sequence's length never influence its output. */
pa_status pa_decode_attention(pa_pool* pool, int layer, void* out,
                              const void* q, int S, int Hq,
                              const int32_t* block_tables, int maxb,
                              const int32_t* context_lens, int max_ctx,
                              float scale, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* pa_write_kv followed by pa_decode_attention for the same layer, in one
 * pass ("fused block operations" of the reading guide's main concepts):
 * the result -- the cache contents and `out` -- equals the two calls in that
 * order when every slot_mapping[s] >= 0 is the slot that position
 * context_lens[s] - 1 of sequence s maps to through block_tables[s] (the
 * decode step's own token) or is negative.  The token's key and value are
 * then taken from k / v directly for that position.  Arguments as for the
 * two separate calls (k, v: device [S][Hkv][d]; slot_mapping: device int64
 * [S]); same errors. */
pa_status pa_write_kv_decode_attention(pa_pool* pool, int layer, const void* k,
                                       const void* v,
                                       const int64_t* slot_mapping, void* out,
                                       const void* q, int S, int Hq,
                                       const int32_t* block_tables, int maxb,
                                       const int32_t* context_lens, int max_ctx,
                                       float scale, void* workspace,
                                       size_t ws_bytes, hipStream_t stream);

/* pa_decode_attention (k, v, slot_mapping all NULL) or
 * pa_write_kv_decode_attention (all three given) with the context
 * partitions launched longest first.  The same attention as those calls
 * ("vLLM PagedAttention and continuous batching", sections "PagedAttention:
 * fixed blocks, non-contiguous physical memory" and "The kernel page"); the
 * difference is only the order of the work.  The host's block manager
 * knows every sequence's length, so the library lists exactly the
 * partitions that hold positions, longest first.  A sequence's partitions
 * share its length equally (no short remainder partitions).  No workgroup
 * is launched past a sequence's end, and the ones that start last are the
 * shortest.
 *   host_context_lens : host int32 [S], equal to what context_lens holds
 *                       when the launch executes (the manager's copy);
 *                       read during the call only.  A value that differs
 *                       gives wrong outputs for that sequence but no access
 *                       outside the arguments.
 * Other arguments, results and errors as for pa_write_kv_decode_attention
 * (k, v: device [S][Hkv][d]; slot_mapping: device int64 [S]) and
 * pa_decode_attention; the same workspace.  INVALID_ARG if only some of k,
 * v and slot_mapping are given, or host_context_lens is NULL while S > 0.
 * The partition boundaries differ from the unordered calls', so outputs
 * agree with theirs within rounding, not bitwise; for given inputs they
 * are deterministic and the same at every block size.  Launches whose
 * partitions do not fit one list (over 512 (sequence, partition) units)
 * run as the unordered calls do. */
pa_status pa_decode_attention_ordered(pa_pool* pool, int layer, const void* k,
                                      const void* v,
                                      const int64_t* slot_mapping, void* out,
                                      const void* q, int S, int Hq,
                                      const int32_t* block_tables, int maxb,
                                      const int32_t* context_lens,
                                      const int32_t* host_context_lens,
                                      int max_ctx, float scale,
                                      void* workspace, size_t ws_bytes,
                                      hipStream_t stream);

/* pa_decode_attention_ordered without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The split-K partial
 * results go to a static device array of the library (32 MiB, one per
 * device, held until the process ends); the call itself allocates nothing.
 * Arguments, results and errors as pa_decode_attention_ordered; the output
 * is bitwise the same as that call's with any large enough workspace.
 * INVALID_ARG when the launch needs more than 32 MiB of partials (e.g. about
 * 330 sequences of 4,096 positions at 8 key/value heads and Hq / Hkv = 4);
 * nothing is launched then.  Every call on one device shares that device's
 * array, so calls that overlap in time on one device (different streams,
 * threads) race and must be serialised by the caller.  Nothing in the array
 * needs to start at zero: every partial a call reads was written by the
 * same call. */
pa_status pa_decode_attention_ordered_noalloc(pa_pool* pool, int layer,
                                              const void* k, const void* v,
                                              const int64_t* slot_mapping,
                                              void* out, const void* q, int S,
                                              int Hq, const int32_t* block_tables,
                                              int maxb,
                                              const int32_t* context_lens,
                                              const int32_t* host_context_lens,
                                              int max_ctx, float scale,
                                              hipStream_t stream);

/* Several query tokens per sequence over the same block tables: chunked
 * prefill ("vLLM PagedAttention and continuous batching", section "Chunked
 * prefill": a prefill that does not fit the step's budget is split, each
 * chunk attending to the cache written so far) and speculative verification
 * ("PagedAttention and Online Inference", section 5: speculative decoding
 * creates several new positions at once).  Sequence s has queries
 * q_start[s] .. q_start[s+1]-1 (nq of them) for its last nq positions,
 * whose keys and values are already in the cache (pa_write_kv): query t
 * sits at position n - nq + t, n = context_lens[s], and attends to
 * positions 0 .. n - nq + t (causal inside the new tokens).
 *   q, out      : device [T][Hq][d], row q_start[s] + t for query t of s
 *   q_start     : device int32 [S+1], nondecreasing, q_start[S] <= T; the
 *                 kernel clamps every entry into [0, T]
 *   max_q       : an upper bound of every nq (queries beyond it are not
 *                 computed); nq must not exceed context_lens[s]
 *   workspace   : >= pa_multi_query_workspace_bytes(pool, S, Hq, max_ctx,
 *                 max_q) bytes, 256-byte aligned, or NULL when that is 0
 * Other arguments, supported shapes and errors as pa_decode_attention; with
 * q_start[s+1] - q_start[s] = 1 for every s the result equals it. */
pa_status pa_multi_query_attention(pa_pool* pool, int layer, void* out,
                                   const void* q, const int32_t* q_start, int T,
                                   int S, int Hq, const int32_t* block_tables,
                                   int maxb, const int32_t* context_lens,
                                   int max_ctx, int max_q, float scale,
                                   void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* pa_multi_query_attention with the context partitions launched longest
 * first, as pa_decode_attention_ordered does, when each sequence's query
 * rows (query tokens x query heads of a key/value head) fit one 16-row
 * matrix-core tile, e.g. 4 speculative tokens at Hq / Hkv = 4.  Other
 * shapes run as pa_multi_query_attention does.
 *   host_context_lens : host int32 [S], equal to what context_lens holds
 *                       when the launch executes; read during the call.
 * Other arguments, results, errors and workspace as for
 * pa_multi_query_attention; INVALID_ARG if host_context_lens is NULL while
 * S > 0.  Outputs agree with pa_multi_query_attention within rounding (the
 * partitions differ), and are deterministic. */
pa_status pa_multi_query_attention_ordered(pa_pool* pool, int layer, void* out,
                                           const void* q, const int32_t* q_start,
                                           int T, int S, int Hq,
                                           const int32_t* block_tables, int maxb,
                                           const int32_t* context_lens,
                                           const int32_t* host_context_lens,
                                           int max_ctx, int max_q, float scale,
                                           void* workspace, size_t ws_bytes,
                                           hipStream_t stream);

/* Decode attention (optionally with the step's cache write, as
 * pa_write_kv_decode_attention) for a batch in which groups of consecutive
 * sequences share a prefix: the parallel samples or beams of one prompt map
 * the same physical blocks for their first positions ("vLLM PagedAttention
 * and continuous batching", section "Sharing with reference counts and
 * copy-on-write"; decode re-reads the cache every step, section "How it
 * works").  The shared positions are read once per group instead of once
 * per sequence: a group pass attends every member's query heads to them
 * (matrix cores), a suffix pass attends each sequence to its own positions,
 * and the two partial results are merged by the eq. (4) rescale.  Equal to
 * pa_decode_attention (up to rounding order) when the promise below holds.
 *   group_start : device int32 [n_groups+1]; group g is sequences
 *                 group_start[g] .. group_start[g+1]-1 (pa_prefix_groups
 *                 builds these arrays); groups with a shared length above 0
 *                 have at most max_group members
 *   group_len   : device int32 [n_groups]; the group's first group_len[g]
 *                 positions are mapped to the same physical blocks by every
 *                 member (the caller's promise) and are below every
 *                 member's context length.  Used rounded down to a multiple
 *                 of 16 and at most max_shared; 0 = nothing shared.
 *   seq_group   : device int32 [S]; the group of each sequence (a value
 *                 outside [0, n_groups) = none)
 *   max_suffix  : an upper bound of every sequence's positions outside its
 *                 group's shared prefix (context length - shared length);
 *                 positions beyond it are not attended to
 *   k, v, slot_mapping: as pa_write_kv_decode_attention, or all NULL
 *   workspace   : >= pa_decode_grouped_workspace_bytes(...) bytes,
 *                 256-byte aligned (always needed)
 * Other arguments, shapes and errors as pa_decode_attention.  A broken
 * promise gives wrong results but no access outside the arguments. */
pa_status pa_decode_attention_grouped(pa_pool* pool, int layer, const void* k,
                                      const void* v, const int64_t* slot_mapping,
                                      void* out, const void* q, int S, int Hq,
                                      const int32_t* block_tables, int maxb,
                                      const int32_t* context_lens, int max_ctx,
                                      const int32_t* group_start,
                                      const int32_t* group_len,
                                      const int32_t* seq_group, int n_groups,
                                      int max_group, int max_shared,
                                      int max_suffix, float scale,
                                      void* workspace, size_t ws_bytes,
                                      hipStream_t stream);

/* pa_decode_attention_grouped with the group pass launched longest first
 * (the partition order of pa_decode_attention_ordered, applied to the
 * prefixes that "vLLM PagedAttention and continuous batching", section
 * "Sharing with reference counts and copy-on-write", lets parallel samples
 * and beams share).  Each group's shared positions are split into
 * partitions of equal length, and only partitions that hold positions are
 * launched.
 *   host_group_len : host int32 [n_groups], equal to what group_len holds
 *                    when the launch executes (pa_prefix_groups' host
 *                    output); read during the call only.  A value that
 *                    differs gives wrong outputs for that group's members
 *                    but no access outside the arguments.
 * Other arguments, results, errors and workspace as for
 * pa_decode_attention_grouped; INVALID_ARG if host_group_len is NULL while
 * n_groups > 0.  Outputs agree with pa_decode_attention_grouped within
 * rounding (the group partitions differ), and are deterministic.  If the
 * groups' partitions do not fit one list (over 512 units), the call runs as
 * pa_decode_attention_grouped does. */
pa_status pa_decode_attention_grouped_ordered(
    pa_pool* pool, int layer, const void* k, const void* v,
    const int64_t* slot_mapping, void* out, const void* q, int S, int Hq,
    const int32_t* block_tables, int maxb, const int32_t* context_lens,
    int max_ctx, const int32_t* group_start, const int32_t* group_len,
    const int32_t* seq_group, const int32_t* host_group_len, int n_groups,
    int max_group, int max_shared, int max_suffix, float scale,
    void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for pa_decode_attention_grouped up to these sizes (never
 * decreasing in any argument); 0 for invalid sizes. */
size_t pa_decode_grouped_workspace_bytes(const pa_pool* pool, int S, int Hq,
                                         int max_ctx, int n_groups,
                                         int max_group, int max_shared,
                                         int max_suffix);

/* Workspace bytes for pa_multi_query_attention up to these sizes (never
 * decreasing in any argument); 0 if none is needed or the shape is
 * unsupported. */
size_t pa_multi_query_workspace_bytes(const pa_pool* pool, int S, int Hq,
                                      int max_ctx, int max_q);

/* Measurement aid: the achievable read rate of decode attention's own
 * access pattern.  "Serving Language Models Within a Memory Budget",
 * section 10, asks that the limiting resource be named before a speed is
 * interpreted; decode attention is bound by reading the cache ("vLLM
 * PagedAttention and continuous batching", section "How it works"), so this
 * call reads exactly the key and value rows pa_decode_attention reads --
 * positions 0 .. context_lens[s]-1 of every sequence and key/value head,
 * through its block table, in 16-byte loads -- spread evenly over a fixed
 * grid, and does no arithmetic but an XOR of every 32-bit word read:
 *   *checksum ^= XOR of all words of the key and value rows read.
 *   checksum : device uint32 [1], 4-byte aligned; the caller sets the
 *              starting value (zero for the plain checksum).
 * At most 2,048 sequences (UNSUPPORTED beyond).  Other arguments, clamping
 * and errors as for pa_decode_attention. */
pa_status pa_stream_tiles(pa_pool* pool, int layer, const int32_t* block_tables,
                          int maxb, const int32_t* context_lens, int S,
                          int max_ctx, uint32_t* checksum, hipStream_t stream);

/* Message describing the calling thread's last failure ("" if none). */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PA_H */
