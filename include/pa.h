/*
 * pa.h -- C ABI of libpa: single-query decode attention over a block-paged
 * KV cache on AMD Instinct MI355X (gfx950), plus the host block allocator
 * that produces its block tables and slot mappings.
 *
 * What the operations are (the pages on PagedAttention this follows):
 *  - The KV cache is cut into fixed-size physical blocks that need not be
 *    adjacent; a request takes a new block only when its current one is
 *    full ("Paged attention in LLMs", section "The fix").
 *  - Each request owns a block table mapping logical block j to a physical
 *    block; attention follows the table to each block in turn, so the
 *    sequence reads in order although storage is scattered (same page,
 *    "Keeping track: the block table").  Position pos lives in block
 *    table[pos / block_size] at offset pos % block_size (PagedAttention MCQ
 *    page, code sketch).
 *  - The attention itself is standard scaled dot-product attention over the
 *    gathered keys and values; only storage changes ("Paged Attention",
 *    chapter introduction; MCQ page, code sketch), and real kernels fold the
 *    table lookup into their tile loop (MCQ page, code sketch).
 *  - Requests with a common prefix point their own tables at the same
 *    blocks ("Paged attention in LLMs", "Sharing blocks"); a shared block is
 *    copied on write (MCQ page, comparison table, beam search / best of N).
 *
 * Conventions for every entry point:
 *  - Device pointers are hipMalloc'd (or torch) device memory owned by the
 *    caller, who keeps them alive until the stream work completes.  The
 *    library keeps no pointer after a call returns, allocates no device
 *    memory and never synchronises the stream.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *  - Every argument is validated on the host before anything is enqueued;
 *    a call that returns an error has enqueued nothing.  A launch failure
 *    reported by the runtime returns PA_ERR_LAUNCH.
 *  - Device data is range-checked where a bad value could address memory
 *    outside a buffer: a slot outside the pool is skipped by the writes; a
 *    block-table entry outside [0, num_blocks) or a sequence longer than its
 *    table turns that sequence's output rows into NaN.  Nothing faults.
 *
 * Device layout of one layer's cache (the pages keep keys and values of a
 * (block, kv-head) pair as [block_size][head_dim]; here the same tile is
 * stored in the order the gfx950 matrix cores consume it).  With
 * X = 16 / sizeof(element) (8 for bf16, 4 for f32) and head_dim % X == 0:
 *    k_cache: [num_blocks][num_kv_heads][head_dim / X][block_size][X]
 *    v_cache: [num_blocks][num_kv_heads][head_dim][block_size]
 * The key of the token in slot s (block s / bs, offset o = s % bs), kv-head
 * h, dimension d is k_cache[s/bs][h][d/X][o][d%X]; its value is
 * v_cache[s/bs][h][d][vpos(o)], where vpos(o) = o for f32 and for bf16 with
 * block_size 8, and for bf16 with block_size 16 or 32 vpos swaps bits 2 and
 * 3 of o (0-3, 8-11, 4-7, 12-15 within each 16 offsets): the 8 values a
 * matrix-core lane needs are then one 16-byte load.  A (block, head) tile is
 * contiguous (block_size * head_dim elements for each of K and V).
 * Pools are written only through this library (pa_cache_write,
 * pa_decode_append, pa_decode_append_noalloc, pa_copy_blocks,
 * pa_swap_blocks), which store in this order; a pool filled any other way
 * must follow the formulas above exactly, or attention reads other values
 * than the caller meant (no check can tell).
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
    PA_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size */
    PA_ERR_UNSUPPORTED = 2, /* a shape or dtype the kernels are not built for */
    PA_ERR_OOM = 3,         /* allocator: not enough free blocks (state unchanged) */
    PA_ERR_NOT_FOUND = 4,   /* allocator: unknown sequence id */
    PA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a launch */
    PA_ERR_EXISTS = 6       /* allocator: sequence id already in use */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status status);

/* ------------------------------------------------------------------------
 * Cache append: write each new token's keys and values into its slot.
 * The cache grows by one token per decode step and each token lands in the
 * slot its request's block table gives it ("Paged attention in LLMs",
 * "The cache being stored"; MCQ page, code sketch).
 *
 *   k, v          device, [num_tokens][num_kv_heads][head_dim], dtype, contiguous
 *   slot_mapping  device, int64 [num_tokens]; token t goes to slot
 *                 slot_mapping[t] = block * block_size + offset.  A negative
 *                 slot means "skip this token"; a slot >= num_blocks *
 *                 block_size is skipped as well.  Slots of one call must be
 *                 distinct (two tokens writing one slot race).
 *   k_cache, v_cache  device, the layout above; only the named slots change.
 *   head_dim      64 or 128;  block_size 8, 16 or 32;  num_tokens >= 0.
 * ------------------------------------------------------------------------ */
pa_status pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                         void* k_cache, void* v_cache,
                         int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                         void* stream);

/* ------------------------------------------------------------------------
 * Host check of a slot mapping before an append (pa_cache_write,
 * pa_decode_append): two tokens of one call writing one slot race on the
 * device, and slots outside the pool are skipped there without notice.
 * Pure host code, no GPU.
 *
 *   slot_mapping  host, int64 [num_tokens]; negative entries ("skip") pass
 *   num_slots     num_blocks * block_size of the pool
 *   first_bad     may be NULL; else the smallest index i whose slot lies in
 *                 [num_slots, inf) or repeats a slot of an earlier index,
 *                 or -1 when there is none
 * Returns PA_OK, or PA_ERR_INVALID_ARG for such an entry, for num_tokens < 0,
 * num_slots < 0, or a NULL slot_mapping with num_tokens > 0.
 * ------------------------------------------------------------------------ */
pa_status pa_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int64_t num_slots, int32_t* first_bad);

/* ------------------------------------------------------------------------
 * Copy whole physical blocks (keys and values of every kv-head): the copy
 * of a shared, partially filled block made before a request writes into it
 * (MCQ page, comparison table, "Copy on write blocks").
 *
 *   pairs   device, int32 [num_pairs][2] = (source block, destination block).
 *           Pairs with a block outside [0, num_blocks) are skipped.  No
 *           destination may also be a source or another pair's destination.
 * ------------------------------------------------------------------------ */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention: for every sequence b and query head h,
 *   out[b][h] = softmax_p(scale * q[b][h] . K[p][g]) . V[p][g],  p in [0, L_b)
 * with g = h / (num_q_heads / num_kv_heads) and K[p], V[p] read through the
 * block table (block block_tables[b][p / bs], offset p % bs).  L_b counts
 * the token being decoded (write it with pa_cache_write first).  L_b = 0
 * gives a zero row.  Entries of a table row past ceil(L_b / bs) are never
 * read, nor is any slot at or past L_b.
 *
 *   q             device, [num_seqs][num_q_heads][head_dim], dtype
 *   k_cache, v_cache  device, the layout above, [num_blocks] blocks
 *   block_tables  device, int32 [num_seqs][max_blocks_per_seq], row-major
 *   seq_lens      device, int32 [num_seqs]
 *   out           device, [num_seqs][num_q_heads][head_dim], dtype (rounded
 *                 to nearest-even from float32 for bf16)
 *   num_q_heads % num_kv_heads == 0 and num_q_heads / num_kv_heads <= 16.
 *   dtype PA_BF16: bf16 inputs, bf16 matrix-core products, float32
 *   accumulation and softmax.  PA_F32: float32 throughout.
 *
 * Splitting a sequence across waves (split-sequence decode).  The result
 * is the same attention whichever way a sequence is cut: each piece j
 * yields its output o_j, maximum m_j and exp-sum l_j, and a log-sum-exp
 * merge combines them:
 *   M = max_j m_j,  w_j = l_j * exp(m_j - M),  out = sum_j w_j o_j / sum_j w_j.
 *  partition_size == 0: no split; one wave per (sequence, kv-head).
 *    workspace may be NULL.
 *  partition_size > 0: fixed partitions of partition_size tokens (a
 *    multiple of 32 and of block_size, at most 64 * block_size), merged by
 *    a second kernel.  A sequence that fits one partition is written
 *    directly.
 *  partition_size == PA_PARTITION_BALANCED: the batch's token steps are
 *    shared out evenly over a fixed grid of waves whatever the length mix;
 *    a (sequence, kv-head) cut between waves is merged inside the same
 *    kernel by the wave that finishes its last piece.  num_seqs <= 1024.
 * workspace: device, 256-byte aligned, at least pa_decode_workspace_bytes()
 * bytes.  Its first pa_decode_counter_bytes() bytes are counters that must
 * be zero before the first PA_PARTITION_BALANCED call on that workspace
 * (allocate it zero-filled); every call leaves them zero again, and the
 * other modes do not touch them.  The rest is scratch whose contents on
 * entry do not matter.  Calls sharing one workspace must not overlap.
 * ------------------------------------------------------------------------ */
#define PA_PARTITION_BALANCED (-1)

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 int32_t partition_size);
/* Bytes at the start of every workspace (pa_decode, pa_prefill,
 * pa_decode_shared_prefix) that hold the balanced split's counters
 * (zero-filled once, see above).  The same for every call, and no call
 * writes anything else there, so one workspace, large enough, serves calls
 * of any size and mode one after another. */
size_t pa_decode_counter_bytes(void);

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    int32_t num_kv_heads, float scale, void* out, void* stream,
                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    pa_dtype dtype, int32_t partition_size,
                    void* workspace, size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * One decode step in one launch: the cache append of each sequence's new
 * token (pa_cache_write with one token per sequence) and pa_decode on the
 * balanced split, with the same results.  The cache grows by the token a
 * step adds and attention reads the table, pos / block_size and
 * pos % block_size ("Paged attention in LLMs", "The cache being stored";
 * MCQ page, code sketch); the launch attends to position L_b - 1 from the
 * new token's row below instead of from its slot, so it never waits for
 * its own stores.
 *
 *   k, v          device, [num_seqs][num_kv_heads][head_dim], dtype: row b
 *                 is sequence b's token at position L_b - 1 (rows of
 *                 sequences with L_b <= 0 are not read)
 *   slot_mapping  device, int64 [num_seqs]: where row b is stored (slot =
 *                 block * block_size + offset, as for pa_cache_write);
 *                 outside [0, num_blocks * block_size) skips the store.  It
 *                 should be position L_b - 1's slot in b's table: the result
 *                 uses row b for that position whatever is stored there.
 *   k_cache, v_cache  written (the new tokens) and read (positions
 *                 0 .. L_b - 2)
 *   workspace     as pa_decode with partition_size PA_PARTITION_BALANCED
 *                 (pa_decode_workspace_bytes(..., PA_PARTITION_BALANCED),
 *                 counters zero-filled once, left zero)
 * Everything else as pa_decode; the same error rows (zeros for L_b <= 0,
 * NaN for a length the table cannot hold or a table entry outside the pool
 * among positions 0 .. L_b - 2); num_seqs <= 1024.  The stores of a call
 * and any read of the same slots by another call must be ordered by the
 * stream.
 * ------------------------------------------------------------------------ */
pa_status pa_decode_append(const void* q, const void* k, const void* v, const int64_t* slot_mapping,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           const int32_t* seq_lens, int32_t num_kv_heads, float scale, void* out,
                           void* stream, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           pa_dtype dtype, void* workspace, size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * pa_decode_append without a workspace and without allocating: for callers
 * that cannot allocate device memory (code under stream capture into a
 * graph, serving loops that forbid allocation, harnesses that disallow it).
 * Arguments, result, pool bytes and errors are those of pa_decode_append;
 * the caller still passes every input and `out`.  The balanced split's
 * merge counters and cut-piece partials live instead in a static device
 * array of the library, 16 MiB, one per GPU the library runs on, held
 * until the process ends.
 *
 * Limit: the scratch a call needs is 8 KiB of counters plus
 * 2 * W * G * (head_dim + 2) * 4 bytes of partials (each 256-byte aligned),
 * W = 2 * the device's compute units (512 on MI355X), G = num_q_heads /
 * num_kv_heads; a shape needing more than 16 MiB returns
 * PA_ERR_UNSUPPORTED with nothing enqueued (on MI355X every supported shape
 * fits: G 16 with head_dim 128 needs about 8.2 MiB).
 * Set-up: the first call on a device takes the array's address on that
 * device and clears its counters with a fill kernel on the call's stream
 * (the split leaves them zero after every call); PA_ERR_LAUNCH if that
 * fails.  The call uses no hipMalloc, hipFree or allocating library
 * routine.
 * Concurrency: every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other host threads without
 * ordering between them) race and give wrong rows; order them.
 * ------------------------------------------------------------------------ */
pa_status pa_decode_append_noalloc(const void* q, const void* k, const void* v, const int64_t* slot_mapping,
                                   void* k_cache, void* v_cache, const int32_t* block_tables,
                                   const int32_t* seq_lens, int32_t num_kv_heads, float scale, void* out,
                                   void* stream, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                   pa_dtype dtype);

/* ------------------------------------------------------------------------
 * Multi-token query over the paged cache: prefill, chunked prefill and
 * speculative verification.  Request b has L_b = seq_lens[b] tokens in the
 * cache, the last M_b of them new (their keys and values already written
 * with pa_cache_write, as the cache grows by what a step adds: "Paged
 * attention in LLMs", "The cache being stored").  Its M_b query tokens are
 * rows query_start[b] .. query_start[b+1] - 1 of q; query token i sits at
 * position p = L_b - M_b + i and attends causally, to positions 0 .. p:
 *   out[t][h] = softmax_k(scale * q[t][h] . K[k][g]) . V[k][g],  k in [0, p]
 * with g = h / (num_q_heads / num_kv_heads) and K, V read through the block
 * table as for pa_decode (MCQ page, code sketch).
 *
 *   q            device, [num_query_tokens][num_q_heads][head_dim], dtype
 *   query_start  device, int32 [num_seqs + 1], non-decreasing from 0 to
 *                num_query_tokens (M_b = query_start[b+1] - query_start[b],
 *                0 allowed)
 *   out          device, [num_query_tokens][num_q_heads][head_dim], dtype
 *   max_query_len  >= every M_b (sizes the launch)
 *   workspace    may be NULL: then a kernel with one wave per (kv-head,
 *                tile of query tokens, request) walks all of each tile's
 *                keys; for bfloat16 chunks of max_query_len * (num_q_heads /
 *                num_kv_heads) >= 128 columns (block size 16 or 32, or head
 *                dim 64; scale > 0), workgroups of four such tiles walk them together,
 *                each key/value step read from the pool once and shared
 *                through LDS.  The same holds with a workspace when
 *                neither path below applies (see pa_prefill_workspace_bytes).
 *                A caller that passes a workspace (256-byte aligned) of at
 *                least pa_prefill_workspace_bytes() bytes, when that is not
 *                0, gets one of two faster paths:
 *                - verification-sized chunks (max_query_len * (num_q_heads /
 *                  num_kv_heads) <= 16, num_seqs <= 1024): pa_decode's
 *                  balanced split, each request's (token, head) pairs one
 *                  wave's columns.  Its counter bytes
 *                  (pa_decode_counter_bytes()) must be zero before the first
 *                  use and are left zero, as for pa_decode;
 *                - short chunks of a batch otherwise (the tile launch would
 *                  hold fewer than 1,024 waves and max_blocks_per_seq *
 *                  block_size spans two 2,048-token key partitions or more):
 *                  the tile kernel with its keys cut into partitions, whose
 *                  partial results a merge kernel combines (log-sum-exp
 *                  rule; a tile whose keys fit the first partition writes
 *                  its rows directly).  The workspace's first
 *                  pa_decode_counter_bytes() bytes are left untouched; the
 *                  rest may hold anything on entry.
 *                A workspace smaller than required gives PA_ERR_INVALID_ARG.
 *                Calls sharing a workspace must not overlap.
 *   num_q_heads / num_kv_heads <= 16; the other arguments as for pa_decode.
 * Error rows: a request with M_b > L_b, M_b > max_query_len, or L_b longer
 * than its table holds gets NaN in all its rows; a table entry outside
 * [0, num_blocks) among a query tile's keys gives NaN rows for that tile
 * (for all four tiles of a workgroup on the workgroup path); a
 * request whose query_start pair is out of order or outside
 * [0, num_query_tokens] writes nothing.  Nothing faults.
 * ------------------------------------------------------------------------ */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t max_query_len);

pa_status pa_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* seq_lens, const int32_t* query_start, int32_t num_kv_heads, float scale,
                     void* out, void* stream, int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                     pa_dtype dtype, int32_t max_query_len, void* workspace, size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * Copy whole blocks from one pool to another with the same block shape:
 * the data movement of swapping a preempted request's blocks out to a host
 * pool and back in (the MCQ page names preemption among what paging makes
 * easy; pa_alloc_move gives the pairs).
 *
 *   src_k, src_v   source pool ([src_num_blocks] blocks, the layout above)
 *   dst_k, dst_v   destination pool ([dst_num_blocks] blocks)
 *   pairs          int32 [num_pairs][2] = (source block, destination block);
 *                  a pair with a block out of range is skipped; no
 *                  destination block may appear twice.
 * Each of the five buffers is device memory or pinned host memory
 * (hipHostMalloc, e.g. a torch tensor made with pin_memory=True), which the
 * kernel reads or writes over the host link; pageable host memory is
 * rejected with PA_ERR_INVALID_ARG before anything is enqueued.  A host
 * destination holds the data once the stream has reached the copy.
 * ------------------------------------------------------------------------ */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks, void* dst_k,
                         void* dst_v, int32_t dst_num_blocks, const int32_t* pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                         void* stream);

/* ------------------------------------------------------------------------
 * Shared-prefix decode: the same result as pa_decode (same arguments, same
 * output, same handling of empty rows and bad tables), computed so that
 * the keys and values of blocks that several requests share are read once
 * for all of them.  Requests forked from one prompt point their tables at
 * the same physical blocks ("Paged attention in LLMs", "Sharing blocks";
 * MCQ page, comparison table, parallel sampling and beam search), so their
 * attention over those blocks can be computed together: one wave loads a
 * key/value step once and scores it against every member's queries.
 *
 *   groups        device, int32 [num_groups][2] = (first request, member
 *                 count).  Members are requests first .. first + count - 1;
 *                 groups do not overlap; requests in no group are allowed.
 *   prefix_blocks device, int32 [num_seqs]: for a group member, the number
 *                 of leading table entries the whole group has in common
 *                 (the same for every member, at most
 *                 floor(L_b / block_size) for each of them); 0 for a request
 *                 in no group.
 *   max_group_size >= every member count; max_group_size * (num_q_heads /
 *                 num_kv_heads) <= 64 (<= 32 for PA_F32 with head_dim 128).
 *   max_prefix_blocks >= every prefix_blocks entry, <= max_blocks_per_seq.
 *   partition_size  as for pa_decode's fixed partitions (a multiple of 32
 *                 and of block_size, at most 64 * block_size); both the
 *                 shared part and each request's own part are cut into
 *                 partitions of this many tokens.
 * The first (prefix_blocks * block_size) / a * a tokens of a member, with
 * a = max(32, block_size), are the shared part; the rest of its tokens are
 * its own.  A prefix_blocks entry above max_prefix_blocks, or a shared
 * part longer than the request, gives NaN rows; a group larger than
 * max_group_size gives NaN rows for its members.  A group that breaks the
 * rules above (members with different prefix_blocks, overlapping groups,
 * tables that differ inside the shared part) gives unspecified values in
 * its members' rows but reads and writes nothing outside the buffers.
 * workspace: device, 256-byte aligned, at least
 * pa_decode_shared_prefix_workspace_bytes() bytes of scratch (contents on
 * entry do not matter); calls sharing a workspace must not overlap.  The
 * call leaves the first pa_decode_counter_bytes() bytes untouched, so one
 * workspace can serve this call and pa_decode's balanced split in turn.
 * The size function returns 0 for arguments the call would reject.
 * ------------------------------------------------------------------------ */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                               int32_t block_size, int32_t max_blocks_per_seq,
                                               int32_t max_prefix_blocks, int32_t partition_size);

pa_status pa_decode_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  int32_t num_kv_heads, float scale, void* out, void* stream,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                  pa_dtype dtype, const int32_t* groups, const int32_t* prefix_blocks,
                                  int32_t num_groups, int32_t max_group_size, int32_t max_prefix_blocks,
                                  int32_t partition_size, void* workspace, size_t workspace_bytes);

/* Host planning for pa_decode_shared_prefix (host memory throughout, no HIP
 * calls).  Walks the batch in order and grows a group from each request
 * while the next request's table starts with the same entries: a request
 * joins when the group then still shares at least min_shared_blocks whole
 * blocks (blocks inside every member's length) and the reads saved,
 * (members - 1) * shared blocks, do not go down; at most max_group_size
 * members.  Only groups of two or more are listed.
 *   block_tables  host int32 [num_seqs][max_blocks_per_seq];  seq_lens host int32 [num_seqs]
 *   groups        out, host int32 [2 * num_seqs] (room for the worst case)
 *   prefix_blocks out, host int32 [num_seqs]
 *   *num_groups, *max_group (>= 1), *max_prefix_blocks   out
 * ------------------------------------------------------------------------ */
pa_status pa_plan_shared_prefix(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                int32_t max_blocks_per_seq, int32_t block_size, int32_t max_group_size,
                                int32_t min_shared_blocks, int32_t* groups, int32_t* prefix_blocks,
                                int32_t* num_groups, int32_t* max_group, int32_t* max_prefix_blocks);

/* ------------------------------------------------------------------------
 * KV-memory accounting of a request trace (host only, no HIP calls): how
 * much of the memory a scheme holds is filled with tokens, under the
 * contiguous reservation the pages start from ("Paged attention in LLMs",
 * "Why the memory gets wasted": each request reserves its prompt plus the
 * largest reply in one unbroken run, placed first fit, so both unreached
 * reserved slots and gaps too small for the next reservation are lost) and
 * under paging ("The fix", "Why this helps so much": whole blocks taken one
 * at a time from anywhere, at most the last block's unfilled tail lost per
 * request; MCQ page, comparison table, "Memory waste" row).
 *
 * Time runs in decode steps.  At step t: requests that completed their
 * reply at t - 1 release their memory; requests with arrival_step == t are
 * admitted in trace order (the prompt is stored at once) or rejected if they
 * do not fit (contiguous: no free run of prompt + max_reply slots, or a reply
 * longer than max_reply; paged: fewer free blocks than the prompt needs);
 * every request admitted before t appends one reply token (a paged request
 * that needs a new block when none is free is dropped and releases its
 * blocks); a request whose reply is complete releases at t + 1.  After each
 * step the held and used slots of the live requests are summed.
 *
 *   arrival_step, prompt_len, reply_len  host int32 [num_requests], arrival
 *                 steps non-decreasing (trace order) and >= 0, prompts >= 1,
 *                 replies >= 0
 *   capacity_slots  token slots of the memory (paged: capacity / block_size blocks)
 *   scheme        PA_MEM_CONTIGUOUS (param = max_reply, the reserved reply
 *                 length) or PA_MEM_PAGED (param = block_size >= 1)
 *   out           host; filled on PA_OK
 * ------------------------------------------------------------------------ */
#define PA_MEM_CONTIGUOUS 0
#define PA_MEM_PAGED 1

typedef struct {
    int64_t steps;              /* steps until the last request released (or the trace ended) */
    int64_t used_slot_steps;    /* sum over steps of slots holding a token */
    int64_t held_slot_steps;    /* sum over steps of slots held by live requests */
    int64_t peak_used;          /* largest per-step used slots */
    int64_t peak_held;          /* largest per-step held slots */
    int64_t max_request_waste;  /* largest held - used of one request at the end of a step */
    int32_t admitted;
    int32_t rejected;           /* did not fit on arrival */
    int32_t dropped;            /* paged: no block left while growing */
    int32_t peak_live;          /* most requests holding memory at the end of a step */
} pa_mem_stats;

pa_status pa_simulate_memory(const int32_t* arrival_step, const int32_t* prompt_len, const int32_t* reply_len,
                             int32_t num_requests, int64_t capacity_slots, int32_t scheme, int32_t param,
                             pa_mem_stats* out);

/* ------------------------------------------------------------------------
 * Host block allocator (no device memory, no HIP calls; not thread-safe).
 * Follows "Paged attention in LLMs" ("The fix", "Keeping track: the block
 * table", "Sharing blocks") and the MCQ page's copy-on-write row:
 *  - free pool: a FIFO queue, initially `free_order` (NULL = 0..num_blocks-1);
 *    freed blocks join its tail, walked from logical block 0 upward;
 *  - append(seq, n): token at position pos takes slot table[pos/bs]*bs +
 *    pos%bs; a new block is popped when pos % bs == 0; if the sequence's
 *    partially filled last block is shared (reference count > 1) the first
 *    appended token first copies it to a fresh block and records the
 *    (source, destination) pair, the last holder writes in place;
 *    all or nothing: PA_ERR_OOM leaves the state unchanged;
 *  - fork(parent, child): child gets a copy of parent's table and length,
 *    every block's reference count goes up by one;
 *  - free(seq): every block's count goes down; blocks reaching 0 are freed.
 * Sequence ids are arbitrary int64 keys.
 * ------------------------------------------------------------------------ */
typedef struct pa_allocator pa_allocator;

/* NULL on a bad argument (num_blocks < 0, block_size <= 0, free_order not a
 * permutation of 0..num_blocks-1).  Host memory `free_order` is copied. */
pa_allocator* pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pa_alloc_destroy(pa_allocator* a);
pa_status pa_alloc_add_seq(pa_allocator* a, int64_t seq);
/* slots_out: host int64 [n_tokens] (may be NULL when n_tokens == 0);
 * cow_pairs_out: host int32 [2 * cow_cap] receives (src, dst) pairs,
 * *n_cow their count (an append copies at most one block, so cow_cap = 1
 * always suffices). */
pa_status pa_alloc_append(pa_allocator* a, int64_t seq, int32_t n_tokens, int64_t* slots_out,
                          int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow);
pa_status pa_alloc_fork(pa_allocator* a, int64_t parent, int64_t child);
pa_status pa_alloc_free(pa_allocator* a, int64_t seq);
/* Copy up to `cap` table entries of seq into host `out`; *n_blocks and
 * *seq_len receive the full table length and token count. */
pa_status pa_alloc_table(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap,
                         int32_t* n_blocks, int32_t* seq_len);
/* Dense decode inputs for a batch: host tables_out [n_seqs][width] (entries
 * past a sequence's blocks are set to `pad`), host seq_lens_out [n_seqs].
 * PA_ERR_INVALID_ARG if a table is wider than `width`. */
pa_status pa_alloc_batch_tables(const pa_allocator* a, const int64_t* seqs, int32_t n_seqs,
                                int32_t* tables_out, int32_t width, int32_t pad,
                                int32_t* seq_lens_out);
/* Move sequences from allocator `from` to allocator `to` (same block size):
 * swap-out (device pool -> host pool) and swap-in (back).  Every distinct
 * block the listed sequences hold in `from` takes one fresh block of `to`,
 * in order of first appearance (sequences in the given order, each table
 * from logical block 0), so blocks the moved sequences share stay shared;
 * host pairs_out [2 * cap] receives (from block, to block) for each, *n_pairs
 * their count — the copies the caller makes with pa_swap_blocks before it
 * reuses the freed blocks.  In `from` the sequences are then freed as by
 * pa_alloc_free in the given order (a block another sequence still holds
 * stays).  All or nothing: PA_ERR_NOT_FOUND (a sequence not in `from`),
 * PA_ERR_EXISTS (already in `to`), PA_ERR_OOM (too few free blocks in `to`),
 * PA_ERR_INVALID_ARG (a sequence listed twice, different block sizes, or
 * cap too small — then *n_pairs is set to the room needed) change nothing. */
pa_status pa_alloc_move(pa_allocator* from, pa_allocator* to, const int64_t* seqs, int32_t n_seqs,
                        int32_t* pairs_out, int32_t cap, int32_t* n_pairs);
/* Reference count of a block (-1 if out of range). */
int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block);
/* Free queue in order, head first: up to `cap` ids into host `out`, *n = its length. */
pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n);
int32_t pa_alloc_num_free(const pa_allocator* a);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
