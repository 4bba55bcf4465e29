/*
 * pa.h -- paged KV cache hot path for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels for the three GPU operations of
 * PagedAttention's decode step:
 *
 *   pa_compute_slots     logical (sequence, position) -> physical cache slot
 *   pa_write_kv          store new tokens' K/V in their slots
 *   pa_write_kv_at       the two above in one launch
 *   pa_copy_blocks       copy whole KV blocks (copy-on-write of shared blocks)
 *   pa_swap_blocks       move whole KV blocks between two pools, e.g. HBM and
 *                        pinned host memory (fine-grained eviction)
 *   pa_decode_attention  one query token per sequence attends to its history,
 *                        reached block by block through its block table
 *   pa_decode_attention_append  the new tokens stored and attended in one call
 *   pa_decode_attention_shared  the same for groups of sequences sharing a
 *                        prefix, each shared block read once per group
 *   pa_prefill_attention  several query tokens per sequence (a prompt chunk),
 *                        causal, over the same pools
 *
 * Sources, cited by page title and section:
 *   [nalar]    "PagedAttention: memetakan blok KV logis ke memori fisik tidak
 *              kontigu" (nalar.dev)
 *   [bicarait] "Melihat Lebih Dalam vLLM v0.7: Bagaimana PagedAttention &
 *              Chunked Prefill ..." (bicarait.com)
 *   [gininih]  "Apa itu PagedAttention (Manajemen Memori KV Cache GPU)?"
 *              (gininih.com)
 *   [gyaansetu] "KV Cache and PagedAttention: Why Your LLM Server Slows Down"
 *              (gyaansetu.com)
 *
 * ---------------------------------------------------------------------------
 * Conventions for every entry point
 * ---------------------------------------------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer on the current HIP
 *   device.  The caller allocates and owns all memory, including the decode
 *   workspace; the library allocates nothing and keeps no pointer after the
 *   call returns (its one static device array, the workspace of
 *   pa_decode_attention_noalloc, is part of the loaded code).  Pools are
 *   updated in place.
 * Streams.  `stream` is a hipStream_t passed as void*; NULL is the null
 *   stream.  Every call only enqueues work and returns; results are visible
 *   in stream order.  Ordering between calls (write -> attend, copy -> attend)
 *   is the caller's stream order.
 * Element types.  PA_F32 (IEEE binary32) or PA_BF16 (bfloat16, the upper
 *   16 bits of a binary32).  K, V, new K/V and Q share one element type.
 * Layouts (row-major, contiguous).  x = 16 / element size (8 for bf16,
 *   4 for f32): a "granule" is 16 bytes.
 *   v_cache            [num_blocks][num_kv_heads][block_size][head_dim]
 *                      -- element d of the token at offset o of a block is
 *                      v_cache[blk][h][o][d]
 *   k_cache            [num_blocks][num_kv_heads][head_dim/x][block_size][x]
 *                      -- element d of the token at offset o of a block is
 *                      k_cache[blk][h][d/x][o][d%x] (granules token-minor,
 *                      so the matrix-core operand of 16 keys x 16 bytes is one
 *                      contiguous run).  In both pools one (block, KV head)
 *                      chunk is block_size*head_dim contiguous elements.
 *                      K is deliberately not token-major like V
 *                      ([NB][Hkv][bs][D]): with token-major rows the four
 *                      lanes of each 64-byte group of the matrix-core K
 *                      operand would read four different 256-byte rows, and
 *                      a gather of that pattern measured ~4.7 TB/s on MI355X
 *                      against ~6.0 TB/s for the granule layout.
 *   block_tables       int32 [num_seqs][max_blocks_per_seq]; entry b is the
 *                      physical block of logical block b; entries past the
 *                      last used block are never read (may hold -1)
 *   context_lens       int32 [num_seqs]
 *   q                  [num_seqs][num_q_heads][head_dim]
 *   out                float32 [num_seqs][num_q_heads][head_dim]
 *   k_new, v_new       [num_tokens][num_kv_heads][head_dim] with a token
 *                      stride (in elements) that may exceed num_kv_heads*head_dim
 *   slot_mapping       int64 [num_tokens]; -1 = padding token (skipped)
 *   block_mapping      int32 [num_pairs][2] = (src, dst)
 * Errors.  Scalar arguments are validated on the host before any HIP call,
 *   so a rejected call has no effect and is safe without a GPU.  The contents
 *   of device arrays are not validated (that would need a synchronisation);
 *   instead every kernel bounds-checks each index it reads from device memory
 *   (slot, block id, sequence id, context length) and skips or clamps an
 *   access that would leave its buffer, so a bad table cannot make the GPU
 *   fault; the affected results are then unspecified.  A launch failure is
 *   reported as PA_ERR_HIP.
 * Threading.  The only state the library keeps is a per-device cache of the
 *   stream-K worker count (resident wave slots of the device, read once per
 *   device and head_dim; written atomically), so concurrent calls on
 *   different streams are safe when their output and workspace buffers are
 *   disjoint.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

/* In C++ the enums get int as their fixed underlying type, so every int a C
 * caller passes is a value of the type (a plain C++ enum would make an
 * out-of-range value undefined behaviour before validation could reject
 * it); in C an enum is an int-sized integer anyway, so the ABI is the same. */
#ifdef __cplusplus
#define PA_ENUM_BASE : int
#else
#define PA_ENUM_BASE
#endif

typedef enum pa_status PA_ENUM_BASE {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL                     */
  PA_ERR_SHAPE = 2,        /* a size is out of range or sizes disagree       */
  PA_ERR_DTYPE = 3,        /* unknown element type                           */
  PA_ERR_UNSUPPORTED = 4,  /* head_dim, block_size or partition not supported*/
  PA_ERR_WORKSPACE = 5,    /* decode workspace missing or too small          */
  PA_ERR_HIP = 6,          /* the HIP runtime reported an error              */
  PA_ERR_CAPACITY = 7      /* block manager: no free block / sequence slot   */
} pa_status;

typedef enum pa_dtype PA_ENUM_BASE { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Supported shapes (checked by every entry point):
 *   head_dim   in {64, 128}
 *   block_size in {8, 16, 32, 64}
 *   num_q_heads a multiple of num_kv_heads, num_q_heads/num_kv_heads <= 16   */

/* ---------------------------------------------------------------------------
 * pa_compute_slots
 *
 * [nalar] "Urutan logis dipisahkan dari penempatan fisik" and [bicarait]
 * "Blueprint Arsitektur 2": a sequence's logical block b lives in physical
 * block block_tables[seq][b]; tokens keep their logical order inside a block.
 * For token j:
 *     p = positions[j], i = seq_ids[j]
 *     slots[j] = block_tables[i][p / block_size] * block_size + p % block_size
 * computed in 64-bit integers.  slots[j] = -1 when p < 0 (padding), and also
 * when i is not in [0, num_seqs), p / block_size >= max_blocks_per_seq, or the
 * table entry is not in [0, num_blocks) -- such a token is then skipped by
 * pa_write_kv.  seq_ids may be NULL: token j then belongs to sequence j
 * (one new token per sequence, the decode step).
 * ------------------------------------------------------------------------- */
pa_status pa_compute_slots(int64_t* slots, const int32_t* block_tables,
                           int32_t num_seqs, int32_t max_blocks_per_seq,
                           const int32_t* seq_ids, const int32_t* positions,
                           int32_t num_tokens, int32_t block_size,
                           int32_t num_blocks, void* stream);

/* ---------------------------------------------------------------------------
 * pa_write_kv  (reshape-and-cache)
 *
 * [gyaansetu] "Apa itu KV Cache?": only the new token's K and V are computed;
 * they are stored so later steps read them back.  For each token j with
 * 0 <= slot_mapping[j] < num_blocks*block_size, each KV head h and dim d,
 * with b = slot / block_size and o = slot % block_size:
 *     k_cache[b][h][d/x][o][d%x] = k_new[j][h][d]
 *     v_cache[b][h][o][d]        = v_new[j][h][d]
 * A bit copy (exact).  Negative slots and slots beyond the pool are skipped.
 * Two tokens with the same slot race (caller error).  new_token_stride is
 * the distance in elements between consecutive tokens of k_new and v_new;
 * 0 means num_kv_heads*head_dim.  It must be a multiple of 8 elements for
 * bf16 and 4 for f32 (16-byte rows), and the pointers 16-byte aligned.
 * ------------------------------------------------------------------------- */
pa_status pa_write_kv(void* k_cache, void* v_cache, const void* k_new,
                      const void* v_new, const int64_t* slot_mapping,
                      int32_t num_tokens, int64_t new_token_stride,
                      int32_t num_blocks, int32_t block_size,
                      int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                      void* stream);

/* ---------------------------------------------------------------------------
 * pa_write_kv_at  (slots and write in one launch)
 *
 * pa_compute_slots followed by pa_write_kv, fused: token j goes to
 *     slot = block_tables[i][p / block_size] * block_size + p % block_size
 * with p = positions[j] and i = seq_ids[j] (or j when seq_ids is NULL), under
 * exactly the rules of pa_compute_slots (slot -1, token skipped, for p < 0 or
 * any index outside its table or the pool), and is stored as pa_write_kv
 * stores it.  slots_out (int64 [num_tokens]) may be NULL; when given it
 * receives the slots, so the call also does what pa_compute_slots does.
 * Same element-type, stride and alignment rules as pa_write_kv.
 * ------------------------------------------------------------------------- */
pa_status pa_write_kv_at(void* k_cache, void* v_cache, const void* k_new,
                         const void* v_new, const int32_t* block_tables,
                         int32_t num_seqs, int32_t max_blocks_per_seq,
                         const int32_t* seq_ids, const int32_t* positions,
                         int32_t num_tokens, int64_t new_token_stride,
                         int32_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                         int64_t* slots_out, void* stream);

/* ---------------------------------------------------------------------------
 * pa_copy_blocks  (copy-on-write)
 *
 * [nalar] "Sharing blok dapat menghindari duplikasi state KV" and [gininih]
 * "Cara kerja PagedAttention": a branch that must modify a shared block gets
 * its own physical copy.  For each pair n: block dst = block_mapping[n][1]
 * receives every KV head of block src = block_mapping[n][0], in both pools
 * (one layer per call).  Bit copy.  Pairs naming a block outside
 * [0, num_blocks) are skipped.  Destinations must be distinct and must not be
 * sources of the same call (otherwise the result depends on the order).
 * ------------------------------------------------------------------------- */
pa_status pa_copy_blocks(void* k_cache, void* v_cache,
                         const int32_t* block_mapping, int32_t num_pairs,
                         int32_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim,
                         pa_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * pa_swap_blocks  (block-granular eviction to, and return from, host memory)
 *
 * [gyaansetu] "The memory problem" and "How PagedAttention fixes this": when
 * HBM runs out, whole sequences need not leave the GPU; small fixed-size
 * pages are moved to CPU memory and brought back.  For each pair n: block
 * dst = block_mapping[n][1] of the destination pools (dst_k, dst_v) receives
 * every KV head of block src = block_mapping[n][0] of the source pools
 * (src_k, src_v); bit copy, one layer per call.  Both pool pairs have the
 * layout of pa.h with the same block_size, num_kv_heads, head_dim and
 * element type; they may have different block counts.  Each of the four pool
 * pointers may be device memory of the current device or pinned host memory
 * (hipHostMalloc; the kernel reads and writes it directly over the host
 * link); block_mapping is int32 [num_pairs][2] in either.  Any other pointer
 * (pageable host memory, another device's memory) gives PA_ERR_UNSUPPORTED
 * before anything is launched.  Swap-out: src = the device pools,
 * dst = the host pools; swap-in: the reverse.  Pairs naming a block outside
 * its pool are skipped.  Destinations must be distinct.  The source and
 * destination pools must be different allocations (PA_ERR_SHAPE when a
 * source and destination pointer are equal; use pa_copy_blocks within a
 * pool).  Results are visible to the host after the stream synchronises.
 * ------------------------------------------------------------------------- */
pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k,
                         const void* src_v, const int32_t* block_mapping,
                         int32_t num_pairs, int32_t src_num_blocks,
                         int32_t dst_num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                         void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_attention
 *
 * [nalar] "Kernel attention harus mengikuti block table": for each sequence's
 * query token the kernel walks the logical context in order and translates
 * each logical block to its physical block before loading K and V.  [nalar]
 * introduction and [gininih] "Batasan dan salah paham umum": the attention
 * equation is unchanged.  For sequence i, query head h, and
 * n = context_lens[i] (tokens 0..n-1 of its logical history):
 *     g     = h / (num_q_heads / num_kv_heads)       (grouped-query heads)
 *     s_t   = scale * dot(q[i][h], K_t[g])           t = 0..n-1
 *     out[i][h] = sum_t softmax(s)_t * V_t[g]        (float32 result)
 * where K_t / V_t is token t's row reached through block_tables[i].
 * n == 0 gives zeros.  n is clamped as described under max_context_len.
 * Scores, softmax and the weighted sum are accumulated in float32 from the
 * exact float32 values of the stored elements.
 *
 * max_context_len is a host-side upper bound of every context_lens[i]; it
 * sizes the fixed-partition grid and workspace (a larger bound is correct,
 * just slower).  On every path a context is clamped to
 *     min(context_lens[i], max_context_len, max_blocks_per_seq*block_size)
 * tokens, so a bound below some context_lens[i] truncates that context to
 * its first max_context_len tokens (and, for the append call, the new token
 * at position context_lens[i]-1 is then neither stored nor attended).
 *
 * Work decomposition.  With partition_size == 0, bf16 K/V, flags == 0 and
 * num_seqs <= 8192 the library splits the (sequence, KV head, 16-token tile)
 * work evenly over one wave per resident wave slot of the device
 * ("stream-K"); a context shared by two waves is merged from float32
 * partials with an exact log-sum-exp rescale.  Otherwise each context is cut
 * into partitions of partition_size tokens (0: the library's choice,
 * pa_decode_partition_size) processed independently and merged the same way;
 * a nonzero partition_size must be a multiple of 16 and of block_size and at
 * most 64 blocks.  The workspace (float32 partials and the decomposition)
 * must hold pa_decode_workspace_size() bytes for the same arguments, be
 * 256-byte aligned, and may be NULL when that size is 0.  Calls that share a
 * workspace must not overlap.
 * flags: 0, or PA_DECODE_VECTOR_ONLY to run the plain vector-ALU kernel
 * (fixed partitions) instead of the matrix-core kernel; both give results
 * within the same tolerance, the flag exists for cross-checking.
 * The result is deterministic: it depends on the logical contents and the
 * decomposition only, never on physical block ids or on timing.  The
 * fixed-partition decomposition is fixed by the arguments; the stream-K one
 * also by the device (its compute-unit count and the kernel's occupancy, see
 * pa_decode_streamk_workers), so two devices of different sizes may round
 * differently, within the same tolerance.
 * ------------------------------------------------------------------------- */
#define PA_DECODE_VECTOR_ONLY 1u

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                 int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size);

/* Waves the stream-K path launches for these arguments on the current
 * device (one per resident wave slot, at most 2048), 0 when the call takes
 * the fixed-partition path, -1 for unsupported arguments or a HIP error.
 * Only the fixed-partition answer is available without a GPU.               */
int32_t pa_decode_streamk_workers(int32_t num_seqs, int32_t head_dim,
                                  int32_t block_size, int32_t partition_size,
                                  pa_dtype dtype, uint32_t flags);

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_context_len,
                                int32_t partition_size, pa_dtype dtype,
                                uint32_t flags);

pa_status pa_decode_attention(float* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale,
                              int32_t partition_size, void* workspace,
                              size_t workspace_bytes, pa_dtype dtype,
                              uint32_t flags, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_attention_append  (write the new tokens, then attend)
 *
 * The decode step of [gyaansetu] "Apa itu KV Cache?": each sequence's new
 * token is stored in the cache and attended together with its history.  For
 * every sequence i with 1 <= context_lens[i] <= max_blocks_per_seq *
 * block_size, row i of k_new / v_new ([num_seqs][num_kv_heads][head_dim],
 * token stride new_token_stride elements, 0 = num_kv_heads*head_dim) is the
 * token at position context_lens[i]-1.  Results equal
 *     pa_write_kv_at(positions[i] = context_lens[i]-1, seq_ids = NULL)
 *     followed by pa_decode_attention with the same arguments:
 * the row is stored at its slot (skipped, as there, when the table entry is
 * outside the pool) and the output attends over positions
 * 0 .. context_lens[i]-1 with the new token's K/V taken from k_new / v_new.
 * Rows of sequences with an empty context are not read.  On the stream-K
 * path the decode kernel itself reads the new rows and stores them (one
 * launch fewer); on the fixed-partition path the rows are stored first.
 * Workspace, decomposition, errors and determinism as pa_decode_attention;
 * k_new / v_new must be 16-byte aligned with 16-byte token strides.
 * ------------------------------------------------------------------------- */
pa_status pa_decode_attention_append(float* out, const void* q, void* k_cache,
                                     void* v_cache, const void* k_new,
                                     const void* v_new, int64_t new_token_stride,
                                     const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, int32_t max_blocks_per_seq,
                                     int32_t max_context_len, float scale,
                                     int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, pa_dtype dtype,
                                     uint32_t flags, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_attention_shared  (decode of groups that share a prefix)
 *
 * [nalar] "Sharing blok dapat menghindari duplikasi state KV" and [gininih]
 * "Cara kerja PagedAttention": sequences sampled from one prompt (parallel
 * sampling, beam candidates) map the blocks of their common prefix to the
 * same physical blocks.  This call computes exactly what
 * pa_decode_attention_append (k_new / v_new given) or pa_decode_attention
 * (both NULL) computes for the same arguments, but reads each shared block
 * once per group instead of once per member: the pages' kernel reads every
 * sequence's context through its own table, so a block shared by m
 * sequences crosses the memory bus m times.
 *
 * Groups are consecutive ranges of sequences: group g holds sequences
 * group_start[g] .. group_start[g+1]-1 (int32 [num_groups+1], increasing,
 * group_start[0] = 0, group_start[num_groups] = num_seqs) whose first
 * shared_len[g] tokens (int32 [num_groups]) map, block by block, to the same
 * physical blocks in every member's table.  The library reads those tokens
 * through the table of the group's first member.  Per group it uses the
 * largest multiple of max(16, block_size) tokens that is <= shared_len[g]
 * and < every member's context length (so each member's last token, the
 * one a step appends, is always its own); only the first 16 / G members
 * (G = num_q_heads / num_kv_heads) of a group are read together, later ones
 * attend over their whole context on their own.  A group with a single
 * member, or nothing left to share, is plain decode.  Both arrays live in
 * device memory and are not validated on the host: a group layout that
 * breaks this contract gives unspecified results, never an access outside
 * a buffer.
 *
 * Two stream-K passes run: one over the (group, KV head) prefixes, the G
 * heads of up to 16 / G members stacked in one matrix-core tile, then one
 * over every (sequence, KV head)'s own tokens; a last kernel combines the
 * two float32 results of each head with their log2-sum-exp (exact in real
 * arithmetic; the rounding differs from the single-pass call within the
 * decode tolerance).  bf16 K/V only, num_seqs <= 4096, 1 <= num_groups <=
 * 2048, block_size >= 8; the workspace must hold
 * pa_decode_shared_workspace_size() bytes, 256-byte aligned.  Other
 * arguments, errors and determinism as pa_decode_attention_append.
 * ------------------------------------------------------------------------- */
size_t pa_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       pa_dtype dtype);

pa_status pa_decode_attention_shared(float* out, const void* q, void* k_cache,
                                     void* v_cache, const void* k_new,
                                     const void* v_new, int64_t new_token_stride,
                                     const int32_t* block_tables,
                                     const int32_t* context_lens,
                                     const int32_t* group_start,
                                     const int32_t* shared_len, int32_t num_groups,
                                     int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq,
                                     int32_t max_context_len, float scale,
                                     void* workspace, size_t workspace_bytes,
                                     pa_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * pa_decode_attention_noalloc  (decode with no allocation and no workspace)
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  With k_new
 * and v_new given it is pa_decode_attention_append, with both NULL it is
 * pa_decode_attention; arguments, results, decomposition and determinism are
 * exactly theirs, except that there is no workspace argument: the partials
 * live in a static device array of PA_NOALLOC_MAX_WORKSPACE bytes that the
 * library holds on every GPU it runs on until the process ends.  A call
 * whose workspace (pa_decode_workspace_size for the same arguments) exceeds
 * that returns PA_ERR_WORKSPACE before anything is launched; the stream-K
 * path of every supported shape fits.  The call allocates nothing (no
 * hipMalloc or other allocating routine); the first call on a device looks
 * up the array's device address once.  All calls on one GPU share the array
 * and its contents between calls are unspecified: calls that may overlap on
 * one GPU (different streams, or host threads) race and must be ordered by
 * the caller.  One of k_new / v_new NULL without the other: PA_ERR_NULL.
 * ------------------------------------------------------------------------- */
#define PA_NOALLOC_MAX_WORKSPACE ((size_t)34 << 20)

pa_status pa_decode_attention_noalloc(float* out, const void* q, void* k_cache,
                                      void* v_cache, const void* k_new,
                                      const void* v_new, int64_t new_token_stride,
                                      const int32_t* block_tables,
                                      const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq,
                                      int32_t max_context_len, float scale,
                                      int32_t partition_size, pa_dtype dtype,
                                      uint32_t flags, void* stream);

/* ---------------------------------------------------------------------------
 * pa_prefill_attention  (multi-query paged attention: a prompt chunk)
 *
 * The prefill side of [bicarait] "Blueprint Arsitektur 3: Chunked Prefill":
 * a long prompt is processed a chunk at a time, every chunk attending to the
 * cache through the same block tables as the decode.  Sequence i has L_i =
 * query_start[i+1] - query_start[i] query tokens, rows query_start[i] ..
 * query_start[i+1]-1 of q and out; its context n_i = context_lens[i]
 * (clamped to [0, max_blocks_per_seq * block_size]) counts the chunk, whose
 * K/V must already be in the cache (pa_write_kv).  Query token j sits at
 * position n_i - L_i + j and attends causally to positions 0 .. n_i - L_i + j
 * (softmax attention as pa_decode_attention, grouped-query heads likewise);
 * a token at a negative position (L_i > n_i) sees nothing and gets zeros.
 * L_i = 1 is exactly the decode.
 *   q      [num_q_tokens][num_q_heads][head_dim] bf16
 *   out    [num_q_tokens][num_q_heads][head_dim] float32
 *   query_start [num_seqs + 1] int32, non-decreasing, query_start[0] >= 0,
 *          query_start[num_seqs] <= num_q_tokens (device memory).  Rows of a
 *          sequence that breaks this are not written; neither are rows of
 *          tokens j >= max_query_len (pass max_query_len >= every L_i).
 * bf16 only, block_size >= 16, num_q_heads / num_kv_heads <= 16, head_dim
 * 64 or 128 (else PA_ERR_UNSUPPORTED).  No workspace; deterministic.
 * Arithmetic: scores, softmax and the running sums in float32 from the
 * stored bf16 values; the weighted sum of V on the fp16 matrix cores, with
 * the weights rounded to fp16 (11 significant bits) and V scaled by 2^-4 into
 * fp16, which holds it exactly for 2^-10 <= |v| <= 1.05e6 (smaller values
 * keep an absolute error under 2^-21; larger ones overflow), accumulated in
 * float32.  The result stays within the decode's 2e-3 tolerance of exact
 * attention (measured 4e-4 on the chunked-prefill workload).
 * ------------------------------------------------------------------------- */
pa_status pa_prefill_attention(float* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens,
                               const int32_t* query_start, int32_t num_seqs,
                               int32_t num_q_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq,
                               int32_t max_query_len, float scale,
                               pa_dtype dtype, void* stream);

/* Text of a status code (static storage).  Takes any integer (a pa_status
 * value or not); codes that are not a pa_status give "unknown status". */
const char* pa_status_string(int status);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
