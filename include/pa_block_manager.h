/*
 * pa_block_manager.h -- host-side KV block manager of the paged KV cache.
 *
 * The memory side of PagedAttention, in C++ behind the same C ABI as the
 * kernels (pa.h).  It owns no device memory: it hands out physical block ids
 * of a pool of num_blocks blocks (the pools themselves are the caller's
 * device tensors), keeps each sequence's block table, counts references to
 * shared blocks, and tells the caller which slots new tokens go to and which
 * blocks to copy before a write.  Its outputs feed pa_write_kv (slots),
 * pa_copy_blocks (copy pairs) and pa_decode_attention (tables, lengths).
 *
 * Sources, cited by page title and section:
 *   [gininih]  "Apa itu PagedAttention (Manajemen Memori KV Cache GPU)?",
 *              "Cara kerja PagedAttention": fixed-size KV blocks, a block
 *              table per sequence, physical blocks taken from anywhere in the
 *              pool when the current one is full, sharing between requests,
 *              copy-on-write when a branch diverges.
 *   [nalar]    "PagedAttention: memetakan blok KV logis ke memori fisik tidak
 *              kontigu", "Urutan logis dipisahkan dari penempatan fisik"
 *              (a new physical block when a sequence crosses a block
 *              boundary), "Sisa alokasi dibatasi oleh granularitas
 *              blok" (waste bounded by the block size), "Sharing blok dapat
 *              menghindari duplikasi state KV" (shared while unchanged; a
 *              writer gets its own copy).
 *   [bicarait] "Melihat Lebih Dalam vLLM v0.7 ...", "Blueprint Arsitektur 2"
 *              (allocate only when the current block is full) and "Berbagi
 *              Memori Fisik" (N samples share the prompt's blocks).
 *   [gyaansetu] "KV Cache and PagedAttention: Why Your LLM Server Slows
 *              Down", "The memory problem" and "How PagedAttention fixes
 *              this" (fine-grained eviction: pages, not whole sequences, move
 *              to CPU memory when HBM is full).
 *
 * Policy (fixed, so that results are reproducible):
 *   * Free blocks form a stack; initially block 0 is on top, then 1, 2, ...
 *     A freed block is pushed back (the most recently freed is reused first).
 *   * Appending token p of a sequence: if p is the first position of a new
 *     logical block, a free block is popped.  Otherwise the token goes into
 *     the sequence's last block; if that block is shared (reference count
 *     > 1) it is first copied into a popped block (copy-on-write: the pair
 *     (old, new) is reported, the sequence's table points at the new block,
 *     the old block loses one reference).
 *   * slot = table[p / block_size] * block_size + p % block_size.
 *   * Sequence ids are dense: the lowest free id is reused first.
 *   * Host blocks (a second pool in pinned host memory, num_host_blocks of
 *     them) follow the same stack policy.  Swapping sequences out moves each
 *     distinct block they hold to a host block, in order of first appearance
 *     (sequence by sequence, table order), keeping the sharing between them;
 *     the GPU blocks are freed in that order.  Swapping in is the reverse.
 *     A swapped sequence can be freed or swapped in, nothing else.
 *
 * Every function is host-only (no HIP call, no GPU needed), returns a
 * pa_status, and leaves the manager unchanged when it fails.  A manager may
 * be used from several threads; calls are serialised internally.
 */
#ifndef PA_BLOCK_MANAGER_H_
#define PA_BLOCK_MANAGER_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* Occupancy of the pool.  A physical block is "used" while some sequence's
 * table holds it, "shared" while two or more do.
 *   logical_blocks   sum over live sequences of their table lengths (what
 *                    private copies of every table would need)
 *   logical_tokens   sum of the live sequences' lengths
 *   stored_tokens    tokens held by used blocks, each block counted once
 *   physical_slots   used_blocks * block_size
 * Tail waste = 1 - stored_tokens / physical_slots; saving from sharing =
 * 1 - used_blocks / logical_blocks.  All of these count GPU blocks and
 * resident sequences only. */
typedef struct pa_bm_stats {
  int32_t num_blocks;
  int32_t free_blocks;
  int32_t used_blocks;
  int32_t shared_blocks;
  int32_t live_sequences;    /* resident (not swapped out) */
  int64_t logical_blocks;
  int64_t logical_tokens;
  int64_t stored_tokens;
  int64_t physical_slots;
  int32_t swapped_sequences;
  int32_t num_host_blocks;
  int32_t free_host_blocks;
} pa_bm_stats;

/* A manager of num_blocks blocks of block_size tokens (block_size >= 1),
 * at most max_seqs live sequences of at most max_blocks_per_seq blocks each,
 * and no host blocks.  *out receives the manager (release with
 * pa_bm_destroy). */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                       int32_t max_blocks_per_seq, pa_block_manager** out);

/* The same with num_host_blocks (>= 0) blocks of host memory to swap to. */
pa_status pa_bm_create_with_host(int32_t num_blocks, int32_t num_host_blocks,
                                 int32_t block_size, int32_t max_seqs,
                                 int32_t max_blocks_per_seq, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new empty sequence; *seq receives its id.  PA_ERR_CAPACITY when max_seqs
 * sequences are live. */
pa_status pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq);

/* A new sequence sharing every block of `parent` (resident; its tokens so
 * far); *child receives its id.  Nothing is copied now: the first write into a shared
 * partial block copies it (copy-on-write). */
pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child);

/* End a sequence: each of its blocks loses one reference; blocks no other
 * sequence holds return to the free stack (in table order, so the last
 * block freed is reused first). */
pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq);

/* Reserve slots for counts[i] new tokens of sequence seq_ids[i], i = 0 ..
 * n-1, in that order (a sequence may appear once).  slots (int64,
 * sum(counts) entries) receives the slot of every new token, sequence by
 * sequence, token by token.  copy_pairs (int32 [n][2], may be NULL when no
 * sequence can need a copy) receives the (src, dst) copy-on-write pairs in
 * the order they occur, and *num_copies their number (at most one per
 * sequence).  All or nothing: PA_ERR_SHAPE for an unknown, swapped or
 * repeated sequence or a negative count (checked first), else PA_ERR_CAPACITY when a
 * table's length or the free blocks would not suffice; either leaves the
 * manager unchanged. */
pa_status pa_bm_append(pa_block_manager* bm, const int32_t* seq_ids, const int32_t* counts,
                       int32_t n, int64_t* slots, int32_t* copy_pairs, int32_t* num_copies);

/* Swap sequences seq_ids[0 .. n-1] (resident, distinct) out to host blocks.
 * pairs (int32 [number of distinct blocks][2]; may be NULL when they hold
 * none) receives the (GPU block, host block) pairs to pass to
 * pa_swap_blocks (source = the device pools), *num_pairs their number.
 * PA_ERR_SHAPE for an unknown, repeated or swapped sequence, or when a block
 * is also held by a sequence not listed; PA_ERR_CAPACITY when the free host
 * blocks do not suffice; either leaves the manager unchanged.  The freed GPU
 * blocks may be reused at once: the caller runs the copy before anything
 * writes them (stream order). */
pa_status pa_bm_swap_out(pa_block_manager* bm, const int32_t* seq_ids, int32_t n,
                         int32_t* pairs, int32_t* num_pairs);

/* Swap sequences seq_ids[0 .. n-1] (swapped, distinct) back in: pairs
 * receives the (host block, GPU block) pairs (source = the host pools).
 * Errors as pa_bm_swap_out, with GPU blocks as the capacity. */
pa_status pa_bm_swap_in(pa_block_manager* bm, const int32_t* seq_ids, int32_t n,
                        int32_t* pairs, int32_t* num_pairs);

/* Block tables and lengths of resident sequences seq_ids[0 .. n-1]: tables
 * (int32 [n][max_blocks_per_seq]) row i receives sequence i's physical
 * blocks followed by -1; lens (int32 [n]) its token count.  PA_ERR_SHAPE for
 * an unknown or swapped sequence. */
pa_status pa_bm_tables(const pa_block_manager* bm, const int32_t* seq_ids, int32_t n,
                       int32_t* tables, int32_t* lens);

/* Current occupancy (see pa_bm_stats). */
pa_status pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H_ */
