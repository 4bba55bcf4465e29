// Internal declarations shared by the HIP sources of libpa (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kWave = 64;

// Launchers: called by the C ABI after validation.  Each enqueues on `stream`
// and returns hipGetLastError() of the launch.
hipError_t launch_compute_slots(int64_t* slots, const int32_t* block_tables, int num_seqs,
                                int max_blocks_per_seq, const int32_t* seq_ids,
                                const int32_t* positions, int num_tokens, int block_size,
                                int num_blocks, hipStream_t stream);

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int num_tokens, int64_t token_stride_bytes,
                           int num_blocks, int block_size, int num_kv_heads, int row_bytes,
                           hipStream_t stream);

hipError_t launch_write_kv_at(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                              const int32_t* block_tables, int num_seqs, int max_blocks_per_seq,
                              const int32_t* seq_ids, const int32_t* positions,
                              int64_t* slots_out, int num_tokens, int64_t token_stride_bytes,
                              int num_blocks, int block_size, int num_kv_heads, int head_bytes,
                              hipStream_t stream);

// Store row i of k_new / v_new at position context_lens[i]-1 of sequence i
// (skipped for an empty context, a context beyond max_tokens <=
// max_blocks*block_size, or an invalid table entry).  One wave per sequence.
hipError_t launch_append_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            int64_t token_stride_bytes, const int32_t* block_tables,
                            const int32_t* context_lens, int num_seqs, int max_blocks_per_seq,
                            int max_tokens, int num_blocks, int block_size, int num_kv_heads,
                            int head_bytes, hipStream_t stream);

// Block block_mapping[n][0] of the source pools -> block block_mapping[n][1]
// of the destination pools (pairs outside either pool are skipped).
hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* block_mapping, int num_pairs, int src_blocks,
                              int dst_blocks, int64_t block_bytes, hipStream_t stream);

struct DecodeParams {
  float* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  // fixed-partition path: partials [S][Hq][P] (m, l) and [S][Hq][P][D] (acc)
  // stream-K path: partials [W][2][G] (m, l) and [W][2][G][D] (acc)
  float* ws_m;        // running maxima (log2 domain; the reference point of l and acc)
  float* ws_l;        // running sums
  float* ws_acc;      // unnormalised outputs
  int32_t* ws_handoff; // stream-K: [max_workers][2] per wave {segment it hands on, last wave
                       // sharing it} or {-1, -1}; every launched wave writes its entry
  // stream-K with the new token appended in the same launch (else null): row
  // i of k_new / v_new ([S][Hkv][D], token stride new_stride elements) is
  // sequence i's token at position ctx-1; it is attended from these rows and
  // stored into its cache slot
  const void* k_new;
  const void* v_new;
  int64_t new_stride;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;          // num_q_heads / num_kv_heads
  int num_blocks;
  int max_blocks_per_seq;
  int block_size;
  int partition;      // fixed-partition path: tokens per partition
  int max_partitions; // fixed-partition path: P = ceil(max_context_len / partition)
  int max_tokens;     // every context length is clamped to it (min of the caller's bound and
                      // max_blocks_per_seq * block_size), so no index leaves its buffer
  int max_workers;    // stream-K path: waves launched (slot capacity of the workspace)
  float scale_log2;   // scale * log2(e)
  // shared-prefix decode (else group_start is null): groups of consecutive
  // sequences sharing the blocks of their first tokens
  const int32_t* group_start;  // [num_groups + 1]
  const int32_t* shared_len;   // [num_groups], tokens
  int num_groups;
  int group_cap;               // most members of a group whose prefix is shared: 16 / group
  float* prefix_out;           // [S][Hq][D]: each member's attention over its group's prefix
  float* prefix_lse;           // [S][Hq]: its log2-sum-exp
  float* lse_out;              // [S][Hq]: log2-sum-exp of the own-token pass's `out`
  int32_t* group_ws;           // written by the prefix pass: [3][num_groups] each group's
                               // first member, members read together, shared tokens used
  int32_t* own_ws;             // written by the own-token pass: [S] each sequence's first
                               // own position (0: not in a sharing group)
};

// Stream-K decomposition limits.
constexpr int kStreamKMaxSeqs = 8192;     // per-sequence prefix kept in LDS
constexpr int kStreamKMaxWorkers = 2048;  // workspace slots (256 CUs x 8 resident waves)
constexpr int kStreamKMinTiles = 8;       // a worker gets at least this many 16-token tiles

enum class DecodePath { kStreamK, kPartition };

// Resident waves per CU of the stream-K kernel for head_dim (-1 on error).
int streamk_workers_per_cu(int head_dim);

// Which path pa_decode_attention takes (host rule shared with the size query).
DecodePath decode_path(int num_seqs, int block_size, pa_dtype dtype, int partition_size,
                       bool vector_only);

hipError_t launch_decode(const DecodeParams& p, int head_dim, int block_size, pa_dtype dtype,
                         bool vector_only, DecodePath path, hipStream_t stream);

// Multi-query (chunked prefill) attention, bf16, block_size >= 16: one
// workgroup per (sequence, KV head, prefill_tokens_per_workgroup(G) chunk
// tokens).
int prefill_tokens_per_workgroup(int group);
int prefill_threads_per_workgroup();
hipError_t launch_prefill(const DecodeParams& p, const int32_t* query_start, int64_t total_q,
                          int max_query_len, int head_dim, int block_size, hipStream_t stream);

// Workspace offsets (bytes); shared by the size query and the launch.
struct DecodeWorkspace {
  size_t m_off, l_off, acc_off, handoff_off, prefix_out_off, prefix_lse_off, lse_off, group_off,
      own_off, total;
};
DecodeWorkspace decode_workspace_partition(int num_seqs, int num_q_heads, int head_dim,
                                           int max_partitions);
DecodeWorkspace decode_workspace_streamk(int num_seqs, int group, int head_dim);
DecodeWorkspace decode_workspace_shared(int num_seqs, int num_q_heads, int head_dim);

// Shared-prefix decode limits (LDS of the stream-K passes).
constexpr int kSharedMaxSeqs = 4096;
constexpr int kSharedMaxGroups = 2048;

}  // namespace pa
