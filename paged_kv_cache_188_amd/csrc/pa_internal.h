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

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                              int num_pairs, int num_blocks, int64_t block_bytes,
                              hipStream_t stream);

struct DecodeParams {
  float* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;        // [S][Hq][P]    running maxima, log2 domain
  float* ws_l;        // [S][Hq][P]    running sums
  float* ws_acc;      // [S][Hq][P][D] unnormalised outputs
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;          // num_q_heads / num_kv_heads
  int num_blocks;
  int max_blocks_per_seq;
  int partition;      // tokens per partition
  int max_partitions; // P = ceil(max_context_len / partition)
  int max_tokens;     // min(max_blocks_per_seq * block_size, P * partition): every
                      // context length is clamped to it, so no index leaves its buffer
  float scale_log2;   // scale * log2(e)
};

hipError_t launch_decode(const DecodeParams& p, int head_dim, int block_size, pa_dtype dtype,
                         bool vector_only, hipStream_t stream);

// Workspace offsets (bytes) for the decode partials; shared by size query and launch.
struct DecodeWorkspace {
  size_t m_off, l_off, acc_off, total;
};
DecodeWorkspace decode_workspace(int num_seqs, int num_q_heads, int head_dim, int max_partitions);

}  // namespace pa
