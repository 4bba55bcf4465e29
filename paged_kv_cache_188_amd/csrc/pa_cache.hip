// Slot computation, slot-mapped KV write and copy-on-write block copy for gfx950.
//
// These three operations move or index data only; they are bit-exact.
//
//  * Slots follow the block table of [nalar] "Urutan logis dipisahkan dari
//    penempatan fisik": logical block b of a sequence lives in physical block
//    table[b]; a token keeps its logical order inside its block.
//  * The write stores only the new tokens' K/V ([gyaansetu] "Apa itu KV
//    Cache?").  V pool [NB][Hkv][bs][D]: one token of one KV head is a
//    D-element row (256 B for bf16, D=128).  K pool [NB][Hkv][D/x][bs][x]: the
//    same row split into 16-byte granules, granule w stored at [w][offset].
//    Every store is a full 16-byte granule.
//  * The block copy gives a diverging branch its own copy of a shared block
//    ([nalar] "Sharing blok dapat menghindari duplikasi state KV"); a block is
//    Hkv*bs*D*e contiguous bytes in each pool, streamed with 16-byte loads.

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte store, for writes that fill whole lines.
// Measured on MI355X: a copy of 256 64 KiB blocks took 18.6 us with ordinary
// stores and 4.3 us with these (the written lines are not left dirty in L2
// for the end-of-kernel write-back), and large copies ran at ~1.6x the rate.
__device__ __forceinline__ void store_stream(uint8_t* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
}

// Slot of token j (-1: padding, or an index outside its table or the pool).
__device__ __forceinline__ int64_t token_slot(const int32_t* __restrict__ block_tables,
                                              int num_seqs, int max_blocks_per_seq,
                                              const int32_t* __restrict__ seq_ids,
                                              const int32_t* __restrict__ positions, int j,
                                              int block_size, int num_blocks) {
  const int p = positions[j];
  const int i = seq_ids ? seq_ids[j] : j;
  int64_t slot = -1;
  if (p >= 0 && i >= 0 && i < num_seqs) {
    const int b = p / block_size;
    if (b < max_blocks_per_seq) {
      const int phys = block_tables[(int64_t)i * max_blocks_per_seq + b];
      if (phys >= 0 && phys < num_blocks)
        slot = (int64_t)phys * block_size + (p - b * block_size);
    }
  }
  return slot;
}

__global__ __launch_bounds__(256) void compute_slots_kernel(
    int64_t* __restrict__ slots, const int32_t* __restrict__ block_tables, int num_seqs,
    int max_blocks_per_seq, const int32_t* __restrict__ seq_ids,
    const int32_t* __restrict__ positions, int num_tokens, int block_size, int num_blocks) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= num_tokens) return;
  slots[j] = token_slot(block_tables, num_seqs, max_blocks_per_seq, seq_ids, positions, j,
                        block_size, num_blocks);
}

// Workgroups are dealt to the 8 XCDs of the chip in turn (workgroup b to XCD
// b mod 8).  Renumbered so that each XCD takes one contiguous run of tokens:
// the K granules of consecutive tokens of a block share cache lines, which
// one L2 then merges whole before writing them back.
__device__ __forceinline__ int xcd_run(int b, int n) {
  const int x = b % 8, k = b / 8, q = n / 8, r = n % 8;
  return x * q + min(x, r) + k;
}

// One wave per token; each lane moves 16-byte granules of the token's
// [Hkv][D] row to their places in the two pools.
constexpr int kWriteWaves = 4;

// Token j's K and V rows into slot `slot` of the two pools (one wave).
__device__ __forceinline__ void write_token(uint8_t* __restrict__ k_cache,
                                            uint8_t* __restrict__ v_cache,
                                            const uint8_t* __restrict__ k_new,
                                            const uint8_t* __restrict__ v_new, int j,
                                            int64_t slot, int64_t token_stride_bytes,
                                            int block_size, int num_kv_heads, int head_chunks,
                                            int lane) {
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int nchunks = num_kv_heads * head_chunks;
  const uint8_t* ksrc = k_new + (int64_t)j * token_stride_bytes;
  const uint8_t* vsrc = v_new + (int64_t)j * token_stride_bytes;
  for (int c = lane; c < nchunks; c += kWave) {
    const int h = c / head_chunks;
    const int w = c - h * head_chunks;
    const int64_t kdst = (((blk * num_kv_heads + h) * head_chunks + w) * block_size + off) * 16;
    const int64_t vdst = (((blk * num_kv_heads + h) * block_size + off) * head_chunks + w) * 16;
    const uint4 a = *reinterpret_cast<const uint4*>(ksrc + (int64_t)c * 16);
    const uint4 b = *reinterpret_cast<const uint4*>(vsrc + (int64_t)c * 16);
    // K granules of consecutive tokens of a block share lines, which
    // ordinary stores let L2 merge before write-back (streaming them made a
    // 131k-token history write 3x slower); a V row is whole lines, streamed
    *reinterpret_cast<uint4*>(k_cache + kdst) = a;
    store_stream(v_cache + vdst, b);
  }
}

__global__ __launch_bounds__(kWriteWaves * kWave) void write_kv_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int64_t token_stride_bytes,
    int64_t pool_slots, int block_size, int num_kv_heads, int head_chunks) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int j = xcd_run(blockIdx.x, gridDim.x) * kWriteWaves + wave;
  if (j >= num_tokens) return;
  const int64_t slot = slot_mapping[j];
  if (slot < 0 || slot >= pool_slots) return;  // padding token, or outside the pool
  write_token(k_cache, v_cache, k_new, v_new, j, slot, token_stride_bytes, block_size,
              num_kv_heads, head_chunks, lane);
}

// The slot computation and the write in one launch (one wave per token); the
// slots are also stored when `slots_out` is given.
__global__ __launch_bounds__(kWriteWaves * kWave) void write_kv_at_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ block_tables, int num_seqs, int max_blocks_per_seq,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions,
    int64_t* __restrict__ slots_out, int num_tokens, int64_t token_stride_bytes, int num_blocks,
    int block_size, int num_kv_heads, int head_chunks) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int j = xcd_run(blockIdx.x, gridDim.x) * kWriteWaves + wave;
  if (j >= num_tokens) return;
  const int64_t slot = token_slot(block_tables, num_seqs, max_blocks_per_seq, seq_ids, positions,
                                  j, block_size, num_blocks);
  if (slots_out && lane == 0) slots_out[j] = slot;
  if (slot < 0) return;  // padding token, or an index outside its table or the pool
  write_token(k_cache, v_cache, k_new, v_new, j, slot, token_stride_bytes, block_size,
              num_kv_heads, head_chunks, lane);
}

// Tokens are taken 16 at a time, one workgroup of four waves per group
// (workgroups renumbered with xcd_run).  The K rows of the group are staged
// in LDS, so that the loads read whole token rows and the stores write, for
// each (head, granule), the 16 tokens' granules with 16 consecutive threads:
// when the tokens sit at consecutive offsets of a block (a prompt chunk or a
// history written in order) those granules are one contiguous 256-byte run
// of the K pool.  V rows go straight through (a token's row is contiguous in
// the V pool).  Every token is stored at its own slot, so any slot pattern
// is handled; tokens with no slot (padding, outside the table or the pool)
// are skipped.  Rows wider than the LDS staging (more than kRunMaxChunks
// granules) take a per-token path, each wave four tokens with all their
// loads issued before their stores.
constexpr int kRunTokens = 16;
constexpr int kRunThreads = kWriteWaves * kWave;
// LDS staging: 16 tokens x (nchunks + 1) granules, kept under 64 KiB
constexpr int kRunMaxChunks = 240;
// Fewer tokens than this (a decode step's one token per sequence) go one
// wave per token instead: the latency of a small write is lower that way
// (64 tokens: ~4 us against ~6 us staged), and there are no runs to gain.
constexpr int kRunMinTokens = 1024;

__global__ __launch_bounds__(kRunThreads) void write_kv_runs_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, const int32_t* __restrict__ block_tables,
    int num_seqs, int max_blocks_per_seq, const int32_t* __restrict__ seq_ids,
    const int32_t* __restrict__ positions, int64_t* __restrict__ slots_out, int num_tokens,
    int64_t token_stride_bytes, int num_blocks, int block_size, int num_kv_heads,
    int head_chunks) {
  extern __shared__ uint4 s_k[];  // [16][nchunks + 1] granules
  // byte offsets of granule 0 of each token's K and V rows in the pools, or -1
  __shared__ int64_t s_kbase[kRunTokens], s_vbase[kRunTokens];
  const int tid = threadIdx.x;
  const int j0 = xcd_run(blockIdx.x, gridDim.x) * kRunTokens;
  const int64_t pool_slots = (int64_t)num_blocks * block_size;
  if (tid < kRunTokens) {
    const int j = j0 + tid;
    int64_t slot = -1;
    if (j < num_tokens) {
      if (slot_mapping) {
        slot = slot_mapping[j];
        if (slot >= pool_slots) slot = -1;  // outside the pool: skipped
      } else {
        slot = token_slot(block_tables, num_seqs, max_blocks_per_seq, seq_ids, positions, j,
                          block_size, num_blocks);
        if (slots_out) slots_out[j] = slot;
      }
    }
    int64_t kb = -1, vb = -1;
    if (slot >= 0) {
      const int64_t blk = slot / block_size, off = slot - blk * block_size;
      // K element (h, granule w) at ((blk*Hkv + h)*hc + w)*bs + off; V at
      // ((blk*Hkv + h)*bs + off)*hc + w (granules of 16 bytes)
      kb = (blk * num_kv_heads * head_chunks * block_size + off) * 16;
      vb = (blk * num_kv_heads * block_size + off) * head_chunks * 16;
    }
    s_kbase[tid] = kb;
    s_vbase[tid] = vb;
  }
  __syncthreads();
  const int nchunks = num_kv_heads * head_chunks;  // granules per token row
  const int64_t vhead = (int64_t)block_size * head_chunks * 16;  // V bytes per (block, head)
  const int64_t kgran = (int64_t)block_size * 16;                // K bytes per (block, head, granule)
  if (nchunks <= kRunMaxChunks) {
    const int row = nchunks + 1;  // padded LDS row: the transposed reads hit distinct banks
    const int total = kRunTokens * nchunks;
    // eight granules of K and of V per thread in flight: all loads of a batch
    // are issued before any of them is stored
    constexpr int kBatch = 8;
    for (int e0 = tid; e0 < total; e0 += kBatch * kRunThreads) {
      uint4 kx[kBatch], vx[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + u * kRunThreads;
        const int i = e / nchunks, c = e - i * nchunks;
        kx[u] = vx[u] = make_uint4(0u, 0u, 0u, 0u);
        if (e < total && s_vbase[i] >= 0) {
          const int64_t src = (int64_t)(j0 + i) * token_stride_bytes + (int64_t)c * 16;
          kx[u] = *reinterpret_cast<const uint4*>(k_new + src);
          vx[u] = *reinterpret_cast<const uint4*>(v_new + src);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + u * kRunThreads;
        const int i = e / nchunks, c = e - i * nchunks;
        if (e < total && s_vbase[i] >= 0) {
          s_k[i * row + c] = kx[u];
          const int h = c / head_chunks, w = c - h * head_chunks;
          store_stream(v_cache + s_vbase[i] + h * vhead + w * 16, vx[u]);
        }
      }
    }
    __syncthreads();
    // Whole runs (the 16 tokens at offsets 16m .. 16m+15 of one block) are
    // streamed; partial runs use ordinary stores, so that L2 merges them with
    // the neighbouring group's part of the same lines (written by the same
    // XCD, see xcd_run) before write-back.
    bool whole = s_kbase[0] >= 0 && block_size % kRunTokens == 0 &&
                 (s_kbase[0] / 16) % kRunTokens == 0;
#pragma unroll
    for (int i = 1; i < kRunTokens; ++i) whole = whole && s_kbase[i] == s_kbase[0] + 16 * i;
    for (int e = tid; e < kRunTokens * nchunks; e += kRunThreads) {
      const int c = e / kRunTokens, i = e - c * kRunTokens;  // (head, granule) c, token i
      const int64_t kb = s_kbase[i];
      if (kb < 0) continue;
      if (whole)
        store_stream(k_cache + kb + c * kgran, s_k[i * row + c]);
      else
        *reinterpret_cast<uint4*>(k_cache + kb + c * kgran) = s_k[i * row + c];
    }
    return;
  }
  // per-token path: wave v takes tokens j0 + 4v .. j0 + 4v + 3
  const int wave = tid / kWave, lane = tid % kWave;
  for (int c = lane; c < nchunks; c += kWave) {
    const int h = c / head_chunks, w = c - h * head_chunks;
    uint4 a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = b[t] = make_uint4(0u, 0u, 0u, 0u);
      if (s_vbase[4 * wave + t] < 0) continue;
      const int64_t src = (int64_t)(j0 + 4 * wave + t) * token_stride_bytes + (int64_t)c * 16;
      a[t] = *reinterpret_cast<const uint4*>(k_new + src);
      b[t] = *reinterpret_cast<const uint4*>(v_new + src);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t kb = s_kbase[4 * wave + t], vb = s_vbase[4 * wave + t];
      if (vb < 0) continue;
      // K granules of consecutive tokens of a block share lines, which
      // ordinary stores let L2 merge before write-back; a V row is whole
      // lines, streamed
      *reinterpret_cast<uint4*>(k_cache + kb + c * kgran) = a[t];
      store_stream(v_cache + vb + h * vhead + w * 16, b[t]);
    }
  }
}

// grid = (pair, pool K/V, 16 KiB piece of the block).  Each thread moves up
// to four 16-byte chunks, all loads issued before the stores.  The loads are
// ordinary (the 8 copies of one shared block read the same source), the
// stores streaming.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyPieceBytes = (int64_t)kCopyThreads * kCopyUnroll * 16;

// Block src of the source pools -> block dst of the destination pools (the
// same pools for a copy-on-write copy; a device pool and a pinned host pool
// for a swap, which the kernel reaches directly over the host link).
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint8_t* dst_k, uint8_t* dst_v, const uint8_t* src_k, const uint8_t* src_v,
    const int32_t* __restrict__ block_mapping, int src_blocks, int dst_blocks,
    int64_t block_bytes) {
  const int pair = blockIdx.x;
  const int src = block_mapping[2 * pair];
  const int dst = block_mapping[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* s = reinterpret_cast<const uint4*>((blockIdx.y ? src_v : src_k) +
                                                  (int64_t)src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>((blockIdx.y ? dst_v : dst_k) + (int64_t)dst * block_bytes);
  const int64_t n = block_bytes / 16;
  const int64_t first = (int64_t)blockIdx.z * (kCopyPieceBytes / 16) + threadIdx.x;
  uint4 r[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = first + (int64_t)u * kCopyThreads;
    if (i < n) r[u] = s[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = first + (int64_t)u * kCopyThreads;
    if (i < n) store_stream(reinterpret_cast<uint8_t*>(d + i), r[u]);
  }
}

}  // namespace

hipError_t launch_compute_slots(int64_t* slots, const int32_t* block_tables, int num_seqs,
                                int max_blocks_per_seq, const int32_t* seq_ids,
                                const int32_t* positions, int num_tokens, int block_size,
                                int num_blocks, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = 256;
  const int grid = (num_tokens + threads - 1) / threads;
  hipLaunchKernelGGL(compute_slots_kernel, dim3(grid), dim3(threads), 0, stream, slots,
                     block_tables, num_seqs, max_blocks_per_seq, seq_ids, positions, num_tokens,
                     block_size, num_blocks);
  return hipGetLastError();
}

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int num_tokens, int64_t token_stride_bytes,
                           int num_blocks, int block_size, int num_kv_heads, int head_bytes,
                           hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  if (num_tokens < kRunMinTokens) {
    const int grid = (num_tokens + kWriteWaves - 1) / kWriteWaves;
    hipLaunchKernelGGL(write_kv_kernel, dim3(grid), dim3(kWriteWaves * kWave), 0, stream,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),
                       slot_mapping, num_tokens, token_stride_bytes,
                       (int64_t)num_blocks * block_size, block_size, num_kv_heads,
                       head_bytes / 16);
    return hipGetLastError();
  }
  const int nchunks = num_kv_heads * (head_bytes / 16);
  const size_t lds = nchunks <= kRunMaxChunks ? (size_t)kRunTokens * (nchunks + 1) * 16 : 0;
  hipLaunchKernelGGL(write_kv_runs_kernel, dim3((num_tokens + kRunTokens - 1) / kRunTokens),
                     dim3(kRunThreads), lds, stream, static_cast<uint8_t*>(k_cache),
                     static_cast<uint8_t*>(v_cache), static_cast<const uint8_t*>(k_new),
                     static_cast<const uint8_t*>(v_new), slot_mapping, nullptr, 0, 0, nullptr,
                     nullptr, nullptr, num_tokens, token_stride_bytes, num_blocks, block_size,
                     num_kv_heads, head_bytes / 16);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(kWriteWaves * kWave) void append_kv_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    int64_t token_stride_bytes, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int num_seqs, int max_blocks_per_seq,
    int max_tokens, int num_blocks, int block_size, int num_kv_heads, int head_chunks) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int i = blockIdx.x * kWriteWaves + wave;
  if (i >= num_seqs) return;
  const int n = context_lens[i];
  if (n < 1 || n > max_tokens) return;  // max_tokens <= max_blocks_per_seq * block_size
  const int pos = n - 1;
  const int b = pos / block_size;
  const int phys = block_tables[(int64_t)i * max_blocks_per_seq + b];
  if (phys < 0 || phys >= num_blocks) return;
  write_token(k_cache, v_cache, k_new, v_new, i, (int64_t)phys * block_size + (pos - b * block_size),
              token_stride_bytes, block_size, num_kv_heads, head_chunks, lane);
}
}  // namespace

hipError_t launch_append_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            int64_t token_stride_bytes, const int32_t* block_tables,
                            const int32_t* context_lens, int num_seqs, int max_blocks_per_seq,
                            int max_tokens, int num_blocks, int block_size, int num_kv_heads,
                            int head_bytes, hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  const int grid = (num_seqs + kWriteWaves - 1) / kWriteWaves;
  hipLaunchKernelGGL(append_kv_kernel, dim3(grid), dim3(kWriteWaves * kWave), 0, stream,
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                     static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),
                     token_stride_bytes, block_tables, context_lens, num_seqs,
                     max_blocks_per_seq, max_tokens, num_blocks, block_size, num_kv_heads,
                     head_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_write_kv_at(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                              const int32_t* block_tables, int num_seqs, int max_blocks_per_seq,
                              const int32_t* seq_ids, const int32_t* positions,
                              int64_t* slots_out, int num_tokens, int64_t token_stride_bytes,
                              int num_blocks, int block_size, int num_kv_heads, int head_bytes,
                              hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  if (num_tokens < kRunMinTokens) {
    const int grid = (num_tokens + kWriteWaves - 1) / kWriteWaves;
    hipLaunchKernelGGL(write_kv_at_kernel, dim3(grid), dim3(kWriteWaves * kWave), 0, stream,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),
                       block_tables, num_seqs, max_blocks_per_seq, seq_ids, positions, slots_out,
                       num_tokens, token_stride_bytes, num_blocks, block_size, num_kv_heads,
                       head_bytes / 16);
    return hipGetLastError();
  }
  const int nchunks = num_kv_heads * (head_bytes / 16);
  const size_t lds = nchunks <= kRunMaxChunks ? (size_t)kRunTokens * (nchunks + 1) * 16 : 0;
  hipLaunchKernelGGL(write_kv_runs_kernel, dim3((num_tokens + kRunTokens - 1) / kRunTokens),
                     dim3(kRunThreads), lds, stream, static_cast<uint8_t*>(k_cache),
                     static_cast<uint8_t*>(v_cache), static_cast<const uint8_t*>(k_new),
                     static_cast<const uint8_t*>(v_new), nullptr, block_tables, num_seqs,
                     max_blocks_per_seq, seq_ids, positions, slots_out, num_tokens,
                     token_stride_bytes, num_blocks, block_size, num_kv_heads, head_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* block_mapping, int num_pairs, int src_blocks,
                              int dst_blocks, int64_t block_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int pieces = (int)((block_bytes + kCopyPieceBytes - 1) / kCopyPieceBytes);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2, pieces), dim3(kCopyThreads), 0,
                     stream, static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v),
                     static_cast<const uint8_t*>(src_k), static_cast<const uint8_t*>(src_v),
                     block_mapping, src_blocks, dst_blocks, block_bytes);
  return hipGetLastError();
}

}  // namespace pa
