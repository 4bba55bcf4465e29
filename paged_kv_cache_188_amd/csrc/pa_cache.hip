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

// Streaming (non-temporal) 16-byte load, for rows read exactly once.
// Measured on MI355X (history writes of 131k / 338k / 524k tokens by the
// run kernel below): 1-3 % faster than ordinary loads, which leave the
// source rows in L2 and the Infinity Cache in place of lines still useful.
__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
  return __builtin_bit_cast(uint4,
                            __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
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

// Large writes: each workgroup of four waves owns a window of 8 tokens
// (windows renumbered with xcd_run), and the K rows are staged in LDS so the
// stores can be laid out by line.  A K pool line (128 bytes) holds one
// 16-byte granule of 8 consecutive slots of a block (slots 8a .. 8a+7 of one
// (block, head, granule)), and the 8 tokens whose slots those are are usually
// consecutive in the write (a prompt chunk or a history written in order),
// but a window of tokens need not start at such a line boundary.  So the
// tokens are cut into RUNS: a token continues the run of the token before it
// when its slot is the next slot and not the first of a line; otherwise it
// leads a run.  A workgroup stores the runs whose leader lies in its window,
// whole, even when they reach up to 7 tokens into the next window, and skips
// the tokens at the start of its window that continue a run led before it.
// Every line written by consecutive tokens is then written by one workgroup
// in one piece, with streaming stores when its 8 slots are all written
// (ordinary stores for a part of a line, so L2 can still merge it with
// another workgroup's part).  Every token is still stored at exactly its
// own slot by exactly one workgroup, so any slot pattern is handled; tokens
// with no slot (padding, outside the table or the pool) are skipped.  V rows
// are whole lines (a token's row per head) and go straight through.  Rows
// wider than the LDS staging (more than kRunMaxChunks granules) take a
// per-token path over the window, each wave two tokens with all their
// loads issued before their stores.
constexpr int kRunTokens = 8;                     // tokens per window
constexpr int kRunLine = 8;                       // slots per K line
constexpr int kRunOwned = kRunTokens + kRunLine - 1;  // most tokens a workgroup stores
constexpr int kRunWaves = kWriteWaves;
constexpr int kRunThreads = kRunWaves * kWave;
// LDS staging: kRunOwned tokens x (nchunks + 1) granules, kept under 64 KiB
constexpr int kRunMaxChunks = 64 * 1024 / (16 * kRunOwned) - 1;
// Fewer tokens than this (a decode step's one token per sequence) go one
// wave per token instead: the latency of a small write is lower that way
// (64 tokens: ~4 us against ~6 us staged), and there are no runs to gain.
constexpr int kRunMinTokens = 1024;
constexpr int kRunWaveTokens = kRunTokens / kRunWaves;  // per-token path: tokens per wave
static_assert(kRunTokens % kRunWaves == 0, "the per-token path splits a window over the waves");

__global__ __launch_bounds__(kRunThreads) void write_kv_runs_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, const int32_t* __restrict__ block_tables,
    int num_seqs, int max_blocks_per_seq, const int32_t* __restrict__ seq_ids,
    const int32_t* __restrict__ positions, int64_t* __restrict__ slots_out, int num_tokens,
    int64_t token_stride_bytes, int num_blocks, int block_size, int num_kv_heads,
    int head_chunks) {
  extern __shared__ uint4 s_k[];  // [kRunOwned][nchunks + 1] granules
  // slots of tokens j0-1 .. j0+kRunOwned-1 (entry t is token j0-1+t), then
  // the owned tokens: their index (relative to j0), slot and run length
  __shared__ int64_t s_slot[kRunOwned + 1];
  __shared__ int s_tok[kRunOwned];
  __shared__ int64_t s_own_slot[kRunOwned];
  __shared__ int s_run_len[kRunOwned];
  __shared__ int s_owned;
  const int tid = threadIdx.x;
  const int j0 = xcd_run(blockIdx.x, gridDim.x) * kRunTokens;
  const int64_t pool_slots = (int64_t)num_blocks * block_size;
  const int nchunks = num_kv_heads * head_chunks;  // granules per token row
  const bool staged = nchunks <= kRunMaxChunks;
  const int span = staged ? kRunOwned + 1 : kRunTokens + 1;
  if (tid < span) {
    const int j = j0 - 1 + tid;
    int64_t slot = -1;
    if (j >= 0 && j < num_tokens) {
      if (slot_mapping) {
        slot = slot_mapping[j];
        if (slot >= pool_slots) slot = -1;  // outside the pool: skipped
      } else {
        slot = token_slot(block_tables, num_seqs, max_blocks_per_seq, seq_ids, positions, j,
                          block_size, num_blocks);
        if (slots_out && tid >= 1 && tid <= kRunTokens) slots_out[j] = slot;
      }
      if (slot < 0) slot = -1;
    }
    s_slot[tid] = slot;
  }
  __syncthreads();
  const int64_t vhead = (int64_t)block_size * head_chunks * 16;  // V bytes per (block, head)
  const int64_t kgran = (int64_t)block_size * 16;                // K bytes per (block, head, granule)
  // byte offsets of granule 0 of a slot's K and V rows in the pools
  auto kbase = [&](int64_t slot) {
    const int64_t blk = slot / block_size, off = slot - blk * block_size;
    return (blk * num_kv_heads * head_chunks * block_size + off) * 16;
  };
  auto vbase = [&](int64_t slot) {
    const int64_t blk = slot / block_size, off = slot - blk * block_size;
    return (blk * num_kv_heads * block_size + off) * head_chunks * 16;
  };
  if (staged) {
    if (tid < kWave) {
      // ownership, in the first wave: lane t holds token j0-1+t; a token
      // continues a run when its slot is the previous token's plus one and
      // not the first of a line
      const int64_t sl = tid <= kRunOwned ? s_slot[tid] : -1;
      const int64_t prev = tid >= 1 && tid <= kRunOwned ? s_slot[tid - 1] : -1;
      const bool cont = tid >= 1 && sl >= 0 && prev >= 0 && sl == prev + 1 &&
                        sl % kRunLine != 0;
      // leaders: every lane that does not continue (lane 0, the token
      // before the window, and lanes past the staging range included)
      const uint64_t lead = __ballot(!cont);
      const int t = tid;
      // the run's leader: the highest leading lane <= t; its end: the lowest
      // leading lane > t (lane kRunOwned + 1 always leads)
      const uint64_t upto = t == 63 ? ~0ull : ((2ull << t) - 1);
      const int first = 63 - __builtin_clzll(lead & upto);
      const uint64_t above = t == 63 ? 0ull : (lead & ~upto);
      const int next = above ? __builtin_ctzll(above) : 64;
      const bool own = t >= 1 && t <= kRunOwned && sl >= 0 && first >= 1 &&
                       first <= kRunTokens;
      const uint64_t owned_mask = __ballot(own);
      if (own) {
        const int n = __builtin_popcountll(owned_mask & ((1ull << t) - 1));
        s_tok[n] = t - 1;
        s_own_slot[n] = sl;
        s_run_len[n] = next - first;
      }
      if (tid == 0) s_owned = __builtin_popcountll(owned_mask);
    }
    __syncthreads();
    const int owned = s_owned;
    const int row = nchunks + 1;  // padded LDS row: the transposed reads hit distinct banks
    const int total = owned * nchunks;
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
        if (e < total) {
          const int64_t src = (int64_t)(j0 + s_tok[i]) * token_stride_bytes + (int64_t)c * 16;
          kx[u] = load_stream(k_new + src);
          vx[u] = load_stream(v_new + src);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + u * kRunThreads;
        const int i = e / nchunks, c = e - i * nchunks;
        if (e < total) {
          s_k[i * row + c] = kx[u];
          const int h = c / head_chunks, w = c - h * head_chunks;
          store_stream(v_cache + vbase(s_own_slot[i]) + h * vhead + w * 16, vx[u]);
        }
      }
    }
    __syncthreads();
    // K: for each (head, granule) c, the owned tokens' granules by
    // consecutive threads, so a run's granules are one contiguous piece of a
    // line; a run of kRunLine tokens fills its line and is streamed
    for (int e = tid; e < owned * nchunks; e += kRunThreads) {
      const int c = e / owned, i = e - c * owned;
      uint8_t* dst = k_cache + kbase(s_own_slot[i]) + c * kgran;
      if (s_run_len[i] == kRunLine)
        store_stream(dst, s_k[i * row + c]);
      else
        *reinterpret_cast<uint4*>(dst) = s_k[i * row + c];
    }
    return;
  }
  // per-token path over the window: wave v takes its kRunWaveTokens tokens
  const int wave = tid / kWave, lane = tid % kWave;
  const int t0 = kRunWaveTokens * wave;
  for (int c = lane; c < nchunks; c += kWave) {
    const int h = c / head_chunks, w = c - h * head_chunks;
    uint4 a[kRunWaveTokens], b[kRunWaveTokens];
#pragma unroll
    for (int t = 0; t < kRunWaveTokens; ++t) {
      a[t] = b[t] = make_uint4(0u, 0u, 0u, 0u);
      if (s_slot[1 + t0 + t] < 0) continue;
      const int64_t src = (int64_t)(j0 + t0 + t) * token_stride_bytes + (int64_t)c * 16;
      a[t] = load_stream(k_new + src);
      b[t] = load_stream(v_new + src);
    }
#pragma unroll
    for (int t = 0; t < kRunWaveTokens; ++t) {
      const int64_t slot = s_slot[1 + t0 + t];
      if (slot < 0) continue;
      // K granules of consecutive tokens of a block share lines, which
      // ordinary stores let L2 merge before write-back; a V row is whole
      // lines, streamed
      *reinterpret_cast<uint4*>(k_cache + kbase(slot) + c * kgran) = a[t];
      store_stream(v_cache + vbase(slot) + h * vhead + w * 16, b[t]);
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
  const size_t lds = nchunks <= kRunMaxChunks ? (size_t)kRunOwned * (nchunks + 1) * 16 : 0;
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
  const size_t lds = nchunks <= kRunMaxChunks ? (size_t)kRunOwned * (nchunks + 1) * 16 : 0;
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
