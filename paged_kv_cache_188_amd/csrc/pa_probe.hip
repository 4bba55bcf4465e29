// Memory bandwidth probes (include/pa_probe.h): plain non-temporal 16-byte
// reads, no arithmetic beyond an XOR that keeps every load alive and lets a
// test check that each byte was read.  A contiguous stream, and the decode
// call's own K/V chunk gather through the block tables.

#include <cstdint>

#include "pa_internal.h"
#include "pa_probe.h"

namespace {

using u32x4_t = uint32_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeWaves = kProbeThreads / pa::kWave;

__device__ __forceinline__ uint32_t load_xor(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return v.x ^ v.y ^ v.z ^ v.w;
}

// XOR of `acc` over the workgroup, stored by thread 0 in sink[blockIdx.x].
__device__ __forceinline__ void store_block_xor(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t part[kProbeWaves];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (threadIdx.x % pa::kWave == 0) part[threadIdx.x / pa::kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kProbeWaves; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

// All workgroups stride over n16 granules together, four loads in flight
// per thread.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ buf,
                                                                  int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint32_t a = load_xor(buf + i);
    const uint32_t b = load_xor(buf + i + stride);
    const uint32_t c = load_xor(buf + i + 2 * stride);
    const uint32_t d = load_xor(buf + i + 3 * stride);
    acc ^= (a ^ b) ^ (c ^ d);
  }
  for (; i < n16; i += stride) acc ^= load_xor(buf + i);
  store_block_xor(acc, sink);
}

struct GatherArgs {
  const uint4* k;
  const uint4* v;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, num_kv_heads, max_blocks_per_seq, block_size, num_blocks;
  int chunk16;  // 16-byte granules per (block, KV head) chunk: a multiple of 64
};

// Blocks sequence i reads: ceil(ctx / block_size) for 0 < ctx <= the table's
// capacity, else none.
__device__ __forceinline__ int seq_blocks(const GatherArgs& a, int i) {
  const int n = a.context_lens[i];
  const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
  return (n > 0 && n <= cap) ? (n + a.block_size - 1) / a.block_size : 0;
}

// s_prefix[i] = blocks of sequences 0 .. i-1 (i = 0 .. S), built by the
// workgroup: each thread sums a slice, thread 0 scans the slice sums.
__device__ void block_prefix(const GatherArgs& a, int* s_prefix) {
  __shared__ int slice_sum[kProbeThreads];
  const int S = a.num_seqs;
  const int per = (S + kProbeThreads - 1) / kProbeThreads;
  const int lo = min(S, (int)threadIdx.x * per), hi = min(S, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += seq_blocks(a, i);
  slice_sum[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int t = 0; t < kProbeThreads; ++t) {
      const int x = slice_sum[t];
      slice_sum[t] = run;
      run += x;
    }
    s_prefix[S] = run;
  }
  __syncthreads();
  int run = slice_sum[threadIdx.x];
  for (int i = lo; i < hi; ++i) {
    s_prefix[i] = run;
    run += seq_blocks(a, i);
  }
  __syncthreads();
}

// Items are (sequence, KV head, logical block) in that order, over the
// blocks each context covers.  Wave w of W takes the contiguous range
// [w*T/W, (w+1)*T/W) of the T items and walks it in order; the table entry
// of the next item is loaded while the current item's K and V chunks are
// read (up to 4 granules of each per lane at once).
__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(const GatherArgs a,
                                                                    uint32_t* sink) {
  extern __shared__ int s_prefix[];  // [S+1]
  block_prefix(a, s_prefix);
  const int S = a.num_seqs, Hkv = a.num_kv_heads;
  const int lane = threadIdx.x % pa::kWave;
  const int64_t W = (int64_t)gridDim.x * kProbeWaves;
  const int64_t w = (int64_t)blockIdx.x * kProbeWaves + threadIdx.x / pa::kWave;
  const int64_t T = (int64_t)Hkv * s_prefix[S];
  const int64_t g0 = w * T / W, g1 = (w + 1) * T / W;
  uint32_t acc = 0;
  if (g0 < g1) {
    // the last sequence whose first item is <= g0 (it is non-empty: an
    // empty one would be followed by one that also qualifies)
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if ((int64_t)Hkv * s_prefix[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    int seq = lo;
    int nb = s_prefix[seq + 1] - s_prefix[seq];
    const int64_t off = g0 - (int64_t)Hkv * s_prefix[seq];
    int kvh = (int)(off / nb), b = (int)(off % nb);
    auto entry = [&](int sq, int blk) {
      return a.block_tables[(int64_t)sq * a.max_blocks_per_seq + blk];
    };
    int phys = entry(seq, b);
    for (int64_t g = g0; g < g1; ++g) {
      // next item and its table entry (issued before this item's loads)
      int nseq = seq, nkvh = kvh, nbk = b + 1, nnb = nb;
      if (nbk == nnb) {
        nbk = 0;
        if (++nkvh == Hkv) {
          nkvh = 0;
          do {
            ++nseq;
          } while (nseq < S && s_prefix[nseq + 1] == s_prefix[nseq]);
          nnb = nseq < S ? s_prefix[nseq + 1] - s_prefix[nseq] : 0;
        }
      }
      const int nphys = (g + 1 < g1) ? entry(nseq, nbk) : 0;
      if (phys >= 0 && phys < a.num_blocks) {
        const int64_t base = ((int64_t)phys * Hkv + kvh) * a.chunk16;
        for (int c = 0; c < a.chunk16; c += 4 * pa::kWave) {
          uint32_t x[8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = c + u * pa::kWave + lane;
            x[u] = i < a.chunk16 ? load_xor(a.k + base + i) : 0u;
            x[4 + u] = i < a.chunk16 ? load_xor(a.v + base + i) : 0u;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) acc ^= x[u];
        }
      }
      seq = nseq, kvh = nkvh, b = nbk, nb = nnb, phys = nphys;
    }
  }
  store_block_xor(acc, sink);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

pa_status pa_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t sink_len,
                        void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || sink_len < 1 || sink_len > PA_PROBE_MAX_SINK)
    return PA_ERR_SHAPE;
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return PA_ERR_NULL;
  if (!aligned16(buf)) return PA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(probe_read_kernel, dim3(sink_len), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_probe_gather(const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, pa_dtype dtype, uint32_t* sink,
                          int32_t sink_len, void* stream) {
  if (num_seqs < 0 || num_kv_heads < 1 || num_blocks < 1 || max_blocks_per_seq < 1 ||
      sink_len < 1 || sink_len > PA_PROBE_MAX_SINK)
    return PA_ERR_SHAPE;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if ((head_dim != 64 && head_dim != 128) ||
      (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs > PA_PROBE_MAX_SEQS) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !sink) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;
  GatherArgs a;
  a.k = static_cast<const uint4*>(k_cache);
  a.v = static_cast<const uint4*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.chunk16 = block_size * head_dim * (dtype == PA_BF16 ? 2 : 4) / 16;
  hipLaunchKernelGGL(probe_gather_kernel, dim3(sink_len), dim3(kProbeThreads),
                     (size_t)(num_seqs + 1) * sizeof(int), static_cast<hipStream_t>(stream), a,
                     sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
