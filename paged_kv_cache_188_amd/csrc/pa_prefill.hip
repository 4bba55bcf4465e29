// Multi-query (chunked prefill) paged attention for gfx950 (MI355X).
//
// What is computed ([bicarait] "Blueprint Arsitektur 3: Chunked Prefill"): a
// prompt is processed a chunk at a time; chunk token j of a sequence whose
// context (chunk included) is n tokens and whose chunk has L tokens sits at
// position n - L + j and attends, with ordinary softmax attention, to the
// positions 0 .. n - L + j, reached block by block through the sequence's
// block table exactly as the decode reaches them ([nalar] "Kernel attention
// harus mengikuti block table").  A token at a negative position (a chunk
// longer than its context) sees no key; its output is zero.
//
// Unlike the decode, this is a dense contraction with reuse: every K/V row of
// the context is used by every query row of the chunk, so the kernel is
// built around the matrix cores and keeps K/V tiles in LDS.
//
// Work decomposition (a gfx950 design, not on the pages).  A "row" is a
// (query token, query head) pair; the G = Hq/Hkv heads of a KV head share its
// K/V, so a workgroup takes the rows of TQ = 128/G consecutive chunk tokens
// of one (sequence, KV head): 128 rows, token-major (row r = token r / G,
// head r % G), 32 per wave.  The workgroup walks the keys from position 0 in
// steps of 32 (two 16-key halves): the 256 threads copy the step's K and V
// rows from the paged pools into LDS (double-buffered: the next step's loads
// are in flight while the current one is used; K goes straight from the pool
// into LDS, V through registers, where it is converted), then every wave
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims (LDS),
//                 B = 32 dims x 16 rows (registers, loaded once);
//                 lane (grp = lane/16, col = lane%16) gets the scores of
//                 row col for keys 4*grp + i of each 16-key half;
//   softmax       online, base 2, the scale applied inside the exponent
//                 (exp2(s*c - m), one fused multiply-add per score), the
//                 running max moved only when a score passes it by 8 (as in
//                 the decode); each row hides keys past its own position
//                 (causal), which only steps on the diagonal need to check;
//   O += P V      v_mfma_f32_16x16x32_f16 with A = P (16 rows x 32 keys,
//                 taken straight from the scores' registers: k index
//                 8*grp + e is key 4*grp + e of half 0 for e < 4 and of half
//                 1 for e >= 4) and B = V in the same key order, both fp16:
//                 the weights (in [0, 256] under the lazy maximum) keep 11
//                 significant bits, and V, scaled by 2^-4 when it is staged
//                 in LDS, is exact in fp16 for 2^-10 <= |v| <= 1.05e6; the
//                 products accumulate in float32.  (bf16 weights would keep
//                 8 bits: on the chunked-prefill workload that puts the
//                 maximum error at 2.8e-3 against the oracle, over the
//                 2e-3 bound; fp16 gives 4.0e-4, and needs one MFMA per tile
//                 where the hi + lo bf16 split of the weights needed two.)
//                 V's B operand (keys along k) is read from the row-major
//                 V tile with gfx950's transposing LDS load
//                 (ds_read_b64_tr_b16), which reads 32 bytes from each of
//                 16 rows; a 32-byte pad per V row starts consecutive rows
//                 8 banks apart, so the 8 rows of each half-wave cover the
//                 64 banks once.  (A 16-byte pad left two-way conflicts:
//                 measured 14.0 M conflict cycles per chunked-prefill call
//                 against 0.1 M, and 1 % more time.)
//                 Output tile nt: lane holds dim 16*nt + col of rows
//                 4*grp + r.
// Latency: the block ids of 64 blocks are fetched at once (one per lane),
// so no K/V load waits for a table lookup; K/V addresses are a uniform
// block base plus a per-lane 32-bit offset fixed for the whole walk; V rows
// past the context are zeroed only on the step that reaches past it, when
// they are stored to LDS; the barrier orders LDS only, so the next step's
// global loads stay in flight across it.  K rows are loaded straight into
// LDS (buffer loads with an LDS destination), so they hold no registers
// while in flight and need no LDS store instructions; the registers this
// frees keep more K operand reads in flight in the score phase (measured:
// 326-334 -> 293-303 us per call).  (Measured on MI355X, the
// chunked-prefill workload of 16 sequences x 512-token chunks: 783 us per
// call with one wave per 16 query rows and no K/V sharing, 605 us with this
// layout; the vector-ALU trims -- uniform base addresses, three-way max, V
// zeroing on one step, transposing V loads instead of byte permutes -- took
// a further 17 %.)
// Occupancy: K and V operands are read from LDS shortly before their MFMAs
// (a few slices or output tiles in flight, not the whole step), which keeps
// the kernel within 168 registers (166 with K bypassing registers): three
// workgroups per CU (three waves per SIMD) instead of two.  The register
// allocation limits how many operand reads are in flight, so registers
// freed elsewhere turn into shorter LDS waits.  (Measured: 417 -> 397 us
// with three workgroups per CU; with two and no spills the fp16 kernel runs
// 10 % slower.  Raising a wave's priority while it issues matrix-core work
// helped when P V ran on the hi + lo pair, 397 -> 388 us, and costs ~1 %
// since the vector ALU is the larger share; interleaving one row half's P V
// with the other half's softmax inside a wave, or one barrier per two steps,
// gained nothing.)
// Scheduling: the work of a (sequence, query tile) pair is its number of key
// steps, known only from device data.  Each workgroup first ranks all pairs
// by decreasing work (a bucketed counting sort in LDS, the same in every
// workgroup, its counts combined with block-wide prefix sums) and takes the
// pair at its own id's rank: workgroups start in id order, so the longest
// items start first and the short ones fill the end.  (Measured: the share
// of workgroup slots in use over the kernel's life was 0.52 with pairs in
// sequence order, the long items of late sequences forming the tail, and
// 0.89 longest first; the ranking itself costs the call ~3 us, against ~31
// us when one thread walked the bucket and per-thread counts.)  The KV heads
// of a pair take consecutive ids.

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// plain vector types (not the uint4 struct) so that register arrays stay in
// registers
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32 * kWaves;  // rows per workgroup
constexpr int kStep = 32;           // keys per step
constexpr float kLazyMax = 8.f;
constexpr float kNegInf = -__builtin_inff();

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight across it (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f16x8_t as_f16x8(u32x4_t v) { return __builtin_bit_cast(f16x8_t, v); }

// Two float32 values as a packed fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// Eight float32 weights as an fp16 A operand.
__device__ __forceinline__ f16x8_t weights_f16(const float (&p)[8]) {
  return as_f16x8(u32x4_t{pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]),
                          pack_f16(p[6], p[7])});
}

// A 16-byte chunk of 8 bf16 V values as 8 fp16 values of V * 2^-4 (an
// exact scaling; the output is scaled back by 2^4).  Values up to
// 65504 * 2^4 (1.05e6) in magnitude keep 11 significant bits (more than
// bf16's 8); below 2^-10 they become fp16 subnormals, with an absolute error
// under 2^-21.
constexpr float kVScale = 1.0f / 16.0f;
__device__ __forceinline__ u32x4_t v_to_f16(u32x4_t v) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_f16(__uint_as_float(v[i] << 16) * kVScale,
                    __uint_as_float(v[i] & 0xffff0000u) * kVScale);
  return r;
}

// Loads of one 16-key half for thread u (0..127) of the half, K straight
// into LDS and V into registers: K chunk c = u + 128 i is granule c / 16 of
// key c % 16, V chunk c is granule c % (D/8) of key c / (D/8); koff / voff
// hold the chunks' byte offsets inside a block's 16 keys, so an address is
// the (wave-uniform) base of (phys, kvh, key0 % BS) plus a 32-bit lane
// offset.  key0 is the half's first position and phys its physical block.
// Every address is inside the pools; V rows past the context are zeroed
// when stored to LDS (not here: a select on the loaded value would wait for
// the load).
// The loads go through buffer descriptors of the (block, KV head) chunk,
// built in scalar registers: the lane supplies only its fixed 32-bit offset
// and the half's position in the block is a scalar offset, so a step's
// addresses cost no vector instructions.  A K load with an LDS destination
// writes lane L's 16 bytes at the (wave-uniform) LDS address + 16 L, so
// chunk i of the wave lands at kdst + 128 i (in 16-byte units), the slots
// the score phase reads.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer, no format conversion

template <int D, int BS>
__device__ __forceinline__ void load_step(const uint16_t* kpool, const uint16_t* vpool, int phys,
                                          int hkv, int kvh, int key0,
                                          const uint32_t (&koff)[D / 64],
                                          const uint32_t (&voff)[D / 64],
                                          u32x4_t* kdst, u32x4_t (&vreg)[D / 64]) {
  const int o = key0 % BS;
  const int64_t cb = ((int64_t)phys * hkv + kvh) * ((int64_t)BS * D);
  constexpr int kChunkBytes = BS * D * 2;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kpool + cb), 0, kChunkBytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vpool + cb), 0, kChunkBytes, kBufferWord3);
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        kr, (__attribute__((address_space(3))) void*)(kdst + 128 * i), 16, (int)koff[i], o * 16, 0,
        0);
    vreg[i] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vr, (int)voff[i], o * D * 2, 0));
  }
}

// max of three (v_max3_f32; fmaxf would first quiet each MFMA result)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Physical block ids of logical blocks 64*chunk .. 64*chunk + 63, one per
// lane (entries past the context, or outside the pool, read as block 0).
template <int BS>
__device__ __forceinline__ int load_ids(const int32_t* bt, int chunk, int n, int num_blocks,
                                        int lane) {
  const int b = chunk * 64 + lane;
  int v = b * BS < n ? bt[b] : 0;
  return (v >= 0 && v < num_blocks) ? v : 0;
}

constexpr int kSortMaxPairs = 16384;  // larger grids keep the natural order
constexpr int kBuckets = 256;

// Key steps of work item pair i = (sequence i / qtiles, query tile i % qtiles):
// 0 for a pair with no chunk token (its workgroups exit at once), else 1 +
// the number of 32-key steps its workgroups walk.
__device__ __forceinline__ int pair_work(const DecodeParams& p, const int32_t* query_start,
                                         int64_t total_q, int tq, int qtiles, int i) {
  const int seq = i / qtiles, qt = i % qtiles;
  const int q0 = query_start[seq];
  const int L = query_start[seq + 1] - q0;
  const int j0 = qt * tq;
  if (q0 < 0 || L < 0 || (int64_t)q0 + L > total_q || j0 >= L) return 0;
  const int n = min(max(p.context_lens[seq], 0), p.max_tokens);
  const int last = n - L + j0 + min(tq, L - j0) - 1;
  return last < 0 ? 1 : last / kStep + 2;
}

// Inclusive prefix sum of v over the workgroup's threads in thread order
// (each wave scans with shuffles; the four wave totals go through `tmp`, 4
// ints of LDS).  Every thread of the workgroup takes part.
__device__ __forceinline__ int block_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += tmp[w];
  __syncthreads();  // `tmp` may be reused
  return v;
}

// The pair at position `rank` when the pairs are ordered by decreasing work
// (bucketed into kBuckets levels, ties in index order): workgroups are
// dispatched in id order, so the longest work starts first and the short
// items fill in at the end (longest-processing-time-first).  Every thread of
// the workgroup takes part and gets the answer; `sm` is kBuckets + kThreads
// + 8 ints of LDS.  The counts are combined with block-wide prefix sums, so
// no thread walks the buckets or the other threads' counts one by one.
__device__ int longest_first_pair(const DecodeParams& p, const int32_t* query_start,
                                  int64_t total_q, int tq, int qtiles, int P, int rank, int* sm) {
  static_assert(kBuckets == kThreads, "one bucket per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* hist = sm;                   // [kBuckets]
  int* res = sm + kBuckets;         // [4]
  int* tmp = res + 4;               // [4]
  // Each thread takes a contiguous slice of the pairs (so index order is kept)
  // and computes the works of its first kCached pairs once.
  constexpr int kCached = 8;
  const int chunk = (P + kThreads - 1) / kThreads;
  const int lo = min(P, tid * chunk), hi = min(P, lo + chunk);
  int wk[kCached];
  int wmax = 0;
#pragma unroll
  for (int k = 0; k < kCached; ++k) {
    wk[k] = lo + k < hi ? pair_work(p, query_start, total_q, tq, qtiles, lo + k) : 0;
    wmax = max(wmax, wk[k]);
  }
  for (int i = lo + kCached; i < hi; ++i)
    wmax = max(wmax, pair_work(p, query_start, total_q, tq, qtiles, i));
  // the largest work of any pair
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wmax = max(wmax, __shfl_xor(wmax, o));
  hist[tid] = 0;
  if (lane == 0) tmp[wave] = wmax;
  __syncthreads();
  wmax = max(max(tmp[0], tmp[1]), max(tmp[2], tmp[3]));
  auto bucket = [&](int w) {
    return w == 0 ? 0 : 1 + (int)((int64_t)(w - 1) * (kBuckets - 2) / max(wmax - 1, 1));
  };
  auto work_at = [&](int k) {  // work of pair lo + k
    return k < kCached ? wk[k] : pair_work(p, query_start, total_q, tq, qtiles, lo + k);
  };
#pragma unroll
  for (int k = 0; k < kCached; ++k)
    if (lo + k < hi) atomicAdd(&hist[bucket(wk[k])], 1);
  for (int i = lo + kCached; i < hi; ++i)
    atomicAdd(&hist[bucket(pair_work(p, query_start, total_q, tq, qtiles, i))], 1);
  __syncthreads();
  // the bucket holding `rank`, buckets taken from the top: thread t holds
  // bucket kBuckets-1-t, and the one whose running count first passes
  // `rank` has it
  {
    const int h = hist[kBuckets - 1 - tid];
    const int cum = block_scan(h, tmp);
    if (cum > rank && cum - h <= rank) {
      res[0] = kBuckets - 1 - tid;
      res[1] = rank - (cum - h);  // position inside the bucket
    }
  }
  __syncthreads();
  const int tb = res[0], want = res[1];
  // the thread whose slice holds that position, then its element
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kCached; ++k) cnt += lo + k < hi && bucket(wk[k]) == tb;
  for (int i = lo + kCached; i < hi; ++i)
    cnt += bucket(pair_work(p, query_start, total_q, tq, qtiles, i)) == tb;
  const int cum = block_scan(cnt, tmp);
  if (cum > want && cum - cnt <= want) {
    int k = want - (cum - cnt);
    for (int i = lo; i < hi; ++i)
      if (bucket(work_at(i - lo)) == tb && k-- == 0) {
        res[2] = i;
        break;
      }
  }
  __syncthreads();
  const int pair = res[2];
  __syncthreads();  // `sm` is reused by the caller
  return pair;
}

template <int D, int BS>
__global__ __launch_bounds__(kThreads, 3) void prefill_flash_kernel(
    const DecodeParams p, const int32_t* __restrict__ query_start, int64_t total_q, int tq,
    int qtiles, int64_t n_items) {
  static_assert(BS >= 16 && BS % 16 == 0, "16-key halves lie in one block");
  constexpr int NS = D / 32;   // 32-dim slices of a row
  constexpr int DV = D / 16;   // output dims per lane per tile
  constexpr int GR = D / 8;    // 16-byte granules per row
  constexpr int HALF = 2 * D;  // 16-byte chunks of K (or V) per 16-key half
  constexpr int CH = D / 64;   // chunks per thread per half, K and V each
  constexpr int VRS = GR + 2;   // V row stride in 16-byte units: two units of padding
  // [buffer][K: half, granule, key | V: key, granule (+ pad)] in 16-byte units
  // [buffer][K (bf16): half, granule, key | V (fp16, scaled): key, granule (+ pad)]
  __shared__ u32x4_t smem[2][2 * HALF + kStep * VRS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;

  // workgroup -> (sequence, query tile) pair, longest work first, and KV head
  const int64_t item = blockIdx.x;
  if (item >= n_items) return;
  const int P = (int)(n_items / p.num_kv_heads);
  const int rank = (int)(item / p.num_kv_heads);
  const int kvh = (int)(item % p.num_kv_heads);
  const bool sorted = P <= kSortMaxPairs;
  const int pair = sorted ? longest_first_pair(p, query_start, total_q, tq, qtiles, P, rank,
                                               reinterpret_cast<int*>(&smem[0][0]))
                          : rank;
  const int seq = pair / qtiles;
  const int qt = sorted ? pair % qtiles : qtiles - 1 - pair % qtiles;  // else: later tiles first
  const int q0 = query_start[seq];
  const int L = query_start[seq + 1] - q0;
  const int j0 = qt * tq;
  if (q0 < 0 || L < 0 || (int64_t)q0 + L > total_q || j0 >= L) return;  // whole workgroup
  const int n = min(max(p.context_lens[seq], 0), p.max_tokens);
  const int G = p.group;
  const int jn = min(tq, L - j0);  // chunk tokens of this workgroup
  const int base = n - L + j0;     // position of token j0

  // scores are scaled by c >= 0 inside the exponent (exp2(s*c - m)); a
  // negative scale is carried by negating Q, which is exact
  const bool neg = p.scale_log2 < 0.f;
  const float c = fmaxf(fabsf(p.scale_log2), 1e-30f);

  // this lane's two rows (one per 16-row half of the wave): query, position
  int pos[2];
  bool live[2];
  bf16x8_t qv[2][NS];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = wave * 32 + h * 16 + col;
    const int tk = rr / G, hd = rr - tk * G;
    live[h] = rr < jn * G && base + tk >= 0;
    pos[h] = live[h] ? base + tk : n - 1;  // a dead row sees every key (results dropped)
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           ((int64_t)(q0 + j0 + (live[h] ? tk : 0)) * p.num_q_heads +
                            (int64_t)kvh * G + (live[h] ? hd : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4_t raw = u32x4_t{0u, 0u, 0u, 0u};
      if (live[h]) raw = *reinterpret_cast<const u32x4_t*>(qrow + 32 * s + 8 * grp);
      if (neg) raw ^= 0x80008000u;
      qv[h][s] = as_bf16x8(raw);
    }
  }
  // the wave's last live position and its rows' first position (wave-uniform)
  int wmax = max(live[0] ? pos[0] : -1, live[1] ? pos[1] : -1);
  int wmin = min(pos[0], pos[1]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    wmax = max(wmax, __shfl_xor(wmax, o));
    wmin = min(wmin, __shfl_xor(wmin, o));
  }
  wmax = __builtin_amdgcn_readfirstlane(wmax);
  wmin = __builtin_amdgcn_readfirstlane(wmin);
  const int last = base + jn - 1;  // the workgroup's last position (<= n - 1)
  const int nsteps = last < 0 ? 0 : last / kStep + 1;

  // loads of one step: thread (half th, index u)
  const int th = tid >> 7, u = tid & 127;
  const uint16_t* kpool = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v_cache);
  const int32_t* bt = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;
  u32x4_t vreg[CH];
  uint32_t koff[CH], voff[CH];  // byte offsets of this thread's chunks in a 16-key half
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = u + 128 * i;
    koff[i] = (uint32_t)(((c >> 4) * BS + (c & 15)) * 16);
    voff[i] = (uint32_t)((c / GR) * D * 2 + (c % GR) * 16);
  }
  // block ids come 64 at a time, one per lane, and are picked with readlane:
  // the K/V loads of a step never wait for a table lookup
  int ids = 0, ids_chunk = -1;
  // this wave's K chunks of a step land in LDS in lane order: chunk
  // u + 128 i of its half at slot th * HALF + u + 128 i
  const int kwave = th * HALF + 64 * ((tid >> 6) & 1);
  auto fetch = [&](int step) {
    const int key0 = __builtin_amdgcn_readfirstlane(step * kStep + th * 16);
    const int blk = key0 / BS;
    if (blk / 64 != ids_chunk) {
      ids_chunk = blk / 64;
      ids = load_ids<BS>(bt, ids_chunk, n, p.num_blocks, lane);
    }
    load_step<D, BS>(kpool, vpool, __builtin_amdgcn_readlane(ids, blk % 64), p.num_kv_heads, kvh,
                     key0, koff, voff, &smem[step & 1][kwave], vreg);
  };
  // byte offset of this lane's transposing-load source in the V tile (key
  // 4*grp + col/4, dims 4*(col%4) .. +3 of dim tile 0)
  const int vlane = (4 * grp + (col >> 2)) * VRS * 16 + (col & 3) * 8;
  f32x4_t acc[2][DV];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int nt = 0; nt < DV; ++nt) acc[h][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};

  // this thread's LDS slots for its V chunks (the same every step)
  int vslot[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = u + 128 * i;
    vslot[i] = 2 * HALF + (th * 16 + c / GR) * VRS + c % GR;
  }
  if (nsteps > 0) fetch(0);
  for (int step = 0; step < nsteps; ++step) {
    u32x4_t* buf = smem[step & 1];
    // first key of this thread's half (the same for the whole wave)
    const int skey0 = __builtin_amdgcn_readfirstlane(step * kStep + th * 16);
    if (skey0 + 16 > n) {  // keys past the context: V rows zeroed (wave-uniform test)
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = u + 128 * i;
        if (skey0 + c / (D / 8) >= n) vreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) buf[vslot[i]] = v_to_f16(vreg[i]);
    // this wave's K chunks, loaded straight into LDS, have landed
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    lds_barrier();
    if (step + 1 < nsteps) fetch(step + 1);
    if (step * kStep > wmax) continue;  // nothing left for this wave's rows

    // S^T = K Q^T: sc[half][row half]; all K operands first, then the four
    // accumulations interleaved
    f32x4_t sc[2][2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int h = 0; h < 2; ++h) sc[kh][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8_t a[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) a[kh] = as_bf16x8(buf[kh * HALF + (4 * s + grp) * 16 + col]);
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sc[kh][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kh], qv[h][s], sc[kh][h], 0, 0, 0);
    }
    // B operands of P V, read before the softmax so the loads overlap it.
    // Dim tile nt: lane (grp, n) holds V at keys 4*grp + j and 16 + 4*grp + j
    // (j = 0..3; the order of P's elements) and dim 16*nt + n, read with two
    // transposing LDS loads: source lane 4*j + r of a 16-lane group supplies
    // key 4*grp + j (+16), dims 16*nt + 4*r .. +3
    const char* vl = reinterpret_cast<const char*>(buf + 2 * HALF) + vlane;
    auto vop = [&](int nt) {
      const v4s_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s_t*)(vl + nt * 32));
      const v4s_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s_t*)(vl + 16 * VRS * 16 + nt * 32));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo4), h2 = __builtin_bit_cast(u32x2_t, hi4);
      return u32x4_t{l2.x, l2.y, h2.x, h2.y};
    };
    // softmax: exponent arguments s * c - m (the causal mask only on steps
    // that reach past some row's position), lazy reference point
    const bool diag = step * kStep + kStep - 1 > wmin;
    float x[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[h][4 * kh + i] = sc[kh][h][i];
    if (diag) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (step * kStep + kh * 16 + 4 * grp + i > pos[h]) x[h][4 * kh + i] = kNegInf;
    }
    float lmax[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      lmax[h] = max3f(max3f(x[h][0], x[h][1], x[h][2]), max3f(x[h][3], x[h][4], x[h][5]),
                      max3f(x[h][6], x[h][7], x[h][7])) * c;
    if (__any(lmax[0] > m_run[0] + kLazyMax || lmax[1] > m_run[1] + kLazyMax)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float mt = fmaxf(lmax[h], __shfl_xor(lmax[h], 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run[h], mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);  // 0 on the first step
        l_run[h] *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = __shfl(alpha, 4 * grp + r);
#pragma unroll
          for (int nt = 0; nt < DV; ++nt) acc[h][nt][r] *= a;
        }
        m_run[h] = m_new;
      }
    }
    float pw[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) pw[h][i] = __builtin_amdgcn_exp2f(fmaf(x[h][i], c, -m_run[h]));
    // O += P V: fp16 weights (in [0, 256]: 11 significant bits) times the
    // scaled fp16 V, float32 accumulation; V's operand of each output tile
    // read just before its MFMAs.  The running sums add the same rounded
    // weights, two per dot-product instruction, in float32.
    f16x8_t ph[2];
    const f16x2_t ones = f16x2_t{(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ph[h] = weights_f16(pw[h]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        l_run[h] = __builtin_amdgcn_fdot2(f16x2_t{ph[h][2 * i], ph[h][2 * i + 1]}, ones, l_run[h],
                                          false);
    }
#pragma unroll
    for (int nt = 0; nt < DV; ++nt) {
      const f16x8_t b = as_f16x8(vop(nt));
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[h][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[h], b, acc[h][nt], 0, 0, 0);
    }
  }

  // normalise and store: acc[h][nt][r] is row wave*32 + 16h + 4*grp + r,
  // dim 16*nt + col
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float l = l_run[h];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float l_c = __shfl(l, 4 * grp + r);
      const int rr = wave * 32 + h * 16 + 4 * grp + r;
      if (rr >= jn * G) continue;
      const int tk = rr / G, hd = rr - tk * G;
      // a row that sees a key has l >= 1 (its largest weight is >= 1); the
      // factor 2^4 undoes V's scaling
      const float inv = base + tk >= 0 ? (1.0f / kVScale) / l_c : 0.f;
      float* dst = p.out + ((int64_t)(q0 + j0 + tk) * p.num_q_heads + (int64_t)kvh * G + hd) * D +
                   col;
      // streaming stores: the output is not read back here, and the lines
      // are not left dirty in L2 for the end-of-kernel write-back
#pragma unroll
      for (int nt = 0; nt < DV; ++nt) __builtin_nontemporal_store(acc[h][nt][r] * inv, dst + 16 * nt);
    }
  }
}

template <int D>
hipError_t launch_d(const DecodeParams& p, const int32_t* query_start, int64_t total_q, int tq,
                    int qtiles, int64_t items, int block_size, hipStream_t stream) {
  const dim3 grid((unsigned)items), block(kThreads);
  if (block_size == 16)
    hipLaunchKernelGGL((prefill_flash_kernel<D, 16>), grid, block, 0, stream, p, query_start,
                       total_q, tq, qtiles, items);
  else if (block_size == 32)
    hipLaunchKernelGGL((prefill_flash_kernel<D, 32>), grid, block, 0, stream, p, query_start,
                       total_q, tq, qtiles, items);
  else
    hipLaunchKernelGGL((prefill_flash_kernel<D, 64>), grid, block, 0, stream, p, query_start,
                       total_q, tq, qtiles, items);
  return hipGetLastError();
}

}  // namespace

int prefill_tokens_per_workgroup(int group) { return kRows / group; }
int prefill_threads_per_workgroup() { return kThreads; }

hipError_t launch_prefill(const DecodeParams& p, const int32_t* query_start, int64_t total_q,
                          int max_query_len, int head_dim, int block_size, hipStream_t stream) {
  const int tq = prefill_tokens_per_workgroup(p.group);
  const int qtiles = (max_query_len + tq - 1) / tq;
  const int64_t items = (int64_t)p.num_seqs * p.num_kv_heads * qtiles;
  if (items == 0) return hipSuccess;
  return head_dim == 128
             ? launch_d<128>(p, query_start, total_q, tq, qtiles, items, block_size, stream)
             : launch_d<64>(p, query_start, total_q, tq, qtiles, items, block_size, stream);
}

}  // namespace pa
