// Paged decode attention for gfx950 (MI355X).
//
// What is computed ([nalar] introduction; [gininih] "Batasan dan salah paham
// umum"): ordinary softmax attention of one query token per sequence over the
// first ctx tokens of its history.  How K/V are reached ([nalar] "Kernel
// attention harus mengikuti block table"): the kernel walks the sequence's
// logical blocks in order and translates each through the block table before
// loading the block's K and V rows.
//
// Work decomposition (not on the pages; a gfx950 design):
//   one wave = one work item (sequence, KV head, context partition).  All
//   G = Hq/Hkv query heads of the KV head are served by that wave, so every
//   K/V row is read from HBM once per KV head.  A context longer than one
//   partition is split over several waves whose float32 partial results
//   (running max, running sum, unnormalised output) are merged exactly by
//   decode_reduce_kernel (log-sum-exp rescale, fixed order).
//
// Matrix-core kernel (bf16 K/V, the serving configurations):
//   a tile is 16 consecutive logical tokens.
//   QK^T : v_mfma_f32_16x16x32_bf16, A = 16 key rows x 32 dims, B = 32 dims x
//          16 query heads (heads >= G are zero).  bf16 x bf16 products are
//          exact in float32 and accumulate in float32.
//          Lane (grp = lane/16, col = lane%16) loads key row `col`, dims
//          32*s + 8*grp .. +7 of each k-step s (16-byte loads).
//          Result: lane holds scores of head `col` for tokens 4*grp + i.
//   softmax: online (running max m, running sum l) per head, base 2 with the
//          scale folded in; masked tokens get -inf by select, never by
//          multiplication, so NaN in unused slots cannot leak.
//   PV   : v_mfma_f32_16x16x4_f32, A = P (16 heads x 4 tokens, full float32),
//          B = V (4 tokens x 16 dims).  The token order inside the k-step is
//          free, so lane (grp, col) uses its own score registers (token
//          4*grp + j in step j) and its own V load: row 4*grp + j, dims
//          (D/16)*col .. +D/16-1 -- 16 lanes read one V row contiguously.
//          Output: lane holds heads 4*grp + r, dims (D/16)*col + nt.
//
// Vector-ALU kernel (float32 K/V, or on request): 16-byte row chunks, LPR
//   lanes per row, each group of LPR lanes an independent online-softmax
//   stream over every (64/LPR)-th token; the streams are merged at the end
//   with a fixed butterfly, so results are deterministic.

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecodeWaves = 4;  // independent work items per workgroup
constexpr int kRing = 4;         // 16-token tiles held in registers per wave (3 in flight)
constexpr float kLazyMax = 8.f;  // headroom (log2) before the running max must move
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

struct Item {
  int seq, kvh, part, n, nparts, start, end;
};

// Decode the flat work-item index; returns false for waves with no work.
__device__ __forceinline__ bool decode_item(const DecodeParams& p, int64_t item, Item& it) {
  const int P = p.max_partitions;
  const int64_t rest = item / P;
  if (rest >= (int64_t)p.num_seqs * p.num_kv_heads) return false;
  it.part = (int)(item - rest * P);
  it.kvh = (int)(rest % p.num_kv_heads);
  it.seq = (int)(rest / p.num_kv_heads);
  int n = p.context_lens[it.seq];
  n = min(max(n, 0), p.max_tokens);
  it.n = n;
  it.nparts = (n + p.partition - 1) / p.partition;
  if (it.part >= max(it.nparts, 1)) return false;
  it.start = it.part * p.partition;
  it.end = min(it.start + p.partition, n);
  return true;
}

// ---------------------------------------------------------------------------
// matrix-core kernel (bf16)
// ---------------------------------------------------------------------------

template <int D, int BS>
__global__ __launch_bounds__(kDecodeWaves * kWave, 2) void decode_mfma_kernel(const DecodeParams p) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KSTEPS = D / 32;  // QK k-steps
  constexpr int DV = D / 16;      // V dims per lane per row == PV n-tiles
  using VRow = typename std::conditional<DV == 8, uint4, uint2>::type;
  struct Tile {
    uint4 k[KSTEPS];  // key row `col`, dims 32*s + 8*grp .. +7
    VRow v[4];        // value rows 4*grp + j, dims DV*col .. +DV-1
  };

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int grp = lane >> 4;
  const int col = lane & 15;
  Item it;
  if (!decode_item(p, (int64_t)blockIdx.x * kDecodeWaves + wave, it)) return;
  const int G = p.group;
  const int hq0 = it.kvh * G;

  // Query heads as the B operand of QK^T (zero rows for col >= G).
  bf16x8_t qv[KSTEPS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           ((int64_t)it.seq * p.num_q_heads + hq0 + (col < G ? col : 0)) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (col < G) raw = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * grp);
      qv[s] = as_bf16x8(raw);
    }
  }

  // Physical ids of the partition's blocks, one per lane (partition <= 64 blocks).
  const int b0 = it.start / BS;
  const int nblk = (it.end - it.start + BS - 1) / BS;
  int my_id = 0;
  if (lane < nblk) {
    const int v = p.block_tables[(int64_t)it.seq * p.max_blocks_per_seq + b0 + lane];
    my_id = (v >= 0 && v < p.num_blocks) ? v : 0;  // a bad entry reads block 0, never faults
  }

  const uint16_t* kpool = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v_cache);
  const int64_t chunk = (int64_t)BS * D;  // elements of one (block, KV head) chunk
  auto chunk_base = [&](int phys) -> int64_t {
    return ((int64_t)phys * p.num_kv_heads + it.kvh) * chunk;
  };
  const int ntiles = (it.end - it.start + 15) / 16;

  // Tile t covers tokens start+16t .. +15.  For BS >= 16 they lie in one
  // block, whose id is wave-uniform (readlane); for BS == 8 a tile spans two
  // blocks and each lane fetches its row's id with a lane shuffle.  Rows past
  // the partition's last block reuse its id (they are masked).  The index is
  // clamped to the last tile, so the ring can be refilled unconditionally:
  // loads past the end re-read the last tile (from cache) and are never used.
  auto load = [&](int t, Tile& b) {
    const int tb = it.start + 16 * min(t, ntiles - 1);
    if constexpr (BS >= 16) {
      const int phys = __builtin_amdgcn_readlane(my_id, tb / BS - b0);
      const int64_t cb = chunk_base(phys) + (int64_t)(tb % BS) * D;
      const uint16_t* kb = kpool + cb + (int64_t)col * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) b.k[s] = *reinterpret_cast<const uint4*>(kb + 32 * s);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b.v[j] = *reinterpret_cast<const VRow*>(vpool + cb + (int64_t)(4 * grp + j) * D + DV * col);
    } else {
      auto row_base = [&](int tok) -> int64_t {
        const int lb = min(tok / BS - b0, nblk - 1);
        return chunk_base(__shfl(my_id, lb)) + (int64_t)(tok % BS) * D;
      };
      const uint16_t* kb = kpool + row_base(tb + col) + 8 * grp;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) b.k[s] = *reinterpret_cast<const uint4*>(kb + 32 * s);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b.v[j] = *reinterpret_cast<const VRow*>(vpool + row_base(tb + 4 * grp + j) + DV * col);
    }
  };

  f32x4_t acc[DV];
#pragma unroll
  for (int nt = 0; nt < DV; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // m_run: reference point of the exponentials of head `col` (log2 domain).
  // It is moved only when a score exceeds it by more than kLazyMax, so every
  // weight 2^(x - m_run) stays <= 2^kLazyMax and the common path needs no
  // cross-lane traffic; results are exact either way (partials carry m_run).
  float m_run = kNegInf;
  float l_run = 0.f;

  auto compute = [&](int t, Tile& b) {
    const int tb = it.start + 16 * t;
    // scores: lane holds head `col`, tokens tb + 4*grp + i
    f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(b.k[s]), qv[s], sc, 0, 0, 0);
    const bool full = tb + 16 <= it.end;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = full || (tb + 4 * grp + i < it.end);
      x[i] = ok ? sc[i] * p.scale_log2 : kNegInf;
    }
    const float lmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__any(lmax > m_run + kLazyMax)) {
      float mt = fmaxf(lmax, __shfl_xor(lmax, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);   // 0 on the first tile
      l_run *= alpha;
      // rows of acc are heads 4*grp + r; their factor lives in lane 4*grp + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = __shfl(alpha, 4 * grp + r);
#pragma unroll
        for (int nt = 0; nt < DV; ++nt) acc[nt][r] *= a;
      }
      m_run = m_new;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[i] - m_run);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    if (!full) {  // zero V rows past the end (they may hold anything, NaN included)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tb + 4 * grp + j >= it.end) b.v[j] = VRow{};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&b.v[j]);
#pragma unroll
      for (int nt = 0; nt < DV; ++nt) {
        const float v = (nt & 1) ? bf16_hi(w[nt >> 1]) : bf16_lo(w[nt >> 1]);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[j], v, acc[nt], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) {
    // The first pass only fills the ring, so every path into a compute has
    // issued the ring's loads in the same order (the compiler can then wait
    // for the oldest tile alone).
    Tile ring[kRing];
    for (int t0 = -kRing; t0 < ntiles; t0 += kRing) {
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        const int t = t0 + i;
        if (t >= 0 && t < ntiles) compute(t, ring[i]);
        load(t + kRing, ring[i]);
      }
    }
  }

  // total running sum per head (lanes of one column hold the same head)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  const bool single = it.nparts <= 1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * grp + r;
    const float l_h = __shfl(l_run, h);
    const float m_h = __shfl(m_run, h);
    if (h >= G) continue;
    const int64_t row = (int64_t)it.seq * p.num_q_heads + hq0 + h;
    if (single) {
      const float inv = l_h > 0.f ? 1.0f / l_h : 0.f;
      float* dst = p.out + row * D + DV * col;
#pragma unroll
      for (int c = 0; c < DV; c += 4)
        *reinterpret_cast<float4*>(dst + c) =
            make_float4(acc[c][r] * inv, acc[c + 1][r] * inv, acc[c + 2][r] * inv, acc[c + 3][r] * inv);
    } else {
      const int64_t prow = row * p.max_partitions + it.part;
      float* dst = p.ws_acc + prow * D + DV * col;
#pragma unroll
      for (int c = 0; c < DV; c += 4)
        *reinterpret_cast<float4*>(dst + c) =
            make_float4(acc[c][r], acc[c + 1][r], acc[c + 2][r], acc[c + 3][r]);
      if (col == 0) {
        p.ws_m[prow] = m_h;
        p.ws_l[prow] = l_h;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// vector-ALU kernel (f32 or bf16)
// ---------------------------------------------------------------------------

template <typename T, int D, int GMAX>
__global__ __launch_bounds__(kDecodeWaves * kWave) void decode_valu_kernel(const DecodeParams p,
                                                                           int block_size) {
  constexpr int E = sizeof(T);
  constexpr int VEC = 16 / E;    // elements per lane per row chunk
  constexpr int LPR = D / VEC;   // lanes per row
  constexpr int RPW = kWave / LPR;
  static_assert(LPR <= kWave && kWave % LPR == 0, "row split");

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int rg = lane / LPR;
  const int ch = lane % LPR;
  Item it;
  if (!decode_item(p, (int64_t)blockIdx.x * kDecodeWaves + wave, it)) return;
  const int G = p.group;
  const int hq0 = it.kvh * G;

  auto load_row = [&](const void* base, int64_t elem_off, float (&f)[VEC]) {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const T*>(base) + elem_off);
    if constexpr (E == 4) {
      f[0] = __uint_as_float(raw.x);
      f[1] = __uint_as_float(raw.y);
      f[2] = __uint_as_float(raw.z);
      f[3] = __uint_as_float(raw.w);
    } else {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_lo(w[e]);
        f[2 * e + 1] = bf16_hi(w[e]);
      }
    }
  };

  float q[GMAX][VEC];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      load_row(p.q, ((int64_t)it.seq * p.num_q_heads + hq0 + h) * D + ch * VEC, q[h]);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[h][e] = 0.f;
    }
  }
  float m[GMAX], l[GMAX], acc[GMAX][VEC];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  }

  const int32_t* bt = p.block_tables + (int64_t)it.seq * p.max_blocks_per_seq;
  for (int tok = it.start + rg; tok < it.end; tok += RPW) {
    const int lb = tok / block_size;
    int phys = bt[lb];
    phys = (phys >= 0 && phys < p.num_blocks) ? phys : 0;
    const int64_t off = (((int64_t)phys * p.num_kv_heads + it.kvh) * block_size +
                         (tok - lb * block_size)) * D + ch * VEC;
    float kf[VEC], vf[VEC];
    load_row(p.k_cache, off, kf);
    load_row(p.v_cache, off, vf);
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) continue;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) s = fmaf(q[h][e], kf[e], s);
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
      const float x = s * p.scale_log2;
      const float mn = fmaxf(m[h], x);
      const float a = fast_exp2(m[h] - mn);
      const float pw = fast_exp2(x - mn);
      l[h] = l[h] * a + pw;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(pw, vf[e], acc[h][e] * a);
      m[h] = mn;
    }
  }

  // merge the RPW independent streams (butterfly; both partners compute the
  // same commutative expression, so every lane ends bit-identical)
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) continue;
      const float mo = __shfl_xor(m[h], o);
      const float lo = __shfl_xor(l[h], o);
      const float mn = fmaxf(m[h], mo);
      const float a = mn == kNegInf ? 0.f : fast_exp2(m[h] - mn);
      const float b = mn == kNegInf ? 0.f : fast_exp2(mo - mn);
      l[h] = l[h] * a + lo * b;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = __shfl_xor(acc[h][e], o);
        acc[h][e] = acc[h][e] * a + ao * b;
      }
      m[h] = mn;
    }
  }
  if (rg != 0) return;

  const bool single = it.nparts <= 1;
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h >= G) continue;
    const int64_t row = (int64_t)it.seq * p.num_q_heads + hq0 + h;
    if (single) {
      const float inv = l[h] > 0.f ? 1.0f / l[h] : 0.f;
      float* dst = p.out + row * D + ch * VEC;
#pragma unroll
      for (int e = 0; e < VEC; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv, acc[h][e + 3] * inv);
    } else {
      const int64_t prow = row * p.max_partitions + it.part;
      float* dst = p.ws_acc + prow * D + ch * VEC;
#pragma unroll
      for (int e = 0; e < VEC; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      if (ch == 0) {
        p.ws_m[prow] = m[h];
        p.ws_l[prow] = l[h];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// cross-partition merge
// ---------------------------------------------------------------------------
//
// One workgroup per (sequence, query head) with more than one partition:
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p
// Partitions are split over PG thread groups in a fixed interleave, then
// summed in a fixed order through LDS: deterministic.

constexpr int kReduceThreads = 256;

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* scratch) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / kWave; ++w) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
  return r;
}

template <int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(const DecodeParams p) {
  constexpr int C = D / 4;                 // float4 chunks per row
  constexpr int PG = kReduceThreads / C;   // partition groups
  __shared__ float scratch[kReduceThreads / kWave];
  __shared__ float4 part_sum[PG][C];

  const int64_t row = blockIdx.x;          // seq * Hq + h
  const int seq = (int)(row / p.num_q_heads);
  int n = p.context_lens[seq];
  n = min(max(n, 0), p.max_tokens);
  const int np = (n + p.partition - 1) / p.partition;
  if (np <= 1) return;                     // written directly by the decode kernel
  const int P = p.max_partitions;
  const float* m = p.ws_m + row * P;
  const float* l = p.ws_l + row * P;
  const int tid = threadIdx.x;

  float mx = kNegInf;
  for (int i = tid; i < np; i += kReduceThreads) mx = fmaxf(mx, m[i]);
  const float M = block_reduce(mx, true, scratch);
  float ls = 0.f;
  for (int i = tid; i < np; i += kReduceThreads) ls += fast_exp2(m[i] - M) * l[i];
  const float L = block_reduce(ls, false, scratch);

  const int c = tid % C;
  const int g = tid / C;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* acc = reinterpret_cast<const float4*>(p.ws_acc + row * P * D);
  for (int i = g; i < np; i += PG) {
    const float w = fast_exp2(m[i] - M);
    const float4 v = acc[(int64_t)i * C + c];
    a.x = fmaf(w, v.x, a.x);
    a.y = fmaf(w, v.y, a.y);
    a.z = fmaf(w, v.z, a.z);
    a.w = fmaf(w, v.w, a.w);
  }
  part_sum[g][c] = a;
  __syncthreads();
  if (g == 0) {
    float4 s = part_sum[0][c];
#pragma unroll
    for (int k = 1; k < PG; ++k) {
      const float4 v = part_sum[k][c];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    reinterpret_cast<float4*>(p.out + row * D)[c] =
        make_float4(s.x * inv, s.y * inv, s.z * inv, s.w * inv);
  }
}

template <int D, int BS>
void launch_mfma(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mfma_kernel<D, BS>), grid, dim3(kDecodeWaves * kWave), 0, stream, p);
}

template <typename T, int D>
void launch_valu(const DecodeParams& p, int block_size, dim3 grid, hipStream_t stream) {
  const int g = p.group;
  if (g <= 1)
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 1>), grid, dim3(kDecodeWaves * kWave), 0, stream, p, block_size);
  else if (g <= 2)
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 2>), grid, dim3(kDecodeWaves * kWave), 0, stream, p, block_size);
  else if (g <= 4)
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 4>), grid, dim3(kDecodeWaves * kWave), 0, stream, p, block_size);
  else if (g <= 8)
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 8>), grid, dim3(kDecodeWaves * kWave), 0, stream, p, block_size);
  else
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 16>), grid, dim3(kDecodeWaves * kWave), 0, stream, p, block_size);
}

template <int D>
void launch_mfma_bs(const DecodeParams& p, int block_size, dim3 grid, hipStream_t stream) {
  switch (block_size) {
    case 8: launch_mfma<D, 8>(p, grid, stream); break;
    case 16: launch_mfma<D, 16>(p, grid, stream); break;
    case 32: launch_mfma<D, 32>(p, grid, stream); break;
    default: launch_mfma<D, 64>(p, grid, stream); break;
  }
}

}  // namespace

DecodeWorkspace decode_workspace(int num_seqs, int num_q_heads, int head_dim, int max_partitions) {
  DecodeWorkspace w{};
  if (max_partitions <= 1) return w;
  const size_t rows = (size_t)num_seqs * num_q_heads * max_partitions;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  w.m_off = 0;
  w.l_off = align(rows * sizeof(float));
  w.acc_off = w.l_off + align(rows * sizeof(float));
  w.total = w.acc_off + align(rows * head_dim * sizeof(float));
  return w;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int block_size, pa_dtype dtype,
                         bool vector_only, hipStream_t stream) {
  const int64_t items = (int64_t)p.num_seqs * p.num_kv_heads * p.max_partitions;
  if (items == 0) return hipSuccess;
  const dim3 grid((unsigned)((items + kDecodeWaves - 1) / kDecodeWaves));
  if (dtype == PA_BF16 && !vector_only) {
    if (head_dim == 128) launch_mfma_bs<128>(p, block_size, grid, stream);
    else launch_mfma_bs<64>(p, block_size, grid, stream);
  } else if (dtype == PA_BF16) {
    if (head_dim == 128) launch_valu<uint16_t, 128>(p, block_size, grid, stream);
    else launch_valu<uint16_t, 64>(p, block_size, grid, stream);
  } else {
    if (head_dim == 128) launch_valu<float, 128>(p, block_size, grid, stream);
    else launch_valu<float, 64>(p, block_size, grid, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_partitions <= 1) return e;
  const dim3 rgrid((unsigned)((int64_t)p.num_seqs * p.num_q_heads));
  if (head_dim == 128)
    hipLaunchKernelGGL((decode_reduce_kernel<128>), rgrid, dim3(kReduceThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<64>), rgrid, dim3(kReduceThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
