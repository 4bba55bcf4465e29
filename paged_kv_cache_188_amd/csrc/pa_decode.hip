// Paged decode attention for gfx950 (MI355X).
//
// What is computed ([nalar] introduction; [gininih] "Batasan dan salah paham
// umum"): ordinary softmax attention of one query token per sequence over the
// first ctx tokens of its history.  How K/V are reached ([nalar] "Kernel
// attention harus mengikuti block table"): the kernel walks the sequence's
// logical blocks in order and translates each through the block table before
// loading the block's K and V rows.
//
// Work decomposition (not on the pages; a gfx950 design).  A "segment" is one
// (sequence, KV head): all G = Hq/Hkv query heads of the KV head are served by
// the same wave, so every K/V row is read from HBM once per KV head.  Segments
// are cut into 16-token tiles.
//   * stream-K path (bf16, the default): persistent waves, one per resident
//     wave slot.  The tiles of all segments, in (sequence, KV head, tile)
//     order, are split into equal contiguous ranges, one per wave, so every
//     wave streams the same number of bytes whatever the length mix.  A wave
//     writes the final output of every segment it covers whole and a float32
//     partial (running max, running sum, unnormalised output) for at most two
//     segments it shares with its neighbours; the first wave of a shared
//     segment records it, and decode_streamk_merge_kernel combines the
//     partials (log-sum-exp rescale, fixed order).
//   * fixed-partition path (float32 K/V, an explicit partition size, or very
//     large batches): one wave per (segment, partition) work item, partials
//     merged by decode_reduce_kernel.
//   With 8-token blocks a 16-token tile covers two blocks; both ids travel in
//   the tile descriptor.
//
// Matrix-core tile loop (bf16 K/V):
//   a tile is 16 consecutive logical tokens.  Loads are laid out so that
//   every group of four consecutive lanes reads 64 contiguous bytes and every
//   group of sixteen reads 256 contiguous bytes.  (Measured on MI355X: a random
//   4 KiB chunk gather reaches ~6.0 TB/s with that pattern but only ~4.7 TB/s
//   when the four lanes of a group read four different 256-byte rows, which is
//   what a token-major K row would need for the matrix-core operand.)  K/V are
//   read once, so the loads are non-temporal.
//   QK^T : v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims, B = 32 dims x 16
//          query heads (heads >= G are zero).  bf16 x bf16 products are exact
//          in float32 and accumulate in float32.  The K pool stores 16-byte
//          granules token-minor, so lane (grp = lane/16, col = lane%16) reads
//          granule 4*s + grp of key `col`.  Result: lane holds the scores of
//          head `col` for tokens 4*grp + i.
//   softmax: online (running max m, running sum l) per head, base 2 with the
//          scale folded in; masked tokens get -inf by select, never by
//          multiplication, so NaN in unused slots cannot leak.
//   PV   : v_mfma_f32_16x16x16_bf16 twice per output tile, A = P split as
//          hi + lo bf16 (16 heads x 16 tokens; hi + lo equals the float32
//          weight to 2^-16 relative, so P is never rounded to bf16), B = V
//          (16 tokens x 16 dims).  Lane (grp, col) holds the scores of tokens
//          4*grp .. 4*grp+3 (the A layout) and loads V rows 4*grp + j, dims
//          (D/16)*col .. +D/16-1 of the token-major V pool (16 lanes read one
//          V row); element nt of its four rows is the B operand of output
//          tile nt.  Output: lane holds heads 4*grp + r, dims (D/16)*col + nt.
//   pipeline: each wave loads one tile, then attends to it; the 8 waves of a
//          CU keep 8 tiles (64 KiB) in flight between them.
//
// Vector-ALU kernel (float32 K/V, or on request): 16-byte granules, LPR
//   lanes per token, each group of LPR lanes an independent online-softmax
//   stream over every (64/LPR)-th token; the streams are merged at the end
//   with a fixed butterfly, so results are deterministic.

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));   // 4 bf16 bit patterns
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kDecodeWaves = 4;  // independent waves per workgroup
constexpr float kLazyMax = 8.f;  // headroom (log2) before the running max must move
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Streaming (non-temporal) loads of K/V data that is read exactly once.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)));
}

// Streaming (non-temporal) stores of results that this kernel does not read
// back: they leave no dirty L2 lines behind for the end-of-kernel write-back.
__device__ __forceinline__ void store_stream(float* p, float4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_stream(uint16_t* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int clamp_ctx(const DecodeParams& p, int seq) {
  return min(max(p.context_lens[seq], 0), p.max_tokens);
}

// ---------------------------------------------------------------------------
// matrix-core building blocks (bf16)
// ---------------------------------------------------------------------------

template <int D>
struct MfmaState {
  f32x4_t acc[D / 16];
  float m_run;  // reference point of the exponentials of head `col` (log2)
  float l_run;  // per-lane partial sum of weights of head `col`
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;
  }
};

// Query heads hq0 .. hq0+G-1 of sequence `seq` as the B operand of QK^T
// (zero rows for col >= G).
template <int D>
__device__ __forceinline__ void mfma_load_q(const DecodeParams& p, int seq, int hq0, int lane,
                                            bf16x8_t (&qv)[D / 32], int heads = 0) {
  // heads > G: a shared-prefix group, tile column col is head hq0 + col % G
  // of the group's member col / G (sequences seq, seq + 1, ...)
  const int grp = lane >> 4, col = lane & 15;
  const int G = p.group;
  const bool valid = col < (heads > 0 ? heads : G);
  const int64_t qr = valid ? (int64_t)(seq + col / G) * p.num_q_heads + hq0 + col % G
                           : (int64_t)seq * p.num_q_heads + hq0;
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + qr * D;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (valid) raw = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * grp);
    qv[s] = as_bf16x8(raw);
  }
}

template <int D>
using VRowT = typename std::conditional<D / 16 == 8, uint4, uint2>::type;

// One 16-token tile in registers.
template <int D>
struct Tile {
  uint4 k[D / 32];  // key `col`, granule 4*s + grp (dims 32*s + 8*grp .. +7)
  VRowT<D> v[4];    // value row 4*grp + j, dims (D/16)*col .. +D/16-1
};

// Load a tile whose 16 tokens lie in one block (BS >= 16): cb is the element
// offset of the (block, KV head) chunk, o the tile's first token in the
// block.  If kk >= 0, token kk of the tile is read from the row pair knew /
// vnew (D elements each) instead of the pools.
template <int D, int BS>
__device__ __forceinline__ void load_tile(const uint16_t* kpool, const uint16_t* vpool, int64_t cb,
                                          int o, int lane, Tile<D>& b,
                                          const uint16_t* knew = nullptr,
                                          const uint16_t* vnew = nullptr, int kk = -1) {
  constexpr int DV = D / 16;
  const int grp = lane >> 4, col = lane & 15;
  const bool k_from_new = col == kk;  // kk = -1: no token is overridden
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    b.k[s] = load_stream(reinterpret_cast<const uint4*>(
        k_from_new ? knew + 32 * s + 8 * grp
                   : kpool + cb + ((int64_t)(4 * s + grp) * BS + o + col) * 8));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool v_from_new = 4 * grp + j == kk;
    b.v[j] = load_stream(reinterpret_cast<const VRowT<D>*>(
        v_from_new ? vnew + DV * col : vpool + cb + (int64_t)(o + 4 * grp + j) * D + DV * col));
  }
}

// Load a tile that spans two blocks (BS < 16, so BS = 8 and the tile starts
// a block): tokens 0 .. BS-1 from the chunk at cb0, the rest from cb1.  The
// new-row override is as in load_tile.
template <int D, int BS>
__device__ __forceinline__ void load_tile2(const uint16_t* kpool, const uint16_t* vpool,
                                           int64_t cb0, int64_t cb1, int lane, Tile<D>& b,
                                           const uint16_t* knew = nullptr,
                                           const uint16_t* vnew = nullptr, int kk = -1) {
  static_assert(16 % BS == 0 && BS < 16, "a tile covers whole blocks");
  constexpr int DV = D / 16;
  const int grp = lane >> 4, col = lane & 15;
  const bool k_from_new = col == kk;
  const int64_t kb = col < BS ? cb0 : cb1;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    b.k[s] = load_stream(reinterpret_cast<const uint4*>(
        k_from_new ? knew + 32 * s + 8 * grp
                   : kpool + kb + ((int64_t)(4 * s + grp) * BS + col % BS) * 8));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * grp + j;
    const bool v_from_new = r == kk;
    b.v[j] = load_stream(reinterpret_cast<const VRowT<D>*>(
        v_from_new ? vnew + DV * col
                   : vpool + (r < BS ? cb0 : cb1) + (int64_t)(r % BS) * D + DV * col));
  }
}

// Attend the G heads to one tile: `valid` (1..16) of its tokens are in the
// context.  The running max is moved only when a score exceeds it by more
// than kLazyMax, so every weight 2^(x - m_run) stays <= 2^kLazyMax and the
// common path needs no cross-lane traffic; results are exact either way
// (partials carry m_run as their reference point).
template <int D>
__device__ __forceinline__ void compute_tile(const DecodeParams& p, MfmaState<D>& st,
                                             const bf16x8_t (&qv)[D / 32], Tile<D>& b, int valid,
                                             int lane) {
  constexpr int DV = D / 16;
  const int grp = lane >> 4;
  // scores: lane holds head `col`, tokens 4*grp + i of the tile
  f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(b.k[s]), qv[s], sc, 0, 0, 0);
  const bool full = valid >= 16;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = full || (4 * grp + i < valid);
    x[i] = ok ? sc[i] * p.scale_log2 : kNegInf;
  }
  const float lmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (__any(lmax > st.m_run + kLazyMax)) {
    float mt = fmaxf(lmax, __shfl_xor(lmax, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(st.m_run, mt);
    const float alpha = fast_exp2(st.m_run - m_new);  // 0 on the first tile
    st.l_run *= alpha;
    // rows of acc are heads 4*grp + r; their factor lives in lane 4*grp + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = __shfl(alpha, 4 * grp + r);
#pragma unroll
      for (int nt = 0; nt < DV; ++nt) st.acc[nt][r] *= a;
    }
    st.m_run = m_new;
  }
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[i] - st.m_run);
  st.l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

  if (!full) {  // zero V rows past the end (they may hold anything, NaN included)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * grp + j >= valid) b.v[j] = VRowT<D>{};
  }
  // PV on the bf16 matrix cores without rounding P to bf16: p = hi + lo with
  // hi = the upper 16 bits of p (exact) and lo = bf16(p - hi) (p - hi is
  // exact in float32), so hi + lo equals p to 2^-16 relative; bf16 x bf16
  // products are exact and accumulate in float32.  A operand: lane (grp,
  // col) holds head col, tokens 4*grp .. 4*grp+3 -- the scores' own layout.
  uint32_t u[4];
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u[i] = __float_as_uint(pr[i]);
    r[i] = pr[i] - __uint_as_float(u[i] & 0xffff0000u);
  }
  const s16x4_t p_hi = __builtin_bit_cast(
      s16x4_t, make_uint2(__builtin_amdgcn_perm(u[1], u[0], 0x07060302u),
                          __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)));
  const s16x4_t p_lo = __builtin_bit_cast(
      s16x4_t,
      make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{r[0], r[1]}, bf16x2_t)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{r[2], r[3]}, bf16x2_t))));
  // B operand of output tile nt: tokens 4*grp .. 4*grp+3 of dim (D/16)*col +
  // nt, i.e. element nt of this lane's four V rows, packed pairwise.
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&b.v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&b.v[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&b.v[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&b.v[3]);
#pragma unroll
  for (int nt = 0; nt < DV; ++nt) {
    const uint32_t sel = (nt & 1) ? 0x07060302u : 0x05040100u;
    const s16x4_t v = __builtin_bit_cast(
        s16x4_t, make_uint2(__builtin_amdgcn_perm(w1[nt >> 1], w0[nt >> 1], sel),
                            __builtin_amdgcn_perm(w3[nt >> 1], w2[nt >> 1], sel)));
    st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_hi, v, st.acc[nt], 0, 0, 0);
    st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_lo, v, st.acc[nt], 0, 0, 0);
  }
}

// Tiles [tile_begin, tile_end) of segment (seq, kvh) whose context is n
// tokens, accumulated into st (fixed-partition path).  The tiles may touch
// at most 64 blocks (one block id per lane).  One tile at a time: load, then
// attend (the other waves of the CU keep the memory system busy meanwhile).
template <int D, int BS>
__device__ __forceinline__ void mfma_tiles(const DecodeParams& p, int seq, int kvh, int n,
                                           int tile_begin, int tile_end,
                                           const bf16x8_t (&qv)[D / 32], MfmaState<D>& st,
                                           int lane) {
  constexpr int DV = D / 16;
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int start = 16 * tile_begin;
  const int end = min(16 * tile_end, n);
  const int ntiles = tile_end - tile_begin;
  if (ntiles <= 0) return;

  // Physical ids of the blocks the tiles touch, one per lane.
  const int b0 = start / BS;
  const int nblk = (end - 1) / BS - b0 + 1;
  int my_id = 0;
  if (lane < nblk) {
    const int v = p.block_tables[(int64_t)seq * p.max_blocks_per_seq + b0 + lane];
    my_id = (v >= 0 && v < p.num_blocks) ? v : 0;  // a bad entry reads block 0, never faults
  }

  const uint16_t* kpool = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v_cache);
  auto chunk_base = [&](int phys) -> int64_t {
    return ((int64_t)phys * p.num_kv_heads + kvh) * ((int64_t)BS * D);
  };

  auto load = [&](int t, Tile<D>& b) {
    const int tb = start + 16 * t;
    if constexpr (BS >= 16) {
      load_tile<D, BS>(kpool, vpool, chunk_base(__builtin_amdgcn_readlane(my_id, tb / BS - b0)),
                       tb % BS, lane, b);
    } else {
      // a tile spans two blocks: each lane fetches its row's id with a shuffle
      auto blk_base = [&](int tok) -> int64_t {
        const int lb = min(tok / BS - b0, nblk - 1);
        return chunk_base(__shfl(my_id, lb));
      };
      const int kt = tb + col;
      const int64_t kb = blk_base(kt);
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        b.k[s] = load_stream(reinterpret_cast<const uint4*>(
            kpool + kb + ((int64_t)(4 * s + grp) * BS + kt % BS) * 8));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int vt = tb + 4 * grp + j;
        b.v[j] = load_stream(reinterpret_cast<const VRowT<D>*>(
            vpool + blk_base(vt) + (int64_t)(vt % BS) * D + DV * col));
      }
    }
  };

  for (int t = 0; t < ntiles; ++t) {
    Tile<D> b;
    load(t, b);
    compute_tile<D>(p, st, qv, b, min(16, end - (start + 16 * t)), lane);
  }
}

// Write the `heads` heads of a finished state: normalised into `out_row0`,
// head h at row (h / per) * member_rows + h % per (per = heads of one
// sequence, member_rows = rows between the sequences of a shared-prefix
// group; one sequence: row h), with its log2-sum-exp m + log2(l) at the same
// row of lse_row0 when that is given; or as a partial: acc at acc_row0 +
// h*acc_stride, m and l at m0/l0 + h*ml_stride.
template <int D>
__device__ __forceinline__ void mfma_finish(MfmaState<D>& st, int heads, int per,
                                            int64_t member_rows, int lane, float* out_row0,
                                            float* lse_row0, float* acc_row0, float* m0,
                                            float* l0, int64_t acc_stride, int64_t ml_stride) {
  constexpr int DV = D / 16;
  const int grp = lane >> 4, col = lane & 15;
  // total running sum per head (lanes of one column hold the same head)
  float l_run = st.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * grp + r;
    const float l_h = __shfl(l_run, h);
    const float m_h = __shfl(st.m_run, h);
    if (h >= heads) continue;
    if (out_row0) {
      const float inv = l_h > 0.f ? 1.0f / l_h : 0.f;
      const int64_t orow = (int64_t)(h / per) * member_rows + h % per;
      if (lse_row0 && col == 0) lse_row0[orow] = l_h > 0.f ? m_h + __log2f(l_h) : kNegInf;
      float* dst = out_row0 + orow * D + DV * col;
#pragma unroll
      for (int c = 0; c < DV; c += 4)
        store_stream(dst + c, make_float4(st.acc[c][r] * inv, st.acc[c + 1][r] * inv,
                                          st.acc[c + 2][r] * inv, st.acc[c + 3][r] * inv));
    } else {
      float* dst = acc_row0 + (int64_t)h * acc_stride + DV * col;
#pragma unroll
      for (int c = 0; c < DV; c += 4)
        *reinterpret_cast<float4*>(dst + c) =
            make_float4(st.acc[c][r], st.acc[c + 1][r], st.acc[c + 2][r], st.acc[c + 3][r]);
      if (col == 0) {
        m0[(int64_t)h * ml_stride] = m_h;
        l0[(int64_t)h * ml_stride] = l_h;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// stream-K matrix-core kernel
// ---------------------------------------------------------------------------

// Passes of the stream-K kernels.  kPlain: every (sequence, KV head) over its
// whole context.  The shared-prefix decode runs two passes: kPrefix, one
// segment per (group, KV head) over the tokens the group's sequences share,
// the G heads of each member stacked into one matrix-core tile of up to 16
// heads, so each shared K/V tile is read once for the whole group; then
// kOwn, every (sequence, KV head) over its own tokens after the shared ones;
// a last kernel combines the two results of each head (log-sum-exp).
enum : int { kPlain = 0, kPrefix = 1, kOwn = 2 };

// Group g as the kernels see it: its first sequence, the members whose
// prefix is shared (at most group_cap = 16 / G of them: the heads of one
// tile), and the shared token count -- the caller's shared_len rounded down
// to whole 16-token tiles and blocks, and cut so that every member keeps at
// least its last token (the one a step appends) as its own.  count = 0: the
// group shares nothing (or has a single member).  Every index is checked, so groups that break the
// contract give wrong results, never an access outside a buffer.
struct GroupInfo {
  int first, count, len;
};

__device__ __forceinline__ GroupInfo group_info(const DecodeParams& p, int g) {
  GroupInfo gi{0, 0, 0};
  const int a = p.group_start[g], b = p.group_start[g + 1];
  if (a < 0 || b <= a || a >= p.num_seqs) return gi;
  const int cnt = min(min(b, p.num_seqs) - a, p.group_cap);
  if (cnt < 2) return gi;  // a lone sequence: plain decode
  const int unit = max(16, p.block_size);
  int len = p.shared_len[g];
  for (int i = 0; i < cnt; ++i) len = min(len, clamp_ctx(p, a + i) - 1);
  len = len > 0 ? len - len % unit : 0;
  if (len > 0) {
    gi.first = a;
    gi.count = cnt;
    gi.len = len;
  }
  return gi;
}

// Exclusive prefix of the pass's tile counts per (virtual) sequence into LDS
// (V + 1 entries; V = S, or the group count for kPrefix), computed by the
// whole workgroup.  s_aux: kPrefix, the groups' first member, member count
// and shared length ([3][V]); kOwn, each sequence's first own position ([S]).
template <int MODE>
__device__ void tile_prefix(const DecodeParams& p, int* s_prefix, int* s_aux) {
  __shared__ int wave_sums[kDecodeWaves];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int V = MODE == kPrefix ? p.num_groups : p.num_seqs;
  if constexpr (MODE == kPrefix) {
    for (int g = tid; g < V; g += blockDim.x) {
      const GroupInfo gi = group_info(p, g);
      s_aux[g] = gi.first;
      s_aux[V + g] = gi.count;
      s_aux[2 * V + g] = gi.len;
    }
  } else if constexpr (MODE == kOwn) {
    for (int i = tid; i < V; i += blockDim.x) s_aux[i] = 0;
    __syncthreads();
    for (int g = tid; g < p.num_groups; g += blockDim.x) {
      const GroupInfo gi = group_info(p, g);
      for (int i = 0; i < gi.count; ++i) s_aux[gi.first + i] = gi.len;
    }
  }
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < V; base += kDecodeWaves * kWave) {
    const int i = base + tid;
    int v = 0;
    if (i < V) {
      if constexpr (MODE == kPrefix) v = s_aux[2 * V + i] / 16;
      else if constexpr (MODE == kOwn) v = (clamp_ctx(p, i) - s_aux[i] + 15) / 16;
      else v = (clamp_ctx(p, i) + 15) / 16;
    }
    // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (lane == kWave - 1) wave_sums[wave] = v;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wave; ++w) before += wave_sums[w];
    if (i < V) s_prefix[i + 1] = before + v;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < kDecodeWaves; ++w) tot += wave_sums[w];
      carry_s += tot;
    }
    __syncthreads();
  }
  if (tid == 0) s_prefix[0] = 0;
  __syncthreads();
}

__device__ __forceinline__ int64_t streamk_workers(int64_t total_tiles, int launched) {
  const int64_t want = (total_tiles + kStreamKMinTiles - 1) / kStreamKMinTiles;
  return want < launched ? (want > 0 ? want : 1) : launched;
}

// Position of a tile in the (sequence, KV head, tile) order of all segments.
struct Pos {
  int seq, kvh, t;
};

// Move q forward by k tiles through the segments (sequences with an empty
// context have no tiles and are stepped over); seq == S past the end.
__device__ __forceinline__ Pos advance(Pos q, int k, const int* s_prefix, int S, int Hkv) {
  q.t += k;
  while (q.seq < S) {
    const int nt = s_prefix[q.seq + 1] - s_prefix[q.seq];
    if (q.t < nt) break;
    q.t -= nt;
    if (++q.kvh == Hkv) {
      q.kvh = 0;
      ++q.seq;
    }
  }
  return q;
}

// Per-lane descriptors of up to 64 consecutive tiles, one per lane: the
// tile's sequence, KV head and tile index, and the raw block-table entry of
// its first token and context length of its sequence.  The two loads are
// issued one chunk ahead of their use and only read (and checked) when the
// tile's loads are issued, so building a chunk never waits for memory.
struct TileDescs {
  int seq, kvh, t, phys_raw, n_raw;
  int phys_raw2;  // block size 8: the block of the tile's second half
  // Make the values register-resident at this point of the program, so the
  // per-tile reads of a chunk never wait for memory where control flow joins.
  __device__ __forceinline__ void settle() {
    asm volatile("" : "+v"(seq), "+v"(kvh), "+v"(t), "+v"(phys_raw), "+v"(n_raw),
                 "+v"(phys_raw2));
  }
};

// The tile's raw context length is its clamped one (so position n-1 really
// is the sequence's last token).
__device__ __forceinline__ bool n_raw_ok(const TileDescs& d, int l, const DecodeParams& p) {
  const int n = __builtin_amdgcn_readlane(d.n_raw, l);
  return n >= 1 && n <= p.max_tokens;
}

// First position of (virtual) sequence v's tiles in the pass, and the table
// its tiles are read through (kPrefix: the group's first member's).
template <int MODE>
__device__ __forceinline__ int pass_pos0(const int* s_aux, int v) {
  if constexpr (MODE == kOwn) return s_aux[v];
  return 0;
}
template <int MODE>
__device__ __forceinline__ int pass_table_seq(const int* s_aux, int v) {
  if constexpr (MODE == kPrefix) return s_aux[v];
  return v;
}

template <int BS, int MODE>
__device__ __forceinline__ TileDescs describe_tiles(const DecodeParams& p, const int* s_prefix,
                                                    const int* s_aux, int V, Pos start, int count,
                                                    int lane) {
  TileDescs d{0, 0, 0, 0, 0, 0};
  if (lane < count) {
    const Pos q = advance(start, lane, s_prefix, V, p.num_kv_heads);
    d.seq = q.seq;
    d.kvh = q.kvh;
    d.t = q.t;
    // the pass's context end: the shared length for a group, else the
    // sequence's raw context length (checked when used)
    d.n_raw = MODE == kPrefix ? s_aux[2 * V + q.seq] : p.context_lens[q.seq];
    const int32_t* row =
        p.block_tables + (int64_t)pass_table_seq<MODE>(s_aux, q.seq) * p.max_blocks_per_seq;
    const int tpos = pass_pos0<MODE>(s_aux, q.seq) + 16 * q.t;
    d.phys_raw = row[tpos / BS];
    if constexpr (BS < 16)  // the second block, when the table has one
      d.phys_raw2 = tpos / BS + 1 < p.max_blocks_per_seq ? row[tpos / BS + 1] : -1;
  }
  return d;
}

template <int D, int BS, int MODE>
__global__ __launch_bounds__(kDecodeWaves * kWave, 2) void decode_mfma_streamk_kernel(
    const DecodeParams p) {
  static_assert(BS >= 16 || BS == 8, "a tile lies in one block, or covers two of 8");
  // LDS: the tile prefix [V+1], then the pass's per-sequence data (tile_prefix)
  extern __shared__ int s_lds[];
  const int S = MODE == kPrefix ? p.num_groups : p.num_seqs;  // the pass's (virtual) sequences
  int* s_prefix = s_lds;
  int* s_aux = s_lds + S + 1;
  tile_prefix<MODE>(p, s_prefix, s_aux);
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  // the pass's per-group / per-sequence data, for the merge and combine
  // kernels that follow (one workgroup writes it)
  if constexpr (MODE != kPlain) {
    if (blockIdx.x == 0) {
      int32_t* dst = MODE == kPrefix ? p.group_ws : p.own_ws;
      const int n = MODE == kPrefix ? 3 * S : S;
      for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = s_aux[i];
    }
  }
  // sequences with nothing to attend in the pass: zeros (and a log-sum-exp
  // of -inf), spread over the workgroups; a group with no shared tokens
  // writes nothing (its members' prefix results are not used)
  if constexpr (MODE != kPrefix) {
    for (int seq = blockIdx.x; seq < S; seq += gridDim.x) {
      if (s_prefix[seq + 1] != s_prefix[seq]) continue;
      float4* o = reinterpret_cast<float4*>(p.out + (int64_t)seq * p.num_q_heads * D);
      for (int i = threadIdx.x; i < p.num_q_heads * (D / 4); i += blockDim.x)
        o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (MODE == kOwn)
        for (int i = threadIdx.x; i < p.num_q_heads; i += blockDim.x)
          p.lse_out[(int64_t)seq * p.num_q_heads + i] = kNegInf;
    }
  }
  const int64_t T = (int64_t)Hkv * s_prefix[S];
  const int64_t W = streamk_workers(T, p.max_workers);
  const int lane = threadIdx.x % kWave;
  const int64_t w = (int64_t)blockIdx.x * kDecodeWaves + wave_id();
  int2* handoff = reinterpret_cast<int2*>(p.ws_handoff) + w;
  if (T == 0 || w >= W) {
    if (lane == 0) *handoff = make_int2(-1, -1);
    return;
  }
  const int64_t g0 = w * T / W;
  const int64_t g1 = (w + 1) * T / W;
  const int ntiles = (int)(g1 - g0);

  // position of tile g0: the last sequence whose first tile is <= g0
  Pos pos0;
  {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if ((int64_t)Hkv * s_prefix[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    const int nt = s_prefix[lo + 1] - s_prefix[lo];
    const int64_t off = g0 - (int64_t)Hkv * s_prefix[lo];
    pos0.seq = lo;
    pos0.kvh = (int)(off / nt);
    pos0.t = (int)(off - (int64_t)pos0.kvh * nt);
  }

  // descriptors: `dc` covers the chunk the loads are in, `dn` the next one
  auto chunk_count = [&](int c) { return min(kWave, ntiles - c * kWave); };
  TileDescs dc = describe_tiles<BS, MODE>(p, s_prefix, s_aux, S, pos0, chunk_count(0), lane);
  dc.settle();
  Pos next_pos = advance(pos0, kWave, s_prefix, S, Hkv);
  TileDescs dn = {0, 0, 0, 0, 0, 0};
  if (ntiles > kWave) {
    dn = describe_tiles<BS, MODE>(p, s_prefix, s_aux, S, next_pos, chunk_count(1), lane);
    next_pos = advance(next_pos, kWave, s_prefix, S, Hkv);
  }
  int chunk = 0;

  const uint16_t* kpool = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v_cache);

  // compute-side state: the piece being accumulated
  MfmaState<D> st;
  st.reset();
  bf16x8_t qv[D / 32];
  int cur_seg = -1, cur_t0 = 0, cur_tlast = 0;
  int2 my_handoff = make_int2(-1, -1);
  const int64_t slot0 = w * 2;

  // heads per partial slot: a shared-prefix group stacks up to 16
  const int HS = MODE == kPrefix ? 16 : G;
  auto finish_piece = [&]() {
    const int seq = cur_seg / Hkv, kvh = cur_seg - (cur_seg / Hkv) * Hkv;
    const int nt = s_prefix[seq + 1] - s_prefix[seq];
    const int hq0 = kvh * G;
    if (cur_t0 == 0 && cur_tlast == nt - 1) {
      if constexpr (MODE == kPrefix) {  // the group's members' prefix results
        const int64_t r0 = (int64_t)s_aux[seq] * p.num_q_heads + hq0;
        mfma_finish<D>(st, s_aux[S + seq] * G, G, p.num_q_heads, lane, p.prefix_out + r0 * D,
                       p.prefix_lse + r0, nullptr, nullptr, nullptr, 0, 0);
      } else {
        const int64_t r0 = (int64_t)seq * p.num_q_heads + hq0;
        mfma_finish<D>(st, G, G, 0, lane, p.out + r0 * D, MODE == kOwn ? p.lse_out + r0 : nullptr,
                       nullptr, nullptr, nullptr, 0, 0);
      }
    } else {
      // slot 0: a segment begun by an earlier wave; slot 1: one continued by
      // later waves -- this wave is its first, so it hands the merge on
      const int64_t slot = slot0 + (cur_t0 > 0 ? 0 : 1);
      mfma_finish<D>(st, MODE == kPrefix ? s_aux[S + seq] * G : G, G, 0, lane, nullptr, nullptr,
                     p.ws_acc + slot * HS * D, p.ws_m + slot * HS, p.ws_l + slot * HS, D, 1);
      if (cur_t0 == 0) {
        const int64_t last_tile = (int64_t)Hkv * s_prefix[seq] + (int64_t)kvh * nt + nt - 1;
        my_handoff = make_int2(cur_seg, (int)(((last_tile + 1) * W - 1) / T));
      }
    }
  };

  // One tile at a time: its descriptor, a new segment's Q (issued before the
  // tile, so it arrives with it), the tile's K/V, then the attention.  A wave
  // keeps one tile in flight; the other waves of the CU overlap its compute.
  // (Measured on MI355X: deeper per-wave pipelines -- rings of 2 to 4 tiles,
  // or batches of 2 to 4 -- were slower: the extra requests in flight
  // lengthen the queues without raising the bandwidth, and the waves finish
  // further apart.)
  for (int u = 0; u < ntiles; ++u) {
    if (u / kWave != chunk) {  // entering the next chunk (its loads were issued a chunk ago)
      chunk = u / kWave;
      dc = dn;
      dc.settle();
      if ((chunk + 1) * kWave < ntiles) {
        dn = describe_tiles<BS, MODE>(p, s_prefix, s_aux, S, next_pos, chunk_count(chunk + 1),
                                      lane);
        next_pos = advance(next_pos, kWave, s_prefix, S, Hkv);
      }
    }
    const int l = u % kWave;
    const int seq = __builtin_amdgcn_readlane(dc.seq, l);
    const int kvh = __builtin_amdgcn_readlane(dc.kvh, l);
    const int t = __builtin_amdgcn_readlane(dc.t, l);
    int phys = __builtin_amdgcn_readlane(dc.phys_raw, l);
    phys = (phys >= 0 && phys < p.num_blocks) ? phys : 0;  // a bad entry reads block 0
    const int n = min(max(__builtin_amdgcn_readlane(dc.n_raw, l), 0), p.max_tokens);
    const int seg = seq * Hkv + kvh;
    const bool new_seg = seg != cur_seg;
    // A new segment's Q and the tile are loaded before the finished piece is
    // stored, so the waits on these loads need not cover those stores.
    if (new_seg) {
      if constexpr (MODE == kPrefix)
        mfma_load_q<D>(p, s_aux[seq], kvh * G, lane, qv, s_aux[S + seq] * G);
      else
        mfma_load_q<D>(p, seq, kvh * G, lane, qv);
    }
    const int64_t cb = ((int64_t)phys * Hkv + kvh) * ((int64_t)BS * D);
    const int tpos = pass_pos0<MODE>(s_aux, seq) + 16 * t;  // the tile's first position
    const int valid = min(16, n - tpos);
    // The tile holding the sequence's new token (position n-1) when the call
    // appends: that token is read from the new rows (the merge kernel stores
    // them into their slots, so no wave here waits for a store).
    const bool append = MODE != kPrefix && p.k_new != nullptr && valid == n - tpos &&
                        n_raw_ok(dc, l, p);
    const int64_t row = (int64_t)seq * p.new_stride + (int64_t)kvh * D;
    Tile<D> b;
    if constexpr (BS >= 16) {
      load_tile<D, BS>(kpool, vpool, cb, tpos % BS, lane, b,
                       static_cast<const uint16_t*>(p.k_new) + row,
                       static_cast<const uint16_t*>(p.v_new) + row, append ? valid - 1 : -1);
    } else {
      // a short tile's second block may be absent from the table: its rows
      // are masked, so block 0 stands in
      int phys2 = __builtin_amdgcn_readlane(dc.phys_raw2, l);
      phys2 = (phys2 >= 0 && phys2 < p.num_blocks) ? phys2 : 0;
      load_tile2<D, BS>(kpool, vpool, cb, ((int64_t)phys2 * Hkv + kvh) * ((int64_t)BS * D), lane,
                        b, static_cast<const uint16_t*>(p.k_new) + row,
                        static_cast<const uint16_t*>(p.v_new) + row, append ? valid - 1 : -1);
    }
    if (new_seg) {
      if (cur_seg >= 0) finish_piece();
      st.reset();
      cur_seg = seg;
      cur_t0 = t;
    }
    compute_tile<D>(p, st, qv, b, valid, lane);
    cur_tlast = t;
  }
  finish_piece();
  if (lane == 0) *handoff = my_handoff;
}

// One workgroup per launched wave slot w.  If wave w handed a segment on, it
// is merged here from slot 1 of wave w and slot 0 of waves w+1 .. last, in
// wave order, with an online log-sum-exp rescale.
template <int D, int MODE>
__global__ __launch_bounds__(256) void decode_streamk_merge_kernel(const DecodeParams p) {
  constexpr int C = D / 4;  // float4 chunks per row
  const int G = p.group;
  const int HS = MODE == kPrefix ? 16 : G;  // heads per partial slot
  if (blockIdx.x >= p.max_workers) {
    // Workgroups past the wave slots store the appended tokens: 8 (sequence,
    // KV head) rows per workgroup, 32 threads per row (16 K granules, 16 V
    // granules of 16 bytes for D = 128; half of them for D = 64).
    const int64_t r = (int64_t)(blockIdx.x - p.max_workers) * 8 + threadIdx.x / 32;
    const int c = threadIdx.x % 32;
    constexpr int kChunks = D / 8;  // 16-byte granules per row
    if (r >= (int64_t)p.num_seqs * p.num_kv_heads || c % 16 >= kChunks) return;
    const int seq = (int)(r / p.num_kv_heads), kvh = (int)(r % p.num_kv_heads);
    const int n = p.context_lens[seq];
    if (n < 1 || n > p.max_tokens) return;
    const int pos = n - 1;
    const int bs = p.block_size;
    const int phys = p.block_tables[(int64_t)seq * p.max_blocks_per_seq + pos / bs];
    if (phys < 0 || phys >= p.num_blocks) return;
    const int o = pos % bs;
    const int64_t cb = ((int64_t)phys * p.num_kv_heads + kvh) * ((int64_t)bs * D);
    const int64_t row = (int64_t)seq * p.new_stride + (int64_t)kvh * D;
    const int w = c % 16;
    if (c < 16) {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k_new) + row + 8 * w);
      store_stream(const_cast<uint16_t*>(static_cast<const uint16_t*>(p.k_cache)) + cb +
                       ((int64_t)w * bs + o) * 8, x);
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v_new) + row + 8 * w);
      store_stream(const_cast<uint16_t*>(static_cast<const uint16_t*>(p.v_cache)) + cb +
                       (int64_t)o * D + 8 * w, x);
    }
    return;
  }
  // Workgroups are dealt to the 8 XCDs in turn, so the decode kernel's
  // workgroup b (waves 4b .. 4b+3) ran on XCD b mod 8.  When the decode grid
  // is a multiple of 8 workgroups, merge workgroup m takes a wave slot whose
  // decode workgroup ran on m's own XCD, m mod 8: the hand-off entry and the
  // partials written there (and those of the neighbouring waves of the same
  // workgroup) can still be in that XCD's L2.
  const int nb = p.max_workers / kDecodeWaves;
  int64_t w1 = blockIdx.x;
  if (nb % 8 == 0) {
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    w1 = (int64_t)(8 * (k / kDecodeWaves) + x) * kDecodeWaves + k % kDecodeWaves;
  }
  const int2 h = reinterpret_cast<const int2*>(p.ws_handoff)[w1];
  if (h.x < 0) return;
  const int seq = h.x / p.num_kv_heads, kvh = h.x % p.num_kv_heads;
  const int64_t w2 = h.y;
  // where head hd of the segment goes: row0 + (hd / G) * member_rows + hd % G
  int heads = G;
  int64_t row0 = (int64_t)seq * p.num_q_heads + kvh * G, member_rows = 0;
  float* out = p.out;
  float* lse = MODE == kOwn ? p.lse_out : nullptr;
  if constexpr (MODE == kPrefix) {  // a group: its members' prefix results
    heads = p.group_ws[p.num_groups + seq] * G;
    row0 = (int64_t)p.group_ws[seq] * p.num_q_heads + kvh * G;
    member_rows = p.num_q_heads;
    out = p.prefix_out;
    lse = p.prefix_lse;
  }
  for (int idx = threadIdx.x; idx < heads * C; idx += blockDim.x) {
    const int hd = idx / C, c = idx % C;
    float M = kNegInf, L = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    // eight partials per round trip: all loads of a batch are issued first
    // (indices past w2 re-read w2's and are not combined)
    constexpr int kBatch = 8;
    for (int64_t wb = w1; wb <= w2; wb += kBatch) {
      float m[kBatch], l[kBatch];
      float4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t w = wb + u <= w2 ? wb + u : w2;
        const int64_t slot = 2 * w + (w == w1 ? 1 : 0);
        m[u] = p.ws_m[slot * HS + hd];
        l[u] = p.ws_l[slot * HS + hd];
        v[u] = reinterpret_cast<const float4*>(p.ws_acc + (slot * HS + hd) * D)[c];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (wb + u > w2) break;
        const float Mn = fmaxf(M, m[u]);
        const float s_old = fast_exp2(M - Mn);   // 0 while M is -inf
        const float s_new = fast_exp2(m[u] - Mn);
        L = L * s_old + l[u] * s_new;
        a.x = a.x * s_old + v[u].x * s_new;
        a.y = a.y * s_old + v[u].y * s_new;
        a.z = a.z * s_old + v[u].z * s_new;
        a.w = a.w * s_old + v[u].w * s_new;
        M = Mn;
      }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const int64_t orow = row0 + (int64_t)(hd / G) * member_rows + hd % G;
    store_stream(out + orow * D + 4 * c, make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv));
    if (lse && c == 0) lse[orow] = L > 0.f ? M + __log2f(L) : kNegInf;
  }
}

// Shared-prefix decode, last step: for every member of a group that shares
// a prefix, each head's prefix result (o_p, log2-sum-exp lp) and own-token
// result (o_t, lt) are combined exactly:
//     out = (2^lp o_p + 2^lt o_t) / (2^lp + 2^lt)
// One workgroup per sequence; sequences outside a sharing group keep their
// own-token result, which is then their whole context's.
template <int D>
__global__ __launch_bounds__(256) void decode_shared_combine_kernel(const DecodeParams p) {
  constexpr int C = D / 4;
  const int seq = blockIdx.x;
  // only members of a sharing group have a prefix result (own start > 0)
  if (p.own_ws[seq] <= 0) return;
  const int64_t r0 = (int64_t)seq * p.num_q_heads;
  for (int idx = threadIdx.x; idx < p.num_q_heads * C; idx += blockDim.x) {
    const int hd = idx / C, c = idx % C;
    const float lp = p.prefix_lse[r0 + hd], lt = p.lse_out[r0 + hd];
    const float M = fmaxf(lp, lt);
    const float wp = M == kNegInf ? 0.f : fast_exp2(lp - M);
    const float wt = M == kNegInf ? 0.f : fast_exp2(lt - M);
    const float inv = wp + wt > 0.f ? 1.0f / (wp + wt) : 0.f;
    const float4 op = reinterpret_cast<const float4*>(p.prefix_out + (r0 + hd) * D)[c];
    float4* dst = reinterpret_cast<float4*>(p.out + (r0 + hd) * D) + c;
    const float4 ot = *dst;
    *dst = make_float4((wp * op.x + wt * ot.x) * inv, (wp * op.y + wt * ot.y) * inv,
                       (wp * op.z + wt * ot.z) * inv, (wp * op.w + wt * ot.w) * inv);
  }
}

// ---------------------------------------------------------------------------
// fixed-partition kernels
// ---------------------------------------------------------------------------

struct Item {
  int seq, kvh, part, n, nparts, start, end;
};

// Decode the flat work-item index (part fastest); false for waves with no work.
__device__ __forceinline__ bool decode_item(const DecodeParams& p, int64_t item, Item& it) {
  const int P = p.max_partitions;
  const int64_t rest = item / P;
  if (rest >= (int64_t)p.num_seqs * p.num_kv_heads) return false;
  it.part = (int)(item - rest * P);
  it.kvh = (int)(rest % p.num_kv_heads);
  it.seq = (int)(rest / p.num_kv_heads);
  it.n = clamp_ctx(p, it.seq);
  it.nparts = (it.n + p.partition - 1) / p.partition;
  if (it.part >= max(it.nparts, 1)) return false;
  it.start = it.part * p.partition;
  it.end = min(it.start + p.partition, it.n);
  return true;
}

template <int D, int BS>
__global__ __launch_bounds__(kDecodeWaves * kWave, 2) void decode_mfma_kernel(const DecodeParams p) {
  const int lane = threadIdx.x % kWave;
  Item it;
  if (!decode_item(p, (int64_t)blockIdx.x * kDecodeWaves + wave_id(), it)) return;
  const int G = p.group;
  const int hq0 = it.kvh * G;
  bf16x8_t qv[D / 32];
  mfma_load_q<D>(p, it.seq, hq0, lane, qv);
  MfmaState<D> st;
  st.reset();
  // a partition is a whole number of tiles and at most 64 blocks
  mfma_tiles<D, BS>(p, it.seq, it.kvh, it.n, it.start / 16, (it.end + 15) / 16, qv, st, lane);
  const int64_t row = (int64_t)it.seq * p.num_q_heads + hq0;
  if (it.nparts <= 1) {
    mfma_finish<D>(st, G, G, 0, lane, p.out + row * D, nullptr, nullptr, nullptr, nullptr, 0, 0);
  } else {
    const int64_t prow = row * p.max_partitions + it.part;
    mfma_finish<D>(st, G, G, 0, lane, nullptr, nullptr, p.ws_acc + prow * D, p.ws_m + prow,
                   p.ws_l + prow, (int64_t)p.max_partitions * D, p.max_partitions);
  }
}

template <typename T, int D, int GMAX>
__global__ __launch_bounds__(kDecodeWaves * kWave) void decode_valu_kernel(const DecodeParams p,
                                                                           int block_size) {
  constexpr int E = sizeof(T);
  constexpr int VEC = 16 / E;    // elements per lane per 16-byte granule
  constexpr int LPR = D / VEC;   // lanes per token
  constexpr int RPW = kWave / LPR;
  static_assert(LPR <= kWave && kWave % LPR == 0, "row split");

  const int lane = threadIdx.x % kWave;
  const int rg = lane / LPR;
  const int ch = lane % LPR;
  Item it;
  if (!decode_item(p, (int64_t)blockIdx.x * kDecodeWaves + wave_id(), it)) return;
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
    const int64_t base = ((int64_t)phys * p.num_kv_heads + it.kvh) * block_size * D;
    const int o = tok - lb * block_size;
    float kf[VEC], vf[VEC];
    load_row(p.k_cache, base + ((int64_t)ch * block_size + o) * VEC, kf);  // granule ch
    load_row(p.v_cache, base + (int64_t)o * D + ch * VEC, vf);
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) continue;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) s = fmaf(q[h][e], kf[e], s);
#pragma unroll
      for (int o2 = 1; o2 < LPR; o2 <<= 1) s += __shfl_xor(s, o2);
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
  const int n = clamp_ctx(p, seq);
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
  // eight partitions per round trip: their loads are issued before any is
  // combined (the combination order is unchanged: partition by partition)
  int i = g;
  for (; i + 7 * PG < np; i += 8 * PG) {
    float mv[8];
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mv[u] = m[i + u * PG];
      v[u] = acc[(int64_t)(i + u * PG) * C + c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = fast_exp2(mv[u] - M);
      a.x = fmaf(w, v[u].x, a.x);
      a.y = fmaf(w, v[u].y, a.y);
      a.z = fmaf(w, v[u].z, a.z);
      a.w = fmaf(w, v[u].w, a.w);
    }
  }
  for (; i < np; i += PG) {
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
    store_stream(p.out + row * D + 4 * c, make_float4(s.x * inv, s.y * inv, s.z * inv, s.w * inv));
  }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------

template <int D, int BS, int MODE>
hipError_t launch_streamk_pass(const DecodeParams& p, hipStream_t stream) {
  const int blocks = p.max_workers / kDecodeWaves;
  const int V = MODE == kPrefix ? p.num_groups : p.num_seqs;
  const size_t lds =
      (size_t)(V + 1 + (MODE == kPrefix ? 3 * V : MODE == kOwn ? V : 0)) * sizeof(int);
  hipLaunchKernelGGL((decode_mfma_streamk_kernel<D, BS, MODE>), dim3(blocks),
                     dim3(kDecodeWaves * kWave), lds, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // merge workgroups (one per wave slot), then the append workgroups
  const int64_t append_rows = p.k_new ? (int64_t)p.num_seqs * p.num_kv_heads : 0;
  const int64_t grid = (int64_t)blocks * kDecodeWaves + (append_rows + 7) / 8;
  hipLaunchKernelGGL((decode_streamk_merge_kernel<D, MODE>), dim3((unsigned)grid), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_streamk(const DecodeParams& p, hipStream_t stream) {
  if (!p.group_start) return launch_streamk_pass<D, BS, kPlain>(p, stream);
  // shared prefixes: the groups' prefixes (nothing appended there: a group's
  // shared tokens end before every member's last token), then every
  // sequence's own tokens (with the new rows), then the combination
  DecodeParams pp = p;
  pp.k_new = pp.v_new = nullptr;
  hipError_t e = launch_streamk_pass<D, BS, kPrefix>(pp, stream);
  if (e != hipSuccess) return e;
  e = launch_streamk_pass<D, BS, kOwn>(p, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_shared_combine_kernel<D>), dim3(p.num_seqs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_streamk_bs(const DecodeParams& p, int block_size, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_streamk<D, 8>(p, stream);
    case 16: return launch_streamk<D, 16>(p, stream);
    case 32: return launch_streamk<D, 32>(p, stream);
    default: return launch_streamk<D, 64>(p, stream);
  }
}

template <int D, int BS>
void launch_mfma(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mfma_kernel<D, BS>), grid, dim3(kDecodeWaves * kWave), 0, stream, p);
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

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int streamk_workers_per_cu(int head_dim) {
  // All instantiations of one head_dim share the register footprint; the
  // LDS of the largest supported batch is assumed.
  int blocks = 0;
  const size_t lds = (size_t)(kStreamKMaxSeqs + 1) * sizeof(int);
  hipError_t e = head_dim == 128
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks,
                                                     decode_mfma_streamk_kernel<128, 16, kPlain>,
                                                     kDecodeWaves * kWave, lds)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks,
                                                     decode_mfma_streamk_kernel<64, 16, kPlain>,
                                                     kDecodeWaves * kWave, lds);
  if (e != hipSuccess || blocks <= 0) return -1;
  return blocks * kDecodeWaves;
}

DecodePath decode_path(int num_seqs, int block_size, pa_dtype dtype, int partition_size,
                       bool vector_only) {
  if (dtype == PA_BF16 && !vector_only && partition_size == 0 && num_seqs <= kStreamKMaxSeqs &&
      block_size >= 8)
    return DecodePath::kStreamK;
  return DecodePath::kPartition;
}

DecodeWorkspace decode_workspace_partition(int num_seqs, int num_q_heads, int head_dim,
                                           int max_partitions) {
  DecodeWorkspace w{};
  if (max_partitions <= 1) return w;
  const size_t rows = (size_t)num_seqs * num_q_heads * max_partitions;
  w.m_off = 0;
  w.l_off = align256(rows * sizeof(float));
  w.acc_off = w.l_off + align256(rows * sizeof(float));
  w.total = w.acc_off + align256(rows * head_dim * sizeof(float));
  return w;
}

DecodeWorkspace decode_workspace_shared(int num_seqs, int num_q_heads, int head_dim) {
  // stream-K partials with 16 heads per slot (the prefix pass's widest
  // segments; the own-token pass reuses them), then the prefix results, the
  // log2-sum-exp of both passes, and the passes' per-group and per-sequence
  // data for the kernels after them
  DecodeWorkspace w = decode_workspace_streamk(num_seqs, 16, head_dim);
  const size_t rows = (size_t)num_seqs * num_q_heads;
  w.prefix_out_off = w.total;
  w.prefix_lse_off = w.prefix_out_off + align256(rows * head_dim * sizeof(float));
  w.lse_off = w.prefix_lse_off + align256(rows * sizeof(float));
  w.group_off = w.lse_off + align256(rows * sizeof(float));
  w.own_off = w.group_off + align256((size_t)3 * kSharedMaxGroups * sizeof(int32_t));
  w.total = w.own_off + align256((size_t)num_seqs * sizeof(int32_t));
  return w;
}

DecodeWorkspace decode_workspace_streamk(int num_seqs, int group, int head_dim) {
  (void)num_seqs;
  DecodeWorkspace w{};
  const size_t slots = (size_t)kStreamKMaxWorkers * 2 * group;
  w.handoff_off = 0;
  w.m_off = align256((size_t)kStreamKMaxWorkers * 2 * sizeof(int32_t));
  w.l_off = w.m_off + align256(slots * sizeof(float));
  w.acc_off = w.l_off + align256(slots * sizeof(float));
  w.total = w.acc_off + align256(slots * head_dim * sizeof(float));
  return w;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int block_size, pa_dtype dtype,
                         bool vector_only, DecodePath path, hipStream_t stream) {
  if (path == DecodePath::kStreamK) {
    return head_dim == 128 ? launch_streamk_bs<128>(p, block_size, stream)
                           : launch_streamk_bs<64>(p, block_size, stream);
  }
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
