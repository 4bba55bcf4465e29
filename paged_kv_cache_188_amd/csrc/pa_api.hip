// C ABI of libpa: argument validation, launch configuration, workspace sizing
// and error mapping.  Validation touches scalars and pointer values only and
// runs before any HIP call, so a rejected call has no effect.

#include <atomic>
#include <cmath>
#include <cstdint>

#include "pa_internal.h"

// Workspace of pa_decode_attention_noalloc: file-scope device memory, one
// copy per GPU the library runs on, held until the process ends.  Its size,
// PA_NOALLOC_MAX_WORKSPACE, covers the stream-K workspace of every supported
// shape (2048 wave slots x 2 partials x 16 heads x (128 + 2) floats, plus
// the hand-off entries) and fixed-partition workspaces up to the same size.
// Nothing in it has to start at zero: every entry a kernel reads was written
// earlier in the same call.  In host code `scratch` is only a handle, never a
// device address; the address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_MAX_WORKSPACE];

namespace {

bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }
bool supported_block_size(int32_t bs) { return bs == 8 || bs == 16 || bs == 32 || bs == 64; }
bool valid_dtype(pa_dtype t) { return t == PA_F32 || t == PA_BF16; }
int elem_bytes(pa_dtype t) { return t == PA_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// A partition is a whole number of 16-token tiles and of blocks, at most 64
// blocks (the decode kernel keeps one block id per lane).
bool valid_partition(int32_t part, int32_t bs) {
  return part > 0 && part % 16 == 0 && part % bs == 0 && part / bs <= 64;
}

// Library choice: start from the largest allowed partition (<= 1024 tokens)
// and halve while the grid would hold fewer than kTargetItems work items --
// enough independent waves to fill 256 CUs with several waves each -- but not
// below max(64, tile, block).
constexpr int64_t kTargetItems = 4096;

int32_t choose_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t bs, int32_t max_ctx) {
  const int32_t unit = bs > 16 ? bs : 16;
  int32_t part = 64 * bs < 1024 ? 64 * bs : 1024;
  part -= part % unit;
  const int32_t floor_part = unit > 64 ? unit : 64;
  auto items = [&](int32_t pt) {
    const int64_t p = max_ctx > 0 ? (max_ctx + (int64_t)pt - 1) / pt : 1;
    return (int64_t)num_seqs * num_kv_heads * p;
  };
  while (part / 2 >= floor_part && (part / 2) % unit == 0 && items(part) < kTargetItems) part /= 2;
  return part;
}

// Stream-K worker count for the current device: one wave per resident wave
// slot, capped by the workspace slots.  Cached per (device, head_dim); the
// only state the library keeps.
int streamk_workers(int head_dim, int* out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  const int k = head_dim == 128 ? 1 : 0;
  if (dev < kMaxDevices) {
    const int c = cache[dev][k].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return 0;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  const int per_cu = pa::streamk_workers_per_cu(head_dim);
  if (per_cu <= 0) return -1;
  int64_t w = (int64_t)cus * per_cu;
  if (w > pa::kStreamKMaxWorkers) w = pa::kStreamKMaxWorkers;
  w -= w % 4;  // whole workgroups of four waves
  if (w < 4) w = 4;
  if (dev < kMaxDevices) cache[dev][k].store((int)w, std::memory_order_relaxed);
  *out = (int)w;
  return 0;
}

// Device address of `scratch` on the current device, looked up once per
// device (nullptr on a HIP error).
void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  addr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(int s) {
  // an int, not a pa_status: an out-of-range enum value would be undefined
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case PA_ERR_DTYPE: return "unknown element type";
    case PA_ERR_UNSUPPORTED: return "head_dim, block_size, partition or alignment not supported";
    case PA_ERR_WORKSPACE: return "decode workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_CAPACITY: return "no free block or sequence slot left";
  }
  return "unknown status";
}

pa_status pa_compute_slots(int64_t* slots, const int32_t* block_tables, int32_t num_seqs,
                           int32_t max_blocks_per_seq, const int32_t* seq_ids,
                           const int32_t* positions, int32_t num_tokens, int32_t block_size,
                           int32_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1)
    return PA_ERR_SHAPE;
  if (!supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!slots || !positions || (num_seqs > 0 && !block_tables)) return PA_ERR_NULL;
  return from_hip(pa::launch_compute_slots(slots, block_tables, num_seqs, max_blocks_per_seq,
                                           seq_ids, positions, num_tokens, block_size, num_blocks,
                                           static_cast<hipStream_t>(stream)));
}

pa_status pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int32_t num_tokens, int64_t new_token_stride,
                      int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                      int32_t head_dim, pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 1 || num_kv_heads < 1) return PA_ERR_SHAPE;
  if (!supported_block_size(block_size) || !supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (new_token_stride == 0) new_token_stride = row;
  if (new_token_stride < row) return PA_ERR_SHAPE;
  const int e = elem_bytes(dtype);
  if ((new_token_stride * e) % 16) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return PA_ERR_UNSUPPORTED;
  return from_hip(pa::launch_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens,
                                      new_token_stride * e, num_blocks, block_size, num_kv_heads,
                                      head_dim * e, static_cast<hipStream_t>(stream)));
}

pa_status pa_write_kv_at(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int32_t* block_tables, int32_t num_seqs,
                         int32_t max_blocks_per_seq, const int32_t* seq_ids,
                         const int32_t* positions, int32_t num_tokens, int64_t new_token_stride,
                         int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, pa_dtype dtype, int64_t* slots_out, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      num_kv_heads < 1)
    return PA_ERR_SHAPE;
  if (!supported_block_size(block_size) || !supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (new_token_stride == 0) new_token_stride = row;
  if (new_token_stride < row) return PA_ERR_SHAPE;
  const int e = elem_bytes(dtype);
  if ((new_token_stride * e) % 16) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !positions || (num_seqs > 0 && !block_tables))
    return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return PA_ERR_UNSUPPORTED;
  return from_hip(pa::launch_write_kv_at(
      k_cache, v_cache, k_new, v_new, block_tables, num_seqs, max_blocks_per_seq, seq_ids,
      positions, slots_out, num_tokens, new_token_stride * e, num_blocks, block_size,
      num_kv_heads, head_dim * e, static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                         int32_t num_pairs, int32_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_pairs < 0 || num_blocks < 1 || num_kv_heads < 1) return PA_ERR_SHAPE;
  if (!supported_block_size(block_size) || !supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  return from_hip(pa::launch_copy_blocks(k_cache, v_cache, k_cache, v_cache, block_mapping,
                                         num_pairs, num_blocks, num_blocks, block_bytes,
                                         static_cast<hipStream_t>(stream)));
}

namespace {

// The address the current device uses for p: p itself for its own device
// memory, the mapped address for pinned host memory.  False for pageable
// host memory, another device's memory, or an unknown pointer (the kernel
// must never touch an address it cannot reach).
bool device_address(const void* p, const void** out) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // do not leave the query's error for the launch check
    return false;
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return false;
  if (a.isManaged) {
    *out = p;
    return true;
  }
  if (a.type == hipMemoryTypeDevice) {
    if (a.device != cur) return false;
    *out = p;
    return true;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer) {
    const char* host = static_cast<const char*>(a.hostPointer ? a.hostPointer : p);
    *out = static_cast<const char*>(a.devicePointer) + (static_cast<const char*>(p) - host);
    return true;
  }
  return false;
}

}  // namespace

pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                         const int32_t* block_mapping, int32_t num_pairs, int32_t src_num_blocks,
                         int32_t dst_num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_pairs < 0 || src_num_blocks < 1 || dst_num_blocks < 1 || num_kv_heads < 1)
    return PA_ERR_SHAPE;
  if (!supported_block_size(block_size) || !supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_mapping) return PA_ERR_NULL;
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v))
    return PA_ERR_UNSUPPORTED;
  if (dst_k == src_k || dst_v == src_v) return PA_ERR_SHAPE;  // within one pool: pa_copy_blocks
  const void *dk, *dv, *sk, *sv, *map;
  if (!device_address(dst_k, &dk) || !device_address(dst_v, &dv) ||
      !device_address(src_k, &sk) || !device_address(src_v, &sv) ||
      !device_address(block_mapping, &map))
    return PA_ERR_UNSUPPORTED;  // not reachable from this device
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  return from_hip(pa::launch_copy_blocks(const_cast<void*>(dk), const_cast<void*>(dv), sk, sv,
                                         static_cast<const int32_t*>(map), num_pairs,
                                         src_num_blocks, dst_num_blocks, block_bytes,
                                         static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                 int32_t max_context_len, int32_t partition_size) {
  if (!supported_block_size(block_size) || num_seqs < 0 || num_kv_heads < 1 || max_context_len < 0)
    return 0;
  if (partition_size != 0) return valid_partition(partition_size, block_size) ? partition_size : 0;
  return choose_partition(num_seqs, num_kv_heads, block_size, max_context_len);
}

int32_t pa_decode_streamk_workers(int32_t num_seqs, int32_t head_dim, int32_t block_size,
                                  int32_t partition_size, pa_dtype dtype, uint32_t flags) {
  if (num_seqs < 0 || !supported_head_dim(head_dim) || !supported_block_size(block_size) ||
      !valid_dtype(dtype) || (flags & ~PA_DECODE_VECTOR_ONLY))
    return -1;
  const bool vector_only = (flags & PA_DECODE_VECTOR_ONLY) != 0;
  if (pa::decode_path(num_seqs, block_size, dtype, partition_size, vector_only) !=
      pa::DecodePath::kStreamK)
    return 0;
  int workers = 0;
  if (streamk_workers(head_dim, &workers) != 0) return -1;
  return workers;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                int32_t partition_size, pa_dtype dtype, uint32_t flags) {
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads ||
      !supported_head_dim(head_dim) || !valid_dtype(dtype) || num_seqs <= 0)
    return 0;  // invalid arguments, or no sequence: nothing to hold
  const bool vector_only = (flags & PA_DECODE_VECTOR_ONLY) != 0;
  if (pa::decode_path(num_seqs, block_size, dtype, partition_size, vector_only) ==
      pa::DecodePath::kStreamK)
    return pa::decode_workspace_streamk(num_seqs, num_q_heads / num_kv_heads, head_dim).total;
  const int32_t part = pa_decode_partition_size(num_seqs, num_kv_heads, block_size,
                                                max_context_len, partition_size);
  if (part <= 0) return 0;
  const int64_t P = max_context_len > 0 ? (max_context_len + (int64_t)part - 1) / part : 1;
  return pa::decode_workspace_partition(num_seqs, num_q_heads, head_dim, (int)P).total;
}

namespace {

// Decode, optionally with each sequence's new token appended first (k_new
// non-null): shared by pa_decode_attention and pa_decode_attention_append.
pa_status decode_impl(float* out, const void* q, const void* k_cache, const void* v_cache,
                      const void* k_new, const void* v_new, int64_t new_token_stride,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t max_context_len, float scale, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, pa_dtype dtype, uint32_t flags,
                      bool append, bool static_scratch, void* stream,
                      const int32_t* group_start = nullptr, const int32_t* shared_len = nullptr,
                      int32_t num_groups = 0) {
  if (!valid_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1 || max_context_len < 0 || num_q_heads % num_kv_heads)
    return PA_ERR_SHAPE;
  if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  if (flags & ~PA_DECODE_VECTOR_ONLY) return PA_ERR_UNSUPPORTED;
  if (partition_size != 0 && !valid_partition(partition_size, block_size)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  // every context is clamped to the caller's bound and to what the table holds
  const int32_t max_tokens = max_context_len < max_blocks_per_seq * block_size
                                 ? max_context_len
                                 : max_blocks_per_seq * block_size;
  const bool vector_only = (flags & PA_DECODE_VECTOR_ONLY) != 0;
  const pa::DecodePath path =
      pa::decode_path(num_seqs, block_size, dtype, partition_size, vector_only);
  // Same partition, partition count and workspace as pa_decode_workspace_size.
  const int32_t part = partition_size ? partition_size
                                      : choose_partition(num_seqs, num_kv_heads, block_size,
                                                         max_context_len);
  const int64_t P = max_context_len > 0 ? (max_context_len + (int64_t)part - 1) / part : 1;
  // a launch holds at most 2^32 - 1 work-items: on the fixed-partition path
  // one wave per work item and 256 threads per (sequence, head) in the merge
  if (path != pa::DecodePath::kStreamK && ((int64_t)num_seqs * num_kv_heads * P * 64 > UINT32_MAX ||
                                           (int64_t)num_seqs * num_q_heads * 256 > UINT32_MAX))
    return PA_ERR_SHAPE;
  const bool shared = group_start != nullptr;
  if (shared) {  // the two stream-K passes only
    if (path != pa::DecodePath::kStreamK) return PA_ERR_UNSUPPORTED;
    if (num_seqs > pa::kSharedMaxSeqs || num_groups < 1 || num_groups > pa::kSharedMaxGroups)
      return PA_ERR_SHAPE;
  }
  if (num_seqs == 0) return PA_OK;
  const pa::DecodeWorkspace ws =
      shared ? pa::decode_workspace_shared(num_seqs, num_q_heads, head_dim)
      : path == pa::DecodePath::kStreamK
          ? pa::decode_workspace_streamk(num_seqs, num_q_heads / num_kv_heads, head_dim)
          : pa::decode_workspace_partition(num_seqs, num_q_heads, head_dim, (int)P);
  if (static_scratch) {
    if (ws.total > PA_NOALLOC_MAX_WORKSPACE) return PA_ERR_WORKSPACE;
  } else {
    if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return PA_ERR_WORKSPACE;
    if (ws.total > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return PA_ERR_WORKSPACE;
  }
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (shared && !shared_len) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const int e = elem_bytes(dtype);
  if (append) {
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (new_token_stride == 0) new_token_stride = row;
    if (new_token_stride < row) return PA_ERR_SHAPE;
    if ((new_token_stride * e) % 16) return PA_ERR_UNSUPPORTED;
    if (!k_new || !v_new) return PA_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_UNSUPPORTED;
  }
  if (static_scratch && ws.total > 0) {  // validation done: the first HIP call
    workspace = noalloc_scratch();
    if (!workspace) return PA_ERR_HIP;
  }

  pa::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  char* wsb = static_cast<char*>(workspace);
  if (ws.total) {
    p.ws_m = reinterpret_cast<float*>(wsb + ws.m_off);
    p.ws_l = reinterpret_cast<float*>(wsb + ws.l_off);
    p.ws_acc = reinterpret_cast<float*>(wsb + ws.acc_off);
    if (path == pa::DecodePath::kStreamK)
      p.ws_handoff = reinterpret_cast<int32_t*>(wsb + ws.handoff_off);
    if (shared) {
      p.prefix_out = reinterpret_cast<float*>(wsb + ws.prefix_out_off);
      p.prefix_lse = reinterpret_cast<float*>(wsb + ws.prefix_lse_off);
      p.lse_out = reinterpret_cast<float*>(wsb + ws.lse_off);
      p.group_ws = reinterpret_cast<int32_t*>(wsb + ws.group_off);
      p.own_ws = reinterpret_cast<int32_t*>(wsb + ws.own_off);
      p.group_start = group_start;
      p.shared_len = shared_len;
      p.num_groups = num_groups;
      p.group_cap = 16 / (num_q_heads / num_kv_heads);
    }
  }
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.block_size = block_size;
  p.scale_log2 = scale * 1.4426950408889634f;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (path == pa::DecodePath::kStreamK) {
    int workers = 0;
    if (streamk_workers(head_dim, &workers) != 0) return PA_ERR_HIP;
    p.max_workers = workers;
    p.partition = 16;
    p.max_partitions = 1;
    p.max_tokens = max_tokens;
    if (append) {  // the decode kernel appends the new tokens itself
      p.k_new = k_new;
      p.v_new = v_new;
      p.new_stride = new_token_stride;
    }
  } else {
    p.partition = part;
    p.max_partitions = (int)P;
    p.max_tokens = max_tokens;  // <= P * part, so every token lies in a partition
    if (append) {  // store the new tokens first, then attend
      const pa_status st = from_hip(pa::launch_append_kv(
          const_cast<void*>(k_cache), const_cast<void*>(v_cache), k_new, v_new,
          new_token_stride * e, block_tables, context_lens, num_seqs, max_blocks_per_seq,
          max_tokens, num_blocks, block_size, num_kv_heads, head_dim * e, hs));
      if (st != PA_OK) return st;
    }
  }
  return from_hip(pa::launch_decode(p, head_dim, block_size, dtype, vector_only, path, hs));
}

}  // namespace

pa_status pa_decode_attention(float* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                              int32_t partition_size, void* workspace, size_t workspace_bytes,
                              pa_dtype dtype, uint32_t flags, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, nullptr, nullptr, 0, block_tables, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, flags, false, false, stream);
}

pa_status pa_decode_attention_append(float* out, const void* q, void* k_cache, void* v_cache,
                                     const void* k_new, const void* v_new,
                                     int64_t new_token_stride, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, pa_dtype dtype, uint32_t flags,
                                     void* stream) {
  return decode_impl(out, q, k_cache, v_cache, k_new, v_new, new_token_stride, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, scale, partition_size,
                     workspace, workspace_bytes, dtype, flags, true, false, stream);
}

size_t pa_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype) {
  if (num_seqs <= 0 || num_seqs > pa::kSharedMaxSeqs || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > 16 ||
      !supported_head_dim(head_dim) || dtype != PA_BF16)
    return 0;
  return pa::decode_workspace_shared(num_seqs, num_q_heads, head_dim).total;
}

pa_status pa_decode_attention_shared(float* out, const void* q, void* k_cache, void* v_cache,
                                     const void* k_new, const void* v_new,
                                     int64_t new_token_stride, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* group_start,
                                     const int32_t* shared_len, int32_t num_groups,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, void* workspace, size_t workspace_bytes,
                                     pa_dtype dtype, void* stream) {
  if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
  if (!group_start) return PA_ERR_NULL;
  return decode_impl(out, q, k_cache, v_cache, k_new, v_new, new_token_stride, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, scale, 0, workspace,
                     workspace_bytes, dtype, 0, k_new != nullptr, false, stream, group_start,
                     shared_len, num_groups);
}

pa_status pa_decode_attention_noalloc(float* out, const void* q, void* k_cache, void* v_cache,
                                      const void* k_new, const void* v_new,
                                      int64_t new_token_stride, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t partition_size, pa_dtype dtype,
                                      uint32_t flags, void* stream) {
  if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
  return decode_impl(out, q, k_cache, v_cache, k_new, v_new, new_token_stride, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, scale, partition_size,
                     nullptr, 0, dtype, flags, k_new != nullptr, true, stream);
}

pa_status pa_prefill_attention(float* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start,
                               int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_query_len, float scale, pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_tokens < 0 || max_query_len < 0 || num_q_heads < 1 ||
      num_kv_heads < 1 || num_blocks < 1 || max_blocks_per_seq < 1 ||
      num_q_heads % num_kv_heads)
    return PA_ERR_SHAPE;
  if (dtype != PA_BF16 || block_size < 16) return PA_ERR_UNSUPPORTED;
  if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  {  // one workgroup per (sequence, KV head, query tile): at most 2^32 - 1
     // work-items in the launch
    const int32_t tq = pa::prefill_tokens_per_workgroup(num_q_heads / num_kv_heads);
    const int64_t items = (int64_t)num_seqs * num_kv_heads * ((max_query_len + tq - 1) / tq);
    if (items * pa::prefill_threads_per_workgroup() > UINT32_MAX) return PA_ERR_SHAPE;
  }
  if (num_seqs == 0 || num_q_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  pa::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.block_size = block_size;
  p.max_tokens = max_blocks_per_seq * block_size;
  p.scale_log2 = scale * 1.4426950408889634f;
  return from_hip(pa::launch_prefill(p, query_start, num_q_tokens, max_query_len, head_dim,
                                     block_size, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
