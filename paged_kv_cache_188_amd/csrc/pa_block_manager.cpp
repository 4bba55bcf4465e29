// Host-side KV block manager: free stack, per-sequence block tables,
// reference counts of shared blocks and copy-on-write (see
// include/pa_block_manager.h for the policy and the passages it follows).

#include "pa_block_manager.h"

#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

struct pa_block_manager {
  struct Seq {
    bool live = false;
    bool swapped = false;         // blocks are host blocks (swapped out)
    int64_t len = 0;              // tokens
    std::vector<int32_t> blocks;  // physical block of each logical block
  };
  // One address space's blocks: reference counts, fill and a free stack.
  struct Space {
    std::vector<int32_t> refs;        // references per block
    std::vector<int32_t> fill;        // tokens held by each block
    std::vector<int32_t> free_stack;  // top = back
    void init(int32_t n) {
      refs.assign(n, 0);
      fill.assign(n, 0);
      free_stack.clear();
      free_stack.reserve(n);
      for (int32_t b = n - 1; b >= 0; --b) free_stack.push_back(b);  // 0 on top
    }
    int32_t pop() {
      const int32_t b = free_stack.back();
      free_stack.pop_back();
      refs[b] = 1;
      fill[b] = 0;
      return b;
    }
    void release(int32_t b) {  // one reference less; free when none is left
      if (--refs[b] == 0) {
        fill[b] = 0;
        free_stack.push_back(b);
      }
    }
  };

  int32_t num_blocks = 0, num_host_blocks = 0, block_size = 0, max_seqs = 0,
          max_blocks_per_seq = 0;
  Space gpu, host;
  // gpu.refs / gpu.fill under their old names for the code below
  std::vector<int32_t>& refs = gpu.refs;
  std::vector<int32_t>& fill = gpu.fill;
  std::vector<int32_t>& free_stack = gpu.free_stack;
  std::vector<Seq> seqs;
  mutable std::mutex mu;

  bool valid_seq(int32_t s) const {
    return s >= 0 && s < static_cast<int32_t>(seqs.size()) && seqs[s].live;
  }
  bool resident_seq(int32_t s) const { return valid_seq(s) && !seqs[s].swapped; }
  int32_t pop_block() { return gpu.pop(); }
  // Lowest free sequence id (or -1).
  int32_t new_seq_id() {
    for (int32_t i = 0; i < static_cast<int32_t>(seqs.size()); ++i)
      if (!seqs[i].live) return i;
    if (static_cast<int32_t>(seqs.size()) < max_seqs) {
      seqs.emplace_back();
      return static_cast<int32_t>(seqs.size()) - 1;
    }
    return -1;
  }
};

extern "C" {

pa_status pa_bm_create_with_host(int32_t num_blocks, int32_t num_host_blocks,
                                 int32_t block_size, int32_t max_seqs,
                                 int32_t max_blocks_per_seq, pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  if (num_blocks < 1 || num_host_blocks < 0 || block_size < 1 || max_seqs < 1 ||
      max_blocks_per_seq < 1)
    return PA_ERR_SHAPE;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_CAPACITY;
  bm->num_blocks = num_blocks;
  bm->num_host_blocks = num_host_blocks;
  bm->block_size = block_size;
  bm->max_seqs = max_seqs;
  bm->max_blocks_per_seq = max_blocks_per_seq;
  bm->gpu.init(num_blocks);
  bm->host.init(num_host_blocks);
  *out = bm;
  return PA_OK;
}

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                       int32_t max_blocks_per_seq, pa_block_manager** out) {
  return pa_bm_create_with_host(num_blocks, 0, block_size, max_seqs, max_blocks_per_seq, out);
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq) {
  if (!bm || !seq) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  const int32_t id = bm->new_seq_id();
  if (id < 0) return PA_ERR_CAPACITY;
  bm->seqs[id] = pa_block_manager::Seq{true, 0, {}};
  *seq = id;
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child) {
  if (!bm || !child) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->resident_seq(parent)) return PA_ERR_SHAPE;
  const int32_t id = bm->new_seq_id();
  if (id < 0) return PA_ERR_CAPACITY;
  pa_block_manager::Seq s = bm->seqs[parent];  // copy before seqs may grow
  for (int32_t b : s.blocks) ++bm->refs[b];
  bm->seqs[id] = std::move(s);
  *child = id;
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq) {
  if (!bm) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->valid_seq(seq)) return PA_ERR_SHAPE;
  pa_block_manager::Seq& s = bm->seqs[seq];
  pa_block_manager::Space& sp = s.swapped ? bm->host : bm->gpu;
  for (int32_t b : s.blocks) sp.release(b);
  s = pa_block_manager::Seq{};
  return PA_OK;
}

namespace {

// Move every block of sequences ids[0..n-1] from space `from` to space `to`
// (swap-out: GPU -> host; swap-in: host -> GPU).  Each distinct block gets
// one block of `to`, in order of first appearance (sequence by sequence,
// table order); the pairs (old, new) go to pairs.  A block also held by a
// sequence outside the list cannot move (PA_ERR_SHAPE); too few free blocks
// in `to` give PA_ERR_CAPACITY; either leaves the manager unchanged.
pa_status move_sequences(pa_block_manager* bm, const int32_t* ids, int32_t n, bool to_host,
                         int32_t* pairs, int32_t* num_pairs) {
  pa_block_manager::Space& from = to_host ? bm->gpu : bm->host;
  pa_block_manager::Space& to = to_host ? bm->host : bm->gpu;
  std::vector<char> seen(bm->seqs.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (!bm->valid_seq(id) || seen[id] || bm->seqs[id].swapped != !to_host) return PA_ERR_SHAPE;
    seen[id] = 1;
  }
  std::unordered_map<int32_t, int32_t> listed;  // block -> references from the listed sequences
  std::vector<int32_t> order;                   // distinct blocks, first appearance
  for (int32_t i = 0; i < n; ++i)
    for (int32_t b : bm->seqs[ids[i]].blocks)
      if (listed[b]++ == 0) order.push_back(b);
  for (int32_t b : order)
    if (from.refs[b] != listed[b]) return PA_ERR_SHAPE;  // held by a sequence not listed
  if (order.size() > to.free_stack.size()) return PA_ERR_CAPACITY;
  if (!order.empty() && !pairs) return PA_ERR_NULL;
  std::unordered_map<int32_t, int32_t> moved;
  for (size_t k = 0; k < order.size(); ++k) {
    const int32_t b = order[k];
    const int32_t nb = to.pop();
    to.refs[nb] = from.refs[b];
    to.fill[nb] = from.fill[b];
    moved[b] = nb;
    pairs[2 * k] = b;
    pairs[2 * k + 1] = nb;
  }
  for (int32_t b : order) {  // freed in pair order
    from.refs[b] = 1;
    from.release(b);
  }
  for (int32_t i = 0; i < n; ++i) {
    pa_block_manager::Seq& s = bm->seqs[ids[i]];
    for (int32_t& b : s.blocks) b = moved[b];
    s.swapped = to_host;
  }
  *num_pairs = static_cast<int32_t>(order.size());
  return PA_OK;
}

}  // namespace

pa_status pa_bm_swap_out(pa_block_manager* bm, const int32_t* seq_ids, int32_t n,
                         int32_t* pairs, int32_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  *num_pairs = 0;
  if (n == 0) return PA_OK;
  if (!seq_ids) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  return move_sequences(bm, seq_ids, n, true, pairs, num_pairs);
}

pa_status pa_bm_swap_in(pa_block_manager* bm, const int32_t* seq_ids, int32_t n,
                        int32_t* pairs, int32_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  *num_pairs = 0;
  if (n == 0) return PA_OK;
  if (!seq_ids) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  return move_sequences(bm, seq_ids, n, false, pairs, num_pairs);
}

pa_status pa_bm_append(pa_block_manager* bm, const int32_t* seq_ids, const int32_t* counts,
                       int32_t n, int64_t* slots, int32_t* copy_pairs, int32_t* num_copies) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) {
    if (num_copies) *num_copies = 0;
    return PA_OK;
  }
  if (!seq_ids || !counts || !num_copies) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  // Check everything first: the call changes nothing unless it succeeds.
  // The count of blocks taken follows the appends in order: a sequence that
  // copies a shared block drops one of its references, so a later sharer in
  // the same call may then own it alone and write in place.
  std::vector<char> seen(bm->seqs.size(), 0);
  std::unordered_map<int32_t, int32_t> dropped;  // references released by copies so far
  int64_t total = 0, need = 0;
  bool any_copy = false;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = seq_ids[i];
    if (!bm->resident_seq(id) || seen[id] || counts[i] < 0) return PA_ERR_SHAPE;
    seen[id] = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    const pa_block_manager::Seq& s = bm->seqs[seq_ids[i]];
    if (s.len + counts[i] > static_cast<int64_t>(bm->max_blocks_per_seq) * bm->block_size)
      return PA_ERR_CAPACITY;
    if (counts[i] == 0) continue;
    total += counts[i];
    const int64_t have = static_cast<int64_t>(s.blocks.size());
    need += (s.len + counts[i] + bm->block_size - 1) / bm->block_size - have;
    if (s.len % bm->block_size != 0) {
      const int32_t last = s.blocks.back();
      auto it = dropped.find(last);
      const int32_t r = bm->refs[last] - (it == dropped.end() ? 0 : it->second);
      if (r > 1) {  // this append copies the block
        ++need;
        ++dropped[last];
        any_copy = true;
      }
    }
  }
  if (need > static_cast<int64_t>(bm->free_stack.size())) return PA_ERR_CAPACITY;
  if (total > 0 && !slots) return PA_ERR_NULL;
  if (any_copy && !copy_pairs) return PA_ERR_NULL;

  int64_t k = 0;
  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    pa_block_manager::Seq& s = bm->seqs[seq_ids[i]];
    for (int32_t c = 0; c < counts[i]; ++c) {
      const int64_t pos = s.len;
      const int64_t lb = pos / bm->block_size;
      const int32_t off = static_cast<int32_t>(pos - lb * bm->block_size);
      if (lb == static_cast<int64_t>(s.blocks.size())) {
        s.blocks.push_back(bm->pop_block());  // crossing into a new logical block
      } else if (bm->refs[s.blocks[lb]] > 1) {  // writing into a shared partial block
        const int32_t old = s.blocks[lb];
        const int32_t fresh = bm->pop_block();
        bm->fill[fresh] = bm->fill[old];
        --bm->refs[old];
        s.blocks[lb] = fresh;
        copy_pairs[2 * copies] = old;
        copy_pairs[2 * copies + 1] = fresh;
        ++copies;
      }
      const int32_t phys = s.blocks[lb];
      slots[k++] = static_cast<int64_t>(phys) * bm->block_size + off;
      if (bm->fill[phys] < off + 1) bm->fill[phys] = off + 1;
      s.len = pos + 1;
    }
  }
  *num_copies = copies;
  return PA_OK;
}

pa_status pa_bm_tables(const pa_block_manager* bm, const int32_t* seq_ids, int32_t n,
                       int32_t* tables, int32_t* lens) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!seq_ids || !tables || !lens) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  for (int32_t i = 0; i < n; ++i)
    if (!bm->resident_seq(seq_ids[i])) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    const pa_block_manager::Seq& s = bm->seqs[seq_ids[i]];
    int32_t* row = tables + static_cast<int64_t>(i) * bm->max_blocks_per_seq;
    for (int32_t b = 0; b < bm->max_blocks_per_seq; ++b)
      row[b] = b < static_cast<int32_t>(s.blocks.size()) ? s.blocks[b] : -1;
    lens[i] = static_cast<int32_t>(s.len);
  }
  return PA_OK;
}

pa_status pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* st) {
  if (!bm || !st) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  pa_bm_stats r{};
  r.num_blocks = bm->num_blocks;
  r.free_blocks = static_cast<int32_t>(bm->free_stack.size());
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->refs[b] > 0) {
      ++r.used_blocks;
      r.stored_tokens += bm->fill[b];
    }
    if (bm->refs[b] > 1) ++r.shared_blocks;
  }
  for (const auto& s : bm->seqs)
    if (s.live && !s.swapped) {
      ++r.live_sequences;
      r.logical_blocks += static_cast<int64_t>(s.blocks.size());
      r.logical_tokens += s.len;
    } else if (s.live) {
      ++r.swapped_sequences;
    }
  r.physical_slots = static_cast<int64_t>(r.used_blocks) * bm->block_size;
  r.num_host_blocks = bm->num_host_blocks;
  r.free_host_blocks = static_cast<int32_t>(bm->host.free_stack.size());
  *st = r;
  return PA_OK;
}

}  // extern "C"
