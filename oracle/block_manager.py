"""Plain reference model of the host KV block manager.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product never
imports this module.

What it models, from the pages (cited by title and section):

* [gininih] "Apa itu PagedAttention (Manajemen Memori KV Cache GPU)?",
  "Cara kerja PagedAttention": the KV cache is cut into fixed-size blocks; a
  block table maps a sequence's logical order to physical blocks, which can be
  anywhere; when the active block is full another free block is taken;
  requests may share physical blocks, and a branch that diverges gets a
  copied block (copy-on-write).
* [nalar] "PagedAttention: memetakan blok KV logis ke memori fisik tidak
  kontigu": "Urutan logis dipisahkan dari penempatan fisik" (a new physical
  block when a sequence crosses a block boundary); "Sisa alokasi tetap ada,
  tetapi dibatasi ukuran blok" (only the last block of a sequence can be
  partly empty); "Sharing blok dapat menghindari duplikasi state KV" (a block
  is shared while its content is unchanged; a writer gets separate storage).
* [bicarait] "Melihat Lebih Dalam vLLM v0.7 ...", "Blueprint Arsitektur 2"
  (allocate only when the current block is full) and "Berbagi Memori Fisik"
  (N samples point at the same prompt blocks).

The pages fix no allocation order; the model uses the policy the library
documents (a free stack with block 0 on top, freed blocks pushed back in
table order, the lowest free sequence id reused first) so that the two can
be compared exactly.  Every operation is all-or-nothing: it runs on a copy
of the state, which replaces the state only when the operation succeeds.
"""

from __future__ import annotations

import copy


class ShapeError(ValueError):
    """Unknown or repeated sequence, negative count (the library's
    PA_ERR_SHAPE)."""


class CapacityError(RuntimeError):
    """No free block, sequence id or table entry left (PA_ERR_CAPACITY)."""


class BlockManager:
    def __init__(self, num_blocks, block_size, max_seqs, max_blocks_per_seq):
        if min(num_blocks, block_size, max_seqs, max_blocks_per_seq) < 1:
            raise ShapeError("sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = list(range(num_blocks - 1, -1, -1))   # a stack: the end is the top
        self.refs = [0] * num_blocks                      # sequences holding each block
        self.fill = [0] * num_blocks                      # tokens stored in each block
        self.seqs = {}                                    # id -> {"len": n, "blocks": [...]}

    # -- helpers -----------------------------------------------------------
    def _take_block(self):
        if not self.free:
            raise CapacityError("no free block")
        b = self.free.pop()
        self.refs[b] = 1
        self.fill[b] = 0
        return b

    def _new_id(self):
        for i in range(self.max_seqs):
            if i not in self.seqs:
                return i
        raise CapacityError("no free sequence id")

    def _commit(self, fn):
        trial = copy.deepcopy(self)
        result = fn(trial)
        self.__dict__.update(trial.__dict__)
        return result

    # -- operations ----------------------------------------------------------
    def add_sequence(self):
        def op(m):
            i = m._new_id()
            m.seqs[i] = {"len": 0, "blocks": []}
            return i
        return self._commit(op)

    def fork(self, parent):
        def op(m):
            if parent not in m.seqs:
                raise ShapeError("unknown sequence")
            i = m._new_id()
            m.seqs[i] = copy.deepcopy(m.seqs[parent])
            for b in m.seqs[i]["blocks"]:
                m.refs[b] += 1
            return i
        return self._commit(op)

    def free_sequence(self, seq):
        def op(m):
            if seq not in m.seqs:
                raise ShapeError("unknown sequence")
            for b in m.seqs[seq]["blocks"]:
                m.refs[b] -= 1
                if m.refs[b] == 0:
                    m.fill[b] = 0
                    m.free.append(b)
            del m.seqs[seq]
        return self._commit(op)

    def append(self, seq_ids, counts):
        """Slots of the new tokens (in order) and the copy-on-write pairs."""
        seq_ids = [int(s) for s in seq_ids]
        counts = [int(c) for c in counts]

        def op(m):
            if len(set(seq_ids)) != len(seq_ids):
                raise ShapeError("a sequence appears twice")
            for s, c in zip(seq_ids, counts):
                if s not in m.seqs or c < 0:
                    raise ShapeError("unknown sequence or negative count")
            for s, c in zip(seq_ids, counts):
                if m.seqs[s]["len"] + c > m.max_blocks_per_seq * m.block_size:
                    raise CapacityError("the table would be too long")
            slots, copies = [], []
            for s, c in zip(seq_ids, counts):
                rec = m.seqs[s]
                for _ in range(c):
                    p = rec["len"]
                    logical, offset = p // m.block_size, p % m.block_size
                    if logical == len(rec["blocks"]):
                        rec["blocks"].append(m._take_block())     # crossing a boundary
                    elif m.refs[rec["blocks"][logical]] > 1:       # shared: copy first
                        old = rec["blocks"][logical]
                        new = m._take_block()
                        m.fill[new] = m.fill[old]
                        m.refs[old] -= 1
                        rec["blocks"][logical] = new
                        copies.append((old, new))
                    phys = rec["blocks"][logical]
                    slots.append(phys * m.block_size + offset)
                    m.fill[phys] = max(m.fill[phys], offset + 1)
                    rec["len"] = p + 1
            return slots, copies
        return self._commit(op)

    def tables(self, seq_ids):
        rows, lens = [], []
        for s in seq_ids:
            if s not in self.seqs:
                raise ShapeError("unknown sequence")
            b = self.seqs[s]["blocks"]
            rows.append(b + [-1] * (self.max_blocks_per_seq - len(b)))
            lens.append(self.seqs[s]["len"])
        return rows, lens

    def stats(self):
        used = [b for b in range(self.num_blocks) if self.refs[b] > 0]
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": len(used),
            "shared_blocks": sum(1 for b in used if self.refs[b] > 1),
            "live_sequences": len(self.seqs),
            "logical_blocks": sum(len(r["blocks"]) for r in self.seqs.values()),
            "logical_tokens": sum(r["len"] for r in self.seqs.values()),
            "stored_tokens": sum(self.fill[b] for b in used),
            "physical_slots": len(used) * self.block_size,
        }
