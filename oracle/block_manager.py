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
  block when a sequence crosses a block boundary); "Sisa alokasi dibatasi
  oleh granularitas blok" (only the last block of a sequence can be
  partly empty); "Sharing blok dapat menghindari duplikasi state KV" (a block
  is shared while its content is unchanged; a writer gets separate storage).
* [bicarait] "Melihat Lebih Dalam vLLM v0.7 ...", "Blueprint Arsitektur 2"
  (allocate only when the current block is full) and "Berbagi Memori Fisik"
  (N samples point at the same prompt blocks).
* [gyaansetu] "KV Cache and PagedAttention: Why Your LLM Server Slows Down",
  "The memory problem" / "How PagedAttention fixes this": when HBM is full,
  pages (not whole sequences) move to CPU memory -- the model keeps a second
  set of blocks in host memory and moves a list of sequences' blocks there
  and back, keeping the sharing between them.

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
    def __init__(self, num_blocks, block_size, max_seqs, max_blocks_per_seq, num_host_blocks=0):
        if min(num_blocks, block_size, max_seqs, max_blocks_per_seq) < 1 or num_host_blocks < 0:
            raise ShapeError("sizes must be positive")
        self.num_blocks = num_blocks
        self.num_host_blocks = num_host_blocks
        self.block_size = block_size
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = list(range(num_blocks - 1, -1, -1))   # a stack: the end is the top
        self.refs = [0] * num_blocks                      # sequences holding each block
        self.fill = [0] * num_blocks                      # tokens stored in each block
        self.hfree = list(range(num_host_blocks - 1, -1, -1))  # host blocks, same policy
        self.hrefs = [0] * num_host_blocks
        self.hfill = [0] * num_host_blocks
        self.seqs = {}          # id -> {"len": n, "blocks": [...], "swapped": bool}

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
    def _resident(self, s):
        return s in self.seqs and not self.seqs[s]["swapped"]

    def add_sequence(self):
        def op(m):
            i = m._new_id()
            m.seqs[i] = {"len": 0, "blocks": [], "swapped": False}
            return i
        return self._commit(op)

    def fork(self, parent):
        def op(m):
            if not m._resident(parent):
                raise ShapeError("unknown or swapped sequence")
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
            host = m.seqs[seq]["swapped"]
            refs, fill, free = (m.hrefs, m.hfill, m.hfree) if host else (m.refs, m.fill, m.free)
            for b in m.seqs[seq]["blocks"]:
                refs[b] -= 1
                if refs[b] == 0:
                    fill[b] = 0
                    free.append(b)
            del m.seqs[seq]
        return self._commit(op)

    def _move(self, seq_ids, to_host):
        """Move the listed sequences' blocks to the other memory; pairs
        (old block, new block) in order of first appearance."""
        seq_ids = [int(s) for s in seq_ids]

        def op(m):
            if len(set(seq_ids)) != len(seq_ids):
                raise ShapeError("a sequence appears twice")
            for s in seq_ids:
                if s not in m.seqs or m.seqs[s]["swapped"] == to_host:
                    raise ShapeError("unknown sequence, or already on that side")
            src = (m.refs, m.fill, m.free) if to_host else (m.hrefs, m.hfill, m.hfree)
            dst = (m.hrefs, m.hfill, m.hfree) if to_host else (m.refs, m.fill, m.free)
            order, count = [], {}
            for s in seq_ids:
                for b in m.seqs[s]["blocks"]:
                    if b not in count:
                        order.append(b)
                        count[b] = 0
                    count[b] += 1
            for b in order:
                if src[0][b] != count[b]:
                    raise ShapeError("a block is also held by a sequence not listed")
            if len(order) > len(dst[2]):
                raise CapacityError("not enough free blocks on the other side")
            new = {}
            for b in order:
                nb = dst[2].pop()
                dst[0][nb] = src[0][b]
                dst[1][nb] = src[1][b]
                new[b] = nb
            for b in order:
                src[0][b] = 0
                src[1][b] = 0
                src[2].append(b)
            for s in seq_ids:
                m.seqs[s]["blocks"] = [new[b] for b in m.seqs[s]["blocks"]]
                m.seqs[s]["swapped"] = to_host
            return [(b, new[b]) for b in order]
        return self._commit(op)

    def swap_out(self, seq_ids):
        return self._move(seq_ids, True)

    def swap_in(self, seq_ids):
        return self._move(seq_ids, False)

    def append(self, seq_ids, counts):
        """Slots of the new tokens (in order) and the copy-on-write pairs."""
        seq_ids = [int(s) for s in seq_ids]
        counts = [int(c) for c in counts]

        def op(m):
            if len(set(seq_ids)) != len(seq_ids):
                raise ShapeError("a sequence appears twice")
            for s, c in zip(seq_ids, counts):
                if not m._resident(s) or c < 0:
                    raise ShapeError("unknown or swapped sequence, or negative count")
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
            if not self._resident(s):
                raise ShapeError("unknown or swapped sequence")
            b = self.seqs[s]["blocks"]
            rows.append(b + [-1] * (self.max_blocks_per_seq - len(b)))
            lens.append(self.seqs[s]["len"])
        return rows, lens

    def stats(self):
        used = [b for b in range(self.num_blocks) if self.refs[b] > 0]
        res = [r for r in self.seqs.values() if not r["swapped"]]
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": len(used),
            "shared_blocks": sum(1 for b in used if self.refs[b] > 1),
            "live_sequences": len(res),
            "logical_blocks": sum(len(r["blocks"]) for r in res),
            "logical_tokens": sum(r["len"] for r in res),
            "stored_tokens": sum(self.fill[b] for b in used),
            "physical_slots": len(used) * self.block_size,
            "swapped_sequences": len(self.seqs) - len(res),
            "num_host_blocks": self.num_host_blocks,
            "free_host_blocks": len(self.hfree),
        }
