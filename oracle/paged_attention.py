"""Plain, slow, float64 reference of the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (the four pages on PagedAttention; cited by page title and section):

* [nalar] "PagedAttention: memetakan blok KV logis ke memori fisik tidak
  kontigu" (nalar.dev) -- the most precise page.  Its introduction says the
  attention equation itself is unchanged by paging; "Urutan logis dipisahkan
  dari penempatan fisik" gives the logical-block -> physical-block table with a
  worked example; "Kernel attention harus mengikuti block table" says the
  kernel walks the logical context and translates each logical block to its
  physical block before loading K and V; "Sharing blok dapat menghindari
  duplikasi state KV" defines sharing and copy-on-write as storage identity,
  not approximation; "Paging tidak mengompresi KV cache secara matematis" says
  no token is dropped or compressed.
* [bicarait] "Melihat Lebih Dalam vLLM v0.7: Bagaimana PagedAttention & Chunked
  Prefill ..." -- "Blueprint Arsitektur 2" maps logical block index L_i to a
  physical location and allocates a new block only when the current one is
  full; the TL;DR diagram shows 16-token logical blocks in frames 41, 08, 93.
* [gininih] "Apa itu PagedAttention (Manajemen Memori KV Cache GPU)?" -- "Cara
  kerja PagedAttention" (fixed-size KV blocks, block table, copy-on-write);
  "Batasan dan salah paham umum" (cached values are identical, so accuracy is
  unchanged).
* [gyaansetu] "KV Cache and PagedAttention: Why Your LLM Server Slows Down" --
  "Apa itu KV Cache?": only the new token's K and V are computed; earlier ones
  are read back from the cache.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* Pool layout: separate K and V pools.  V is ``[num_blocks][num_kv_heads]
  [block_size][head_dim]`` (one row per token).  K keeps each token's row as
  16-byte granules of ``x = 16 / element_bytes`` elements, token-minor:
  ``[num_blocks][num_kv_heads][head_dim / x][block_size][x]``; element ``d`` of
  token ``o`` of a block is ``K[blk][h][d // x][o][d % x]``.  (The pages fix
  no in-block layout; this one makes the matrix-core operand loads of the GPU
  kernel contiguous.)
* Offset inside a block: token ``p`` sits at offset ``p mod block_size`` of
  logical block ``p // block_size`` (tokens in logical order inside a block,
  as in a page table).
* Slot = ``table[p // bs] * bs + p mod bs``; a negative position is a padding
  token whose slot is -1 and whose write is skipped.
* Grouped-query attention: query head ``h`` reads KV head ``h // (Hq/Hkv)``.
* The query attends to exactly the first ``ctx`` logical tokens; ``ctx == 0``
  gives an all-zero output.
* ``scale`` is a float32 number; the oracle uses its exact float32 value.
"""

from __future__ import annotations

import numpy as np

BF16 = "bf16"
F32 = "f32"
ORACLE_DTYPES = (BF16, F32)


class ContractError(ValueError):
    """An input violates the documented contract (the oracle refuses it)."""


# ---------------------------------------------------------------------------
# values
# ---------------------------------------------------------------------------

def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements.

    bf16 elements are stored as their uint16 bit patterns: the float32 with the
    same top 16 bits is their exact value.  float32 widens exactly.
    """
    if dtype == BF16:
        b = np.ascontiguousarray(bits).view(np.uint16)
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        return np.ascontiguousarray(bits).view(np.float32).astype(np.float64)
    raise ContractError(f"unknown dtype {dtype!r}")


def pool_dims(k_pool: np.ndarray, v_pool: np.ndarray):
    """(num_blocks, num_kv_heads, block_size, head_dim, x) of a K/V pool pair."""
    if k_pool.ndim != 5 or v_pool.ndim != 4:
        raise ContractError("K pool must be [NB][Hkv][D/x][bs][x], V pool [NB][Hkv][bs][D]")
    nb, hkv, dx, bs, x = k_pool.shape
    if v_pool.shape != (nb, hkv, bs, dx * x):
        raise ContractError("K and V pools disagree")
    return nb, hkv, bs, dx * x, x


def _k_rows(k_pool: np.ndarray, blocks, heads, offsets) -> np.ndarray:
    """K rows ``[n][D]`` of tokens (blocks[i], heads, offsets[i]) from the
    granule layout (a pure re-indexing)."""
    g = k_pool[blocks, heads, :, offsets, :]          # [n][D/x][x]
    return g.reshape(g.shape[0], -1)


# ---------------------------------------------------------------------------
# a1: logical position -> physical slot
# ---------------------------------------------------------------------------

def _logical_block(p: int, block_size: int) -> int:
    """Logical block that holds logical token ``p`` (fixed-size blocks)."""
    return p // block_size


def _offset_in_block(p: int, block_size: int) -> int:
    """Offset of logical token ``p`` inside its block (tokens kept in order)."""
    return p % block_size


def slot_mapping(block_tables: np.ndarray, seq_ids: np.ndarray,
                 positions: np.ndarray, block_size: int,
                 num_blocks: int) -> np.ndarray:
    """Physical slot of each (sequence, logical position) pair.

    [nalar] "Urutan logis ...": the block table maps logical block b of a
    sequence to physical block ``table[b]``; [bicarait] "Blueprint Arsitektur
    2": the table maps logical block index L_i to a physical location.  The
    slot is ``physical_block * block_size + offset``.

    ``positions[j] < 0`` marks a padding token: its slot is -1.  Any other
    violation (bad sequence id, position beyond the table, an entry outside
    ``[0, num_blocks)``) is a caller error and raises.
    """
    bt = np.asarray(block_tables)
    seq_ids = np.asarray(seq_ids)
    positions = np.asarray(positions)
    if bt.ndim != 2 or seq_ids.shape != positions.shape or positions.ndim != 1:
        raise ContractError("block_tables must be 2-D; seq_ids/positions 1-D and equal length")
    num_seqs, max_blocks = bt.shape
    out = np.empty(positions.shape[0], dtype=np.int64)
    for j in range(positions.shape[0]):
        p = int(positions[j])
        if p < 0:
            out[j] = -1
            continue
        i = int(seq_ids[j])
        if not 0 <= i < num_seqs:
            raise ContractError(f"token {j}: sequence id {i} out of range")
        b = _logical_block(p, block_size)
        if b >= max_blocks:
            raise ContractError(f"token {j}: position {p} beyond the block table")
        phys = int(bt[i, b])
        if not 0 <= phys < num_blocks:
            raise ContractError(f"token {j}: table entry {phys} is not a pool block")
        out[j] = np.int64(phys) * block_size + _offset_in_block(p, block_size)
    return out


# ---------------------------------------------------------------------------
# a2: store the new tokens' K and V in their slots
# ---------------------------------------------------------------------------

def write_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
             v_new: np.ndarray, slots: np.ndarray):
    """Return copies of the pools with each new token's K/V stored in its slot.

    [gyaansetu] "Apa itu KV Cache?": K and V are computed for the new token only
    and kept for later steps.  Pools are K ``[NB][Hkv][D/x][bs][x]`` and V
    ``[NB][Hkv][bs][D]``; ``k_new`` and
    ``v_new`` are ``[T][Hkv][D]``.  The copy is of bits, so it is exact for any
    element type.  Slot -1 skips the token; a slot outside the pool or two
    tokens with the same slot raise.  K rows are stored as granules (see the
    module notes on the layout).
    """
    num_blocks, num_kv_heads, block_size, head_dim, x = pool_dims(k_pool, v_pool)
    slots = np.asarray(slots, dtype=np.int64)
    if k_new.shape != (slots.shape[0], num_kv_heads, head_dim) or v_new.shape != k_new.shape:
        raise ContractError("new K/V must be [T][Hkv][D] matching the slots")
    used = slots[slots >= 0]
    if used.size and int(used.max()) >= num_blocks * block_size:
        raise ContractError("slot beyond the pool")
    if np.unique(used).size != used.size:
        raise ContractError("two tokens write the same slot")
    if np.any(slots < -1):
        raise ContractError("slots below -1 are not defined")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for j, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), block_size)
        k_out[b, :, :, o, :] = k_new[j].reshape(num_kv_heads, head_dim // x, x)
        v_out[b, :, o, :] = v_new[j]
    return k_out, v_out


# ---------------------------------------------------------------------------
# a3: copy-on-write block copy
# ---------------------------------------------------------------------------

def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs: np.ndarray):
    """Return copies of the pools where block ``dst`` holds block ``src``.

    [nalar] "Sharing blok ...": a branch that must change a shared block gets
    its own physical storage (copy-on-write); [gininih] "Cara kerja": a new block
    is copied when a branch diverges.  A whole block is copied, every KV head,
    K and V.  Pairs must name pool blocks, destinations must be distinct and no
    destination may also be a source (otherwise the result would depend on the
    order of the copies): these raise.
    """
    pairs = np.asarray(pairs).reshape(-1, 2)
    num_blocks = pool_dims(k_pool, v_pool)[0]
    if pairs.size and (pairs.min() < 0 or pairs.max() >= num_blocks):
        raise ContractError("pair names a block outside the pool")
    src, dst = pairs[:, 0], pairs[:, 1]
    if np.unique(dst).size != dst.size:
        raise ContractError("two pairs write the same destination block")
    if np.intersect1d(src, dst).size:
        raise ContractError("a destination block is also a source")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for s, d in pairs:
        k_out[d] = k_pool[s]
        v_out[d] = v_pool[s]
    return k_out, v_out


# ---------------------------------------------------------------------------
# a4..a10: decode attention through the block table
# ---------------------------------------------------------------------------

def _kv_head(q_head: int, group: int) -> int:
    """KV head read by query head ``q_head`` (consecutive groups of ``group``)."""
    return q_head // group


def decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     block_tables: np.ndarray, context_lens: np.ndarray,
                     scale: float, dtype: str, seqs=None, heads=None) -> np.ndarray:
    """Exact softmax attention of one query token per sequence, float64.

    [nalar] "Kernel attention harus mengikuti block table": for the query, walk
    the logical context in order; translate each logical block through the
    table; then load K and V.  [nalar] introduction and [gininih] "Batasan":
    the attention equation is the ordinary one, so for each query head h

        s_t   = scale * <q_h, K_t>          t = 0 .. ctx-1
        out_h = sum_t softmax(s)_t * V_t

    q is ``[S][Hq][D]``; pools as in the module notes; the table ``[S][MB]``
    (entries past the last used block are never read).  Returns
    ``[S][Hq][D]`` float64; a sequence with ``ctx == 0`` gets zeros.

    ``seqs`` / ``heads`` (optional index lists) restrict the work to those
    sequences and query heads, for checking samples of a large batch; rows not
    computed are NaN.
    """
    num_seqs, num_q_heads, head_dim = q.shape
    num_blocks, num_kv_heads, block_size, head_dim_kv, _ = pool_dims(k_pool, v_pool)
    if head_dim_kv != head_dim:
        raise ContractError("q, K and V disagree in head_dim")
    if num_q_heads % num_kv_heads:
        raise ContractError("num_q_heads must be a multiple of num_kv_heads")
    group = num_q_heads // num_kv_heads
    bt = np.asarray(block_tables)
    ctx = np.asarray(context_lens)
    scale64 = np.float64(np.float32(scale))
    q64 = to_f64(q, dtype)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    if seqs is not None or heads is not None:
        out[:] = np.nan
    seq_list = range(num_seqs) if seqs is None else [int(i) for i in seqs]
    head_list = range(num_q_heads) if heads is None else [int(h) for h in heads]
    for i in seq_list:
        n = int(ctx[i])
        if n < 0 or n > bt.shape[1] * block_size:
            raise ContractError(f"sequence {i}: context length {n} outside the table")
        if n == 0:
            out[i, list(head_list)] = 0.0
            continue
        t = np.arange(n)
        lb = np.array([_logical_block(int(p), block_size) for p in t])
        off = np.array([_offset_in_block(int(p), block_size) for p in t])
        phys = bt[i, lb]
        if phys.min() < 0 or phys.max() >= num_blocks:
            raise ContractError(f"sequence {i}: table entry is not a pool block")
        for h in head_list:
            g = _kv_head(h, group)
            k_t = to_f64(_k_rows(k_pool, phys, g, off), dtype)  # [n][D]
            v_t = to_f64(v_pool[phys, g, off, :], dtype)        # [n][D]
            s = scale64 * (k_t @ q64[i, h])                     # [n]
            w = np.exp(s - s.max())
            out[i, h] = (w @ v_t) / w.sum()
    return out


# ---------------------------------------------------------------------------
# multi-query attention of a prompt chunk (chunked prefill)
# ---------------------------------------------------------------------------

def prefill_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                      block_tables: np.ndarray, context_lens: np.ndarray,
                      query_start: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Exact causal softmax attention of a chunk of query tokens per sequence,
    float64.

    [bicarait] "Blueprint Arsitektur 3: Chunked Prefill": a prompt is
    processed a chunk (e.g. 512 tokens) at a time, interleaved with decode
    steps; each chunk's tokens attend to everything before them through the
    same block table as the decode ([nalar] "Kernel attention harus mengikuti
    block table").  Reading (the page gives no formula): sequence i's chunk is
    the last ``L = query_start[i+1] - query_start[i]`` of its ``n =
    context_lens[i]`` tokens, already in the cache; chunk token j is logical
    position ``n - L + j`` and, as in ordinary causal self-attention, sees
    positions ``0 .. n - L + j``:

        s_t   = scale * <q_{j,h}, K_t>          t = 0 .. n - L + j
        out   = sum_t softmax(s)_t * V_t

    A token whose position is negative (a chunk longer than its context) sees
    no key and gets zeros, like an empty decode context.  q and the result are
    ``[T][Hq][D]`` with T = query_start[-1]; head h reads KV head h // G.
    """
    total, num_q_heads, head_dim = q.shape
    num_blocks, num_kv_heads, block_size, head_dim_kv, _ = pool_dims(k_pool, v_pool)
    if head_dim_kv != head_dim or num_q_heads % num_kv_heads:
        raise ContractError("q and the pools disagree")
    group = num_q_heads // num_kv_heads
    bt = np.asarray(block_tables)
    ctx = np.asarray(context_lens)
    qs = np.asarray(query_start, dtype=np.int64)
    if qs.shape != (ctx.size + 1,) or qs[0] < 0 or np.any(np.diff(qs) < 0) or qs[-1] > total:
        raise ContractError("query_start must be non-decreasing within the query rows")
    scale64 = np.float64(np.float32(scale))
    q64 = to_f64(q, dtype)
    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    for i in range(ctx.size):
        n, L = int(ctx[i]), int(qs[i + 1] - qs[i])
        if n < 0 or n > bt.shape[1] * block_size:
            raise ContractError(f"sequence {i}: context length {n} outside the table")
        if L == 0 or n == 0:
            continue
        t = np.arange(n)
        lb = np.array([_logical_block(int(p), block_size) for p in t])
        off = np.array([_offset_in_block(int(p), block_size) for p in t])
        phys = bt[i, lb]
        if phys.min() < 0 or phys.max() >= num_blocks:
            raise ContractError(f"sequence {i}: table entry is not a pool block")
        pos = n - L + np.arange(L)                   # position of each chunk token
        visible = t[None, :] <= pos[:, None]         # [L][n]: key t seen by token j
        seen = visible.any(axis=1)                   # tokens at a position >= 0
        for g in range(num_kv_heads):
            k_t = to_f64(_k_rows(k_pool, phys, g, off), dtype)   # [n][D]
            v_t = to_f64(v_pool[phys, g, off, :], dtype)         # [n][D]
            for h in range(g * group, (g + 1) * group):
                s = scale64 * (q64[qs[i]:qs[i + 1], h] @ k_t.T)  # [L][n]
                s = np.where(visible, s, -np.inf)
                top = np.where(seen, s.max(axis=1), 0.0)
                w = np.where(visible, np.exp(s - top[:, None]), 0.0)
                den = np.where(seen, w.sum(axis=1), 1.0)
                out[qs[i]:qs[i + 1], h] = (w @ v_t) / den[:, None]
    return out


# ---------------------------------------------------------------------------
# block swap between two pools (eviction to host memory and return)
# ---------------------------------------------------------------------------

def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray,
                pairs: np.ndarray):
    """Return copies of the destination pools where block ``dst`` holds block
    ``src`` of the source pools, for each (src, dst) pair.

    [gyaansetu] "How PagedAttention fixes this" (fine-grained eviction):
    fixed-size pages, not whole sequences, move between GPU and CPU memory.
    Moving a page changes where its bytes live, never the bytes.  Both pool
    pairs have the same block shape; a pair naming a block outside its pool is
    a contract error here (the GPU skips it).
    """
    if src_k.shape[1:] != dst_k.shape[1:] or src_v.shape[1:] != dst_v.shape[1:]:
        raise ContractError("the pools disagree in block shape")
    k_out, v_out = dst_k.copy(), dst_v.copy()
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if len(set(pairs[:, 1].tolist())) != len(pairs):
        raise ContractError("destinations must be distinct")
    for s, d in pairs:
        if not (0 <= s < src_k.shape[0]) or not (0 <= d < dst_k.shape[0]):
            raise ContractError("pair outside a pool")
        k_out[d] = src_k[s]
        v_out[d] = src_v[s]
    return k_out, v_out
