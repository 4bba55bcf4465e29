"""Seeded synthetic inputs shaped like the pages' serving workloads.

This module draws numbers and lays out buffers; it holds none of the method's
arithmetic (no slot formula, no attention).  Both the HIP path and the CPU
oracle consume what it returns, and each side executes the returned *plan*
with its own code:

    setup: a list of ops run once (history writes, and copy-on-write for the
           observable-CoW variant of the shared-prefix workload)
    step:  the ops of one decode step, timed by the benchmark
           ([copy,] write of the new token per sequence, decode attention)

An op is ``("write", Write)`` -- compute the slot of every (sequence, position)
pair through the named block table, then store K/V there -- or
``("copy", pairs)``.  Pools start as all-NaN bit patterns, so every slot and
block the plan never writes stays poisoned; table padding is -1.

Random draws: ``numpy.random.default_rng(SeedSequence([188, config_id]))``,
drawn in the fixed order context lengths -> block permutation -> Q ->
new-token K -> new-token V; the (large) history K and V come from child
seeds of ``SeedSequence([188, config_id, stream, 0 or 1])``, one per
32768-token chunk.  float32 draws are rounded to
bfloat16 by round-to-nearest-even once, here, so both sides see the same bits.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"

BF16_NAN = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)
SEED_ROOT = 188


# ---------------------------------------------------------------------------
# element encodings
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def draw_normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws in the element encoding of ``dtype``."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    return x


def nan_pool(shape, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return np.full(shape, BF16_NAN, dtype=np.uint16)
    return np.full(shape, F32_NAN_BITS, dtype=np.uint32).view(np.float32)


def elem_bytes(dtype: str) -> int:
    return 2 if dtype == BF16 else 4


def granule(dtype: str) -> int:
    """Elements per 16-byte granule of the K pool layout."""
    return 16 // elem_bytes(dtype)


# ---------------------------------------------------------------------------
# plan containers
# ---------------------------------------------------------------------------

@dataclass
class Write:
    """Tokens to store: token j is logical position ``positions[j]`` of
    sequence ``seq_ids[j]``, addressed through block table ``table``."""
    table: str
    seq_ids: np.ndarray        # int32 [T]
    positions: np.ndarray      # int32 [T]
    k: np.ndarray              # [T][Hkv][D] element bits
    v: np.ndarray


@dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float                       # a float32 value
    q: np.ndarray                      # [S][Hq][D]
    tables: dict                       # name -> int32 [S][MB]; "final" is decoded
    context_lens: np.ndarray           # int32 [S], after the step's write
    setup: list = field(default_factory=list)
    step: list = field(default_factory=list)
    partition_size: int = 0            # 0: the library picks
    seed: tuple = ()
    notes: dict = field(default_factory=dict)
    # multi-query (chunked prefill) workloads: sequence i owns query rows
    # query_start[i] .. query_start[i+1]-1 of q ([T][Hq][D])
    query_start: np.ndarray = None

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def empty_pools(self):
        """NaN-filled K pool [NB][Hkv][D/x][bs][x] (x = 16-byte granule) and
        V pool [NB][Hkv][bs][D]."""
        x = granule(self.dtype)
        kshape = (self.num_blocks, self.num_kv_heads, self.head_dim // x, self.block_size, x)
        vshape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        return nan_pool(kshape, self.dtype), nan_pool(vshape, self.dtype)

    # --- accounting (algorithmic bytes of one decode step) -----------------
    def kv_bytes_read(self) -> int:
        """K and V bytes the decode must read: every context token, once per KV
        head (nothing is pruned or compressed)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads \
            * self.head_dim * 2 * elem_bytes(self.dtype)

    def decode_bytes(self) -> int:
        """KV + query + fp32 output + block-table entries + context lengths."""
        e = elem_bytes(self.dtype)
        blocks = int(sum(math.ceil(int(c) / self.block_size) for c in self.context_lens))
        return (self.kv_bytes_read()
                + self.num_seqs * self.num_q_heads * self.head_dim * (e + 4)
                + 4 * blocks + 4 * self.num_seqs)

    # --- accounting of a chunked-prefill step ------------------------------
    @property
    def max_query_len(self) -> int:
        return int(np.diff(self.query_start).max()) if self.num_seqs else 0

    def prefill_flops(self) -> int:
        """Multiply-adds x 2 of QK^T and PV over the keys each chunk token
        sees (positions 0 .. its own): the causal work, nothing masked."""
        qs, ctx = self.query_start.astype(np.int64), self.context_lens.astype(np.int64)
        L = np.diff(qs)
        # sum over j < L of (n - L + j + 1) keys
        keys = int((L * (ctx - L) + L * (L + 1) // 2).sum())
        return 4 * keys * self.num_q_heads * self.head_dim

    def prefill_bytes(self) -> int:
        """Each context token's K and V once per KV head, Q in, fp32 out."""
        e = elem_bytes(self.dtype)
        t = int(self.query_start[-1])
        return (self.kv_bytes_read() + t * self.num_q_heads * self.head_dim * (e + 4))

    def shared_decode_bytes(self, group_start, shared_len) -> int:
        """decode_bytes() for a call that reads each group's shared tokens
        once: group g's first min(members, 16 // G) sequences share the largest
        multiple of max(16, block_size) tokens <= shared_len[g] and < each
        one's context (the tokens the shared-prefix call reads once)."""
        unit = max(16, self.block_size)
        cap = 16 // self.group
        per_token = self.num_kv_heads * self.head_dim * 2 * elem_bytes(self.dtype)
        saved = 0
        for g in range(len(shared_len)):
            a, b = int(group_start[g]), int(group_start[g + 1])
            cnt = min(b - a, cap)
            if cnt < 2:
                continue
            n = min(int(shared_len[g]), int(self.context_lens[a:a + cnt].min()) - 1)
            n = n - n % unit if n > 0 else 0
            saved += (cnt - 1) * n * per_token
        return self.decode_bytes() - saved

    def unique_kv_bytes(self) -> int:
        """KV bytes of distinct physical blocks referenced by the final tables."""
        bt = self.tables["final"]
        ids = set()
        for i in range(self.num_seqs):
            nb = math.ceil(int(self.context_lens[i]) / self.block_size)
            ids.update(int(x) for x in bt[i, :nb])
        return len(ids) * self.num_kv_heads * self.block_size * self.head_dim \
            * 2 * elem_bytes(self.dtype)


def _rng(config_id) -> tuple:
    seq = np.random.SeedSequence([SEED_ROOT, int(config_id)])
    return np.random.default_rng(seq), (SEED_ROOT, int(config_id))


def _blocks_for(ctx: int, block_size: int) -> int:
    """Blocks a sequence of ``ctx`` tokens occupies (allocation bookkeeping)."""
    return -(-ctx // block_size)


def _positions(lengths, starts=None):
    """Concatenated (seq_id, position) lists: sequence i gets positions
    ``starts[i] .. starts[i]+lengths[i]-1``."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if lengths.size == 0:
        return np.zeros(0, np.int32), np.zeros(0, np.int32)
    if starts is None:
        starts = np.zeros_like(lengths)
    seq_ids = np.repeat(np.arange(lengths.size, dtype=np.int32), lengths)
    first = np.repeat(np.asarray(starts, dtype=np.int64) - np.concatenate(
        [[0], np.cumsum(lengths)[:-1]]), lengths)
    pos = (np.arange(int(lengths.sum()), dtype=np.int64) + first).astype(np.int32)
    return seq_ids, pos


HISTORY_CHUNK_TOKENS = 1 << 15


def _history_kv(seed, stream_id, n_tokens, num_kv_heads, head_dim, dtype):
    """History K then V for ``n_tokens`` tokens.

    Token chunk c of K (V) is drawn from child c of
    ``SeedSequence([*seed, stream_id, 0 (K) / 1 (V)])``, so the values do not
    depend on how many threads draw them; chunks are drawn in parallel."""
    import concurrent.futures as cf
    import os
    workers = max(1, min(16, os.cpu_count() or 1))
    out = []
    for which in range(2):
        buf = np.empty((n_tokens, num_kv_heads, head_dim),
                       dtype=np.uint16 if dtype == BF16 else np.float32)
        n_chunks = -(-n_tokens // HISTORY_CHUNK_TOKENS)
        children = np.random.SeedSequence([*seed, stream_id, which]).spawn(n_chunks)

        def fill(c, buf=buf, children=children):
            s = c * HISTORY_CHUNK_TOKENS
            e = min(n_tokens, s + HISTORY_CHUNK_TOKENS)
            buf[s:e] = draw_normal(np.random.default_rng(children[c]),
                                   (e - s, num_kv_heads, head_dim), dtype)

        if n_chunks:
            with cf.ThreadPoolExecutor(max_workers=min(workers, n_chunks)) as ex:
                list(ex.map(fill, range(n_chunks)))
        out.append(buf)
    return out[0], out[1]


# ---------------------------------------------------------------------------
# generic decode workload (configs 1, 2, 3, 5 and custom test shapes)
# ---------------------------------------------------------------------------

def decode_workload(name, dtype, ctx_lens, num_q_heads, num_kv_heads, head_dim,
                    block_size, *, rng, seed=(), pool_slack=1.1, num_blocks=None,
                    max_blocks_per_seq=None, partition_size=0, scale=None,
                    table_prefix_only=False, shuffle=True):
    """One new token per sequence at position ``ctx-1``; history ``0..ctx-2``
    is written in setup.  Physical blocks come from a seeded permutation of the
    pool (``shuffle=False``: the identity, i.e. every sequence's blocks
    contiguous), taken in (sequence, logical block) order.  ``ctx == 0``
    sequences get no token and no block."""
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    S = ctx.size
    if not seed:
        seed = tuple(int(x) for x in rng.integers(0, 2**31 - 1, size=2))
    need_each = np.array([_blocks_for(int(c), block_size) for c in ctx], dtype=np.int64)
    need = int(need_each.sum())
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_slack * need))
    if num_blocks < need:
        raise ValueError("pool smaller than the blocks needed")
    mb = max_blocks_per_seq or (max(1, int(need_each.max())) if S else 1)
    perm = (rng.permutation(num_blocks) if shuffle else np.arange(num_blocks)).astype(np.int32)
    bt = np.full((S, mb), -1, dtype=np.int32)
    cursor = 0
    for i in range(S):
        n = int(need_each[i])
        bt[i, :n] = perm[cursor:cursor + n]
        cursor += n
    q = draw_normal(rng, (S, num_q_heads, head_dim), dtype)
    hist_len = np.maximum(ctx.astype(np.int64) - 1, 0)
    hk, hv = _history_kv(seed, 1, int(hist_len.sum()), num_kv_heads, head_dim, dtype)
    hs, hp = _positions(hist_len)
    has_new = ctx > 0
    new_seq = np.nonzero(has_new)[0].astype(np.int32)
    new_pos = (ctx[has_new] - 1).astype(np.int32)
    nk = draw_normal(rng, (new_seq.size, num_kv_heads, head_dim), dtype)
    nv = draw_normal(rng, (new_seq.size, num_kv_heads, head_dim), dtype)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    wl = Workload(name=name, dtype=dtype, num_seqs=S, num_q_heads=num_q_heads,
                  num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                  num_blocks=num_blocks, max_blocks_per_seq=mb, scale=scale, q=q,
                  tables={"final": bt}, context_lens=ctx,
                  partition_size=partition_size, seed=seed)
    wl.setup.append(("write", Write("final", hs, hp, hk, hv)))
    wl.step.append(("write", Write("final", new_seq, new_pos, nk, nv)))
    wl.step.append(("decode", "final"))
    return wl


# ---------------------------------------------------------------------------
# chunked prefill: a chunk of query tokens per sequence
# ---------------------------------------------------------------------------

def prefill_workload(name, dtype, prefix_lens, chunk_lens, num_q_heads, num_kv_heads, head_dim,
                     block_size, *, rng, seed=(), pool_slack=1.1, shuffle=True):
    """Sequence i has ``prefix_lens[i]`` tokens in the cache (written in
    setup) and a chunk of ``chunk_lens[i]`` new prompt tokens at positions
    prefix .. prefix+chunk-1: the step writes their K/V and runs the
    multi-query attention of the chunk (context = prefix + chunk).  Blocks
    are drawn as in decode_workload.  Draw order: block permutation -> Q ->
    chunk K -> chunk V; the prefix K/V come from _history_kv."""
    pre = np.asarray(prefix_lens, dtype=np.int32)
    L = np.asarray(chunk_lens, dtype=np.int32)
    ctx = (pre + L).astype(np.int32)
    S = ctx.size
    if not seed:
        seed = tuple(int(x) for x in rng.integers(0, 2**31 - 1, size=2))
    need_each = np.array([_blocks_for(int(c), block_size) for c in ctx], dtype=np.int64)
    need = int(need_each.sum())
    num_blocks = max(1, math.ceil(pool_slack * need))
    mb = max(1, int(need_each.max())) if S else 1
    perm = (rng.permutation(num_blocks) if shuffle else np.arange(num_blocks)).astype(np.int32)
    bt = np.full((S, mb), -1, dtype=np.int32)
    cursor = 0
    for i in range(S):
        n = int(need_each[i])
        bt[i, :n] = perm[cursor:cursor + n]
        cursor += n
    qs = np.concatenate([[0], np.cumsum(L, dtype=np.int64)]).astype(np.int32)
    q = draw_normal(rng, (int(qs[-1]), num_q_heads, head_dim), dtype)
    hk, hv = _history_kv(seed, 1, int(pre.astype(np.int64).sum()), num_kv_heads, head_dim, dtype)
    hs, hp = _positions(pre)
    cs, cp = _positions(L, starts=pre)
    ck = draw_normal(rng, (cs.size, num_kv_heads, head_dim), dtype)
    cv = draw_normal(rng, (cs.size, num_kv_heads, head_dim), dtype)
    wl = Workload(name=name, dtype=dtype, num_seqs=S, num_q_heads=num_q_heads,
                  num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                  num_blocks=num_blocks, max_blocks_per_seq=mb,
                  scale=float(np.float32(1.0 / math.sqrt(head_dim))), q=q,
                  tables={"final": bt}, context_lens=ctx, seed=seed, query_start=qs)
    wl.setup.append(("write", Write("final", hs, hp, hk, hv)))
    wl.step.append(("write", Write("final", cs, cp, ck, cv)))
    wl.step.append(("prefill", "final"))
    return wl


PREFILL_NAME = "chunked prefill Llama-3-8B-shape 16 seqs x 512-token chunks, prefix U[0,3584]"


def make_prefill(small: bool = False, *, block_size: int = 16) -> Workload:
    """The chunked-prefill workload: 512-token prompt chunks ([bicarait]
    "Blueprint Arsitektur 3"), Llama-3-8B attention shape (32 query heads,
    8 KV heads, head_dim 128), bf16, 16-token blocks.  16 sequences with a
    prefix already cached (uniform in [0, 3584], so contexts reach 4096);
    12 chunks are full 512-token chunks and 4 are a prompt's last, shorter
    chunk (uniform in [1, 511]).  ``small``: 4 sequences, prefixes in
    [0, 200], chunks of up to 70 tokens (several tiles, ragged tails)."""
    rng, seed = _rng(600 if small else 60)
    if small:
        pre = rng.integers(0, 200, size=4, endpoint=True)
        chunk = np.array([70, 33, 1, int(rng.integers(2, 70))])
        name = PREFILL_NAME + " [small]"
    else:
        pre = rng.integers(0, 3584, size=16, endpoint=True)
        chunk = np.full(16, 512)
        chunk[12:] = rng.integers(1, 511, size=4, endpoint=True)
        name = PREFILL_NAME
    return prefill_workload(name, BF16, pre, chunk, 32, 8, 128, block_size, rng=rng, seed=seed)


# ---------------------------------------------------------------------------
# shared-prefix / parallel-sampling workload (config 4)
# ---------------------------------------------------------------------------

def shared_prefix_workload(name, *, rng, seed=(), groups=32, samples=8, prefix=2048,
                           tail_lo=64, tail_hi=512, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16, dtype=BF16, pool_slack=1.1,
                           cow_in_step=True):
    """``groups`` prompts x ``samples`` samples.  Each group's prefix is written
    once, through sample 0's table, into blocks every sample's table shares.
    Copy-on-write gives every sample a private copy of the group's last prefix
    block (logical block ``(prefix-1)//bs``), remapped in the "final" table.
    Tails ``U[tail_lo, tail_hi]`` tokens are private.  ``ctx = prefix + tail``.

    With ``cow_in_step`` the copy is part of every timed step (it is then
    idempotent, which needs the prefix to end on a block boundary so that no
    tail token lands in the copied block).  Otherwise the copy runs once in
    setup, before the tails are written; with a prefix that ends inside a block
    the first tail tokens then land in the private copy and the copy-on-write
    is observable."""
    S = groups * samples
    if not seed:
        seed = tuple(int(x) for x in rng.integers(0, 2**31 - 1, size=2))
    tails = rng.integers(tail_lo, tail_hi, size=S, endpoint=True).astype(np.int64)
    ctx = (prefix + tails).astype(np.int32)
    n_prefix_blocks = _blocks_for(prefix, block_size)
    last_shared = n_prefix_blocks - 1
    if cow_in_step and prefix % block_size:
        raise ValueError("a copy in every step needs a prefix on a block boundary")
    total_blocks = np.array([_blocks_for(int(c), block_size) for c in ctx])
    tail_blocks = total_blocks - n_prefix_blocks
    unique_need = groups * n_prefix_blocks + S + int(tail_blocks.sum())
    num_blocks = math.ceil(pool_slack * unique_need)
    mb = int(total_blocks.max())
    perm = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0

    def take(n):
        nonlocal cursor
        out = perm[cursor:cursor + n]
        cursor += n
        return out

    pre = np.full((S, mb), -1, dtype=np.int32)
    fin = np.full((S, mb), -1, dtype=np.int32)
    pairs = np.empty((S, 2), dtype=np.int32)
    for a in range(groups):
        shared = take(n_prefix_blocks)
        for s in range(samples):
            i = a * samples + s
            pre[i, :n_prefix_blocks] = shared
            fin[i, :n_prefix_blocks] = shared
            private = take(1)[0]
            pairs[i] = (shared[last_shared], private)
            fin[i, last_shared] = private
            nt = int(tail_blocks[i])
            fin[i, n_prefix_blocks:n_prefix_blocks + nt] = take(nt)
            pre[i, n_prefix_blocks:n_prefix_blocks + nt] = fin[i, n_prefix_blocks:n_prefix_blocks + nt]
    q = draw_normal(rng, (S, num_q_heads, head_dim), dtype)
    pk, pv = _history_kv(seed, 1, groups * prefix, num_kv_heads, head_dim, dtype)
    tail_hist = tails - 1                       # the last token is the step's
    tk, tv = _history_kv(seed, 2, int(tail_hist.sum()), num_kv_heads, head_dim, dtype)
    nk = draw_normal(rng, (S, num_kv_heads, head_dim), dtype)
    nv = draw_normal(rng, (S, num_kv_heads, head_dim), dtype)
    ps, pp = _positions(np.full(groups, prefix))
    ps = (ps * samples).astype(np.int32)          # sample 0 of each group
    ts, tp = _positions(tail_hist, starts=np.full(S, prefix))
    scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    wl = Workload(name=name, dtype=dtype, num_seqs=S, num_q_heads=num_q_heads,
                  num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                  num_blocks=num_blocks, max_blocks_per_seq=mb, scale=scale, q=q,
                  tables={"pre": pre, "final": fin}, context_lens=ctx, seed=seed)
    wl.setup.append(("write", Write("pre", ps, pp, pk, pv)))
    if not cow_in_step:
        wl.setup.append(("copy", pairs))
    wl.setup.append(("write", Write("final", ts, tp, tk, tv)))
    if cow_in_step:
        wl.step.append(("copy", pairs))
    wl.step.append(("write", Write("final", np.arange(S, dtype=np.int32),
                                   (ctx - 1).astype(np.int32), nk, nv)))
    wl.step.append(("decode", "final"))
    wl.notes.update(groups=groups, samples=samples, prefix=prefix,
                    prefix_blocks_shared=groups * n_prefix_blocks,
                    cow_pairs=S)
    return wl


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-fp32: S=4 ctx{5,16,17,40} Hq=Hkv=4 D=64 bs=16 NB=32",
    2: "llama3-8b-decode: S=64 Hq=32 Hkv=8 D=128 bs=16 ctx~U[128,4096] bf16",
    3: "llama3.1-70b-decode: S=256 Hq=64 Hkv=8 D=128 bs=16 ctx~lognormal(1024,0.8)[16,8192] bf16",
    4: "shared-prefix: 32x8 samples prefix=2048 tails~U[64,512] Hq=32 Hkv=8 D=128 bs=16 bf16 +CoW",
    5: "long-context: S=4 ctx=131072 Hq=64 Hkv=8 D=128 bs=32 NB=16384 part=512 bf16",
}


def make(config_id: int, *, small: bool = False) -> Workload:
    """The workload of one of the five configurations.

    ``small=True`` keeps every per-token shape (heads, head_dim, block_size,
    dtype) and the length distribution's form but shrinks the batch and the
    lengths so the oracle finishes in seconds; it still spans many 16-token
    tiles, several split-K partitions and ragged tails."""
    rng, seed = _rng(config_id if not small else 100 + config_id)
    if config_id == 1:
        ctx = np.array([5, 16, 17, 40], dtype=np.int32)
        return decode_workload(CONFIG_NAMES[1], F32, ctx, 4, 4, 64, 16, rng=rng,
                               seed=seed, num_blocks=32, max_blocks_per_seq=3)
    if config_id == 2:
        S, lo, hi = (64, 128, 4096) if not small else (6, 1, 700)
        ctx = rng.integers(lo, hi, size=S, endpoint=True).astype(np.int32)
        return decode_workload(CONFIG_NAMES[2] + (" [small]" if small else ""), BF16, ctx,
                               32, 8, 128, 16, rng=rng, seed=seed,
                               max_blocks_per_seq=_blocks_for(hi, 16))
    if config_id == 3:
        S, med, lo, hi = (256, 1024, 16, 8192) if not small else (12, 96, 1, 900)
        raw = rng.lognormal(mean=math.log(med), sigma=0.8, size=S)
        ctx = np.clip(np.rint(raw), lo, hi).astype(np.int32)
        return decode_workload(CONFIG_NAMES[3] + (" [small]" if small else ""), BF16, ctx,
                               64, 8, 128, 16, rng=rng, seed=seed,
                               max_blocks_per_seq=_blocks_for(hi, 16))
    if config_id == 4:
        if not small:
            return shared_prefix_workload(CONFIG_NAMES[4], rng=rng, seed=seed)
        return shared_prefix_workload(CONFIG_NAMES[4] + " [small]", rng=rng, seed=seed,
                                      groups=2, samples=4, prefix=96, tail_lo=5,
                                      tail_hi=60)
    if config_id == 5:
        S, n, nb = (4, 131072, 16384) if not small else (2, 2080, 130)
        ctx = np.full(S, n, dtype=np.int32)
        return decode_workload(CONFIG_NAMES[5] + (" [small]" if small else ""), BF16, ctx,
                               64, 8, 128, 32, rng=rng, seed=seed, num_blocks=nb,
                               partition_size=512)
    raise ValueError(f"no configuration {config_id}")


def make_cow_observable(small: bool = True) -> Workload:
    """Shared-prefix variant whose prefix ends inside a block, with the copy in
    setup, so the first tail tokens of every sample land in its private copy."""
    rng, seed = _rng(404 if small else 44)
    if small:
        return shared_prefix_workload("shared-prefix CoW-observable [small]", rng=rng,
                                      seed=seed, groups=2, samples=4, prefix=88,
                                      tail_lo=3, tail_hi=40, cow_in_step=False)
    return shared_prefix_workload("shared-prefix CoW-observable prefix=2040", rng=rng,
                                  seed=seed, prefix=2040, cow_in_step=False)


# ---------------------------------------------------------------------------
# inputs whose attention scores climb along the context
# ---------------------------------------------------------------------------

def bits_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Element bits of ``dtype`` (bf16 as uint16) as float32 values (exact)."""
    if dtype == BF16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(np.float32)


def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in the element encoding of ``dtype`` (bf16: rounded to
    nearest, ties to even)."""
    return f32_to_bf16_bits(x) if dtype == BF16 else x.astype(np.float32)


def climbing_scores(wl: Workload, *, slope: float = 0.0, spike_at=(), spike_gain: float = 8.0,
                    name: str = None) -> Workload:
    """A copy of ``wl`` whose scores rise with the key position.

    Every query element is made non-negative (|q|) and the key row stored at
    logical position p becomes ``|k| * g + c * p`` (rounded once to the
    element type), with g = ``spike_gain`` at the positions in ``spike_at``
    and 1 elsewhere.  c is chosen so that the expected score, in log2 units
    (score * scale / ln 2), grows by ``slope`` per position: with
    E|q_d| = sqrt(2/pi), c = slope / (scale * log2(e) * sqrt(2/pi) * D).
    Such inputs move any softmax reference point again and again along the
    context, and a spiked key outweighs every other by many powers of two.
    Placement, V rows, tables and lengths are unchanged."""
    import copy
    w2 = copy.copy(wl)
    w2.q = f32_to_bits(np.abs(bits_to_f32(wl.q, wl.dtype)), wl.dtype)
    c = slope / (wl.scale * math.log2(math.e) * math.sqrt(2.0 / math.pi) * wl.head_dim)
    spikes = np.asarray(sorted(spike_at), dtype=np.int64)

    def steer(ops):
        out = []
        for kind, x in ops:
            if kind == "write":
                p = x.positions.astype(np.float32)[:, None, None]
                g = np.where(np.isin(x.positions, spikes), np.float32(spike_gain),
                             np.float32(1.0))[:, None, None]
                k = np.abs(bits_to_f32(x.k, wl.dtype)) * g + np.float32(c) * p
                x = Write(x.table, x.seq_ids, x.positions, f32_to_bits(k, wl.dtype), x.v)
            out.append((kind, x))
        return out

    w2.setup, w2.step = steer(wl.setup), steer(wl.step)
    w2.tables = dict(wl.tables)
    w2.notes = dict(wl.notes)
    w2.name = name or f"{wl.name} climbing scores slope={slope:g} spikes={len(spikes)}"
    return w2
