"""Pins for the CPU oracle: checks against facts that do not come from it.

Each ``pin_*`` function takes an oracle module (the real one, or a copy with a
planted mistake) and raises AssertionError (or any exception) when the oracle
disagrees with:

* the block tables the pages print (worked examples, ``tests/golden``);
* pure-Python brute-force attention on the logical (unpaged) arrays, with its
  own bf16 decoding (``struct``) and its own pool construction;
* torch's CPU scaled_dot_product_attention in float64 (library special case);
* closed forms (one token, equal keys, constant values, two tokens, a very
  large scale);
* the sharing and copy-on-write invariants.

The pool construction below restates the layout reading independently of the
oracle's own code: token p of a sequence lives in block ``table[p // bs]`` at
offset ``o = p % bs``; V element d of it is ``V[blk][h][o][d]``, K element d is
``K[blk][h][d // x][o][d % x]`` (granules of x elements; the GPU library uses
16-byte granules, the oracle accepts any x that divides D).
"""

from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# independent helpers
# ---------------------------------------------------------------------------

def bf16_bits_to_float(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def f32_to_float(x) -> float:
    return float(np.float32(x))


def as_float(bits, dtype) -> float:
    return bf16_bits_to_float(bits) if dtype == "bf16" else f32_to_float(bits)


def random_values(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)   # truncation is fine here
    return x


def nan_like_pool(shape, dtype):
    if dtype == "bf16":
        return np.full(shape, 0x7FC0, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


def k_pool_shape(nb, hkv, bs, d, x):
    return (nb, hkv, d // x, bs, x)


def build_pool(k_logical, v_logical, tables, num_blocks, block_size, dtype, x=1):
    """Scatter per-sequence logical K/V ``[ctx][Hkv][D]`` into NaN pools by
    explicit loops over tokens, heads and dims."""
    hkv, d = k_logical[0].shape[1], k_logical[0].shape[2]
    assert d % x == 0
    kp = nan_like_pool(k_pool_shape(num_blocks, hkv, block_size, d, x), dtype)
    vp = nan_like_pool((num_blocks, hkv, block_size, d), dtype)
    for i, (ks, vs) in enumerate(zip(k_logical, v_logical)):
        for p in range(ks.shape[0]):
            blk = tables[i][p // block_size]
            off = p % block_size
            for g in range(hkv):
                for e in range(d):
                    kp[blk, g, e // x, off, e % x] = ks[p, g, e]
                    vp[blk, g, off, e] = vs[p, g, e]
    return kp, vp


def dense_attention_loops(q, k_logical, v_logical, scale, dtype):
    """Textbook softmax attention with Python floats and math.exp."""
    s_n, hq, d = q.shape
    out = np.zeros((s_n, hq, d))
    sc = float(np.float32(scale))
    for i in range(s_n):
        ks, vs = k_logical[i], v_logical[i]
        n = ks.shape[0]
        if n == 0:
            continue
        hkv = ks.shape[1]
        grp = hq // hkv
        for h in range(hq):
            g = h // grp
            qh = [as_float(q[i, h, e], dtype) for e in range(d)]
            scores = []
            for t in range(n):
                kt = [as_float(ks[t, g, e], dtype) for e in range(d)]
                scores.append(sc * sum(a * b for a, b in zip(qh, kt)))
            m = max(scores)
            w = [math.exp(x - m) for x in scores]
            z = sum(w)
            for e in range(d):
                out[i, h, e] = sum(w[t] * as_float(vs[t, g, e], dtype) for t in range(n)) / z
    return out


def random_case(rng, *, num_seqs, hq, hkv, d, bs, ctx_max, dtype, slack=3, ctx=None, x=1):
    """Logical K/V per sequence, a random non-sharing table over a shuffled
    pool, and Q.  Returns everything the oracle and brute force need."""
    if ctx is None:
        ctx = [int(rng.integers(0, ctx_max + 1)) for _ in range(num_seqs)]
    need = [-(-c // bs) for c in ctx]
    mb = max(1, max(need) if need else 1)
    nb = sum(need) + slack
    perm = rng.permutation(nb)
    tables = np.full((num_seqs, mb), -1, dtype=np.int32)
    cur = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[cur:cur + n]
        cur += n
    k_logical = [random_values(rng, (c, hkv, d), dtype) for c in ctx]
    v_logical = [random_values(rng, (c, hkv, d), dtype) for c in ctx]
    q = random_values(rng, (num_seqs, hq, d), dtype)
    kp, vp = build_pool(k_logical, v_logical, tables, nb, bs, dtype, x=x)
    return dict(q=q, kp=kp, vp=vp, tables=tables, ctx=np.array(ctx, dtype=np.int32),
                k_logical=k_logical, v_logical=v_logical, nb=nb, bs=bs, dtype=dtype, x=x)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_value_decoding(O):
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x8000, 0x7F7F], dtype=np.uint16)
    want = [bf16_bits_to_float(b) for b in bits]
    got = O.to_f64(bits, "bf16")
    assert want[0] == 1.0 and want[1] == -2.0 and want[2] == 1.0078125
    assert np.array_equal(got, np.array(want)), (got, want)
    f = np.array([1.5, -0.1, 3.4028235e38, 1e-45], dtype=np.float32)
    assert np.array_equal(O.to_f64(f, "f32"), np.array([float(x) for x in f]))


def pin_worked_tables(O):
    g = load_golden("worked_block_tables.json")
    cases = [(g["nalar_mapping_diagram"], 16), (g["nalar_mapping_diagram"], 32),
             (g["bicarait_tldr_diagram"], g["bicarait_tldr_diagram"]["block_size"])]
    for entry, bs in cases:
        phys = entry["physical_blocks"]
        table = np.array([phys], dtype=np.int32)
        n = len(phys) * bs
        pos = np.arange(n, dtype=np.int32)
        slots = O.slot_mapping(table, np.zeros(n, np.int32), pos, bs, max(phys) + 1)
        for b, pb in zip(entry["logical_blocks"], phys):
            blk = slots[b * bs:(b + 1) * bs]
            # every token of logical block b lies in physical block table[b] ...
            assert np.all(blk // bs == pb), (b, pb, blk)
            # ... in logical order, one slot per token
            assert np.array_equal(blk % bs, np.arange(bs)), blk
    # A few explicit values (derived from the printed tables with bs = 16).
    t = np.array([[17, 4, 29, 8]], dtype=np.int32)
    pos = np.array([0, 15, 16, 31, 40, 63], dtype=np.int32)
    got = O.slot_mapping(t, np.zeros(6, np.int32), pos, 16, 30)
    assert list(got) == [272, 287, 64, 79, 472, 143], list(got)
    t = np.array([[41, 8, 93]], dtype=np.int32)
    pos = np.array([0, 17, 47], dtype=np.int32)
    assert list(O.slot_mapping(t, np.zeros(3, np.int32), pos, 16, 94)) == [656, 129, 1503]


def pin_slot_bijection(O):
    rng = np.random.default_rng(7)
    for bs in (1, 3, 8, 16):
        c = random_case(rng, num_seqs=4, hq=1, hkv=1, d=1, bs=bs, ctx_max=50, dtype="f32")
        seq_ids = np.concatenate([np.full(n, i, np.int32) for i, n in enumerate(c["ctx"])])
        pos = np.concatenate([np.arange(n, dtype=np.int32) for n in c["ctx"]])
        slots = O.slot_mapping(c["tables"], seq_ids, pos, bs, c["nb"])
        assert np.unique(slots).size == slots.size
        assigned = set()
        for i, n in enumerate(c["ctx"]):
            for b in range(-(-int(n) // bs)):
                assigned.update(range(int(c["tables"][i, b]) * bs, int(c["tables"][i, b]) * bs + bs))
        assert set(int(s) for s in slots) <= assigned
        # with pad tokens mixed in, pads map to -1 and the rest is unchanged
        pos2 = pos.copy()
        pos2[::5] = -1
        s2 = O.slot_mapping(c["tables"], seq_ids, pos2, bs, c["nb"])
        assert np.all(s2[::5] == -1)
        keep = np.ones(pos.size, bool)
        keep[::5] = False
        assert np.array_equal(s2[keep], slots[keep])


def pin_write_bruteforce(O):
    rng = np.random.default_rng(11)
    for dtype, d, x in (("f32", 5, 1), ("bf16", 6, 3), ("bf16", 8, 8), ("f32", 4, 2)):
        nb, hkv, bs, t = 6, 3, 4, 9
        kp = random_values(rng, k_pool_shape(nb, hkv, bs, d, x), dtype)
        vp = random_values(rng, (nb, hkv, bs, d), dtype)
        kn = random_values(rng, (t, hkv, d), dtype)
        vn = random_values(rng, (t, hkv, d), dtype)
        slots = rng.permutation(nb * bs)[:t].astype(np.int64)
        slots[3] = -1
        k2, v2 = O.write_kv(kp, vp, kn, vn, slots)
        # independent element-by-element expectation
        ek, ev = kp.copy(), vp.copy()
        for j in range(t):
            if slots[j] < 0:
                continue
            blk, off = int(slots[j]) // bs, int(slots[j]) % bs
            for g in range(hkv):
                for e in range(d):
                    ek[blk, g, e // x, off, e % x] = kn[j, g, e]
                    ev[blk, g, off, e] = vn[j, g, e]
        assert k2.tobytes() == ek.tobytes() and v2.tobytes() == ev.tobytes()
        # inputs are not modified in place
        assert not np.shares_memory(k2, kp)


def pin_write_roundtrip(O):
    """Writing a sequence's tokens through its table, then gathering them back
    through the same table, returns the written vectors bit for bit; every
    other slot keeps its sentinel."""
    rng = np.random.default_rng(12)
    c = random_case(rng, num_seqs=3, hq=2, hkv=2, d=4, bs=4, ctx_max=13, dtype="bf16",
                    ctx=[13, 0, 6], x=2)
    kp, vp = nan_like_pool(c["kp"].shape, "bf16"), nan_like_pool(c["vp"].shape, "bf16")
    seq_ids = np.concatenate([np.full(n, i, np.int32) for i, n in enumerate(c["ctx"])])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in c["ctx"]])
    kn = np.concatenate([x for x in c["k_logical"]])
    vn = np.concatenate([x for x in c["v_logical"]])
    slots = O.slot_mapping(c["tables"], seq_ids, pos, c["bs"], c["nb"])
    k2, v2 = O.write_kv(kp, vp, kn, vn, slots)
    assert k2.tobytes() == c["kp"].tobytes() and v2.tobytes() == c["vp"].tobytes()


def pin_copy(O):
    rng = np.random.default_rng(13)
    nb, hkv, bs, d = 8, 2, 4, 3
    kp = random_values(rng, k_pool_shape(nb, hkv, bs, d, 1), "bf16")
    vp = random_values(rng, (nb, hkv, bs, d), "bf16")
    pairs = np.array([[1, 5], [1, 6], [3, 0]], dtype=np.int32)
    k2, v2 = O.copy_blocks(kp, vp, pairs)
    for s, dd in pairs:
        assert k2[dd].tobytes() == kp[s].tobytes() and v2[dd].tobytes() == vp[s].tobytes()
    for b in (1, 2, 3, 4, 7):
        assert k2[b].tobytes() == kp[b].tobytes() and v2[b].tobytes() == vp[b].tobytes()
    for bad in ([[1, 1]], [[1, 2], [2, 3]], [[0, 9]], [[1, 4], [2, 4]]):
        try:
            O.copy_blocks(kp, vp, np.array(bad, dtype=np.int32))
        except ValueError:
            continue
        raise AssertionError(f"copy accepted a contract violation {bad}")


DENSE_CASES = [
    # (num_seqs, hq, hkv, d, bs, ctx_max, dtype, seed, x)
    (3, 4, 2, 4, 4, 30, "f32", 1, 2),
    (2, 4, 1, 3, 3, 20, "bf16", 2, 1),
    (2, 2, 2, 5, 1, 9, "f32", 3, 5),
    (3, 6, 3, 2, 8, 40, "bf16", 4, 1),
    (1, 8, 2, 4, 16, 37, "bf16", 5, 4),
    (4, 1, 1, 6, 2, 11, "f32", 6, 3),
    (2, 4, 2, 8, 4, 19, "bf16", 7, 2),
]


def pin_attention_dense(O, cases=DENSE_CASES, tol=1e-12):
    for (s_n, hq, hkv, d, bs, cmax, dtype, seed, x) in cases:
        rng = np.random.default_rng(100 + seed)
        c = random_case(rng, num_seqs=s_n, hq=hq, hkv=hkv, d=d, bs=bs, ctx_max=cmax, dtype=dtype,
                        x=x)
        scale = float(np.float32(1 / math.sqrt(d)))
        got = O.decode_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], scale, dtype)
        want = dense_attention_loops(c["q"], c["k_logical"], c["v_logical"], scale, dtype)
        err = np.max(np.abs(got - want)) if got.size else 0.0
        assert err <= tol, (s_n, hq, hkv, d, bs, dtype, x, err)


def pin_attention_sdpa(O):
    import torch
    rng = np.random.default_rng(21)
    for (hq, hkv, d, n, dtype, x) in ((8, 2, 16, 37, "bf16", 8), (4, 4, 8, 5, "f32", 4),
                                      (6, 1, 4, 64, "f32", 1)):
        bs = n  # identity table, one block holds the whole context
        c = random_case(rng, num_seqs=1, hq=hq, hkv=hkv, d=d, bs=bs, ctx_max=n, dtype=dtype,
                        ctx=[n], slack=0, x=x)
        scale = float(np.float32(0.37))
        got = O.decode_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], scale, dtype)
        conv = (lambda a: np.vectorize(bf16_bits_to_float)(a)) if dtype == "bf16" else (lambda a: a.astype(np.float64))
        q = torch.tensor(conv(c["q"]), dtype=torch.float64).reshape(1, hq, 1, d)
        k = torch.tensor(conv(c["k_logical"][0]), dtype=torch.float64).permute(1, 0, 2)
        v = torch.tensor(conv(c["v_logical"][0]), dtype=torch.float64).permute(1, 0, 2)
        k = k.repeat_interleave(hq // hkv, dim=0).unsqueeze(0).contiguous()
        v = v.repeat_interleave(hq // hkv, dim=0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
        ref = ref.reshape(1, hq, d).numpy()
        assert np.max(np.abs(got - ref)) <= 1e-12, np.max(np.abs(got - ref))


def _single(O, q, ks, vs, scale, bs=4, dtype="f32"):
    """Run the oracle on one sequence given logical [n][1][D] arrays."""
    n = ks.shape[0]
    nb = -(-n // bs) + 2
    rng = np.random.default_rng(n)
    perm = rng.permutation(nb)
    table = np.full((1, max(1, -(-n // bs))), -1, np.int32)
    table[0, :-(-n // bs)] = perm[:-(-n // bs)]
    kp, vp = build_pool([ks], [vs], table, nb, bs, dtype, x=2 if ks.shape[2] % 2 == 0 else 1)
    return O.decode_attention(q, kp, vp, table, np.array([n], np.int32), scale, dtype)[0, 0]


def pin_closed_forms(O):
    rng = np.random.default_rng(31)
    d = 6
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    # one token: the output is that token's V row exactly
    k1 = rng.standard_normal((1, 1, d)).astype(np.float32)
    v1 = rng.standard_normal((1, 1, d)).astype(np.float32)
    assert np.array_equal(_single(O, q, k1, v1, 0.5), v1[0, 0].astype(np.float64))
    # q = 0 (all scores equal): the mean of the V rows
    n = 11
    ks = rng.standard_normal((n, 1, d)).astype(np.float32)
    vs = rng.standard_normal((n, 1, d)).astype(np.float32)
    got = _single(O, np.zeros((1, 1, d), np.float32), ks, vs, 0.5)
    assert np.allclose(got, vs[:, 0].astype(np.float64).mean(0), rtol=0, atol=1e-14)
    # equal V rows: the output is that row whatever the scores
    c = rng.standard_normal(d).astype(np.float32)
    vc = np.broadcast_to(c, (n, 1, d)).copy()
    assert np.allclose(_single(O, q, ks, vc, 0.9), c.astype(np.float64), rtol=0, atol=1e-14)
    # two tokens: (v0 + e^D v1) / (1 + e^D), D = s1 - s0
    k2 = rng.standard_normal((2, 1, d)).astype(np.float32)
    v2 = rng.standard_normal((2, 1, d)).astype(np.float32)
    sc = float(np.float32(0.25))
    s = [sc * float(np.dot(q[0, 0].astype(np.float64), k2[t, 0].astype(np.float64))) for t in range(2)]
    dlt = s[1] - s[0]
    want = (v2[0, 0].astype(np.float64) + math.exp(dlt) * v2[1, 0].astype(np.float64)) / (1 + math.exp(dlt))
    assert np.allclose(_single(O, q, k2, v2, sc), want, rtol=0, atol=1e-14)
    # very large scale: the V row of the largest score
    n = 9
    ks = rng.standard_normal((n, 1, d)).astype(np.float32)
    vs = rng.standard_normal((n, 1, d)).astype(np.float32)
    sc_raw = ks[:, 0].astype(np.float64) @ q[0, 0].astype(np.float64)
    best = int(np.argmax(sc_raw))
    gap = np.sort(sc_raw)[-1] - np.sort(sc_raw)[-2]
    big = float(np.float32(60.0 / gap))
    assert np.allclose(_single(O, q, ks, vs, big), vs[best, 0].astype(np.float64), rtol=0, atol=1e-12)


def pin_shared_vs_private(O):
    """Invariant (b): sequences whose tables share physical prefix blocks get
    exactly the output they get with private copies of those blocks."""
    rng = np.random.default_rng(41)
    bs, hkv, hq, d, prefix, samples = 4, 2, 4, 3, 10, 3
    pk = random_values(rng, (prefix, hkv, d), "bf16")
    pv = random_values(rng, (prefix, hkv, d), "bf16")
    tails = [int(x) for x in rng.integers(1, 9, samples)]
    ks = [np.concatenate([pk, random_values(rng, (t, hkv, d), "bf16")]) for t in tails]
    vs = [np.concatenate([pv, random_values(rng, (t, hkv, d), "bf16")]) for t in tails]
    q = random_values(rng, (samples, hq, d), "bf16")
    ctx = np.array([prefix + t for t in tails], np.int32)
    nblk = [-(-int(c) // bs) for c in ctx]
    npre = prefix // bs                       # full prefix blocks that can be shared
    # private layout: every sequence owns all its blocks
    nb_priv = sum(nblk)
    perm = rng.permutation(nb_priv)
    t_priv = np.full((samples, max(nblk)), -1, np.int32)
    cur = 0
    for i, n in enumerate(nblk):
        t_priv[i, :n] = perm[cur:cur + n]
        cur += n
    kp1, vp1 = build_pool(ks, vs, t_priv, nb_priv, bs, "bf16", x=3)
    # shared layout: the full prefix blocks are stored once
    nb_sh = npre + sum(n - npre for n in nblk)
    perm = rng.permutation(nb_sh)
    shared = perm[:npre]
    t_sh = np.full((samples, max(nblk)), -1, np.int32)
    cur = npre
    for i, n in enumerate(nblk):
        t_sh[i, :npre] = shared
        t_sh[i, npre:n] = perm[cur:cur + n - npre]
        cur += n - npre
    kp2, vp2 = build_pool(ks, vs, t_sh, nb_sh, bs, "bf16", x=3)
    assert nb_sh < nb_priv
    o1 = O.decode_attention(q, kp1, vp1, t_priv, ctx, 0.5, "bf16")
    o2 = O.decode_attention(q, kp2, vp2, t_sh, ctx, 0.5, "bf16")
    assert o1.tobytes() == o2.tobytes()


def pin_cow_isolation(O):
    """Invariant (c): after sample 0 copies a shared block and then writes into
    its copy, the other sharers' outputs are bit-identical to before and
    sample 0's output changes."""
    rng = np.random.default_rng(51)
    bs, hkv, hq, d, samples, ctx0 = 4, 1, 2, 4, 3, 6      # the shared block 1 holds 2 tokens
    ks = random_values(rng, (ctx0, hkv, d), "bf16")
    vs = random_values(rng, (ctx0, hkv, d), "bf16")
    nb = 6
    table = np.full((samples, 2), -1, np.int32)
    table[:, 0], table[:, 1] = 2, 4
    kp, vp = build_pool([ks], [vs], table[:1], nb, bs, "bf16", x=2)
    q = random_values(rng, (samples, hq, d), "bf16")
    ctx = np.full(samples, ctx0, np.int32)
    before = O.decode_attention(q, kp, vp, table, ctx, 0.5, "bf16")
    k2, v2 = O.copy_blocks(kp, vp, np.array([[4, 5]], np.int32))
    t2 = table.copy()
    t2[0, 1] = 5
    mid = O.decode_attention(q, k2, v2, t2, ctx, 0.5, "bf16")
    assert mid.tobytes() == before.tobytes()        # the copy alone changes nothing
    # sample 0 now writes position 6 (offset 2 of its private block 5)
    kn = random_values(rng, (1, hkv, d), "bf16")
    vn = random_values(rng, (1, hkv, d), "bf16")
    slot = O.slot_mapping(t2, np.array([0], np.int32), np.array([6], np.int32), bs, nb)
    assert int(slot[0]) == 5 * bs + 2
    k3, v3 = O.write_kv(k2, v2, kn, vn, slot)
    ctx3 = ctx.copy()
    ctx3[0] = 7
    after = O.decode_attention(q, k3, v3, t2, ctx3, 0.5, "bf16")
    assert after[1:].tobytes() == before[1:].tobytes()
    assert not np.array_equal(after[0], before[0])
    # the shared original block 4 is untouched
    assert k3[4].tobytes() == kp[4].tobytes() and v3[4].tobytes() == vp[4].tobytes()


# ---------------------------------------------------------------------------
# multi-query attention of a prompt chunk (chunked prefill)
# ---------------------------------------------------------------------------

def prefill_case(rng, *, ctx, chunk, hq, hkv, d, bs, dtype, x=1, slack=3):
    """random_case plus, for each sequence, a chunk of ``chunk[i]`` query
    tokens (the last ones of its context) and their start offsets."""
    c = random_case(rng, num_seqs=len(ctx), hq=hq, hkv=hkv, d=d, bs=bs, ctx_max=max(ctx),
                    dtype=dtype, ctx=list(ctx), x=x, slack=slack)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    c["qs"] = qs
    c["q"] = random_values(rng, (int(qs[-1]), hq, d), dtype)
    return c


def prefill_bruteforce(c, scale):
    """Chunk token j of sequence i (position n - L + j) by the textbook loops
    over its visible prefix K[0 .. n-L+j], one query at a time."""
    qs, q = c["qs"], c["q"]
    out = np.zeros(q.shape)
    for i, n in enumerate(c["ctx"]):
        L = int(qs[i + 1] - qs[i])
        for j in range(L):
            pos = int(n) - L + j
            if pos < 0:
                continue
            row = q[qs[i] + j][None]
            out[qs[i] + j] = dense_attention_loops(
                row, [c["k_logical"][i][:pos + 1]], [c["v_logical"][i][:pos + 1]], scale,
                c["dtype"])[0]
    return out


PREFILL_CASES = [  # (ctx, chunk, hq, hkv, d, bs, dtype, x, seed)
    ([9, 5, 12], [4, 5, 3], 4, 2, 4, 4, "bf16", 2, 1),      # prefix + chunk, whole prompt
    ([7, 16], [7, 1], 2, 1, 3, 2, "f32", 1, 2),            # L = 1 is a decode
    ([3, 10], [5, 0], 6, 3, 2, 8, "f32", 2, 3),            # chunk longer than its context
]


def pin_prefill_bruteforce(O):
    """Each chunk token equals textbook attention of its own query over the
    keys up to its position ([bicarait] "Blueprint Arsitektur 3": a chunk
    sees the whole prompt before it; causal inside the chunk)."""
    for (ctx, chunk, hq, hkv, d, bs, dtype, x, seed) in PREFILL_CASES:
        c = prefill_case(np.random.default_rng(300 + seed), ctx=ctx, chunk=chunk, hq=hq,
                         hkv=hkv, d=d, bs=bs, dtype=dtype, x=x)
        scale = float(np.float32(0.61))
        got = O.prefill_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], c["qs"],
                                  scale, dtype)
        want = prefill_bruteforce(c, scale)
        assert np.max(np.abs(got - want), initial=0.0) <= 1e-12, (ctx, chunk)


def pin_prefill_sdpa(O):
    """A chunk's rows are the last L rows of ordinary causal self-attention
    over the whole context (torch's float64 scaled_dot_product_attention with
    is_causal, grouped heads expanded)."""
    import torch
    rng = np.random.default_rng(41)
    for (n, L, hq, hkv, d, bs, x) in ((37, 37, 8, 2, 16, 8, 8), (50, 13, 4, 4, 8, 16, 4),
                                      (24, 24, 6, 1, 4, 4, 1)):
        c = prefill_case(rng, ctx=[n], chunk=[L], hq=hq, hkv=hkv, d=d, bs=bs, dtype="bf16", x=x)
        scale = float(np.float32(0.29))
        got = O.prefill_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], c["qs"],
                                  scale, "bf16")
        conv = np.vectorize(bf16_bits_to_float)
        # queries: positions 0 .. n-L-1 are zero rows (not compared), then the chunk
        qf = np.zeros((n, hq, d))
        qf[n - L:] = conv(c["q"])
        q = torch.tensor(qf).permute(1, 0, 2).unsqueeze(0).contiguous()
        k = torch.tensor(conv(c["k_logical"][0])).permute(1, 0, 2)
        v = torch.tensor(conv(c["v_logical"][0])).permute(1, 0, 2)
        k = k.repeat_interleave(hq // hkv, dim=0).unsqueeze(0).contiguous()
        v = v.repeat_interleave(hq // hkv, dim=0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                               scale=scale)
        ref = ref[0].permute(1, 0, 2).numpy()[n - L:]
        assert np.max(np.abs(got - ref)) <= 1e-12, np.max(np.abs(got - ref))


def pin_prefill_chunks_compose(O):
    """Chunking changes nothing: a prompt attended in three chunks (each with
    the context it has at that point) gives the rows of the one-chunk run;
    and L = 1 gives the decode result."""
    rng = np.random.default_rng(43)
    n, hq, hkv, d, bs = 29, 4, 2, 4, 4
    c = prefill_case(rng, ctx=[n], chunk=[n], hq=hq, hkv=hkv, d=d, bs=bs, dtype="f32", x=2)
    whole = O.prefill_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], c["qs"], 0.5,
                                "f32")
    for a, b in ((0, 11), (11, 12), (12, 29)):
        part = O.prefill_attention(c["q"][a:b], c["kp"], c["vp"], c["tables"],
                                   np.array([b], np.int32), np.array([0, b - a], np.int32), 0.5,
                                   "f32")
        assert np.max(np.abs(part - whole[a:b])) <= 1e-13
    for pos in (0, 5, 28):
        dec = O.decode_attention(c["q"][pos][None], c["kp"], c["vp"], c["tables"],
                                 np.array([pos + 1], np.int32), 0.5, "f32")
        assert np.max(np.abs(dec[0] - whole[pos])) <= 1e-13


def pin_swap(O):
    """[gyaansetu] "How PagedAttention fixes this" (fine-grained eviction):
    a page moved to host memory and back holds the same bytes; nothing else
    moves; attention through the new placement is unchanged, bit for bit."""
    rng = np.random.default_rng(61)
    c = random_case(rng, num_seqs=2, hq=4, hkv=2, d=4, bs=4, ctx_max=0, dtype="bf16",
                    ctx=[9, 6], x=2, slack=4)
    kp, vp, t = c["kp"], c["vp"], c["tables"]
    hk = nan_like_pool((6,) + kp.shape[1:], "bf16")
    hv = nan_like_pool((6,) + vp.shape[1:], "bf16")
    out_pairs = np.array([[t[0, 0], 4], [t[0, 1], 0], [t[0, 2], 5]], np.int32)
    hk2, hv2 = O.swap_blocks(hk, hv, kp, vp, out_pairs)
    for s_, d_ in out_pairs:
        assert hk2[d_].tobytes() == kp[s_].tobytes() and hv2[d_].tobytes() == vp[s_].tobytes()
    for b in (1, 2, 3):                                    # untouched host blocks
        assert hk2[b].tobytes() == hk[b].tobytes() and hv2[b].tobytes() == hv[b].tobytes()
    # back into free device blocks (the ones past the two tables' blocks)
    used = set(t[t >= 0].tolist())
    free = [b for b in range(kp.shape[0]) if b not in used][:3]
    in_pairs = np.array([[4, free[0]], [0, free[1]], [5, free[2]]], np.int32)
    kp2, vp2 = O.swap_blocks(kp, vp, hk2, hv2, in_pairs)
    t2 = t.copy()
    t2[0, :3] = free
    a = O.decode_attention(c["q"], kp, vp, t, c["ctx"], 0.5, "bf16")
    b = O.decode_attention(c["q"], kp2, vp2, t2, c["ctx"], 0.5, "bf16")
    assert a.tobytes() == b.tobytes()
    for blk in range(kp.shape[0]):                         # only the targets changed
        if blk not in free:
            assert kp2[blk].tobytes() == kp[blk].tobytes()


ALL_PINS = [pin_value_decoding, pin_worked_tables, pin_slot_bijection, pin_write_bruteforce,
            pin_write_roundtrip, pin_copy, pin_attention_dense, pin_attention_sdpa,
            pin_closed_forms, pin_shared_vs_private, pin_cow_isolation, pin_prefill_bruteforce,
            pin_prefill_sdpa, pin_prefill_chunks_compose, pin_swap]
