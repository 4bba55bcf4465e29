"""GPU parity: libpa's HIP kernels against the CPU oracle, through the C ABI.

Bar (from the method's accuracy target):
  * slots, cache writes, block copies: bit-exact -- whole pools compared,
    including every NaN-poisoned slot the plan never writes;
  * decode attention: max |gpu - oracle| <= 2e-3 for bf16 K/V, <= 1e-5 for
    float32 K/V (float32 accumulation on the GPU, float64 in the oracle).
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import climbing_cases as C
import workloads as W
from plan_oracle import max_abs_err, run_oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _device():
    from workloads.device import DeviceWorkload
    return DeviceWorkload


def run_both(wl, *, partition=None, vector_only=False, seqs=None, heads=None,
             check_pools=True, fused_write=True, append=False):
    """Run the plan on the GPU and in the oracle; check slots and pools
    bit-exactly; return (gpu_out, oracle_out).  Writes go through
    pa_write_kv_at, or pa_compute_slots + pa_write_kv with fused_write=False;
    with append=True the step's new tokens are stored and attended by one
    pa_decode_attention_append call."""
    DeviceWorkload = _device()
    _say(f"[case] {wl.name} partition={partition} vector_only={vector_only} "
         f"fused_write={fused_write} append={append}")
    dev = DeviceWorkload(wl)
    if append:
        assert dev.step_uses_append()
    dev.run_setup(fused_write=fused_write)
    out = dev.run_step(partition_size=partition, vector_only=vector_only,
                       fused_write=fused_write, append=append).cpu().numpy()
    torch.cuda.synchronize()
    kp, vp, ref, slots_ref = run_oracle(wl, wl.setup + wl.step, seqs=seqs, heads=heads)
    got_slots = dev.slots_of(dev.setup_ops + dev.step_ops)
    assert len(got_slots) == len(slots_ref)
    for a, b in zip(got_slots, slots_ref):
        assert np.array_equal(a, b), "slot mismatch"
    if check_pools:
        gk, gv = dev.pool_bits()
        assert np.array_equal(gk.view(np.uint8), kp.view(np.uint8)), "K pool differs"
        assert np.array_equal(gv.view(np.uint8), vp.view(np.uint8)), "V pool differs"
    return out, ref


# ---------------------------------------------------------------------------
# the five workloads (small versions: full oracle comparison)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_parity_small(cid):
    wl = W.make(cid, small=(cid != 1))
    out, ref = run_both(wl)
    err = max_abs_err(out, ref)
    _say(f"  max_abs_err={err:.3e}")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_append_parity(cid):
    """pa_decode_attention_append: the new tokens land in their slots (pools
    bit-exact) and the output matches the oracle; on the stream-K path the
    decode kernel itself reads and stores them."""
    wl = W.make(cid, small=(cid != 1))
    out, ref = run_both(wl, append=True)
    assert max_abs_err(out, ref) <= TOL[wl.dtype]


@pytest.mark.parametrize("cid", [2, 4])
@pytest.mark.parametrize("partition", [None, 64])
def test_append_equals_write_then_decode_bitwise(cid, partition):
    """Appending inside the decode call changes where the new rows come from,
    not the arithmetic: outputs and pools equal the two-call result bit for
    bit, on the stream-K path and on fixed partitions."""
    wl = W.make(cid, small=True)
    DeviceWorkload = _device()
    res = []
    for append in (False, True):
        dev = DeviceWorkload(wl)
        dev.run_setup()
        o = dev.run_step(partition_size=partition, append=append).cpu().numpy()
        res.append((o, dev.pool_bits()))
    assert res[0][0].tobytes() == res[1][0].tobytes()
    assert res[0][1][0].tobytes() == res[1][1][0].tobytes()
    assert res[0][1][1].tobytes() == res[1][1][1].tobytes()


@pytest.mark.parametrize("cid", [1, 4])
def test_separate_slot_and_write_calls(cid):
    """pa_compute_slots + pa_write_kv (two launches) give the same slots and
    pools as the fused pa_write_kv_at, bit for bit."""
    wl = W.make(cid, small=(cid != 1))
    out, ref = run_both(wl, fused_write=False)
    assert max_abs_err(out, ref) <= TOL[wl.dtype]


def test_cow_observable_parity():
    wl = W.make_cow_observable(small=True)
    out, ref = run_both(wl)
    assert max_abs_err(out, ref) <= TOL[wl.dtype]


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_vector_kernel_parity(cid):
    wl = W.make(cid, small=True)
    out, ref = run_both(wl, vector_only=True, check_pools=False)
    assert max_abs_err(out, ref) <= TOL[wl.dtype]


@pytest.mark.parametrize("part", [16, 32, 64, 128, 256, 512, 1024])
def test_partition_sweep(part):
    wl = W.make(2, small=True)
    out, ref = run_both(wl, partition=part, check_pools=False)
    assert max_abs_err(out, ref) <= TOL[wl.dtype]


# ---------------------------------------------------------------------------
# edge cases: empty and ragged contexts, every block size and head_dim, GQA
# group sizes from 1 to 16, both element types
# ---------------------------------------------------------------------------

EDGE_CTX = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 200, 257, 600]

EDGE_SHAPES = [
    # dtype, Hq, Hkv, D, bs
    ("bf16", 8, 8, 128, 16),     # G = 1
    ("bf16", 16, 8, 128, 8),     # G = 2, block 8 (two blocks per 16-token tile)
    ("bf16", 32, 2, 128, 64),    # G = 16
    ("bf16", 12, 4, 64, 32),     # G = 3 (not a power of two), head_dim 64
    ("bf16", 8, 1, 64, 16),      # one KV head, G = 8
    ("f32", 4, 4, 64, 16),       # float32 path
    ("f32", 16, 2, 128, 8),      # float32, G = 8, block 8
    ("f32", 6, 3, 128, 64),
]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_edge_shapes(shape):
    dtype, hq, hkv, d, bs = shape
    # a fixed integer seed per shape (string hashes change between interpreters)
    rng = np.random.default_rng([7, EDGE_SHAPES.index(shape), hq, hkv, d, bs])
    wl = W.decode_workload(f"edge {shape}", dtype, EDGE_CTX, hq, hkv, d, bs, rng=rng,
                           seed=(7, hq, hkv, d, bs))
    for part, append in ((None, False), (max(16, bs), False), (4 * max(16, bs), False),
                         (None, True)):
        out, ref = run_both(wl, partition=part, check_pools=(part is None), append=append)
        err = max_abs_err(out, ref)
        _say(f"  partition={part} append={append} max_abs_err={err:.3e}")
        assert err <= TOL[dtype]
        assert np.all(out[0] == 0.0)           # ctx == 0 gives zeros
        assert np.isfinite(out).all()


# Work splits of the stream-K path (bf16): many segments
# per wave (segment switches inside a wave's pipeline), contexts of one tile,
# empty contexts between non-empty ones, and one context split over ~150
# waves whose partials are merged.
def _mixed_ctx(rng, n):
    c = rng.integers(1, 49, size=n)
    c[rng.random(n) < 0.2] = 0
    return c


STREAMK_CASES = [
    # name, ctx recipe, Hq, Hkv, D, bs
    ("many-short", lambda r: _mixed_ctx(r, 3000), 8, 2, 128, 16),
    ("many-short-g16-d64", lambda r: _mixed_ctx(r, 1500), 16, 1, 64, 64),
    ("one-long", lambda r: [20000], 4, 1, 128, 32),
    ("long-and-empty", lambda r: [0, 9000, 0, 0, 1, 17, 5000, 0], 16, 4, 128, 16),
    # block size 8: each 16-token tile covers two blocks
    ("many-short-bs8", lambda r: _mixed_ctx(r, 2000), 8, 2, 128, 8),
    ("one-long-bs8-d64", lambda r: [0, 12345, 9], 4, 1, 64, 8),
]


@pytest.mark.parametrize("case", STREAMK_CASES, ids=lambda c: c[0])
def test_streamk_splits(case):
    name, recipe, hq, hkv, d, bs = case
    rng = np.random.default_rng(sum(map(ord, name)))
    ctx = np.asarray(recipe(rng), dtype=np.int32)
    wl = W.decode_workload(f"streamk {name}", "bf16", ctx, hq, hkv, d, bs, rng=rng,
                           seed=(11, len(ctx), hq, hkv, d, bs))
    out, ref = run_both(wl, check_pools=False)
    err = max_abs_err(out, ref)
    _say(f"  max_abs_err={err:.3e}")
    assert err <= TOL["bf16"]
    assert np.all(out[ctx == 0] == 0.0)
    assert np.isfinite(out).all()


# Scores that climb along the context, and spiked keys (tests/climbing_cases):
# the kernels' softmax reference point moves many times inside a wave's run of
# tiles, partials of one split context carry reference points hundreds of
# log2 units apart, and a spike's weight drowns every other key's.
@pytest.mark.parametrize("case", C.DECODE, ids=lambda c: c[0])
def test_climbing_scores(case):
    wl = C.decode_case(case)
    forms = ((None, False, False), (16, False, False), (64, False, False), (None, True, False),
             (None, False, True))
    for part, append, vector_only in forms:
        out, ref = run_both(wl, partition=part, check_pools=(part is None and not vector_only),
                            append=append, vector_only=vector_only)
        err = max_abs_err(out, ref)
        _say(f"  partition={part} append={append} vector_only={vector_only} "
             f"max_abs_err={err:.3e}")
        assert err <= TOL["bf16"]
        assert np.isfinite(out).all() and np.all(out[wl.context_lens == 0] == 0.0)


@pytest.mark.parametrize("num_seqs", [8192, 8193], ids=["streamk-max-batch", "partition-batch"])
def test_largest_batches(num_seqs):
    """The largest batch the stream-K path takes (its tile prefix of S+1
    ints sits in LDS) and one more, which takes fixed partitions: short
    mixed contexts (empties included), every output checked against the
    oracle on a sample of sequences (the rest: finite, zero for empty)."""
    rng = np.random.default_rng(num_seqs)
    ctx = _mixed_ctx(rng, num_seqs)
    wl = W.decode_workload(f"largest batch S={num_seqs}", "bf16", ctx, 8, 2, 128, 16, rng=rng,
                           seed=(13, num_seqs))
    pick = sorted(set([0, num_seqs - 1] + [int(x) for x in rng.choice(num_seqs, 120, replace=False)]))
    out, ref = run_both(wl, seqs=pick, check_pools=False)
    assert max_abs_err(out, ref) <= TOL["bf16"]
    assert np.isfinite(out).all() and np.all(out[ctx == 0] == 0.0)


def test_single_token_is_exact_value_row():
    """ctx == 1: the output equals the only V row (exact in float32)."""
    rng = np.random.default_rng(3)
    wl = W.decode_workload("ctx1", "bf16", [1, 1, 1], 16, 4, 128, 16, rng=rng, seed=(3,))
    out, ref = run_both(wl)
    assert np.array_equal(out.astype(np.float64), ref)


def test_max_context_len_upper_bound_is_harmless():
    import paged_kv_cache_188_amd as pa
    wl = W.make(3, small=True)
    DeviceWorkload = _device()
    dev = DeviceWorkload(wl)
    dev.run_setup()
    a = dev.run_step().clone()
    dev.max_ctx = wl.max_context_len * 3 + 17
    b = dev.run_step()
    torch.cuda.synchronize()
    _, _, ref, _ = run_oracle(wl, wl.setup + wl.step)
    assert max_abs_err(b.cpu().numpy(), ref) <= TOL[wl.dtype]
    assert max_abs_err(a.cpu().numpy(), ref) <= TOL[wl.dtype]


@pytest.mark.parametrize("partition,append", [(None, False), (None, True), (64, False),
                                              (64, True)])
def test_max_context_len_below_a_context_truncates(partition, append):
    """A max_context_len below some context truncates that context to its
    first max_context_len tokens on both decompositions (and the append call
    then neither stores nor attends its new token)."""
    import copy
    wl = W.make(3, small=True)
    bound = int(np.median(wl.context_lens))
    _say(f"[case] truncation bound={bound} partition={partition} append={append}")
    DeviceWorkload = _device()
    dev = DeviceWorkload(wl)
    dev.run_setup()
    dev.max_ctx = bound
    out = dev.run_step(partition_size=partition, append=append).cpu().numpy()
    torch.cuda.synchronize()
    from oracle import paged_attention as O
    kp, vp, _, _ = run_oracle(wl, wl.setup + (wl.step if not append else []))
    if append:  # the untruncated sequences' new tokens are stored by the call
        w2 = copy.copy(wl)
        keep = wl.context_lens <= bound
        x = [op for op in wl.step if op[0] == "write"][0][1]
        sel = keep[x.seq_ids]
        xs = W.Write(x.table, x.seq_ids[sel], x.positions[sel], x.k[sel], x.v[sel])
        kp, vp, _, _ = run_oracle(w2, [("write", xs)], kp=kp, vp=vp)
        gk, gv = dev.pool_bits()
        assert np.array_equal(gk.view(np.uint8), kp.view(np.uint8)), "K pool differs"
        assert np.array_equal(gv.view(np.uint8), vp.view(np.uint8)), "V pool differs"
    ctx = np.minimum(wl.context_lens, bound).astype(np.int32)
    ref = O.decode_attention(wl.q, kp, vp, wl.tables["final"], ctx, wl.scale, wl.dtype)
    err = max_abs_err(out, ref)
    _say(f"  max_abs_err={err:.3e}")
    assert err <= TOL[wl.dtype]


# ---------------------------------------------------------------------------
# invariants on the device
# ---------------------------------------------------------------------------

def _relabel(wl, seed):
    """Same logical data, different physical placement: apply a random
    permutation of the pool to every block table and copy pair."""
    import copy
    rng = np.random.default_rng(seed)
    perm = rng.permutation(wl.num_blocks).astype(np.int32)
    w2 = copy.copy(wl)
    w2.tables = {k: np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32)
                 for k, t in wl.tables.items()}
    w2.setup = [(k, perm[x].astype(np.int32)) if k == "copy" else (k, x) for k, x in wl.setup]
    w2.step = [(k, perm[x].astype(np.int32)) if k == "copy" else (k, x) for k, x in wl.step]
    return w2


@pytest.mark.parametrize("cid", [2, 4, 5])
def test_placement_invariance_bitwise(cid):
    """Invariant (a) on the device: moving blocks in the pool changes nothing,
    bit for bit (the arithmetic order depends on logical positions only)."""
    wl = W.make(cid, small=True)
    DeviceWorkload = _device()
    outs = []
    for w in (wl, _relabel(wl, 1), _relabel(wl, 2)):
        dev = DeviceWorkload(w)
        dev.run_setup()
        outs.append(dev.run_step().cpu().numpy())
    assert outs[0].tobytes() == outs[1].tobytes() == outs[2].tobytes()


def test_run_to_run_determinism():
    wl = W.make(3, small=True)
    DeviceWorkload = _device()
    dev = DeviceWorkload(wl)
    dev.run_setup()
    a = dev.run_step().cpu().numpy()
    b = dev.run_step().cpu().numpy()
    c = dev.decode_only(vector_only=False).cpu().numpy()
    assert a.tobytes() == b.tobytes() == c.tobytes()


@pytest.mark.parametrize("cid", [1, 2, 4])
def test_prepared_call_equals_direct_call_bitwise(cid):
    """A PreparedCall (arguments marshalled once, issued several times) runs
    the same launches as the direct call: equal outputs and pools, bit for
    bit, and every re-issue gives the same answer."""
    wl = W.make(cid, small=(cid != 1))
    DeviceWorkload = _device()
    res = []
    for prepared in (False, True):
        dev = DeviceWorkload(wl)
        dev.run_setup()
        if prepared:
            ops = dev.step_ops_append
            calls = dev.prepare(ops)
            outs = []
            for _ in range(2):
                for c in calls:
                    c()
                outs.append(dev.out.cpu().numpy())
            assert outs[0].tobytes() == outs[1].tobytes()
            o = outs[0]
        else:
            o = dev.run_step(append=True).cpu().numpy()
            o2 = dev.run_step(append=True).cpu().numpy()
            assert o.tobytes() == o2.tobytes()
        res.append((o, dev.pool_bits()))
    assert res[0][0].tobytes() == res[1][0].tobytes()
    assert res[0][1][0].tobytes() == res[1][1][0].tobytes()
    assert res[0][1][1].tobytes() == res[1][1][1].tobytes()


@pytest.mark.parametrize("cid", [2, 3])
def test_append_with_bad_table_entry_writes_nothing_there(cid):
    """A table entry outside the pool in the block that would receive a new
    token: the append call skips that store (the pools equal the good call's
    pools with that one slot left as it was), never writes block 0 in its
    place, and every other sequence's output is unchanged bit for bit."""
    wl = W.make(cid, small=True)
    DeviceWorkload = _device()
    good = DeviceWorkload(wl)
    good.run_setup()
    before_k, before_v = good.pool_bits()
    out_good = good.run_step(append=True).cpu().numpy()
    gk, gv = good.pool_bits()
    bad = DeviceWorkload(wl)
    bad.run_setup()
    table = [x for kind, x in wl.step if kind == "decode"][0]
    n0 = int(wl.context_lens[0])
    blk = (n0 - 1) // wl.block_size
    phys = int(wl.tables[table][0, blk])
    bad.tables[table][0, blk] = wl.num_blocks + 5
    out_bad = bad.run_step(append=True).cpu().numpy()
    bk, bv = bad.pool_bits()
    # the good call's pools with sequence 0's new slot as before the step
    o = (n0 - 1) % wl.block_size
    ek, ev = gk.copy(), gv.copy()
    ek[phys, :, :, o, :] = before_k[phys, :, :, o, :]
    ev[phys, :, o, :] = before_v[phys, :, o, :]
    assert bk.tobytes() == ek.tobytes()
    assert bv.tobytes() == ev.tobytes()
    assert out_bad[1:].tobytes() == out_good[1:].tobytes()


def test_workspace_reuse_with_new_queries():
    """Consecutive calls on one workspace: partials and arrival counters left
    by a call never leak into the next (new queries give the oracle's new
    answer; the old queries give the old answer again, bit for bit)."""
    import copy
    from workloads.device import to_device
    for cid in (2, 3):
        wl = W.make(cid, small=True)
        DeviceWorkload = _device()
        dev = DeviceWorkload(wl)
        dev.run_setup()
        a = dev.run_step().cpu().numpy()
        w2 = copy.copy(wl)
        w2.q = W.draw_normal(np.random.default_rng(99 + cid), wl.q.shape, wl.dtype)
        q_old = dev.q
        dev.q = to_device(w2.q, wl.dtype)
        b = dev.decode_only().cpu().numpy()
        dev.q = q_old
        c = dev.decode_only().cpu().numpy()
        torch.cuda.synchronize()
        _, _, ref_b, _ = run_oracle(w2, w2.setup + w2.step)
        err = max_abs_err(b, ref_b)
        _say(f"  config {cid}: new-query max_abs_err={err:.3e}")
        assert err <= TOL[wl.dtype]
        assert a.tobytes() == c.tobytes()


def test_shared_prefix_equals_private_copies():
    """Invariant (b): samples that share physical prefix blocks get, bit for
    bit, the outputs they get when every sample owns a private copy."""
    wl = W.make(4, small=True)
    groups, samples = wl.notes["groups"], wl.notes["samples"]
    npb = -(-wl.notes["prefix"] // wl.block_size)
    # private variant: give every sample its own copy of every shared block
    import copy
    priv = copy.copy(wl)
    fin = wl.tables["final"].copy()
    pre = wl.tables["pre"].copy()
    extra = []
    nxt = wl.num_blocks
    for a in range(groups):
        for s in range(1, samples):
            i = a * samples + s
            for b in range(npb - 1):          # the last prefix block is already private
                fin[i, b] = nxt
                pre[i, b] = nxt
                extra.append(nxt)
                nxt += 1
    priv.num_blocks = nxt
    priv.tables = {"final": fin, "pre": pre}
    # the prefix write now goes to every sample (each through its own table)
    new_setup = []
    for kind, x in wl.setup:
        if kind == "write" and x.table == "pre":
            # sample 0 writes the whole prefix; the others write the blocks
            # they now own privately (the last prefix block stays shared
            # until copy-on-write), so no slot is written twice
            reps = [x]
            own = x.positions < (npb - 1) * wl.block_size
            for s in range(1, samples):
                reps.append(W.Write("pre", x.seq_ids[own] + s, x.positions[own], x.k[own], x.v[own]))
            new_setup.append(("write", W.Write(
                "pre", np.concatenate([r.seq_ids for r in reps]).astype(np.int32),
                np.concatenate([r.positions for r in reps]),
                np.concatenate([r.k for r in reps]), np.concatenate([r.v for r in reps]))))
        else:
            new_setup.append((kind, x))
    priv.setup = new_setup
    DeviceWorkload = _device()
    outs = []
    for w in (wl, priv):
        dev = DeviceWorkload(w)
        dev.run_setup()
        outs.append(dev.run_step().cpu().numpy())
    assert outs[0].tobytes() == outs[1].tobytes()
    _, _, ref, _ = run_oracle(wl, wl.setup + wl.step)
    assert max_abs_err(outs[0], ref) <= TOL[wl.dtype]


def test_copy_on_write_isolates_the_writer():
    """Invariant (c): after a sample's private copy is modified, every other
    sharer's output is bit-identical to before, and the shared original block
    is untouched."""
    import paged_kv_cache_188_amd as pa
    from workloads.device import to_device
    wl = W.make_cow_observable(small=True)
    DeviceWorkload = _device()
    dev = DeviceWorkload(wl)
    dev.run_setup()
    before = dev.run_step().cpu().numpy()
    k, v = dev.pools[0]
    kb, vb = k.clone(), v.clone()
    # overwrite the first tail token of sample 0 (it lies in its private copy)
    prefix = wl.notes["prefix"]
    tbl = dev.tables["final"]
    pos = torch.tensor([prefix], dtype=torch.int32, device="cuda")
    slot = pa.compute_slots(tbl, pos, wl.block_size, wl.num_blocks,
                            seq_ids=torch.tensor([0], dtype=torch.int32, device="cuda"))
    rng = np.random.default_rng(9)
    kn = to_device(W.draw_normal(rng, (1, wl.num_kv_heads, wl.head_dim), wl.dtype), wl.dtype)
    vn = to_device(W.draw_normal(rng, (1, wl.num_kv_heads, wl.head_dim), wl.dtype), wl.dtype)
    pa.write_kv(k, v, kn, vn, slot)
    after = dev.decode_only().cpu().numpy()
    assert after[1:].tobytes() == before[1:].tobytes()
    assert not np.array_equal(after[0], before[0])
    # only the private block of sample 0 changed
    changed = (k.view(torch.int16) != kb.view(torch.int16)).flatten(1).any(1)
    changed = changed.nonzero().flatten().tolist()
    assert changed == [int(wl.tables["final"][0, prefix // wl.block_size])]
    shared = int(wl.tables["pre"][0, prefix // wl.block_size])
    assert torch.equal(k[shared].view(torch.int16), kb[shared].view(torch.int16))
    assert torch.equal(v[shared].view(torch.int16), vb[shared].view(torch.int16))


# ---------------------------------------------------------------------------
# full sizes, in the launch configuration the benchmark times; sampled outputs
# ---------------------------------------------------------------------------

FULL_SAMPLES = {
    2: dict(n_seqs=4, heads=None),
    3: dict(n_seqs=5, heads=None),
    4: dict(n_seqs=4, heads=None),
    5: dict(n_seqs=2, heads=[0, 7, 8, 33, 63]),
}


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size_sampled(cid):
    wl = W.make(cid)
    ctx = wl.context_lens
    order = np.argsort(ctx, kind="stable")
    n = FULL_SAMPLES[cid]["n_seqs"]
    pick = sorted(set([int(order[0]), int(order[-1])] +
                      [int(x) for x in np.random.default_rng(cid).choice(wl.num_seqs, n, replace=False)]))
    out, ref = run_both(wl, seqs=pick, heads=FULL_SAMPLES[cid]["heads"])
    err = max_abs_err(out, ref)
    _say(f"  sampled seqs={pick} max_abs_err={err:.3e}")
    assert err <= TOL[wl.dtype]
    # properties that hold at every size: finite, and each output row lies in
    # the convex hull of its V rows, so |out| <= max |V| (here < 6 sigma)
    assert np.isfinite(out).all()
    assert np.abs(out).max() < 6.5
