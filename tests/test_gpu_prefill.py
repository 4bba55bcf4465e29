"""GPU parity of the multi-query (chunked prefill) paged attention.

A chunk of prompt tokens per sequence ([bicarait] "Blueprint Arsitektur 3:
Chunked Prefill", 512-token chunks) is written into the paged cache and
attends causally to everything before it through the block table.  Checked
against the oracle's prefill_attention, element by element, at the full
chunked-prefill workload too (16 sequences, 6877 query tokens: the oracle
takes seconds).  Bar: max |gpu - oracle| <= 2e-3 (bf16 K/V/Q, float32
accumulation), pools bit-exact.  P V runs in fp16 (weights rounded to 11
significant bits, V scaled by 2^-4): its range is checked with V scaled far
up and far down.
"""

from __future__ import annotations

import copy
import sys

import numpy as np
import pytest
import torch

import climbing_cases as C
import paged_kv_cache_188_amd as pa
import workloads as W
from oracle import paged_attention as O
from plan_oracle import max_abs_err, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(wl):
    from workloads.device import DeviceWorkload
    _say(f"[case] {wl.name} S={wl.num_seqs} T={int(wl.query_start[-1])} Hq={wl.num_q_heads} "
         f"Hkv={wl.num_kv_heads} D={wl.head_dim} bs={wl.block_size}")
    dev = DeviceWorkload(wl)
    dev.run_setup()
    out = dev.run_step().cpu().numpy()
    torch.cuda.synchronize()
    return dev, out


def _check(wl, dev, out):
    kp, vp, ref, _ = run_oracle(wl, wl.setup + wl.step)
    gk, gv = dev.pool_bits()
    assert gk.tobytes() == kp.tobytes() and gv.tobytes() == vp.tobytes(), "pools differ"
    err = max_abs_err(out, ref)
    _say(f"  max_abs_err={err:.3e}")
    assert err <= TOL
    return kp, vp, ref


@pytest.mark.parametrize("small", [True, False], ids=["small", "full"])
def test_prefill_workload_parity(small):
    wl = W.make_prefill(small=small)
    dev, out = _run(wl)
    _check(wl, dev, out)


def _custom(rng, pre, chunk, hq, hkv, d, bs):
    return W.prefill_workload(f"prefill custom G={hq // hkv} D={d} bs={bs}", W.BF16, pre, chunk,
                              hq, hkv, d, bs, rng=rng)


# (prefix lengths, chunk lengths, Hq, Hkv, D, bs): every group size G = 1, 2,
# 4, 6, 8, 16 (128 / G chunk tokens per workgroup, 128 - 128 % G rows used),
# both head dims, every block size, empty chunks, one-token chunks, chunks
# starting at position 0, contexts over 64 blocks (of 16, 32 and 64 tokens),
# a 2048-token chunk
EDGE = [
    ([0, 40, 3], [37, 16, 1], 8, 8, 64, 32),
    ([100, 0, 17], [64, 0, 129], 16, 8, 128, 16),
    ([5, 260], [33, 7], 16, 2, 128, 64),
    ([31, 2], [50, 19], 12, 2, 128, 16),
    ([0, 1100], [21, 40], 16, 1, 64, 16),
    ([1500, 0], [300, 200], 32, 8, 128, 16),
    ([2000, 37], [2048, 700], 16, 2, 128, 32),   # a 2048-token chunk over a long prefix
    # 64-token blocks past 64 blocks (4096 positions): the walk crosses a
    # chunk of 64 table entries
    ([4200, 3], [300, 90], 8, 8, 64, 64),
    ([4100, 0], [64, 129], 32, 8, 128, 64),
    # a long walk: ~2000 key steps through ~32 chunks of table entries
    ([65000], [40], 8, 8, 128, 32),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"G{c[2] // c[3]}-D{c[4]}-bs{c[5]}")
def test_prefill_shapes(case):
    pre, chunk, hq, hkv, d, bs = case
    wl = _custom(np.random.default_rng(sum(pre) + hq), pre, chunk, hq, hkv, d, bs)
    dev, out = _run(wl)
    _check(wl, dev, out)


@pytest.mark.parametrize("case", C.PREFILL, ids=lambda c: c[0])
def test_prefill_climbing_scores(case):
    """Scores that climb along the context, and spiked keys
    (tests/climbing_cases): each query row's reference point moves many
    times over its causal window and spikes drown the other keys' weights."""
    wl = C.prefill_case(case)
    dev, out = _run(wl)
    _check(wl, dev, out)
    assert np.isfinite(out).all()


def test_chunk_longer_than_context_gives_zeros():
    """Tokens at negative positions (context shorter than the chunk) see no
    key: zero rows; the others attend over the shortened context."""
    wl = _custom(np.random.default_rng(7), [20, 3], [30, 9], 32, 8, 128, 16)
    from workloads.device import DeviceWorkload
    dev = DeviceWorkload(wl)
    dev.run_setup()
    dev.run_step()
    kp, vp = dev.pool_bits()
    short = np.array([25, 4], np.int32)            # chunks of 30 and 9 tokens
    out = pa.prefill_attention(dev.q, *dev.pools[0], dev.tables["final"],
                               torch.from_numpy(short).cuda(), dev.qs, wl.scale,
                               wl.max_query_len).cpu().numpy()
    ref = O.prefill_attention(wl.q, kp, vp, wl.tables["final"], short, wl.query_start, wl.scale,
                              wl.dtype)
    assert max_abs_err(out, ref) <= TOL
    assert not out[:5].any() and not out[30:35].any()   # positions -5 .. -1
    assert out[5:30].any() and out[35:].any()


def test_one_token_chunks_match_the_decode():
    """L = 1 for every sequence is a decode: the prefill kernel and the
    decode path agree with each other and with the oracle."""
    wl = _custom(np.random.default_rng(9), [0, 77, 300, 1023], [1, 1, 1, 1], 32, 8, 128, 16)
    dev, out = _run(wl)
    kp, vp, ref = _check(wl, dev, out)
    dec = pa.decode_attention(dev.q, *dev.pools[0], dev.tables["final"], dev.ctx, wl.scale,
                              int(wl.context_lens.max())).cpu().numpy()
    assert max_abs_err(dec, ref) <= TOL
    assert np.abs(dec - out).max() <= 2 * TOL


def test_prefill_placement_invariance_bitwise():
    """Moving blocks in the pool changes nothing, bit for bit."""
    wl = W.make_prefill(small=True)
    outs = []
    for seed in (None, 1, 2):
        w = wl
        if seed is not None:
            perm = np.random.default_rng(seed).permutation(wl.num_blocks).astype(np.int32)
            w = copy.copy(wl)
            t = wl.tables["final"]
            w.tables = {"final": np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32)}
        _, out = _run(w)
        outs.append(out)
    assert outs[0].tobytes() == outs[1].tobytes() == outs[2].tobytes()


def test_prefill_more_pairs_than_the_sort_takes():
    """16400 one-token chunks: more (sequence, query tile) pairs than the
    kernel's in-LDS longest-first ranking handles (16384), so the workgroups
    take the pairs in index order -- the results are the same."""
    rng = np.random.default_rng(11)
    S = 16400
    wl = W.prefill_workload("prefill 16400 one-token chunks", W.BF16, rng.integers(0, 40, size=S),
                            np.ones(S, np.int64), 8, 8, 64, 16, rng=rng)
    dev, out = _run(wl)
    _check(wl, dev, out)


def _scale_v(wl, f):
    """The workload with every written V row multiplied by f (rounded to
    bf16): same keys, queries and placement."""
    w2 = copy.copy(wl)

    def scaled(ops):
        out = []
        for kind, x in ops:
            if kind == "write":
                v = (O.to_f64(x.v, wl.dtype) * f).astype(np.float32)
                x = W.Write(x.table, x.seq_ids, x.positions, x.k, W.f32_to_bf16_bits(v))
            out.append((kind, x))
        return out

    w2.setup, w2.step = scaled(wl.setup), scaled(wl.step)
    w2.name = f"{wl.name} V x {f:g}"
    return w2


@pytest.mark.parametrize("f", [3e4, 1e-3])
def test_prefill_value_range(f):
    """P V runs on the fp16 matrix cores with V scaled by 2^-4: values far
    beyond fp16's 65504 (here up to ~1.5e5) and values mostly below 2^-10
    (fp16 subnormals after scaling) keep the decode's bar relative to the
    size of V: max |gpu - oracle| <= 2e-3 * f."""
    wl = _scale_v(_custom(np.random.default_rng(11), [300, 17], [200, 64], 32, 8, 128, 16), f)
    dev, out = _run(wl)
    kp, vp, ref, _ = run_oracle(wl, wl.setup + wl.step)
    assert np.isfinite(out).all()
    err = max_abs_err(out, ref)
    _say(f"  max_abs_err={err:.3e} (bar {TOL * f:.3e})")
    assert err <= TOL * f
