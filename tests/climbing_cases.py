"""Inputs whose attention scores climb along the context (test infrastructure).

Gaussian queries and keys keep every score within a few units of the first
tile's, so a kernel that moves its softmax reference point only when a score
passes it by a margin (8 in log2 units here) seldom does so after the first
tile.  These workloads (workloads.climbing_scores: |q|, keys |k| * g + c * p)
force that move many times per sequence, inside a wave's run of tiles, between
the partials of a split context and across the causal rows of a prefill chunk,
and add spiked keys that outweigh all others by tens of powers of two.  The
GPU parity tests run them against the oracle; test_workloads checks on the CPU
that they really move the reference point.
"""

from __future__ import annotations

import numpy as np

import workloads as W

LAZY_SLACK = 8.0   # log2 units a score may pass the reference before it moves
TILE = 16          # keys scored together before that test is made

RAGGED_CTX = [0, 1, 2, 15, 16, 17, 31, 33, 64, 127, 200, 257, 600]

# name, contexts, Hq, Hkv, D, bs, slope (log2 per position), spiked positions
DECODE = [
    ("ramp-ragged", RAGGED_CTX, 16, 4, 128, 16, 0.33, ()),
    ("ramp-g8-d64-bs8", [3, 100, 700, 40], 8, 1, 64, 8, 0.5, ()),
    ("spikes-ragged", RAGGED_CTX, 16, 4, 128, 16, 0.0, (0, 16, 47, 200, 511)),
    ("ramp-and-spike-long", [0, 5000, 17, 1200, 3], 8, 2, 128, 16, 0.05, (900, 2500)),
]


def decode_case(case):
    name, ctx, hq, hkv, d, bs, slope, spikes = case
    rng = np.random.default_rng(sum(map(ord, name)))
    wl = W.decode_workload(f"climbing {name}", W.BF16, ctx, hq, hkv, d, bs, rng=rng,
                           seed=(17, len(ctx), hq, hkv, d, bs))
    return W.climbing_scores(wl, slope=slope, spike_at=spikes, name=f"climbing {name}")


# name, prefix lengths, chunk lengths, Hq, Hkv, D, bs, slope, spiked positions
PREFILL = [
    ("ramp", [300, 17, 0], [200, 64, 40], 32, 8, 128, 16, 0.33, ()),
    ("ramp-and-spikes-g1-d64", [0, 130], [150, 90], 8, 8, 64, 32, 0.33, (150, 200)),
]


def prefill_case(case):
    name, pre, chunk, hq, hkv, d, bs, slope, spikes = case
    rng = np.random.default_rng(sum(map(ord, name)))
    wl = W.prefill_workload(f"climbing prefill {name}", W.BF16, pre, chunk, hq, hkv, d, bs,
                            rng=rng)
    return W.climbing_scores(wl, slope=slope, spike_at=spikes,
                             name=f"climbing prefill {name}")


def key_rows(wl, seq):
    """float64 key rows [ctx][Hkv][D] of one sequence, by position, from the
    plan's writes (decode and prefill plans write every position once)."""
    n = int(wl.context_lens[seq])
    rows = np.full((n, wl.num_kv_heads, wl.head_dim), np.nan)
    for kind, x in wl.setup + wl.step:
        if kind != "write":
            continue
        sel = x.seq_ids == seq
        rows[x.positions[sel]] = W.bits_to_f32(x.k[sel], wl.dtype)
    assert not np.isnan(rows).any()
    return rows


def log2_scores(wl, q_row, seq, head):
    """Scores of one query row of head ``head`` against every key of ``seq``,
    in log2 units (float64)."""
    k = key_rows(wl, seq)[:, head // wl.group, :]
    q = W.bits_to_f32(q_row[head], wl.dtype).astype(np.float64)
    return (k @ q) * wl.scale / np.log(2.0)


def reference_moves(scores):
    """How often a reference point that starts at the first tile's maximum
    and moves only when a 16-key tile's maximum passes it by the slack has
    to move."""
    ref, moves = -np.inf, -1
    for t in range(0, len(scores), TILE):
        tmax = scores[t:t + TILE].max()
        if tmax > ref + LAZY_SLACK:
            ref, moves = max(ref, tmax), moves + 1
    return moves
