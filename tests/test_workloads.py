"""Seeded generators and the byte accounting the benchmark reports (CPU)."""

import math

import numpy as np
import pytest

import workloads as W
import oracle_pins as P


def test_bf16_rounding_is_nearest_even():
    # exact ties go to the even neighbour; above/below a tie round to nearest
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing in [1, 2)
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2 ** -20,
                  one + ulp / 2 - 2 ** -20, -2.5, 3.0e38], dtype=np.float32)
    got = [P.bf16_bits_to_float(b) for b in W.f32_to_bf16_bits(x)]
    assert got[0] == 1.0
    assert got[1] == 1.0                  # tie -> even (1.0)
    assert got[2] == one + 2 * ulp        # tie -> even (mantissa ...10)
    assert got[3] == one + ulp
    assert got[4] == 1.0
    assert got[5] == -2.5
    assert math.isclose(got[6], 3.0e38, rel_tol=2 ** -8)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_small_workloads_are_deterministic_and_well_formed(cid):
    a, b = W.make(cid, small=True), W.make(cid, small=True)
    assert a.q.tobytes() == b.q.tobytes()
    for (ka, xa), (kb, xb) in zip(a.setup + a.step, b.setup + b.step):
        assert ka == kb
        if ka == "write":
            assert xa.k.tobytes() == xb.k.tobytes() and xa.positions.tobytes() == xb.positions.tobytes()
    bt = a.tables["final"]
    for i, c in enumerate(a.context_lens):
        nb = -(-int(c) // a.block_size)
        assert np.all(bt[i, :nb] >= 0) and np.all(bt[i, :nb] < a.num_blocks)
        assert np.all(bt[i, nb:] == -1)
    # every written token is distinct: no (sequence, position) pair twice
    seen = set()
    for kind, op in a.setup + a.step:
        if kind == "write":
            t = op.table
            for s_, p_ in zip(op.seq_ids, op.positions):
                key = (t, int(s_), int(p_)) if t == "final" else ("pre", int(s_), int(p_))
                assert key not in seen
                seen.add(key)


def test_tiny_config_matches_its_description():
    w = W.make(1)
    assert list(w.context_lens) == [5, 16, 17, 40]
    assert (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks) == \
        (4, 4, 4, 64, 16, 32)
    assert w.dtype == "f32" and w.scale == 0.125
    used = w.tables["final"][w.tables["final"] >= 0]
    assert used.size == 7 and np.unique(used).size == 7


def test_kv_bytes_formula_matches_the_pages_70b_figure():
    """The memory-problem section of the gyaansetu page prints about 1.3 GB of
    KV for one 4096-token Llama 3.1 70B sequence, and 336 GB for 256 users."""
    g = P.load_golden("closed_forms.json")["kv_bytes_70b"]
    wl = W.Workload(name="70b-one-seq", dtype="bf16", num_seqs=1, num_q_heads=64,
                    num_kv_heads=g["num_kv_heads"], head_dim=g["head_dim"], block_size=16,
                    num_blocks=256, max_blocks_per_seq=256, scale=1.0, q=None,
                    tables={"final": np.arange(256, dtype=np.int32)[None]},
                    context_lens=np.array([g["tokens"]], np.int32))
    per_layer = wl.kv_bytes_read()
    total = per_layer * g["num_layers"]
    assert total == 2 * 80 * 8 * 128 * 2 * 4096
    assert round(total / 1e9, 1) == g["printed_gb_per_sequence"]
    # 256 users: the formula gives 343.6 GB; the page's 336 GB is 256 x 1.3125,
    # a rounded per-sequence figure, so agreement is to within 3 %
    assert abs(g["users"] * total / 1e9 - g["printed_gb_for_users"]) / g["printed_gb_for_users"] < 0.03


def test_fragmentation_and_sharing_closed_forms():
    g = P.load_golden("closed_forms.json")
    f = g["internal_fragmentation"]
    assert round(100 * (1 - f["used"] / f["reserved"])) == f["printed_waste_percent"]
    assert f["reserved"] - f["used"] == f["printed_wasted_tokens"]
    s = g["prompt_sharing"]
    assert 100 * (s["samples"] - 1) / s["samples"] == s["printed_saving_percent"]


def test_shared_prefix_accounting():
    w = W.make(4, small=True)
    groups, samples = w.notes["groups"], w.notes["samples"]
    fin, pre = w.tables["final"], w.tables["pre"]
    npb = -(-w.notes["prefix"] // w.block_size)
    for a in range(groups):
        rows = range(a * samples, (a + 1) * samples)
        # all samples of a group share the prefix blocks except the copied last one
        assert all(np.array_equal(fin[r, :npb - 1], fin[a * samples, :npb - 1]) for r in rows)
        assert len({int(fin[r, npb - 1]) for r in rows}) == samples
        assert len({int(pre[r, npb - 1]) for r in rows}) == 1
    # unique KV is well below the logical KV: the prefix is stored once per group
    assert w.unique_kv_bytes() < w.kv_bytes_read()


def test_climbing_inputs_move_the_reference_point():
    """The climbing-score workloads the GPU parity tests run do what they are
    for: along the longest context the reference point of a lazy softmax
    (slack 8 in log2, 16-key tiles) moves many times -- about once per 8
    log2 of rise where only the ramp lifts the scores, at least 4 times where
    spikes lift the reference point above the ramp for a while -- and every
    spiked key outweighs every key that is not spiked by >= 2^30."""
    import climbing_cases as C
    for case in C.DECODE:
        wl = C.decode_case(case)
        slope, spikes = case[6], case[7]
        s = int(np.argmax(wl.context_lens))
        n = int(wl.context_lens[s])
        for h in (0, wl.num_q_heads - 1):
            sc = C.log2_scores(wl, wl.q[s], s, h)
            if slope:
                # the expected rise over the context, in steps of the slack
                want = 0.5 * slope * n / C.LAZY_SLACK if not spikes else 4
                assert C.reference_moves(sc) >= want, (case[0], h)
            plain = np.delete(sc, [p for p in spikes if p < n])
            for p in spikes:
                if p < n and not slope:
                    assert sc[p] - plain.max() >= 30, (case[0], p)
    for case in C.PREFILL:
        wl = C.prefill_case(case)
        s = int(np.argmax(wl.context_lens))
        last = int(wl.query_start[s + 1]) - 1
        sc = C.log2_scores(wl, wl.q[last], s, 0)
        want = 0.5 * case[7] * sc.size / C.LAZY_SLACK if not case[8] else 4
        assert C.reference_moves(sc) >= want, case[0]
