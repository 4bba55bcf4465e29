"""pa_decode_attention_shared on the GPU against the oracle's plain decode.

The shared-prefix call must compute exactly what pa_decode_attention(_append)
computes (the oracle's decode over each sequence's own table); only the
number of times a shared block is read changes.  Groups come from
pa.shared_prefix_groups over the host copy of the table.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from plan_oracle import max_abs_err, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-3  # bf16 decode tolerance, as for the single-pass call


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dev(wl):
    from workloads.device import DeviceWorkload
    dev = DeviceWorkload(wl)
    dev.run_setup()
    return dev


def _shared_wl(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, samples=4,
               groups=3, prefix=96, tail=(5, 60), seed=7, cow_in_step=True):
    rng = np.random.default_rng(seed)
    name = (f"shared-prefix {groups}x{samples} prefix={prefix} Hq={num_q_heads} "
            f"Hkv={num_kv_heads} D={head_dim} bs={block_size} [small]")
    return W.shared_prefix_workload(name, rng=rng, groups=groups, samples=samples, prefix=prefix,
                                    tail_lo=tail[0], tail_hi=tail[1], num_q_heads=num_q_heads,
                                    num_kv_heads=num_kv_heads, head_dim=head_dim,
                                    block_size=block_size, cow_in_step=cow_in_step)


def _check(wl, append, seqs=None, heads=None):
    _say(f"[case] {wl.name} append={append} seqs={seqs}")
    dev = _dev(wl)
    gs, sl, _ = dev.shared_args("final")
    _say(f"  groups={gs.cpu().tolist()} shared_len={sl.cpu().tolist()[:8]}")
    out = dev.run_step(append=append, shared=True).cpu().numpy()
    torch.cuda.synchronize()
    kp, vp, ref, _ = run_oracle(wl, wl.setup + wl.step, seqs=seqs, heads=heads)
    gk, gv = dev.pool_bits()
    assert np.array_equal(gk.view(np.uint8), kp.view(np.uint8)), "K pool differs"
    assert np.array_equal(gv.view(np.uint8), vp.view(np.uint8)), "V pool differs"
    err = max_abs_err(out, ref)
    _say(f"  max_abs_err={err:.3e}")
    assert err <= TOL
    return out


@pytest.mark.parametrize("append", [False, True])
def test_shared_parity_config_small(append):
    """The shared-prefix workload (small): groups of 4 samples (G = 4)."""
    _check(W.make(4, small=True), append)


@pytest.mark.parametrize("append", [False, True])
def test_shared_parity_cow_observable(append):
    """Prefix ending inside a block whose private copies then diverge: only
    whole blocks before it are read as shared."""
    _check(W.make_cow_observable(small=True), append)


@pytest.mark.parametrize("shape", [
    dict(num_q_heads=64, num_kv_heads=8),                    # G = 8: pairs
    dict(num_q_heads=8, num_kv_heads=8, samples=8),          # G = 1: eight members
    dict(num_q_heads=16, num_kv_heads=8, samples=8),         # G = 2: eight members
    dict(num_q_heads=32, num_kv_heads=8, head_dim=64),
    dict(num_q_heads=32, num_kv_heads=8, block_size=8),
    dict(num_q_heads=32, num_kv_heads=8, block_size=32),
    dict(num_q_heads=16, num_kv_heads=1, samples=3, prefix=256, tail=(1, 40)),  # G = 16: none
    # a 20,000-token prefix: each group's prefix segment split over many
    # waves, long merge chains in the prefix pass
    dict(num_q_heads=32, num_kv_heads=8, samples=4, groups=2, prefix=20000, tail=(5, 300)),
])
def test_shared_parity_shapes(shape):
    _check(_shared_wl(**shape), append=True)


@pytest.mark.parametrize("append", [False, True])
def test_shared_climbing_scores(append):
    """Scores that climb along the context with one spiked key in the shared
    prefix and one in the own tokens: the prefix pass and the own-token pass
    end on reference points far apart, which the combine must reconcile."""
    wl = W.climbing_scores(_shared_wl(prefix=160, tail=(20, 90), seed=23), slope=0.33,
                           spike_at=(70, 200), name="shared-prefix climbing scores")
    _check(wl, append)


def test_shared_full_size_sampled():
    """The full shared-prefix workload (32 prompts x 8 samples, prefix 2048)
    in the benchmark's launch configuration; sampled outputs."""
    wl = W.make(4)
    pick = [0, 3, 4, 7, 100, 255]
    dev = _dev(wl)
    out = dev.run_step(append=True, shared=True).cpu().numpy()
    _, _, ref, _ = run_oracle(wl, wl.setup + wl.step, seqs=pick)
    err = max_abs_err(out, ref)
    _say(f"  sampled seqs={pick} max_abs_err={err:.3e}")
    assert err <= TOL
    assert np.isfinite(out).all()


@pytest.mark.parametrize("cid", [2, 3])
def test_no_sharing_equals_plain_call_bitwise(cid):
    """Without shared blocks every group is a lone sequence: the own-token
    pass is the plain stream-K pass and the result is bit-identical."""
    wl = W.make(cid, small=True)
    res = []
    for shared in (False, True):
        dev = _dev(wl)
        if shared:
            gs, sl, _ = dev.shared_args("final")
            assert int(sl.max()) == 0
        res.append((dev.run_step(append=True, shared=shared).cpu().numpy(), dev.pool_bits()))
    assert res[0][0].tobytes() == res[1][0].tobytes()
    assert res[0][1][0].tobytes() == res[1][1][0].tobytes()


def test_group_larger_than_a_tile_and_unaligned_shared_len():
    """Groups of 8 samples with G = 4 (only the first 4 are read together)
    and a shared length that is not a multiple of 16: the result is still
    the plain decode's."""
    wl = W.make(4, small=True)
    dev = _dev(wl)
    gs, sl, ws = dev.shared_args("final")
    samples = wl.notes["samples"]
    gs8 = torch.arange(0, wl.num_seqs + 1, samples, dtype=torch.int32, device="cuda")
    sl8 = torch.full((gs8.numel() - 1,), 75, dtype=torch.int32, device="cuda")
    dev._shared["final"] = (gs8, sl8, ws)
    out = dev.run_step(append=True, shared=True).cpu().numpy()
    _, _, ref, _ = run_oracle(wl, wl.setup + wl.step)
    assert max_abs_err(out, ref) <= TOL


def test_shared_run_to_run_determinism():
    wl = W.make(4, small=True)
    outs = []
    for _ in range(2):
        dev = _dev(wl)
        outs.append(dev.run_step(append=True, shared=True).cpu().numpy())
    assert outs[0].tobytes() == outs[1].tobytes()


def test_prepared_shared_call_repeats():
    """A prepared shared call issued twice (workspace reused) gives the same
    bits as the direct call."""
    wl = W.make(4, small=True)
    dev = _dev(wl)
    direct = dev.decode_only(shared=True).cpu().numpy().copy()
    calls = dev.prepare([op for op in dev.step_ops if op[0] == "decode"], shared=True)
    for _ in range(2):
        for c in calls:
            c()
        assert dev.out.cpu().numpy().tobytes() == direct.tobytes()
