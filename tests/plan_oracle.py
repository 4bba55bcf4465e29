"""Execute a workload plan with the CPU oracle (test infrastructure)."""

from __future__ import annotations

import numpy as np

from oracle import paged_attention as O


def run_oracle(wl, ops, kp=None, vp=None, seqs=None, heads=None):
    """Returns (k_pool, v_pool, decode output or None, [slots of each write])."""
    if kp is None:
        kp, vp = wl.empty_pools()
    out = None
    slots_all = []
    for kind, x in ops:
        if kind == "write":
            s = O.slot_mapping(wl.tables[x.table], x.seq_ids, x.positions, wl.block_size,
                               wl.num_blocks)
            slots_all.append(s)
            kp, vp = O.write_kv(kp, vp, x.k, x.v, s)
        elif kind == "copy":
            kp, vp = O.copy_blocks(kp, vp, x)
        elif kind == "prefill":
            out = O.prefill_attention(wl.q, kp, vp, wl.tables[x], wl.context_lens,
                                      wl.query_start, wl.scale, wl.dtype)
        else:
            out = O.decode_attention(wl.q, kp, vp, wl.tables[x], wl.context_lens, wl.scale,
                                     wl.dtype, seqs=seqs, heads=heads)
    return kp, vp, out, slots_all


def max_abs_err(got, ref):
    """Max |got - ref| over entries the oracle computed (non-NaN in ref).
    A NaN in `got` at a computed entry counts as an infinite error."""
    got = np.asarray(got, dtype=np.float64)
    mask = ~np.isnan(ref)
    if not mask.any():
        return 0.0
    diff = np.abs(got[mask] - ref[mask])
    if np.isnan(diff).any():
        return float("inf")
    return float(diff.max())
