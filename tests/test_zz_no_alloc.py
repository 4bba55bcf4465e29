"""pa_decode_attention_noalloc against the entry points it stands in for.

The allocation-free call keeps its partials in the library's static device
array instead of a caller workspace; everything else is the same code, so
its outputs and pools must equal those of pa_decode_attention_append (and of
pa_decode_attention without new rows) bit for bit, and the oracle within the
attention tolerance.  Two calls in a row, the second on a smaller batch, so
the second must not depend on what the first left in the shared array.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from plan_oracle import max_abs_err, run_oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _one(wl, partition, append):
    import paged_kv_cache_188_amd as pa
    from workloads.device import DeviceWorkload
    _say(f"[case] noalloc {wl.name} partition={partition} append={append}")
    dev = DeviceWorkload(wl)
    dev.run_setup()
    dev.add_pool_copies(1)
    op = [x for kind, x in dev.step_ops_append if kind == "decode_append"][0]
    table = dev.tables[op["table"]]
    part = wl.partition_size if partition is None else partition
    kw = dict(k_new=op["k"], v_new=op["v"]) if append else {}
    if not append:  # the new tokens stored first, as the plain decode expects
        for p in (0, 1):
            k, v = dev.pools[p]
            w = op["write"]
            pa.write_kv_at(k, v, w["k"], w["v"], table, w["positions"], seq_ids=w["seq_ids"])
    k0, v0 = dev.pools[0]
    ref = pa.decode_attention(dev.q, k0, v0, table, dev.ctx, wl.scale, dev.max_ctx,
                              partition_size=part, **kw)
    k1, v1 = dev.pools[1]
    got = pa.decode_attention_noalloc(dev.q, k1, v1, table, dev.ctx, wl.scale, dev.max_ctx,
                                      partition_size=part, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), "output differs"
    assert torch.equal(k0.view(torch.int16), k1.view(torch.int16)), "K pool differs"
    assert torch.equal(v0.view(torch.int16), v1.view(torch.int16)), "V pool differs"
    _, _, oref, _ = run_oracle(wl, wl.setup + wl.step)
    err = max_abs_err(got.cpu().numpy(), oref)
    _say(f"  max_abs_err={err:.3e}")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("partition,append", [(None, True), (None, False), (256, True)])
def test_noalloc_matches_workspace_call_twice(partition, append):
    big = W.make(2)                  # 64 sequences, contexts up to 4096
    small = W.make(3, small=True)    # then 12 sequences, shorter contexts
    assert small.num_seqs < big.num_seqs
    _one(big, partition, append)
    _one(small, partition, append)


def test_noalloc_refuses_a_workspace_beyond_its_array():
    import paged_kv_cache_188_amd as pa
    wl = W.make(3, small=True)
    from workloads.device import DeviceWorkload
    dev = DeviceWorkload(wl)
    # fixed partitions of 16 tokens over a declared 1M-token context: far
    # more partials than the static array holds
    need = pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                    wl.block_size, 1 << 20, 16, dev.torch_dtype)
    assert need > pa.PA_NOALLOC_MAX_WORKSPACE
    k, v = dev.pools[0]
    with pytest.raises(pa.PAError, match="WORKSPACE"):
        pa.decode_attention_noalloc(dev.q, k, v, dev.tables["final"], dev.ctx, wl.scale,
                                    1 << 20, partition_size=16)
