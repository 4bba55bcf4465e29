"""GPU: the bandwidth probes read exactly the bytes they claim.

Each workgroup stores the XOR of the 32-bit words it loaded; the XOR of the
whole sink must equal the XOR, computed here with numpy, of every word of
the buffer (contiguous probe) or of every K/V chunk a decode over the same
pools, tables and context lengths reads (gather probe; a chunk that two
sequences share is read twice and cancels).  Bit-exact.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_188_amd as pa
import workloads as W

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _xor(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel(),
                                     initial=np.uint32(0)))


@pytest.mark.parametrize("nbytes,sink_len", [(16, 1), (4096 * 16 + 48, 7), (3 << 20, 2048)])
def test_probe_read_xor(nbytes, sink_len):
    _say(f"[case] probe_read bytes={nbytes} sink_len={sink_len}")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = pa.probe_read(buf, sink_len=sink_len).cpu().numpy()
    assert _xor(sink) == _xor(host)


def _expected_gather_xor(wl, kp, vp):
    """XOR of the K and V chunk words of every (sequence, KV head, logical
    block) a decode over the workload's step table reads."""
    table = wl.tables[[x for kind, x in wl.step if kind == "decode"][0]]
    nb, hkv = kp.shape[0], kp.shape[1]
    kc = kp.reshape(nb, hkv, -1).view(np.uint32)
    vc = vp.reshape(nb, hkv, -1).view(np.uint32)
    acc = 0
    for i, n in enumerate(wl.context_lens):
        if n <= 0:
            continue
        ids = table[i, : -(-int(n) // wl.block_size)]
        acc ^= _xor(kc[ids]) ^ _xor(vc[ids])
    return acc, table


@pytest.mark.parametrize("cid,sink_len", [(1, 3), (2, 512), (4, 2048), (5, 300)])
def test_probe_gather_xor(cid, sink_len):
    from workloads.device import DeviceWorkload
    wl = W.make(cid, small=(cid != 1))
    _say(f"[case] probe_gather {wl.name} sink_len={sink_len}")
    dev = DeviceWorkload(wl)
    dev.run_setup()
    k, v = dev.pools[0]
    kp, vp = dev.pool_bits()
    want, table = _expected_gather_xor(wl, kp, vp)
    bt = torch.from_numpy(np.ascontiguousarray(table)).cuda()
    sink = pa.probe_gather(k, v, bt, dev.ctx, sink_len=sink_len).cpu().numpy()
    assert _xor(sink) == want
