"""Parallel sampling driven end to end by the host block manager.

Two prompts are prefilled, each forked into three samples ([bicarait]
"Berbagi Memori Fisik"); every decode step the manager hands out the new
tokens' slots and the copy-on-write pairs of shared partial blocks ([gininih]
"Cara kerja PagedAttention"), the GPU copies the blocks, writes the tokens
and attends through the manager's tables.  Checked at every step:

  * against the oracle run on the same slots, copies and tables: output
    within 2e-3, pools bit-exact (including never-written NaN slots);
  * against dense attention over each sample's own logical history (its
    prompt followed by its own tokens) -- independent of the manager, so a
    wrong table, slot or missing copy fails it;
  * the sharing the pages describe: the prompts' full blocks stay shared.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_188_amd as pa
import workloads as W
from oracle import paged_attention as O
from plan_oracle import max_abs_err
from workloads.device import to_device, to_host_bits

pytestmark = pytest.mark.gpu

BS, NB, HQ, HKV, D = 16, 96, 8, 2, 128
X = 8  # bf16 elements per 16-byte K granule


def _dense(q, ks, vs, scale):
    """Softmax attention of q [Hq][D] over logical rows ks, vs [n][Hkv][D]
    (float64), grouped-query heads."""
    g = HQ // HKV
    out = np.zeros((HQ, D))
    for h in range(HQ):
        kk, vv = ks[:, h // g, :], vs[:, h // g, :]
        s = float(np.float32(scale)) * (kk @ q[h])
        w = np.exp(s - s.max())
        out[h] = (w @ vv) / w.sum()
    return out


def test_parallel_sampling_through_the_block_manager():
    rng = np.random.default_rng(2024)
    bm = pa.BlockManager(NB, BS, 16, 24)
    kp = W.nan_pool((NB, HKV, D // X, BS, X), W.BF16)
    vp = W.nan_pool((NB, HKV, BS, D), W.BF16)
    kd, vd = to_device(kp, W.BF16), to_device(vp, W.BF16)
    scale = float(np.float32(1 / np.sqrt(D)))

    # prefill two prompts (100 and 37 tokens: both end in a partial block)
    prompts = [bm.add_sequence(), bm.add_sequence()]
    plen = [100, 37]
    slots, copies = bm.append(prompts, plen)
    assert copies.size == 0
    k_new = W.draw_normal(rng, (sum(plen), HKV, D), W.BF16)
    v_new = W.draw_normal(rng, (sum(plen), HKV, D), W.BF16)
    pa.write_kv(kd, vd, to_device(k_new, W.BF16), to_device(v_new, W.BF16),
                torch.from_numpy(slots).cuda())
    kp, vp = O.write_kv(kp, vp, k_new, v_new, slots)
    hist = {prompts[0]: (O.to_f64(k_new[:100], W.BF16), O.to_f64(v_new[:100], W.BF16)),
            prompts[1]: (O.to_f64(k_new[100:], W.BF16), O.to_f64(v_new[100:], W.BF16))}

    samples = []
    for p in prompts:
        kids = [bm.fork(p), bm.fork(p)]
        for c in kids:
            hist[c] = hist[p]
        samples += [p] + kids
    st = bm.stats()
    assert st["used_blocks"] == 7 + 3 and st["shared_blocks"] == 10

    total_copies = 0
    for step in range(20):
        slots, copies = bm.append(samples, [1] * len(samples))
        if step == 0:
            # each prompt's partial last block is copied for two of its three
            # samples; the third then owns it alone and writes in place
            assert copies.shape[0] == 4
        total_copies += copies.shape[0]
        if copies.size:
            pa.copy_blocks(kd, vd, torch.from_numpy(copies).cuda())
            kp, vp = O.copy_blocks(kp, vp, copies)
        kn = W.draw_normal(rng, (len(samples), HKV, D), W.BF16)
        vn = W.draw_normal(rng, (len(samples), HKV, D), W.BF16)
        pa.write_kv(kd, vd, to_device(kn, W.BF16), to_device(vn, W.BF16),
                    torch.from_numpy(slots).cuda())
        kp, vp = O.write_kv(kp, vp, kn, vn, slots)
        for j, s in enumerate(samples):
            hk, hv = hist[s]
            hist[s] = (np.concatenate([hk, O.to_f64(kn[j:j + 1], W.BF16)]),
                       np.concatenate([hv, O.to_f64(vn[j:j + 1], W.BF16)]))

        tables, lens = bm.tables(samples)
        q = W.draw_normal(rng, (len(samples), HQ, D), W.BF16)
        out = pa.decode_attention(to_device(q, W.BF16), kd, vd,
                                  torch.from_numpy(tables).cuda(),
                                  torch.from_numpy(lens).cuda(), scale,
                                  int(lens.max())).cpu().numpy()
        ref = O.decode_attention(q, kp, vp, tables, lens, scale, W.BF16)
        assert max_abs_err(out, ref) <= 2e-3
        q64 = O.to_f64(q, W.BF16)
        for j, s in enumerate(samples):
            hk, hv = hist[s]
            assert hk.shape[0] == lens[j]
            dense = _dense(q64[j], hk, hv, scale)
            assert np.abs(out[j] - dense).max() <= 2e-3, (step, s)

    assert total_copies == 4
    gk, gv = to_host_bits(kd, W.BF16), to_host_bits(vd, W.BF16)
    assert gk.tobytes() == kp.tobytes() and gv.tobytes() == vp.tobytes()
    st = bm.stats()
    # the prompts' full blocks (6 + 2) are still shared by three samples each
    assert st["shared_blocks"] == 8
    for s in samples:
        bm.free_sequence(s)
    assert bm.stats()["free_blocks"] == NB
