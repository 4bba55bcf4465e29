"""The oracle against its pins, plus planted-mistake (mutation) checks.

CPU only.  Every pin in ``oracle_pins`` must pass on the real oracle, and each
planted mistake below -- a dropped term, a wrong sign or index, a transposed
operand, swapped K/V -- must make at least one pin fail.
"""

import math
import types

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from oracle import paged_attention as real
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(real)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(num_seqs=st.integers(1, 3), hkv=st.integers(1, 2), grp=st.sampled_from([1, 2, 4]),
       d=st.integers(1, 5), bs=st.sampled_from([1, 2, 3, 4, 8, 16, 32, 64]),
       ctx_max=st.integers(0, 45), dtype=st.sampled_from(["f32", "bf16"]),
       seed=st.integers(0, 2**31 - 1), xsel=st.integers(0, 3))
def test_paged_equals_dense_any_block_size_and_permutation(num_seqs, hkv, grp, d, bs, ctx_max,
                                                           dtype, seed, xsel):
    """Invariant (a): paging changes placement only -- the oracle equals
    brute-force dense attention for any block size and any physical order."""
    rng = np.random.default_rng(seed)
    divisors = [x for x in range(1, d + 1) if d % x == 0]
    x = divisors[xsel % len(divisors)]
    c = P.random_case(rng, num_seqs=num_seqs, hq=hkv * grp, hkv=hkv, d=d, bs=bs,
                      ctx_max=ctx_max, dtype=dtype, x=x)
    scale = float(np.float32(1 / math.sqrt(d)))
    got = real.decode_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], scale, dtype)
    want = P.dense_attention_loops(c["q"], c["k_logical"], c["v_logical"], scale, dtype)
    assert np.max(np.abs(got - want), initial=0.0) <= 1e-12


def test_placement_invariance_bitwise():
    """Two different physical placements of the same logical data give
    bit-identical oracle outputs."""
    rng = np.random.default_rng(5)
    c = P.random_case(rng, num_seqs=3, hq=4, hkv=2, d=4, bs=4, ctx_max=30, dtype="bf16",
                      ctx=[30, 7, 12], x=2)
    rng2 = np.random.default_rng(6)
    nb = c["nb"] + 4
    perm = rng2.permutation(nb)
    t2 = np.full_like(c["tables"], -1)
    cur = 0
    for i, n in enumerate(c["ctx"]):
        k = -(-int(n) // 4)
        t2[i, :k] = perm[cur:cur + k]
        cur += k
    kp2, vp2 = P.build_pool(c["k_logical"], c["v_logical"], t2, nb, 4, "bf16", x=2)
    o1 = real.decode_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], 0.3, "bf16")
    o2 = real.decode_attention(c["q"], kp2, vp2, t2, c["ctx"], 0.3, "bf16")
    assert o1.tobytes() == o2.tobytes()


def test_zero_context_gives_zeros_and_unused_entries_never_read():
    rng = np.random.default_rng(8)
    c = P.random_case(rng, num_seqs=2, hq=2, hkv=1, d=3, bs=4, ctx_max=9, dtype="f32", ctx=[0, 5])
    out = real.decode_attention(c["q"], c["kp"], c["vp"], c["tables"], c["ctx"], 0.5, "f32")
    assert np.all(out[0] == 0) and np.all(np.isfinite(out[1]))


def test_contract_errors_raise():
    kp = np.zeros((4, 1, 1, 2, 1), np.float32)
    vp = np.zeros((4, 1, 2, 1), np.float32)
    with pytest.raises(oracle.paged_attention.ContractError):
        real.write_kv(kp, vp, np.zeros((2, 1, 1), np.float32), np.zeros((2, 1, 1), np.float32),
                      np.array([3, 3]))
    with pytest.raises(oracle.paged_attention.ContractError):
        real.write_kv(kp, vp, np.zeros((1, 1, 1), np.float32), np.zeros((1, 1, 1), np.float32),
                      np.array([8]))
    with pytest.raises(oracle.paged_attention.ContractError):
        real.write_kv(vp, vp, np.zeros((1, 1, 1), np.float32), np.zeros((1, 1, 1), np.float32),
                      np.array([1]))                                     # K pool not granular
    t = np.array([[0, -1]], np.int32)
    with pytest.raises(oracle.paged_attention.ContractError):
        real.slot_mapping(t, np.array([0]), np.array([2]), 2, 4)     # entry -1
    with pytest.raises(oracle.paged_attention.ContractError):
        real.slot_mapping(t, np.array([0]), np.array([4]), 2, 4)     # beyond the table
    with pytest.raises(oracle.paged_attention.ContractError):
        real.slot_mapping(t, np.array([1]), np.array([0]), 2, 4)     # no such sequence
    with pytest.raises(oracle.paged_attention.ContractError):
        kp2, vp2 = np.zeros((4, 2, 1, 2, 1), np.float32), np.zeros((4, 2, 2, 1), np.float32)
        real.decode_attention(np.zeros((1, 3, 1), np.float32), kp2, vp2, t, np.array([1]), 1.0, "f32")
    with pytest.raises(oracle.paged_attention.ContractError):
        real.decode_attention(np.zeros((1, 1, 1), np.float32), kp, vp, t, np.array([3]), 1.0, "f32")


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------

MUTATIONS = {
    "dropped-scale": ("s = scale64 * (k_t @ q64[i, h])", "s = (k_t @ q64[i, h])"),
    "wrong-sign-in-softmax": ("np.exp(s - s.max())", "np.exp(s.max() - s)"),
    "dropped-normalisation": ("(w @ v_t) / w.sum()", "(w @ v_t)"),
    "gqa-modulo-grouping": ("return q_head // group", "return q_head % group"),
    "reversed-offset": ("return p % block_size", "return block_size - 1 - p % block_size"),
    "swapped-block-and-offset": ("return p // block_size", "return p % block_size"),
    "context-off-by-one": ("t = np.arange(n)", "t = np.arange(max(n - 1, 1))"),
    "values-from-k-pool": ("v_t = to_f64(v_pool[phys, g, off, :], dtype)",
                           "v_t = to_f64(k_pool[phys, g, off, :], dtype)"),
    "transposed-operand": ("(w @ v_t) / w.sum()", "(w @ k_t) / w.sum()"),
    "bf16-shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "slot-no-offset": ("* block_size + _offset_in_block(p, block_size)", "* block_size"),
    "write-k-gets-v": ("= k_new[j].reshape(num_kv_heads, head_dim // x, x)",
                       "= v_new[j].reshape(num_kv_heads, head_dim // x, x)"),
    "write-swapped-divmod": ("b, o = divmod(int(s), block_size)", "o, b = divmod(int(s), block_size)"),
    "granule-order-swapped": ("return g.reshape(g.shape[0], -1)",
                              "return g.transpose(0, 2, 1).reshape(g.shape[0], -1)"),
    "write-granule-order-swapped": (
        "k_new[j].reshape(num_kv_heads, head_dim // x, x)",
        "k_new[j].reshape(num_kv_heads, x, head_dim // x).transpose(0, 2, 1)"),
    "copy-reversed": ("k_out[d] = k_pool[s]", "k_out[s] = k_pool[d]"),
    "scale-not-float32": ("np.float64(np.float32(scale))", "np.float64(scale) * 1.001"),
    "swap-reversed": ("k_out[d] = src_k[s]", "k_out[d] = src_k[d]"),
    "prefill-causal-off-by-one": ("t[None, :] <= pos[:, None]", "t[None, :] < pos[:, None]"),
    "prefill-chunk-at-start": ("pos = n - L + np.arange(L)", "pos = np.arange(L)"),
    "prefill-heads-interleaved": ("range(g * group, (g + 1) * group)",
                                  "range(g, num_q_heads, num_kv_heads)"),
    "prefill-no-causal-mask": ("visible = t[None, :] <= pos[:, None]",
                               "visible = np.ones((L, n), bool)"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    with open(real.__file__) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not in the oracle"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = real.__file__
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    m = _mutant(name)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(m)
        except Exception as e:  # noqa: BLE001 - any failure is a detection
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects the planted mistake {name!r}"
