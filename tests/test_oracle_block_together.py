"""Pins of the oracle's attention for a block whose tokens are predicted
together (a block-diffusion drafter's step: page "Deep dive into Muse
Glimmer", shishifenxi.com, section 04).  Every query of the block at
positions p0 .. p0+n-1 sees the context 0 .. p0-1 and the whole block.

The pins do not repeat the oracle's reduction to the causal routine:
* a materialised mask (every block row sees keys 0 .. p0+n-1, nothing past
  the block) in an independent numpy softmax, on a stream that also holds
  positions after the block;
* reordering the block's keys and values together leaves every output
  unchanged (a causal mask inside the block would not);
* a needle at the block's last position is found by the block's first query.
Planted mistakes in a copy of the function (a causal mask inside the block,
the last visible position off by one either way) must each fail a pin."""
import inspect
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth_inputs as si


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _masked_softmax_attention(qb, kb, vb, mask, hq, hkv):
    q, k, v = _widen(qb), _widen(kb), _widen(vb)
    K = np.repeat(k, hq // hkv, axis=1)
    V = np.repeat(v, hq // hkv, axis=1)
    S = np.einsum("nhd,khd->hnk", q, K) / math.sqrt(q.shape[-1])
    S = np.where(mask[None], S, -np.inf)
    return np.einsum("hnk,khd->nhd", scipy.special.softmax(S, axis=-1), V)


def pin_bruteforce(fn):
    hq, hkv, d = 4, 2, 8
    for p0, n, total in ((20, 5, 31), (0, 3, 9), (7, 1, 12), (40, 16, 64)):
        g = si.gen(300 + p0 + n)
        kb = si.bits(si.randn_bf16((total, hkv, d), generator=g))
        vb = si.bits(si.randn_bf16((total, hkv, d), generator=g))
        qb = si.bits(si.randn_bf16((n, hq, d), generator=g))
        mask = np.zeros((n, total), dtype=bool)
        mask[:, :p0 + n] = True   # context and whole block, nothing after
        want = _masked_softmax_attention(qb, kb, vb, mask, hq, hkv)
        got = fn(qb, p0, kb, vb, 0, hq=hq, hkv=hkv, d=d)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_block_order_free(fn):
    hq, hkv, d, p0, n = 8, 2, 16, 33, 7
    g = si.gen(311)
    kb = si.bits(si.randn_bf16((p0 + n + 4, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((p0 + n + 4, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((n, hq, d), generator=g))
    base = fn(qb, p0, kb, vb, 0, hq=hq, hkv=hkv, d=d)
    perm = np.random.default_rng(5).permutation(n)
    assert (perm != np.arange(n)).any()
    kp, vp = kb.copy(), vb.copy()
    kp[p0:p0 + n] = kb[p0 + perm]
    vp[p0:p0 + n] = vb[p0 + perm]
    got = fn(qb, p0, kp, vp, 0, hq=hq, hkv=hkv, d=d)
    np.testing.assert_allclose(got, base, rtol=0, atol=1e-13)


def pin_needle_at_block_end(fn):
    p0, n = 100, 16
    k, v, u = si.needle_stream(17, p0 + n, [p0 + n - 1], direction_seed=18,
                               magnitude=16.0)
    q = (u.float().repeat_interleave(16, dim=0) * 8.0)
    q = q[None].repeat(n, 1, 1).to(k.dtype)
    got = fn(si.bits(q), p0, si.bits(k), si.bits(v), 0, hq=32, hkv=2, d=128)
    V = _widen(si.bits(v))
    for h in range(32):   # query 0 already sees the block's last key
        np.testing.assert_allclose(got[0, h], V[p0 + n - 1, h // 16],
                                   rtol=0, atol=1e-3)


PINS = [pin_bruteforce, pin_block_order_free, pin_needle_at_block_end]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attend_block_together)


def test_causal_inside_block_would_differ():
    """The order-free pin is sensitive: the causal oracle changes when the
    block is reordered."""
    hq, hkv, d, p0, n = 8, 2, 16, 33, 7
    g = si.gen(311)
    kb = si.bits(si.randn_bf16((p0 + n, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((p0 + n, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((n, hq, d), generator=g))
    qpos = p0 + np.arange(n)
    base = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d, window=0,
                         rope=False)
    kp, vp = kb.copy(), vb.copy()
    kp[p0:] = kb[p0:][::-1]
    vp[p0:] = vb[p0:][::-1]
    got = oracle.attend(qb, qpos, kp, vp, 0, hq=hq, hkv=hkv, d=d, window=0,
                        rope=False)
    assert np.abs(got - base).max() > 1e-3


MUTANTS = {
    "causal_inside_block": (
        "see = np.full(n, int(pos0) + n - 1, dtype=np.int64)",
        "see = int(pos0) + np.arange(n, dtype=np.int64)"),
    "last_key_dropped": ("int(pos0) + n - 1", "int(pos0) + n - 2"),
    "key_after_block": ("int(pos0) + n - 1", "int(pos0) + n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(oracle.attend_block_together)
    assert src.count(old) == 1, "mutation anchor moved: %s" % name
    ns = dict(vars(oracle))
    exec(src.replace(old, new), ns)
    mutant = ns["attend_block_together"]
    caught = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleRangeError):
            caught += 1
    assert caught, "no pin caught mutant %s" % name
