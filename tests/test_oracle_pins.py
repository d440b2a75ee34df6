"""Pins for the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each one checks it against a
printed figure (tests/golden/page_figures.json), an independent brute-force
formulation written here (full mask matrix, complex-number rotation, scipy
softmax), an identity of the definition (GQA as MHA with repeated KV heads,
window >= length equals full causal, rotation invariances), or a special case
whose answer is known in closed form (zero query -> window mean of V, constant
V, single key, needle)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synth_inputs as si

HERE = os.path.dirname(os.path.abspath(__file__))
GiB = float(1 << 30)
MiB = float(1 << 20)


def _figures():
    with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
        return {e["name"]: e for e in json.load(f)["figures"]}


def _close(value, fig):
    tol = fig["rel_tol"]
    return abs(value - fig["value"]) <= tol * abs(fig["value"]) + 1e-12


# ---------------------------------------------------------------- figures

def test_page_figures_bytes():
    F = _figures()
    assert oracle.kv_bytes_per_token_layer() == F["kv_bytes_per_token_layer"]["value"]
    g_all, l_all = oracle.kv_cache_bytes(all_global=True)
    assert l_all == 0
    assert _close(g_all / GiB, F["kv_all_global_131072"])
    assert g_all == 52 * 131072 * 1024
    g, l = oracle.kv_cache_bytes()
    assert _close(g / GiB, F["kv_hybrid_global_131072"])
    assert _close(l / MiB, F["kv_hybrid_local_filled"])
    assert _close((g + l) / GiB, F["kv_hybrid_total_131072"])


def test_page_figures_mha_ratio():
    F = _figures()
    gqa = oracle.kv_bytes_per_token_layer(hkv=2)
    mha = oracle.kv_bytes_per_token_layer(hkv=32)
    assert mha // gqa == F["mha_over_gqa_ratio"]["value"]
    g, l = oracle.kv_cache_bytes(hkv=32)
    assert (g + l) / GiB > F["mha_hybrid_total_min"]["value"]


def test_page_figures_pairs_and_schedule():
    F = _figures()
    dense = oracle.pair_count(131072, causal=False)
    assert _close(dense, F["dense_pairs_per_layer_131072"])
    kinds = [oracle.layer_kind(l) for l in range(52)]
    assert kinds.count(oracle.LOCAL) == F["n_local_layers"]["value"]
    assert kinds.count(oracle.GLOBAL) == F["n_global_layers"]["value"]
    assert kinds[:8] == [0, 0, 0, 1, 0, 0, 0, 1]


def test_pair_count_small_bruteforce():
    for T in (1, 5, 17):
        for W in (0, 1, 3, 8):
            want = sum(1 for i in range(T) for j in range(T)
                       if j <= i and (W == 0 or j > i - W))
            assert oracle.pair_count(T, window=W) == want


# ---------------------------------------------------------------- brute force

def _widen(bits):
    return si.from_bits(bits).float().numpy().astype(np.float64)


def _rot_complex(x, pos, theta):
    """RoPE written as complex multiplication of (x_c + i x_{c+d/2})."""
    d = x.shape[-1]
    half = d // 2
    freq = theta ** (-np.arange(half) / half)
    z = x[..., :half] + 1j * x[..., half:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None, None] * freq)
    return np.concatenate([z.real, z.imag], axis=-1)


def brute(qb, qpos, kb, vb, kpos0, hq, hkv, window, rope, theta=10000.0):
    q = _widen(qb)
    k = _widen(kb)
    v = _widen(vb)
    nk = k.shape[0]
    kpos = kpos0 + np.arange(nk)
    qpos = np.asarray(qpos)
    if rope:
        q = _rot_complex(q, qpos, theta)
        k = _rot_complex(k, kpos, theta)
    rep = hq // hkv
    K = np.repeat(k, rep, axis=1)   # [nk, hq, d]
    V = np.repeat(v, rep, axis=1)
    S = np.einsum("nhd,khd->hnk", q, K) / math.sqrt(q.shape[-1])
    mask = kpos[None, :] <= qpos[:, None]
    if window:
        mask &= kpos[None, :] > qpos[:, None] - window
    S = np.where(mask[None], S, -np.inf)
    P = scipy.special.softmax(S, axis=-1)
    return np.einsum("hnk,khd->nhd", P, V)


CASES = [
    # hq, hkv, d, T, window, rope
    (4, 2, 8, 23, 0, False),
    (4, 2, 8, 23, 5, True),
    (6, 3, 16, 40, 8, True),
    (8, 2, 4, 64, 4, True),
    (8, 1, 12, 33, 0, False),
    (2, 2, 6, 9, 3, False),
]


@pytest.mark.parametrize("hq,hkv,d,T,window,rope", CASES)
def test_bruteforce_tiny(hq, hkv, d, T, window, rope):
    seed = 100 + hq * 7 + T
    g = si.gen(seed)
    kb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((T, hq, d), generator=g))
    qpos = np.arange(T)
    got = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d,
                        window=window, rope=rope)
    want = brute(qb, qpos, kb, vb, 0, hq, hkv, window, rope)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_bruteforce_offset_stream_and_sparse_queries():
    hq, hkv, d, W = 8, 2, 16, 6
    g = si.gen(7)
    kb = si.bits(si.randn_bf16((30, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((30, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((4, hq, d), generator=g))
    kpos0 = 100
    qpos = np.array([105, 110, 129, 120])
    got = oracle.attend(qb, qpos, kb, vb, kpos0, hq=hq, hkv=hkv, d=d,
                        window=W, rope=True)
    want = brute(qb, qpos, kb, vb, kpos0, hq, hkv, W, True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    with pytest.raises(oracle.OracleRangeError):
        oracle.attend(qb[:1], np.array([102]), kb, vb, kpos0, hq=hq, hkv=hkv,
                      d=d, window=W, rope=True)  # needs positions < 100


# ---------------------------------------------------------------- identities

def test_gqa_equals_mha_with_repeated_kv():
    hq, hkv, d, T = 32, 2, 128, 40
    g = si.gen(11)
    k = si.randn_bf16((T, hkv, d), generator=g)
    v = si.randn_bf16((T, hkv, d), generator=g)
    q = si.randn_bf16((T, hq, d), generator=g)
    qpos = np.arange(T)
    for window, rope in ((0, False), (16, True)):
        a = oracle.attend(si.bits(q), qpos, si.bits(k), si.bits(v), 0, hq=hq,
                          hkv=hkv, d=d, window=window, rope=rope)
        kk = k.repeat_interleave(hq // hkv, dim=1)
        vv = v.repeat_interleave(hq // hkv, dim=1)
        b = oracle.attend(si.bits(q), qpos, si.bits(kk), si.bits(vv), 0,
                          hq=hq, hkv=hq, d=d, window=window, rope=rope)
        np.testing.assert_array_equal(a, b)


def test_window_at_least_length_equals_global():
    hq, hkv, d, T = 32, 2, 128, 50
    g = si.gen(12)
    kb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((T, hq, d), generator=g))
    qpos = np.arange(T)
    glob = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d, window=0,
                         rope=False)
    for W in (T, T + 1, 2048):
        loc = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d,
                            window=W, rope=False)
        np.testing.assert_array_equal(glob, loc)
    smaller = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d,
                            window=T - 1, rope=False)
    assert np.abs(smaller[-1] - glob[-1]).max() > 1e-6  # the edge matters


def test_rope_identity_norm_and_relative():
    g = si.gen(13)
    x = si.randn_bf16((5, 128), generator=g).double().numpy()
    np.testing.assert_array_equal(oracle.rope(x, 0.0), x)         # R_0 = I
    for t in (1.0, 2047.0, 131071.0):
        y = oracle.rope(x, t)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1),
                                   np.linalg.norm(x, axis=-1), rtol=1e-13)
        np.testing.assert_allclose(y, _rot_complex(x, np.float64(t), 10000.0)[0]
                                   if y.ndim == 1 else
                                   _rot_complex(x[None], np.array([t]), 10000.0)[0],
                                   rtol=0, atol=1e-9)
    # <R_i a, R_j b> depends on i - j only
    a, b = x[0], x[1]
    base = np.dot(oracle.rope(a, 7.0), oracle.rope(b, 3.0))
    for c in (0.0, 100.0, 2048.0, 131000.0):
        np.testing.assert_allclose(
            np.dot(oracle.rope(a, 7.0 + c), oracle.rope(b, 3.0 + c)), base,
            rtol=0, atol=1e-9)


def test_position_shift_invariance_local():
    hq, hkv, d, W, T = 32, 2, 128, 16, 48
    g = si.gen(14)
    kb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((8, hq, d), generator=g))
    qpos = np.arange(T - 8, T)
    a = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d, window=W,
                      rope=True)
    for c in (5, 2048, 131024 - T):
        b = oracle.attend(qb, qpos + c, kb, vb, c, hq=hq, hkv=hkv, d=d,
                          window=W, rope=True)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-10)


# ---------------------------------------------------------------- special cases

@pytest.mark.parametrize("window,rope", [(0, False), (8, True), (2048, True)])
def test_zero_query_gives_window_mean(window, rope):
    hq, hkv, d, T = 32, 2, 128, 64
    g = si.gen(15)
    kb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    qb = si.bits(si.zeros_bf16((T, hq, d)))
    qpos = np.arange(T)
    got = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d,
                        window=window, rope=rope)
    V = _widen(vb)
    for i in (0, 1, 7, 8, 9, 63):
        lo = 0 if window == 0 else max(0, i - window + 1)
        mean = V[lo:i + 1].mean(axis=0)          # [hkv, d]
        for h in range(hq):
            np.testing.assert_allclose(got[i, h], mean[h // (hq // hkv)],
                                       rtol=0, atol=1e-12)


def test_constant_v_and_single_key():
    hq, hkv, d, T = 32, 2, 128, 30
    g = si.gen(16)
    kb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((T, hq, d), generator=g))
    vb = si.bits(si.constant_bf16((T, hkv, d), -1.25))
    got = oracle.attend(qb, np.arange(T), kb, vb, 0, hq=hq, hkv=hkv, d=d,
                        window=4, rope=True)
    np.testing.assert_allclose(got, -1.25, rtol=0, atol=1e-13)
    vb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    one = oracle.attend(qb[:1], [0], kb, vb, 0, hq=hq, hkv=hkv, d=d,
                        window=0, rope=False)
    V = _widen(vb)
    for h in range(hq):
        np.testing.assert_array_equal(one[0, h], V[0, h // 16])
    # a window of one sees only itself
    w1 = oracle.attend(qb, np.arange(T), kb, vb, 0, hq=hq, hkv=hkv, d=d,
                       window=1, rope=True)
    for h in range(hq):
        np.testing.assert_allclose(w1[:, h], V[:, h // 16], rtol=0, atol=1e-13)


def test_needle_retrieval():
    T = 300
    needles = [0, 127, 128, 255, 299]
    k, v, u = si.needle_stream(17, T, needles, direction_seed=18,
                               magnitude=16.0)
    hq = 32
    q = u.float().repeat_interleave(16, dim=0)[None].repeat(len(needles), 1, 1)
    q = (q * 8.0).to(k.dtype)
    # each query sits right at its needle; the window is 1 position wide
    # around nothing else, so the needle dominates through its score.
    got = oracle.attend(si.bits(q), needles, si.bits(k), si.bits(v), 0, hq=hq,
                        hkv=2, d=128, window=0, rope=False)
    V = _widen(si.bits(v))
    for n, p in enumerate(needles):
        # the latest needle at or before p wins (all needles score equally)
        earlier = [x for x in needles if x <= p]
        want = V[earlier].mean(axis=0)
        for h in range(hq):
            np.testing.assert_allclose(got[n, h], want[h // 16], rtol=0,
                                       atol=1e-3)


# ---------------------------------------------------------------- merge

def test_split_merge_identity():
    hq, hkv, d, T = 32, 2, 128, 200
    g = si.gen(19)
    kb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((T, hkv, d), generator=g))
    qb = si.bits(si.randn_bf16((3, hq, d), generator=g))
    qpos = np.array([199, 150, 64])
    for window, rope in ((0, False), (64, True)):
        full = oracle.attend(qb, qpos, kb, vb, 0, hq=hq, hkv=hkv, d=d,
                             window=window, rope=rope)
        for cuts in ([0, 200], [0, 1, 2, 200], [0, 37, 64, 65, 128, 199, 200],
                     [0, 100, 200]):
            parts = [oracle.partial(qb, qpos, kb, vb, 0, a, b, hq=hq, hkv=hkv,
                                    d=d, window=window, rope=rope)
                     for a, b in zip(cuts[:-1], cuts[1:])]
            np.testing.assert_allclose(oracle.merge(parts), full, rtol=0,
                                       atol=1e-13)


# ---------------------------------------------------------------- cache

def test_cache_oracle_global_identity_and_ring_latest():
    hkv, d, W = 2, 4, 8
    P = 45
    g = si.gen(20)
    kb = si.bits(si.randn_bf16((P, hkv, d), generator=g))
    vb = si.bits(si.randn_bf16((P, hkv, d), generator=g))
    Kg, Vg = oracle.expected_cache(oracle.GLOBAL, 64, [(0, 0, kb, vb)],
                                   hkv=hkv, d=d)
    np.testing.assert_array_equal(Kg[0, :P], kb)
    assert (Kg[0, P:] == 0xFFFF).all()
    Kl, Vl = oracle.expected_cache(oracle.LOCAL, W, [(0, 0, kb[:20], vb[:20]),
                                                     (0, 20, kb[20:], vb[20:])],
                                   window=W, hkv=hkv, d=d)
    for s in range(W):
        latest = (P - 1) - ((P - 1 - s) % W)      # largest p < P with p = s mod W
        np.testing.assert_array_equal(Kl[0, s], kb[latest])
        np.testing.assert_array_equal(Vl[0, s], vb[latest])
    # a short stream leaves the slots it never reached untouched
    Ks, _ = oracle.expected_cache(oracle.LOCAL, W, [(0, 0, kb[:3], vb[:3])],
                                  window=W, hkv=hkv, d=d)
    assert (Ks[0, 3:] == 0xFFFF).all()
