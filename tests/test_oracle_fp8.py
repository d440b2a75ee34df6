"""Pins for the oracle's fp8 (E4M3) KV cache against the format definition
and the mathematics (CPU only).

The reading (oracle/fp8.py; page "Tomas Koutsky explains how Meta fits
Muse Glimmer into 24 GB", runtimewire.com, "Narrow cache", names cache
quantisation without a format): OCP FP8 E4M3 codes, one fp32 scale per
(token, KV head) s = amax / 448, code = round-to-nearest-even of
clamp(x / s, +-448), fp32 divisions, amax = 0 -> s = 0 and zero codes.

None of these retypes the quantiser: the code table is checked against
values the E4M3 definition fixes, rounding against a brute-force nearest
search over all 254 finite codes, the quantiser against exact
representability, the rounding error bound, exact power-of-two rescaling
and sign symmetry, and attention over the dequantised cache against an
independent numpy brute force.  Planted mistakes in a copy of the module
(ties away from zero, truncation, a wrong maximum, a shifted subnormal
step, a lost sign, no clamp, a wrong exponent bias) are each caught.
Attention of a block of new bf16 tokens over the fp8 cache (verification)
is pinned by the same brute force on the concatenated stream, by a closed
form with a zero prior, and by the bf16 oracle on exactly held caches."""
import importlib.util
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth_inputs as si
from oracle import fp8 as fp8_mod

SRC = fp8_mod.__file__


# ----------------------------------------------------------------- pins

def pin_code_table(m):
    """Values the E4M3 definition fixes (sign, 4-bit exponent with bias 7,
    3-bit mantissa, subnormals, 0x7F / 0xFF NaN, largest finite 448)."""
    v = m.e4m3_value(np.arange(256, dtype=np.uint8))
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x09: 1.125 * 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
             0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for c, want in fixed.items():
        assert v[c] == want, (hex(c), v[c], want)
    assert np.signbit(v[0x80]) and v[0x80] == 0.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()          # codes 0..0x7E ascend
    assert np.array_equal(v[0x80:0xFF], -pos)


def pin_round_trip(m):
    codes = np.arange(256, dtype=np.uint8)
    v = m.e4m3_value(codes)
    fin = np.isfinite(v)
    assert np.array_equal(m.e4m3_round(v[fin]), codes[fin])


def _brute_round(y, table_codes, table_vals):
    """Nearest finite E4M3 value by search; ties to the even code; zero
    keeps the sign of y."""
    out = np.empty(y.shape, dtype=np.uint8)
    for i, t in enumerate(y):
        d = np.abs(table_vals - t)
        best = np.flatnonzero(d == d.min())
        cand = table_codes[best]
        if t == 0 or (cand & 0x7F).max() == 0:     # rounds to zero
            out[i] = 0x80 if np.signbit(t) else 0x00
            continue
        cand = cand[(cand >> 7) == (1 if t < 0 else 0)]
        even = cand[(cand & 1) == 0]
        out[i] = even[0] if len(even) else cand[0]
    return out


def pin_round_brute_force(m):
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8_mod.e4m3_value(codes)                 # the pinned table
    fin = np.isfinite(vals)
    tc, tv = codes[fin], vals[fin]
    rng = np.random.default_rng(11)
    pos = np.sort(tv[tv > 0])
    mids = 0.5 * (pos[1:] + pos[:-1])                # exact ties
    y = np.concatenate([
        rng.uniform(-448, 448, 400),
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448), 400)) *
        rng.choice([-1, 1], 400),
        mids, -mids, mids * (1 + 2.0 ** -30), mids * (1 - 2.0 ** -30),
        [0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -10, 3 * 2.0 ** -10,
         448.0, -448.0, 464.0 - 1e-6]])
    y = y[np.abs(y) <= 448]
    got = m.e4m3_round(y)
    want = _brute_round(y, tc, tv)
    bad = np.flatnonzero(got != want)
    assert len(bad) == 0, [(y[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def _bf16_rows(seed, n, hkv=2, d=128, scale=1.0):
    x = si.randn_bf16((n, hkv, d), seed=seed)
    if scale != 1.0:
        x = (x.float() * scale).to(x.dtype)
    return si.bits(x)


def _f(bits):
    return si.from_bits(bits).float().numpy().astype(np.float64)


def pin_quantise_properties(m):
    xb = np.concatenate([_bf16_rows(21, 64), _bf16_rows(22, 64, scale=1e-3),
                         _bf16_rows(23, 32, scale=300.0)])
    codes, scales = m.quantize(xb)
    x = _f(xb)
    deq = fp8_mod.dequantize(codes, scales)
    amax = np.abs(x).max(axis=-1)
    # rounding bound: half a step of the binade (relative 2^-4 for normals)
    # or half the subnormal step 2^-10 * s
    bound = np.abs(x) * 2.0 ** -4 + scales[..., None].astype(np.float64) * \
        2.0 ** -10 * (1 + 1e-6)
    assert (np.abs(deq - x) <= bound).all()
    # the largest magnitude maps to +-448 and comes back within fp32 rounding
    idx = np.abs(x).argmax(axis=-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0]
    assert ((top & 0x7F) == 0x7E).all()
    back = np.take_along_axis(deq, idx[..., None], -1)[..., 0]
    assert np.allclose(np.abs(back), amax, rtol=2.0 ** -21, atol=0)
    # scale within an ulp of amax / 448
    assert np.allclose(scales, amax / 448.0, rtol=2.0 ** -23, atol=0)
    # sign symmetry
    c2, s2 = m.quantize(xb ^ np.uint16(0x8000))
    assert np.array_equal(c2, codes ^ np.uint8(0x80))
    assert np.array_equal(s2, scales)
    # an exact power-of-two rescale leaves the codes unchanged
    for k in (-3, 5):
        xk = si.bits(si.from_bits(xb).float().mul(2.0 ** k).to(
            si.from_bits(xb).dtype))
        ck, sk = m.quantize(xk)
        assert np.array_equal(ck, codes)
        assert np.array_equal(sk, scales * np.float32(2.0 ** k))


def pin_exact_when_representable(m):
    """Rows of E4M3 values whose largest magnitude is 448: the scale is 1,
    every value is kept exactly."""
    rng = np.random.default_rng(31)
    table = fp8_mod.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    vals = rng.choice(table, size=(8, 2, 128)) * rng.choice([-1, 1],
                                                            (8, 2, 128))
    vals[:, :, 0] = 448.0
    xb = si.bits(__import__("torch").from_numpy(vals).to(
        __import__("torch").bfloat16))
    assert np.array_equal(_f(xb), vals)
    codes, scales = m.quantize(xb)
    assert (scales == 1.0).all()
    assert np.array_equal(fp8_mod.dequantize(codes, scales), vals)


def pin_zero_rows(m):
    xb = _bf16_rows(41, 4)
    xb[1, 0] = 0                      # +0 row in head 0
    xb[2, 1] = 0x8000                 # -0 row in head 1
    codes, scales = m.quantize(xb)
    assert scales[1, 0] == 0 and scales[2, 1] == 0
    assert not codes[1, 0].any() and not codes[2, 1].any()
    assert scales[1, 1] > 0 and scales[2, 0] > 0
    assert not fp8_mod.dequantize(codes, scales)[1, 0].any()


PINS = [pin_code_table, pin_round_trip, pin_round_brute_force,
        pin_quantise_properties, pin_exact_when_representable, pin_zero_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_pin(pin):
    pin(fp8_mod)


# ---------------------------------------------- attention over the cache

def _brute64(q, qpos, k, v, kpos0, hq, hkv, window, rope, theta=10000.0):
    """Masked softmax attention in fp64 on given float keys and values, with
    RoPE as complex multiplication."""
    def rot(x, pos):
        half = x.shape[-1] // 2
        freq = theta ** (-np.arange(half) / half)
        z = (x[..., :half] + 1j * x[..., half:]) * np.exp(
            1j * np.asarray(pos, dtype=np.float64)[..., None, None] * freq)
        return np.concatenate([z.real, z.imag], axis=-1)
    kpos = kpos0 + np.arange(k.shape[0])
    qpos = np.asarray(qpos)
    if rope:
        q, k = rot(q, qpos), rot(k, kpos)
    K = np.repeat(k, hq // hkv, axis=1)
    V = np.repeat(v, hq // hkv, axis=1)
    S = np.einsum("nhd,khd->hnk", q, K) / math.sqrt(q.shape[-1])
    mask = kpos[None, :] <= qpos[:, None]
    if window:
        mask &= kpos[None, :] > qpos[:, None] - window
    P = scipy.special.softmax(np.where(mask[None], S, -np.inf), axis=-1)
    return np.einsum("hnk,khd->nhd", P, V)


@pytest.mark.parametrize("window,rope", [(0, False), (8, True), (5, False)])
def test_attend_over_dequantised_cache_bruteforce(window, rope):
    hq, hkv, d, T = 8, 2, 16, 40
    kb = si.bits(si.randn_bf16((T, hkv, d), seed=51))
    vb = si.bits(si.randn_bf16((T, hkv, d), seed=52))
    qb = si.bits(si.randn_bf16((6, hq, d), seed=53))
    kc, ks = fp8_mod.quantize(kb, hkv, d)
    vc, vs = fp8_mod.quantize(vb, hkv, d)
    qpos = [0, 3, 17, 30, 38, 39]
    got = fp8_mod.attend(qb, qpos, kc, ks, vc, vs, 0, hq=hq, hkv=hkv, d=d,
                         window=window, rope=rope)
    want = _brute64(_f(qb), qpos, fp8_mod.dequantize(kc, ks),
                    fp8_mod.dequantize(vc, vs), 0, hq, hkv, window, rope)
    assert np.abs(got - want).max() < 1e-12


def test_attend_fp8_equals_bf16_attend_when_exact():
    """K and V made of E4M3 values times 2^-6 with largest magnitude
    448 * 2^-6 = 7 (scale exactly 2^-6) are kept exactly: the fp8 attention
    equals the bf16 attention on them."""
    import torch
    rng = np.random.default_rng(61)
    table = fp8_mod.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    T, hq, hkv, d = 64, 32, 2, 128
    kv = []
    for _ in range(2):
        vals = rng.choice(table, size=(T, hkv, d)) * \
            rng.choice([-1, 1], (T, hkv, d)) * 2.0 ** -6
        vals[:, :, 0] = 7.0
        kv.append(si.bits(torch.from_numpy(vals).to(torch.bfloat16)))
    qb = si.bits(si.randn_bf16((3, hq, d), seed=62))
    kc, ks = fp8_mod.quantize(kv[0])
    vc, vs = fp8_mod.quantize(kv[1])
    assert (ks == np.float32(2.0 ** -6)).all() and (vs == ks).all()
    for window, rope in ((0, False), (16, True)):
        a = fp8_mod.attend(qb, [10, 40, 63], kc, ks, vc, vs, 0, hq=hq,
                           hkv=hkv, d=d, window=window, rope=rope)
        b = oracle.attend(qb, [10, 40, 63], kv[0], kv[1], 0, hq=hq, hkv=hkv,
                          d=d, window=window, rope=rope)
        assert np.abs(a - b).max() < 1e-12


# ------------------------------------------------------- planted mistakes

MUTANTS = {
    "ties_away": ("q = np.rint(a / step).astype(np.int64)",
                  "q = np.floor(a / step + 0.5).astype(np.int64)"),
    "truncate": ("q = np.rint(a / step).astype(np.int64)",
                 "q = np.floor(a / step).astype(np.int64)"),
    "wrong_max": ("scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)",
                  "scale = (amax / np.float32(240.0)).astype(np.float32)"),
    "subnormal_step": ("_MIN_NORMAL_EXP = -6 ", "_MIN_NORMAL_EXP = -7 "),
    "sign_lost": ("code = (sign << 7) | (E << 3) | M",
                  "code = (E << 3) | M"),
    "no_clamp": ("y = np.minimum(np.maximum(y, np.float32(-E4M3_MAX)), "
                 "np.float32(E4M3_MAX))", "pass"),
    "exponent_bias": ("(1.0 + m / 8.0) * np.ldexp(1.0, e - 7)",
                      "(1.0 + m / 8.0) * np.ldexp(1.0, e - 8)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor moved: %s" % name
    path = tmp_path / ("fp8_%s.py" % name)
    path.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location("fp8_mutant_" + name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "no pin caught mutant %s" % name


# ------------------------- a block of new tokens over the cache (verify)

def _mixed_stream(seed, nc, n, hkv=2, d=16):
    """An fp8 prior stream of nc cached tokens (quantised from bf16 rows) and
    n new bf16 tokens."""
    kb = si.bits(si.randn_bf16((nc, hkv, d), seed=seed))
    vb = si.bits(si.randn_bf16((nc, hkv, d), seed=seed + 1))
    kn = si.bits(si.randn_bf16((n, hkv, d), seed=seed + 2))
    vn = si.bits(si.randn_bf16((n, hkv, d), seed=seed + 3))
    kc, ks = fp8_mod.quantize(kb, hkv, d)
    vc, vs = fp8_mod.quantize(vb, hkv, d)
    return kc, ks, vc, vs, kn, vn


@pytest.mark.parametrize("window,rope", [(0, False), (8, True), (5, False)])
def test_attend_mixed_bruteforce(window, rope):
    """Queries of a block at positions kpos0+nc .. against the dequantised
    prior then the block's own bf16 keys, causal inside the block: the numpy
    brute force on the concatenated float stream."""
    hq, hkv, d, nc, n = 8, 2, 16, 30, 6
    kpos0 = 4 if window else 0  # a global query needs every key from 0
    kc, ks, vc, vs, kn, vn = _mixed_stream(71, nc, n, hkv, d)
    qb = si.bits(si.randn_bf16((n, hq, d), seed=75))
    qpos = kpos0 + nc + np.arange(n)
    got = fp8_mod.attend_mixed(qb, qpos, kc, ks, vc, vs, kn, vn, kpos0, hq=hq,
                               hkv=hkv, d=d, window=window, rope=rope)
    k = np.concatenate([fp8_mod.dequantize(kc, ks), _f(kn)])
    v = np.concatenate([fp8_mod.dequantize(vc, vs), _f(vn)])
    want = _brute64(_f(qb), qpos, k, v, kpos0, hq, hkv, window, rope)
    assert np.abs(got - want).max() < 1e-12


def test_attend_mixed_block_enters_unquantised():
    """The block's rows are taken at their bf16 values: quantising them too
    changes the result, and the last query attends to its own key and value
    exactly as the brute force on bf16 block rows says."""
    hq, hkv, d, nc, n = 8, 2, 16, 20, 4
    kc, ks, vc, vs, kn, vn = _mixed_stream(81, nc, n, hkv, d)
    qb = si.bits(si.randn_bf16((n, hq, d), seed=85))
    qpos = nc + np.arange(n)
    got = fp8_mod.attend_mixed(qb, qpos, kc, ks, vc, vs, kn, vn, 0, hq=hq,
                               hkv=hkv, d=d, window=0, rope=False)
    knc, kns = fp8_mod.quantize(kn, hkv, d)
    vnc, vns = fp8_mod.quantize(vn, hkv, d)
    allq = fp8_mod.attend(qb, qpos, np.concatenate([kc, knc]),
                          np.concatenate([ks, kns]), np.concatenate([vc, vnc]),
                          np.concatenate([vs, vns]), 0, hq=hq, hkv=hkv, d=d,
                          window=0, rope=False)
    assert np.abs(got - allq).max() > 1e-4
    # with a prior of zero scales (zero keys and values) the first query
    # weighs its nc + 1 keys equally except its own, whose score is exact
    zs = np.zeros_like(ks)
    got0 = fp8_mod.attend_mixed(qb, qpos, kc, zs, vc, zs, kn, vn, 0, hq=hq,
                                hkv=hkv, d=d, window=0, rope=False)
    q0 = _f(qb)[0]
    g = np.repeat(np.arange(hkv), hq // hkv)
    s = (q0 * _f(kn)[0][g]).sum(-1) / math.sqrt(d)
    w = np.exp(s) / (nc + np.exp(s))
    assert np.abs(got0[0] - w[:, None] * _f(vn)[0][g]).max() < 1e-12


def test_attend_mixed_equals_bf16_attend_when_exact():
    """A prior made of E4M3 values times 2^-6 (largest 7, so scale 2^-6) is
    held exactly: the mixed attention equals the bf16 oracle's attention on
    the prior's bf16 values followed by the block."""
    import torch
    rng = np.random.default_rng(91)
    table = fp8_mod.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    nc, n, hq, hkv, d = 48, 16, 32, 2, 128
    prior = []
    for _ in range(2):
        vals = rng.choice(table, size=(nc, hkv, d)) * \
            rng.choice([-1, 1], (nc, hkv, d)) * 2.0 ** -6
        vals[:, :, 0] = 7.0
        prior.append(si.bits(torch.from_numpy(vals).to(torch.bfloat16)))
    kn = si.bits(si.randn_bf16((n, hkv, d), seed=92))
    vn = si.bits(si.randn_bf16((n, hkv, d), seed=93))
    qb = si.bits(si.randn_bf16((n, hq, d), seed=94))
    kc, ks = fp8_mod.quantize(prior[0])
    vc, vs = fp8_mod.quantize(prior[1])
    for window, rope in ((0, False), (16, True)):
        kpos0 = 100 if window else 0  # a global query needs every key from 0
        qpos = kpos0 + nc + np.arange(n)
        a = fp8_mod.attend_mixed(qb, qpos, kc, ks, vc, vs, kn, vn, kpos0,
                                 hq=hq, hkv=hkv, d=d, window=window, rope=rope)
        b = oracle.attend(qb, qpos, np.concatenate([prior[0], kn]),
                          np.concatenate([prior[1], vn]), kpos0, hq=hq,
                          hkv=hkv, d=d, window=window, rope=rope)
        assert np.abs(a - b).max() < 1e-12
