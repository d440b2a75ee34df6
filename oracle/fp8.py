"""fp8 KV cache in the oracle: quantiser, dequantiser and attention over the
dequantised cache.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Page: "Tomas Koutsky explains how Meta fits Muse Glimmer into 24 GB"
(runtimewire.com), "Narrow cache": cache quantisation is one of the things
that change how much memory the cache really takes.  The page names no
format; the reading taken here:

* codes are OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals, no infinities, 0x7F / 0xFF are NaN, largest
  finite value 448);
* one fp32 scale per (token, KV head), separately for K and V:
  s = amax / 448, amax = the largest magnitude among the head's 128 values;
* code_i = round-to-nearest-even to E4M3 of clamp(x_i / s, -448, 448);
* both divisions are fp32 operations rounded to nearest (the precision the
  GPU decides the codes in), the rounding to E4M3 is exact;
* amax = 0 gives s = 0 and all codes 0;
* the cache holds the codes and the scales; attention reads the dequantised
  values code_value * s exactly (fp64 here).
"""
from __future__ import annotations

import ctypes

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6        # smallest normal binade: [2^-6, 2^-5)
_MANT_BITS = 3


def e4m3_value(code):
    """Value of each E4M3 code (uint8), as float64; NaN for 0x7F / 0xFF."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS),
                   (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.where(sign == 1, -val, val)


def e4m3_round(y):
    """Codes of float values |y| <= 448, rounded to the nearest E4M3 value,
    ties to the even code.  A value rounding to zero keeps its sign."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if not (a <= E4M3_MAX).all():
        raise ValueError("e4m3_round takes |y| <= 448")
    sign = np.signbit(y).astype(np.int64)
    # the binade of a, with subnormals sharing the smallest normal's step
    _, ex = np.frexp(np.where(a > 0, a, 1.0))   # a = f 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, _MIN_NORMAL_EXP)
    step = np.ldexp(1.0, e - _MANT_BITS)       # spacing of the binade
    q = np.rint(a / step).astype(np.int64)     # exact quotient; ties to even
    up = q == 16                               # rounded into the next binade
    e = np.where(up, e + 1, e)
    q = np.where(up, 8, q)
    normal = q >= 8
    E = np.where(normal, e + 7, 0)
    M = np.where(normal, q - 8, q)
    code = (sign << 7) | (E << 3) | M
    code = np.where(a > 0, code, sign << 7)
    return code.astype(np.uint8)


def _as_f32_bf16(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def quantize(x_bits, hkv=2, d=128):
    """Quantise K or V rows: x_bits [n, hkv, d] bf16 bit patterns.
    Returns (codes uint8 [n, hkv, d], scales float32 [n, hkv])."""
    x = _as_f32_bf16(x_bits).reshape(-1, hkv, d)
    amax = np.max(np.abs(x), axis=-1)                        # exact
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)  # fp32 division
    nz = amax > 0
    div = np.where(nz, scale, np.float32(1.0)).astype(np.float32)
    y = (x / div[..., None]).astype(np.float32)               # fp32 division
    y = np.minimum(np.maximum(y, np.float32(-E4M3_MAX)), np.float32(E4M3_MAX))
    codes = e4m3_round(y)
    codes = np.where(nz[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize(codes, scales):
    """code value x scale, exactly (float64): codes [n, hkv, d], scales
    [n, hkv]."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def attend(q, qpos, k_codes, k_scales, v_codes, v_scales, kpos0, *, hq, hkv,
           d, window, rope, theta=10000.0, scale=None, nthreads=None):
    """Attention (as :func:`oracle.attend`) over a quantised K/V stream: row r
    of the codes / scales is position kpos0 + r.  The keys and values are the
    exact dequantised values."""
    return _attend64(q, qpos, dequantize(k_codes, k_scales),
                     dequantize(v_codes, v_scales), kpos0, hq=hq, hkv=hkv, d=d,
                     window=window, rope=rope, theta=theta, scale=scale,
                     nthreads=nthreads)


def attend_mixed(q, qpos, k_codes, k_scales, v_codes, v_scales, k_blk, v_blk,
                 kpos0, *, hq, hkv, d, window, rope, theta=10000.0, scale=None,
                 nthreads=None):
    """Attention of a block of new tokens over an fp8 cache (speculative
    verification, page "Deep dive into Muse Glimmer", shishifenxi.com,
    section 04: the main model checks a drafted block in one pass).  The
    stream's first rows are cached tokens, read as their exact dequantised
    values (codes / scales [nc, hkv, d] / [nc, hkv], positions kpos0 ..
    kpos0+nc-1); the block's own tokens follow (k_blk, v_blk bf16 bits
    [n, hkv, d] at positions kpos0+nc ..) and enter with their bf16 values:
    they arrive with the call and are not in the cache yet, so nothing has
    quantised them.  Queries q [nq, hq, d] at positions qpos."""
    kb = _as_f32_bf16(k_blk).reshape(-1, hkv, d).astype(np.float64)
    vb = _as_f32_bf16(v_blk).reshape(-1, hkv, d).astype(np.float64)
    k = np.concatenate([dequantize(k_codes, k_scales).reshape(-1, hkv, d), kb])
    v = np.concatenate([dequantize(v_codes, v_scales).reshape(-1, hkv, d), vb])
    return _attend64(q, qpos, k, v, kpos0, hq=hq, hkv=hkv, d=d, window=window,
                     rope=rope, theta=theta, scale=scale, nthreads=nthreads)


def _attend64(q, qpos, k, v, kpos0, *, hq, hkv, d, window, rope, theta,
              scale, nthreads):
    """The oracle's attention on float64 keys and values."""
    from oracle import _bits, _cfg, _load, _nthreads, _ptr, OracleRangeError
    q = _bits(q).reshape(-1, hq, d)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    qpos = np.ascontiguousarray(qpos, dtype=np.int64).reshape(-1)
    nq, nk = q.shape[0], k.shape[0]
    out = np.zeros((nq, hq, d), dtype=np.float64)
    cfg = _cfg(hq, hkv, d, window, rope, theta, scale)
    lib = _load()
    fn = lib.gqa_oracle_attend_kv64
    rc = fn(ctypes.byref(cfg), _ptr(q), _ptr(qpos), nq, _ptr(k), _ptr(v),
            int(kpos0), nk, _ptr(out), _nthreads(nthreads))
    if rc == -2:
        raise OracleRangeError("a query needs a key outside the given stream")
    if rc != 0:
        raise ValueError("oracle rejected its arguments (%d)" % rc)
    return out
