"""Plain fp64 CPU oracle for the hybrid local/global GQA attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never loads it, and it shares no code with the HIP path (the only
common module is the seeded input generator, which holds none of the method's
arithmetic).

What it defines, each cited by page and section:

* :func:`attend` / :func:`partial` -- the attention itself, in C
  (``gqa_oracle.c``), fp64, over a logical position-indexed K/V stream.
  Page "Deep dive into Muse Glimmer" (shishifenxi.com) section 01 and page
  "Tomas Koutsky explains how Meta fits Muse Glimmer into 24 GB"
  (runtimewire.com) sections "Narrow cache" and "Long context still costs
  compute".
* :func:`merge` -- recombining partial sums over disjoint key sets (the
  log-sum-exp identity; the pages only require that the result is the plain
  one, "memory-efficient kernels" in "Long context still costs compute").
* :func:`attend_block_together` -- a block of tokens predicted together
  (block-diffusion drafting, section 04 of the shishifenxi.com page): every
  query of the block sees the context and the whole block.
* :mod:`oracle.fp8` -- an fp8 (E4M3) cache with one scale per token and KV
  head: the quantiser, the dequantised values and attention over them
  ("Narrow cache": cache quantisation changes the measured cache use).
* :func:`expected_cache` -- integer-only cache contents after a sequence of
  appends: global slot = position, local slot = position mod window, latest
  write wins ("Narrow cache": the engine must evict or cyclically reuse stale
  sliding-window entries).
* :func:`layer_kind`, :func:`kv_bytes_per_token_layer`, :func:`kv_cache_bytes`,
  :func:`pair_count` -- the schedule and the byte / pair counts the pages print
  (section 01 of the shishifenxi.com page; "Narrow cache"; "Trick 2: hybrid
  attention" on the kongchang.com page "Meta open-sources the 30B Muse
  Glimmer").
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgqa_oracle.so")
_lock = threading.Lock()
_lib = None

GLOBAL = 1
LOCAL = 0


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc into ``oracle/libgqa_oracle.so``."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("theta", ctypes.c_double), ("scale", ctypes.c_double)]


def _configure(lib):
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.gqa_oracle_attend.argtypes = [ctypes.POINTER(_Cfg), p, p, i64,
                                      p, p, i64, i64, p, ctypes.c_int32]
    lib.gqa_oracle_attend.restype = ctypes.c_int
    lib.gqa_oracle_partial.argtypes = [ctypes.POINTER(_Cfg), p, p, i64,
                                       p, p, i64, i64, i64, i64, p, p,
                                       p, ctypes.c_int32]
    lib.gqa_oracle_partial.restype = ctypes.c_int
    lib.gqa_oracle_attend_kv64.argtypes = [ctypes.POINTER(_Cfg), p, p, i64,
                                           p, p, i64, i64, p, ctypes.c_int32]
    lib.gqa_oracle_attend_kv64.restype = ctypes.c_int
    lib.gqa_oracle_rope.argtypes = [p, ctypes.c_int32, ctypes.c_double,
                                    ctypes.c_double, p]
    lib.gqa_oracle_rope.restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call through another build of the
    same source (used by the tests that plant mistakes in the oracle)."""
    global _lib
    old = _load()
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = old


def _nthreads(n):
    if n:
        return int(n)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def _cfg(hq, hkv, d, window, rope, theta, scale):
    return _Cfg(hq, hkv, d, window, 1 if rope else 0, 0, float(theta),
                float(scale if scale is not None else 1.0 / math.sqrt(d)))


def _bits(x):
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        a = a.view(np.uint16) if a.dtype.itemsize == 2 else a.astype(np.uint16)
    return a


class OracleRangeError(ValueError):
    pass


def attend(q, qpos, k, v, kpos0, *, hq, hkv, d, window, rope, theta=10000.0,
           scale=None, nthreads=None):
    """Attention outputs in fp64.

    q: [nq, hq, d] bf16 bits (uint16); qpos: [nq] positions;
    k, v: [nk, hkv, d] bf16 bits, row r is position kpos0 + r.
    window: 0 for full causal, W > 0 for a W-token window including self.
    rope: rotate q at its position and k at its position (local layers).
    Returns float64 [nq, hq, d]."""
    q = _bits(q).reshape(-1, hq, d)
    k = _bits(k).reshape(-1, hkv, d)
    v = _bits(v).reshape(-1, hkv, d)
    qpos = np.ascontiguousarray(qpos, dtype=np.int64).reshape(-1)
    nq, nk = q.shape[0], k.shape[0]
    assert qpos.shape[0] == nq and v.shape[0] == nk
    out = np.zeros((nq, hq, d), dtype=np.float64)
    cfg = _cfg(hq, hkv, d, window, rope, theta, scale)
    rc = _load().gqa_oracle_attend(ctypes.byref(cfg), _ptr(q), _ptr(qpos), nq,
                                   _ptr(k), _ptr(v), int(kpos0), nk, _ptr(out),
                                   _nthreads(nthreads))
    if rc == -2:
        raise OracleRangeError("a query needs a key outside the given stream")
    if rc != 0:
        raise ValueError("oracle rejected its arguments (%d)" % rc)
    return out


def partial(q, qpos, k, v, kpos0, jlo, jhi, *, hq, hkv, d, window, rope,
            theta=10000.0, scale=None, nthreads=None):
    """Unnormalised sums over the visible keys with position in [jlo, jhi).

    Returns (m [nq,hq], l [nq,hq], o [nq,hq,d]) with o = sum e^(s-m) v."""
    q = _bits(q).reshape(-1, hq, d)
    k = _bits(k).reshape(-1, hkv, d)
    v = _bits(v).reshape(-1, hkv, d)
    qpos = np.ascontiguousarray(qpos, dtype=np.int64).reshape(-1)
    nq, nk = q.shape[0], k.shape[0]
    m = np.zeros((nq, hq), dtype=np.float64)
    l = np.zeros((nq, hq), dtype=np.float64)
    o = np.zeros((nq, hq, d), dtype=np.float64)
    cfg = _cfg(hq, hkv, d, window, rope, theta, scale)
    rc = _load().gqa_oracle_partial(ctypes.byref(cfg), _ptr(q), _ptr(qpos), nq,
                                    _ptr(k), _ptr(v), int(kpos0), nk, int(jlo),
                                    int(jhi), _ptr(m), _ptr(l), _ptr(o),
                                    _nthreads(nthreads))
    if rc == -2:
        raise OracleRangeError("a query needs a key outside the given stream")
    if rc != 0:
        raise ValueError("oracle rejected its arguments (%d)" % rc)
    return m, l, o


def merge(parts):
    """Combine partial sums over disjoint key sets: with M = max_s m_s,
    o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s."""
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    Msafe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - Msafe[None]), 0.0)
    L = sum(w[i] * parts[i][1] for i in range(len(parts)))
    O = sum(w[i][..., None] * parts[i][2] for i in range(len(parts)))
    return O / L[..., None]


def attend_block_together(q, pos0, k, v, kpos0, *, hq, hkv, d, nthreads=None):
    """Attention of a block of n tokens at positions pos0 .. pos0+n-1 that are
    predicted together, as in a block-diffusion drafter's step (page "Deep
    dive into Muse Glimmer", shishifenxi.com, section 04: the drafter
    predicts a 16-token block in parallel rather than token by token, and the
    target's hidden features from five layers enter every drafter layer's
    keys and values).  With no order inside the block, every query of the
    block sees every key at positions 0 .. pos0+n-1: the context before the
    block and the whole block.  Only for layers without RoPE and without a
    window (the pages give the drafter neither).

    On such a layer a query's position enters the result only through its
    visible set, and the set {j <= pos0+n-1} is the causal set of position
    pos0+n-1; so each row is the plain attention of that query placed at the
    block's last position, which :func:`attend` computes.

    q: [n, hq, d] bf16 bits; k, v: [nk, hkv, d] bf16 bits, row r at position
    kpos0 + r, covering 0 .. pos0+n-1.  Returns float64 [n, hq, d]."""
    q = _bits(q).reshape(-1, hq, d)
    n = q.shape[0]
    see = np.full(n, int(pos0) + n - 1, dtype=np.int64)
    return attend(q, see, k, v, kpos0, hq=hq, hkv=hkv, d=d, window=0,
                  rope=False, nthreads=nthreads)


def rope(x, t, theta=10000.0):
    """Rotate the head vectors x[..., d] (float64) by position t."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    out = np.empty_like(flat)
    lib = _load()
    for r in range(flat.shape[0]):
        lib.gqa_oracle_rope(_ptr(flat[r]), d, float(t), float(theta),
                            out[r].ctypes.data_as(ctypes.c_void_p))
    return out.reshape(x.shape)


# --------------------------------------------------------------------------
# integer-only parts

def layer_kind(layer: int) -> int:
    """Three local layers, then one global: layer l is global iff l % 4 == 3
    (shishifenxi.com page, section 01: the cycle of three local then one
    global; runtimewire.com page, "Narrow cache": every fourth layer)."""
    return GLOBAL if layer % 4 == 3 else LOCAL


def kv_bytes_per_token_layer(hkv=2, d=128, elem_bytes=2) -> int:
    """K and V for one token in one layer: hkv heads x d x {K,V} x bytes
    (section 01 of the shishifenxi.com page: about 1024 B in BF16)."""
    return hkv * d * 2 * elem_bytes


def kv_cache_bytes(n_layers=52, ctx=131072, window=2048, hkv=2, d=128,
                   elem_bytes=2, all_global=False):
    """Bytes held by the caches at context ``ctx``: global layers keep every
    token, local layers keep min(ctx, window) tokens.  Returns
    (global_bytes, local_bytes)."""
    per = kv_bytes_per_token_layer(hkv, d, elem_bytes)
    n_glob = sum(1 for l in range(n_layers)
                 if all_global or layer_kind(l) == GLOBAL)
    n_loc = n_layers - n_glob
    return n_glob * ctx * per, n_loc * min(ctx, window) * per


def pair_count(T: int, window: int = 0, causal: bool = True) -> int:
    """Number of (query, key) pairs a layer evaluates over T tokens: every
    pair when not causal, j <= i when causal, and i - window < j <= i with a
    window.  Counted by summing over queries (no closed form is used)."""
    i = np.arange(T, dtype=np.int64)
    if not causal:
        return int(T) * int(T)
    per = i + 1
    if window > 0:
        per = np.minimum(per, window)
    return int(per.sum())


def expected_cache(kind, capacity, appends, window=2048, hkv=2, d=128,
                   sentinel=0xFFFF, nseq=1):
    """Integer cache contents after a sequence of appends, per sequence.

    appends: list of (b, pos0, k_bits[n, hkv, d], v_bits[n, hkv, d]).
    Global: slot = position.  Local: slot = position mod window, the latest
    write to a slot wins.  Slots never written keep ``sentinel``.
    Returns (K, V) uint16 arrays [nseq, capacity, hkv, d]."""
    K = np.full((nseq, capacity, hkv, d), sentinel, dtype=np.uint16)
    V = np.full((nseq, capacity, hkv, d), sentinel, dtype=np.uint16)
    for (b, pos0, kb, vb) in appends:
        kb = _bits(kb).reshape(-1, hkv, d)
        vb = _bits(vb).reshape(-1, hkv, d)
        for t in range(kb.shape[0]):
            pos = pos0 + t
            slot = pos if kind == GLOBAL else pos % window
            assert 0 <= slot < capacity
            K[b, slot] = kb[t]
            V[b, slot] = vb[t]
    return K, V
