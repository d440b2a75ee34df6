"""Verify (drafted block, n <= 16) and chunked prefill on the GPU against
the fp64 oracle.

Tolerance: max abs <= 2e-2, mean abs <= 2e-3.  Beyond random inputs: the
cache must be left untouched by both calls, verify row r must agree with a
decode at pos0 + r once block tokens 0..r are appended (the two entry points
compute the same function), a zero query must give the exact window mean,
and the full-size shapes (verify at 131056 + 16, prefill's last 4096-token
chunk of 131072) are checked on sampled rows plus the edge rows.  At full
size the prefill also has gates a tolerance alone would miss there: a zero
query on every row of the last chunk against the exact mean of its visible
values, needles at the prior's ends, a tile edge, the causal diagonal and
the window edge, and every row of the first chunk; the whole prompt in one
131072-token chunk is checked on sampled rows."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import oracle
import synth_inputs as si
from tests._util import (check_close, fill_layer, same_path_excess,
                         sentinel_cache)

pytestmark = pytest.mark.gpu


def _oracle_rows(kind, q_cpu, streams, pos0, rows):
    """fp64 oracle for block tokens `rows` of each sequence."""
    out = []
    for b, (k, v) in enumerate(streams):
        qpos = [pos0[b] + r for r in rows]
        lo = 0 if kind == ga.GLOBAL else max(0, min(qpos) - ga.WINDOW + 1)
        hi = max(qpos) + 1
        out.append(oracle.attend(
            si.bits(q_cpu[b, rows]), qpos, si.bits(k[lo:hi]), si.bits(v[lo:hi]),
            lo, hq=ga.HQ, hkv=ga.HKV, d=ga.D,
            window=ga.WINDOW if kind == ga.LOCAL else 0,
            rope=kind == ga.LOCAL, theta=10000.0))
    return np.stack(out)


def _setup(kind, pos0, n, seed, capacity=None, v_scale=1.0):
    """Caches holding every position before pos0[b]; returns the layer,
    the logical streams (positions 0 .. pos0+n-1), the block tensors.
    v_scale (a power of two, so the bf16 values scale exactly) multiplies
    every value vector."""
    B = len(pos0)
    streams = [si.stream(si.seq_seed(seed, b), pos0[b] + n) for b in range(B)]
    if v_scale != 1.0:
        streams = [(k, (v.float() * v_scale).to(torch.bfloat16))
                   for k, v in streams]
    if kind == ga.GLOBAL and capacity is None:
        capacity = max(pos0) + n
    layer = sentinel_cache(kind, B, capacity)
    for b in range(B):
        if pos0[b] > 0:
            sub = ga.Layer(kind, layer.k[b:b + 1], layer.v[b:b + 1])
            lo = 0 if kind == ga.GLOBAL else max(0, pos0[b] - ga.WINDOW)
            ga.kv_append(sub, streams[b][0][None, lo:pos0[b]].contiguous().cuda(),
                         streams[b][1][None, lo:pos0[b]].contiguous().cuda(), [lo])
    kb = torch.stack([streams[b][0][pos0[b]:pos0[b] + n] for b in range(B)])
    vb = torch.stack([streams[b][1][pos0[b]:pos0[b] + n] for b in range(B)])
    q = torch.stack([si.queries(si.seq_seed(seed, b) + 555, n) for b in range(B)])
    return layer, streams, q, kb, vb


def _snapshot(layer):
    return (layer.k.view(torch.int16).clone(), layer.v.view(torch.int16).clone())


def _unchanged(layer, snap):
    return (torch.equal(layer.k.view(torch.int16), snap[0]) and
            torch.equal(layer.v.view(torch.int16), snap[1]))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
@pytest.mark.parametrize("n", [1, 5, 16])
def test_verify_ragged(kind, n):
    pos0 = [0, 63, 2047, 2048, 5000]
    print("verify kind=%d n=%d pos0=%s" % (kind, n, pos0), flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=2001 + n)
    snap = _snapshot(layer)
    out = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    assert _unchanged(layer, snap), "verify must not write the cache"
    want = _oracle_rows(kind, q, streams, pos0, list(range(n)))
    check_close(out.cpu().numpy(), want, "verify kind=%d n=%d" % (kind, n))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
@pytest.mark.parametrize("log2c", [18, -100])
def test_verify_value_scale(kind, log2c):
    """Attention is linear in the values: with every value vector times
    c = 2^log2c (exact in bf16) the output is c times the oracle's for the
    unscaled cache, so got / c meets the usual bar.  At c = 2^18 the values
    (up to ~10^6) lie beyond fp16's range and at c = 2^-100 far below its
    normal range, where the key splits' 2-byte partial rows would overflow
    or flush without their per-row scale."""
    pos0, n = [3000, 9000], 16
    c = 2.0 ** log2c
    print("verify value scale kind=%d c=2^%d" % (kind, log2c), flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=2060,
                                       capacity=20000 if kind == ga.GLOBAL
                                       else None, v_scale=c)
    out = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64) / c
    want = _oracle_rows(kind, q, streams, pos0, list(range(n))) / c
    check_close(got, want, "verify value scale kind=%d c=2^%d" % (kind, log2c))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_verify_full_size_131056(kind):
    # 16 drafted tokens at 131056..131071 over a 131056-token prior context
    pos0 = [131056]
    cap = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    print("verify full kind=%d" % kind, flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, 16, seed=1004, capacity=cap)
    out = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    want = _oracle_rows(kind, q, streams, pos0, list(range(16)))
    check_close(out.cpu().numpy(), want, "verify 131056+16 kind=%d" % kind,
                ctx=131072 if kind == ga.GLOBAL else ga.WINDOW)


@pytest.mark.parametrize("kind,needle", [
    (ga.GLOBAL, 0), (ga.GLOBAL, 64 * 37 - 1), (ga.GLOBAL, 64 * 37),
    (ga.GLOBAL, 131055), (ga.GLOBAL, 131056 + 3),
    (ga.LOCAL, 131056 - 2047 + 5), (ga.LOCAL, 131056 - 2047 + 64 * 3),
    (ga.LOCAL, 131055), (ga.LOCAL, 131056 + 9)])
def test_verify_needle(kind, needle):
    """A key far above the rest at a key-split boundary (splits are whole
    64-key tiles), at the first or last prior key, inside the block (seen
    only by the rows at or after it), or at the window edge of a local layer
    (seen by the first rows only): every row must match the oracle, and on a
    global layer every row that sees the needle must return its value."""
    pos0, n = [131056], 16
    k, v, u = si.needle_stream(si.seq_seed(1040, 0), pos0[0] + n, [needle],
                               1041, magnitude=16.0)
    cap = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    layer = sentinel_cache(kind, 1, cap)
    fill_layer(layer, [(k, v)], [pos0[0] - 1])
    kb = k[pos0[0]:pos0[0] + n][None].contiguous()
    vb = v[pos0[0]:pos0[0] + n][None].contiguous()
    q = (u.float().repeat_interleave(16, dim=0) * 8.0).to(torch.bfloat16)
    q = q[None, None].expand(1, n, ga.HQ, ga.D).contiguous()
    print("verify needle kind=%d at %d" % (kind, needle), flush=True)
    out = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = _oracle_rows(kind, q, [(k, v)], pos0, list(range(n)))
    check_close(got, want, "verify needle kind=%d at %d" % (kind, needle),
                ctx=131072 if kind == ga.GLOBAL else ga.WINDOW)
    if kind == ga.GLOBAL:
        target = np.repeat(v[needle].double().numpy(), 16, axis=0)
        for r in range(n):
            if pos0[0] + r >= needle:
                assert np.abs(got[0, r] - target).max() < 0.05, r


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_verify_rows_equal_decode_after_append(kind):
    """Verify token r == decode at pos0 + r once tokens 0..r are appended."""
    pos0, n = [3000, 9000], 16
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=2010,
                                       capacity=20000 if kind == ga.GLOBAL
                                       else None)
    ver = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    ver = ver.cpu().numpy()
    ws = ga.workspace(ga.OP_DECODE, kind, 2, 1, 20000)
    for r in range(n):
        pos = [p + r for p in pos0]
        dec = ga.attn_decode_append(layer, q[:, r].contiguous().cuda(),
                                    kb[:, r:r + 1].contiguous().cuda(),
                                    vb[:, r:r + 1].contiguous().cuda(), pos,
                                    ws=ws)
        torch.cuda.synchronize()
        err = np.abs(dec.cpu().numpy() - ver[:, r]).max()
        assert err < 1e-2, "row %d differs by %.3e" % (r, err)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
@pytest.mark.parametrize("pos0,n", [([0], 300), ([0, 4096], 257), ([4096], 4096),
                                    ([2000], 100), ([1], 8)])
def test_prefill_small(kind, pos0, n):
    print("prefill kind=%d pos0=%s n=%d" % (kind, pos0, n), flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=3001 + n)
    snap = _snapshot(layer)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    assert _unchanged(layer, snap), "prefill must not write the cache"
    rows = sorted(set(list(range(min(n, 40))) + list(range(max(0, n - 40), n)) +
                      [int(x) for x in np.random.default_rng(n).integers(0, n, 64)]))
    want = _oracle_rows(kind, q, streams, pos0, rows)
    got = out.float().cpu().numpy()[:, rows]
    check_close(got, want, "prefill kind=%d pos0=%s n=%d" % (kind, pos0, n))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_zero_query_window_mean(kind):
    pos0, n = [5000], 64
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=3100)
    q = torch.zeros_like(q)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    v = streams[0][1].double().numpy()
    got = out.float().cpu().numpy()[0]
    for r in (0, 1, 31, 63):
        i = pos0[0] + r
        lo = 0 if kind == ga.GLOBAL else i - ga.WINDOW + 1
        mean = np.repeat(v[lo:i + 1].mean(axis=0), 16, axis=0)
        err = np.abs(got[r] - mean).max()
        assert err < 4e-3, "row %d: %.3e (bf16 output)" % (r, err)


def test_prefill_then_append_chunks_match_single_chunk():
    """Two chunks (prefill + append, prefill) reproduce one big chunk."""
    kind, n = ga.GLOBAL, 1024
    layer, streams, q, kb, vb = _setup(kind, [0], 2 * n, seed=3200)
    whole = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), [0])
    first = ga.attn_prefill(layer, q[:, :n].contiguous().cuda(),
                            kb[:, :n].contiguous().cuda(),
                            vb[:, :n].contiguous().cuda(), [0])
    ga.kv_append(layer, kb[:, :n].contiguous().cuda(),
                 vb[:, :n].contiguous().cuda(), [0])
    second = ga.attn_prefill(layer, q[:, n:].contiguous().cuda(),
                             kb[:, n:].contiguous().cuda(),
                             vb[:, n:].contiguous().cuda(), [n])
    torch.cuda.synchronize()
    both = torch.cat([first, second], dim=1)
    diff = (both.float() - whole.float()).abs().max().item()
    assert same_path_excess(both.float().cpu().numpy(),
                            whole.float().cpu().numpy()) <= 0, diff


LAST0 = 131072 - 4096  # first position of the last 4096-token chunk


def _edge_rows(n):
    return [0, 1, 7, 8, 15, 16, 63, 64, 65, 127, 128, 2046, 2047, 2048, 2049,
            n - 65, n - 64, n - 2, n - 1]


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_last_chunk_131072_sampled(kind):
    """The last 4096-token chunk of a 131072-token prompt (the quadratic
    worst case), checked on 256 random rows plus the edge rows (tiles,
    query groups, the local window's width)."""
    pos0, n = [LAST0], 4096
    cap = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    print("prefill last chunk kind=%d" % kind, flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=1005, capacity=cap)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = sorted(set(_edge_rows(n) +
                      [int(x) for x in rng.choice(n, 256, replace=False)]))
    assert len(rows) >= 256
    want = _oracle_rows(kind, q, streams, pos0, rows)
    got = out.float().cpu().numpy()[:, rows]
    check_close(got, want, "prefill last chunk kind=%d (%d rows)" %
                (kind, len(rows)),
                ctx=131072 if kind == ga.GLOBAL else ga.WINDOW)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_last_chunk_131072_zero_query_every_row(kind):
    """A zero query weighs every visible key equally, so each of the 4096
    rows must equal the exact mean of V over its own visible keys (global:
    positions 0 .. i, up to 131072 keys; local: i - 2047 .. i).  The only
    rounding left on the GPU is the fp32 sum and the bf16 output (round to
    nearest: relative 2^-8 at most), so the gate is relative: one 64-key
    tile lost anywhere in a row's range moves its mean by ~6e-5 (global) or
    ~4e-3 (local), far above it."""
    pos0, n = [LAST0], 4096
    cap = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    print("prefill last chunk zero query kind=%d" % kind, flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=3150, capacity=cap)
    q = torch.zeros_like(q)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()[0]                  # [n, 32, 128]
    v = streams[0][1].double().numpy()                  # [131072, 2, 128]
    csum = np.concatenate([np.zeros((1,) + v.shape[1:]), np.cumsum(v, axis=0)])
    i = pos0[0] + np.arange(n)
    lo = np.zeros(n, dtype=np.int64) if kind == ga.GLOBAL else \
        np.maximum(i - ga.WINDOW + 1, 0)
    mean = (csum[i + 1] - csum[lo]) / (i + 1 - lo)[:, None, None]
    exact = np.repeat(mean, ga.HQ // ga.HKV, axis=1)    # [n, 32, 128]
    err = np.abs(got - exact)
    bound = np.abs(exact) * 2.0 ** -8 + 1e-6
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    print("zero-query rows: max abs err %.3e, max err/|mean| %.3e" %
          (err.max(), (err / (np.abs(exact) + 1e-30)).max()), flush=True)
    assert (err <= bound).all(), ("row %d head %d dim %d: got %.6e want %.6e"
                                  % (worst + (got[worst], exact[worst])))


@pytest.mark.parametrize("kind,needle", [
    (ga.GLOBAL, 0), (ga.GLOBAL, 64 * 1000 - 1), (ga.GLOBAL, 64 * 1000),
    (ga.GLOBAL, LAST0 - 1), (ga.GLOBAL, LAST0 + 100),
    (ga.GLOBAL, LAST0 + 4095),
    (ga.LOCAL, LAST0 - 2047 + 5), (ga.LOCAL, LAST0 - 1),
    (ga.LOCAL, LAST0 + 64 * 10), (ga.LOCAL, LAST0 + 4095)])
def test_prefill_last_chunk_131072_needle(kind, needle):
    """One key far above the rest at the first or last prior key, on both
    sides of a 64-key tile edge, on the causal diagonal inside the chunk, at
    the chunk's last key, or (local) at the window's edge, seen only by the
    chunk's first six rows.  On a global layer every row at or after the
    needle must return its value (all 4096 rows are checked); rows before
    it, and every local row sampled around where the needle enters and
    leaves the window, must match the oracle."""
    pos0, n = [LAST0], 4096
    # On a local layer the needle's score depends on its offset to the query
    # (RoPE), so many rows see it only partly dominant; there a needle
    # scoring ~45 nats (magnitude 16) turns the bf16 rounding of the rotated,
    # pre-scaled query (relative 2^-9 of the score: ~0.09 nats) plus the
    # bf16 output into errors just above 2e-2.  Magnitude 8 (~23 nats, still
    # e^23 against the window's 2048 background keys) keeps the scores in
    # the range the tolerance was set for.
    mag = 16.0 if kind == ga.GLOBAL else 8.0
    k, v, u = si.needle_stream(si.seq_seed(1050, 0), pos0[0] + n, [needle],
                               1051, magnitude=mag)
    cap = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    layer = sentinel_cache(kind, 1, cap)
    fill_layer(layer, [(k, v)], [pos0[0] - 1])
    kb = k[pos0[0]:pos0[0] + n][None].contiguous()
    vb = v[pos0[0]:pos0[0] + n][None].contiguous()
    q = (u.float().repeat_interleave(16, dim=0) * 8.0).to(torch.bfloat16)
    q = q[None, None].expand(1, n, ga.HQ, ga.D).contiguous()
    print("prefill needle kind=%d at %d" % (kind, needle), flush=True)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()[0]
    first_seen = max(0, needle - pos0[0])               # first row seeing it
    last_seen = min(n - 1, needle + ga.WINDOW - 1 - pos0[0]) \
        if kind == ga.LOCAL else n - 1
    if kind == ga.GLOBAL:
        target = np.repeat(v[needle].double().numpy(), 16, axis=0)
        err = np.abs(got[first_seen:] - target[None]).max()
        print("rows %d..%d return the needle: max err %.3e" %
              (first_seen, n - 1, err), flush=True)
        assert err < 0.05
    rng = np.random.default_rng(needle)
    rows = set(_edge_rows(n)) | {int(x) for x in rng.integers(0, n, 24)}
    for e in (first_seen, last_seen):
        rows |= {r for r in range(e - 2, e + 3) if 0 <= r < n}
    rows = sorted(rows)
    want = _oracle_rows(kind, q, [(k, v)], pos0, rows)
    check_close(got[None, rows], want, "prefill needle kind=%d at %d" %
                (kind, needle),
                ctx=131072 if kind == ga.GLOBAL else ga.WINDOW)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_first_chunk_every_row(kind):
    """Chunk 0 of a long prompt (positions 0 .. 4095, empty cache): every
    one of its 4096 rows against the oracle."""
    pos0, n = [0], 4096
    print("prefill chunk 0 every row kind=%d" % kind, flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=3300,
                                       capacity=n if kind == ga.GLOBAL
                                       else None)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    want = _oracle_rows(kind, q, streams, pos0, list(range(n)))
    check_close(out.float().cpu().numpy(), want,
                "prefill chunk 0 kind=%d (all rows)" % kind)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_one_chunk_of_131072(kind):
    """The largest chunk the library takes: the whole 131072-token prompt in
    one call from an empty cache, checked on the edge rows, the last rows and
    64 random rows."""
    pos0, n = [0], ga.MAX_CONTEXT
    print("prefill one chunk of 131072 kind=%d" % kind, flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=3310,
                                       capacity=n if kind == ga.GLOBAL
                                       else None)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = sorted(set(_edge_rows(n) + [n - 4097, n - 4096] +
                      [int(x) for x in rng.choice(n, 64, replace=False)]))
    want = _oracle_rows(kind, q, streams, pos0, rows)
    got = out[:, rows].float().cpu().numpy()
    check_close(got, want, "prefill one chunk of 131072 kind=%d (%d rows)" %
                (kind, len(rows)),
                ctx=131072 if kind == ga.GLOBAL else ga.WINDOW)
