"""Verification and drafted blocks over the fp8 (E4M3) cache on the GPU,
against the oracle.

The cache is filled with the library's fp8 append; the expected values come
from the oracle's own quantisation of the same bf16 stream
(oracle/fp8.py: ``attend_mixed``): cached tokens at their exact dequantised
values, the block's own tokens (which arrive with the call, not yet in the
cache) at their bf16 values.  Bar: max abs <= 2e-2, mean abs <= 2e-3, and the
max/RMS gate beyond 32K keys.  Covered: both layer kinds, blocks of 1, 5 and
16 tokens, prefill chunks (every row of chunks up to 2500 tokens, sampled
and edge rows of the last 4096-token chunk of 131072), ragged batches (an
empty prior, a prior shorter than a tile, a local window that wraps the
ring), the largest batch (64 sequences), the full 131056-token prior,
needles at key-split and tile edges and inside the block, the drafted block
predicted together, and an exactly held cache against the bf16 verification."""
import random

import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import synth_inputs as si
from oracle import fp8
from tests._util import check_close

pytestmark = pytest.mark.gpu


def _fill_prior(kind, streams, pos0, capacity):
    """fp8 caches holding each sequence's positions before its block
    (global: 0 .. pos0-1; local: the last 2048 of them) through the
    library's append; returns the layer and the oracle's quantisation of the
    same rows (first position, codes and scales)."""
    B = len(pos0)
    layer = ga.LayerFp8.allocate(kind, B, capacity, device="cuda", fill=0xA5)
    layer.k_scale.fill_(-1.0)
    layer.v_scale.fill_(-1.0)
    prior = []
    for b, (k, v) in enumerate(streams):
        p = pos0[b]
        lo = 0 if kind == ga.GLOBAL else max(0, p - ga.WINDOW)
        if p > lo:
            sub = ga.LayerFp8(kind, layer.k[b:b + 1], layer.v[b:b + 1],
                              layer.k_scale[b:b + 1], layer.v_scale[b:b + 1])
            ga.kv_append_fp8(sub, k[None, lo:p].contiguous().cuda(),
                             v[None, lo:p].contiguous().cuda(), [lo])
        kc, ks = fp8.quantize(si.bits(k[lo:p])) if p > lo else (
            np.zeros((0, 2, 128), np.uint8), np.zeros((0, 2), np.float32))
        vc, vs = fp8.quantize(si.bits(v[lo:p])) if p > lo else (
            np.zeros((0, 2, 128), np.uint8), np.zeros((0, 2), np.float32))
        prior.append((lo, kc, ks, vc, vs))
    return layer, prior


def _run(kind, pos0, n, seed, together=False, capacity=None, streams=None,
         q=None, prefill=False, rows=None):
    """The library's call and the oracle's values; rows: the query tokens
    the oracle computes (all by default)."""
    B = len(pos0)
    print("fp8 %s kind=%d B=%d n=%d pos0=%s" %
          ("prefill" if prefill else "draft" if together else "verify",
           kind, B, n, pos0[:4]), flush=True)
    if streams is None:
        streams = [si.stream(si.seq_seed(seed, b), pos0[b] + n)
                   for b in range(B)]
    if q is None:
        q = torch.stack([si.queries(si.seq_seed(seed, b) + 77, n)
                         for b in range(B)])
    if capacity is None and kind == ga.GLOBAL:
        # scales of sequence b start at b * 2 * capacity floats: a multiple
        # of 64 keeps every sequence's scales 16-byte aligned
        capacity = min(ga.MAX_CONTEXT, (max(pos0) + n + 63) // 64 * 64)
    layer, prior = _fill_prior(kind, streams, pos0, capacity)
    kb = torch.stack([streams[b][0][pos0[b]:pos0[b] + n] for b in range(B)])
    vb = torch.stack([streams[b][1][pos0[b]:pos0[b] + n] for b in range(B)])
    fn = (ga.attn_prefill_fp8 if prefill else
          ga.attn_draft_block_fp8 if together else ga.attn_verify_fp8)
    got = fn(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    rows = np.arange(n) if rows is None else np.asarray(rows)
    want = []
    for b in range(B):
        lo, kc, ks, vc, vs = prior[b]
        qpos = (np.full(len(rows), pos0[b] + n - 1) if together
                else pos0[b] + rows)
        want.append(fp8.attend_mixed(
            si.bits(q[b][rows]), qpos, kc, ks, vc, vs, si.bits(kb[b]),
            si.bits(vb[b]), lo, hq=ga.HQ, hkv=ga.HKV, d=ga.D,
            window=ga.WINDOW if kind == ga.LOCAL else 0,
            rope=kind == ga.LOCAL, theta=10000.0))
    return got.float().cpu().numpy()[:, rows], np.stack(want), prior


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
@pytest.mark.parametrize("n", [1, 5, 16])
def test_verify_fp8_ragged(kind, n):
    pos0 = [0, 37, 2040, 5000]
    got, want, _ = _run(kind, pos0, n, 8201 + n)
    check_close(got, want, "verify fp8 kind=%d n=%d" % (kind, n))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_verify_fp8_full_size_131056(kind):
    pos0 = [ga.MAX_CONTEXT - 16]
    got, want, _ = _run(kind, pos0, 16, 8211,
                        capacity=ga.MAX_CONTEXT if kind == ga.GLOBAL
                        else None)
    check_close(got, want, "verify fp8 131056 kind=%d" % kind,
                ctx=ga.MAX_CONTEXT if kind == ga.GLOBAL else ga.WINDOW)


@pytest.mark.parametrize("kind,pos0,needle", [
    (ga.GLOBAL, 131056, 0), (ga.GLOBAL, 131056, 131055),
    (ga.GLOBAL, 131056, 1024 * 16 - 1), (ga.GLOBAL, 131056, 1024 * 16),
    (ga.GLOBAL, 131056, 131060),           # inside the block (bf16 row)
    (ga.LOCAL, 131056, 131056 - 2048), (ga.LOCAL, 131056, 131055),
    (ga.LOCAL, 131056, 131058), (ga.LOCAL, 4096, 4096 - 2000)])
def test_verify_fp8_needle(kind, pos0, needle):
    n = 16
    k, v, u = si.needle_stream(si.seq_seed(8221, 0), pos0 + n, [needle], 8222,
                               magnitude=16.0)
    q = (u.float().repeat_interleave(16, dim=0) * 8.0).to(torch.bfloat16)
    q = q[None].expand(n, -1, -1).contiguous()[None]
    got, want, _ = _run(kind, [pos0], n, 8221, streams=[(k, v)], q=q,
                        capacity=ga.MAX_CONTEXT if kind == ga.GLOBAL
                        else None)
    check_close(got, want, "verify fp8 needle kind=%d at %d" % (kind, needle),
                ctx=pos0 + n if kind == ga.GLOBAL else ga.WINDOW)


@pytest.mark.parametrize("pos0,n", [(0, 16), (5000, 16), (77777, 7),
                                    (131056, 16)])
def test_draft_block_fp8(pos0, n):
    got, want, _ = _run(ga.GLOBAL, [pos0], n, 8231, together=True,
                        capacity=ga.MAX_CONTEXT)
    check_close(got, want, "draft fp8 pos0=%d n=%d" % (pos0, n),
                ctx=pos0 + n)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_verify_fp8_exact_cache_matches_bf16_verify(kind):
    """A prior made of E4M3 values times 2^-6 with largest magnitude 7
    (scale exactly 2^-6) is held exactly by the fp8 cache: fp8 and bf16
    verification see the same keys and values and agree to the bar."""
    rng = np.random.default_rng(8241)
    table = fp8.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    pos0, n = 6000, 16
    kv = []
    for _ in range(2):
        vals = rng.choice(table, size=(pos0 + n, 2, 128)) * \
            rng.choice([-1, 1], (pos0 + n, 2, 128)) * 2.0 ** -6
        vals[:, :, 0] = 7.0
        kv.append(torch.from_numpy(vals).to(torch.bfloat16))
    q = si.queries(8242, n)[None]
    got8, want, prior = _run(kind, [pos0], n, 8241, streams=[tuple(kv)], q=q)
    assert (prior[0][2] == np.float32(2.0 ** -6)).all()
    cap = pos0 + n if kind == ga.GLOBAL else None
    layer = ga.Layer.allocate(kind, 1, cap, device="cuda")
    lo = 0 if kind == ga.GLOBAL else pos0 - ga.WINDOW
    ga.kv_append(layer, kv[0][None, lo:pos0].contiguous().cuda(),
                 kv[1][None, lo:pos0].contiguous().cuda(), [lo])
    got16 = ga.attn_verify(layer, q.cuda(),
                           kv[0][None, pos0:].contiguous().cuda(),
                           kv[1][None, pos0:].contiguous().cuda(), [pos0])
    torch.cuda.synchronize()
    check_close(got8, want, "verify fp8 exact cache kind=%d" % kind)
    check_close(got8, got16.cpu().numpy(), "fp8 vs bf16 verify kind=%d" % kind)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
@pytest.mark.parametrize("pos0,n", [([0, 3000], 300), ([37, 2100], 129),
                                    ([5000], 2500)])
def test_prefill_fp8_every_row(kind, pos0, n):
    """Chunks over the fp8 cache against the oracle, every row (bf16 out):
    an empty prior, a local window across the ring's end, a chunk longer
    than the window."""
    got, want, _ = _run(kind, pos0, n, 8251 + n, prefill=True)
    check_close(got, want, "prefill fp8 kind=%d n=%d" % (kind, n))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_fp8_last_chunk_131072_sampled(kind):
    """The last 4096-token chunk of a 131072-token prompt over the fp8
    cache: 256 sampled rows plus the chunk's edge rows."""
    n, pos0 = 4096, ga.MAX_CONTEXT - 4096
    rng = np.random.default_rng(8261)
    rows = np.unique(np.concatenate([
        rng.choice(n, 256, replace=False),
        [0, 1, 15, 16, 63, 64, 2046, 2047, 2048, 4094, 4095]]))
    got, want, _ = _run(kind, [pos0], n, 8261, prefill=True, rows=rows,
                        capacity=ga.MAX_CONTEXT if kind == ga.GLOBAL
                        else None)
    check_close(got, want, "prefill fp8 131072 kind=%d" % kind,
                ctx=ga.MAX_CONTEXT if kind == ga.GLOBAL else ga.WINDOW)


def _random_cases(count=48):
    rng = random.Random(20261204)
    out = []
    for _ in range(count):
        op = rng.choice(["verify", "draft", "prefill"])
        kind = ga.GLOBAL if op == "draft" else rng.choice([ga.LOCAL, ga.GLOBAL])
        B = rng.randint(1, 4)
        n = rng.randint(1, 16) if op != "prefill" else rng.randint(1, 600)
        pos0 = [rng.choice([rng.randint(0, 100), rng.randint(0, 12000)])
                for _ in range(B)]
        rows = (list(range(n)) if n <= 48 else sorted(
            set([0, 1, n - 2, n - 1] + rng.sample(range(n), 40))))
        out.append((op, kind, pos0, n, rng.randint(1, 10 ** 6), rows))
    return out


@pytest.mark.parametrize("case", _random_cases(),
                         ids=lambda c: "%s-%d" % (c[0], c[1]))
def test_fp8_block_random_case(case):
    """Randomly drawn shapes (fixed seed) of the three calls over the fp8
    cache: ragged batches of 1-4 sequences mixing short (< 100) and long (up
    to 12000) priors, 1-16 block tokens, 1-600 prefill tokens (prefill:
    first two, last two and 40 sampled rows)."""
    op, kind, pos0, n, seed, rows = case
    got, want, _ = _run(kind, pos0, n, seed, together=op == "draft",
                        prefill=op == "prefill", rows=rows)
    check_close(got, want, "fp8 %s kind=%d pos0=%s n=%d seed=%d" %
                (op, kind, pos0, n, seed))


@pytest.mark.parametrize("op,kind", [
    ("verify", ga.LOCAL), ("verify", ga.GLOBAL), ("draft", ga.GLOBAL),
    ("prefill", ga.LOCAL), ("prefill", ga.GLOBAL)])
def test_fp8_block_max_batch_64(op, kind):
    """The largest batch the library takes (64 sequences), ragged priors of
    0 to 3000 tokens (an empty prior first, a wrapped local ring last):
    verification and the drafted block with 16 tokens, prefill with 100
    (every row)."""
    rng = random.Random(8290 + kind)
    pos0 = [rng.randrange(0, 3000) for _ in range(ga.MAX_BATCH)]
    pos0[0], pos0[-1] = 0, 2999
    n = 100 if op == "prefill" else 16
    got, want, _ = _run(kind, pos0, n, 8290 + kind, together=op == "draft",
                        prefill=op == "prefill")
    check_close(got, want, "fp8 %s B=64 kind=%d" % (op, kind))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_fp8_block_calls_in_a_graph(kind):
    """Verification and prefill over the fp8 cache captured in a HIP graph:
    every replay, with eager work and synchronisation between replays,
    equals the eager call bit for bit."""
    pos0, n, npf = [3000, 700], 16, 300
    B = len(pos0)
    streams = [si.stream(si.seq_seed(8271, b), pos0[b] + npf)
               for b in range(B)]
    cap = None if kind == ga.LOCAL else 4096
    layer, _ = _fill_prior(kind, streams, pos0, cap)
    dev = "cuda"
    qv = torch.stack([si.queries(si.seq_seed(8271, b) + 1, n)
                      for b in range(B)]).to(dev)
    qp = torch.stack([si.queries(si.seq_seed(8271, b) + 2, npf)
                      for b in range(B)]).to(dev)
    kv = torch.stack([streams[b][0][pos0[b]:pos0[b] + npf]
                      for b in range(B)]).to(dev)
    vv = torch.stack([streams[b][1][pos0[b]:pos0[b] + npf]
                      for b in range(B)]).to(dev)
    kb, vb = kv[:, :n].contiguous(), vv[:, :n].contiguous()
    ctx = max(pos0) + npf
    wsv = ga.workspace(ga.OP_VERIFY, kind, B, n, ctx)
    wsp = ga.workspace(ga.OP_PREFILL_FP8, kind, B, npf, ctx)
    ov = torch.empty(B, n, ga.HQ, ga.D, dtype=torch.float32, device=dev)
    op = torch.empty(B, npf, ga.HQ, ga.D, dtype=torch.bfloat16, device=dev)

    def step():
        ga.attn_verify_fp8(layer, qv, kb, vb, pos0, ov, wsv)
        ga.attn_prefill_fp8(layer, qp, kv, vv, pos0, op, wsp)

    step()
    torch.cuda.synchronize()
    ref_v, ref_p = ov.clone(), op.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        ov.zero_()
        op.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ov, ref_v), "verify replay %d" % rep
        assert torch.equal(op, ref_p), "prefill replay %d" % rep
