"""GPU checks that relate the entry points to each other and to the
structure of the method, beyond element-wise parity with the oracle:

* RoPE makes a score depend on the query and key positions only through
  their difference, so moving a whole local window (queries and keys) by c
  positions must leave the outputs unchanged up to the rounding of the
  rotated operands.  A shift that is not a multiple of 2048 also moves
  every key to another ring slot.
* Prefill row r and a decode at pos0 + r (after appending rows 0..r) are
  the same function of the same inputs.
* A decode step captured in a HIP graph and replayed gives the eager result
  on every replay (the library records no memset nodes).
* Verification at the largest batch, ragged positions."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import synth_inputs as si
from tests._util import check_close, fill_layer, sentinel_cache
from tests.test_gpu_block import _oracle_rows, _setup

pytestmark = pytest.mark.gpu


def _shifted_stream(k, v, lo, hi, c):
    """A stream whose positions lo + c .. hi + c hold the rows that
    positions lo .. hi hold in (k, v); earlier rows are filler."""
    n = hi + c + 1
    k2 = torch.zeros((n,) + tuple(k.shape[1:]), dtype=k.dtype)
    v2 = torch.zeros((n,) + tuple(v.shape[1:]), dtype=v.dtype)
    k2[lo + c:] = k[lo:hi + 1]
    v2[lo + c:] = v[lo:hi + 1]
    return k2, v2


@pytest.mark.parametrize("c", [777, 3 * ga.WINDOW, 100000])
def test_local_decode_shift_invariance(c):
    p = 5000
    k, v = si.stream(si.seq_seed(4001, 0), p + 1)
    q = si.queries(si.seq_seed(4001, 0) + 9, 1)
    base = sentinel_cache(ga.LOCAL, 1)
    fill_layer(base, [(k, v)], [p])
    k2, v2 = _shifted_stream(k, v, p - ga.WINDOW + 1, p, c)
    moved = sentinel_cache(ga.LOCAL, 1)
    fill_layer(moved, [(k2, v2)], [p + c])
    a = ga.attn_decode(base, q.cuda(), [p]).cpu().numpy()
    b = ga.attn_decode(moved, q.cuda(), [p + c]).cpu().numpy()
    print("shift %d" % c, flush=True)
    # the kernels rotate by offsets to the query, so the two runs do the
    # same arithmetic (measured: identical); the tolerance allows a kernel
    # that rotates by absolute position instead
    check_close(b, a.astype(np.float64), "local decode shifted by %d" % c,
                max_abs=5e-3, mean_abs=5e-4)


@pytest.mark.parametrize("c", [777, 2 * ga.WINDOW])
def test_local_verify_shift_invariance(c):
    pos0, n = 6000, 16
    k, v = si.stream(si.seq_seed(4002, 0), pos0 + n)
    q = si.queries(si.seq_seed(4002, 0) + 9, n)[None]
    outs = []
    for shift in (0, c):
        kk, vv = _shifted_stream(k, v, pos0 - ga.WINDOW + 1, pos0 + n - 1,
                                 shift)
        layer = sentinel_cache(ga.LOCAL, 1)
        p0 = pos0 + shift
        fill_layer(layer, [(kk, vv)], [p0 - 1])
        kb = kk[p0:p0 + n][None].contiguous()
        vb = vv[p0:p0 + n][None].contiguous()
        outs.append(ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(),
                                   [p0]).cpu().numpy())
    check_close(outs[1], outs[0].astype(np.float64),
                "local verify shifted by %d" % c, max_abs=5e-3, mean_abs=5e-4)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_rows_equal_decode(kind):
    """Prefill row r == decode at pos0 + r with rows 0..r appended."""
    pos0, n = [3000], 48
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=4010,
                                       capacity=4096 if kind == ga.GLOBAL
                                       else None)
    pre = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    pre = pre.float().cpu().numpy()
    ws = ga.workspace(ga.OP_DECODE, kind, 1, 1, 4096)
    worst = 0.0
    for r in range(n):
        dec = ga.attn_decode_append(layer, q[:, r].contiguous().cuda(),
                                    kb[:, r:r + 1].contiguous().cuda(),
                                    vb[:, r:r + 1].contiguous().cuda(),
                                    [pos0[0] + r], ws=ws)
        torch.cuda.synchronize()
        worst = max(worst, float(np.abs(dec.cpu().numpy() - pre[:, r]).max()))
    print("prefill vs decode kind=%d: max %.3e" % (kind, worst), flush=True)
    # prefill rounds its output to bf16 (relative 2^-9 of |o| <= ~4)
    assert worst < 1.5e-2


def test_decode_append_graph_replay():
    """Two local and two global layers, batch 4, appended and attended in a
    captured graph: every replay equals an eager run of the same calls."""
    B, p = 4, 9000
    kinds = [ga.LOCAL, ga.LOCAL, ga.GLOBAL, ga.GLOBAL]
    g = torch.Generator(device="cuda").manual_seed(4020)
    layers, qs, kn, vn = [], [], [], []
    for kind in kinds:
        cap = ga.WINDOW if kind == ga.LOCAL else 10000
        k = torch.randn((B, cap, ga.HKV, ga.D), generator=g,
                        device="cuda").to(torch.bfloat16)
        v = torch.randn((B, cap, ga.HKV, ga.D), generator=g,
                        device="cuda").to(torch.bfloat16)
        layers.append(ga.Layer(kind, k, v))
        qs.append(torch.randn((B, ga.HQ, ga.D), generator=g,
                              device="cuda").to(torch.bfloat16))
        kn.append(torch.randn((B, 1, ga.HKV, ga.D), generator=g,
                              device="cuda").to(torch.bfloat16))
        vn.append(torch.randn((B, 1, ga.HKV, ga.D), generator=g,
                              device="cuda").to(torch.bfloat16))
    ws = torch.empty(max(ga.workspace_bytes(ga.OP_DECODE, k, B, 1, 10000)
                         for k in (ga.LOCAL, ga.GLOBAL)),
                     dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, ga.HQ, ga.D), dtype=torch.float32, device="cuda")
            for _ in kinds]
    pos = [p - 3 * b for b in range(B)]

    def step():
        for i in range(len(kinds)):
            ga.attn_decode_append(layers[i], qs[i], kn[i], vn[i], pos,
                                  outs[i], ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(kinds)):
            assert torch.equal(outs[i], eager[i]), "replay %d layer %d" % (rep, i)
        # eager work between replays
        step()
        torch.cuda.synchronize()


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_verify_max_batch_64(kind):
    rng = np.random.default_rng(4030)
    pos0 = [int(x) for x in rng.integers(0, 5000, 64)]
    pos0[0], pos0[-1] = 0, 4984
    n = 16
    print("verify B=64 kind=%d" % kind, flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=4031)
    out = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sample = [0, 1, 17, 40, 63]
    want = _oracle_rows(kind, q[sample], [streams[b] for b in sample],
                        [pos0[b] for b in sample], list(range(n)))
    check_close(got[sample], want, "verify B=64 kind=%d" % kind)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_prefill_max_batch_64(kind):
    """Prefill of 100 tokens for 64 sequences at ragged positions (an empty
    prior first, a wrapped local ring last); every row of five sequences."""
    rng = np.random.default_rng(4040 + kind)
    pos0 = [int(x) for x in rng.integers(0, 5000, 64)]
    pos0[0], pos0[-1] = 0, 4900
    n = 100
    print("prefill B=64 kind=%d" % kind, flush=True)
    layer, streams, q, kb, vb = _setup(kind, pos0, n, seed=4041 + kind)
    out = ga.attn_prefill(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    sample = [0, 1, 17, 40, 63]
    want = _oracle_rows(kind, q[sample], [streams[b] for b in sample],
                        [pos0[b] for b in sample], list(range(n)))
    check_close(got[sample], want, "prefill B=64 kind=%d" % kind)


def test_draft_block_max_batch_64():
    """A drafted block of 16 tokens predicted together for 64 sequences at
    ragged positions; five sequences checked against the oracle."""
    from tests.test_gpu_draft import _oracle_together
    rng = np.random.default_rng(4050)
    pos0 = [int(x) for x in rng.integers(0, 5000, 64)]
    pos0[0], pos0[-1] = 0, 4984
    n = 16
    print("draft B=64", flush=True)
    layer, streams, q, kb, vb = _setup(ga.GLOBAL, pos0, n, seed=4051)
    out = ga.attn_draft_block(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sample = [0, 1, 17, 40, 63]
    want = _oracle_together(q[sample], [streams[b] for b in sample],
                            [pos0[b] for b in sample], n)
    check_close(got[sample], want, "draft B=64")
