"""The 52-layer decode step on the GPU, with the layer kinds taken from the
library's schedule (``gqa_layer_kind``: three local layers then one global),
checked layer by layer against the fp64 oracle.

The step is run as the benchmark runs it: for every layer in order, the new
token's K/V is appended and attended in one call (``attn_decode_append``),
all 52 calls share one workspace, and the step is captured once in a HIP
graph and replayed.  Every output row of every layer is compared with the
oracle (max abs <= 2e-2, mean abs <= 2e-3), and the replays must reproduce
the first one bit for bit.

Shapes: a single sequence at context 32768 (52 layers: local rings wrapped
many times, global caches linear), and a ragged pair of sequences at
contexts 32768 and 5001."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import oracle
import synth_inputs as si
from tests._util import check_close, sentinel_cache

pytestmark = pytest.mark.gpu


def _build_step(positions, seed):
    """Caches of all 52 layers holding every visible position before each
    sequence's query, plus the query token's own K/V and the queries.
    Returns (kinds, layers, streams, q, k_new, v_new), where streams[l][b] =
    (k, v, lo): rows of positions lo .. p (the query's own at the end)."""
    B = len(positions)
    kinds = [ga.layer_kind(l) for l in range(ga.NUM_LAYERS)]
    cap = max(positions) + 1
    layers, streams, qs, kn, vn = [], [], [], [], []
    for l, kind in enumerate(kinds):
        layer = sentinel_cache(kind, B, cap if kind == ga.GLOBAL else None)
        per = []
        for b, p in enumerate(positions):
            lo = 0 if kind == ga.GLOBAL else max(0, p - ga.WINDOW + 1)
            k, v = si.stream(si.seq_seed(seed + l, b), p + 1 - lo)
            if p > lo:
                sub = ga.Layer(kind, layer.k[b:b + 1], layer.v[b:b + 1])
                ga.kv_append(sub, k[None, :-1].contiguous().cuda(),
                             v[None, :-1].contiguous().cuda(), [lo])
            per.append((k, v, lo))
        q = torch.cat([si.queries(si.seq_seed(seed + l, b) + 999, 1)
                       for b in range(B)])
        layers.append(layer)
        streams.append(per)
        qs.append(q)
        kn.append(torch.stack([per[b][0][-1:] for b in range(B)]))
        vn.append(torch.stack([per[b][1][-1:] for b in range(B)]))
    return kinds, layers, streams, qs, kn, vn


def _oracle_layer(kind, q, per, positions):
    out = []
    for b, p in enumerate(positions):
        k, v, lo = per[b]
        out.append(oracle.attend(
            si.bits(q[b:b + 1]), [p], si.bits(k), si.bits(v), lo, hq=ga.HQ,
            hkv=ga.HKV, d=ga.D, window=ga.WINDOW if kind == ga.LOCAL else 0,
            rope=kind == ga.LOCAL, theta=10000.0)[0])
    return np.stack(out)


@pytest.mark.parametrize("positions", [[32767], [32767, 5000]])
def test_52_layer_decode_step_graph(positions):
    print("52-layer step positions=%s" % positions, flush=True)
    B = len(positions)
    kinds, layers, streams, qs, kn, vn = _build_step(positions, seed=1002)
    assert kinds.count(ga.GLOBAL) == 13
    qd = [q.cuda() for q in qs]
    knd = [k.contiguous().cuda() for k in kn]
    vnd = [v.contiguous().cuda() for v in vn]
    outs = [torch.empty((B, ga.HQ, ga.D), dtype=torch.float32, device="cuda")
            for _ in kinds]
    ws = torch.empty(max(ga.workspace_bytes(ga.OP_DECODE, k, B, 1,
                                            max(positions) + 1)
                         for k in (ga.LOCAL, ga.GLOBAL)),
                     dtype=torch.uint8, device="cuda")

    def step():
        for l in range(ga.NUM_LAYERS):
            ga.attn_decode_append(layers[l], qd[l], knd[l], vnd[l], positions,
                                  outs[l], ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # eager once before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for o in outs:
        o.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    first = [o.cpu().numpy().copy() for o in outs]

    worst = 0.0
    for l, kind in enumerate(kinds):
        want = _oracle_layer(kind, qs[l], streams[l], positions)
        err = check_close(first[l], want, "layer %d kind %d" % (l, kind))
        worst = max(worst, float(err.max()))
    print("worst max abs over 52 layers: %.3e" % worst, flush=True)

    # the new tokens were stored to their slots (global: slot p; local ring:
    # p mod 2048)
    for l, kind in enumerate(kinds):
        for b, p in enumerate(positions):
            slot = p if kind == ga.GLOBAL else p % ga.WINDOW
            assert torch.equal(layers[l].k[b, slot].cpu().view(torch.int16),
                               kn[l][b, 0].view(torch.int16)), (l, b)
            assert torch.equal(layers[l].v[b, slot].cpu().view(torch.int16),
                               vn[l][b, 0].view(torch.int16)), (l, b)

    # replays with eager work in between reproduce the first replay exactly
    for r in range(2):
        torch.randn(1 << 20, device="cuda").sum().item()
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l in range(ga.NUM_LAYERS):
            assert np.array_equal(outs[l].cpu().numpy(), first[l]), (r, l)
