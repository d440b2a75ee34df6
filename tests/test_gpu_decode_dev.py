"""Decode with device-resident positions (gqa_attn_decode_dev).

The same kernels read the positions from device memory instead of the call,
so the results must be bit-identical to the host-position entry points; a
step captured in a HIP graph, with the positions advanced inside the graph,
must reproduce an eager run that passes the advancing positions from the
host (up to summation order when the two plan different key splits); and a
device position beyond the validated bound gives NaN rows and appends
nothing, leaving the other sequences of the call intact."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import synth_inputs as si
from tests._util import check_close, fill_layer, oracle_decode, sentinel_cache

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_device_positions_equal_host_positions(kind):
    positions = [131071 if kind == ga.GLOBAL else 70000, 2047, 5000, 64]
    B = len(positions)
    streams = [si.stream(si.seq_seed(4200, b), positions[b] + 1)
               for b in range(B)]
    q = torch.cat([si.queries(si.seq_seed(4200, b) + 3, 1) for b in range(B)])
    layer = sentinel_cache(kind, B, ga.MAX_CONTEXT if kind == ga.GLOBAL
                           else None)
    fill_layer(layer, streams, positions)
    host = ga.attn_decode(layer, q.cuda(), positions)
    pos_dev = torch.tensor(positions, dtype=torch.int64, device="cuda")
    dev = ga.attn_decode_dev(layer, q.cuda(), pos_dev, max(positions))
    torch.cuda.synchronize()
    assert torch.equal(dev, host)
    check_close(dev.cpu().numpy(), oracle_decode(kind, q, streams, positions),
                "decode_dev kind=%d" % kind)


def test_graph_replay_with_advancing_device_positions():
    """Two local and two global layers, batch 4, append + attend; the graph
    also adds 1 to every position, so replay r works at pos + r."""
    B, steps = 4, 5
    kinds = [ga.LOCAL, ga.GLOBAL, ga.LOCAL, ga.GLOBAL]
    start = [9000, 2040, 30, 7000]
    max_pos = max(start) + steps
    g = torch.Generator(device="cuda").manual_seed(4210)

    def make_layers():
        ls = []
        for kind in kinds:
            cap = ga.WINDOW if kind == ga.LOCAL else 12000
            k = torch.randn((B, cap, ga.HKV, ga.D), generator=g,
                            device="cuda").to(torch.bfloat16)
            v = torch.randn((B, cap, ga.HKV, ga.D), generator=g,
                            device="cuda").to(torch.bfloat16)
            ls.append(ga.Layer(kind, k, v))
        return ls
    layers = make_layers()
    ref = [ga.Layer(l.kind, l.k.clone(), l.v.clone()) for l in layers]
    qs = [torch.randn((B, ga.HQ, ga.D), generator=g, device="cuda")
          .to(torch.bfloat16) for _ in kinds]
    kn = [torch.randn((B, 1, ga.HKV, ga.D), generator=g, device="cuda")
          .to(torch.bfloat16) for _ in kinds]
    vn = [torch.randn((B, 1, ga.HKV, ga.D), generator=g, device="cuda")
          .to(torch.bfloat16) for _ in kinds]
    ws = torch.empty(max(ga.workspace_bytes(ga.OP_DECODE, k, B, 1, max_pos + 1)
                         for k in (ga.LOCAL, ga.GLOBAL)),
                     dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, ga.HQ, ga.D), dtype=torch.float32, device="cuda")
            for _ in kinds]
    pos_dev = torch.tensor(start, dtype=torch.int64, device="cuda")

    def step():
        for i in range(len(kinds)):
            ga.attn_decode_dev(layers[i], qs[i], pos_dev, max_pos, outs[i], ws,
                               kn[i], vn[i])
        pos_dev.add_(1)

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the graph, then rewind
        step()
        pos_dev.sub_(1)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # the warm-up appended at `start`: redo that on the reference caches
    for i in range(len(kinds)):
        ga.attn_decode_append(ref[i], qs[i], kn[i], vn[i], start)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ref_ws = ga.workspace(ga.OP_DECODE, ga.GLOBAL, B, 1, max_pos + 1)
    for r in range(steps):
        graph.replay()
        torch.cuda.synchronize()
        pos = [p + r for p in start]
        for i in range(len(kinds)):
            want = ga.attn_decode_append(ref[i], qs[i], kn[i], vn[i], pos,
                                         ws=ref_ws)
            torch.cuda.synchronize()
            # same kernels; the graph plans its key splits for max_pos and
            # the eager call for the current positions, so allow for a
            # different summation order
            err = (outs[i] - want).abs().max().item()
            assert err <= 1e-5, "replay %d layer %d: %g" % (r, i, err)
    assert pos_dev.tolist() == [p + steps for p in start]
    for i in range(len(kinds)):
        assert torch.equal(layers[i].k.view(torch.int16),
                           ref[i].k.view(torch.int16))
        assert torch.equal(layers[i].v.view(torch.int16),
                           ref[i].v.view(torch.int16))


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_device_position_beyond_bound(kind):
    positions = [3000, 3000]
    B = 2
    streams = [si.stream(si.seq_seed(4220, b), positions[b] + 2)
               for b in range(B)]
    q = torch.cat([si.queries(si.seq_seed(4220, b) + 3, 1) for b in range(B)])
    layer = sentinel_cache(kind, B, 8192 if kind == ga.GLOBAL else None)
    fill_layer(layer, streams, [p - 1 for p in positions])
    kn = torch.stack([streams[b][0][positions[b]:positions[b] + 1]
                      for b in range(B)]).cuda()
    vn = torch.stack([streams[b][1][positions[b]:positions[b] + 1]
                      for b in range(B)]).cuda()
    before = layer.k.view(torch.int16).clone()
    max_pos = 3000
    pos_dev = torch.tensor([3000, 3001], dtype=torch.int64, device="cuda")
    out = ga.attn_decode_dev(layer, q.cuda(), pos_dev, max_pos, k_new=kn,
                             v_new=vn)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[1]).all(), "sequence beyond the bound must be NaN"
    check_close(got[:1], oracle_decode(kind, q[:1], streams[:1], [3000]),
                "in-range sequence kind=%d" % kind)
    slot = 3001 if kind == ga.GLOBAL else 3001 % ga.WINDOW
    after = layer.k.view(torch.int16)
    assert torch.equal(after[1, slot], before[1, slot]), "no append beyond bound"
    slot0 = 3000 if kind == ga.GLOBAL else 3000 % ga.WINDOW
    assert torch.equal(after[0, slot0].cpu(), kn[0, 0].cpu().view(torch.int16))
