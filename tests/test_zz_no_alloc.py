"""gqa_attn_decode_noalloc -- decode without a workspace, for callers that
cannot allocate -- against the workspace entry points it mirrors.

Through the C ABI (the binding's argument marshalling only), on two calls
in a row, the second with a smaller input: the outputs must equal those of
gqa_attn_decode_append / gqa_attn_decode on identical caches bit for bit
(same kernels, same plan; only where the partials live differs), match the
fp64 oracle within the tolerance, and leave the same cache bytes.  The
scratch keeps the previous call's partials, so the smaller second call also
shows that nothing of the first leaks into it.  A graph capture of the call
(no allocation inside) replays to the same result."""
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import synth_inputs as si
from tests._util import check_close, fill_layer, oracle_decode, sentinel_cache

pytestmark = pytest.mark.gpu


def _case(kind, positions, seed, capacity):
    """Two identical caches holding each sequence's stream up to (not
    including) its query position, plus the query token's K/V and q."""
    B = len(positions)
    streams = [si.stream(si.seq_seed(seed, b), positions[b] + 1)
               for b in range(B)]
    q = torch.cat([si.queries(si.seq_seed(seed, b) + 4242, 1)
                   for b in range(B)])
    layers = []
    for _ in range(2):
        layer = sentinel_cache(kind, B, capacity)
        fill_layer(layer, [(k[:-1], v[:-1]) for k, v in streams],
                   [p - 1 for p in positions])
        layers.append(layer)
    kn = torch.stack([k[-1:] for k, _ in streams]).contiguous()
    vn = torch.stack([v[-1:] for _, v in streams]).contiguous()
    return layers, streams, q, kn, vn


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_noalloc_matches_workspace_entry_points(kind):
    cap = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    # first call: batch 4 up to the full context; second: smaller
    for positions, seed in (([131071, 100000, 5000, 77], 7001),
                            ([3000], 7002)):
        print("noalloc kind=%d positions=%s" % (kind, positions), flush=True)
        (la, lb), streams, q, kn, vn = _case(kind, positions, seed, cap)
        qd, knd, vnd = q.cuda(), kn.cuda(), vn.cuda()
        want = ga.attn_decode_append(la, qd, knd, vnd, positions)
        got = ga.attn_decode_noalloc(lb, qd, positions, k_new=knd, v_new=vnd)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "append+attend differs"
        assert torch.equal(la.k.view(torch.int16), lb.k.view(torch.int16))
        assert torch.equal(la.v.view(torch.int16), lb.v.view(torch.int16))
        check_close(got.cpu().numpy(),
                    oracle_decode(kind, q, streams, positions),
                    "noalloc kind=%d B=%d" % (kind, len(positions)),
                    ctx=max(positions) + 1 if kind == ga.GLOBAL else ga.WINDOW)
        # attend only (the token is in the cache now)
        want2 = ga.attn_decode(la, qd, positions)
        got2 = ga.attn_decode_noalloc(lb, qd, positions)
        torch.cuda.synchronize()
        assert torch.equal(got2, want2), "attend-only differs"
        assert torch.equal(got2, got)


def test_noalloc_under_graph_capture():
    """Captured in a HIP graph (the first call on the device, which looks up
    the scratch's address, happened eagerly before), replayed with eager
    work in between: every replay equals the eager result."""
    positions = [40000, 123]
    (la, lb), streams, q, kn, vn = _case(ga.GLOBAL, positions, 7003, 65536)
    qd = q.cuda()
    for b, p in enumerate(positions):
        sub = ga.Layer(ga.GLOBAL, lb.k[b:b + 1], lb.v[b:b + 1])
        ga.kv_append(sub, kn[b:b + 1].cuda(), vn[b:b + 1].cuda(), [p])
    eager = ga.attn_decode_noalloc(lb, qd, positions)
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ga.attn_decode_noalloc(lb, qd, positions, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ga.attn_decode_noalloc(lb, qd, positions, out=out)
    for r in range(3):
        out.fill_(float("nan"))
        ga.attn_decode_noalloc(lb, qd[:1].contiguous(), positions[:1])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
    check_close(eager.cpu().numpy(),
                oracle_decode(ga.GLOBAL, q, streams, positions),
                "noalloc graph", ctx=max(positions) + 1)
