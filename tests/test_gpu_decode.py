"""Decode attention on the GPU against the fp64 oracle.

Tolerance: max abs <= 2e-2 and mean abs <= 2e-3 (bf16 inputs, fp32
accumulation).  Besides random N(0,1) inputs the structured cases pin what a
tolerance alone could miss: a zero query must return the exact mean of V over
the visible window (window extent and ring contents), constant V must come
back unchanged (the split merge's weights sum to one), and a needle key placed
at tile, split and ring boundaries must dominate the output."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import synth_inputs as si
from tests._util import check_close, fill_layer, oracle_decode, sentinel_cache

pytestmark = pytest.mark.gpu


def _decode_case(kind, positions, seed, capacity=None, q_cpu=None,
                 streams=None):
    B = len(positions)
    print("decode kind=%d B=%d pos=%s seed=%d" % (kind, B, positions[:4], seed),
          flush=True)
    if streams is None:
        streams = [si.stream(si.seq_seed(seed, b), positions[b] + 1)
                   for b in range(B)]
    if q_cpu is None:
        q_cpu = torch.cat([si.queries(si.seq_seed(seed, b) + 7777, 1)
                           for b in range(B)])
    if capacity is None and kind == ga.GLOBAL:
        capacity = max(positions) + 1
    layer = sentinel_cache(kind, B, capacity)
    fill_layer(layer, streams, positions)
    out = ga.attn_decode(layer, q_cpu.cuda(), positions)
    torch.cuda.synchronize()
    want = oracle_decode(kind, q_cpu, streams, positions)
    return out.cpu().numpy(), want, streams, q_cpu


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_config_ctx4096(kind):
    # one local + one global layer, batch 1, context 4096 (query at 4095)
    got, want, _, _ = _decode_case(kind, [4095], seed=1001)
    check_close(got, want, "decode ctx4096 kind=%d" % kind)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_ragged_batch_and_edges(kind):
    positions = [0, 1, 62, 63, 64, 65, 127, 2046, 2047, 2048, 2049, 3000, 4095,
                 5001]
    got, want, _, _ = _decode_case(kind, positions, seed=1002)
    check_close(got, want, "decode ragged kind=%d" % kind)


def test_decode_global_wave_key_groups():
    """Global layers split each 64-key tile over four waves of 16 keys and
    merge the waves' sums at the end of the split: contexts of 1 .. 18 keys
    (only the first wave sees keys), tiles ending on and next to the 16-key
    group edges, and longer sequences whose last tile is partial, in one
    ragged batch."""
    positions = list(range(18)) + [31, 32, 47, 48, 63, 64 * 40 + 5,
                                    20000 + 17]
    got, want, _, _ = _decode_case(ga.GLOBAL, positions, seed=1012)
    check_close(got, want, "decode global wave groups")


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_full_context_131072(kind):
    got, want, _, _ = _decode_case(
        kind, [131071], seed=1003,
        capacity=ga.MAX_CONTEXT if kind == ga.GLOBAL else None)
    check_close(got, want, "decode ctx131072 kind=%d" % kind,
                ctx=131072 if kind == ga.GLOBAL else ga.WINDOW)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_max_batch_64(kind):
    # the largest batch the library takes, ragged positions up to 6000:
    # the planner's smallest split count per sequence
    positions = [int(x) for x in np.random.default_rng(64).integers(0, 6000, 64)]
    positions[0], positions[-1] = 0, 5999
    got, want, _, _ = _decode_case(kind, positions, seed=1010)
    check_close(got, want, "decode B=64 kind=%d" % kind)


def test_decode_batch4_131072_global():
    positions = [131071, 131071, 100000, 77777]
    got, want, _, _ = _decode_case(ga.GLOBAL, positions, seed=1004,
                                   capacity=ga.MAX_CONTEXT)
    check_close(got, want, "decode B=4 ctx131072 global", ctx=131072)


@pytest.mark.parametrize("kind,p", [(ga.LOCAL, 5000), (ga.LOCAL, 1000),
                                    (ga.GLOBAL, 70000), (ga.GLOBAL, 130)])
def test_decode_zero_query_is_window_mean(kind, p):
    streams = [si.stream(si.seq_seed(1005, 0), p + 1)]
    q = torch.zeros(1, ga.HQ, ga.D, dtype=torch.bfloat16)
    got, want, streams, _ = _decode_case(kind, [p], seed=1005, q_cpu=q,
                                         streams=streams)
    lo = 0 if kind == ga.GLOBAL else max(0, p - ga.WINDOW + 1)
    v = streams[0][1][lo:p + 1].double().numpy()
    mean = v.mean(axis=0)
    exact = np.repeat(mean, ga.HQ // ga.HKV, axis=0)
    np.testing.assert_allclose(want[0], exact, atol=1e-12)
    # uniform weights 1 are exact in bf16, so only summation order differs
    err = np.abs(got[0] - exact).max()
    print("zero-query mean err %.3e" % err, flush=True)
    assert err < 1e-4


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_constant_v(kind):
    p = 20000 if kind == ga.GLOBAL else 9000
    k, v = si.stream(si.seq_seed(1006, 0), p + 1)
    v = torch.full_like(v, 0.75)
    got, _, _, _ = _decode_case(kind, [p], seed=1006, streams=[(k, v)])
    err = np.abs(got - 0.75).max()
    print("constant-V err %.3e" % err, flush=True)
    assert err < 1e-5


@pytest.mark.parametrize("kind,p,needle", [
    (ga.GLOBAL, 131071, 0), (ga.GLOBAL, 131071, 131071),
    (ga.GLOBAL, 131071, 64 * 37), (ga.GLOBAL, 131071, 64 * 37 - 1),
    (ga.GLOBAL, 50000, 49999), (ga.GLOBAL, 40, 15), (ga.GLOBAL, 40, 16),
    (ga.GLOBAL, 3000, 64 * 20 + 47), (ga.GLOBAL, 3000, 64 * 20 + 48),
    (ga.LOCAL, 131071, 131071 - 2047),
    (ga.LOCAL, 131071, 131071), (ga.LOCAL, 10000, 10000 - 2047 + 64),
    (ga.LOCAL, 4095, 2048), (ga.LOCAL, 4095, 2047 + 2048)])
def test_decode_needle(kind, p, needle):
    k, v, u = si.needle_stream(si.seq_seed(1007, 0), p + 1, [needle], 1008,
                               magnitude=16.0)
    q = (u.float().repeat_interleave(16, dim=0) * 8.0).to(torch.bfloat16)[None]
    capacity = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    got, want, _, _ = _decode_case(kind, [p], seed=1007, q_cpu=q,
                                   streams=[(k, v)], capacity=capacity)
    check_close(got, want, "needle kind=%d p=%d at %d" % (kind, p, needle),
                ctx=p + 1 if kind == ga.GLOBAL else ga.WINDOW)
    vn = v[needle].double().numpy()
    target = np.repeat(vn, 16, axis=0)
    if kind == ga.LOCAL:
        # RoPE turns the needle's score with its relative offset; the
        # oracle decides how strongly it wins, the kernel must agree
        return
    assert np.abs(got[0] - target).max() < 0.05


def test_decode_matches_after_second_call_same_workspace():
    # the workspace carries nothing between calls: reuse it across shapes
    kind = ga.GLOBAL
    ws = ga.workspace(ga.OP_DECODE, kind, 4, 1, 131072)
    for positions in ([131071, 5, 70000, 64], [300]):
        B = len(positions)
        streams = [si.stream(si.seq_seed(1009, b), positions[b] + 1)
                   for b in range(B)]
        q = torch.cat([si.queries(si.seq_seed(1009, b) + 1, 1) for b in range(B)])
        layer = sentinel_cache(kind, B, ga.MAX_CONTEXT)
        fill_layer(layer, streams, positions)
        out = ga.attn_decode(layer, q.cuda(), positions, ws=ws)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), oracle_decode(kind, q, streams, positions),
                    "ws reuse %s" % positions[:2])


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_append_fused(kind):
    """decode_append = append the token at pos, then attend: the output must
    match the oracle over the stream including the new token, and the cache
    must hold the new token's bytes at its slot afterwards.  Repeated over
    consecutive positions with one shared workspace."""
    positions = [4095, 2047, 131069 if kind == ga.GLOBAL else 70000, 64]
    B = len(positions)
    streams = [si.stream(si.seq_seed(1010, b), positions[b] + 3)
               for b in range(B)]
    cap = ga.MAX_CONTEXT if kind == ga.GLOBAL else None
    layer = sentinel_cache(kind, B, cap)
    fill_layer(layer, streams, [p - 1 for p in positions])
    ws = ga.workspace(ga.OP_DECODE, kind, B, 1, max(positions) + 3)
    for step in range(3):
        pos = [p + step for p in positions]
        q = torch.cat([si.queries(si.seq_seed(1010, b) + 100 + step, 1)
                       for b in range(B)])
        kn = torch.stack([streams[b][0][pos[b]:pos[b] + 1] for b in range(B)])
        vn = torch.stack([streams[b][1][pos[b]:pos[b] + 1] for b in range(B)])
        print("decode_append kind=%d step %d pos=%s" % (kind, step, pos),
              flush=True)
        out = ga.attn_decode_append(layer, q.cuda(), kn.cuda(), vn.cuda(), pos,
                                    ws=ws)
        torch.cuda.synchronize()
        want = oracle_decode(kind, q, streams, pos)
        check_close(out.cpu().numpy(), want, "decode_append step %d" % step)
        for b in range(B):
            slot = pos[b] if kind == ga.GLOBAL else pos[b] % ga.WINDOW
            assert torch.equal(layer.k[b, slot].cpu().view(torch.int16),
                               kn[b, 0].view(torch.int16))
            assert torch.equal(layer.v[b, slot].cpu().view(torch.int16),
                               vn[b, 0].view(torch.int16))


def test_one_workspace_for_every_operation_and_kind():
    """One workspace, sized for the largest request, serves global and
    local decode, verify and prefill in any order: no call may depend on
    what an earlier call of another kind left in it."""
    B = 4
    pos_l = [5000, 2047, 3000, 64]
    pos_g = [8000, 5, 4000, 64]
    sl = [si.stream(si.seq_seed(1011, b), pos_l[b] + 1) for b in range(B)]
    sg = [si.stream(si.seq_seed(1012, b), pos_g[b] + 1) for b in range(B)]
    loc = sentinel_cache(ga.LOCAL, B)
    glo = sentinel_cache(ga.GLOBAL, B, 8192)
    fill_layer(loc, sl, pos_l)
    fill_layer(glo, sg, pos_g)
    need = max(ga.workspace_bytes(op, kind, B, n, 8192)
               for op, n in ((ga.OP_DECODE, 1), (ga.OP_VERIFY, 16),
                             (ga.OP_PREFILL, 300))
               for kind in (ga.LOCAL, ga.GLOBAL))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    g = torch.Generator().manual_seed(1013)
    qb = torch.randn((B, 16, ga.HQ, ga.D), generator=g).to(torch.bfloat16).cuda()
    kb = torch.randn((B, 16, ga.HKV, ga.D), generator=g).to(torch.bfloat16).cuda()
    vb = torch.randn((B, 16, ga.HKV, ga.D), generator=g).to(torch.bfloat16).cuda()
    qp = torch.randn((1, 300, ga.HQ, ga.D), generator=g).to(torch.bfloat16).cuda()
    kp = torch.randn((1, 300, ga.HKV, ga.D), generator=g).to(torch.bfloat16).cuda()
    vp = torch.randn((1, 300, ga.HKV, ga.D), generator=g).to(torch.bfloat16).cuda()
    want_l = None
    others = [
        lambda: ga.attn_decode(glo, qb[:, 0].contiguous(), pos_g, ws=ws),
        lambda: ga.attn_verify(glo, qb, kb, vb, [p + 1 for p in pos_g], ws=ws),
        lambda: ga.attn_verify(loc, qb, kb, vb, [p + 1 for p in pos_l], ws=ws),
        lambda: ga.attn_prefill(loc, qp, kp, vp, [4096], ws=ws),
        lambda: ga.attn_prefill(glo, qp, kp, vp, [4096], ws=ws),
    ]
    for i, other in enumerate(others * 2):
        print("shared workspace: call %d, then a local decode" % i, flush=True)
        other()
        q = torch.cat([si.queries(si.seq_seed(1011, b) + 50 + i, 1)
                       for b in range(B)])
        out = ga.attn_decode(loc, q.cuda(), pos_l, ws=ws)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), oracle_decode(ga.LOCAL, q, sl, pos_l),
                    "local decode after call %d" % i)
