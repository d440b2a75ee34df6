"""A drafted block predicted together (gqa_attn_draft_block) on the GPU
against the fp64 oracle (oracle.attend_block_together): every block token
sees the cached context and the whole block.

Tolerance as the other block tests: max abs <= 2e-2, mean abs <= 2e-3.
Beyond random inputs: the cache is left untouched; a needle inside the block
is returned by every row, including the rows before it (which a causal
block would hide it from); the last row, whose visible set is the same
under both rules, equals the verify call's last row bit for bit; local
layers are refused."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import oracle
import synth_inputs as si
from tests._util import check_close, fill_layer, sentinel_cache
from tests.test_gpu_block import _setup, _snapshot, _unchanged

pytestmark = pytest.mark.gpu


def _oracle_together(q_cpu, streams, pos0, n):
    out = []
    for b, (k, v) in enumerate(streams):
        hi = pos0[b] + n
        out.append(oracle.attend_block_together(
            si.bits(q_cpu[b]), pos0[b], si.bits(k[:hi]), si.bits(v[:hi]), 0,
            hq=ga.HQ, hkv=ga.HKV, d=ga.D))
    return np.stack(out)


@pytest.mark.parametrize("n", [1, 5, 16])
def test_draft_ragged(n):
    pos0 = [0, 63, 2048, 5000]
    print("draft n=%d pos0=%s" % (n, pos0), flush=True)
    layer, streams, q, kb, vb = _setup(ga.GLOBAL, pos0, n, seed=2101 + n)
    snap = _snapshot(layer)
    out = ga.attn_draft_block(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    assert _unchanged(layer, snap), "the drafted block must not write the cache"
    want = _oracle_together(q, streams, pos0, n)
    check_close(out.cpu().numpy(), want, "draft n=%d" % n)


def test_draft_full_size_131056():
    pos0, n = [131056], 16
    print("draft full 131056+16", flush=True)
    layer, streams, q, kb, vb = _setup(ga.GLOBAL, pos0, n, seed=1104,
                                       capacity=ga.MAX_CONTEXT)
    out = ga.attn_draft_block(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    want = _oracle_together(q, streams, pos0, n)
    check_close(out.cpu().numpy(), want, "draft 131056+16", ctx=131072)


@pytest.mark.parametrize("needle", [0, 64 * 37 - 1, 64 * 37, 131055,
                                    131056, 131056 + 12, 131056 + 15])
def test_draft_needle(needle):
    """A key far above the rest at a split boundary, at the first or last
    context key, or inside the block: every row must match the oracle and
    return the needle's value -- also the rows before a needle inside the
    block."""
    pos0, n = [131056], 16
    k, v, u = si.needle_stream(si.seq_seed(1140, 0), pos0[0] + n, [needle],
                               1141, magnitude=16.0)
    layer = sentinel_cache(ga.GLOBAL, 1, ga.MAX_CONTEXT)
    fill_layer(layer, [(k, v)], [pos0[0] - 1])
    kb = k[pos0[0]:pos0[0] + n][None].contiguous()
    vb = v[pos0[0]:pos0[0] + n][None].contiguous()
    q = (u.float().repeat_interleave(16, dim=0) * 8.0).to(torch.bfloat16)
    q = q[None, None].expand(1, n, ga.HQ, ga.D).contiguous()
    print("draft needle at %d" % needle, flush=True)
    out = ga.attn_draft_block(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = _oracle_together(q, [(k, v)], pos0, n)
    check_close(got, want, "draft needle at %d" % needle, ctx=131072)
    target = np.repeat(v[needle].double().numpy(), 16, axis=0)
    for r in range(n):
        assert np.abs(got[0, r] - target).max() < 0.05, r


def test_draft_last_row_equals_verify():
    pos0, n = [777, 40000], 16
    print("draft vs verify last row", flush=True)
    layer, streams, q, kb, vb = _setup(ga.GLOBAL, pos0, n, seed=1150)
    d = ga.attn_draft_block(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    ver = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    assert torch.equal(d[:, n - 1], ver[:, n - 1])
    # the other rows see later block keys under this rule, so they differ
    assert (d[:, 0] - ver[:, 0]).abs().max().item() > 1e-4


def test_draft_local_layer_refused():
    layer = sentinel_cache(ga.LOCAL, 1)
    q = torch.zeros((1, 4, ga.HQ, ga.D), dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros((1, 4, ga.HKV, ga.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(ga.GqaError) as e:
        ga.attn_draft_block(layer, q, kb, kb, [100], ws=ws)
    assert e.value.status == -5
