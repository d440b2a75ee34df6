"""Speculative decoding rounds on the GPU: verify a drafted block of 16,
commit only the accepted prefix with kv_append, draft again from the new
position.  The pages describe the drafter proposing a block that the main
model checks in one pass, causal within the block, and only accepted tokens
becoming part of the sequence ("Deep dive into Muse Glimmer", section 04;
"Meta open-sources the 30B Muse Glimmer", "Trick 3: D-Flash").

Acceptance counts are synthetic and differ between the two sequences, so
their positions drift apart; a count of 0 commits nothing, 16 the whole
block.  Each round's verify output is compared with the fp64 oracle over the
committed prefix plus that round's block, which also checks that rejected
drafts never reached the cache (a local ring overwritten by a rejected draft
would change the window of later rounds)."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import oracle
import synth_inputs as si
from tests._util import check_close, fill_layer, sentinel_cache

pytestmark = pytest.mark.gpu

ACCEPTS = [[5, 16], [0, 7], [16, 1], [3, 0]]


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_verify_commit_rounds(kind):
    B, n = 2, 16
    pos0 = [3000, 9000]
    prefix = [si.stream(si.seq_seed(4100, b), pos0[b]) for b in range(B)]
    layer = sentinel_cache(kind, B, 10000 if kind == ga.GLOBAL else None)
    fill_layer(layer, prefix, [p - 1 for p in pos0])
    for rnd, accepts in enumerate(ACCEPTS):
        blocks = [si.stream(si.seq_seed(4101 + rnd, b), n) for b in range(B)]
        q = torch.stack([si.queries(si.seq_seed(4120 + rnd, b), n)
                         for b in range(B)])
        kb = torch.stack([blk[0] for blk in blocks])
        vb = torch.stack([blk[1] for blk in blocks])
        print("round %d pos0=%s accept=%s kind=%d" % (rnd, pos0, accepts, kind),
              flush=True)
        out = ga.attn_verify(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
        torch.cuda.synchronize()
        want = []
        for b in range(B):
            k_all = torch.cat([prefix[b][0], blocks[b][0]])
            v_all = torch.cat([prefix[b][1], blocks[b][1]])
            qpos = [pos0[b] + r for r in range(n)]
            lo = 0 if kind == ga.GLOBAL else max(0, pos0[b] - ga.WINDOW + 1)
            want.append(oracle.attend(
                si.bits(q[b]), qpos, si.bits(k_all[lo:]), si.bits(v_all[lo:]),
                lo, hq=ga.HQ, hkv=ga.HKV, d=ga.D,
                window=ga.WINDOW if kind == ga.LOCAL else 0,
                rope=kind == ga.LOCAL, theta=10000.0))
        check_close(out.cpu().numpy(), np.stack(want),
                    "round %d kind=%d" % (rnd, kind))
        # commit the accepted prefix of each sequence
        for b in range(B):
            a = accepts[b]
            if a == 0:
                continue
            sub = ga.Layer(kind, layer.k[b:b + 1], layer.v[b:b + 1])
            ga.kv_append(sub, kb[b:b + 1, :a].contiguous().cuda(),
                         vb[b:b + 1, :a].contiguous().cuda(), [pos0[b]])
            prefix[b] = (torch.cat([prefix[b][0], blocks[b][0][:a]]),
                         torch.cat([prefix[b][1], blocks[b][1][:a]]))
            pos0[b] += a
