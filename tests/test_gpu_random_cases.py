"""Randomly drawn shapes (fixed seed) for every attention call against the
fp64 oracle: decode, verify, the drafted block and prefill, both layer kinds,
ragged batches of 1-6 sequences whose positions mix short (< 200) and long
(up to 20000) contexts, 1-16 block tokens for verify and the drafted block
and 1-700 for prefill.  Tolerance as everywhere: max abs <= 2e-2, mean abs
<= 2e-3.  Prefill compares its first two, last two and 40 sampled rows,
the other calls every row."""
import random

import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
from tests._util import check_close
from tests.test_gpu_block import _oracle_rows, _setup
from tests.test_gpu_decode import _decode_case
from tests.test_gpu_draft import _oracle_together

pytestmark = pytest.mark.gpu

N_CASES = 96


def _cases():
    rng = random.Random(20261203)
    out = []
    for _ in range(N_CASES):
        op = rng.choice(["decode", "verify", "prefill", "draft"])
        kind = ga.GLOBAL if op == "draft" else rng.choice([ga.LOCAL, ga.GLOBAL])
        B = rng.randint(1, 6)
        seed = rng.randint(1, 10 ** 6)
        if op == "decode":
            pos = [rng.choice([rng.randint(0, 200), rng.randint(0, 20000)])
                   for _ in range(B)]
            out.append((op, kind, pos, 1, seed))
        else:
            n = rng.randint(1, 16) if op != "prefill" else rng.randint(1, 700)
            pos0 = [rng.choice([rng.randint(0, 100), rng.randint(0, 12000)])
                    for _ in range(B)]
            rows = (list(range(n)) if n <= 48 else sorted(
                set([0, 1, n - 2, n - 1] + rng.sample(range(n), 40))))
            out.append((op, kind, pos0, n, seed, rows))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "%s-%d" % (c[0], c[1]))
def test_random_case(case):
    op, kind = case[0], case[1]
    what = "%s kind=%d pos=%s n=%d seed=%d" % (op, kind, case[2], case[3],
                                               case[4])
    print(what, flush=True)
    if op == "decode":
        got, want, _, _ = _decode_case(kind, case[2], case[4])
        check_close(got, want, what)
        return
    pos0, n, seed, rows = case[2], case[3], case[4], case[5]
    layer, streams, q, kb, vb = _setup(
        kind, pos0, n, seed,
        capacity=max(pos0) + n if kind == ga.GLOBAL else None)
    call = {"verify": ga.attn_verify, "draft": ga.attn_draft_block,
            "prefill": ga.attn_prefill}[op]
    out = call(layer, q.cuda(), kb.cuda(), vb.cuda(), pos0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    if op == "draft":
        want = _oracle_together(q, streams, pos0, n)
    else:
        want = _oracle_rows(kind, q, streams, pos0, rows)
        got = got[:, rows]
    check_close(got, want, what)
