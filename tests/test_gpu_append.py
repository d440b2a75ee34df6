"""kv_append on the GPU against the integer cache oracle: bit-exact bytes,
ring wraparound, blocks longer than the ring, chunking invariance and
untouched sentinel slots."""
import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import oracle
import synth_inputs as si
from tests._util import sentinel_cache

pytestmark = pytest.mark.gpu


def _bits_gpu(t):
    return si.bits(t.cpu())


def _run(kind, capacity, B, chunks, seed):
    layer = sentinel_cache(kind, B, capacity)
    total = sum(chunks)
    appends = []
    streams = []
    for b in range(B):
        k, v = si.stream(si.seq_seed(seed, b), total)
        streams.append((k, v))
    pos = 0
    for n in chunks:
        kk = torch.stack([s[0][pos:pos + n] for s in streams]).cuda()
        vv = torch.stack([s[1][pos:pos + n] for s in streams]).cuda()
        ga.kv_append(layer, kk, vv, [pos] * B)
        for b in range(B):
            appends.append((b, pos, si.bits(streams[b][0][pos:pos + n]),
                            si.bits(streams[b][1][pos:pos + n])))
        pos += n
    torch.cuda.synchronize()
    K, V = oracle.expected_cache(kind, capacity, appends, nseq=B)
    return layer, K, V


@pytest.mark.parametrize("chunks", [[1] * 40, [5, 64, 3, 1, 100], [333],
                                    [4096], [1, 4095]])
def test_append_global_bit_exact(chunks):
    print("append global chunks", chunks[:5], flush=True)
    layer, K, V = _run(ga.GLOBAL, 4096, 2, chunks, seed=31)
    np.testing.assert_array_equal(_bits_gpu(layer.k), K)
    np.testing.assert_array_equal(_bits_gpu(layer.v), V)


@pytest.mark.parametrize("chunks", [[2047], [2048], [2049], [100, 2000, 7],
                                    [4096, 1], [1] * 10 + [3000, 2048, 5000],
                                    [32768]])
def test_append_local_ring_bit_exact(chunks):
    print("append local chunks", chunks[:5], flush=True)
    layer, K, V = _run(ga.LOCAL, ga.WINDOW, 2, chunks, seed=32)
    np.testing.assert_array_equal(_bits_gpu(layer.k), K)
    np.testing.assert_array_equal(_bits_gpu(layer.v), V)


def test_append_chunking_invariance_ring():
    a, _, _ = _run(ga.LOCAL, ga.WINDOW, 1, [32768], seed=33)
    b, _, _ = _run(ga.LOCAL, ga.WINDOW, 1, [1, 2, 4093, 8192, 20000, 480],
                   seed=33)
    assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16))
    assert torch.equal(a.v.view(torch.int16), b.v.view(torch.int16))


def test_append_full_global_capacity_edge():
    # the last slot of a full-size cache is writable, one past is rejected
    layer = sentinel_cache(ga.GLOBAL, 1, ga.MAX_CONTEXT)
    k, v = si.stream(34, 2)
    ga.kv_append(layer, k[None, :1].cuda(), v[None, :1].cuda(),
                 [ga.MAX_CONTEXT - 1])
    torch.cuda.synchronize()
    assert torch.equal(layer.k[0, -1].cpu().view(torch.int16),
                       k[0].view(torch.int16))
    assert (layer.k[0, :-1].view(torch.int16) == -1).all()
    with pytest.raises(ga.GqaError):
        ga.kv_append(layer, k[None].cuda(), v[None].cuda(),
                     [ga.MAX_CONTEXT - 1])
