"""The fp8 (E4M3) KV cache on the GPU against the oracle.

Append: the codes and scales the library writes must equal the oracle's
quantiser bit for bit (oracle/fp8.py: one fp32 scale per token and KV head,
s = amax / 448, round-to-nearest-even of clamp(x / s, +-448)), in the slots
the bf16 cache uses (global: position; local ring: position mod 2048, the
latest write wins), for chunkings from 1 token to more than the ring, with
slots never written left untouched, and on rows with edge values (zero and
negative-zero rows, values far below a row's maximum that land on E4M3
subnormals or zero, a row spanning 2^-40 .. 2^40).

Decode: attention over the fp8 cache against the oracle's attention over the
dequantised values of its own quantisation of the same bf16 stream (nothing
of the GPU's cache feeds the expected values), max abs <= 2e-2 and mean abs
<= 2e-3, at context 4096, ragged batches across tile and ring edges, the full
131072 context, a zero query (exact mean of the dequantised values), constant
V and needles."""
import random

import numpy as np
import pytest
import torch

import global_gqa_attention_kv_amd as ga
import synth_inputs as si
from oracle import fp8
from tests._util import check_close

pytestmark = pytest.mark.gpu

SENT_CODE = 0xA5


def _sentinel_layer(kind, B, capacity=None):
    layer = ga.LayerFp8.allocate(kind, B, capacity, device="cuda",
                                 fill=SENT_CODE)
    layer.k_scale.fill_(-1.0)       # the quantiser never writes a negative
    layer.v_scale.fill_(-1.0)
    return layer


def _expected(kind, capacity, appends, B):
    """Oracle cache contents: codes [B, cap, 2, 128] and scales
    [B, 2, cap] after the appends (b, pos0, k bits, v bits)."""
    kc = np.full((B, capacity, 2, 128), SENT_CODE, dtype=np.uint8)
    vc = kc.copy()
    ks = np.full((B, 2, capacity), -1.0, dtype=np.float32)
    vs = ks.copy()
    for b, pos0, kb, vb in appends:      # in order: the latest write wins
        ck, sk = fp8.quantize(kb)
        cv, sv = fp8.quantize(vb)
        pos = pos0 + np.arange(kb.shape[0])
        slot = pos if kind == ga.GLOBAL else pos % ga.WINDOW
        assert len(np.unique(slot)) == len(slot)   # <= 2048 kept per append
        kc[b, slot], vc[b, slot] = ck, cv
        ks[b, :, slot], vs[b, :, slot] = sk, sv
    return kc, vc, ks, vs


def _check_cache(layer, want):
    kc, vc, ks, vs = want
    assert np.array_equal(layer.k.cpu().numpy(), kc), "K codes differ"
    assert np.array_equal(layer.v.cpu().numpy(), vc), "V codes differ"
    # scales bit for bit
    assert np.array_equal(layer.k_scale.cpu().numpy().view(np.uint32),
                          ks.view(np.uint32)), "K scales differ"
    assert np.array_equal(layer.v_scale.cpu().numpy().view(np.uint32),
                          vs.view(np.uint32)), "V scales differ"


def _edge_stream(seed, n):
    """A bf16 K/V stream of n tokens with edge rows planted: zero rows,
    negative-zero rows, rows whose small entries fall to E4M3 subnormals or
    to zero next to a large maximum, and a row spanning 2^-40 .. 2^40."""
    k, v = si.stream(seed, n)
    for x in (k, v):
        x[3] = 0.0
        x[4] = -0.0
        if n > 10:
            x[5, 0] = (x[5, 0].float() * 1e-4).to(torch.bfloat16)
            x[5, 0, 7] = 3.0
            x[6, 1] = (x[6, 1].float() * 2.0 ** -16).to(torch.bfloat16)
            x[6, 1, 0] = 1.0
            x[7, 0] = torch.tensor(
                [2.0 ** (-40 + 80 * i / 127) for i in range(128)]).to(
                    torch.bfloat16)
            x[8, 1] = -x[8, 1].abs()
    return k, v


@pytest.mark.parametrize("kind,total,chunks", [
    (ga.GLOBAL, 5000, [1, 7, 64, 1000, 3928]),
    (ga.GLOBAL, 131072, [131072]),
    (ga.LOCAL, 9000, [1, 2047, 2, 64, 4096, 2790]),
    (ga.LOCAL, 32768, [32768])])
def test_append_fp8_bit_exact(kind, total, chunks):
    assert sum(chunks) == total
    print("append fp8 kind=%d total=%d chunks=%s" % (kind, total, chunks),
          flush=True)
    cap = min(total + 100, ga.MAX_CONTEXT) if kind == ga.GLOBAL else None
    B = 2
    layer = _sentinel_layer(kind, B, cap)
    appends = []
    for b in range(B):
        k, v = _edge_stream(si.seq_seed(8001, b), total)
        p0 = 0
        for c in chunks:
            sub = ga.LayerFp8(kind, layer.k[b:b + 1], layer.v[b:b + 1],
                              layer.k_scale[b:b + 1], layer.v_scale[b:b + 1])
            ga.kv_append_fp8(sub, k[None, p0:p0 + c].contiguous().cuda(),
                             v[None, p0:p0 + c].contiguous().cuda(), [p0])
            # a block longer than the ring only keeps its last 2048 tokens
            keep = max(0, c - ga.WINDOW) if kind == ga.LOCAL else 0
            appends.append((b, p0 + keep, si.bits(k[p0 + keep:p0 + c]),
                            si.bits(v[p0 + keep:p0 + c])))
            p0 += c
    torch.cuda.synchronize()
    _check_cache(layer, _expected(kind, layer.capacity, appends, B))


def _fill(kind, streams, positions, capacity=None):
    """An fp8 cache holding each sequence's stream up to its query position
    (global: 0..p; local: the last 2048 of them) via the library's append;
    returns the layer and the oracle's quantisation of the same rows."""
    B = len(positions)
    layer = _sentinel_layer(kind, B, capacity)
    quant = []
    for b, (k, v) in enumerate(streams):
        p = positions[b]
        lo = 0 if kind == ga.GLOBAL else max(0, p - ga.WINDOW + 1)
        sub = ga.LayerFp8(kind, layer.k[b:b + 1], layer.v[b:b + 1],
                          layer.k_scale[b:b + 1], layer.v_scale[b:b + 1])
        ga.kv_append_fp8(sub, k[None, lo:p + 1].contiguous().cuda(),
                         v[None, lo:p + 1].contiguous().cuda(), [lo])
        kc, ks = fp8.quantize(si.bits(k[lo:p + 1]))
        vc, vs = fp8.quantize(si.bits(v[lo:p + 1]))
        quant.append((lo, kc, ks, vc, vs))
    return layer, quant


def _oracle(kind, q, positions, quant):
    out = []
    for b, p in enumerate(positions):
        lo, kc, ks, vc, vs = quant[b]
        out.append(fp8.attend(si.bits(q[b:b + 1]), [p], kc, ks, vc, vs, lo,
                              hq=ga.HQ, hkv=ga.HKV, d=ga.D,
                              window=ga.WINDOW if kind == ga.LOCAL else 0,
                              rope=kind == ga.LOCAL, theta=10000.0)[0])
    return np.stack(out)


def _case(kind, positions, seed, capacity=None, q=None, streams=None):
    B = len(positions)
    print("decode fp8 kind=%d B=%d pos=%s" % (kind, B, positions[:4]),
          flush=True)
    if streams is None:
        streams = [si.stream(si.seq_seed(seed, b), positions[b] + 1)
                   for b in range(B)]
    if q is None:
        q = torch.cat([si.queries(si.seq_seed(seed, b) + 99, 1)
                       for b in range(B)])
    if capacity is None and kind == ga.GLOBAL:
        capacity = max(positions) + 1
    layer, quant = _fill(kind, streams, positions, capacity)
    out = ga.attn_decode_fp8(layer, q.cuda(), positions)
    torch.cuda.synchronize()
    return out.cpu().numpy(), _oracle(kind, q, positions, quant), quant


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_fp8_ctx4096(kind):
    got, want, _ = _case(kind, [4095], 8101)
    check_close(got, want, "decode fp8 ctx4096 kind=%d" % kind)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_fp8_ragged(kind):
    positions = [0, 1, 15, 16, 63, 64, 65, 2046, 2047, 2048, 2049, 3000,
                 4095, 5001]
    got, want, _ = _case(kind, positions, 8102)
    check_close(got, want, "decode fp8 ragged kind=%d" % kind)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_fp8_max_batch_64(kind):
    """The largest batch the library takes: 64 sequences at ragged positions
    0 .. 2999 (position 0 first, a wrapped local ring last)."""
    rng = random.Random(8111 + kind)
    positions = [rng.randrange(0, 3000) for _ in range(ga.MAX_BATCH)]
    positions[0], positions[-1] = 0, 2999
    got, want, _ = _case(kind, positions, 8111,
                         capacity=3008 if kind == ga.GLOBAL else None)
    check_close(got, want, "decode fp8 B=64 kind=%d" % kind)


@pytest.mark.parametrize("kind,positions", [
    (ga.LOCAL, [131071]), (ga.GLOBAL, [131071]),
    (ga.GLOBAL, [131071, 77777, 4100, 64 * 500])])
def test_decode_fp8_full_context(kind, positions):
    got, want, _ = _case(kind, positions, 8103,
                         capacity=ga.MAX_CONTEXT if kind == ga.GLOBAL
                         else None)
    check_close(got, want, "decode fp8 ctx131072 kind=%d B=%d" %
                (kind, len(positions)),
                ctx=max(positions) + 1 if kind == ga.GLOBAL else ga.WINDOW)


@pytest.mark.parametrize("kind,p", [(ga.LOCAL, 5000), (ga.GLOBAL, 70000)])
def test_decode_fp8_zero_query_is_dequantised_mean(kind, p):
    q = torch.zeros(1, ga.HQ, ga.D, dtype=torch.bfloat16)
    got, want, quant = _case(kind, [p], 8104, q=q)
    lo, kc, ks, vc, vs = quant[0]
    mean = fp8.dequantize(vc, vs).mean(axis=0)
    exact = np.repeat(mean, ga.HQ // ga.HKV, axis=0)
    np.testing.assert_allclose(want[0], exact, atol=1e-12)
    # weights are all 1; each value goes through bf16(1 * v scale), so the
    # only rounding is that product's (relative 2^-8 per term) and fp32 sums
    err = np.abs(got[0] - exact).max()
    print("fp8 zero-query mean err %.3e" % err, flush=True)
    assert err < 2e-4


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_decode_fp8_constant_v(kind):
    p = 20000 if kind == ga.GLOBAL else 9000
    k, v = si.stream(si.seq_seed(8105, 0), p + 1)
    v = torch.full_like(v, 0.75)
    got, _, quant = _case(kind, [p], 8105, streams=[(k, v)])
    # constant rows quantise to code 448 with scale 0.75 / 448
    assert (quant[0][3] == 0x7E).all()
    err = np.abs(got - 0.75).max()
    print("fp8 constant-V err %.3e" % err, flush=True)
    assert err < 1e-3


@pytest.mark.parametrize("kind,p,needle", [
    (ga.GLOBAL, 131071, 0), (ga.GLOBAL, 131071, 131071),
    (ga.GLOBAL, 131071, 64 * 1000 - 1), (ga.GLOBAL, 131071, 64 * 1000),
    (ga.GLOBAL, 3000, 64 * 20 + 47), (ga.GLOBAL, 3000, 64 * 20 + 48),
    (ga.LOCAL, 131071, 131071 - 2047), (ga.LOCAL, 131071, 131071),
    (ga.LOCAL, 4095, 2048), (ga.LOCAL, 4095, 2047 + 2048)])
def test_decode_fp8_needle(kind, p, needle):
    k, v, u = si.needle_stream(si.seq_seed(8106, 0), p + 1, [needle], 8107,
                               magnitude=16.0)
    q = (u.float().repeat_interleave(16, dim=0) * 8.0).to(torch.bfloat16)[None]
    got, want, quant = _case(kind, [p], 8106, q=q, streams=[(k, v)],
                             capacity=ga.MAX_CONTEXT if kind == ga.GLOBAL
                             else None)
    check_close(got, want, "fp8 needle kind=%d p=%d at %d" % (kind, p, needle),
                ctx=p + 1 if kind == ga.GLOBAL else ga.WINDOW)
    if kind == ga.GLOBAL:
        lo, kc, ks, vc, vs = quant[0]
        target = np.repeat(fp8.dequantize(vc[needle - lo:needle - lo + 1],
                                          vs[needle - lo:needle - lo + 1])[0],
                           16, axis=0)
        assert np.abs(got[0] - target).max() < 0.05
