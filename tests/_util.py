"""Shared helpers of the GPU parity tests: cache set-up through the library's
own append, oracle calls on the same bytes, and the tolerance check."""
import numpy as np
import torch

import global_gqa_attention_kv_amd as ga
import oracle
import synth_inputs as si

# bf16 inputs, fp32 accumulation, compared with the fp64 oracle
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# Beyond 32768 keys the outputs of N(0,1) inputs are small (RMS ~ sqrt(e/N):
# 0.005 at 131072), so the absolute bounds alone would pass a kernel that
# lost a tenth of the keys; there the largest error must also stay below a
# tenth of the output's RMS.
LONG_CONTEXT = 32768
MAX_REL_LONG = 0.1
# Two library paths that compute the same rows with bf16 outputs (a chunked
# prefill and a whole one) round at different points, so their outputs may
# sit on neighbouring bf16 values: one bf16 step is 2^-6 = 0.0156 for
# magnitudes in [2, 4).  Such comparisons allow the larger of SAME_ABS and
# one bf16 step at the element's magnitude.
SAME_ABS = 1e-2


def same_path_excess(a, b):
    """Largest amount by which |a - b| exceeds max(SAME_ABS, one bf16 step
    at max(|a|, |b|)), elementwise (<= 0 when the two outputs agree)."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    mag = np.maximum(np.abs(a), np.abs(b))
    step = np.spacing(mag) * np.float32(2 ** 16)  # bf16 keeps 8 of fp32's 24 bits
    return float((np.abs(a - b) - np.maximum(SAME_ABS, step)).max())


def sentinel_cache(kind, B, capacity=None, device="cuda"):
    """A layer whose caches are filled with the 0xFFFF bit pattern."""
    if capacity is None:
        capacity = ga.WINDOW if kind == ga.LOCAL else ga.MAX_CONTEXT
    shape = (B, capacity, ga.HKV, ga.D)
    k = torch.full(shape, -1, dtype=torch.int16, device=device).view(torch.bfloat16)
    v = torch.full(shape, -1, dtype=torch.int16, device=device).view(torch.bfloat16)
    return ga.Layer(kind, k, v)


def fill_layer(layer, streams, positions):
    """Append each sequence's logical stream up to and including its query
    position: global layers get positions 0..p, local layers the last 2048
    of them.  streams[b] = (k [n,2,128], v) on the CPU, row r = position r."""
    for b, (k, v) in enumerate(streams):
        p = positions[b]
        lo = 0 if layer.kind == ga.GLOBAL else max(0, p - ga.WINDOW + 1)
        kk = k[lo:p + 1].unsqueeze(0).contiguous().cuda()
        vv = v[lo:p + 1].unsqueeze(0).contiguous().cuda()
        sub = ga.Layer(layer.kind, layer.k[b:b + 1], layer.v[b:b + 1],
                       layer.rope_theta)
        ga.kv_append(sub, kk, vv, [lo])


def oracle_decode(kind, q_cpu, streams, positions):
    """fp64 oracle for one decode query per sequence."""
    outs = []
    for b, (k, v) in enumerate(streams):
        p = positions[b]
        lo = 0 if kind == ga.GLOBAL else max(0, p - ga.WINDOW + 1)
        outs.append(oracle.attend(
            si.bits(q_cpu[b:b + 1]), [p], si.bits(k[lo:p + 1]),
            si.bits(v[lo:p + 1]), lo, hq=ga.HQ, hkv=ga.HKV, d=ga.D,
            window=ga.WINDOW if kind == ga.LOCAL else 0,
            rope=kind == ga.LOCAL, theta=10000.0)[0])
    return np.stack(outs)


def check_close(got, want, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS,
                ctx=0, max_rel=None):
    """Element-wise comparison with the oracle.  ctx: the largest number of
    keys a compared row sees; beyond LONG_CONTEXT the max/RMS gate applies
    (max_rel overrides its bound)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    rms = float(np.sqrt(np.mean(want ** 2))) or 1.0
    msg = "%s: max abs %.3e, mean abs %.3e, max/rms %.3e" % (
        what, err.max(), err.mean(), err.max() / rms)
    print(msg, flush=True)
    assert np.isfinite(got).all(), what + ": non-finite output"
    assert err.max() <= max_abs and err.mean() <= mean_abs, msg
    if max_rel is None and ctx > LONG_CONTEXT:
        max_rel = MAX_REL_LONG
    if max_rel is not None:
        assert err.max() <= max_rel * rms, msg + " (max/rms gate %g)" % max_rel
    return err
