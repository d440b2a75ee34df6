"""Benchmark of the hybrid local/global GQA attention path on one MI355X.

Default workload: one full 52-layer decode step (three local layers then one
global, repeated 13 times) at the maximum context of 131072 tokens, batch 4
(independent sequences).  A step is, for every layer in order: append the new
token's K/V to the layer cache and attend (split-K decode + merge), fused
into one call per layer.  The 52
layers run on one stream, captured once as a HIP graph and replayed.

Printed: ONE JSON line.  ``value`` = KV bytes the step must read (every
visible key of every layer, 1024 B per token per layer) / step time, in GB/s.
``roofline`` covers the dominant kernel, the global-layer decode at 131072
keys, timed with HIP events on the stream it is launched on.  ``cpu_baseline``
is the fp64 oracle timed on this host on a bounded sample of the same
workload.

Inputs are synthetic: caches and queries are i.i.d. N(0,1) bf16 drawn from
seeded generators on the GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
N_LAYERS = 52
CTX = 131072


def _ensure_built():
    import global_gqa_attention_kv_amd as ga
    if not os.path.exists(ga.library_path()):
        from global_gqa_attention_kv_amd import build
        build.build()
    return ga


def measured_traffic(B):
    """HBM bytes per launch of the global-layer decode kernel from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by a plain copy
    (profiles/decode_131072_hbm_counters.md).  None when the
    counters were taken on other kernel sources or another batch size."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "decode_global_traffic.json")) as f:
            rec = json.load(f)
        csrc = os.path.join(ROOT, "global_gqa_attention_kv_amd", "csrc")
        h = hashlib.sha256(b"".join(
            open(os.path.join(csrc, n), "rb").read()
            for n in ("decode.hip", "device_common.h", "internal.h"))).hexdigest()
    except (OSError, ValueError):
        return None
    if h != rec.get("source_sha256") or B != 4:
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def kv_bytes_step(kinds, positions):
    """Algorithmic KV bytes of one decode step: each layer reads every
    visible key's K and V for both KV heads (1024 B per token)."""
    total = 0
    for kind in kinds:
        for p in positions:
            keys = p + 1 if kind == 1 else min(p + 1, 2048)
            total += keys * 1024
    return total


def build_decode_step(ga, torch, B, pos, seed=1003):
    dev = torch.device("cuda")
    kinds = [ga.layer_kind(l) for l in range(N_LAYERS)]
    gen = torch.Generator(device=dev)
    layers, qs, knews, vnews = [], [], [], []
    for l, kind in enumerate(kinds):
        gen.manual_seed(seed * 1000 + l)
        cap = ga.WINDOW if kind == ga.LOCAL else CTX
        shape = (B, cap, ga.HKV, ga.D)
        k = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
        layers.append(ga.Layer(kind, k, v))
        qs.append(torch.randn((B, ga.HQ, ga.D), generator=gen,
                              device=dev).to(torch.bfloat16))
        knews.append(torch.randn((B, 1, ga.HKV, ga.D), generator=gen,
                                 device=dev).to(torch.bfloat16))
        vnews.append(torch.randn((B, 1, ga.HKV, ga.D), generator=gen,
                                 device=dev).to(torch.bfloat16))
    ws = torch.empty(max(ga.workspace_bytes(ga.OP_DECODE, k, B, 1, CTX)
                         for k in (ga.LOCAL, ga.GLOBAL)),
                     dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, ga.HQ, ga.D), dtype=torch.float32, device=dev)
            for _ in kinds]
    positions = [pos] * B

    def step():
        for l in range(N_LAYERS):
            ga.attn_decode_append(layers[l], qs[l], knews[l], vnews[l],
                                  positions, outs[l], ws)

    def step_kind(kind):
        def f():
            for l in range(N_LAYERS):
                if kinds[l] == kind:
                    ga.attn_decode_append(layers[l], qs[l], knews[l],
                                          vnews[l], positions, outs[l], ws)
        return f

    step.local_only = step_kind(ga.LOCAL)
    step.global_only = step_kind(ga.GLOBAL)
    step.knews, step.vnews = knews, vnews
    return kinds, layers, qs, outs, ws, positions, step


def check_step_outputs(ga, torch, layers, qs, outs, positions, kinds):
    """The replayed step shares one workspace across all 52 layers; a
    local and a global layer's outputs must equal a fresh eager call's with
    a workspace of its own (same kernels, same merge order: bit-identical)."""
    for l in (kinds.index(ga.LOCAL), kinds.index(ga.GLOBAL)):
        again = ga.attn_decode(layers[l], qs[l], positions)
        torch.cuda.synchronize()
        diff = (again - outs[l]).abs().max().item()
        if not diff <= 1e-6:
            raise RuntimeError("decode step output of layer %d differs from "
                               "an eager call by %g" % (l, diff))


def bench_decode_b1(ga, torch, steps, warmup):
    """Single-sequence decode steps (append + attend per layer, HIP graph):
    one local + one global layer at context 4096, and all 52 layers at
    contexts 32768 and 131072."""
    res = {}
    for ctx in (4096, 32768, CTX):
        kinds, layers, qs, outs, ws, positions, step = build_decode_step(
            ga, torch, 1, ctx - 1)
        if ctx == 4096:
            pair = [kinds.index(ga.LOCAL), kinds.index(ga.GLOBAL)]

            def fn():
                for l in pair:
                    ga.attn_decode_append(layers[l], qs[l], step.knews[l],
                                          step.vnews[l], positions, outs[l], ws)
            ms, _, _ = time_graph(torch, fn, steps, warmup)
            nbytes = sum(kv_bytes_step([kinds[l]], positions) for l in pair)
            name, what = "b1_ctx4096_1local_1global", "2 layers"
        else:
            ms, _, _ = time_graph(torch, step, steps, warmup)
            nbytes = kv_bytes_step(kinds, positions)
            name, what = "b1_ctx%d_52layers" % ctx, "52 layers"
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"us_per_step": round(ms * 1000, 2), "kv_GBps": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "layers": what}
        del layers, qs, outs, ws, step
        torch.cuda.empty_cache()
    return res


def time_graph(torch, fn, steps, warmup):
    """Capture fn once in a HIP graph, replay it `warmup` times untimed,
    then `steps` times with an event between replays.  Returns (median ms
    per replay, the graph, mean ms per replay)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager run once before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return median(per), g, sum(per) / len(per)


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def time_global_decode(ga, torch, layers, qs, outs, ws, positions, kinds,
                       reps):
    """Duration of one global-layer decode call (split kernel + merge
    kernel) at the step's context, rotating over the 13 global layers so the
    256 MB last-level cache cannot serve repeats.  HIP events on the stream
    the calls are launched on, one between consecutive calls.  Returns
    (mean ms, median ms) per call."""
    glob = [l for l, k in enumerate(kinds) if k == ga.GLOBAL]
    for l in glob:
        ga.attn_decode(layers[l], qs[l], positions, outs[l], ws)
    torch.cuda.synchronize()
    calls = [l for _ in range(reps) for l in glob]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    ev[0].record()
    for i, l in enumerate(calls):
        ga.attn_decode(layers[l], qs[l], positions, outs[l], ws)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(calls))]
    return sum(per) / len(per), median(per)


FP8_TOKEN_BYTES = 2 * 128 * 2 + 2 * 2 * 4  # codes + scales, K and V


def bench_decode_fp8(ga, torch, layers, qs, outs, ws, positions, kinds,
                     steps, warmup, kernel_reps):
    """The 52-layer decode step over fp8 caches (E4M3 codes plus one fp32
    scale per token and KV head): the bf16 caches of the bf16 step are
    quantised once by the library's fp8 append; a step appends each layer's
    new token (quantising it) and attends.  Also the global-layer fp8 call
    alone (split + merge kernels), timed like the roofline kernel.  Bytes
    counted: 528 per visible token per layer (codes and scales)."""
    B = len(positions)
    pos = positions[0]
    dev = layers[0].k.device
    l8 = []
    for l, kind in enumerate(kinds):
        cap = layers[l].capacity
        lay = ga.LayerFp8.allocate(kind, B, cap, device=dev)
        ga.kv_append_fp8(lay, layers[l].k, layers[l].v, [0] * B)
        l8.append(lay)
    torch.cuda.synchronize()
    gen = torch.Generator(device=dev)
    gen.manual_seed(6006)
    kn = [torch.randn((B, 1, ga.HKV, ga.D), generator=gen, device=dev)
          .to(torch.bfloat16) for _ in kinds]
    vn = [torch.randn((B, 1, ga.HKV, ga.D), generator=gen, device=dev)
          .to(torch.bfloat16) for _ in kinds]
    out8 = [torch.empty_like(o) for o in outs]

    def step():
        for l in range(N_LAYERS):
            ga.kv_append_fp8(l8[l], kn[l], vn[l], positions)
            ga.attn_decode_fp8(l8[l], qs[l], positions, out8[l], ws)

    ms, _, _ = time_graph(torch, step, steps, warmup)
    # the fp8 step's outputs against the bf16 step's on the same tokens:
    # only the quantisation of K and V differs
    for l in (kinds.index(ga.LOCAL), kinds.index(ga.GLOBAL)):
        ref = torch.empty_like(outs[l])
        ga.kv_append(layers[l], kn[l], vn[l], positions)
        ga.attn_decode(layers[l], qs[l], positions, ref)
        torch.cuda.synchronize()
        diff = (ref - out8[l]).abs().max().item()
        if not diff < 0.05:
            raise RuntimeError("fp8 decode of layer %d differs from bf16 by "
                               "%g" % (l, diff))
    glob = [l for l, k in enumerate(kinds) if k == ga.GLOBAL]
    for l in glob:
        ga.attn_decode_fp8(l8[l], qs[l], positions, out8[l], ws)
    torch.cuda.synchronize()
    calls = [l for _ in range(kernel_reps) for l in glob]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    ev[0].record()
    for i, l in enumerate(calls):
        ga.attn_decode_fp8(l8[l], qs[l], positions, out8[l], ws)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(calls))]
    kms = sum(per) / len(per)
    step_bytes = kv_bytes_step(kinds, positions) // 1024 * FP8_TOKEN_BYTES
    call_bytes = B * (pos + 1) * FP8_TOKEN_BYTES
    verify = bench_verify_fp8(ga, torch, layers, l8, kinds)
    del l8
    return {"ms_per_step": round(ms, 4),
            "kv_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 2),
            "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              4),
            "global_call_ms": round(kms, 5),
            "global_call_median_ms": round(median(per), 5),
            "global_call_GBps": round(call_bytes / (kms * 1e-3) / 1e9, 2),
            "global_call_hbm_frac": round(call_bytes / (kms * 1e-3) / 1e9 /
                                          HBM_PEAK_GBS, 4),
            "bytes_per_token_layer": FP8_TOKEN_BYTES,
            "verify_fp8": verify,
            "workload": "52-layer decode step over fp8 caches (E4M3 + one "
                        "fp32 scale per token and KV head), context 131072, "
                        "batch %d: fp8 append + attend per layer, HIP graph"
                        % B}


def pairs_block(kind, pos0, n, window=2048):
    """Unmasked (query, key) pairs of a block of n tokens at pos0."""
    total = 0
    for r in range(n):
        i = pos0 + r
        total += i + 1 if kind == 1 else min(i + 1, window)
    return total


def pairs_block_together(pos0, n):
    """Pairs of a block of n tokens at pos0 predicted together: every token
    sees positions 0 .. pos0+n-1."""
    return n * (pos0 + n)


def bench_verify_fp8(ga, torch, layers, l8, kinds, reps=5, seed=4004):
    """52-layer verification of a 16-token block at 131056..131071 over the
    fp8 caches of sequence 0 (their first 131056 positions are the prior),
    batch 1, the same block inputs as the bf16 verification; a local and a
    global layer are checked against the bf16 verification of the same
    tokens (only the quantisation of the prior differs)."""
    dev = layers[0].k.device
    n, pos0 = 16, CTX - 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    blk = []
    for l in range(N_LAYERS):
        q = torch.randn((1, n, ga.HQ, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        kb = torch.randn((1, n, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        vb = torch.randn((1, n, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        blk.append((q, kb, vb))
    sub = [ga.LayerFp8(kinds[l], x.k[0:1], x.v[0:1], x.k_scale[0:1],
                       x.v_scale[0:1]) for l, x in enumerate(l8)]
    ws = torch.empty(max(ga.workspace_bytes(ga.OP_VERIFY, k, 1, n, CTX)
                         for k in (ga.LOCAL, ga.GLOBAL)), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((1, n, ga.HQ, ga.D), dtype=torch.float32, device=dev)

    def step():
        for l in range(N_LAYERS):
            q, kb, vb = blk[l]
            ga.attn_verify_fp8(sub[l], q, kb, vb, [pos0], out, ws)

    ms, _, _ = time_graph(torch, step, reps, 2)
    for l in (kinds.index(ga.LOCAL), kinds.index(ga.GLOBAL)):
        q, kb, vb = blk[l]
        a = ga.attn_verify_fp8(sub[l], q, kb, vb, [pos0], None, ws)
        ref = ga.Layer(kinds[l], layers[l].k[0:1], layers[l].v[0:1])
        b = ga.attn_verify(ref, q, kb, vb, [pos0], None, ws)
        torch.cuda.synchronize()
        diff = (a - b).abs().max().item()
        if not diff < 0.05:
            raise RuntimeError("fp8 verify of layer %d differs from bf16 by "
                               "%g" % (l, diff))
    flops = kvb = 0
    for kind in kinds:
        flops += pairs_block(kind, pos0, n) * 4 * ga.HQ * ga.D
        keys = CTX if kind == ga.GLOBAL else min(CTX, 2048 + n - 1)
        kvb += keys * FP8_TOKEN_BYTES
    return {"ms_per_step": round(ms, 4),
            "kv_GBps": round(kvb / (ms * 1e-3) / 1e9, 2),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "workload": "52-layer verify over fp8 caches, 16 drafted tokens "
                        "at 131056..131071, batch 1"}


def bench_verify(ga, torch, layers, kinds, B, reps=5, seed=4004):
    """52-layer verification of a 16-token drafted block at 131056..131071
    over the caches of the decode step (their first 131056 positions serve as
    the prior context).  Returns a dict of figures."""
    dev = torch.device("cuda")
    n, pos0 = 16, CTX - 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    blk = []
    for l in range(N_LAYERS):
        q = torch.randn((B, n, ga.HQ, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        kb = torch.randn((B, n, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        vb = torch.randn((B, n, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        blk.append((q, kb, vb))
    ws = torch.empty(max(ga.workspace_bytes(ga.OP_VERIFY, k, B, n, CTX)
                         for k in (ga.LOCAL, ga.GLOBAL)), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, n, ga.HQ, ga.D), dtype=torch.float32, device=dev)
    positions = [pos0] * B

    def step():
        for l in range(N_LAYERS):
            q, kb, vb = blk[l]
            ga.attn_verify(layers[l], q, kb, vb, positions, out, ws)

    ms, _, _ = time_graph(torch, step, reps, 2)
    flops = 0
    kvb = 0
    for kind in kinds:
        pr = pairs_block(kind, pos0, n)
        flops += B * pr * 4 * ga.HQ * ga.D
        keys = CTX if kind == ga.GLOBAL else min(CTX, 2048 + n - 1)
        kvb += B * keys * 1024
    return {"ms_per_step": round(ms, 4),
            "kv_GBps": round(kvb / (ms * 1e-3) / 1e9, 2),
            "hbm_frac": round(kvb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "workload": "52-layer verify, 16 drafted tokens at 131056..131071, "
                        "batch %d" % B}


def bench_draft(ga, torch, layers, kinds, B, n_drafter=5, reps=5, seed=4404):
    """A 5-layer drafter's attention over a 16-token block predicted together
    at 131056..131071 (every block token sees the context and the whole
    block).  The first five global caches of the decode step stand in for
    the drafter's context keys and values.  Returns a dict of figures."""
    dev = torch.device("cuda")
    n, pos0 = 16, CTX - 16
    glob = [l for l in range(N_LAYERS) if kinds[l] == ga.GLOBAL][:n_drafter]
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    blk = []
    for _ in glob:
        q = torch.randn((B, n, ga.HQ, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        kb = torch.randn((B, n, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        vb = torch.randn((B, n, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        blk.append((q, kb, vb))
    ws = torch.empty(ga.workspace_bytes(ga.OP_DRAFT, ga.GLOBAL, B, n, CTX),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((B, n, ga.HQ, ga.D), dtype=torch.float32, device=dev)
    positions = [pos0] * B

    def step():
        for i, l in enumerate(glob):
            q, kb, vb = blk[i]
            ga.attn_draft_block(layers[l], q, kb, vb, positions, out, ws)

    ms, _, _ = time_graph(torch, step, reps, 2)
    flops = len(glob) * B * pairs_block_together(pos0, n) * 4 * ga.HQ * ga.D
    kvb = len(glob) * B * CTX * 1024
    return {"ms_per_step": round(ms, 4),
            "kv_GBps": round(kvb / (ms * 1e-3) / 1e9, 2),
            "hbm_frac": round(kvb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "workload": "%d drafter layers, a 16-token block predicted "
                        "together at 131056..131071 over a 131056-token "
                        "context, batch %d" % (len(glob), B)}


def prefill_oracle_sample(ga, torch, kind, q, k, v, out, c0, nrows,
                          seed=5115):
    """The fp64 oracle on this host for `nrows` randomly drawn rows of the
    last prefill chunk (positions c0 ..), each checked against the GPU's
    bf16 output of that chunk (max abs <= 2e-2, mean abs <= 2e-3; a miss
    raises).  Returns the oracle's rate over the sample."""
    import numpy as np
    import oracle
    import synth_inputs as si

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    n = out.shape[1]
    rows = np.sort(np.random.default_rng(seed).choice(n, nrows,
                                                      replace=False))
    pos = c0 + rows
    lo = 0 if kind == ga.GLOBAL else max(0, c0 - ga.WINDOW + 1)
    kb = si.bits(k[0, lo:c0 + n])
    vb = si.bits(v[0, lo:c0 + n])
    qb = si.bits(q[0, torch.as_tensor(c0 + rows, device=q.device)])
    ts = time.perf_counter()
    want = oracle.attend(qb, pos, kb, vb, lo, hq=32, hkv=2, d=128,
                         window=ga.WINDOW if kind == ga.LOCAL else 0,
                         rope=kind == ga.LOCAL, nthreads=cores)
    elapsed = time.perf_counter() - ts
    got = out[0, torch.as_tensor(rows, device=out.device)].float().cpu() \
        .double().numpy()
    err = np.abs(got - want)
    if not (err.max() <= 2e-2 and err.mean() <= 2e-3):
        raise RuntimeError("prefill rows differ from the oracle: max abs "
                           "%.3e, mean abs %.3e" % (err.max(), err.mean()))
    pairs = int(sum(p + 1 - max(lo, p - ga.WINDOW + 1 if kind == ga.LOCAL
                                else 0) for p in pos))
    flops = pairs * 4 * ga.HQ * ga.D
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": "fp64 oracle, %d random rows of the last %d-token "
                      "chunk (positions %d..), %.3g flop in %.2f s; the "
                      "GPU's rows match it (max abs %.2e, mean abs %.2e)" %
                      (nrows, n, c0, flops, elapsed, err.max(), err.mean())}


def bench_prefill(ga, torch, chunk=4096, total=CTX, reps=1, seed=5005,
                  fp8=False, with_oracle=True):
    """Chunked causal prefill of `total` tokens in `chunk`-token chunks on
    one local and one global layer: prefill then append per chunk (fp8:
    over fp8 caches, appending with the quantiser)."""
    dev = torch.device("cuda")
    res = {}
    for kind in (ga.LOCAL, ga.GLOBAL):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed + kind)
        layer = (ga.LayerFp8 if fp8 else ga.Layer).allocate(kind, 1,
                                                              device=dev)
        attend = ga.attn_prefill_fp8 if fp8 else ga.attn_prefill
        append = ga.kv_append_fp8 if fp8 else ga.kv_append
        q = torch.randn((1, total, ga.HQ, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((1, total, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((1, total, ga.HKV, ga.D), generator=gen, device=dev).to(torch.bfloat16)
        op = ga.OP_PREFILL_FP8 if fp8 else ga.OP_PREFILL
        ws = torch.empty(ga.workspace_bytes(op, kind, 1, chunk, total),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((1, chunk, ga.HQ, ga.D), dtype=torch.bfloat16, device=dev)

        def run():
            for c0 in range(0, total, chunk):
                sl = slice(c0, c0 + chunk)
                attend(layer, q[:, sl], k[:, sl], v[:, sl], [c0], out, ws)
                append(layer, k[:, sl], v[:, sl], [c0])

        run()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = pairs_block(kind, 0, total) * 4 * ga.HQ * ga.D
        name = "local" if kind == ga.LOCAL else "global"
        res[name] = {"ms": round(ms, 3),
                     "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                     "mfma_frac": round(flops / (ms * 1e-3) / 1e12 /
                                        MFMA_PEAK_TFLOPS, 4),
                     "algorithmic_flop": flops}
        if not fp8 and with_oracle:
            res[name]["cpu_baseline"] = prefill_oracle_sample(
                ga, torch, kind, q, k, v, out, total - chunk,
                64 if kind == ga.GLOBAL else 512)
        del q, k, v, layer, ws, out
        torch.cuda.empty_cache()
    res["workload"] = ("prefill of %d tokens in %d-token chunks (prefill + "
                       "append per chunk), batch 1%s" %
                       (total, chunk, ", over fp8 caches" if fp8 else ""))
    if not fp8:
        res["fp8"] = bench_prefill(ga, torch, chunk, total, reps, seed, True,
                                   False)
    return res


def cpu_baseline(ga, torch, layers, qs, outs, positions, kinds,
                 budget_s=20.0):
    """The fp64 oracle on this host: the timed decode step, sequence by
    sequence and layer by layer in step order, for as many (sequence, layer)
    pairs as fit the time budget (the whole step at the default sizes).
    The oracle's outputs are also compared with the timed step's outputs
    (max abs <= 2e-2, mean abs <= 2e-3); a miss raises, so no figure is
    printed for a wrong result."""
    import numpy as np
    import oracle
    import synth_inputs as si

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    done_bytes, done_pairs = 0, 0
    worst_max, worst_mean = 0.0, 0.0
    t0 = time.perf_counter()
    elapsed = 0.0
    B = len(positions)
    for b in range(B):
        p = positions[b]
        for l, kind in enumerate(kinds):
            lo = 0 if kind == ga.GLOBAL else max(0, p - ga.WINDOW + 1)
            if kind == ga.GLOBAL:
                kb = si.bits(layers[l].k[b, lo:p + 1])
                vb = si.bits(layers[l].v[b, lo:p + 1])
            else:
                idx = torch.arange(lo, p + 1,
                                   device=layers[l].k.device) % ga.WINDOW
                kb = si.bits(layers[l].k[b, idx])
                vb = si.bits(layers[l].v[b, idx])
            qb = si.bits(qs[l][b:b + 1])
            ts = time.perf_counter()
            want = oracle.attend(qb, [p], kb, vb, lo, hq=32, hkv=2, d=128,
                                 window=ga.WINDOW if kind == ga.LOCAL else 0,
                                 rope=kind == ga.LOCAL, nthreads=cores)
            elapsed += time.perf_counter() - ts
            err = np.abs(outs[l][b].cpu().double().numpy() - want[0])
            worst_max = max(worst_max, float(err.max()))
            worst_mean = max(worst_mean, float(err.mean()))
            if not (err.max() <= 2e-2 and err.mean() <= 2e-3):
                raise RuntimeError(
                    "sequence %d, layer %d (kind %d) of the decode step "
                    "differs from the oracle: max abs %.3e, mean abs %.3e" %
                    (b, l, kind, err.max(), err.mean()))
            done_bytes += (p + 1 - lo) * 1024
            done_pairs += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "fp64 oracle, the timed decode step (%d sequences x 52 "
                  "layers at context %d): %d of its %d (sequence, layer) "
                  "pairs, %.1f MB of KV, %.2f s of oracle time; the step's "
                  "outputs for those pairs match it (worst max abs %.2e, "
                  "mean abs %.2e)" %
                  (B, max(positions) + 1, done_pairs, B * len(kinds),
                   done_bytes / 1e6, elapsed, worst_max, worst_mean),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (also lets the GPU clocks ramp "
                         "up; ~0.2 s at batch 4)")
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true",
                    help="decode step only (skip verify and prefill)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the chunked-prefill measurement and print "
                         "its JSON (for hardware-counter runs)")
    ap.add_argument("--global-decode-calls", type=int, default=0,
                    help="run only the global-layer decode call this many "
                         "times over each of the 13 global layers and print "
                         "its average (for hardware-counter runs)")
    ap.add_argument("--fp8-only", action="store_true",
                    help="after the bf16 decode step, run only the fp8 "
                         "decode measurement (skip verify and prefill)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB, "
                         "to scale hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the attention path has no "
              "multi-GPU execution (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    ga = _ensure_built()
    torch.cuda.set_device(0)
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill(
            ga, torch, with_oracle=not args.no_cpu_baseline)}), flush=True)
        return
    if args.calibrate_copy_mib:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads and writes exactly nbytes each
        torch.cuda.synchronize()
        del src, dst
    B = args.batch
    pos = CTX - 1
    kinds, layers, qs, outs, ws, positions, step = build_decode_step(
        ga, torch, B, pos)
    torch.cuda.synchronize()
    print("# setup done: %d layers, batch %d, context %d" % (N_LAYERS, B, CTX),
          file=sys.stderr, flush=True)
    if args.global_decode_calls:
        kms, _ = time_global_decode(ga, torch, layers, qs, outs, ws,
                                    positions, kinds, args.global_decode_calls)
        print(json.dumps({"global_decode_call_ms": round(kms, 5),
                          "batch": B, "keys": pos + 1}), flush=True)
        return

    ms, _graph, ms_mean = time_graph(torch, step, args.steps, args.warmup)
    check_step_outputs(ga, torch, layers, qs, outs, positions, kinds)
    kvb = kv_bytes_step(kinds, positions)
    value = kvb / (ms * 1e-3) / 1e9

    ms_local, _, _ = time_graph(torch, step.local_only, args.steps,
                                args.warmup)
    ms_global, _, _ = time_graph(torch, step.global_only, args.steps,
                                 args.warmup)

    kms, kms_med = time_global_decode(ga, torch, layers, qs, outs, ws,
                                      positions, kinds, args.kernel_reps)
    kbytes = B * (pos + 1) * 1024
    achieved = kbytes / (kms * 1e-3) / 1e9

    line = {
        "metric": "decode attn KV GB/s (% HBM peak) at 131K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "52-layer decode step (39 local W=2048 RoPE + "
                               "13 global), context 131072, append + attend "
                               "per layer, HIP graph",
                   "global_batch": B, "seq_len": CTX,
                   "parallelism": "none (1 GPU)"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "breakdown_ms": {"39 local layers": round(ms_local, 4),
                         "13 global layers": round(ms_global, 4)},
        "roofline": {
            "bound": "hbm",
            "kernel": "global-layer decode call (split-K kernel + merge "
                      "kernel), %d keys x batch %d" % (pos + 1, B),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(B),
            "traffic_unit": "bytes per launch (HBM fetched + written)",
            "avg_ms": round(kms, 5),
            "median_ms": round(kms_med, 5),
            "algorithmic_bytes": kbytes,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(ga, torch, layers, qs, outs,
                                            positions, kinds)
    if not args.no_extras or args.fp8_only:
        line["decode_fp8"] = bench_decode_fp8(
            ga, torch, layers, qs, outs, ws, positions, kinds, args.steps,
            args.warmup, args.kernel_reps)
        line["decode_fp8"]["global_call_vs_bf16"] = round(
            kms / line["decode_fp8"]["global_call_ms"], 3)
        print("# fp8 decode done", file=sys.stderr, flush=True)
    if not args.no_extras and not args.fp8_only:
        line["verify"] = bench_verify(ga, torch, layers, kinds, 1)
        print("# verify done", file=sys.stderr, flush=True)
        line["draft_block"] = bench_draft(ga, torch, layers, kinds, 1)
        print("# drafted block done", file=sys.stderr, flush=True)
        del layers, qs, outs, ws, step
        torch.cuda.empty_cache()
        line["decode_b1"] = bench_decode_b1(ga, torch, args.steps, args.warmup)
        print("# single-sequence decode done", file=sys.stderr, flush=True)
        line["prefill"] = bench_prefill(
            ga, torch, with_oracle=not args.no_cpu_baseline)
        print("# prefill done", file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
