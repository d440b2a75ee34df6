"""Host checks of bench.py: its byte and pair accounting against closed forms
of the workloads (so the reported throughput divides the right numerator),
and the one-GPU guard.  No GPU needed."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LOCAL, GLOBAL = 0, 1


def _kinds():
    # three local layers then one global, 13 times
    return [GLOBAL if l % 4 == 3 else LOCAL for l in range(52)]


def test_kv_bytes_of_the_decode_steps():
    kinds = _kinds()
    assert kinds.count(LOCAL) == 39 and kinds.count(GLOBAL) == 13
    # 13 x 131072 x 1024 B of global caches + 39 x 2048 x 1024 B of rings
    assert bench.kv_bytes_step(kinds, [131071]) == 1826619392
    assert bench.kv_bytes_step(kinds, [131071] * 4) == 4 * 1826619392
    # 13 x 32 MiB + 39 x 2 MiB at context 32768
    assert bench.kv_bytes_step(kinds, [32767]) == 13 * (32 << 20) + 39 * (2 << 20)
    # one local + one global layer at context 4096: 2 MiB + 4 MiB
    assert bench.kv_bytes_step([LOCAL, GLOBAL], [4095]) == 6291456
    # short contexts: a local layer sees every key before the window fills
    assert bench.kv_bytes_step([LOCAL], [99]) == 100 * 1024


def test_prefill_pair_counts():
    chunk, total = 4096, 131072
    glob = sum(bench.pairs_block(GLOBAL, c, chunk) for c in range(0, total, chunk))
    loc = sum(bench.pairs_block(LOCAL, c, chunk) for c in range(0, total, chunk))
    assert glob == total * (total + 1) // 2 == 8590000128
    # the first 2048 queries see 1..2048 keys, every later one 2048
    assert loc == 2048 * 2049 // 2 + (total - 2048) * 2048 == 266339328


def test_verify_pairs():
    # 16 drafted tokens at 131056..131071: 131057 .. 131072 visible keys each
    assert bench.pairs_block(GLOBAL, 131056, 16) == sum(range(131057, 131073))
    assert bench.pairs_block(LOCAL, 131056, 16) == 16 * 2048


def test_block_together_pairs():
    # every one of the 16 tokens sees the 131056 context keys and all 16
    assert bench.pairs_block_together(131056, 16) == 16 * 131072
    assert bench.pairs_block_together(0, 1) == 1
    # the causal block's last token sees as many as any token here
    assert bench.pairs_block_together(131056, 16) >= bench.pairs_block(
        GLOBAL, 131056, 16)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
