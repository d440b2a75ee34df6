"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutant is the oracle source with one textual edit: a window edge off by
one, the wrong query-to-KV head mapping, a RoPE sign or frequency slip, a
dropped softmax scale, a causal mask that drops the query's own key.  The
mutant is compiled with gcc into a temporary library, all oracle calls are
routed through it, and the pin tests are run; at least one must fail."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gqa_oracle.c")

MUTANTS = {
    "window_edge": ("int64_t lo = i - (int64_t)cfg->window + 1;",
                    "int64_t lo = i - (int64_t)cfg->window;"),
    "head_map": ("const int32_t g = h / group;",
                 "const int32_t g = h % hkv;"),
    "rope_sign": ("out[c + half] = x1 * cs + x0 * sn;",
                  "out[c + half] = x1 * cs - x0 * sn;"),
    "rope_freq": ("pow(theta, -(double)c / (double)half)",
                  "pow(theta, -(double)c / (double)d)"),
    "no_scale": ("s[t] = dot * cfg->scale;", "s[t] = dot;"),
    "no_self_key": ("int64_t jlo = visible_lo(cfg, i), jhi = i + 1;",
                    "int64_t jlo = visible_lo(cfg, i), jhi = i;"),
    "k_not_rotated": ("if (cfg->rope && nk > 0) {", "if (0) {"),
}

PIN_TESTS = [
    lambda: [pins.test_bruteforce_tiny(*c) for c in pins.CASES],
    pins.test_bruteforce_offset_stream_and_sparse_queries,
    pins.test_rope_identity_norm_and_relative,
    lambda: [pins.test_zero_query_gives_window_mean(w, r)
             for w, r in [(0, False), (8, True), (2048, True)]],
    pins.test_constant_v_and_single_key,
    pins.test_gqa_equals_mha_with_repeated_kv,
    pins.test_split_merge_identity,
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation anchor moved: %s" % name
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "gqa_oracle.c")
        with open(src, "w") as f:
            f.write(text.replace(old, new))
        shutil.copy(os.path.join(os.path.dirname(SRC), "gqa_oracle.h"), tmp)
        lib = os.path.join(tmp, "libmutant.so")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                        "-pthread", "-o", lib, src, "-lm"], check=True)
        caught = []
        with oracle.use_library(lib):
            for t in PIN_TESTS:
                try:
                    t()
                except (AssertionError, oracle.OracleRangeError):
                    caught.append(t)
        assert caught, "no pin caught mutant %s" % name
