"""The launch planners on the host, for devices of any shape (no GPU).

``csrc/plan.cpp`` is plain C++: it is built here with g++ together with a
small shim that exposes the plans with C types, and driven with faked
compute-unit and XCD counts (a full MI355X, partitioned parts, larger and
smaller devices).  Every plan must cover its keys with non-empty splits,
stay within what the merge kernels take (256 splits), fill the device in
one round where it can, and size its workspace for what the kernels write.
On a full MI355X (256 CUs) the plans must be the ones the kernels were
measured with."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "global_gqa_attention_kv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

SHIM = r"""
#include "plan.h"
using namespace gqa;
extern "C" {
void shim_plan_decode(int kind, int B, long long keys, int cus, int xcds,
                      long long* out) {
  const DecodePlan p = plan_decode(kind, B, keys, DeviceShape{cus, xcds});
  out[0] = p.splits;
  out[1] = p.tiles_per_split;
  out[2] = p.heads_per_wg;
  out[3] = (long long)decode_ws_bytes(B, p);
}
void shim_plan_block(int kind, int B, int n, long long keys, int cus,
                     int xcds, int always_split, long long* out) {
  const BlockPlan p = plan_block(kind, B, n, keys, DeviceShape{cus, xcds},
                                 always_split != 0);
  out[0] = p.qpw;
  out[1] = p.qgroups;
  out[2] = p.splits;
  out[3] = p.grid;
  out[4] = p.walks;
  out[5] = (long long)p.klin_bytes;
  out[6] = (long long)p.part_bytes;
  out[7] = (long long)block_ws_bytes(p);
}
}
"""

LOCAL, GLOBAL = 0, 1
TILE, W, MAX_SPLITS, BLK_MAX_SPLITS = 64, 2048, 256, 128
SHAPES = [(256, 8), (304, 8), (240, 8), (128, 4), (80, 2), (64, 2), (38, 1),
          (32, 1), (8, 1), (1, 1)]


@pytest.fixture(scope="module")
def plans(tmp_path_factory):
    d = tmp_path_factory.mktemp("plan")
    shim = d / "shim.cpp"
    shim.write_text(SHIM)
    so = d / "libplan.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I",
                    INCLUDE, "-I", CSRC, os.path.join(CSRC, "plan.cpp"),
                    str(shim), "-o", str(so)], check=True)
    lib = ctypes.CDLL(str(so))
    i, ll = ctypes.c_int, ctypes.c_longlong
    lib.shim_plan_decode.argtypes = [i, i, ll, i, i, ctypes.POINTER(ll)]
    lib.shim_plan_block.argtypes = [i, i, i, ll, i, i, i,
                                    ctypes.POINTER(ll)]

    def decode(kind, B, keys, cus, xcds=8):
        out = (ll * 4)()
        lib.shim_plan_decode(kind, B, keys, cus, xcds, out)
        return dict(zip(("splits", "tps", "hpw", "ws"), out))

    def block(kind, B, n, keys, cus, xcds=8, always_split=False):
        out = (ll * 8)()
        lib.shim_plan_block(kind, B, n, keys, cus, xcds, int(always_split),
                            out)
        return dict(zip(("qpw", "qgroups", "splits", "grid", "walks", "klin",
                         "part", "ws"), out))
    return decode, block


@pytest.mark.parametrize("cus,xcds", SHAPES)
def test_decode_plans_cover_and_fit(plans, cus, xcds):
    decode, _ = plans
    for kind in (LOCAL, GLOBAL):
        for B in (1, 2, 3, 4, 7, 8, 16, 33, 64):
            for ctx in (1, 63, 64, 65, 2048, 4096, 32768, 131072):
                keys = min(ctx, W) if kind == LOCAL else ctx
                p = decode(kind, B, keys, cus, xcds)
                tiles = -(-keys // TILE)
                s, t = p["splits"], p["tps"]
                assert 1 <= s <= MAX_SPLITS
                assert s * t >= tiles and (s - 1) * t < tiles, p
                # one round on the device where the keys allow it
                wgs = B * 2 * s
                if kind == GLOBAL:
                    assert wgs <= max(2 * cus, 2 * B), (B, ctx, p)
                    if 2 * cus // (2 * B) >= tiles:
                        assert t == 1      # as many splits as tiles
                else:
                    assert wgs <= max(2 * cus, 2 * B), (B, ctx, p)
                    assert p["hpw"] == (8 if B <= 2 else 16)
                assert p["ws"] >= B * 2 * s * 16 * 130 * 4
                assert p["ws"] % 256 == 0


def test_decode_plans_on_a_full_mi355x(plans):
    """256 CUs: the plans the kernels were measured with."""
    decode, _ = plans
    for B in range(1, 65):
        g = decode(GLOBAL, B, 131072, 256)
        want = max(1, 512 // (2 * B))
        per = -(-2048 // want)
        assert (g["tps"], g["splits"]) == (per, -(-2048 // per)), B
        loc = decode(LOCAL, B, 2048, 256)
        tps = min(32, B // 4 if B >= 8 else 1)
        assert (loc["tps"], loc["splits"]) == (tps, -(-32 // tps)), B
    assert decode(GLOBAL, 4, 131072, 256)["splits"] == 64
    assert decode(GLOBAL, 1, 131072, 256)["splits"] == 256


def test_noalloc_scratch_holds_every_decode_on_a_full_mi355x(plans):
    """The no-allocation entry point's 8 MiB scratch holds the partials of
    every decode call a 256-CU device plans (at most 4.3 MB)."""
    decode, _ = plans
    worst = 0
    for kind in (LOCAL, GLOBAL):
        for B in range(1, 65):
            for ctx in (1, 64, 2048, 2049, 4096, 32768, 100000, 131072):
                keys = min(ctx, W) if kind == LOCAL else ctx
                worst = max(worst, decode(kind, B, keys, 256)["ws"])
    assert worst <= 8 << 20
    assert worst == 2 * 256 * 16 * 130 * 4        # batch 1, 256 splits


@pytest.mark.parametrize("cus,xcds", SHAPES)
def test_block_plans_cover_and_fit(plans, cus, xcds):
    _, block = plans
    for kind in (LOCAL, GLOBAL):
        for B in (1, 4, 64):
            for n, ctx in ((1, 100), (16, 131072), (16, 2064), (100, 5000),
                           (4096, 4096), (4096, 131072)):
                keys = min(ctx, W) if kind == LOCAL else ctx
                p = block(kind, B, n, keys, cus, xcds)
                qpw = p["qpw"]
                # 8-token groups only for local layers with key splits, and
                # whenever those still leave CUs over
                if qpw == 8:
                    assert kind == LOCAL and p["splits"] > 1
                else:
                    assert qpw == 16
                    if kind == LOCAL and p["splits"] > 1:
                        assert -(-n // 8) * 2 * B >= cus
                groups = p["qgroups"] * 2 * B
                assert p["qgroups"] == -(-n // qpw)
                wg_keys = W - 1 + qpw if kind == LOCAL else keys
                assert 1 <= p["splits"] <= min(BLK_MAX_SPLITS,
                                               -(-wg_keys // TILE))
                items = p["splits"] * groups
                if p["splits"] > 1:
                    assert p["grid"] == items and p["walks"] == 1
                    assert groups < cus
                    assert p["part"] >= groups * p["splits"] * qpw * 16 * 272
                else:
                    assert p["part"] == 0
                    assert p["grid"] <= cus
                    assert p["grid"] * p["walks"] >= items
                    assert (p["grid"] - 1) * p["walks"] < items
                if kind == LOCAL and p["splits"] == 1:
                    assert p["klin"] >= B * (W + n) * 512
                assert p["ws"] >= p["klin"] + p["part"]


def test_block_plans_on_a_full_mi355x(plans):
    _, block = plans
    # verify at 131056 + 16, batch 1: 256 workgroups of 16 tiles (global),
    # 33 splits of one tile per KV head and 8-token group (local)
    g = block(GLOBAL, 1, 16, 131072, 256)
    assert (g["qpw"], g["splits"], g["grid"]) == (16, 128, 256)
    loc = block(LOCAL, 1, 16, 2048, 256)
    assert (loc["qpw"], loc["splits"], loc["grid"]) == (8, 33, 132)
    # prefill chunk of 4096: 512 work items walked by 256 workgroups
    pf = block(GLOBAL, 1, 4096, 131072, 256)
    assert (pf["splits"], pf["grid"], pf["walks"]) == (1, 256, 2)


@pytest.mark.parametrize("cus,xcds", SHAPES)
def test_block_plans_always_split(plans, cus, xcds):
    """Calls over fp8 caches (verification, drafted blocks) always take the
    key-split kernels: one or more splits, partials for every split, no
    rotated-key copy, one work item per workgroup, and 8-token workgroups on
    local layers."""
    _, block = plans
    for kind in (LOCAL, GLOBAL):
        for B in (1, 4, 64):
            for n, ctx in ((1, 1), (16, 16), (1, 100), (16, 2064),
                           (16, 131072)):
                keys = min(ctx, W) if kind == LOCAL else ctx
                p = block(kind, B, n, keys, cus, xcds, always_split=True)
                qpw = 8 if kind == LOCAL else 16
                assert p["qpw"] == qpw
                groups = -(-n // qpw) * 2 * B
                wg_keys = W - 1 + qpw if kind == LOCAL else keys
                assert 1 <= p["splits"] <= min(BLK_MAX_SPLITS,
                                               -(-wg_keys // TILE))
                assert p["walks"] == 1 and p["klin"] == 0
                assert p["grid"] == p["splits"] * groups
                assert p["part"] >= groups * p["splits"] * qpw * 16 * 272
                assert p["ws"] >= p["part"]

