"""Host-only checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function include/gqa_attn.h declares,
agree with the header's constants, and reject bad arguments with the
documented status codes before it touches the GPU.  Device pointers here are
fake addresses: validation never dereferences them, and every call below
fails validation, so no HIP call is made."""
import ctypes
import os
import re

import pytest

import global_gqa_attention_kv_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f)
           for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


def _header_text():
    return "\n".join(open(h).read() for h in HEADERS)


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", text)))


def _defines():
    out = {}
    for name, val in re.findall(r"#define\s+(GQA_\w+)\s+\(?(-?\d+)\)?",
                                _header_text()):
        out[name] = int(val)
    return out


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ga.library_path()):
        pytest.fail("libgqa_attn.so is not built (run __graft_entry__.build())")
    return ga._load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert "gqa_attn_decode" in names and "gqa_kv_append" in names
    for n in names:
        assert hasattr(lib, n), "missing export %s" % n


def test_constants_match_header(lib):
    D = _defines()
    assert lib.gqa_abi_version() == D["GQA_ABI_VERSION"]
    assert (ga.HQ, ga.HKV, ga.D, ga.WINDOW, ga.MAX_CONTEXT, ga.MAX_BATCH) == (
        D["GQA_NUM_Q_HEADS"], D["GQA_NUM_KV_HEADS"], D["GQA_HEAD_DIM"],
        D["GQA_WINDOW"], D["GQA_MAX_CONTEXT"], D["GQA_MAX_BATCH"])
    assert (ga.LOCAL, ga.GLOBAL) == (D["GQA_LOCAL"], D["GQA_GLOBAL"])
    for code in ("GQA_OK", "GQA_ERR_INVALID_ARG", "GQA_ERR_POS_RANGE",
                 "GQA_ERR_MISALIGNED", "GQA_ERR_WS_TOO_SMALL",
                 "GQA_ERR_UNSUPPORTED", "GQA_ERR_HIP"):
        s = ga.status_string(D[code])
        assert s and s != "unknown status"
    assert ga.status_string(-99) == "unknown status"


def test_workspace_bytes():
    for kind in (ga.LOCAL, ga.GLOBAL):
        prev = 0
        for ctx in (1, 63, 64, 65, 2048, 4096, 32768, 131072):
            n = ga.workspace_bytes(ga.OP_DECODE, kind, 1, 1, ctx)
            assert n > 0 and n % 16 == 0 and n >= prev
            prev = n
        assert ga.workspace_bytes(ga.OP_DECODE, kind, 4, 1, 131072) >= prev
    assert ga.workspace_bytes(ga.OP_DECODE, ga.GLOBAL, 1, 1, 131073) == 0
    assert ga.workspace_bytes(ga.OP_DECODE, ga.GLOBAL, 0, 1, 10) == 0
    assert ga.workspace_bytes(ga.OP_DECODE, ga.GLOBAL, 65, 1, 10) == 0
    assert ga.workspace_bytes(ga.OP_DECODE, 7, 1, 1, 10) == 0
    assert ga.workspace_bytes(99, ga.GLOBAL, 1, 1, 10) == 0
    # local layers never see more than the window
    assert (ga.workspace_bytes(ga.OP_DECODE, ga.LOCAL, 1, 1, 131072) ==
            ga.workspace_bytes(ga.OP_DECODE, ga.LOCAL, 1, 1, 2048))


FAKE = 0x7f0000000000  # 16-byte aligned, never dereferenced


def _layer(kind=ga.GLOBAL, capacity=4096, window=None, theta=None, k=FAKE,
           v=FAKE + (1 << 30), stride=None):
    if window is None:
        window = ga.WINDOW if kind == ga.LOCAL else 0
    if theta is None:
        theta = 10000.0 if kind == ga.LOCAL else 0.0
    if kind == ga.LOCAL and capacity == 4096:
        capacity = ga.WINDOW
    if stride is None:
        stride = capacity * 256
    return ga._CLayer(kind, window, capacity, theta, k, v, stride)


def _pos(*vals):
    return (ctypes.c_int64 * len(vals))(*vals)


D_ = _defines()
E_ARG, E_POS, E_ALN = (D_["GQA_ERR_INVALID_ARG"], D_["GQA_ERR_POS_RANGE"],
                       D_["GQA_ERR_MISALIGNED"])
E_WS, E_UNS = D_["GQA_ERR_WS_TOO_SMALL"], D_["GQA_ERR_UNSUPPORTED"]


def _append(lib, L, B=1, n=1, k=FAKE, v=FAKE, pos=None):
    pos = pos if pos is not None else _pos(*([0] * B))
    return lib.gqa_kv_append(ctypes.byref(L) if L is not None else None, k, v,
                             pos, B, n, None)


def test_append_validation(lib):
    L = _layer()
    assert _append(lib, None) == E_ARG
    assert _append(lib, L, k=None) == E_ARG
    assert _append(lib, L, B=0) == E_ARG
    assert _append(lib, L, B=65, pos=_pos(*([0] * 65))) == E_ARG
    assert _append(lib, L, n=0) == E_ARG
    assert _append(lib, _layer(k=0)) == E_ARG
    assert _append(lib, _layer(kind=5)) == E_UNS
    assert _append(lib, _layer(kind=ga.LOCAL, capacity=4096 * 2)) == E_UNS
    assert _append(lib, _layer(kind=ga.LOCAL, theta=0.0)) == E_UNS
    assert _append(lib, _layer(kind=ga.LOCAL, window=1024)) == E_UNS
    assert _append(lib, _layer(theta=10000.0)) == E_UNS     # global with RoPE
    assert _append(lib, _layer(capacity=131073)) == E_UNS
    assert _append(lib, _layer(stride=100)) == E_ARG
    assert _append(lib, _layer(stride=4096 * 256 + 4)) == E_ALN
    assert _append(lib, _layer(k=FAKE + 8)) == E_ALN
    assert _append(lib, L, k=FAKE + 2) == E_ALN
    assert _append(lib, L, pos=_pos(-1)) == E_POS
    assert _append(lib, L, n=2, pos=_pos(4095)) == E_POS        # past capacity
    assert _append(lib, L, B=2, n=1, pos=_pos(0, 4096)) == E_POS


def _decode(lib, L, B=1, q=FAKE, out=FAKE, pos=None, ws=FAKE, ws_bytes=1 << 30):
    pos = pos if pos is not None else _pos(*([0] * B))
    return lib.gqa_attn_decode(ctypes.byref(L) if L is not None else None, q,
                               pos, B, out, ws, ws_bytes, None)


def test_decode_validation(lib):
    L = _layer()
    assert _decode(lib, None) == E_ARG
    assert _decode(lib, L, q=None) == E_ARG
    assert _decode(lib, L, out=None) == E_ARG
    assert _decode(lib, L, B=0) == E_ARG
    assert _decode(lib, L, ws=None) == E_ARG
    assert _decode(lib, _layer(kind=3)) == E_UNS
    assert _decode(lib, L, q=FAKE + 4) == E_ALN
    assert _decode(lib, L, out=FAKE + 4) == E_ALN
    assert _decode(lib, L, ws=FAKE + 8) == E_ALN
    assert _decode(lib, L, pos=_pos(4096)) == E_POS              # pos < capacity
    assert _decode(lib, L, pos=_pos(-3)) == E_POS
    assert _decode(lib, _layer(kind=ga.LOCAL), pos=_pos(1 << 40)) == E_POS
    need = ga.workspace_bytes(ga.OP_DECODE, ga.GLOBAL, 1, 1, 4096)
    assert _decode(lib, L, pos=_pos(4095), ws_bytes=need - 1) == E_WS
    assert _decode(lib, L, pos=_pos(4095), ws_bytes=0) == E_WS


def test_decode_append_validation(lib):
    L = _layer()
    pos = _pos(10)

    def call(kn=FAKE, vn=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.gqa_attn_decode_append(ctypes.byref(L), FAKE, kn, vn, pos, 1,
                                          FAKE, ws, ws_bytes, None)
    assert call(kn=None) == E_ARG
    assert call(vn=None) == E_ARG
    assert call(kn=FAKE + 2) == E_ALN
    assert call(ws=FAKE + 16) == E_ALN     # workspace needs 256-byte alignment
    assert call(ws_bytes=8) == E_WS


def test_decode_dev_validation(lib):
    """Device positions: the host checks the bound max_pos like a position
    (the positions themselves are read by the kernels)."""
    L = _layer()   # global, capacity 4096

    def call(pos_dev=FAKE, max_pos=10, kn=None, vn=None, B=1, ws_bytes=1 << 30):
        return lib.gqa_attn_decode_dev(ctypes.byref(L), FAKE, kn, vn, pos_dev,
                                       max_pos, B, FAKE, FAKE, ws_bytes, None)
    assert call(pos_dev=None) == E_ARG
    assert call(pos_dev=FAKE + 4) == E_ALN
    assert call(B=0) == E_ARG
    assert call(max_pos=4096) == E_POS
    assert call(max_pos=-1) == E_POS
    assert call(kn=FAKE) == E_ARG            # k_new and v_new go together
    need = ga.workspace_bytes(ga.OP_DECODE, ga.GLOBAL, 1, 1, 4096)
    assert call(max_pos=4095, ws_bytes=need - 1) == E_WS


@pytest.mark.parametrize("fn", ["gqa_attn_verify", "gqa_attn_draft_block",
                                "gqa_attn_prefill"])
def test_block_validation(lib, fn):
    f = getattr(lib, fn)
    L = _layer()

    def call(layer=L, q=FAKE, kb=FAKE, vb=FAKE, pos=None, B=1, n=16, out=FAKE,
             ws=FAKE, ws_bytes=1 << 30):
        pos = pos if pos is not None else _pos(*([0] * B))
        return f(ctypes.byref(layer) if layer is not None else None, q, kb, vb,
                 pos, B, n, out, ws, ws_bytes, None)
    assert call(layer=None) == E_ARG
    assert call(q=None) == E_ARG
    assert call(kb=None) == E_ARG
    assert call(out=None) == E_ARG
    assert call(n=0) == E_ARG
    assert call(B=0) == E_ARG
    assert call(ws=None) == E_ARG
    if fn != "gqa_attn_prefill":
        assert call(n=17) == E_ARG                      # block of at most 16
    else:
        assert call(n=17, pos=_pos(0), ws_bytes=0) == E_WS
    assert call(layer=_layer(kind=9)) == E_UNS
    assert call(vb=FAKE + 4) == E_ALN
    assert call(ws=FAKE + 64) == E_ALN
    assert call(pos=_pos(4096 - 15)) == E_POS           # pos0 + n > capacity
    assert call(pos=_pos(-1)) == E_POS
    op = {"gqa_attn_verify": ga.OP_VERIFY, "gqa_attn_draft_block": ga.OP_DRAFT,
          "gqa_attn_prefill": ga.OP_PREFILL}[fn]
    need = ga.workspace_bytes(op, ga.GLOBAL, 1, 16, 4096)
    assert need > 0
    assert call(pos=_pos(4080), ws_bytes=need - 1) == E_WS
    if fn == "gqa_attn_draft_block":
        # a block predicted together is defined on global layers only
        assert ga.workspace_bytes(op, ga.LOCAL, 1, 16, 4096) == 0
        assert call(layer=_layer(kind=ga.LOCAL)) == E_UNS
        assert need == ga.workspace_bytes(ga.OP_VERIFY, ga.GLOBAL, 1, 16, 4096)
    # local layers need room for the rotated window in the workspace
    loc = ga.workspace_bytes(ga.OP_PREFILL, ga.LOCAL, 1, 4096, 131072)
    assert loc >= (2048 + 4096) * 512


def test_layer_kind_schedule(lib):
    """The library's layer schedule equals the oracle's reading of the pages
    (three local layers then one global: 39 + 13 of 52) and refuses indices
    outside the stack."""
    import oracle
    D = _defines()
    n = D["GQA_NUM_LAYERS"]
    assert n == 52 == ga.NUM_LAYERS
    kinds = [lib.gqa_layer_kind(l) for l in range(n)]
    assert kinds == [oracle.layer_kind(l) for l in range(n)]
    assert kinds == [ga.layer_kind(l) for l in range(n)]
    assert kinds.count(ga.LOCAL) == 39 and kinds.count(ga.GLOBAL) == 13
    assert kinds[:4] == [ga.LOCAL, ga.LOCAL, ga.LOCAL, ga.GLOBAL]
    for bad in (-1, n, 1 << 20):
        assert lib.gqa_layer_kind(bad) == E_ARG
    with pytest.raises(ga.GqaError):
        ga.layer_kind(n)


def test_position_bound(lib):
    """Positions above GQA_MAX_POSITION are refused before any launch (the
    kernels' 32-bit key-range arithmetic would wrap near 2^31); positions at
    the bound pass validation and stop at the (empty) workspace check."""
    top = _defines()["GQA_MAX_POSITION"]
    assert top == 2 ** 31 - 4097
    L = _layer(kind=ga.LOCAL)
    for fn in ("gqa_attn_verify", "gqa_attn_prefill"):
        f = getattr(lib, fn)
        assert f(ctypes.byref(L), FAKE, FAKE, FAKE, _pos(top - 14), 1, 16,
                 FAKE, FAKE, 1 << 30, None) == E_POS
        assert f(ctypes.byref(L), FAKE, FAKE, FAKE, _pos(top - 15), 1, 16,
                 FAKE, FAKE, 0, None) == E_WS
    assert _decode(lib, L, pos=_pos(top + 1)) == E_POS
    assert _decode(lib, L, pos=_pos(top), ws_bytes=0) == E_WS
    assert _append(lib, L, n=2, pos=_pos(top)) == E_POS


def test_decode_noalloc_validation(lib):
    """The entry point without a workspace validates like gqa_attn_decode
    before it touches its device scratch (these calls launch nothing)."""
    L = _layer()   # global, capacity 4096

    def call(layer=L, q=FAKE, kn=None, vn=None, pos=None, B=1, out=FAKE):
        pos = pos if pos is not None else _pos(*([10] * B))
        return lib.gqa_attn_decode_noalloc(
            ctypes.byref(layer) if layer is not None else None, q, kn, vn,
            pos, B, out, None)
    assert call(layer=None) == E_ARG
    assert call(q=None) == E_ARG
    assert call(out=None) == E_ARG
    assert call(B=0) == E_ARG
    assert call(kn=FAKE) == E_ARG            # k_new and v_new go together
    assert call(kn=FAKE, vn=FAKE + 2) == E_ALN
    assert call(layer=_layer(kind=7)) == E_UNS
    assert call(pos=_pos(4096)) == E_POS
    assert call(pos=_pos(-1)) == E_POS
    assert _defines()["GQA_NOALLOC_SCRATCH_BYTES"] == 8 << 20


def _layer8(kind=ga.GLOBAL, capacity=4096, k=FAKE, v=FAKE + (1 << 30),
            ks=FAKE + (2 << 30), vs=FAKE + (3 << 30), stride=None,
            sstride=None, theta=None, window=None):
    if kind == ga.LOCAL and capacity == 4096:
        capacity = ga.WINDOW
    if window is None:
        window = ga.WINDOW if kind == ga.LOCAL else 0
    if theta is None:
        theta = 10000.0 if kind == ga.LOCAL else 0.0
    return ga._CLayerFp8(kind, window, capacity, theta, k, v, ks, vs,
                         capacity * 256 if stride is None else stride,
                         2 * capacity if sstride is None else sstride)


def test_fp8_append_validation(lib):
    def call(L, B=1, n=1, kn=FAKE, vn=FAKE, pos=None):
        pos = pos if pos is not None else _pos(*([0] * B))
        return lib.gqa_kv_append_fp8(ctypes.byref(L) if L is not None else
                                     None, kn, vn, pos, B, n, None)
    L = _layer8()
    assert call(None) == E_ARG
    assert call(L, kn=None) == E_ARG
    assert call(L, B=0) == E_ARG
    assert call(L, n=0) == E_ARG
    assert call(_layer8(ks=0)) == E_ARG
    assert call(_layer8(vs=0)) == E_ARG
    assert call(_layer8(k=0)) == E_ARG
    assert call(_layer8(kind=4)) == E_UNS
    assert call(_layer8(kind=ga.LOCAL, capacity=4096 * 2)) == E_UNS
    assert call(_layer8(kind=ga.LOCAL, theta=0.0)) == E_UNS
    assert call(_layer8(stride=4096 * 256 - 16)) == E_ARG
    assert call(_layer8(sstride=2 * 4096 - 4)) == E_ARG
    assert call(_layer8(stride=4096 * 256 + 8)) == E_ALN
    assert call(_layer8(ks=FAKE + 4)) == E_ALN
    assert call(_layer8(v=FAKE + 8)) == E_ALN
    assert call(L, kn=FAKE + 2) == E_ALN
    assert call(L, pos=_pos(-1)) == E_POS
    assert call(L, n=2, pos=_pos(4095)) == E_POS


def test_fp8_decode_validation(lib):
    def call(L, B=1, q=FAKE, out=FAKE, pos=None, ws=FAKE, ws_bytes=1 << 30):
        pos = pos if pos is not None else _pos(*([10] * B))
        return lib.gqa_attn_decode_fp8(ctypes.byref(L) if L is not None else
                                       None, q, pos, B, out, ws, ws_bytes,
                                       None)
    L = _layer8()
    assert call(None) == E_ARG
    assert call(L, q=None) == E_ARG
    assert call(L, out=None) == E_ARG
    assert call(L, ws=None) == E_ARG
    assert call(L, B=65, pos=_pos(*([1] * 65))) == E_ARG
    assert call(_layer8(vs=0)) == E_ARG
    assert call(_layer8(kind=2)) == E_UNS
    assert call(L, q=FAKE + 4) == E_ALN
    assert call(L, ws=FAKE + 16) == E_ALN
    assert call(L, pos=_pos(4096)) == E_POS
    assert call(_layer8(kind=ga.LOCAL), pos=_pos(1 << 40)) == E_POS
    need = ga.workspace_bytes(ga.OP_DECODE, ga.GLOBAL, 1, 1, 4096)
    assert call(L, pos=_pos(4095), ws_bytes=need - 1) == E_WS


@pytest.mark.parametrize("fn", ["gqa_attn_verify_fp8",
                                "gqa_attn_draft_block_fp8",
                                "gqa_attn_prefill_fp8"])
def test_fp8_block_validation(lib, fn):
    f = getattr(lib, fn)
    L = _layer8()

    def call(layer=L, q=FAKE, kb=FAKE, vb=FAKE, pos=None, B=1, n=16,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30):
        pos = pos if pos is not None else _pos(*([0] * B))
        return f(ctypes.byref(layer) if layer is not None else None, q, kb, vb,
                 pos, B, n, out, ws, ws_bytes, None)
    assert call(layer=None) == E_ARG
    assert call(q=None) == E_ARG
    assert call(kb=None) == E_ARG
    assert call(vb=None) == E_ARG
    assert call(out=None) == E_ARG
    assert call(n=0) == E_ARG
    if fn != "gqa_attn_prefill_fp8":
        assert call(n=17) == E_ARG                      # block of at most 16
    else:
        assert call(n=17, pos=_pos(0), ws_bytes=0) == E_WS
        assert call(n=ga.MAX_CONTEXT + 1) == E_ARG
    assert call(B=0) == E_ARG
    assert call(ws=None) == E_ARG
    assert call(layer=_layer8(ks=0)) == E_ARG
    assert call(layer=_layer8(kind=5)) == E_UNS
    assert call(kb=FAKE + 4) == E_ALN
    assert call(layer=_layer8(vs=FAKE + 4)) == E_ALN
    assert call(ws=FAKE + 64) == E_ALN
    assert call(pos=_pos(4096 - 15)) == E_POS           # pos0 + n > capacity
    assert call(pos=_pos(-1)) == E_POS
    op = {"gqa_attn_verify_fp8": ga.OP_VERIFY,
          "gqa_attn_draft_block_fp8": ga.OP_DRAFT,
          "gqa_attn_prefill_fp8": ga.OP_PREFILL}[fn]
    if fn == "gqa_attn_prefill_fp8":
        op = ga.OP_PREFILL_FP8
    need = ga.workspace_bytes(op, ga.GLOBAL, 1, 16, 4096)
    assert call(pos=_pos(4080), ws_bytes=need - 1) == E_WS
    if fn == "gqa_attn_draft_block_fp8":
        assert call(layer=_layer8(kind=ga.LOCAL)) == E_UNS
    elif fn == "gqa_attn_prefill_fp8":
        # the bf16 prefill's workspace plus a bf16 copy of the prior
        # (1 KiB per token: positions before the chunk, or the ring)
        bf = ga.workspace_bytes(ga.OP_PREFILL, ga.GLOBAL, 1, 16, 4096)
        assert need >= bf + (4096 - 1) * 1024
        loc = ga.workspace_bytes(op, ga.LOCAL, 1, 16, 4096)
        assert loc >= 2048 * 1024
        assert call(layer=_layer8(kind=ga.LOCAL), pos=_pos(4080),
                    ws_bytes=loc - 1) == E_WS
    else:
        # the local workspace query covers the fp8 call's key splits
        need = ga.workspace_bytes(op, ga.LOCAL, 1, 16, 4096)
        assert call(layer=_layer8(kind=ga.LOCAL), pos=_pos(4080),
                    ws_bytes=need - 1) == E_WS
