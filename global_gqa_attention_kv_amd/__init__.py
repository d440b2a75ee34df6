"""Python binding of libgqa_attn.so: grouped-query attention (32 query heads,
2 KV heads, head dim 128) with a hybrid local / global KV cache on MI355X.

This module only marshals arguments: it checks tensor placement, dtype and
shape, then calls the C ABI declared in ``include/gqa_attn.h`` with raw device
pointers and the current HIP stream.  Every step of the computation runs in
the library's HIP kernels; there is no fallback.  If the library has not been
built, importing works but the first call raises :class:`LibraryMissing`.

PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LOCAL", "GLOBAL", "OP_DECODE", "OP_VERIFY", "OP_PREFILL", "OP_DRAFT",
    "OP_PREFILL_FP8",
    "MAX_VERIFY", "attn_verify", "attn_draft_block", "attn_prefill", "HQ", "HKV", "D", "WINDOW", "MAX_CONTEXT",
    "MAX_BATCH", "GqaError", "LibraryMissing", "Layer", "kv_append",
    "attn_decode", "attn_decode_append", "attn_decode_dev",
    "attn_decode_noalloc", "LayerFp8", "kv_append_fp8", "attn_decode_fp8",
    "attn_verify_fp8", "attn_draft_block_fp8", "attn_prefill_fp8", "workspace_bytes", "workspace", "status_string", "abi_version",
    "library_path", "layer_kind", "NUM_LAYERS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libgqa_attn.so")

LOCAL, GLOBAL = 0, 1
OP_DECODE, OP_VERIFY, OP_PREFILL, OP_DRAFT, OP_PREFILL_FP8 = 0, 1, 2, 3, 4
MAX_VERIFY = 16
HQ, HKV, D, WINDOW, MAX_CONTEXT, MAX_BATCH = 32, 2, 128, 2048, 131072, 64
NUM_LAYERS = 52
ROPE_THETA = 10000.0

_lib = None


class LibraryMissing(RuntimeError):
    pass


class GqaError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s failed: %s (%d)" % (what, status_string(status),
                                                 status))
        self.status = status


class _CLayer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("rope_theta", ctypes.c_double),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("seq_stride", ctypes.c_int64)]


class _CLayerFp8(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("rope_theta", ctypes.c_double),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("seq_stride", ctypes.c_int64),
                ("scale_stride", ctypes.c_int64)]


def library_path() -> str:
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                "libgqa_attn.so is not built; run "
                "`python -m global_gqa_attention_kv_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L = ctypes.POINTER(_CLayer)
        lib.gqa_abi_version.restype = i32
        lib.gqa_layer_kind.restype = i32
        lib.gqa_layer_kind.argtypes = [i32]
        lib.gqa_status_string.restype = ctypes.c_char_p
        lib.gqa_status_string.argtypes = [i32]
        lib.gqa_workspace_bytes.restype = ctypes.c_size_t
        lib.gqa_workspace_bytes.argtypes = [i32, i32, i32, i32, i64]
        lib.gqa_kv_append.restype = i32
        lib.gqa_kv_append.argtypes = [L, p, p, p, i32, i32, p]
        lib.gqa_attn_decode.restype = i32
        lib.gqa_attn_decode.argtypes = [L, p, p, i32, p, p, ctypes.c_size_t, p]
        lib.gqa_attn_verify.restype = i32
        lib.gqa_attn_verify.argtypes = [L, p, p, p, p, i32, i32, p, p,
                                        ctypes.c_size_t, p]
        lib.gqa_attn_draft_block.restype = i32
        lib.gqa_attn_draft_block.argtypes = [L, p, p, p, p, i32, i32, p, p,
                                             ctypes.c_size_t, p]
        lib.gqa_attn_prefill.restype = i32
        lib.gqa_attn_prefill.argtypes = [L, p, p, p, p, i32, i32, p, p,
                                         ctypes.c_size_t, p]
        lib.gqa_attn_decode_append.restype = i32
        lib.gqa_attn_decode_append.argtypes = [L, p, p, p, p, i32, p, p,
                                               ctypes.c_size_t, p]
        lib.gqa_attn_decode_dev.restype = i32
        lib.gqa_attn_decode_dev.argtypes = [L, p, p, p, p, i64, i32, p, p,
                                            ctypes.c_size_t, p]
        L8 = ctypes.POINTER(_CLayerFp8)
        lib.gqa_kv_append_fp8.restype = i32
        lib.gqa_kv_append_fp8.argtypes = [L8, p, p, p, i32, i32, p]
        lib.gqa_attn_decode_fp8.restype = i32
        lib.gqa_attn_decode_fp8.argtypes = [L8, p, p, i32, p, p,
                                            ctypes.c_size_t, p]
        for name in ("gqa_attn_verify_fp8", "gqa_attn_draft_block_fp8",
                     "gqa_attn_prefill_fp8"):
            f = getattr(lib, name)
            f.restype = i32
            f.argtypes = [L8, p, p, p, p, i32, i32, p, p, ctypes.c_size_t, p]
        lib.gqa_attn_decode_noalloc.restype = i32
        lib.gqa_attn_decode_noalloc.argtypes = [L, p, p, p, p, i32, p, p]
        _lib = lib
    return _lib


def abi_version() -> int:
    return _load().gqa_abi_version()


def status_string(status: int) -> str:
    return _load().gqa_status_string(int(status)).decode()


def workspace_bytes(op: int, kind: int, B: int, n: int, max_ctx: int) -> int:
    return int(_load().gqa_workspace_bytes(op, kind, B, n, int(max_ctx)))


def layer_kind(layer_index: int) -> int:
    """Kind of layer ``layer_index`` (0 .. NUM_LAYERS-1) of the stack, as the
    library's schedule gives it (``gqa_layer_kind``: three local layers, then
    one global layer, repeating)."""
    kind = _load().gqa_layer_kind(int(layer_index))
    if kind < 0:
        raise GqaError(kind, "gqa_layer_kind")
    return kind


class Layer:
    """One attention layer's K/V cache, held in caller-owned torch tensors.

    k, v: bf16 [B, capacity, 2, 128] on the GPU.  Local layers have capacity
    2048 (a ring, slot = position mod 2048) and RoPE base ``rope_theta``;
    global layers have capacity up to 131072 (slot = position) and no RoPE."""

    def __init__(self, kind, k, v, rope_theta=None):
        self.kind = int(kind)
        self.k = k
        self.v = v
        if rope_theta is None:
            rope_theta = ROPE_THETA if self.kind == LOCAL else 0.0
        self.rope_theta = float(rope_theta)
        assert k.shape == v.shape and k.dim() == 4
        self.batch, self.capacity = int(k.shape[0]), int(k.shape[1])
        self._c = _CLayer(self.kind, WINDOW if self.kind == LOCAL else 0,
                          self.capacity, self.rope_theta, k.data_ptr(),
                          v.data_ptr(), int(k.stride(0)))
        if k.stride(0) != v.stride(0):
            raise ValueError("k and v must share the sequence stride")

    @classmethod
    def allocate(cls, kind, batch, capacity=None, device="cuda", fill=None):
        if capacity is None:
            capacity = WINDOW if kind == LOCAL else MAX_CONTEXT
        shape = (batch, capacity, HKV, D)
        if fill is None:
            k = torch.empty(shape, dtype=torch.bfloat16, device=device)
            v = torch.empty(shape, dtype=torch.bfloat16, device=device)
        else:
            k = torch.full(shape, fill, dtype=torch.bfloat16, device=device)
            v = torch.full(shape, fill, dtype=torch.bfloat16, device=device)
        return cls(kind, k, v)

    @property
    def c_ref(self):
        return ctypes.byref(self._c)


class LayerFp8:
    """One attention layer's fp8 cache in caller-owned torch tensors: E4M3
    codes k, v (uint8 [B, capacity, 2, 128]) and one fp32 scale per (token,
    KV head), k_scale, v_scale (float32 [B, 2, capacity]).  Kinds, capacities
    and RoPE as :class:`Layer`."""

    def __init__(self, kind, k, v, k_scale, v_scale, rope_theta=None):
        self.kind = int(kind)
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        if rope_theta is None:
            rope_theta = ROPE_THETA if self.kind == LOCAL else 0.0
        self.rope_theta = float(rope_theta)
        assert k.shape == v.shape and k.dim() == 4 and k.dtype == torch.uint8
        assert k_scale.shape == v_scale.shape and k_scale.dim() == 3
        assert k_scale.dtype == torch.float32
        self.batch, self.capacity = int(k.shape[0]), int(k.shape[1])
        if tuple(k_scale.shape) != (self.batch, HKV, self.capacity) or \
                k_scale.stride(1) != self.capacity or k_scale.stride(2) != 1:
            raise ValueError("scales must be [B, 2, capacity] with unit stride")
        if k.stride(0) != v.stride(0) or k_scale.stride(0) != v_scale.stride(0):
            raise ValueError("k and v (and their scales) share their strides")
        self._c = _CLayerFp8(self.kind, WINDOW if self.kind == LOCAL else 0,
                             self.capacity, self.rope_theta, k.data_ptr(),
                             v.data_ptr(), k_scale.data_ptr(),
                             v_scale.data_ptr(), int(k.stride(0)),
                             int(k_scale.stride(0)))

    @classmethod
    def allocate(cls, kind, batch, capacity=None, device="cuda", fill=0):
        """Codes filled with the byte ``fill``, scales with 0."""
        if capacity is None:
            capacity = WINDOW if kind == LOCAL else MAX_CONTEXT
        shape = (batch, capacity, HKV, D)
        k = torch.full(shape, fill, dtype=torch.uint8, device=device)
        v = torch.full(shape, fill, dtype=torch.uint8, device=device)
        ks = torch.zeros((batch, HKV, capacity), dtype=torch.float32,
                         device=device)
        vs = torch.zeros_like(ks)
        return cls(kind, k, v, ks, vs)

    @property
    def c_ref(self):
        return ctypes.byref(self._c)


def kv_append_fp8(layer: LayerFp8, k_new, v_new, pos0, stream=None):
    """Quantise n new tokens per sequence (k_new, v_new: bf16 [B, n, 2, 128])
    into the layer's fp8 cache at positions pos0[b] .. pos0[b]+n-1."""
    B, n = int(k_new.shape[0]), int(k_new.shape[1])
    kp = _dev(k_new, torch.bfloat16, (B, n, HKV, D), "k_new")
    vp = _dev(v_new, torch.bfloat16, (B, n, HKV, D), "v_new")
    rc = _load().gqa_kv_append_fp8(layer.c_ref, kp, vp, _positions(pos0, B),
                                   B, n, _stream(stream))
    if rc != 0:
        raise GqaError(rc, "gqa_kv_append_fp8")


def attn_decode_fp8(layer: LayerFp8, q, pos, out=None, ws=None, stream=None):
    """One decode step over an fp8 cache: q bf16 [B, 32, 128] at host
    positions pos (the token already appended).  Returns fp32
    [B, 32, 128]."""
    return _decode_common(_load().gqa_attn_decode_fp8, "gqa_attn_decode_fp8",
                          layer, q, pos, out, ws, stream)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape),
                                                             tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


def _positions(pos, B):
    arr = (ctypes.c_int64 * B)()
    vals = pos.tolist() if isinstance(pos, torch.Tensor) else list(pos)
    if len(vals) != B:
        raise ValueError("need %d positions, got %d" % (B, len(vals)))
    for i, x in enumerate(vals):
        arr[i] = int(x)
    return arr


def kv_append(layer: Layer, k_new, v_new, pos0, stream=None):
    """Write n new tokens per sequence into the layer cache.
    k_new, v_new: bf16 [B, n, 2, 128]; pos0: B host positions."""
    B, n = int(k_new.shape[0]), int(k_new.shape[1])
    kp = _dev(k_new, torch.bfloat16, (B, n, HKV, D), "k_new")
    vp = _dev(v_new, torch.bfloat16, (B, n, HKV, D), "v_new")
    rc = _load().gqa_kv_append(layer.c_ref, kp, vp, _positions(pos0, B), B, n,
                               _stream(stream))
    if rc != 0:
        raise GqaError(rc, "gqa_kv_append")


def workspace(op, kind, B, n, max_ctx, device="cuda"):
    """A workspace tensor for the given operation and shape (no
    initialisation needed; one tensor may serve every operation issued in
    order on a stream)."""
    need = workspace_bytes(op, kind, B, n, max_ctx)
    if need == 0:
        raise ValueError("invalid workspace request")
    return torch.empty(need, dtype=torch.uint8, device=device)


def _decode_common(fn, name, layer, q, pos, out, ws, stream, extra=()):
    B = int(q.shape[0])
    qp = _dev(q, torch.bfloat16, (B, HQ, D), "q")
    if out is None:
        out = torch.empty((B, HQ, D), dtype=torch.float32, device=q.device)
    op = _dev(out, torch.float32, (B, HQ, D), "out")
    posc = _positions(pos, B)
    if ws is None:
        ws = workspace(OP_DECODE, layer.kind, B, 1,
                       max(int(x) for x in posc) + 1, device=q.device)
    wp = _dev(ws, ws.dtype, None, "ws")
    args = (layer.c_ref, qp) + tuple(extra) + (posc, B, op, wp,
                                               ws.numel() * ws.element_size(),
                                               _stream(stream))
    rc = fn(*args)
    if rc != 0:
        raise GqaError(rc, name)
    return out


def attn_decode(layer: Layer, q, pos, out=None, ws=None, stream=None):
    """One decode step.  q: bf16 [B, 32, 128]; pos: B host positions of the
    query tokens (already appended).  ws: workspace (see
    :func:`workspace`), allocated per call when omitted.
    Returns out: fp32 [B, 32, 128]."""
    return _decode_common(_load().gqa_attn_decode, "gqa_attn_decode", layer,
                          q, pos, out, ws, stream)


def attn_decode_append(layer: Layer, q, k_new, v_new, pos, out=None, ws=None,
                       stream=None):
    """Append the new token (k_new, v_new: bf16 [B, 1, 2, 128]) at pos and
    attend, in one launch.  Returns out: fp32 [B, 32, 128]."""
    B = int(q.shape[0])
    kp = _dev(k_new, torch.bfloat16, (B, 1, HKV, D), "k_new")
    vp = _dev(v_new, torch.bfloat16, (B, 1, HKV, D), "v_new")
    return _decode_common(_load().gqa_attn_decode_append,
                          "gqa_attn_decode_append", layer, q, pos, out, ws,
                          stream, extra=(kp, vp))


def attn_decode_dev(layer: Layer, q, pos_dev, max_pos, out=None, ws=None,
                    k_new=None, v_new=None, stream=None):
    """Decode with device-resident positions (for graph replays that
    advance them).  pos_dev: int64 GPU tensor [B], read when the kernels
    run; max_pos: host bound on every entry (a position outside 0..max_pos
    gives NaN rows and appends nothing).  k_new / v_new: both None (attend
    only) or bf16 [B, 1, 2, 128] (append at pos_dev, then attend).
    Returns out: fp32 [B, 32, 128]."""
    B = int(q.shape[0])
    qp = _dev(q, torch.bfloat16, (B, HQ, D), "q")
    pp = _dev(pos_dev, torch.int64, (B,), "pos_dev")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    kp = vp = None
    if k_new is not None:
        kp = _dev(k_new, torch.bfloat16, (B, 1, HKV, D), "k_new")
        vp = _dev(v_new, torch.bfloat16, (B, 1, HKV, D), "v_new")
    if out is None:
        out = torch.empty((B, HQ, D), dtype=torch.float32, device=q.device)
    op = _dev(out, torch.float32, (B, HQ, D), "out")
    if ws is None:
        ws = workspace(OP_DECODE, layer.kind, B, 1, int(max_pos) + 1,
                       device=q.device)
    wp = _dev(ws, ws.dtype, None, "ws")
    rc = _load().gqa_attn_decode_dev(layer.c_ref, qp, kp, vp, pp,
                                     int(max_pos), B, op, wp,
                                     ws.numel() * ws.element_size(),
                                     _stream(stream))
    if rc != 0:
        raise GqaError(rc, "gqa_attn_decode_dev")
    return out


def attn_decode_noalloc(layer: Layer, q, pos, out=None, k_new=None,
                        v_new=None, stream=None):
    """Decode without a workspace (the library's device-resident scratch
    holds the split partials), for callers that cannot allocate, e.g. under
    graph capture.  k_new / v_new: both None (attend only) or bf16
    [B, 1, 2, 128] (append at pos, then attend).  Pass ``out`` to allocate
    nothing here either.  Calls overlapping in time on one GPU race; make the
    first call on a device outside a graph capture.
    Returns out: fp32 [B, 32, 128]."""
    B = int(q.shape[0])
    qp = _dev(q, torch.bfloat16, (B, HQ, D), "q")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    kp = vp = None
    if k_new is not None:
        kp = _dev(k_new, torch.bfloat16, (B, 1, HKV, D), "k_new")
        vp = _dev(v_new, torch.bfloat16, (B, 1, HKV, D), "v_new")
    if out is None:
        out = torch.empty((B, HQ, D), dtype=torch.float32, device=q.device)
    op = _dev(out, torch.float32, (B, HQ, D), "out")
    rc = _load().gqa_attn_decode_noalloc(layer.c_ref, qp, kp, vp,
                                         _positions(pos, B), B, op,
                                         _stream(stream))
    if rc != 0:
        raise GqaError(rc, "gqa_attn_decode_noalloc")
    return out


def _block_common(fn, name, op, out_dtype, layer, q, k_blk, v_blk, pos0, out,
                  ws, stream):
    B, n = int(q.shape[0]), int(q.shape[1])
    qp = _dev(q, torch.bfloat16, (B, n, HQ, D), "q")
    kp = _dev(k_blk, torch.bfloat16, (B, n, HKV, D), "k_blk")
    vp = _dev(v_blk, torch.bfloat16, (B, n, HKV, D), "v_blk")
    if out is None:
        out = torch.empty((B, n, HQ, D), dtype=out_dtype, device=q.device)
    op_ = _dev(out, out_dtype, (B, n, HQ, D), "out")
    posc = _positions(pos0, B)
    if ws is None:
        need = workspace_bytes(op, layer.kind, B, n,
                               max(int(x) for x in posc) + n)
        if need == 0:
            raise GqaError(-1, name)
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp = _dev(ws, ws.dtype, None, "ws")
    rc = fn(layer.c_ref, qp, kp, vp, posc, B, n, op_, wp,
            ws.numel() * ws.element_size(), _stream(stream))
    if rc != 0:
        raise GqaError(rc, name)
    return out


def attn_verify(layer: Layer, q, k_blk, v_blk, pos0, out=None, ws=None,
                stream=None):
    """Verify a drafted block: q bf16 [B, n, 32, 128] (n <= 16) at positions
    pos0[b] .. pos0[b]+n-1; k_blk, v_blk bf16 [B, n, 2, 128] (not yet in the
    cache).  Returns fp32 [B, n, 32, 128].  The cache is not modified."""
    return _block_common(_load().gqa_attn_verify, "gqa_attn_verify",
                         OP_VERIFY, torch.float32, layer, q, k_blk, v_blk,
                         pos0, out, ws, stream)


def attn_verify_fp8(layer: LayerFp8, q, k_blk, v_blk, pos0, out=None,
                    ws=None, stream=None):
    """:func:`attn_verify` over an fp8 cache: the cached tokens are read as
    their dequantised values, the block's own tokens (k_blk, v_blk bf16, not
    in the cache) at their bf16 values.  Returns fp32 [B, n, 32, 128]."""
    return _block_common(_load().gqa_attn_verify_fp8, "gqa_attn_verify_fp8",
                         OP_VERIFY, torch.float32, layer, q, k_blk, v_blk,
                         pos0, out, ws, stream)


def attn_draft_block_fp8(layer: LayerFp8, q, k_blk, v_blk, pos0, out=None,
                         ws=None, stream=None):
    """:func:`attn_draft_block` over an fp8 cache (global layers)."""
    return _block_common(_load().gqa_attn_draft_block_fp8,
                         "gqa_attn_draft_block_fp8", OP_DRAFT, torch.float32,
                         layer, q, k_blk, v_blk, pos0, out, ws, stream)


def attn_prefill_fp8(layer: LayerFp8, q, k_chunk, v_chunk, pos0, out=None,
                     ws=None, stream=None):
    """:func:`attn_prefill` over an fp8 cache: the cached tokens are read as
    their dequantised values, the chunk's own tokens at their bf16 values.
    Returns bf16 [B, n, 32, 128]; append the chunk with
    :func:`kv_append_fp8` afterwards."""
    return _block_common(_load().gqa_attn_prefill_fp8, "gqa_attn_prefill_fp8",
                         OP_PREFILL_FP8, torch.bfloat16, layer, q, k_chunk,
                         v_chunk, pos0, out, ws, stream)


def attn_draft_block(layer: Layer, q, k_blk, v_blk, pos0, out=None, ws=None,
                     stream=None):
    """Attention of a drafted block predicted together (one block-diffusion
    drafting step): q bf16 [B, n, 32, 128] (n <= 16) at positions pos0[b] ..
    pos0[b]+n-1, k_blk, v_blk bf16 [B, n, 2, 128] (not in the cache); every
    block token sees the cached context and the whole block.  Global layers
    only.  Returns fp32 [B, n, 32, 128]; the cache is not modified."""
    return _block_common(_load().gqa_attn_draft_block, "gqa_attn_draft_block",
                         OP_DRAFT, torch.float32, layer, q, k_blk, v_blk,
                         pos0, out, ws, stream)


def attn_prefill(layer: Layer, q, k_chunk, v_chunk, pos0, out=None, ws=None,
                 stream=None):
    """Prefill a chunk: q bf16 [B, n, 32, 128] at positions pos0[b] ..
    pos0[b]+n-1 with its own K/V (k_chunk, v_chunk bf16 [B, n, 2, 128], not
    yet in the cache).  Returns bf16 [B, n, 32, 128].  The cache is not
    modified; append the chunk with :func:`kv_append` afterwards."""
    return _block_common(_load().gqa_attn_prefill, "gqa_attn_prefill",
                         OP_PREFILL, torch.bfloat16, layer, q, k_chunk,
                         v_chunk, pos0, out, ws, stream)
