"""ctypes binding of libsqg.so.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Torch supplies device memory (tensor storage) and the current HIP
stream.  There is no CPU fallback: if libsqg.so is missing or a tensor is not on
the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsqg.so")

SQG_INT4_ROT = 0
SQG_INT8_ROT = 1
SQG_BF16_ROT = 2
SQG_F32, SQG_BF16, SQG_F16 = 0, 1, 2
SQG_EMIT_QKV, SQG_EMIT_Q, SQG_EMIT_KV = 0, 1, 2
SQG_QK_EXACT, SQG_QK_FP8 = 0, 1
MAX_SEGMENTS = 16
HEAD_DIM = 128

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class SqgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("sqg status %d: %s" % (status, message))
        self.status = status


class Range(ctypes.Structure):
    _fields_ = [("begin", _c_i64), ("end", _c_i64), ("fmt", _c_i32), ("reserved", _c_i32),
                ("int8_heads", ctypes.c_uint64)]


class Layout(ctypes.Structure):
    _fields_ = [("n_tokens", _c_i64), ("n_heads", _c_i32), ("n_segments", _c_i32),
                ("seg_begin", _c_i64 * MAX_SEGMENTS), ("seg_end", _c_i64 * MAX_SEGMENTS),
                ("seg_offset", _c_i64 * MAX_SEGMENTS), ("seg_fmt", _c_i32 * MAX_SEGMENTS),
                ("seg_row_bytes", _c_i32 * MAX_SEGMENTS),
                ("seg_int8_heads", ctypes.c_uint64 * MAX_SEGMENTS), ("q_bytes", _c_i64),
                ("pack_bytes", _c_i64), ("scale_bytes", _c_i64), ("bf16_qkv_bytes", _c_i64)]


class QkvArgs(ctypes.Structure):
    _fields_ = [("n_tokens", _c_i64), ("d_model", _c_i32), ("n_heads", _c_i32),
                ("x", _vp), ("ldx", _c_i64), ("w_qkv", _vp), ("ldw", _c_i64),
                ("q_norm_w", _vp), ("k_norm_w", _vp), ("eps", ctypes.c_float),
                ("rope_cos", _vp), ("rope_sin", _vp),
                ("ranges", ctypes.POINTER(Range)), ("n_ranges", _c_i32), ("emit", _c_i32),
                ("chunk_rows", _c_i64), ("min_tail", _c_i64),
                ("q", _vp), ("ldq", _c_i64), ("kpack", _vp), ("vpack", _vp),
                ("kscale", _vp), ("vscale", _vp)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("n_tokens", _c_i64), ("d_model", _c_i32), ("n_heads", _c_i32),
                ("q", _vp), ("ldq", _c_i64), ("kpack", _vp), ("vpack", _vp),
                ("kscale", _vp), ("vscale", _vp),
                ("ranges", ctypes.POINTER(Range)), ("n_ranges", _c_i32), ("o_dtype", _c_i32),
                ("q_begin", _c_i64), ("q_end", _c_i64), ("kv_begin", _c_i64), ("kv_end", _c_i64),
                ("kv_block", _c_i64), ("accumulate", _c_i32), ("softmax_scale", ctypes.c_float),
                ("o", _vp), ("ldo", _c_i64), ("lse", _vp), ("qk_mode", _c_i32),
                ("reserved", _c_i32)]


class StagedKV(ctypes.Structure):
    _fields_ = [("block_rows", _c_i64), ("host_kpack", _vp), ("host_vpack", _vp),
                ("host_kscale", _vp), ("host_vscale", _vp), ("dev_kpack", _vp * 2),
                ("dev_vpack", _vp * 2), ("dev_kscale", _vp * 2), ("dev_vscale", _vp * 2),
                ("copy_stream", _vp)]


class QRecomputeArgs(ctypes.Structure):
    _fields_ = [("attn", AttnArgs), ("x", _vp), ("ldx", _c_i64), ("w_qkv", _vp), ("ldw", _c_i64),
                ("q_norm_w", _vp), ("rope_cos", _vp), ("rope_sin", _vp), ("eps", ctypes.c_float),
                ("reserved", _c_i32), ("q_chunk_rows", _c_i64), ("workspace", _vp),
                ("workspace_bytes", _c_i64)]


_lib = None


def load(path: Optional[str] = None):
    """Load libsqg.so (built by __graft_entry__.build() / streamed_qkv_gemm_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError("libsqg.so not found at %s: build it first with "
                           "`python -m streamed_qkv_gemm_amd.build`" % path)
    lib = ctypes.CDLL(path)
    lib.sqg_version.restype = ctypes.c_int
    lib.sqg_status_string.restype = ctypes.c_char_p
    lib.sqg_status_string.argtypes = [ctypes.c_int]
    lib.sqg_last_error.restype = ctypes.c_char_p
    lib.sqg_struct_size.restype = _c_i64
    lib.sqg_struct_size.argtypes = [ctypes.c_int]
    lib.sqg_chunk_ranges.argtypes = [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_i64),
                                     ctypes.POINTER(_c_i64), _c_i32, ctypes.POINTER(_c_i32)]
    lib.sqg_kv_layout.argtypes = [_c_i64, _c_i32, _c_i32, ctypes.POINTER(Range), _c_i32,
                                  ctypes.POINTER(Layout)]
    lib.sqg_rope_table.argtypes = [_c_i64, _c_i64, ctypes.c_double, _vp, _vp]
    lib.sqg_streamed_qkv_quant.argtypes = [ctypes.POINTER(QkvArgs), _vp]
    lib.sqg_packed_kv_attention.argtypes = [ctypes.POINTER(AttnArgs), _vp]
    lib.sqg_kv_row_offset.restype = _c_i64
    lib.sqg_kv_row_offset.argtypes = [ctypes.POINTER(Layout), _c_i32, _c_i64]
    lib.sqg_kv_block_layout.argtypes = [_c_i64, _c_i32, _c_i32, ctypes.POINTER(Range), _c_i32,
                                        _c_i64, _c_i64, ctypes.POINTER(Layout)]
    lib.sqg_staged_sizes.argtypes = [_c_i64, _c_i32, _c_i32, ctypes.POINTER(Range), _c_i32, _c_i64,
                                     ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i32)]
    lib.sqg_streamed_qkv_quant_staged.argtypes = [ctypes.POINTER(QkvArgs), ctypes.POINTER(StagedKV), _vp]
    lib.sqg_packed_kv_attention_staged.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(StagedKV), _vp]
    lib.sqg_qrecompute_workspace_bytes.restype = _c_i64
    lib.sqg_qrecompute_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i32]
    lib.sqg_packed_kv_attention_qrecompute.argtypes = [ctypes.POINTER(QRecomputeArgs), _vp]
    lib.sqg_packed_kv_attention_qrecompute_noalloc.argtypes = [ctypes.POINTER(QRecomputeArgs), _vp]
    lib.sqg_noalloc_scratch_bytes.restype = _c_i64
    lib.sqg_test_quant_pack_f32.argtypes = [_vp, _c_i64, _c_i32, _vp, _vp, _vp]
    lib.sqg_test_fwht_f32.argtypes = [_vp, _vp, _c_i64, _c_i32, _vp]
    for name, cls in ((0, Range), (1, Layout), (2, QkvArgs), (3, AttnArgs), (4, QRecomputeArgs),
                      (5, StagedKV)):
        got = lib.sqg_struct_size(name)
        if got != ctypes.sizeof(cls):
            raise RuntimeError("ABI mismatch: %s is %d bytes in the library, %d in the binding"
                               % (cls.__name__, got, ctypes.sizeof(cls)))
    _lib = lib
    return lib


def lib_path() -> str:
    return LIB_PATH


def _check(status: int):
    if status != 0:
        lib = load()
        raise SqgError(status, lib.sqg_last_error().decode())


def _ranges_array(ranges: Optional[Sequence[Tuple[int, int, int]]]):
    if not ranges:
        return None, 0
    arr = (Range * len(ranges))()
    for i, r in enumerate(ranges):
        arr[i].begin, arr[i].end, arr[i].fmt, arr[i].reserved = int(r[0]), int(r[1]), int(r[2]), 0
        arr[i].int8_heads = int(r[3]) if len(r) > 3 else 0
    return arr, len(ranges)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev_ptr(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (the library has no CPU path)" % name)
    return t.data_ptr()


def version() -> int:
    return load().sqg_version()


def chunk_ranges(n: int, size: int, min_tail: int = 512):
    lib = load()
    count = _c_i32(0)
    _check(lib.sqg_chunk_ranges(n, size, min_tail, None, None, 0, ctypes.byref(count)))
    cap = count.value
    b = (_c_i64 * max(cap, 1))()
    e = (_c_i64 * max(cap, 1))()
    _check(lib.sqg_chunk_ranges(n, size, min_tail, b, e, cap, ctypes.byref(count)))
    return [(b[i], e[i]) for i in range(count.value)]


def _layout_dict(L) -> Dict:
    segs = [{"begin": L.seg_begin[i], "end": L.seg_end[i], "fmt": L.seg_fmt[i],
             "int8_heads": L.seg_int8_heads[i], "offset": L.seg_offset[i],
             "row_bytes": L.seg_row_bytes[i]} for i in range(L.n_segments)]
    return {"n_tokens": L.n_tokens, "n_heads": L.n_heads, "segments": segs,
            "q_bytes": L.q_bytes, "pack_bytes": L.pack_bytes, "scale_bytes": L.scale_bytes,
            "bf16_qkv_bytes": L.bf16_qkv_bytes, "_struct": L}


def kv_row_offset(layout: Dict, head: int, token: int) -> int:
    """Byte offset of the row of (head, token) in a store laid out by `layout`."""
    return load().sqg_kv_row_offset(ctypes.byref(layout["_struct"]), head, token)


def kv_block_layout(n_tokens: int, d_model: int, key_begin: int, key_end: int, ranges=None) -> Dict:
    """Layout of the block store that holds keys [key_begin, key_end)."""
    lib = load()
    arr, nr = _ranges_array(ranges)
    L = Layout()
    _check(lib.sqg_kv_block_layout(n_tokens, d_model, d_model // HEAD_DIM, arr, nr, key_begin,
                                   key_end, ctypes.byref(L)))
    return _layout_dict(L)


def kv_layout(n_tokens: int, d_model: int, ranges=None) -> Dict:
    lib = load()
    arr, nr = _ranges_array(ranges)
    L = Layout()
    _check(lib.sqg_kv_layout(n_tokens, d_model, d_model // HEAD_DIM, arr, nr, ctypes.byref(L)))
    return _layout_dict(L)


def rope_table(n_tokens: int, theta: float = 10000.0, pos0: int = 0, device="cuda"):
    """fp32 [N, 64] cos and sin tables built by the library on the host (fp64 -> fp32)."""
    lib = load()
    cos = torch.empty((n_tokens, 64), dtype=torch.float32)
    sin = torch.empty((n_tokens, 64), dtype=torch.float32)
    _check(lib.sqg_rope_table(pos0, n_tokens, theta, cos.data_ptr(), sin.data_ptr()))
    return cos.to(device), sin.to(device)


def alloc_store(n_tokens: int, d_model: int, ranges=None, device="cuda", emit: int = SQG_EMIT_QKV):
    """Empty output buffers of the streamed QKV-quant: Q, packed K/V and scales.

    With emit SQG_EMIT_KV there is no Q buffer ("q" is None); with SQG_EMIT_Q no
    packed store."""
    L = kv_layout(n_tokens, d_model, ranges)
    H = d_model // HEAD_DIM
    want_q, want_kv = emit != SQG_EMIT_KV, emit != SQG_EMIT_Q
    empty = lambda *shape, dtype: torch.empty(shape, dtype=dtype, device=device)  # noqa: E731
    return {
        "q": empty(n_tokens, d_model, dtype=torch.bfloat16) if want_q else None,
        "kpack": empty(max(L["pack_bytes"], 16), dtype=torch.uint8) if want_kv else None,
        "vpack": empty(max(L["pack_bytes"], 16), dtype=torch.uint8) if want_kv else None,
        "kscale": empty(H, n_tokens, 4, dtype=torch.float16) if want_kv else None,
        "vscale": empty(H, n_tokens, 4, dtype=torch.float16) if want_kv else None,
        "layout": L,
        "ranges": list(ranges) if ranges else None,
        "n_tokens": n_tokens,
        "d_model": d_model,
    }


def streamed_qkv_quant(x: torch.Tensor, w_qkv: torch.Tensor, ranges=None, chunk_rows: int = 0,
                       min_tail: int = 512, q_norm_w: Optional[torch.Tensor] = None,
                       k_norm_w: Optional[torch.Tensor] = None, eps: float = 1e-6,
                       rope_cos: Optional[torch.Tensor] = None,
                       rope_sin: Optional[torch.Tensor] = None, out: Optional[Dict] = None,
                       emit: int = SQG_EMIT_QKV):
    """streamed_qkv_quant(x, W_qkv, range_policy) -> {q, kpack, vpack, kscale, vscale}.

    x bf16 [N, d], w_qkv bf16 [d, 3d] row-major.  emit picks Q and K/V (default),
    Q only or K/V only.  Enqueued on the current stream."""
    lib = load()
    N, d = x.shape
    if out is None:
        out = alloc_store(N, d, ranges, device=x.device, emit=emit)
    arr, nr = _ranges_array(ranges)
    a = QkvArgs()
    a.n_tokens, a.d_model, a.n_heads = N, d, d // HEAD_DIM
    a.x, a.ldx = _dev_ptr(x, "x"), x.stride(0)
    a.w_qkv, a.ldw = _dev_ptr(w_qkv, "w_qkv"), w_qkv.stride(0)
    a.q_norm_w, a.k_norm_w = _dev_ptr(q_norm_w, "q_norm_w"), _dev_ptr(k_norm_w, "k_norm_w")
    a.eps = eps
    a.rope_cos, a.rope_sin = _dev_ptr(rope_cos, "rope_cos"), _dev_ptr(rope_sin, "rope_sin")
    a.ranges = ctypes.cast(arr, ctypes.POINTER(Range)) if arr is not None else None
    a.n_ranges, a.emit = nr, emit
    a.chunk_rows, a.min_tail = chunk_rows, min_tail
    if out.get("q") is not None:
        a.q, a.ldq = _dev_ptr(out["q"], "q"), out["q"].stride(0)
    a.kpack, a.vpack = _dev_ptr(out["kpack"], "kpack"), _dev_ptr(out["vpack"], "vpack")
    a.kscale, a.vscale = _dev_ptr(out["kscale"], "kscale"), _dev_ptr(out["vscale"], "vscale")
    for t, nm in ((x, "x"), (w_qkv, "w_qkv")):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1:
            raise ValueError("%s must be a row-major bf16 tensor" % nm)
    _check(lib.sqg_streamed_qkv_quant(ctypes.byref(a), _stream(x.device)))
    return out


_ODT = {torch.float32: SQG_F32, torch.bfloat16: SQG_BF16, torch.float16: SQG_F16}


def _attn_args(store: Dict, N: int, d: int, device, q_begin, q_end, kv_begin, kv_end, kv_block,
               accumulate, o, lse, o_dtype, softmax_scale, want_lse, qk_mode=SQG_QK_EXACT):
    H = d // HEAD_DIM
    if o is None:
        o = torch.empty((N, d), dtype=o_dtype, device=device)
    if lse is None and (want_lse or accumulate or kv_block > 0):
        lse = torch.empty((H, N), dtype=torch.float32, device=device)
    arr, nr = _ranges_array(store.get("ranges"))
    a = AttnArgs()
    a.n_tokens, a.d_model, a.n_heads = N, d, H
    a.kpack, a.vpack = _dev_ptr(store["kpack"], "kpack"), _dev_ptr(store["vpack"], "vpack")
    a.kscale, a.vscale = _dev_ptr(store["kscale"], "kscale"), _dev_ptr(store["vscale"], "vscale")
    a.ranges = ctypes.cast(arr, ctypes.POINTER(Range)) if arr is not None else None
    a.n_ranges = nr
    a.o_dtype = _ODT[o.dtype]
    a.q_begin, a.q_end, a.kv_begin, a.kv_end = q_begin, q_end, kv_begin, kv_end
    a.kv_block, a.accumulate, a.softmax_scale = kv_block, int(bool(accumulate)), softmax_scale
    a.o, a.ldo = _dev_ptr(o, "o"), o.stride(0)
    a.lse = _dev_ptr(lse, "lse")
    a.qk_mode, a.reserved = qk_mode, 0
    # keep the ranges array alive as long as the struct
    return a, arr, o, lse


def packed_kv_attention(store: Dict, q: Optional[torch.Tensor] = None, q_begin: int = 0,
                        q_end: int = 0, kv_begin: int = 0, kv_end: int = 0, kv_block: int = 0,
                        accumulate: bool = False, o: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, o_dtype=torch.float32,
                        softmax_scale: float = 0.0, want_lse: bool = True,
                        qk_mode: int = SQG_QK_EXACT):
    """packed_kv_attention(Q, Kpack, Vpack, scales) -> (O, lse).

    `store` is what streamed_qkv_quant returned (or the same keys).  O is [N, d]
    in the model basis; lse is fp32 [H, N] (natural log).  qk_mode SQG_QK_FP8 takes
    the scores on block-scaled fp8 operands (approximation tier)."""
    lib = load()
    q = store["q"] if q is None else q
    if q is None:
        raise ValueError("no Q: the store was built without one, pass q=")
    N, d = q.shape
    a, _keep, o, lse = _attn_args(store, N, d, q.device, q_begin, q_end, kv_begin, kv_end, kv_block,
                                  accumulate, o, lse, o_dtype, softmax_scale, want_lse, qk_mode)
    a.q, a.ldq = _dev_ptr(q, "q"), q.stride(0)
    _check(lib.sqg_packed_kv_attention(ctypes.byref(a), _stream(q.device)))
    return o, lse


def qrecompute_workspace_bytes(n_query_rows: int, d_model: int, q_chunk_rows: int = 0) -> int:
    """Bytes of Q workspace packed_kv_attention_qrecompute needs."""
    got = load().sqg_qrecompute_workspace_bytes(n_query_rows, q_chunk_rows, d_model)
    if got < 0:
        raise ValueError("invalid arguments to qrecompute_workspace_bytes")
    return got


def packed_kv_attention_qrecompute(store: Dict, x: torch.Tensor, w_qkv: torch.Tensor,
                                   q_norm_w: Optional[torch.Tensor] = None,
                                   rope_cos: Optional[torch.Tensor] = None,
                                   rope_sin: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                   q_chunk_rows: int = 0, workspace: Optional[torch.Tensor] = None,
                                   q_begin: int = 0, q_end: int = 0, kv_begin: int = 0,
                                   kv_end: int = 0, kv_block: int = 0, accumulate: bool = False,
                                   o: Optional[torch.Tensor] = None,
                                   lse: Optional[torch.Tensor] = None, o_dtype=torch.float32,
                                   softmax_scale: float = 0.0, want_lse: bool = True,
                                   qk_mode: int = SQG_QK_EXACT):
    """Attention over the packed store with Q recomputed from x chunk by chunk -> (O, lse).

    The store may come from streamed_qkv_quant(..., emit=SQG_EMIT_KV): no [N, d] Q
    is ever held.  Same results as packed_kv_attention on the Q a full call writes."""
    lib = load()
    N, d = x.shape
    for t, nm in ((x, "x"), (w_qkv, "w_qkv")):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1:
            raise ValueError("%s must be a row-major bf16 tensor" % nm)
    a, _keep, o, lse = _attn_args(store, N, d, x.device, q_begin, q_end, kv_begin, kv_end, kv_block,
                                  accumulate, o, lse, o_dtype, softmax_scale, want_lse, qk_mode)
    n_q = (q_end if q_end else N) - q_begin
    if workspace is None:
        need = qrecompute_workspace_bytes(max(n_q, 0), d, q_chunk_rows)
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    r = QRecomputeArgs()
    r.attn = a
    r.x, r.ldx = _dev_ptr(x, "x"), x.stride(0)
    r.w_qkv, r.ldw = _dev_ptr(w_qkv, "w_qkv"), w_qkv.stride(0)
    r.q_norm_w = _dev_ptr(q_norm_w, "q_norm_w")
    r.rope_cos, r.rope_sin = _dev_ptr(rope_cos, "rope_cos"), _dev_ptr(rope_sin, "rope_sin")
    r.eps, r.reserved, r.q_chunk_rows = eps, 0, q_chunk_rows
    r.workspace = _dev_ptr(workspace, "workspace")
    r.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.sqg_packed_kv_attention_qrecompute(ctypes.byref(r), _stream(x.device)))
    return o, lse


def noalloc_scratch_bytes() -> int:
    """Bytes of the device scratch the allocation-free Q-recompute entry point uses."""
    return load().sqg_noalloc_scratch_bytes()


def packed_kv_attention_qrecompute_noalloc(store: Dict, x: torch.Tensor, w_qkv: torch.Tensor,
                                           o: torch.Tensor, lse: Optional[torch.Tensor] = None,
                                           q_norm_w: Optional[torch.Tensor] = None,
                                           rope_cos: Optional[torch.Tensor] = None,
                                           rope_sin: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                           q_chunk_rows: int = 0, q_begin: int = 0, q_end: int = 0,
                                           kv_begin: int = 0, kv_end: int = 0, kv_block: int = 0,
                                           accumulate: bool = False, softmax_scale: float = 0.0,
                                           qk_mode: int = SQG_QK_EXACT):
    """packed_kv_attention_qrecompute whose Q workspace is the library's own device scratch:
    the call allocates nothing, so the caller passes the outputs (o, and lse when the call
    merges: accumulate or kv_block > 0).  Calls overlapping on one GPU race on the scratch."""
    lib = load()
    N, d = x.shape
    for t, nm in ((x, "x"), (w_qkv, "w_qkv")):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1:
            raise ValueError("%s must be a row-major bf16 tensor" % nm)
    if o is None or (lse is None and (accumulate or kv_block > 0)):
        raise ValueError("the allocation-free entry point takes its outputs from the caller (o, and "
                         "lse when the call merges: accumulate or kv_block > 0)")
    a, _keep, o, lse = _attn_args(store, N, d, x.device, q_begin, q_end, kv_begin, kv_end, kv_block,
                                  accumulate, o, lse, o.dtype, softmax_scale, False, qk_mode)
    r = QRecomputeArgs()
    r.attn = a
    r.x, r.ldx = _dev_ptr(x, "x"), x.stride(0)
    r.w_qkv, r.ldw = _dev_ptr(w_qkv, "w_qkv"), w_qkv.stride(0)
    r.q_norm_w = _dev_ptr(q_norm_w, "q_norm_w")
    r.rope_cos, r.rope_sin = _dev_ptr(rope_cos, "rope_cos"), _dev_ptr(rope_sin, "rope_sin")
    r.eps, r.reserved, r.q_chunk_rows = eps, 0, q_chunk_rows
    r.workspace, r.workspace_bytes = None, 0
    _check(lib.sqg_packed_kv_attention_qrecompute_noalloc(ctypes.byref(r), _stream(x.device)))
    return o, lse


def staged_sizes(n_tokens: int, d_model: int, block_rows: int, ranges=None):
    """(host pack bytes, host scale bytes, staging pack bytes, staging scale bytes), n_blocks."""
    lib = load()
    arr, nr = _ranges_array(ranges)
    sizes = (_c_i64 * 4)()
    nb = _c_i32(0)
    _check(lib.sqg_staged_sizes(n_tokens, d_model, d_model // HEAD_DIM, arr, nr, block_rows, sizes,
                                ctypes.byref(nb)))
    return tuple(sizes), nb.value


def alloc_staged(n_tokens: int, d_model: int, block_rows: int, ranges=None, device="cuda",
                 overlap: bool = True) -> Dict:
    """A host-staged K/V store: pinned host buffers for every block, two device staging
    block stores, the block plan, and (overlap) a stream of default priority on which the
    copies run beside the kernels."""
    (hp, hs, dp, ds), nb = staged_sizes(n_tokens, d_model, block_rows, ranges)
    pinned = lambda n: torch.empty((max(n, 16),), dtype=torch.uint8, pin_memory=True)  # noqa: E731
    dev = lambda n: torch.empty((max(n, 16),), dtype=torch.uint8, device=device)  # noqa: E731
    st = {"block_rows": block_rows, "n_blocks": nb, "ranges": list(ranges) if ranges else None,
          "n_tokens": n_tokens, "d_model": d_model,
          "host_kpack": pinned(hp), "host_vpack": pinned(hp), "host_kscale": pinned(hs),
          "host_vscale": pinned(hs),
          "dev_kpack": [dev(dp), dev(dp)], "dev_vpack": [dev(dp), dev(dp)],
          "dev_kscale": [dev(ds), dev(ds)], "dev_vscale": [dev(ds), dev(ds)],
          "copy_stream": torch.cuda.Stream(device=device) if overlap else None}
    return st


def _staged_struct(st: Dict) -> StagedKV:
    s = StagedKV()
    s.block_rows = st["block_rows"]
    for k in ("host_kpack", "host_vpack", "host_kscale", "host_vscale"):
        t = st[k]
        if not t.is_pinned():
            raise ValueError("%s must be pinned host memory" % k)
        setattr(s, k, t.data_ptr())
    for k in ("dev_kpack", "dev_vpack", "dev_kscale", "dev_vscale"):
        arr = getattr(s, k)
        for i in range(2):
            arr[i] = _dev_ptr(st[k][i], k)
    cs = st.get("copy_stream")
    s.copy_stream = cs.cuda_stream if cs is not None else None
    return s


def streamed_qkv_quant_staged(x: torch.Tensor, w_qkv: torch.Tensor, staged: Dict,
                              q: Optional[torch.Tensor] = None, emit: int = SQG_EMIT_QKV,
                              q_norm_w: Optional[torch.Tensor] = None,
                              k_norm_w: Optional[torch.Tensor] = None, eps: float = 1e-6,
                              rope_cos: Optional[torch.Tensor] = None,
                              rope_sin: Optional[torch.Tensor] = None):
    """streamed_qkv_quant with the packed K/V written block by block into the host store
    `staged` (alloc_staged).  Returns Q (None with emit SQG_EMIT_KV)."""
    lib = load()
    N, d = x.shape
    for t, nm in ((x, "x"), (w_qkv, "w_qkv")):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1:
            raise ValueError("%s must be a row-major bf16 tensor" % nm)
    if q is None and emit != SQG_EMIT_KV:
        q = torch.empty((N, d), dtype=torch.bfloat16, device=x.device)
    arr, nr = _ranges_array(staged.get("ranges"))
    a = QkvArgs()
    a.n_tokens, a.d_model, a.n_heads = N, d, d // HEAD_DIM
    a.x, a.ldx = _dev_ptr(x, "x"), x.stride(0)
    a.w_qkv, a.ldw = _dev_ptr(w_qkv, "w_qkv"), w_qkv.stride(0)
    a.q_norm_w, a.k_norm_w = _dev_ptr(q_norm_w, "q_norm_w"), _dev_ptr(k_norm_w, "k_norm_w")
    a.eps = eps
    a.rope_cos, a.rope_sin = _dev_ptr(rope_cos, "rope_cos"), _dev_ptr(rope_sin, "rope_sin")
    a.ranges = ctypes.cast(arr, ctypes.POINTER(Range)) if arr is not None else None
    a.n_ranges, a.emit = nr, emit
    if q is not None:
        a.q, a.ldq = _dev_ptr(q, "q"), q.stride(0)
    s = _staged_struct(staged)
    _check(lib.sqg_streamed_qkv_quant_staged(ctypes.byref(a), ctypes.byref(s), _stream(x.device)))
    return q


def packed_kv_attention_staged(staged: Dict, q: torch.Tensor, q_begin: int = 0, q_end: int = 0,
                               kv_begin: int = 0, kv_end: int = 0, accumulate: bool = False,
                               o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                               o_dtype=torch.float32, softmax_scale: float = 0.0,
                               want_lse: bool = True, qk_mode: int = SQG_QK_EXACT):
    """packed_kv_attention against the host-staged store: blocks are copied in one at a
    time and merged through the LSE.  -> (O, lse)."""
    lib = load()
    N, d = q.shape
    a, _keep, o, lse = _attn_args(staged_view(staged), N, d, q.device, q_begin, q_end, kv_begin,
                                  kv_end, 0, accumulate, o, lse, o_dtype, softmax_scale,
                                  want_lse or staged["n_blocks"] > 1, qk_mode)
    a.q, a.ldq = _dev_ptr(q, "q"), q.stride(0)
    s = _staged_struct(staged)
    _check(lib.sqg_packed_kv_attention_staged(ctypes.byref(a), ctypes.byref(s), _stream(q.device)))
    return o, lse


def staged_view(staged: Dict) -> Dict:
    """Store-shaped view for argument marshalling (the store pointers are ignored)."""
    return {"kpack": staged["dev_kpack"][0], "vpack": staged["dev_vpack"][0],
            "kscale": staged["dev_kscale"][0], "vscale": staged["dev_vscale"][0],
            "ranges": staged.get("ranges")}


def test_quant_pack_f32(r: torch.Tensor, fmt: int):
    """The kernels' quantise/pack step on fp32 rotated rows r [rows, 128] (GPU)."""
    lib = load()
    rows = r.shape[0]
    rb = 64 if fmt == SQG_INT4_ROT else 128
    codes = torch.empty((rows, rb), dtype=torch.uint8, device=r.device)
    scales = torch.empty((rows, 4), dtype=torch.float16, device=r.device)
    _check(lib.sqg_test_quant_pack_f32(_dev_ptr(r, "r"), rows, fmt, codes.data_ptr(),
                                       scales.data_ptr(), _stream(r.device)))
    return codes, scales


def test_fwht_f32(x: torch.Tensor, normalize: bool = False):
    """The kernels' 128-point Hadamard butterfly on fp32 rows x [rows, 128] (GPU)."""
    lib = load()
    out = torch.empty_like(x)
    _check(lib.sqg_test_fwht_f32(_dev_ptr(x, "x"), out.data_ptr(), x.shape[0], int(normalize),
                                 _stream(x.device)))
    return out
