"""Plain numpy oracle (float64) of the streamed QKV-quant + packed-K/V attention path.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py.  Shares no code with the HIP library.

Page names used in citations:
  [FR]  feature request "Streamed QKV Projection and Packed Low-Bit K/V Support for
        Extreme Long-Sequence Attention" (comfy-kitchen issue and its mirror)
  [VL]  "VRAM Lab" module page (ComfyUI-MAINodes vram_lab.py)
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "HEAD_DIM", "GROUP", "INT4", "INT8", "BF16", "FORMATS", "QMAX", "ROW_BYTES", "INT4_SCALE_BITS",
    "INT8_SCALE_FACTOR", "round_up_bits", "group_scales", "segment_parts", "head_formats", "gather_bf16_rows",
    "hadamard_pm1", "rotation_matrix",
    "f32_to_bf16_bits", "bf16_bits_to_f64", "f32_to_f16",
    "chunk_ranges", "range_segments", "token_formats",
    "project", "split_heads", "rms_norm", "rope_angles", "rope_split_half",
    "rotate", "quantize_groups", "pack_int4", "unpack_int4", "pack_codes", "unpack_codes",
    "dequantize", "qkv_quant_rows",
    "packed_layout", "gather_packed_rows", "decode_head",
    "softmax_attention", "online_merge", "attention_blockwise",
    "attention_rotated_rows", "attention_model_rows", "attention_rows_from_store",
    "working_set_bytes", "quality_vs_unquantised",
    "E4M3_MAX", "f32_to_e4m3", "e4m3_to_f64", "e8m0_exponent", "fp8_block_quantize",
    "fp8_block_dequantize", "attention_fp8qk_rotated",
]

HEAD_DIM = 128          # head dimension of every workload ([VL] docstring: 7168 = 56 x 128)
GROUP = 32              # quantisation group along head_dim (the workloads' "group 32")
INT4 = 0                # token-range formats ([FR] "Mixed precision for conditioning":
INT8 = 1                # conditioning ranges at BF16 or INT8, generated tokens at
BF16 = 2                # rotated INT4)
FORMATS = (INT4, INT8, BF16)
QMAX = {INT4: 7, INT8: 127}
ROW_BYTES = {INT4: HEAD_DIM // 2, INT8: HEAD_DIM, BF16: 2 * HEAD_DIM}
# INT4 group scales keep 8 significant bits (rounded up), so that code * scale is exact in
# fp16 (3 code bits + 8 scale bits = 11): the attention kernel decodes INT4 without rounding
INT4_SCALE_BITS = 8
# INT8 group scales follow [VL] kvi8r `_Int8KV.store`: the absmax times 1/127 enlarged by
# (1 + 2^-7) so that the fp16 rounding of the scale can never push a code past 127.  The
# page multiplies an fp32 tensor by a Python float, i.e. by that constant rounded to fp32.
INT8_SCALE_FACTOR = np.float32(1.0 / 127.0 * (1.0 + 2.0 ** -7))


# --------------------------------------------------------------------------- rotation
def hadamard_pm1(n: int = HEAD_DIM) -> np.ndarray:
    """Sylvester Hadamard matrix with +-1 entries, n a power of two.

    [VL] kvi8r section, `_hadamard`: start from the 1x1 matrix [1] and repeat the
    2x2 block doubling [[h, h], [h, -h]] until the size reaches n.  (The page then
    divides by sqrt(n); `rotation_matrix` does that.)"""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(n: int = HEAD_DIM) -> np.ndarray:
    """Orthonormal rotation H/sqrt(n) in float64 ([VL] kvi8r, `_hadamard`)."""
    return hadamard_pm1(n).astype(np.float64) / math.sqrt(n)


# --------------------------------------------------------------------------- rounding
def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_f16(x) -> np.ndarray:
    """fp32 -> fp16, IEEE round to nearest even (numpy's conversion)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------- chunk plan and range policy
def chunk_ranges(n: int, size: int, min_tail: int = 512) -> List[Tuple[int, int]]:
    """Row chunks of `size` rows over [0, n); a remainder shorter than `min_tail` rows
    joins the last full chunk.  size <= 0 or size >= n gives one chunk.

    The rule of the [VL] helpers section (`_ranges`), computed from the counts: n rows
    make n // size full chunks and a remainder of n % size rows; the remainder is a
    chunk of its own unless it is shorter than min_tail, in which case the last full
    chunk runs on to n."""
    if size <= 0 or size >= n:
        return [(0, n)]
    n_full, rest = divmod(n, size)
    n_chunks = n_full + (1 if rest >= max(min_tail, 1) else 0)
    starts = [size * i for i in range(n_chunks)]
    ends = starts[1:] + [n]
    return list(zip(starts, ends))


def range_segments(n: int, ranges: Optional[Sequence[Tuple[int, int, int]]],
                   boundary_multiple: int = 128,
                   n_heads: Optional[int] = None) -> List[Tuple[int, int, int]]:
    """Validate a token-range precision policy and return its segments.

    [FR] "Mixed precision for conditioning": different K/V precision per token
    range of the packed sequence (conditioning ranges at BF16 or 8 bits, generated
    tokens at rotated 4 bits).  [VL] segments are half-open (a, b) pairs in order.
    Reading: the ranges must be sorted, contiguous, non-empty and cover [0, n);
    every interior boundary is a multiple of `boundary_multiple` so that key tiles
    never straddle two formats.  No ranges means one INT4 range.

    A range may carry a fourth entry, a bit mask of heads whose K/V are kept at
    INT8 inside an INT4 range ([VL] kvmix section: a per-head 4/8-bit split, "hi"
    heads at 8 bits and the rest at 4).  Reading: the mask applies to INT4 ranges
    only; segments with a non-zero mask come back as (b, e, f, mask)."""
    if not ranges:
        return [(0, n, INT4)] if n > 0 else []
    segs = []
    pos = 0
    for r in ranges:
        b, e, f = int(r[0]), int(r[1]), int(r[2])
        m = int(r[3]) if len(r) > 3 else 0
        if f not in FORMATS:
            raise ValueError("unknown format %r" % f)
        if m < 0 or m >= 1 << 64:
            raise ValueError("head mask out of range")
        if m and f != INT4:
            raise ValueError("a head mask applies to INT4 ranges only")
        if n_heads is not None and m >> n_heads:
            raise ValueError("head mask names a head >= n_heads")
        if b != pos:
            raise ValueError("ranges must be contiguous from 0 (gap or overlap at %d)" % b)
        if e <= b:
            raise ValueError("empty or reversed range")
        if e < n and e % boundary_multiple:
            raise ValueError("interior boundary %d is not a multiple of %d" % (e, boundary_multiple))
        segs.append((b, e, f, m) if m else (b, e, f))
        pos = e
    if pos != n:
        raise ValueError("ranges end at %d, not at n=%d" % (pos, n))
    return segs


def segment_parts(seg) -> Tuple[int, int, int, int]:
    """(begin, end, format, INT8 head mask) of a segment given as 3 or 4 entries."""
    return int(seg[0]), int(seg[1]), int(seg[2]), int(seg[3]) if len(seg) > 3 else 0


def token_formats(n: int, segments: Sequence[Tuple[int, int, int]]) -> np.ndarray:
    """Format of each token's range (the per-head INT8 mask aside)."""
    fm = np.empty(n, dtype=np.int64)
    for seg in segments:
        b, e, f, _ = segment_parts(seg)
        fm[b:e] = f
    return fm


def head_formats(n: int, n_heads: int, segments) -> np.ndarray:
    """Format of each (token, head): the range's format, or INT8 for a head whose
    bit is set in an INT4 range's mask ([VL] kvmix)."""
    fm = np.empty((n, n_heads), dtype=np.int64)
    for seg in segments:
        b, e, f, m = segment_parts(seg)
        for h in range(n_heads):
            fm[b:e, h] = INT8 if (f == INT4 and (m >> h) & 1) else f
    return fm


# --------------------------------------------------------------------------- projection and per-head ops
def project(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """y = x . W in float64 (bf16 products are exact in fp64; the sum is not rounded
    to bf16, because the streamed projection never stores a bf16 QKV tensor:
    [FR] "Proposed backend capability")."""
    return bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(w_bits)


def split_heads(y: np.ndarray, n_heads: int):
    """Fused QKV columns are q | k | v, head h at columns [128h, 128h+128) of each
    ([VL] block section, `_phase1_kv`: split of the fused projection into three
    equal parts, each viewed as heads x 128)."""
    d = n_heads * HEAD_DIM
    assert y.shape[-1] == 3 * d
    r = y.shape[0]
    return (y[:, :d].reshape(r, n_heads, HEAD_DIM),
            y[:, d:2 * d].reshape(r, n_heads, HEAD_DIM),
            y[:, 2 * d:].reshape(r, n_heads, HEAD_DIM))


def rms_norm(u: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm over the last (head_dim) axis: u / sqrt(mean(u^2) + eps) * w.
    [VL] helpers section, `_norm_rope` (q_norm / k_norm before RoPE)."""
    u = np.asarray(u, dtype=np.float64)
    ms = np.mean(u * u, axis=-1, keepdims=True)
    return u / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_angles(positions: np.ndarray, theta: float = 10000.0, rot_dim: int = HEAD_DIM):
    """cos/sin of pos * theta^(-2i/rot_dim), i < rot_dim/2, in float64 [R, rot_dim/2].
    The workloads name a 1D RoPE with theta 10000 over token positions."""
    half = rot_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv = theta ** (-2.0 * i / rot_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope_split_half(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Split-half RoPE ([VL] helpers, `_norm_rope`: "split-half" rotation over
    rot_dim = 2 x table width): pairs (i, i + 64) rotate by the angle of row i:
    (a, b) -> (a cos - b sin, b cos + a sin).  u is [R, H, 128]; cos/sin [R, 64]."""
    half = cos.shape[-1]
    a = u[..., :half]
    b = u[..., half:2 * half]
    c = cos[:, None, :]
    s = sin[:, None, :]
    out = np.array(u, dtype=np.float64, copy=True)
    out[..., :half] = a * c - b * s
    out[..., half:2 * half] = b * c + a * s
    return out


def rotate(u: np.ndarray) -> np.ndarray:
    """r = u . H / sqrt(128) per 128-vector, computed in float64 and rounded once to
    fp32.  [FR] "Quality-oriented low-bit format" (orthogonal / Hadamard-style
    rotation before quantising); [VL] kvi8r `_Int8KV.store` (rotate by the
    orthonormal Hadamard along the head dim).  Reading: no bf16/fp16 rounding
    between the fp32 accumulator and the quantiser."""
    H = hadamard_pm1(HEAD_DIM).astype(np.float64)
    return ((np.asarray(u, dtype=np.float64) @ H) / math.sqrt(HEAD_DIM)).astype(np.float32)


# --------------------------------------------------------------------------- quantise / pack
def round_up_bits(t: np.ndarray, bits: int) -> np.ndarray:
    """Smallest fp32 value with at most `bits` significant bits that is >= t (t >= 0),
    found on the bit pattern: clear the low 24 - bits significand bits, carrying up
    when any of them was set."""
    u = np.ascontiguousarray(np.asarray(t, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    mask = (1 << (24 - bits)) - 1
    u = np.where(u & mask, (u | mask) + 1, u)
    return u.astype(np.uint32).view(np.float32)


def group_scales(a: np.ndarray, qmax: int) -> np.ndarray:
    """fp16 scale of each group from its fp32 absmax a.

    INT4 (qmax 7): t = a / 7 in IEEE fp32, rounded UP to INT4_SCALE_BITS significant
    bits, stored as fp16 (exact).  The round-up enlarges the step by less than 2^-7,
    the page's own enlargement factor for its int8 scale.  [VL] precision-probe
    section, `_fq_int4` (absmax / 7).
    INT8 (qmax 127): s = fp16_RNE(fp32(a * INT8_SCALE_FACTOR)), the scale rule of [VL]
    kvi8r `_Int8KV.store` (absmax * (1/127) * (1 + 2^-7) in fp32, then cast to the
    16-bit store dtype)."""
    a = np.asarray(a, dtype=np.float32)
    if qmax == QMAX[INT4]:
        return round_up_bits((a / np.float32(qmax)).astype(np.float32), INT4_SCALE_BITS).astype(np.float16)
    if qmax == QMAX[INT8]:
        return (a * INT8_SCALE_FACTOR).astype(np.float32).astype(np.float16)
    raise ValueError("qmax must be 7 (INT4) or 127 (INT8)")


def quantize_groups(r: np.ndarray, qmax: int):
    """Group quantisation of fp32 rotated vectors [..., 128] in groups of 32.

    For each group: a = max |r| (fp32); s = `group_scales(a, qmax)` (fp16); if s == 0
    every code is 0; otherwise c = clamp(rne(r / fp32(s)), -qmax, qmax) with
    round-half-to-even and IEEE fp32 division.
    [VL] precision-probe section, `_fq_int4` (absmax / 7, round, clamp) and kvi8r
    `_Int8KV.store` (scale from absmax / 127, torch.round, clamp to +-127); the
    workloads give group 32 along head_dim and fp16 scales.
    Returns (codes int8, scales fp16)."""
    r = np.ascontiguousarray(np.asarray(r, dtype=np.float32))
    lead = r.shape[:-1]
    g = r.reshape(lead + (HEAD_DIM // GROUP, GROUP))
    a = np.max(np.abs(g), axis=-1)                                  # fp32, exact
    s16 = group_scales(a, qmax)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    q = np.rint(g / safe[..., None])                                # fp32 division, RNE
    q = np.clip(q, -qmax, qmax)
    q = np.where((s32 == 0)[..., None], 0, q)
    return q.astype(np.int8).reshape(r.shape), s16


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, code 2i in bits 0-3 and code 2i+1 in bits 4-7."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_codes(codes: np.ndarray, fmt: int) -> np.ndarray:
    if fmt == INT4:
        return pack_int4(codes)
    return np.asarray(codes, dtype=np.int8).view(np.uint8)


def unpack_codes(packed: np.ndarray, fmt: int) -> np.ndarray:
    if fmt == INT4:
        return unpack_int4(packed)
    return np.asarray(packed, dtype=np.uint8).view(np.int8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """k_r = code * scale per group, exact in float64 (rotated basis)."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    lead = c.shape[:-1]
    return (c.reshape(lead + (HEAD_DIM // GROUP, GROUP)) * s[..., None]).reshape(c.shape)


# --------------------------------------------------------------------------- the streamed QKV-quant step for chosen rows
def qkv_quant_rows(x_bits_rows: np.ndarray, w_bits: np.ndarray, n_heads: int,
                   positions: np.ndarray, fmts: np.ndarray,
                   q_norm_w: Optional[np.ndarray] = None, k_norm_w: Optional[np.ndarray] = None,
                   eps: float = 1e-6, rope_theta: Optional[float] = None) -> Dict[str, np.ndarray]:
    """What the streamed QKV-quant computes for the given token rows.

    [FR] "Proposed backend capability": hidden states go through a tiled QKV
    projection; Q is kept in bf16; K and V are rotated, quantised and packed.
    [VL] block section, `_phase1_kv`: projection -> split -> (RMSNorm + RoPE of q
    and k) -> store.  Row r uses token position positions[r] for RoPE and format
    fmts[r] (INT4, INT8 or BF16; or fmts[r, h] per head) for its K/V.

    Returns q_bits [R, d] uint16 (bf16, model basis), k_codes / v_codes
    [R, H, 128] int8, k_scales / v_scales [R, H, 4] fp16 (zero where the format
    is BF16) and k_bf16 / v_bf16 [R, H, 128] uint16: the rotated fp32 values
    rounded to bf16 where the format is BF16 (zero elsewhere).  Reading of [FR]
    "Mixed precision for conditioning": a BF16 range keeps K/V at 16 bits in the
    same rotated basis as the low-bit ranges (the rotation is orthogonal, so this
    keeps what bf16 K/V in the model basis keep: 8 significant bits)."""
    y = project(x_bits_rows, w_bits)
    q, k, v = split_heads(y, n_heads)
    if q_norm_w is not None:
        q = rms_norm(q, q_norm_w, eps)
        k = rms_norm(k, k_norm_w, eps)
    if rope_theta is not None:
        cos, sin = rope_angles(positions, rope_theta)
        q = rope_split_half(q, cos, sin)
        k = rope_split_half(k, cos, sin)
    r_rows = q.shape[0]
    q_bits = f32_to_bf16_bits(q.astype(np.float32)).reshape(r_rows, n_heads * HEAD_DIM)
    kr = rotate(k)
    vr = rotate(v)
    out = {"q_bits": q_bits}
    fm = np.asarray(fmts, dtype=np.int64)
    if fm.ndim == 1:
        fm = np.repeat(fm[:, None], n_heads, axis=1)
    for name, rr in (("k", kr), ("v", vr)):
        codes = np.zeros(rr.shape, dtype=np.int8)
        scales = np.zeros(rr.shape[:-1] + (HEAD_DIM // GROUP,), dtype=np.float16)
        bf = np.zeros(rr.shape, dtype=np.uint16)
        for f in (INT4, INT8):
            sel = fm == f
            if np.any(sel):
                c, s = quantize_groups(rr[sel], QMAX[f])
                codes[sel] = c
                scales[sel] = s
        sel = fm == BF16
        if np.any(sel):
            bf[sel] = f32_to_bf16_bits(rr[sel])
        out[name + "_codes"] = codes
        out[name + "_scales"] = scales
        out[name + "_bf16"] = bf
    out["k_rot_f32"] = kr
    out["v_rot_f32"] = vr
    return out


# --------------------------------------------------------------------------- packed store layout
def packed_layout(n: int, n_heads: int, segments: Sequence[Tuple[int, int, int]]):
    """Byte layout of a packed K (or V) store.

    Reading of [FR] "Proposed backend capability" / "Quality-oriented low-bit
    format" (fixed-width packed tiles a kernel can address directly) and of [VL]
    kvi8r (head-major [heads, tokens, head_dim] store): each segment [b, e) holds
    its rows head-major, head after head; head h of the segment uses format
    fmt(h) (the segment's, or INT8 for a masked head of an INT4 segment) and
    starts at offset_s + (e - b) * (sum of row_bytes(fmt(h')) over h' < h); row
    (h, t) sits at that start + (t - b) * row_bytes(fmt(h)).  Segments follow each
    other.  Scales are separate, fp16 [H, N, 4] over the whole sequence (zero and
    unused for BF16 rows)."""
    out = []
    off = 0
    for seg in segments:
        b, e, f, m = segment_parts(seg)
        hf = [INT8 if (f == INT4 and (m >> h) & 1) else f for h in range(n_heads)]
        hrb = [ROW_BYTES[x] for x in hf]
        hoff = []
        o = off
        for h in range(n_heads):
            hoff.append(o)
            o += (e - b) * hrb[h]
        out.append({"begin": b, "end": e, "fmt": f, "int8_heads": m, "offset": off,
                    "row_bytes": ROW_BYTES[f], "head_fmt": hf, "head_row_bytes": hrb,
                    "head_offset": hoff})
        off = o
    return out, off


def gather_packed_rows(packed: np.ndarray, scales: np.ndarray, layout, n_heads: int,
                       rows: np.ndarray):
    """Codes [R, H, 128] int8 and scales [R, H, 4] fp16 of the given token rows
    (codes stay zero for BF16 rows: see gather_bf16_rows)."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    sc = np.asarray(scales).reshape(n_heads, -1, HEAD_DIM // GROUP)
    rows = np.asarray(rows, dtype=np.int64)
    codes = np.zeros((rows.size, n_heads, HEAD_DIM), dtype=np.int8)
    for seg in layout:
        sel = np.nonzero((rows >= seg["begin"]) & (rows < seg["end"]))[0]
        if sel.size == 0:
            continue
        for h in range(n_heads):
            f, rb = seg["head_fmt"][h], seg["head_row_bytes"][h]
            if f == BF16:
                continue
            start = seg["head_offset"][h] + (rows[sel] - seg["begin"]) * rb
            idx = start[:, None] + np.arange(rb)[None, :]
            codes[sel, h] = unpack_codes(packed[idx], f)
    return codes, np.ascontiguousarray(sc[:, rows, :].transpose(1, 0, 2))


def gather_bf16_rows(packed: np.ndarray, layout, n_heads: int, rows: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [R, H, 128] uint16 of the given rows where the format is
    BF16 (zero elsewhere); each row is 128 little-endian bf16 values."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, n_heads, HEAD_DIM), dtype=np.uint16)
    for seg in layout:
        sel = np.nonzero((rows >= seg["begin"]) & (rows < seg["end"]))[0]
        if sel.size == 0:
            continue
        for h in range(n_heads):
            if seg["head_fmt"][h] != BF16:
                continue
            start = seg["head_offset"][h] + (rows[sel] - seg["begin"]) * ROW_BYTES[BF16]
            idx = start[:, None] + np.arange(ROW_BYTES[BF16])[None, :]
            out[sel, h] = np.ascontiguousarray(packed[idx]).view(np.uint16)
    return out


def decode_head(packed: np.ndarray, scales: np.ndarray, layout, n_heads: int, head: int,
                begin: int, end: int) -> np.ndarray:
    """Dequantised rotated-basis vectors of one head for tokens [begin, end), float64."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    sc = np.asarray(scales).reshape(n_heads, -1, HEAD_DIM // GROUP)
    out = np.empty((end - begin, HEAD_DIM), dtype=np.float64)
    for seg in layout:
        lo, hi = max(begin, seg["begin"]), min(end, seg["end"])
        if lo >= hi:
            continue
        f, rb = seg["head_fmt"][head], seg["head_row_bytes"][head]
        start = seg["head_offset"][head] + (lo - seg["begin"]) * rb
        blob = np.ascontiguousarray(packed[start:start + (hi - lo) * rb].reshape(hi - lo, rb))
        if f == BF16:
            out[lo - begin:hi - begin] = bf16_bits_to_f64(blob.view(np.uint16))
        else:
            out[lo - begin:hi - begin] = dequantize(unpack_codes(blob, f), sc[head, lo:hi])
    return out


# --------------------------------------------------------------------------- attention
def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Exact single-pass softmax attention in float64 for one head.

    q [R, D], k [S, D], v [S, D] -> o [R, D], lse [R] (natural log).  Scores
    s = scale * q.k; the row maximum is subtracted before exp; lse = m + ln sum e^(s-m).
    Non-causal, no mask ([VL] helpers, `_blockwise_attention`: flash call without
    mask or causality; softmax scale head_dim^-1/2)."""
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=-1, keepdims=True)
    o = (p @ np.asarray(v, np.float64)) / l
    return o, (m + np.log(l))[:, 0]


def online_merge(o_acc, lse_acc, o, lse):
    """Online-softmax merge of a partial (o, lse) into (o_acc, lse_acc).

    [VL] kvi8r section, `_online_combine`: lse' = logaddexp(lse_acc, lse);
    o' = o_acc * exp(lse_acc - lse') + o * exp(lse - lse').  A None accumulator
    takes the partial as is."""
    if o_acc is None:
        return np.array(o, dtype=np.float64, copy=True), np.array(lse, dtype=np.float64, copy=True)
    new = np.logaddexp(lse_acc, lse)
    return (o_acc * np.exp(lse_acc - new)[:, None] + o * np.exp(lse - new)[:, None]), new


def attention_blockwise(q, k, v, scale, block: int, min_tail: int = 512):
    """Attention over K/V blocks `chunk_ranges(S, block, min_tail)` merged with
    `online_merge` ([VL] helpers, `_blockwise_attention`; kvi8r
    `_blockwise_attention_q`)."""
    o_acc = lse_acc = None
    for a, b in chunk_ranges(k.shape[0], block, min_tail):
        o, lse = softmax_attention(q, k[a:b], v[a:b], scale)
        o_acc, lse_acc = online_merge(o_acc, lse_acc, o, lse)
    return o_acc, lse_acc


def attention_rotated_rows(q_bits_head: np.ndarray, k_rot: np.ndarray, v_rot: np.ndarray,
                           scale: float, kv_block: int = 0):
    """Attention of bf16 query rows (model basis) against dequantised K/V kept in
    the rotated basis.

    [VL] kvi8r `_Int8KV` docstring and `_blockwise_attention_q`: since H/sqrt(n)
    is orthogonal, q.k = (qH).(kH) and P.V = (P.(VH)).H^T; so the queries are
    rotated once, attention runs against the rotated store, and the output is
    rotated back once (H is symmetric, so H^T = H).  kv_block > 0 merges KV blocks
    by log-sum-exp.  Returns o [R, 128] (model basis) and lse [R]."""
    R = rotation_matrix(HEAD_DIM)
    qr = bf16_bits_to_f64(q_bits_head) @ R
    if kv_block and kv_block > 0:
        o_r, lse = attention_blockwise(qr, k_rot, v_rot, scale, kv_block)
    else:
        o_r, lse = softmax_attention(qr, k_rot, v_rot, scale)
    return o_r @ R.T, lse


def attention_model_rows(q_bits_head: np.ndarray, k_rot: np.ndarray, v_rot: np.ndarray,
                         scale: float):
    """The same attention in the model basis: the dequantised K and V are rotated
    back first (k = k_r . (H/sqrt(128))^T) and the queries are used as stored."""
    R = rotation_matrix(HEAD_DIM)
    return softmax_attention(bf16_bits_to_f64(q_bits_head), k_rot @ R.T, v_rot @ R.T, scale)


def attention_rows_from_store(q_bits: np.ndarray, rows: np.ndarray, kpack, vpack, kscale,
                              vscale, layout, n_heads: int, n_tokens: int,
                              scale: Optional[float] = None, kv_block: int = 0,
                              kv_begin: int = 0, kv_end: Optional[int] = None,
                              heads: Optional[Sequence[int]] = None, qk: str = "exact"):
    """Packed-K/V attention for the query rows `rows` against keys [kv_begin, kv_end).

    q_bits is [R, d] bf16 bits of those rows (model basis).  [FR] "Dense fallback
    is important": keys are decoded from the packed store (here: head by head, in
    float64), never from a bf16 K/V.  qk = "fp8" takes the scores on block-scaled
    fp8 operands (`attention_fp8qk_rotated`).  Returns o [R, d] and lse [H, R]."""
    if scale is None:
        scale = HEAD_DIM ** -0.5
    if kv_end is None:
        kv_end = n_tokens
    heads = range(n_heads) if heads is None else heads
    Rn = len(rows)
    o = np.zeros((Rn, n_heads * HEAD_DIM), dtype=np.float64)
    lse = np.zeros((n_heads, Rn), dtype=np.float64)
    for h in heads:
        kr = decode_head(kpack, kscale, layout, n_heads, h, kv_begin, kv_end)
        vr = decode_head(vpack, vscale, layout, n_heads, h, kv_begin, kv_end)
        qh = q_bits[:, h * HEAD_DIM:(h + 1) * HEAD_DIM]
        if qk == "fp8":
            R = rotation_matrix(HEAD_DIM)
            qr = (bf16_bits_to_f64(qh) @ R).astype(np.float32)
            o_r, lh = attention_fp8qk_rotated(qr, kr, vr, scale, kv_block)
            oh = o_r @ R.T
        else:
            oh, lh = attention_rotated_rows(qh, kr, vr, scale, kv_block)
        o[:, h * HEAD_DIM:(h + 1) * HEAD_DIM] = oh
        lse[h] = lh
    return o, lse


# --------------------------------------------------------------------------- low-precision QK^T tier
E4M3_MAX = 448.0


def f32_to_e4m3(x) -> np.ndarray:
    """OCP FP8 E4M3 code of each value: sign bit, 4-bit exponent with bias 7, 3-bit
    mantissa, subnormals below 2^-6 in steps of 2^-9, no infinities, largest finite
    value 448 (code 0x7e); round to nearest, ties to even; magnitudes above 448
    saturate to 448.  Inputs are finite fp32 values (exact in float64)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    f, E = np.frexp(a)                        # a = f * 2^E, f in [0.5, 1)
    e = np.maximum(np.where(a > 0, E - 1, -6), -6)   # binade of a (subnormals share -6)
    step = np.ldexp(1.0, e - 3)              # spacing of the 3-bit mantissa
    v = np.minimum(np.rint(a / step) * step, E4M3_MAX)   # rint: half to even
    f2, E2 = np.frexp(v)
    ev = E2 - 1
    normal = v >= 2.0 ** -6
    exp_field = np.where(normal, ev + 7, 0)
    mant = np.where(normal, np.rint((v / np.ldexp(1.0, ev) - 1.0) * 8), np.rint(v / 2.0 ** -9))
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def e4m3_to_f64(codes) -> np.ndarray:
    """Value of each OCP FP8 E4M3 code (NaN for 0x7f and 0xff)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e8m0_exponent(amax) -> np.ndarray:
    """Power-of-two block scale exponent: the smallest e with amax <= 448 * 2^e, so the
    block's largest magnitude lands in (224, 448] after division by 2^e; clamped to
    [-127, 127] (the E8M0 range); e = -127 for an all-zero block."""
    a = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(a)                       # a = f * 2^E; 448 = 0.875 * 2^9
    e = np.where(f <= 0.875, E - 9, E - 8)
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def fp8_block_quantize(r: np.ndarray):
    """MX-style fp8 of rotated vectors [..., 128]: per group of 32 values an E8M0
    exponent e (`e8m0_exponent` of the group's max |r|) and the E4M3 codes of r / 2^e.
    Returns (codes uint8 [..., 128], exponents int64 [..., 4])."""
    r = np.asarray(r, dtype=np.float64)
    g = r.reshape(r.shape[:-1] + (HEAD_DIM // GROUP, GROUP))
    e = e8m0_exponent(np.max(np.abs(g), axis=-1))
    codes = f32_to_e4m3(g / np.ldexp(1.0, e)[..., None])
    return codes.reshape(r.shape), e


def fp8_block_dequantize(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    c = e4m3_to_f64(codes)
    g = c.reshape(c.shape[:-1] + (HEAD_DIM // GROUP, GROUP))
    return (g * np.ldexp(1.0, np.asarray(exps))[..., None]).reshape(c.shape)


def attention_fp8qk_rotated(q_rot: np.ndarray, k_rot: np.ndarray, v_rot: np.ndarray,
                            scale: float, kv_block: int = 0):
    """Attention with the scores taken on block-scaled fp8 operands, in the rotated
    basis.  Reading of [VL] kvi8s section (an approximation tier: Hadamard-rotated Q
    and K, QK^T on low-precision tensor cores straight from the store, no dequantised
    K) carried to the MX formats of the MFMA unit: the rotated query (fp32) and the
    decoded rotated keys are each quantised by `fp8_block_quantize` (one E8M0
    exponent per group of 32 dims, E4M3 values); the scores are the exact dot
    products of the dequantised operands; softmax, P.V with the decoded V, and the
    KV-block merge are as in the exact tier.  Returns o [R, 128] in the rotated basis
    and lse [R]."""
    qd = fp8_block_dequantize(*fp8_block_quantize(np.asarray(q_rot, dtype=np.float32)))
    kd = fp8_block_dequantize(*fp8_block_quantize(k_rot))
    if kv_block and kv_block > 0:
        return attention_blockwise(qd, kd, v_rot, scale, kv_block)
    return softmax_attention(qd, kd, v_rot, scale)


# --------------------------------------------------------------------------- memory
def working_set_bytes(n: int, d_model: int, segments: Sequence[Tuple[int, int, int]]):
    """Closed-form bytes of the fused bf16 QKV versus Q bf16 + packed K/V + scales.
    [FR] "Potential reduction": Q kept at bf16, K and V at 4 bits, plus metadata."""
    H = d_model // HEAD_DIM
    _, codes = packed_layout(n, H, segments)
    scales = n * H * (HEAD_DIM // GROUP) * 2
    q = 2 * n * d_model
    return {"bf16_qkv": 6 * n * d_model, "q": q, "k_codes": codes, "v_codes": codes,
            "k_scales": scales, "v_scales": scales,
            "packed_total": q + 2 * codes + 2 * scales}


def quality_vs_unquantised(q_bits_head, k_model, v_model, k_rot_hat, v_rot_hat):
    """Relative L2 error of attention over dequantised K/V against the same
    attention over the unquantised K/V (information only; parity unpinned: the
    pages give no value for this format on these inputs)."""
    scale = HEAD_DIM ** -0.5
    o_ref, _ = softmax_attention(bf16_bits_to_f64(q_bits_head), k_model, v_model, scale)
    o_q, _ = attention_rotated_rows(q_bits_head, k_rot_hat, v_rot_hat, scale)
    return float(np.linalg.norm(o_q - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
