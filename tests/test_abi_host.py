"""CPU tests of the C ABI: the library loads, exports every declared symbol, and its
host-side logic (chunk plan, range policy, layout, RoPE table, argument checks)
agrees with the oracle.  No kernel is launched: every call here either is host-only
or fails validation before the first launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import streamed_qkv_gemm_amd as sqg
from streamed_qkv_gemm_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sqg.h")

FAKE = 0x7f0000000000  # 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"SQG_API\s+[\w\s\*]+?\b(sqg_\w+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    lib = sqg.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sqg.version() == 140


def test_struct_sizes_match_binding():
    lib = sqg.load()
    assert lib.sqg_struct_size(0) == ctypes.sizeof(B.Range)
    assert lib.sqg_struct_size(1) == ctypes.sizeof(B.Layout)
    assert lib.sqg_struct_size(2) == ctypes.sizeof(B.QkvArgs)
    assert lib.sqg_struct_size(3) == ctypes.sizeof(B.AttnArgs)
    assert lib.sqg_struct_size(4) == ctypes.sizeof(B.QRecomputeArgs)
    assert lib.sqg_struct_size(5) == ctypes.sizeof(B.StagedKV)
    assert lib.sqg_struct_size(9) == -1


def test_status_strings():
    lib = sqg.load()
    assert lib.sqg_status_string(0) == b"ok"
    assert lib.sqg_status_string(-3).startswith(b"misaligned")


@pytest.mark.parametrize("n,size,tail", [(152263, 8192, 512), (16484, 8192, 512), (65536, 16384, 512),
                                         (217088, 16384, 512), (1024, 0, 512), (100, 100, 512),
                                         (0, 64, 512), (5000, 128, 0), (16896, 8192, 600)])
def test_chunk_plan_matches_oracle(n, size, tail):
    assert sqg.chunk_ranges(n, size, tail) == oracle.chunk_ranges(n, size, tail)


def test_chunk_plan_random_matches_oracle():
    rng = np.random.default_rng(1)
    for _ in range(200):
        n, size, tail = (int(v) for v in (rng.integers(0, 40000), rng.integers(-5, 9000),
                                          rng.integers(0, 1000)))
        assert sqg.chunk_ranges(n, size, tail) == oracle.chunk_ranges(n, size, tail)


@pytest.mark.parametrize("n,d,ranges", [
    (65536, 7168, [(0, 512, 1), (512, 8704, 1), (8704, 65536, 0)]),
    (152263, 7168, None),
    (1000, 512, [(0, 128, 1), (128, 1000, 0)]),
    (777, 256, [(0, 256, 0), (256, 384, 1), (384, 777, 0)]),
    (2000, 768, [(0, 256, 2), (256, 640, 1), (640, 1536, 0, 0b100101), (1536, 2000, 2)]),
    (65536, 7168, [(0, 512, 2), (512, 8704, 1), (8704, 65536, 0, (1 << 56) - 1 - (1 << 7))]),
])
def test_layout_matches_oracle(n, d, ranges):
    L = sqg.kv_layout(n, d, ranges)
    segs = oracle.range_segments(n, ranges)
    H = d // 128
    ol, total = oracle.packed_layout(n, H, segs)
    assert L["pack_bytes"] == total
    keys = ("begin", "end", "fmt", "int8_heads", "offset", "row_bytes")
    assert [tuple(s[k] for k in keys) for s in L["segments"]] == [tuple(s[k] for k in keys) for s in ol]
    for seg in ol:
        for h in sorted({0, 1, H // 2, H - 1}):
            for t in (seg["begin"], seg["end"] - 1):
                want = seg["head_offset"][h] + (t - seg["begin"]) * seg["head_row_bytes"][h]
                assert sqg.kv_row_offset(L, h, t) == want
    ws = oracle.working_set_bytes(n, d, segs)
    assert L["q_bytes"] == ws["q"] and L["bf16_qkv_bytes"] == ws["bf16_qkv"]
    assert L["scale_bytes"] == ws["k_scales"]


@pytest.mark.parametrize("ranges", [
    [(0, 512, 1), (640, 1024, 0)],
    [(0, 640, 1), (512, 1024, 0)],
    [(0, 500, 1), (500, 1024, 0)],
    [(0, 512, 7), (512, 1024, 0)],
    [(0, 512, 1), (512, 1000, 0)],
    [(128, 1024, 0)],
    [(0, 512, 3), (512, 1024, 0)],                # unknown format
    [(0, 512, 1, 1), (512, 1024, 0)],             # head mask on an INT8 range
    [(0, 512, 2, 4), (512, 1024, 0)],             # head mask on a BF16 range
    [(0, 512, 0, 1 << 4), (512, 1024, 0)],        # head 4 of 4
])
def test_layout_rejects_bad_policies_like_the_oracle(ranges):
    with pytest.raises(ValueError):
        oracle.range_segments(1024, ranges, n_heads=4)
    with pytest.raises(sqg.SqgError) as e:
        sqg.kv_layout(1024, 512, ranges)
    assert e.value.status == -1
    assert sqg.load().sqg_last_error()


def test_layout_too_many_segments():
    ranges = [(128 * i, 128 * (i + 1), i % 2) for i in range(17)]
    with pytest.raises(sqg.SqgError):
        sqg.kv_layout(128 * 17, 512, ranges)


def test_rope_table_matches_oracle_angles():
    lib = sqg.load()
    n = 300
    for pos0 in (0, 216788):
        cos = np.zeros((n, 64), np.float32)
        sin = np.zeros((n, 64), np.float32)
        assert lib.sqg_rope_table(pos0, n, 10000.0, cos.ctypes.data, sin.ctypes.data) == 0
        c, s = oracle.rope_angles(np.arange(pos0, pos0 + n))
        assert np.max(np.abs(cos - c)) <= 6e-8 and np.max(np.abs(sin - s)) <= 6e-8


# ----------------------------------------------------------------------------- argument checks
def qkv_args(**kw):
    a = B.QkvArgs()
    a.n_tokens, a.d_model, a.n_heads = 1024, 512, 4
    a.x, a.ldx, a.w_qkv, a.ldw = FAKE, 512, FAKE, 1536
    a.q, a.ldq, a.kpack, a.vpack, a.kscale, a.vscale = FAKE, 512, FAKE, FAKE, FAKE, FAKE
    a.eps, a.chunk_rows, a.min_tail = 1e-6, 0, 512
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def attn_args(**kw):
    a = B.AttnArgs()
    a.n_tokens, a.d_model, a.n_heads = 1024, 512, 4
    a.q, a.ldq, a.kpack, a.vpack, a.kscale, a.vscale = FAKE, 512, FAKE, FAKE, FAKE, FAKE
    a.o, a.ldo, a.lse = FAKE, 512, FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=384, n_heads=3), -2),            # d not a multiple of 256
    (dict(d_model=512, n_heads=3), -1),            # d != 128 H
    (dict(n_tokens=-1), -1),
    (dict(x=FAKE + 8), -3),                        # misaligned pointer
    (dict(ldx=500), -1),                           # stride shorter than a row
    (dict(ldq=516), -3),                           # stride not a multiple of 8
    (dict(chunk_rows=100), -1),                    # chunk not a multiple of 128
    (dict(chunk_rows=-128), -1),
    (dict(x=None), -1),
    (dict(q_norm_w=FAKE), -1),                     # q norm without k norm
    (dict(rope_cos=FAKE), -1),                     # cos without sin
    (dict(emit=3), -1),                            # unknown emit mode
    (dict(emit=1, q=None), -1),                    # Q only needs q
    (dict(emit=2, kscale=None), -1),               # K/V only needs the store
])
def test_qkv_argument_errors(kw, status):
    lib = sqg.load()
    a = qkv_args(**kw)
    assert lib.sqg_streamed_qkv_quant(ctypes.byref(a), None) == status
    assert len(lib.sqg_last_error()) > 0


def test_qkv_emit_modes_drop_the_unused_pointers():
    """Q only needs no store pointers, K/V only needs no q: a later check fires instead."""
    lib = sqg.load()
    a = qkv_args(emit=1, kpack=None, vpack=None, kscale=None, vscale=None, ldx=500)
    assert lib.sqg_streamed_qkv_quant(ctypes.byref(a), None) == -1
    assert b"row strides" in lib.sqg_last_error()
    a = qkv_args(emit=2, q=None, ldq=0, x=FAKE + 8)
    assert lib.sqg_streamed_qkv_quant(ctypes.byref(a), None) == -3
    assert b"aligned" in lib.sqg_last_error()


def qrec_args(**kw):
    r = B.QRecomputeArgs()
    r.attn = attn_args(q=None, ldq=0)
    r.x, r.ldx, r.w_qkv, r.ldw = FAKE, 512, FAKE, 1536
    r.eps, r.q_chunk_rows = 1e-6, 0
    r.workspace, r.workspace_bytes = FAKE, 1024 * 512 * 2
    for k, v in kw.items():
        if k.startswith("attn_"):
            setattr(r.attn, k[5:], v)
        else:
            setattr(r, k, v)
    return r


@pytest.mark.parametrize("kw,status,msg", [
    (dict(workspace_bytes=1024 * 512 * 2 - 2), -4, b"workspace"),
    (dict(q_chunk_rows=256, workspace_bytes=256 * 512 * 2 - 2), -4, b"workspace"),
    (dict(workspace=None), -1, b"NULL"),
    (dict(x=None), -1, b"NULL"),
    (dict(reserved=1), -1, b"reserved"),
    (dict(q_chunk_rows=100), -1, b"q_chunk_rows"),
    (dict(q_chunk_rows=-128), -1, b"q_chunk_rows"),
    (dict(rope_cos=FAKE), -1, b"rope_sin"),
    (dict(ldx=500), -1, b"row strides"),
    (dict(ldw=1000), -1, b"row strides"),
    (dict(x=FAKE + 8), -3, b"aligned"),
    (dict(workspace=FAKE + 8), -3, b"aligned"),
    (dict(attn_d_model=384, attn_n_heads=3), -2, b"multiple of 256"),
    (dict(attn_kv_begin=64), -1, b"kv_begin"),
    (dict(attn_kpack=None), -1, b"NULL"),
    (dict(attn_accumulate=1, attn_lse=None), -1, b"lse"),
])
def test_qrecompute_argument_errors(kw, status, msg):
    lib = sqg.load()
    r = qrec_args(**kw)
    assert lib.sqg_packed_kv_attention_qrecompute(ctypes.byref(r), None) == status
    assert msg in lib.sqg_last_error()


def test_qrecompute_empty_query_range_is_a_noop():
    lib = sqg.load()
    r = qrec_args(attn_q_begin=300, attn_q_end=300, workspace=None, workspace_bytes=0)
    assert lib.sqg_packed_kv_attention_qrecompute(ctypes.byref(r), None) == 0


@pytest.mark.parametrize("n,chunk,d,want", [
    (1000, 0, 512, 1000 * 1024),                   # one chunk
    (300000, 0, 512, 131072 * 1024),               # 4 heads: default chunk 256 * 512 rows
    (131584, 0, 512, 131072 * 1024),               # 512-row tail stays a chunk of its own...
    (131583, 0, 512, 131583 * 1024),               # ...511 rows join the chunk before it
    (217088, 0, 7168, 16384 * 14336),              # 56 heads: default chunk 16384 rows
    (1000, 256, 384, 488 * 768),                   # 232-row tail joins the chunk at 512
    (1200, 512, 384, 688 * 768),                   # 176-row tail joins the second chunk
    (0, 0, 512, 0),
    (-1, 0, 512, -1),
    (1000, 100, 512, -1),
    (1000, 0, 0, -1),
])
def test_qrecompute_workspace_bytes(n, chunk, d, want):
    assert sqg.load().sqg_qrecompute_workspace_bytes(n, chunk, d) == want


def test_qkv_bad_policy_rejected():
    lib = sqg.load()
    arr = (B.Range * 2)()
    arr[0].begin, arr[0].end, arr[0].fmt = 0, 500, 1
    arr[1].begin, arr[1].end, arr[1].fmt = 500, 1024, 0
    a = qkv_args()
    a.ranges, a.n_ranges = ctypes.cast(arr, ctypes.POINTER(B.Range)), 2
    assert lib.sqg_streamed_qkv_quant(ctypes.byref(a), None) == -1
    assert b"multiple of 128" in lib.sqg_last_error()


def test_zero_tokens_is_a_noop():
    lib = sqg.load()
    a = qkv_args(n_tokens=0, x=None, w_qkv=None, q=None, kpack=None, vpack=None, kscale=None,
                 vscale=None)
    assert lib.sqg_streamed_qkv_quant(ctypes.byref(a), None) == 0
    b = attn_args(n_tokens=0)
    assert lib.sqg_packed_kv_attention(ctypes.byref(b), None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(o_dtype=5), -1),
    (dict(q_begin=10, q_end=5), -1),
    (dict(q_end=2000), -1),
    (dict(kv_begin=64), -1),                       # kv_begin not a multiple of 128
    (dict(kv_begin=512, kv_end=512), -1),          # empty key range
    (dict(kv_block=100), -1),
    (dict(accumulate=1, lse=None), -1),
    (dict(kv_block=256, o_dtype=1), -1),           # merging needs fp32 O
    (dict(softmax_scale=-1.0), -1),
    (dict(o=FAKE + 4), -3),
    (dict(ldo=500), -1),
    (dict(kpack=None), -1),
    (dict(qk_mode=2), -1),
    (dict(reserved=1), -1),
])
def test_attention_argument_errors(kw, status):
    lib = sqg.load()
    a = attn_args(**kw)
    assert lib.sqg_packed_kv_attention(ctypes.byref(a), None) == status
    assert len(lib.sqg_last_error()) > 0


def test_test_entry_argument_errors():
    lib = sqg.load()
    assert lib.sqg_test_quant_pack_f32(FAKE, 10, 3, FAKE, FAKE, None) == -1
    assert lib.sqg_test_quant_pack_f32(FAKE + 4, 10, 0, FAKE, FAKE, None) == -3
    assert lib.sqg_test_quant_pack_f32(FAKE, 0, 0, None, None, None) == 0
    assert lib.sqg_test_fwht_f32(FAKE, FAKE, -1, 0, None) == -1


@pytest.mark.parametrize("n,ranges", [
    # one head's BF16 codes of an 8,388,736-token range: 256 B x N > 2^31 - 1
    (8388736, [(0, 8388736, 2)]),
    # INT8 rows of a masked head inside an INT4 range: 128 B x N > 2^31 - 1
    (16777344, [(0, 16777344, 0, 1)]),
    # INT4 rows: 64 B x N > 2^31 - 1
    (33554560, None),
    # scales: 8 B x N > 2^31 - 1 for every head, whatever the codes need
    (268435584, [(0, 128, 0), (128, 268435584, 0)]),
])
def test_attention_rejects_stores_beyond_32bit_resources(n, ranges):
    # the kernel addresses each (range, head) block of codes and each head's scales
    # through buffer resources with a 32-bit byte length: larger stores are refused
    # before anything is enqueued
    lib = sqg.load()
    arr, nr = B._ranges_array(ranges)
    a = attn_args(n_tokens=n, d_model=128, n_heads=1, ldq=128, ldo=128,
                  ranges=ctypes.cast(arr, ctypes.POINTER(B.Range)) if arr is not None else None,
                  n_ranges=nr)
    assert lib.sqg_packed_kv_attention(ctypes.byref(a), None) == -2
    assert b"2 GiB" in lib.sqg_last_error()


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((256, 256), dtype=torch.bfloat16)
    w = torch.zeros((256, 768), dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        sqg.streamed_qkv_quant(x, w, out={"q": x, "kpack": x, "vpack": x, "kscale": x, "vscale": x})


# ----------------------------------------------------------------------------- host-staged store
STAGE_POLICY = [(0, 384, 1), (384, 1024, 0), (1024, 2304, 1), (2304, 2900, 0)]


@pytest.mark.parametrize("k0,k1", [(0, 2900), (0, 512), (256, 1280), (1024, 2900), (2816, 2900),
                                   (384, 1000)])
def test_block_layout_is_the_layout_of_the_clipped_policy(k0, k1):
    # a block store is the store of the shorter sequence whose policy is the clipped one
    H = 4
    B_ = sqg.kv_block_layout(2900, 512, k0, k1, STAGE_POLICY)
    clipped = [(max(b, k0) - k0, min(e, k1) - k0, f) for b, e, f in STAGE_POLICY if min(e, k1) > max(b, k0)]
    want, total = oracle.packed_layout(k1 - k0, H, clipped)
    assert B_["n_tokens"] == k1 - k0
    assert len(B_["segments"]) == len(want)
    for got, w in zip(B_["segments"], want):
        assert (got["begin"] - k0, got["end"] - k0, got["fmt"], got["offset"], got["row_bytes"]) == \
            (w["begin"], w["end"], w["fmt"], w["offset"], w["row_bytes"])
    assert B_["scale_bytes"] == H * (k1 - k0) * 8 and B_["pack_bytes"] == total


@pytest.mark.parametrize("k0,k1", [(100, 900), (0, 0), (512, 256), (0, 3000), (-128, 128)])
def test_block_layout_rejects_bad_blocks(k0, k1):
    with pytest.raises(sqg.SqgError):
        sqg.kv_block_layout(2900, 512, k0, k1, STAGE_POLICY)


@pytest.mark.parametrize("block,nb", [(512, 5), (1024, 3), (128, 22), (4096, 1)])
def test_staged_sizes_sum_the_blocks(block, nb):
    (hp, hs, dp, ds), n_blocks = sqg.staged_sizes(2900, 512, block, STAGE_POLICY)
    full = sqg.kv_layout(2900, 512, STAGE_POLICY)
    assert n_blocks == nb
    assert hp == full["pack_bytes"] and hs == full["scale_bytes"]
    plan = sqg.chunk_ranges(2900, block, 512)
    assert len(plan) == nb
    blocks = [sqg.kv_block_layout(2900, 512, b, e, STAGE_POLICY) for b, e in plan]
    assert sum(b["pack_bytes"] for b in blocks) == hp
    assert dp == max(b["pack_bytes"] for b in blocks) and ds == max(b["scale_bytes"] for b in blocks)


def staged_struct(**kw):
    s = B.StagedKV()
    s.block_rows = 512
    s.host_kpack = s.host_vpack = s.host_kscale = s.host_vscale = FAKE
    for k in ("dev_kpack", "dev_vpack", "dev_kscale", "dev_vscale"):
        arr = getattr(s, k)
        arr[0], arr[1] = FAKE, FAKE + 4096
    for k, v in kw.items():
        if k.endswith("_1"):
            getattr(s, k[:-2])[1] = v
        else:
            setattr(s, k, v)
    return s


@pytest.mark.parametrize("kw,status,msg", [
    (dict(block_rows=100), -1, b"block_rows"),
    (dict(block_rows=0), -1, b"block_rows"),
    (dict(host_vscale=None), -1, b"host"),
    (dict(dev_vpack_1=None), -1, b"staging"),
    (dict(dev_kscale_1=FAKE + 8), -3, b"aligned"),
])
def test_staged_argument_errors(kw, status, msg):
    lib = sqg.load()
    s = staged_struct(**kw)
    a = qkv_args(kpack=None, vpack=None, kscale=None, vscale=None)
    assert lib.sqg_streamed_qkv_quant_staged(ctypes.byref(a), ctypes.byref(s), None) == status
    assert msg in lib.sqg_last_error()
    b = attn_args(kpack=None, vpack=None, kscale=None, vscale=None)
    assert lib.sqg_packed_kv_attention_staged(ctypes.byref(b), ctypes.byref(s), None) == status
    assert msg in lib.sqg_last_error()


def test_staged_entry_specific_errors():
    lib = sqg.load()
    s = staged_struct()
    assert lib.sqg_streamed_qkv_quant_staged(ctypes.byref(qkv_args(emit=1)), ctypes.byref(s), None) == -1
    assert b"SQG_EMIT_Q" in lib.sqg_last_error()
    assert lib.sqg_streamed_qkv_quant_staged(ctypes.byref(qkv_args()), None, None) == -1
    # 1024 keys in 512-key blocks: two blocks need the LSE merge
    b = attn_args(lse=None)
    assert lib.sqg_packed_kv_attention_staged(ctypes.byref(b), ctypes.byref(s), None) == -1
    assert b"spans 2 blocks" in lib.sqg_last_error()
    b = attn_args(o_dtype=1)
    assert lib.sqg_packed_kv_attention_staged(ctypes.byref(b), ctypes.byref(s), None) == -1
    # empty query range: nothing to do
    b = attn_args(q_begin=5, q_end=5)
    assert lib.sqg_packed_kv_attention_staged(ctypes.byref(b), ctypes.byref(s), None) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(workspace=FAKE), -1, b"workspace must be NULL"),
    (dict(workspace=None, workspace_bytes=4096), -1, b"workspace must be NULL"),
    # explicit chunks of 65536 rows of d 512 need 64 MiB + the folded tail: beyond the scratch
    (dict(workspace=None, workspace_bytes=0, q_chunk_rows=65536, attn_n_tokens=66000), -4, b"scratch"),
    (dict(workspace=None, workspace_bytes=0, x=None), -1, b"NULL"),
])
def test_noalloc_qrecompute_argument_errors(kw, status, msg):
    # the allocation-free entry point checks its arguments like the Q-recompute entry and
    # refuses a workspace of its own or chunks beyond its device scratch, before any launch
    lib = sqg.load()
    r = qrec_args(**kw)
    assert lib.sqg_packed_kv_attention_qrecompute_noalloc(ctypes.byref(r), None) == status
    assert msg in lib.sqg_last_error()


def test_noalloc_scratch_size():
    assert sqg.noalloc_scratch_bytes() == 64 << 20
