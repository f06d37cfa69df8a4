"""GPU tests of the host-staged K/V store: the packed K/V lives in pinned host memory
as consecutive block stores and is carried to and from the GPU one block at a time
(the VRAM Lab page names host-staged K/V as the real fix for the K/V peak).  Every
block must hold exactly the bytes the device store holds for its keys, and attention
over the staged blocks must equal the device path over the same key blocks bit for
bit (and meet the oracle gate on its own).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import BF16, INT4, INT8

pytestmark = pytest.mark.gpu

DEV = "cuda"
N, D = 2900, 512
POLICY = [(0, 384, INT8), (384, 1024, INT4), (1024, 2304, INT8), (2304, N, INT4)]


def make(lib, seed, ranges=POLICY):
    x = synth.make_x(N, D, 0.01, seed=seed, device=DEV)
    w = synth.make_w(D, seed=seed + 1, device=DEV)
    qn, kn = synth.make_norm_weights(seed + 2)
    cos, sin = lib.rope_table(N, 10000.0, device=DEV)
    kw = dict(q_norm_w=qn.to(DEV), k_norm_w=kn.to(DEV), rope_cos=cos, rope_sin=sin)
    return x, w, kw


def host(t):
    return t.detach().cpu().numpy()


def block_rows_of(lib, staged, full_ranges):
    """(k0, k1, codes/scales of K and V) per block, decoded from the host store."""
    H = D // 128
    out = []
    po = so = 0
    for k0, k1 in lib.chunk_ranges(N, staged["block_rows"], 512):
        L = lib.kv_block_layout(N, D, k0, k1, full_ranges)
        # the oracle's layout of the clipped policy, in block coordinates
        clipped = [(max(r[0], k0) - k0, min(r[1], k1) - k0) + tuple(r[2:])
                   for r in full_ranges if min(r[1], k1) > max(r[0], k0)]
        lay, total = oracle.packed_layout(k1 - k0, H, oracle.range_segments(k1 - k0, clipped))
        assert total == L["pack_bytes"]
        rows = np.arange(k1 - k0)
        got = {}
        for t in ("k", "v"):
            pk = host(staged["host_%spack" % t])[po:po + L["pack_bytes"]]
            sc = host(staged["host_%sscale" % t])[so:so + L["scale_bytes"]].view(np.float16)
            got[t] = oracle.gather_packed_rows(pk, sc.reshape(H, k1 - k0, 4), lay, H, rows) + \
                (oracle.gather_bf16_rows(pk, lay, H, rows),)
        out.append((k0, k1, got))
        po += L["pack_bytes"]
        so += L["scale_bytes"]
    return out


MIXED = [(0, 256, BF16), (256, 640, INT8), (640, 2304, INT4, 0b1010), (2304, N, BF16)]


@pytest.mark.parametrize("block,policy", [(512, POLICY), (1024, POLICY), (512, MIXED)])
def test_staged_store_holds_the_device_store_bytes(lib, block, policy):
    H = D // 128
    x, w, kw = make(lib, 301)
    full = lib.streamed_qkv_quant(x, w, ranges=policy, **kw)
    staged = lib.alloc_staged(N, D, block, policy, device=DEV)
    q = lib.streamed_qkv_quant_staged(x, w, staged, **kw)
    torch.cuda.synchronize()
    assert torch.equal(q, full["q"])
    layout, _ = oracle.packed_layout(N, H, oracle.range_segments(N, policy))
    for k0, k1, got in block_rows_of(lib, staged, policy):
        rows = np.arange(k0, k1)
        for t in ("k", "v"):
            want = oracle.gather_packed_rows(host(full[t + "pack"]), host(full[t + "scale"]), layout, H, rows)
            assert np.array_equal(got[t][0], want[0]), (t, k0)
            assert np.array_equal(got[t][1].view(np.uint16), want[1].view(np.uint16)), (t, k0)
            assert np.array_equal(got[t][2], oracle.gather_bf16_rows(host(full[t + "pack"]), layout, H, rows))


def test_staged_kv_only_build_matches(lib):
    x, w, kw = make(lib, 311)
    a = lib.alloc_staged(N, D, 512, POLICY, device=DEV)
    b = lib.alloc_staged(N, D, 512, POLICY, device=DEV)
    lib.streamed_qkv_quant_staged(x, w, a, **kw)
    q = lib.streamed_qkv_quant_staged(x, w, b, emit=lib.SQG_EMIT_KV, **kw)
    torch.cuda.synchronize()
    assert q is None
    for k in ("host_kpack", "host_vpack", "host_kscale", "host_vscale"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("block,policy", [(512, POLICY), (1024, POLICY), (1024, MIXED)])
def test_staged_attention_equals_device_blocks(lib, block, policy):
    x, w, kw = make(lib, 321)
    full = lib.streamed_qkv_quant(x, w, ranges=policy, **kw)
    staged = lib.alloc_staged(N, D, block, policy, device=DEV)
    lib.streamed_qkv_quant_staged(x, w, staged, emit=lib.SQG_EMIT_KV, **kw)
    # the staged call runs one launch per block merged through the LSE: bit for bit the
    # device store attended block by block through explicit key ranges
    o_ref = torch.empty((N, D), dtype=torch.float32, device=DEV)
    l_ref = torch.empty((D // 128, N), dtype=torch.float32, device=DEV)
    for i, (k0, k1) in enumerate(lib.chunk_ranges(N, block, 512)):
        lib.packed_kv_attention(full, kv_begin=k0, kv_end=k1, accumulate=i > 0, o=o_ref, lse=l_ref)
    o, l = lib.packed_kv_attention_staged(staged, full["q"])
    # the device path with kv_block walks the blocks in one launch: equal up to rounding
    o_one, l_one = lib.packed_kv_attention(full, kv_block=block)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    assert float((o - o_one).abs().max()) <= 2e-3 and float((l - l_one).abs().max()) <= 1e-4
    # G3 on its own against the oracle, sampled rows
    H = D // 128
    layout, _ = oracle.packed_layout(N, H, oracle.range_segments(N, policy))
    rows = np.arange(0, N, 29)
    want, lse_want = oracle.attention_rows_from_store(
        synth.bf16_bits(full["q"])[rows], rows, host(full["kpack"]), host(full["vpack"]),
        host(full["kscale"]), host(full["vscale"]), layout, H, N, kv_block=block)
    got = host(o)[rows].astype(np.float64)
    assert np.abs(got - want).max() <= 2e-2
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= 5e-3
    assert np.max(np.abs(host(l)[:, rows] - lse_want)) <= 2e-3


def test_staged_attention_subranges_and_accumulate(lib):
    # keys [256, 2688) in 512-key blocks meet blocks [0,512) ... [2048,2900) partially;
    # the device path makes the same launches through explicit key ranges
    x, w, kw = make(lib, 331)
    full = lib.streamed_qkv_quant(x, w, ranges=POLICY, **kw)
    staged = lib.alloc_staged(N, D, 512, POLICY, device=DEV)
    lib.streamed_qkv_quant_staged(x, w, staged, emit=lib.SQG_EMIT_KV, **kw)
    q = full["q"]
    o_ref = torch.full((N, D), 3.0, device=DEV)
    l_ref = torch.full((D // 128, N), 3.0, device=DEV)
    o, l = o_ref.clone(), l_ref.clone()
    cuts = [256, 512, 1024, 1536, 2048, 2688]
    for i in range(len(cuts) - 1):
        lib.packed_kv_attention(full, q=q, q_begin=77, q_end=2000, kv_begin=cuts[i], kv_end=cuts[i + 1],
                                accumulate=i > 0, o=o_ref, lse=l_ref)
    lib.packed_kv_attention_staged(staged, q, q_begin=77, q_end=2000, kv_begin=256, kv_end=2688, o=o, lse=l)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    assert bool((o[:77] == 3.0).all()) and bool((o[2000:] == 3.0).all())
    # the rest of the keys merged on top, starting from the partial result
    lib.packed_kv_attention(full, q=q, q_begin=77, q_end=2000, kv_begin=0, kv_end=256, accumulate=True,
                            o=o_ref, lse=l_ref)
    lib.packed_kv_attention(full, q=q, q_begin=77, q_end=2000, kv_begin=2688, accumulate=True,
                            o=o_ref, lse=l_ref)
    lib.packed_kv_attention_staged(staged, q, q_begin=77, q_end=2000, kv_begin=0, kv_end=256,
                                   accumulate=True, o=o, lse=l)
    lib.packed_kv_attention_staged(staged, q, q_begin=77, q_end=2000, kv_begin=2688, accumulate=True,
                                   o=o, lse=l)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_overlapped_and_in_order_copies_agree(lib):
    # the copies on a stream of their own (the default) and in order on the call's stream
    # must leave the same host bytes and give the same attention, block for block
    x, w, kw = make(lib, 341)
    full = lib.streamed_qkv_quant(x, w, ranges=POLICY, **kw)
    a = lib.alloc_staged(N, D, 512, POLICY, device=DEV)
    b = lib.alloc_staged(N, D, 512, POLICY, device=DEV, overlap=False)
    assert a["copy_stream"] is not None and b["copy_stream"] is None
    lib.streamed_qkv_quant_staged(x, w, a, emit=lib.SQG_EMIT_KV, **kw)
    lib.streamed_qkv_quant_staged(x, w, b, emit=lib.SQG_EMIT_KV, **kw)
    oa, la = lib.packed_kv_attention_staged(a, full["q"])
    ob, lb = lib.packed_kv_attention_staged(b, full["q"])
    # back to back on the same stream: the second call's copies follow the first's kernels
    oa2, la2 = lib.packed_kv_attention_staged(a, full["q"])
    torch.cuda.synchronize()
    for k in ("host_kpack", "host_vpack", "host_kscale", "host_vscale"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(oa2, oa) and torch.equal(la2, la)
