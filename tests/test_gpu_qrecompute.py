"""GPU tests of the Q-recompute mode: the K/V-only projection, the Q-only projection
and attention with Q recomputed per query chunk.  The streamed block on the VRAM Lab
page keeps only the packed K/V of the whole sequence and rebuilds Q chunk by chunk;
every piece here must equal the matching part of the one-pass path bit for bit, and
the attention output also meets the oracle gate on its own.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import INT4, INT8

pytestmark = pytest.mark.gpu

DEV = "cuda"
STORE_KEYS = ("kpack", "vpack", "kscale", "vscale")


def inputs(N, d, seed, norm=True, rope=True):
    x = synth.make_x(N, d, 0.01, seed=seed, device=DEV)
    w = synth.make_w(d, seed=seed + 1, device=DEV)
    kw = {}
    if norm:
        qn, kn = synth.make_norm_weights(seed + 2)
        kw["q_norm_w"], kw["k_norm_w"] = qn.to(DEV), kn.to(DEV)
    if rope:
        import streamed_qkv_gemm_amd as sqg
        kw["rope_cos"], kw["rope_sin"] = sqg.rope_table(N, 10000.0, device=DEV)
    return x, w, kw


def q_kw(kw):
    return {k: v for k, v in kw.items() if k != "k_norm_w"}


def host(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("N,d,ranges,chunk", [
    (1000, 512, [(0, 256, INT8), (256, 1000, INT4)], 0),
    (777, 768, None, 256),
])
def test_emit_modes_equal_the_full_call(lib, N, d, ranges, chunk):
    x, w, kw = inputs(N, d, seed=201)
    full = lib.streamed_qkv_quant(x, w, ranges=ranges, chunk_rows=chunk, **kw)
    kv = lib.streamed_qkv_quant(x, w, ranges=ranges, chunk_rows=chunk, emit=lib.SQG_EMIT_KV, **kw)
    qo = lib.streamed_qkv_quant(x, w, ranges=ranges, chunk_rows=chunk, emit=lib.SQG_EMIT_Q, **kw)
    torch.cuda.synchronize()
    assert kv["q"] is None and all(qo[k] is None for k in STORE_KEYS)
    for k in STORE_KEYS:
        assert torch.equal(kv[k], full[k]), k
    assert torch.equal(qo["q"], full["q"])


def test_emit_kv_leaves_a_given_q_untouched(lib):
    N, d = 640, 512
    x, w, kw = inputs(N, d, seed=211, norm=False, rope=False)
    out = lib.alloc_store(N, d, device=DEV)
    out["q"].fill_(3.0)
    lib.streamed_qkv_quant(x, w, out=out, emit=lib.SQG_EMIT_KV)
    torch.cuda.synchronize()
    assert bool((out["q"] == 3.0).all())


@pytest.mark.parametrize("chunk", [0, 128, 256])
def test_qrecompute_equals_two_step_path(lib, chunk):
    # N = 1000: with 128- and 256-row chunks the short last chunk joins the one before,
    # so chunks start at rows that are not multiples of the 256-row query tile.
    N, d = 1000, 512
    ranges = [(0, 128, INT8), (128, N, INT4)]
    x, w, kw = inputs(N, d, seed=221)
    full = lib.streamed_qkv_quant(x, w, ranges=ranges, **kw)
    kv = lib.streamed_qkv_quant(x, w, ranges=ranges, emit=lib.SQG_EMIT_KV, **kw)
    o_ref, l_ref = lib.packed_kv_attention(full)
    o, l = lib.packed_kv_attention_qrecompute(kv, x, w, q_chunk_rows=chunk, **q_kw(kw))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    # and on its own against the oracle (the G3 gate)
    H = d // 128
    layout, _ = oracle.packed_layout(N, H, oracle.range_segments(N, ranges))
    rows = np.arange(0, N, 9)
    want, lse_want = oracle.attention_rows_from_store(
        synth.bf16_bits(full["q"])[rows], rows, host(kv["kpack"]), host(kv["vpack"]),
        host(kv["kscale"]), host(kv["vscale"]), layout, H, N)
    err = np.abs(host(o)[rows].astype(np.float64) - want)
    rel = np.linalg.norm(host(o)[rows] - want) / np.linalg.norm(want)
    assert err.max() <= 2e-2 and rel <= 5e-3
    assert np.max(np.abs(host(l)[:, rows] - lse_want)) <= 2e-3


def test_qrecompute_subranges_blocks_and_accumulate(lib):
    N, d = 1100, 512
    x, w, kw = inputs(N, d, seed=231)
    full = lib.streamed_qkv_quant(x, w, **kw)
    kv = lib.streamed_qkv_quant(x, w, emit=lib.SQG_EMIT_KV, **kw)
    args = dict(q_begin=77, q_end=1011, kv_begin=128, kv_end=1024, kv_block=256)
    o_ref = torch.full((N, d), 5.0, device=DEV)
    l_ref = torch.full((d // 128, N), 5.0, device=DEV)
    o = o_ref.clone()
    l = l_ref.clone()
    lib.packed_kv_attention(full, o=o_ref, lse=l_ref, **args)
    lib.packed_kv_attention_qrecompute(kv, x, w, q_chunk_rows=384, o=o, lse=l, **args, **q_kw(kw))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    assert bool((o[:77] == 5.0).all()) and bool((o[1011:] == 5.0).all())
    # second half of the keys merged into the first through the LSE
    lib.packed_kv_attention(full, o=o_ref, lse=l_ref, q_begin=77, q_end=1011, kv_begin=1024,
                            accumulate=True)
    lib.packed_kv_attention_qrecompute(kv, x, w, q_chunk_rows=384, o=o, lse=l, q_begin=77,
                                       q_end=1011, kv_begin=1024, accumulate=True, **q_kw(kw))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_qrecompute_workspace_too_small_raises(lib):
    N, d = 1000, 512
    x, w, kw = inputs(N, d, seed=241, norm=False, rope=False)
    kv = lib.streamed_qkv_quant(x, w, emit=lib.SQG_EMIT_KV)
    need = lib.qrecompute_workspace_bytes(N, d, 256)
    ws = torch.empty((need - 16,), dtype=torch.uint8, device=DEV)
    with pytest.raises(lib.SqgError):
        lib.packed_kv_attention_qrecompute(kv, x, w, q_chunk_rows=256, workspace=ws)
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
    o, _ = lib.packed_kv_attention_qrecompute(kv, x, w, q_chunk_rows=256, workspace=ws)
    full = lib.streamed_qkv_quant(x, w)
    o_ref, _ = lib.packed_kv_attention(full)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
