"""GPU parity under the richer precision policy: BF16 ranges ([FR] "Mixed precision for
conditioning") and INT8 heads inside INT4 ranges ([VL] kvmix section), against the
oracle at sizes it finishes in seconds (several tiles, ragged tails).

Gates: integer entries as G2 (>= 99.9% of codes identical, the rest one step apart;
scales at most one grid step apart, >= 98% identical); BF16 entries >= 99% of bit
patterns identical and every value within one bf16 step plus a floor of 1e-5 of the
row's norm (the GPU rotates in fp32, the oracle in fp64 rounded once to fp32, so a
value that cancels can round differently); attention as G3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import BF16, INT4, INT8

pytestmark = pytest.mark.gpu

DEV = "cuda"


def host(t):
    return t.detach().cpu().numpy()


def run_case(lib, N, d, ranges, seed, chunk=0, norm_rope=True):
    H = d // 128
    x = synth.make_x(N, d, 0.01, seed=seed, device=DEV)
    w = synth.make_w(d, seed=seed + 1, device=DEV)
    kw, okw = {}, {}
    if norm_rope:
        qn, kn = synth.make_norm_weights(seed + 2)
        kw = dict(q_norm_w=qn.to(DEV), k_norm_w=kn.to(DEV))
        kw["rope_cos"], kw["rope_sin"] = lib.rope_table(N, 10000.0, device=DEV)
        okw = dict(q_norm_w=qn.numpy(), k_norm_w=kn.numpy(), eps=1e-6, rope_theta=10000.0)
    store = lib.streamed_qkv_quant(x, w, ranges=ranges, chunk_rows=chunk, **kw)
    torch.cuda.synchronize()
    segs = oracle.range_segments(N, ranges, n_heads=H)
    layout, total = oracle.packed_layout(N, H, segs)
    assert total == store["layout"]["pack_bytes"]
    return x, w, store, segs, layout, okw


def check_store(lib, x, w, store, segs, layout, okw, rows):
    N, d = x.shape
    H = d // 128
    fm = oracle.head_formats(N, H, segs)[rows]
    ref = oracle.qkv_quant_rows(synth.bf16_bits(x.cpu())[rows], synth.bf16_bits(w.cpu()), H, rows, fm, **okw)
    for t in ("k", "v"):
        pk, sc = host(store[t + "pack"]), host(store[t + "scale"])
        codes, scales = oracle.gather_packed_rows(pk, sc, layout, H, rows)
        bits = oracle.gather_bf16_rows(pk, layout, H, rows)
        integer = fm != BF16
        if integer.any():
            d_codes = np.abs(codes[integer].astype(np.int64) - ref[t + "_codes"][integer].astype(np.int64))
            assert d_codes.max() <= 1 and np.mean(d_codes == 0) >= 0.999, t
            g, r = scales[integer].astype(np.float64), ref[t + "_scales"][integer].astype(np.float64)
            # one step: of the 8-bit INT4 grid, or one fp16 step for INT8
            rel = np.where(fm[integer] == INT4, 2.0 ** (1 - oracle.INT4_SCALE_BITS), 2.0 ** -10)
            assert np.all(np.abs(g - r) <= r * rel[:, None] * 1.0001), t
            assert np.mean(g == r) >= 0.98, t
        bf = fm == BF16
        assert np.all(scales[bf] == 0), t
        gb, rb = bits[bf], ref[t + "_bf16"][bf]
        assert np.mean(gb == rb) >= 0.99, t
        gv, rv = oracle.bf16_bits_to_f64(gb), oracle.bf16_bits_to_f64(rb)
        # one bf16 step, plus a floor for values that cancel in the fp32 transform
        # (its error is absolute: a few fp32 steps of the row's magnitude)
        floor = 1e-5 * np.linalg.norm(rv, axis=-1, keepdims=True)
        assert np.all(np.abs(gv - rv) <= np.abs(rv) * 2.0 ** -7 + floor), t
        assert np.all(bits[integer] == 0)


POLICIES = [
    (2000, 768, [(0, 256, BF16), (256, 640, INT8), (640, 1536, INT4, 0b100101), (1536, 2000, BF16)]),
    (1000, 512, [(0, 128, INT4, 0b1111), (128, 1000, BF16)]),
    (700, 512, [(0, 700, BF16)]),
]


@pytest.mark.parametrize("N,d,ranges", POLICIES)
def test_g2_mixed_policy(lib, N, d, ranges):
    x, w, store, segs, layout, okw = run_case(lib, N, d, ranges, seed=501, chunk=512)
    rows = np.unique(np.concatenate([np.arange(0, N, 7), [0, 127, 128, 255, 256, N - 1]]))
    rows = rows[rows < N]
    check_store(lib, x, w, store, segs, layout, okw, rows)


@pytest.mark.parametrize("N,d,ranges", POLICIES)
def test_g3_mixed_policy(lib, N, d, ranges):
    x, w, store, segs, layout, _ = run_case(lib, N, d, ranges, seed=511)
    H = d // 128
    o, lse = lib.packed_kv_attention(store)
    o2, lse2 = lib.packed_kv_attention(store, kv_block=256)
    torch.cuda.synchronize()
    rows = np.arange(0, N, 5)
    qb = synth.bf16_bits(store["q"])[rows]
    args = (host(store["kpack"]), host(store["vpack"]), host(store["kscale"]), host(store["vscale"]),
            layout, H, N)
    want, lse_want = oracle.attention_rows_from_store(qb, rows, *args)
    got = host(o)[rows].astype(np.float64)
    assert np.abs(got - want).max() <= 2e-2
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= 5e-3
    assert np.max(np.abs(host(lse)[:, rows] - lse_want)) <= 2e-3
    want2, _ = oracle.attention_rows_from_store(qb, rows, *args, kv_block=256)
    got2 = host(o2)[rows].astype(np.float64)
    assert np.abs(got2 - want2).max() <= 2e-2
    assert np.linalg.norm(got2 - want2) / np.linalg.norm(want2) <= 5e-3


def test_mixed_policy_qrecompute_and_subranges(lib):
    N, d, ranges = POLICIES[0]
    x, w, store, segs, layout, _ = run_case(lib, N, d, ranges, seed=521, norm_rope=False)
    kv = lib.streamed_qkv_quant(x, w, ranges=ranges, emit=lib.SQG_EMIT_KV)
    o_ref, l_ref = lib.packed_kv_attention(store, q_begin=100, q_end=1900, kv_begin=128, kv_end=1792)
    o, l = lib.packed_kv_attention_qrecompute(kv, x, w, q_chunk_rows=512, q_begin=100, q_end=1900,
                                              kv_begin=128, kv_end=1792)
    torch.cuda.synchronize()
    assert torch.equal(o[100:1900], o_ref[100:1900]) and torch.equal(l[:, 100:1900], l_ref[:, 100:1900])
