"""Pins of the oracle's attention, log-sum-exp merge and packed-store decode
(CPU only)."""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import HEAD_DIM, INT4, INT8

SCALE = HEAD_DIM ** -0.5


def rnd(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def test_matches_scipy_softmax_and_logsumexp():
    q, k, v = rnd((5, 128), 1), rnd((40, 128), 2), rnd((40, 128), 3)
    o, lse = oracle.softmax_attention(q, k, v, SCALE)
    s = (q @ k.T) * SCALE
    assert np.allclose(o, scipy.special.softmax(s, axis=-1) @ v, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-13)


def test_zero_query_gives_mean_of_values():
    k, v = rnd((33, 128), 4, 5), rnd((33, 128), 5)
    o, lse = oracle.softmax_attention(np.zeros((2, 128)), k, v, SCALE)
    assert np.allclose(o, v.mean(0), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, math.log(33), rtol=1e-14)


def test_single_key_returns_its_value():
    q, k, v = rnd((3, 128), 6), rnd((1, 128), 7), rnd((1, 128), 8)
    o, lse = oracle.softmax_attention(q, k, v, SCALE)
    assert np.allclose(o, v[0], rtol=1e-14)
    assert np.allclose(lse, (q @ k[0]) * SCALE, rtol=1e-13)


def test_two_keys_by_hand():
    q = np.zeros((1, 128))
    q[0, 0] = 1.0
    k = np.zeros((2, 128))
    k[0, 0], k[1, 0] = 2.0, -1.0
    v = np.zeros((2, 128))
    v[0, 1], v[1, 1] = 10.0, 4.0
    o, lse = oracle.softmax_attention(q, k, v, 1.0)
    p0 = math.exp(2) / (math.exp(2) + math.exp(-1))
    assert math.isclose(o[0, 1], 10 * p0 + 4 * (1 - p0), rel_tol=1e-14)
    assert math.isclose(lse[0], math.log(math.exp(2) + math.exp(-1)), rel_tol=1e-14)


def test_identical_keys_and_constant_values():
    q = rnd((4, 128), 9)
    k = np.repeat(rnd((1, 128), 10), 17, axis=0)
    v = rnd((17, 128), 11)
    o, _ = oracle.softmax_attention(q, k, v, SCALE)
    assert np.allclose(o, v.mean(0), rtol=1e-12, atol=1e-13)
    vc = np.repeat(rnd((1, 128), 12), 17, axis=0)
    o2, _ = oracle.softmax_attention(q, rnd((17, 128), 13), vc, SCALE)
    assert np.allclose(o2, vc[0], rtol=1e-12)


def test_key_permutation_and_constant_shift_invariance():
    # softmax ignores a constant added to every score of a row; adding one vector c to
    # every key adds q.c to every score of row q (VRAM Lab, kvfp4s section: centring
    # keys plus rotation is an exact reference)
    q, k, v = rnd((6, 128), 14), rnd((50, 128), 15), rnd((50, 128), 16)
    o, lse = oracle.softmax_attention(q, k, v, SCALE)
    perm = np.random.default_rng(17).permutation(50)
    o2, lse2 = oracle.softmax_attention(q, k[perm], v[perm], SCALE)
    assert np.allclose(o, o2, rtol=1e-12) and np.allclose(lse, lse2, rtol=1e-12)
    c = rnd((128,), 18, 3)
    o3, lse3 = oracle.softmax_attention(q, k + c, v, SCALE)
    assert np.allclose(o, o3, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse3, lse + (q @ c) * SCALE, rtol=1e-12)


def test_rotation_invariance():
    # attention(qR, kR, vR) R^T = attention(q, k, v) for the orthonormal R = H/sqrt(128)
    q, k, v = rnd((6, 128), 19), rnd((30, 128), 20), rnd((30, 128), 21)
    R = oracle.rotation_matrix()
    o, lse = oracle.softmax_attention(q, k, v, SCALE)
    o_r, lse_r = oracle.softmax_attention(q @ R, k @ R, v @ R, SCALE)
    assert np.allclose(o_r @ R.T, o, rtol=1e-11, atol=1e-12)
    assert np.allclose(lse_r, lse, rtol=1e-13)


@pytest.mark.parametrize("S,block,min_tail", [(64, 16, 1), (64, 20, 1), (50, 7, 3), (9, 1, 1), (64, 64, 1)])
def test_blockwise_merge_equals_single_pass(S, block, min_tail):
    q, k, v = rnd((4, 128), 22, 2), rnd((S, 128), 23, 2), rnd((S, 128), 24)
    o, lse = oracle.softmax_attention(q, k, v, SCALE)
    ob, lseb = oracle.attention_blockwise(q, k, v, SCALE, block, min_tail)
    assert np.allclose(ob, o, rtol=1e-12, atol=1e-13)
    assert np.allclose(lseb, lse, rtol=1e-13)


def test_online_merge_of_two_halves_by_hand():
    # two one-key partials: o1 = v1 with lse1 = s1, o2 = v2 with lse2 = s2
    o1, o2 = np.array([[1.0]]), np.array([[3.0]])
    l1, l2 = np.array([0.5]), np.array([-0.25])
    o, lse = oracle.online_merge(o1, l1, o2, l2)
    w1 = math.exp(0.5) / (math.exp(0.5) + math.exp(-0.25))
    assert math.isclose(o[0, 0], w1 * 1 + (1 - w1) * 3, rel_tol=1e-14)
    assert math.isclose(lse[0], math.log(math.exp(0.5) + math.exp(-0.25)), rel_tol=1e-14)
    o0, l0 = oracle.online_merge(None, None, o1, l1)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_model_and_rotated_forms_agree():
    rng = np.random.default_rng(25)
    qb = oracle.f32_to_bf16_bits(rng.standard_normal((5, 128)).astype(np.float32))
    kr = rnd((70, 128), 26, 2)
    vr = rnd((70, 128), 27)
    o1, l1 = oracle.attention_rotated_rows(qb, kr, vr, SCALE)
    o2, l2 = oracle.attention_model_rows(qb, kr, vr, SCALE)
    assert np.allclose(o1, o2, rtol=1e-11, atol=1e-12) and np.allclose(l1, l2, rtol=1e-13)
    o3, l3 = oracle.attention_rotated_rows(qb, kr, vr, SCALE, kv_block=16)
    assert np.allclose(o1, o3, rtol=1e-11, atol=1e-12) and np.allclose(l1, l3, rtol=1e-13)


# ----------------------------------------------------------------------------- packed store
def _store(n, H, segs, seed):
    """Quantise random rotated vectors and lay them out with oracle.packed_layout."""
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal((n, H, 128)) * 2).astype(np.float32)
    fm = oracle.token_formats(n, segs)
    codes = np.zeros((n, H, 128), np.int8)
    scales = np.zeros((n, H, 4), np.float16)
    for f in (INT4, INT8):
        sel = fm == f
        codes[sel], scales[sel] = oracle.quantize_groups(r[sel], oracle.QMAX[f])
    layout, total = oracle.packed_layout(n, H, segs)
    blob = np.zeros(total, np.uint8)
    for seg in layout:
        b, e, rb = seg["begin"], seg["end"], seg["row_bytes"]
        for h in range(H):
            rows = oracle.pack_codes(codes[b:e, h], seg["fmt"])
            start = seg["offset"] + h * (e - b) * rb
            blob[start:start + (e - b) * rb] = rows.reshape(-1)
    return codes, scales, np.ascontiguousarray(scales.transpose(1, 0, 2)), layout, blob, total


def test_packed_layout_sizes_closed_form():
    segs = oracle.range_segments(65536, [(0, 512, INT8), (512, 8704, INT8), (8704, 65536, INT4)])
    layout, total = oracle.packed_layout(65536, 56, segs)
    assert total == 56 * (8704 * 128 + (65536 - 8704) * 64)
    assert [s["offset"] for s in layout] == [0, 56 * 512 * 128, 56 * 8704 * 128]


def test_gather_and_decode_agree_with_quantised_rows():
    segs = [(0, 128, INT8), (128, 300, INT4)]
    codes, scales, sc_hn, layout, blob, _ = _store(300, 3, segs, 28)
    rows = np.array([0, 5, 127, 128, 129, 299])
    c, s = oracle.gather_packed_rows(blob, sc_hn, layout, 3, rows)
    assert np.array_equal(c, codes[rows]) and np.array_equal(s, scales[rows])
    for h in range(3):
        dec = oracle.decode_head(blob, sc_hn, layout, 3, h, 100, 260)
        assert np.array_equal(dec, oracle.dequantize(codes[100:260, h], scales[100:260, h]))


def test_attention_from_store_matches_direct():
    segs = [(0, 128, INT8), (128, 200, INT4)]
    codes, scales, sc_hn, layout, blob, _ = _store(200, 2, segs, 29)
    _, _, sc_hn_v, _, blob_v, _ = _store(200, 2, segs, 30)
    rng = np.random.default_rng(31)
    qb = oracle.f32_to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    o, lse = oracle.attention_rows_from_store(qb, np.arange(4), blob, blob_v, sc_hn, sc_hn_v,
                                              layout, 2, 200)
    for h in range(2):
        kr = oracle.decode_head(blob, sc_hn, layout, 2, h, 0, 200)
        vr = oracle.decode_head(blob_v, sc_hn_v, layout, 2, h, 0, 200)
        R = oracle.rotation_matrix()
        ref, lref = oracle.softmax_attention(oracle.bf16_bits_to_f64(qb[:, h * 128:(h + 1) * 128]),
                                             kr @ R.T, vr @ R.T, SCALE)
        assert np.allclose(o[:, h * 128:(h + 1) * 128], ref, rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[h], lref, rtol=1e-13)
