"""Pins of the oracle's richer precision policy: BF16 ranges ([FR] "Mixed precision
for conditioning": conditioning ranges at BF16 or INT8) and INT8 heads inside INT4
ranges ([VL] kvmix section: a per-head 4/8-bit split).  Each test checks the oracle
against a property the mathematics fixes, not against a retyped formula."""
import numpy as np
import pytest

import oracle
import synth
from oracle import BF16, INT4, INT8

POLICY = [(0, 256, BF16), (256, 640, INT8), (640, 1536, INT4, 0b100101), (1536, 2000, BF16)]


def _rows(n, d, seed, fmts, positions=None):
    x = synth.make_x(n, d, 0.01, seed=seed)
    w = synth.make_w(d, seed=seed + 1)
    xb, wb = synth.bf16_bits(x), synth.bf16_bits(w)
    pos = np.arange(n) if positions is None else positions
    return oracle.qkv_quant_rows(xb, wb, d // 128, pos, fmts), xb, wb


def test_layout_rows_tile_the_buffer_exactly():
    # every (segment, head, token) row owns its bytes: the rows cover [0, total) once
    H, n = 6, 2000
    segs = oracle.range_segments(n, POLICY, n_heads=H)
    layout, total = oracle.packed_layout(n, H, segs)
    owner = np.zeros(total, np.int64)
    for seg in layout:
        for h in range(H):
            rb = seg["head_row_bytes"][h]
            for t in range(seg["begin"], seg["end"]):
                a = seg["head_offset"][h] + (t - seg["begin"]) * rb
                owner[a:a + rb] += 1
    assert np.all(owner == 1)
    # closed form of the total: heads 0, 2, 5 of the INT4 range take 128 B per row
    want = (256 + 464) * H * 256 + 384 * H * 128 + 896 * (3 * 128 + 3 * 64)
    assert total == want


def test_head_formats_follow_the_mask():
    fm = oracle.head_formats(2000, 6, oracle.range_segments(2000, POLICY))
    assert np.all(fm[:256] == BF16) and np.all(fm[256:640] == INT8) and np.all(fm[1536:] == BF16)
    assert list(fm[700]) == [INT8, INT4, INT8, INT4, INT4, INT8]


def test_bf16_rows_hold_the_rotated_vector():
    # rotating a BF16 row back gives the model-basis k within bf16 rounding: each
    # rotated value is off by at most 2^-9 of itself, and the rotation keeps norms
    n, d = 24, 256
    ref, xb, wb = _rows(n, d, 401, np.full(n, BF16))
    y = oracle.project(xb, wb)
    _, k, v = oracle.split_heads(y, d // 128)
    R = oracle.rotation_matrix()
    for name, model in (("k", k), ("v", v)):
        back = oracle.bf16_bits_to_f64(ref[name + "_bf16"]) @ R.T
        err = np.linalg.norm(back - model, axis=-1)
        assert np.all(err <= 2.0 ** -8 * np.linalg.norm(model, axis=-1))
        assert np.all(ref[name + "_codes"] == 0) and np.all(ref[name + "_scales"] == 0)


def test_int8_heads_match_an_int8_range():
    # a masked head of an INT4 range is quantised exactly as an INT8 range would be,
    # the other heads exactly as INT4
    n, d = 16, 512
    mask = 0b0101
    fm = np.array([[INT8 if (mask >> h) & 1 else INT4 for h in range(4)]] * n)
    mixed, _, _ = _rows(n, d, 411, fm)
    all8, _, _ = _rows(n, d, 411, np.full(n, INT8))
    all4, _, _ = _rows(n, d, 411, np.full(n, INT4))
    for h in range(4):
        src = all8 if (mask >> h) & 1 else all4
        for key in ("k_codes", "k_scales", "v_codes", "v_scales"):
            assert np.array_equal(mixed[key][:, h], src[key][:, h]), (key, h)


def _mixed_store(n, H, segs, seed):
    """Random rotated rows laid out by oracle.packed_layout under a mixed policy."""
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal((n, H, 128)) * 2).astype(np.float32)
    fm = oracle.head_formats(n, H, segs)
    layout, total = oracle.packed_layout(n, H, segs)
    blob = np.zeros(total, np.uint8)
    scales = np.zeros((n, H, 4), np.float16)
    for seg in layout:
        b, e = seg["begin"], seg["end"]
        for h in range(H):
            f, rb, off = seg["head_fmt"][h], seg["head_row_bytes"][h], seg["head_offset"][h]
            if f == BF16:
                rows = oracle.f32_to_bf16_bits(r[b:e, h]).view(np.uint8)
            else:
                c, s = oracle.quantize_groups(r[b:e, h], oracle.QMAX[f])
                scales[b:e, h] = s
                rows = oracle.pack_codes(c, f)
            blob[off:off + (e - b) * rb] = np.ascontiguousarray(rows).reshape(-1)
    return r, fm, layout, blob, np.ascontiguousarray(scales.transpose(1, 0, 2))


def test_decode_under_a_mixed_policy():
    n, H = 2000, 6
    segs = oracle.range_segments(n, POLICY, n_heads=H)
    r, fm, layout, blob, sc = _mixed_store(n, H, segs, 421)
    rows = np.array([0, 255, 256, 639, 640, 1000, 1535, 1536, 1999])
    bits = oracle.gather_bf16_rows(blob, layout, H, rows)
    codes, _ = oracle.gather_packed_rows(blob, sc, layout, H, rows)
    for h in range(H):
        dec = oracle.decode_head(blob, sc, layout, H, h, 0, n)
        err = np.abs(dec - r[:, h].astype(np.float64))
        for f, bound in ((BF16, 2.0 ** -8), (INT8, 1.0 / 127), (INT4, 1.0 / 7)):
            sel = fm[:, h] == f
            if not sel.any():
                continue
            amax = np.abs(r[sel, h]).max()
            assert err[sel].max() <= bound * amax, (h, f)
        bf_rows = fm[rows, h] == BF16
        assert np.array_equal(oracle.bf16_bits_to_f64(bits[bf_rows, h]), dec[rows[bf_rows]])
        assert np.all(bits[~bf_rows, h] == 0) and np.all(codes[bf_rows, h] == 0)


def test_attention_error_orders_with_precision():
    # the same keys and values at BF16, INT8 and INT4: the attention error against the
    # unquantised rows shrinks with the precision
    n, H = 512, 1
    rng = np.random.default_rng(431)
    qb = oracle.f32_to_bf16_bits(rng.standard_normal((8, 128)).astype(np.float32))
    errs = {}
    for f in (BF16, INT8, INT4):
        segs = oracle.range_segments(n, [(0, n, f)])
        r, _, layout, blob, sc = _mixed_store(n, H, segs, 432)
        rv, _, _, blob_v, sc_v = _mixed_store(n, H, segs, 433)
        o, _ = oracle.attention_rows_from_store(qb, np.arange(8), blob, blob_v, sc, sc_v, layout, H, n)
        R = oracle.rotation_matrix()
        ref, _ = oracle.softmax_attention(oracle.bf16_bits_to_f64(qb), r[:, 0].astype(np.float64) @ R.T,
                                          rv[:, 0].astype(np.float64) @ R.T, 128 ** -0.5)
        errs[f] = np.linalg.norm(o - ref) / np.linalg.norm(ref)
    assert errs[BF16] < errs[INT8] < errs[INT4]
    assert errs[BF16] < 1e-2


@pytest.mark.parametrize("ranges", [
    [(0, 512, INT8, 1), (512, 1024, INT4)],
    [(0, 512, BF16, 2), (512, 1024, INT4)],
    [(0, 512, 3), (512, 1024, INT4)],
])
def test_bad_mixed_policies_rejected(ranges):
    with pytest.raises(ValueError):
        oracle.range_segments(1024, ranges, n_heads=4)
