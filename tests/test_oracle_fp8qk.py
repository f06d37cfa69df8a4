"""Pins of the oracle's low-precision QK^T tier: OCP FP8 E4M3 rounding, the E8M0 block
exponent, block quantisation, and attention with scores on block-scaled fp8 operands
([VL] kvi8s section: an approximation tier with Hadamard-rotated Q and K and QK^T on
low-precision tensor cores).  The E4M3 values come from the format's definition
(bias 7, 3 mantissa bits, largest finite 448, subnormal step 2^-9)."""
import numpy as np
import pytest

import oracle

SCALE = 128 ** -0.5


@pytest.mark.parametrize("x,code", [
    (0.0, 0x00), (1.0, 0x38), (-1.5, 0xBC), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -6, 0x08),
    (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (240.0, 0x77), (0.1015625, 0x1D),
    # ties go to the even mantissa
    (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
    (1.9375, 0x40),                       # carries into the next binade (2.0)
    (464.0, 0x7E), (1e6, 0x7E),           # beyond 448: saturate
])
def test_e4m3_known_codes(x, code):
    assert int(oracle.f32_to_e4m3(np.float32(x))) == code


def test_e4m3_every_code_round_trips_and_orders():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_to_f64(c)
    ok = ~np.isnan(v)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and ok.sum() == 254
    assert np.array_equal(oracle.f32_to_e4m3(v[ok]), c[ok])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0          # codes 0..0x7e ascend


def test_e4m3_rounds_to_the_nearest_value():
    rng = np.random.default_rng(601)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 9, 20000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = oracle.e4m3_to_f64(oracle.f32_to_e4m3(x))
    grid = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    grid = np.concatenate([-grid[::-1], grid])
    nearest = np.min(np.abs(x.astype(np.float64)[:, None] - grid[None, :]), axis=1)
    assert np.allclose(np.abs(got - x), nearest, rtol=0, atol=0)


def test_e8m0_exponent_puts_the_block_max_in_the_top_binade():
    rng = np.random.default_rng(602)
    a = np.exp2(rng.uniform(-60, 60, 5000))
    e = oracle.e8m0_exponent(a)
    r = a / np.exp2(e)
    assert np.all(r <= 448.0) and np.all(r > 224.0)
    assert oracle.e8m0_exponent(448.0) == 0 and oracle.e8m0_exponent(448.5) == 1
    assert oracle.e8m0_exponent(224.0) == -1 and oracle.e8m0_exponent(0.0) == -127


def test_block_quantisation_error_bound():
    # E4M3 keeps 4 significant bits: each value is within 2^-4 of itself, or within
    # half the subnormal step 2^-10 * 2^e of the group
    rng = np.random.default_rng(603)
    r = (rng.standard_normal((64, 128)) * np.exp2(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    codes, e = oracle.fp8_block_quantize(r)
    d = oracle.fp8_block_dequantize(codes, e)
    floor = np.repeat(np.exp2(e.astype(np.float64) - 10), 32, axis=-1)
    assert np.all(np.abs(d - r) <= np.abs(r) * 2.0 ** -4 + floor)
    g = np.abs(r).reshape(64, 4, 32).max(-1)
    assert np.all(g / np.exp2(e) <= 448) and np.all(g / np.exp2(e) > 224)


def _representable(rng, shape):
    """Rotated vectors whose groups quantise without loss: every group holds an
    exact E4M3 value times 2^e and its largest magnitude in (224, 448] * 2^e."""
    codes = rng.integers(0, 0x7F, size=shape).astype(np.uint8)
    codes = np.where(rng.random(shape) < 0.5, codes | 0x80, codes).astype(np.uint8)
    g = codes.reshape(shape[:-1] + (4, 32))
    g[..., 0] = 0x7A                      # 320: puts the group maximum in the top binade
    e = rng.integers(-12, -6, size=shape[:-1] + (4,))
    return oracle.fp8_block_dequantize(g.reshape(shape), e)


def test_fp8_scores_are_exact_when_operands_are_representable():
    rng = np.random.default_rng(604)
    q = _representable(rng, (6, 128))
    k = _representable(rng, (90, 128))
    v = rng.standard_normal((90, 128))
    o8, l8 = oracle.attention_fp8qk_rotated(q.astype(np.float32), k, v, SCALE * 0.05)
    o, l = oracle.softmax_attention(q, k, v, SCALE * 0.05)
    assert np.allclose(o8, o, rtol=0, atol=1e-12) and np.allclose(l8, l, rtol=0, atol=1e-12)
    o8b, l8b = oracle.attention_fp8qk_rotated(q.astype(np.float32), k, v, SCALE * 0.05, kv_block=32)
    assert np.allclose(o8b, o, rtol=0, atol=1e-11) and np.allclose(l8b, l, rtol=0, atol=1e-12)


def test_fp8_scores_cost_bounded_accuracy():
    # on random rotated data the fp8 scores move the output, but by far less than the
    # output itself (4-bit significands, errors averaging over 128 dims)
    rng = np.random.default_rng(605)
    q = rng.standard_normal((16, 128)).astype(np.float32) * 2
    k = rng.standard_normal((300, 128)) * 2
    v = rng.standard_normal((300, 128))
    o8, _ = oracle.attention_fp8qk_rotated(q, k, v, SCALE)
    o, _ = oracle.softmax_attention(q.astype(np.float64), k, v, SCALE)
    rel = np.linalg.norm(o8 - o) / np.linalg.norm(o)
    assert 1e-3 < rel < 0.1
