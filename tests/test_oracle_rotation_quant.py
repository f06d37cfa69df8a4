"""Pins of the oracle's rotation, quantiser and packing against closed forms,
brute force and invariants (CPU only)."""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import HEAD_DIM, INT4, INT8, QMAX


def popcount(x):
    return bin(x).count("1")


# ----------------------------------------------------------------------------- Hadamard
def test_hadamard_closed_form_entries():
    # Sylvester construction in natural order: H[i, j] = (-1)^popcount(i & j)
    H = oracle.hadamard_pm1(128)
    ref = np.array([[(-1) ** popcount(i & j) for j in range(128)] for i in range(128)])
    assert np.array_equal(H, ref)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_orthogonal_integer(n):
    H = oracle.hadamard_pm1(n)
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64))
    assert np.array_equal(H, H.T)


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard_pm1(96)


def test_rotate_one_hot_is_hadamard_row():
    for j in (0, 1, 5, 64, 127):
        e = np.zeros(128)
        e[j] = 1.0
        r = oracle.rotate(e)
        H = oracle.hadamard_pm1(128)
        assert np.array_equal(r, (H[j] / math.sqrt(128)).astype(np.float32))


def test_rotate_integer_input_exact():
    # integer input: u.H is an exact integer; r = fp32(u.H / sqrt(128))
    rng = np.random.default_rng(1)
    u = rng.integers(-50, 50, size=(16, 128)).astype(np.float64)
    H = oracle.hadamard_pm1(128)
    exact = (u.astype(np.int64) @ H).astype(np.float64) / math.sqrt(128)
    assert np.array_equal(oracle.rotate(u), exact.astype(np.float32))


def test_rotate_preserves_norm_and_is_involution():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((64, 128)) * 3
    r = oracle.rotate(u).astype(np.float64)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(u, axis=1), rtol=1e-6)
    back = oracle.rotate(r).astype(np.float64)
    assert np.allclose(back, u, rtol=0, atol=1e-5 * np.abs(u).max())


# ----------------------------------------------------------------------------- quantiser
def brute_force_codes(r_group, s16, qmax):
    """Nearest integer in [-qmax, qmax] to fp32(r / s) with ties to the even integer,
    found by scanning every candidate (independent of np.rint / np.clip)."""
    s = np.float32(s16)
    out = []
    for x in r_group:
        if s == 0:
            out.append(0)
            continue
        t = float(np.float32(np.float32(x) / s))
        best = None
        for c in range(-qmax, qmax + 1):
            d = abs(t - c)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        out.append(best[1])
    return np.array(out)


def scale_by_definition(a, qmax):
    """The group scale computed from the two rules' statements, independently of the
    oracle's bit-pattern code:
      INT4: the smallest number with 8 significant bits that is >= fp32(a / 7), as fp16
            (float64 arithmetic on exponent and step);
      INT8: the fp16 value nearest to t = fp32(a * fp32((1 + 2^-7) / 127)), ties to an
            even significand, found by scanning the fp16 grid around t ([VL] kvi8r
            `_Int8KV.store`)."""
    if qmax == QMAX[INT4]:
        t = float(np.float32(np.float32(a) / np.float32(qmax)))
        if t == 0.0:
            return np.float16(0.0)
        e = math.floor(math.log2(t))
        step = 2.0 ** (e - 8 + 1)
        return np.float16(math.ceil(t / step) * step)
    c8 = np.float32(129.0 / (127.0 * 128.0))
    t = float(np.float32(np.float32(a) * c8))
    if t == 0.0:
        return np.float16(0.0)
    e = max(math.floor(math.log2(t)), -14)        # fp16 binade (subnormals share -14)
    step = 2.0 ** (e - 10)
    lo = math.floor(t / step) * step
    cands = [lo, lo + step]
    best = min(cands, key=lambda v: (abs(v - t), (int(round(v / step)) & 1)))
    return np.float16(best)


def test_round_up_bits_examples():
    vals = np.array([1.0, 1.0 + 2 ** -20, 1.5, 1.00390625, 0.0, 3.0 * 2 ** -10], np.float32)
    got = oracle.round_up_bits(vals, 8)
    assert list(got) == [1.0, 1.0078125, 1.5, 1.0078125, 0.0, 3.0 * 2 ** -10]
    assert oracle.round_up_bits(np.float32(1.9999), 4) == 2.0
    assert oracle.round_up_bits(np.float32(1.0625), 4) == 1.125


def test_int8_scale_factor_is_the_pages_constant():
    # [VL] kvi8r `_Int8KV.store`: absmax * (1/127) * (1 + 2^-7), i.e. 129 / 16256, as the
    # fp32 value the page's fp32 tensor is multiplied by
    exact = 129.0 / 16256.0
    assert abs(float(oracle.INT8_SCALE_FACTOR) - exact) <= 2.0 ** -24 * exact
    assert oracle.INT8_SCALE_FACTOR.dtype == np.float32


def test_int8_worked_example_group_max_127():
    # A group whose largest magnitude is 127: the scale is 127 * 129/16256 = 1.0078125
    # (exact in fp16), so the largest element maps to round(127 / 1.0078125) = 126, not
    # 127 -- the enlargement keeps the row maximum inside the code range.  Dropping the
    # factor would give scale 1 and code 127.
    r = np.zeros((1, 128), np.float32)
    r[0, :32] = np.linspace(-127.0, 127.0, 32, dtype=np.float32)
    codes, scales = oracle.quantize_groups(r, QMAX[INT8])
    assert float(scales[0, 0]) == 1.0078125
    assert codes[0, 0] == -126 and codes[0, 31] == 126
    assert float(scales[0, 1]) == 0.0 and np.all(codes[0, 32:] == 0)


def test_int4_scale_keeps_8_bits_and_code_times_scale_is_exact_in_fp16():
    rng = np.random.default_rng(8)
    r = (rng.standard_normal((500, 128)) * rng.uniform(0.01, 50, size=(500, 1))).astype(np.float32)
    codes, scales = oracle.quantize_groups(r, QMAX[INT4])
    prod = codes.reshape(500, 4, 32).astype(np.float64) * scales.astype(np.float64)[..., None]
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)


def test_int8_scale_within_the_pages_factor():
    # fp32 product then fp16 rounding: s / (a / 127) lies within one fp16 half-step of
    # the page's factor (1 + 2^-7) for normal fp16 scales, so |r / s| < 127 always
    rng = np.random.default_rng(9)
    r = (rng.standard_normal((2000, 128)) * rng.uniform(0.05, 50, size=(2000, 1))).astype(np.float32)
    codes, scales = oracle.quantize_groups(r, QMAX[INT8])
    a = np.max(np.abs(r.reshape(2000, 4, 32)), axis=-1).astype(np.float64)
    ratio = scales.astype(np.float64) / (a / 127.0)
    f = 1.0 + 2.0 ** -7
    assert np.all(ratio >= f * (1 - 2.0 ** -11) * (1 - 2.0 ** -23))
    assert np.all(ratio <= f * (1 + 2.0 ** -11) * (1 + 2.0 ** -23))
    assert np.all(np.abs(codes.astype(np.int64)) <= 127)


@pytest.mark.parametrize("fmt", [INT4, INT8])
def test_quantizer_matches_brute_force(fmt):
    qmax = QMAX[fmt]
    rng = np.random.default_rng(3 + fmt)
    r = (rng.standard_normal((6, 128)) * rng.uniform(0.01, 5, size=(6, 1))).astype(np.float32)
    r[5] *= 1e-4                                    # small scales (subnormal fp16 for INT8)
    codes, scales = oracle.quantize_groups(r, qmax)
    assert codes.dtype == np.int8 and scales.dtype == np.float16
    for row in range(r.shape[0]):
        for g in range(4):
            grp = r[row, 32 * g:32 * g + 32]
            a = float(np.max(np.abs(grp)))
            s16 = scale_by_definition(a, qmax)
            assert scales[row, g] == s16, (fmt, row, g, float(scales[row, g]), float(s16))
            assert np.array_equal(codes[row, 32 * g:32 * g + 32], brute_force_codes(grp, s16, qmax))


@pytest.mark.parametrize("fmt", [INT4, INT8])
def test_dequant_error_at_most_half_scale(fmt):
    qmax = QMAX[fmt]
    rng = np.random.default_rng(5)
    r = (rng.standard_normal((256, 128)) * 2).astype(np.float32)
    codes, scales = oracle.quantize_groups(r, qmax)
    assert np.all(np.abs(scales.astype(np.float64)) >= 6.103515625e-05)  # normal fp16 scales
    deq = oracle.dequantize(codes, scales)
    s = np.repeat(scales.astype(np.float64), 32, axis=-1)
    assert np.all(np.abs(deq - r) <= s / 2 + 1e-12)


def test_absmax_element_maps_to_qmax():
    rng = np.random.default_rng(6)
    r = (rng.standard_normal((64, 128))).astype(np.float32)
    for fmt, lo in ((INT4, 7), (INT8, 126)):
        codes, _ = oracle.quantize_groups(r, QMAX[fmt])
        g = r.reshape(64, 4, 32)
        c = codes.reshape(64, 4, 32)
        idx = np.argmax(np.abs(g), axis=-1)
        top = np.take_along_axis(c, idx[..., None], -1)[..., 0]
        # INT4: the 8-bit round-up moves a / s by less than 2^-7, so the top code is 7;
        # INT8: the page's (1 + 2^-7) enlargement puts the top element at 126 or 127
        assert np.all(np.abs(top) <= QMAX[fmt]) and np.all(np.abs(top) >= lo)


def test_quantisation_error_of_each_scale_rule_against_unquantised_rows():
    # rms error of the dequantised rows against the unquantised rotated rows, for the
    # rules in the oracle and two alternatives: the unrounded scale a / qmax (the floor
    # any fp16 rule sits on) and, for INT8, a scale grid of 4 significant bits.  The
    # page's INT8 rule stays within 1% of the floor; a 4-bit grid costs >= 4% more.
    rng = np.random.default_rng(12)
    u = rng.standard_normal((20000, 128))
    r = oracle.rotate(u)
    g = r.reshape(-1, 4, 32).astype(np.float64)
    a = np.max(np.abs(g), axis=-1)

    def rms(scale, qmax):
        s = np.where(scale == 0, 1.0, scale)[..., None]
        c = np.clip(np.rint(g / s), -qmax, qmax)
        return float(np.sqrt(np.mean((c * s - g) ** 2)))

    for fmt in (INT4, INT8):
        qmax = QMAX[fmt]
        codes, scales = oracle.quantize_groups(r, qmax)
        err = float(np.sqrt(np.mean((oracle.dequantize(codes, scales) - r.astype(np.float64)) ** 2)))
        floor = rms(a / qmax, qmax)
        assert floor <= err <= 1.01 * floor, (fmt, err, floor)
    grid4 = oracle.round_up_bits((a / 127.0).astype(np.float32), 4).astype(np.float16).astype(np.float64)
    codes, scales = oracle.quantize_groups(r, 127)
    page = float(np.sqrt(np.mean((oracle.dequantize(codes, scales) - r.astype(np.float64)) ** 2)))
    assert rms(grid4, 127) >= 1.04 * page


def test_one_hot_vector_codes_follow_hadamard_signs():
    # a one-hot k rotates to +-1/sqrt(128) everywhere: every INT4 code is +-7 with the
    # sign of Hadamard row j, and every scale is fp16(fp32(1/sqrt(128)) / 7)
    H = oracle.hadamard_pm1(128)
    for j in (0, 3, 77):
        e = np.zeros((1, 128))
        e[0, j] = 1.0
        r = oracle.rotate(e)
        codes, scales = oracle.quantize_groups(r, 7)
        assert np.array_equal(codes[0], 7 * H[j])
        expect = scale_by_definition(np.float32(1 / math.sqrt(128)), 7)
        assert np.all(scales == expect)


def test_zero_group_gives_zero_codes_and_scale():
    r = np.zeros((2, 128), dtype=np.float32)
    r[1, 40] = 3.0  # groups 0, 2, 3 of row 1 stay zero
    codes, scales = oracle.quantize_groups(r, 7)
    assert np.all(codes[0] == 0) and np.all(scales[0] == 0)
    assert scales[1, 1] != 0 and np.all(scales[1, [0, 2, 3]] == 0)
    assert np.all(codes[1, :32] == 0) and codes[1, 40] == 7


def test_exact_ties_round_to_even():
    # r = (k + 1/2) * s exactly, s a power of two: ties go to the even integer
    s = np.float32(0.25)
    r = np.zeros((1, 128), dtype=np.float32)
    halves = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, -3.5]
    r[0, :8] = np.array(halves, dtype=np.float32) * s
    r[0, 8] = 7 * s  # absmax 1.75 -> scale 1.75 / 7 = 0.25 exactly
    codes, scales = oracle.quantize_groups(r, 7)
    assert scales[0, 0] == np.float16(0.25)
    assert list(codes[0, :8]) == [0, 2, 2, 0, -2, -2, 4, -4]


def test_int4_never_reaches_minus_eight_for_normal_scales():
    # the scale is rounded up from a/7, so |r/s| <= 7: the pages' [-8, 7] clamp and the
    # symmetric [-7, 7] clamp agree
    rng = np.random.default_rng(7)
    r = (rng.standard_normal((2000, 128)) * rng.uniform(0.01, 100, size=(2000, 1))).astype(np.float32)
    g = r.reshape(-1, 4, 32)
    a = np.max(np.abs(g), axis=-1)
    _, s = oracle.quantize_groups(r, 7)
    t = g / s.astype(np.float32)[..., None]
    assert np.max(np.abs(t)) <= 7.0


# ----------------------------------------------------------------------------- packing
def test_pack_known_bytes():
    c = np.zeros(128, dtype=np.int8)
    c[0], c[1] = -1, 3      # 0xF | 0x3 << 4
    c[2], c[3] = 7, -8      # 0x7 | 0x8 << 4
    c[4], c[5] = -7, 1      # 0x9 | 0x1 << 4
    p = oracle.pack_int4(c)
    assert p.shape == (64,)
    assert (p[0], p[1], p[2], p[3]) == (0x3F, 0x87, 0x19, 0x00)


def test_pack_unpack_all_nibble_pairs():
    pairs = np.array(list(itertools.product(range(-8, 8), repeat=2)), dtype=np.int8)  # 256 pairs
    codes = pairs.reshape(-1, 128)
    packed = oracle.pack_int4(codes)
    assert sorted(set(packed.reshape(-1).tolist())) == list(range(256))
    assert np.array_equal(oracle.unpack_int4(packed), codes)


def test_unpack_pack_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(4, 64)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(b)), b)
    assert np.array_equal(oracle.pack_codes(oracle.unpack_codes(b, INT8), INT8), b)


def test_int8_codes_twos_complement():
    c = np.array([-128, -127, -1, 0, 1, 127] + [0] * 122, dtype=np.int8)
    assert list(oracle.pack_codes(c, INT8)[:6]) == [0x80, 0x81, 0xFF, 0x00, 0x01, 0x7F]


# ----------------------------------------------------------------------------- rounding helpers
def test_bf16_rounding_ties_and_values():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    bits = oracle.f32_to_bf16_bits(vals)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0])


def test_f16_rounding_is_nearest_even():
    x = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 6.1e-5, 65504.0], dtype=np.float32)
    y = oracle.f32_to_f16(x)
    assert y[0] == np.float16(1.0) and y[1] == np.float16(1 + 2 ** -9)
    assert y[3] == np.float16(65504.0)
