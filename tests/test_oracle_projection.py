"""Pins of the oracle's projection, RMSNorm, RoPE and end-to-end QKV-quant rows
(CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import HEAD_DIM, INT4, INT8


def test_projection_integer_inputs_exact():
    # integer-valued bf16 x and W: the product is an exact integer matrix
    x = synth.make_integer_x(64, 512, seed=11)
    w = synth.make_integer_w(512, seed=12)
    y = oracle.project(synth.bf16_bits(x), synth.bf16_bits(w))
    ref = x.to(torch.int64) @ w.to(torch.int64)
    assert np.array_equal(y, ref.numpy().astype(np.float64))


def test_projection_matches_library_matmul():
    x = synth.make_bf16_matrix(32, 256, seed=13)
    w = synth.make_bf16_matrix(256, 768, seed=14, std=1 / 16)
    y = oracle.project(synth.bf16_bits(x), synth.bf16_bits(w))
    ref = x.double() @ w.double()
    assert np.allclose(y, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_projection_row_chunking_is_exact():
    x = synth.make_bf16_matrix(100, 256, seed=15)
    w = synth.make_bf16_matrix(256, 768, seed=16, std=1 / 16)
    xb, wb = synth.bf16_bits(x), synth.bf16_bits(w)
    full = oracle.project(xb, wb)
    parts = np.concatenate([oracle.project(xb[a:b], wb) for a, b in oracle.chunk_ranges(100, 32, 8)])
    assert np.array_equal(full, parts)


def test_split_heads_column_order():
    H = 3
    d = H * HEAD_DIM
    y = np.arange(2 * 3 * d, dtype=np.float64).reshape(2, 3 * d)
    q, k, v = oracle.split_heads(y, H)
    assert q[1, 2, 5] == y[1, 2 * HEAD_DIM + 5]
    assert k[0, 1, 0] == y[0, d + HEAD_DIM]
    assert v[1, 0, 127] == y[1, 2 * d + 127]


# ----------------------------------------------------------------------------- RMSNorm
def test_rms_norm_unit_weight_gives_unit_rms():
    rng = np.random.default_rng(20)
    u = rng.standard_normal((10, 4, 128)) * 7
    out = oracle.rms_norm(u, np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, rtol=1e-12)


def test_rms_norm_closed_form_small():
    # u = (3, 4, 0, ..., 0): mean(u^2) = 25/128, so out = u * sqrt(128/25) * w
    u = np.zeros(128)
    u[0], u[1] = 3.0, 4.0
    w = np.full(128, 2.0)
    out = oracle.rms_norm(u, w, 0.0)
    f = math.sqrt(128 / 25) * 2.0
    assert math.isclose(out[0], 3 * f, rel_tol=1e-14) and math.isclose(out[1], 4 * f, rel_tol=1e-14)
    # eps enters under the root
    out2 = oracle.rms_norm(u, np.ones(128), 1.0)
    assert math.isclose(out2[0], 3 / math.sqrt(25 / 128 + 1.0), rel_tol=1e-14)


# ----------------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(21)
    u = rng.standard_normal((1, 2, 128))
    c, s = oracle.rope_angles(np.array([0]))
    assert np.array_equal(oracle.rope_split_half(u, c, s), u)


def test_rope_hand_computed_pair():
    # pair (0, 64) at position 1 rotates by exactly 1 radian (inv_freq_0 = 1);
    # pair (1, 65) by theta^(-2/128) radians
    u = np.zeros((1, 1, 128))
    u[0, 0, 0], u[0, 0, 64] = 1.0, 2.0
    u[0, 0, 1], u[0, 0, 65] = -1.0, 0.5
    c, s = oracle.rope_angles(np.array([1]), theta=10000.0)
    out = oracle.rope_split_half(u, c, s)
    assert math.isclose(out[0, 0, 0], math.cos(1) - 2 * math.sin(1), rel_tol=1e-14)
    assert math.isclose(out[0, 0, 64], 2 * math.cos(1) + math.sin(1), rel_tol=1e-14)
    a1 = 10000.0 ** (-2 / 128)
    assert math.isclose(out[0, 0, 1], -math.cos(a1) - 0.5 * math.sin(a1), rel_tol=1e-13)
    assert math.isclose(out[0, 0, 65], 0.5 * math.cos(a1) - math.sin(a1), rel_tol=1e-13)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(22)
    u = rng.standard_normal((5, 3, 128))
    pos = np.array([0, 1, 1000, 150000, 217087])
    c, s = oracle.rope_angles(pos)
    out = oracle.rope_split_half(u, c, s)
    n_in = u[..., :64] ** 2 + u[..., 64:] ** 2
    n_out = out[..., :64] ** 2 + out[..., 64:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))

    def score(pq, pk):
        cq, sq = oracle.rope_angles(np.array([pq]))
        ck, sk = oracle.rope_angles(np.array([pk]))
        return float(np.sum(oracle.rope_split_half(q, cq, sq) * oracle.rope_split_half(k, ck, sk)))

    base = score(10, 3)
    for shift in (1, 77, 5000):
        assert math.isclose(score(10 + shift, 3 + shift), base, rel_tol=1e-9, abs_tol=1e-9)
    assert not math.isclose(score(11, 3), base, rel_tol=1e-6)


# ----------------------------------------------------------------------------- QKV-quant rows
def _tiny_problem(n=48, d=256, seed=30):
    x = synth.make_x(n, d, 0.02, seed=seed)
    w = synth.make_w(d, seed=seed + 1)
    return synth.bf16_bits(x), synth.bf16_bits(w), x, w


def test_qkv_rows_q_is_bf16_of_projection():
    xb, wb, x, w = _tiny_problem()
    H = 2
    out = oracle.qkv_quant_rows(xb, wb, H, np.arange(48), np.zeros(48, np.int64))
    y = (x.double() @ w.double()).float()
    q_ref = y[:, :H * HEAD_DIM].to(torch.bfloat16)
    assert np.array_equal(out["q_bits"], synth.bf16_bits(q_ref))


def test_qkv_rows_kv_codes_reconstruct_projection():
    xb, wb, x, w = _tiny_problem()
    H = 2
    fm = np.where(np.arange(48) < 16, INT8, INT4)
    out = oracle.qkv_quant_rows(xb, wb, H, np.arange(48), fm)
    y = x.double() @ w.double()
    R = oracle.rotation_matrix()
    for name, col0 in (("k", H * HEAD_DIM), ("v", 2 * H * HEAD_DIM)):
        u = y[:, col0:col0 + H * HEAD_DIM].numpy().reshape(48, H, HEAD_DIM)
        deq = oracle.dequantize(out[name + "_codes"], out[name + "_scales"])
        back = deq @ R.T  # rotate back to the model basis
        s = np.repeat(out[name + "_scales"].astype(np.float64), 32, axis=-1)
        # each rotated element is within half a step; the rotation keeps the L2 error
        err = np.linalg.norm(back - u, axis=-1)
        bound = np.sqrt(np.sum((s / 2) ** 2, axis=-1)) + 1e-6 * np.linalg.norm(u, axis=-1)
        assert np.all(err <= bound)
        # INT8 rows are ~16x finer than INT4 rows
        assert np.median(err[:16]) < np.median(err[16:]) / 8


def test_qkv_rows_norm_rope_path():
    xb, wb, x, w = _tiny_problem()
    H = 2
    qn = np.ones(128)
    kn = np.ones(128)
    pos = np.zeros(48)
    out = oracle.qkv_quant_rows(xb, wb, H, pos, np.zeros(48, np.int64), q_norm_w=qn, k_norm_w=kn,
                                eps=0.0, rope_theta=10000.0)
    y = x.double() @ w.double()
    q = y[:, :H * HEAD_DIM].numpy().reshape(48, H, HEAD_DIM)
    qn_ref = q / np.sqrt(np.mean(q ** 2, axis=-1, keepdims=True))
    got = oracle.bf16_bits_to_f64(out["q_bits"]).reshape(48, H, HEAD_DIM)
    assert np.allclose(got, qn_ref, rtol=2 ** -8, atol=0)
    kr = out["k_rot_f32"].astype(np.float64)
    assert np.allclose(np.sqrt(np.mean(kr ** 2, axis=-1)), 1.0, rtol=1e-6)


def test_qkv_rows_independent_of_row_subset():
    xb, wb, _, _ = _tiny_problem()
    full = oracle.qkv_quant_rows(xb, wb, 2, np.arange(48), np.zeros(48, np.int64))
    rows = np.array([0, 7, 47])
    part = oracle.qkv_quant_rows(xb[rows], wb, 2, rows, np.zeros(3, np.int64))
    for key in ("q_bits", "k_codes", "k_scales", "v_codes", "v_scales"):
        assert np.array_equal(full[key][rows], part[key])
