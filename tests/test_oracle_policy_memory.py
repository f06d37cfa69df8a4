"""Pins of the oracle's chunk plan, range policy and working-set closed forms,
including the memory figures printed on the pages (tests/golden)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import INT4, INT8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GIB = float(1 << 30)


# ----------------------------------------------------------------------------- chunk plan
def test_chunk_ranges_odd_sequence():
    # 152,263 rows in 8192-row chunks: 18 full chunks and a 4,807-row tail (>= 512: kept)
    r = oracle.chunk_ranges(152263, 8192, 512)
    assert len(r) == 19
    assert r[-1] == (147456, 152263) and r[-1][1] - r[-1][0] == 4807
    assert all(b - a == 8192 for a, b in r[:-1])


def test_chunk_ranges_folds_short_tail():
    assert oracle.chunk_ranges(16484, 8192, 512) == [(0, 8192), (8192, 16484)]
    assert oracle.chunk_ranges(16384 + 511, 8192, 512) == [(0, 8192), (8192, 16895)]
    assert oracle.chunk_ranges(16384 + 512, 8192, 512) == [(0, 8192), (8192, 16384), (16384, 16896)]


@pytest.mark.parametrize("n,size", [(1000, 0), (1000, -5), (1000, 1000), (1000, 5000), (0, 16)])
def test_chunk_ranges_single_chunk(n, size):
    assert oracle.chunk_ranges(n, size) == [(0, n)]


def test_chunk_ranges_cover_in_order():
    rng = np.random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(1, 5000))
        size = int(rng.integers(1, 2000))
        tail = int(rng.integers(0, 700))
        r = oracle.chunk_ranges(n, size, tail)
        assert r[0][0] == 0 and r[-1][1] == n
        assert all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1))
        if len(r) > 1:
            assert r[-1][1] - r[-1][0] >= min(tail, size)
            assert all(b - a == size for a, b in r[:-1])


# ----------------------------------------------------------------------------- range policy
def test_range_policy_valid_mixed():
    segs = oracle.range_segments(65536, [(0, 512, INT8), (512, 8704, INT8), (8704, 65536, INT4)])
    fm = oracle.token_formats(65536, segs)
    assert fm[511] == INT8 and fm[8703] == INT8 and fm[8704] == INT4 and fm[-1] == INT4


def test_range_policy_default_is_int4():
    assert oracle.range_segments(100, None) == [(0, 100, INT4)]


@pytest.mark.parametrize("ranges", [
    [(0, 512, INT8), (640, 1024, INT4)],            # gap
    [(0, 640, INT8), (512, 1024, INT4)],            # overlap
    [(0, 500, INT8), (500, 1024, INT4)],            # interior boundary not a multiple of 128
    [(0, 512, 7), (512, 1024, INT4)],               # unknown format
    [(0, 512, INT8), (512, 1000, INT4)],            # does not reach n
    [(128, 1024, INT4)],                            # does not start at 0
    [(0, 0, INT8), (0, 1024, INT4)],                # empty range
])
def test_range_policy_rejects(ranges):
    with pytest.raises(ValueError):
        oracle.range_segments(1024, ranges)


# ----------------------------------------------------------------------------- working set
def test_working_set_closed_forms():
    ws = oracle.working_set_bytes(152263, 7168, [(0, 152263, INT4)])
    assert ws["bf16_qkv"] == 152263 * 3 * 7168 * 2
    assert ws["q"] == 152263 * 7168 * 2
    assert ws["k_codes"] == 152263 * 56 * 64
    assert ws["k_scales"] == 152263 * 56 * 4 * 2
    ratio = ws["packed_total"] / ws["bf16_qkv"]
    assert abs(ratio - (2 + 1 + 1 / 8) / 6) < 1e-12   # 0.5208: below the 0.55 target


def test_working_set_mixed_policy_ratio():
    segs = [(0, 512, INT8), (512, 8704, INT8), (8704, 65536, INT4)]
    ws = oracle.working_set_bytes(65536, 7168, segs)
    assert 0.54 < ws["packed_total"] / ws["bf16_qkv"] < 0.545


def test_page_memory_figures():
    with open(os.path.join(GOLDEN, "page_memory_figures.json")) as f:
        data = json.load(f)
    for e in data["entries"]:
        ws = oracle.working_set_bytes(e["n_tokens"], e["d_model"], [(0, e["n_tokens"], INT4)])
        got = sum(ws[k] for k in e["quantity"].split("+")) / GIB
        assert abs(got - e["gib"]) <= e["rel_tol"] * e["gib"], (e["cite"], e["what"], got)
