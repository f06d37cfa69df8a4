"""Seeded synthetic inputs for the streamed QKV-quant + packed-K/V attention path.

This module is shared by the tests, the smoke check and the benchmark, and feeds
both the HIP path and the CPU oracle.  It holds no arithmetic of the method: only
random draws, the shapes of the five workloads, and the token-range policies they
name.  Every draw is seeded; the same call on the same device gives the same bytes.

Workload shapes follow the pages' MiniMax-H3 example: d_model = 7168 = 56 heads x
128 (VRAM Lab module, docstring and kvi8r section), packed sequences of ~152k and
~217k tokens (feature request "Streamed QKV Projection and Packed Low-Bit K/V
Support...", section "Example: MiniMax H3"; VRAM Lab docstring), and a packed
text / reference / generated layout whose leading ranges keep 8-bit K/V
(feature request, section "Mixed precision for conditioning").  The pages' own
captured activations are not available; these Gaussian inputs with outlier
channels stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import torch

INT4 = 0
INT8 = 1

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    d_model: int
    outlier_frac: float
    # half-open token ranges (begin, end, fmt); None means one INT4 range over [0, N)
    ranges: Optional[Tuple[Tuple[int, int, int], ...]]
    chunk_rows: int          # 0: one launch over all rows
    kv_block: int            # 0: single-pass attention; >0: KV blocks merged by log-sum-exp
    norm_rope: bool          # per-head RMSNorm on q,k then split-half RoPE before rotation
    seed_base: int

    @property
    def n_heads(self) -> int:
        return self.d_model // HEAD_DIM

    def range_list(self) -> List[Tuple[int, int, int]]:
        if self.ranges is None:
            return [(0, self.n_tokens, INT4)]
        return [tuple(r) for r in self.ranges]

    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.d_model))


WORKLOADS = {
    "tiny_1k": Workload("tiny_1k", 1024, 512, 0.01, None, 0, 0, False, 1000),
    "h3_16k": Workload("h3_16k", 16384, 7168, 0.005, None, 4096, 0, False, 2000),
    "h3_64k_mixed": Workload(
        "h3_64k_mixed", 65536, 7168, 0.005,
        ((0, 512, INT8), (512, 8704, INT8), (8704, 65536, INT4)),
        16384, 0, False, 3000),
    "h3_152k_odd": Workload("h3_152k_odd", 152263, 7168, 0.005, None, 8192, 0, False, 4000),
    "h3_217k_normrope": Workload("h3_217k_normrope", 217088, 7168, 0.01, None, 16384, 16384,
                                 True, 5000),
}

# order of the workloads as listed in the benchmark definition
WORKLOAD_ORDER = ["tiny_1k", "h3_16k", "h3_64k_mixed", "h3_152k_odd", "h3_217k_normrope"]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def outlier_channels(d_model: int, count: int, seed: int) -> torch.Tensor:
    """`count` distinct channel indices drawn without replacement (CPU generator)."""
    g = _gen(seed, "cpu")
    return torch.randperm(d_model, generator=g)[:count].sort().values


def make_x(n_tokens: int, d_model: int, outlier_frac: float, seed: int, device="cpu",
           outlier_seed: Optional[int] = None, outlier_gain: float = 20.0,
           block_rows: int = 16384) -> torch.Tensor:
    """Hidden states x [N, d] bf16: N(0,1) draws with a seeded set of outlier
    channels multiplied by `outlier_gain` before the bf16 cast (round to nearest even)."""
    if outlier_seed is None:
        outlier_seed = seed + 2
    count = int(round(outlier_frac * d_model))
    cols = outlier_channels(d_model, count, outlier_seed).to(device)
    out = torch.empty((n_tokens, d_model), dtype=torch.bfloat16, device=device)
    g = _gen(seed, device)
    for a in range(0, n_tokens, block_rows):
        b = min(a + block_rows, n_tokens)
        blk = torch.randn((b - a, d_model), generator=g, device=device, dtype=torch.float32)
        if count:
            blk[:, cols] *= outlier_gain
        out[a:b] = blk.to(torch.bfloat16)
        del blk
    return out


def make_w(d_model: int, seed: int, device="cpu") -> torch.Tensor:
    """Projection weight W [d, 3d] bf16, entries N(0, 1/d), row-major."""
    g = _gen(seed, device)
    w = torch.randn((d_model, 3 * d_model), generator=g, device=device, dtype=torch.float32)
    w *= d_model ** -0.5
    return w.to(torch.bfloat16)


def make_norm_weights(seed: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """RMSNorm gains for q and k, [128] fp32 each, U(0.5, 1.5) (CPU tensors)."""
    g = _gen(seed, "cpu")
    w = torch.rand((2, HEAD_DIM), generator=g, dtype=torch.float32) + 0.5
    return w[0].contiguous(), w[1].contiguous()


def make_integer_x(n_tokens: int, d_model: int, seed: int, lo=-4, hi=4, device="cpu"):
    """Integer-valued bf16 x in [lo, hi]: partial sums of the projection stay exact in fp32."""
    g = _gen(seed, device)
    return torch.randint(lo, hi + 1, (n_tokens, d_model), generator=g,
                         device=device).to(torch.bfloat16)


def make_integer_w(d_model: int, seed: int, lo=-4, hi=4, device="cpu"):
    g = _gen(seed, device)
    return torch.randint(lo, hi + 1, (d_model, 3 * d_model), generator=g,
                         device=device).to(torch.bfloat16)


def make_rotated_rows(rows: int, seed: int, scale: float = 2.0) -> torch.Tensor:
    """fp32 [rows, 128] values standing in for rotated K/V vectors (CPU)."""
    g = _gen(seed, "cpu")
    return torch.randn((rows, HEAD_DIM), generator=g, dtype=torch.float32) * scale


def make_bf16_matrix(rows: int, cols: int, seed: int, std: float = 1.0, device="cpu"):
    g = _gen(seed, device)
    return (torch.randn((rows, cols), generator=g, device=device) * std).to(torch.bfloat16)


def sample_rows(n_tokens: int, count: int, seed: int,
                must: Sequence[int] = ()) -> torch.Tensor:
    """Sorted distinct row indices: rows 0 and N-1, every row in `must`, and seeded
    uniform draws up to `count` rows in total (all rows when N <= count)."""
    if n_tokens <= count:
        return torch.arange(n_tokens, dtype=torch.int64)
    keep = {0, n_tokens - 1}
    keep.update(int(r) for r in must if 0 <= int(r) < n_tokens)
    g = _gen(seed, "cpu")
    while len(keep) < count:
        keep.add(int(torch.randint(0, n_tokens, (1,), generator=g)))
    return torch.tensor(sorted(keep), dtype=torch.int64)


def boundary_rows(n_tokens: int, step: int, extra: Sequence[int] = ()) -> List[int]:
    """Rows on both sides of every multiple of `step` (and of each value in `extra`)."""
    rows = []
    if step > 0:
        for m in range(step, n_tokens, step):
            rows += [m - 1, m]
    for e in extra:
        rows += [e - 1, e]
    return [r for r in rows if 0 <= r < n_tokens]


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a tensor, as a numpy uint16 array on the host."""
    import numpy as np
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
