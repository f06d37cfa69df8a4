"""CPU oracle for the streamed QKV-quant + packed-K/V attention path.

TEST INFRASTRUCTURE.  Only the tests under tests/, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py may import or call
anything in this package.  The HIP library never calls it, and this package never
imports the HIP library or its Python binding: the two share no code.  The only
thing both sides consume is the seeded input generator in synth/.

Everything here is plain numpy in float64 (floating-point steps whose precision
the method fixes are rounded explicitly: fp32 rotation output, fp16 scales, bf16
Q).  It is slow on purpose and written to be checked by eye against the pages:

* Feature request "Streamed QKV Projection and Packed Low-Bit K/V Support for
  Extreme Long-Sequence Attention" (comfy-kitchen issue page and its mirror),
  sections "Proposed backend capability", "Potential reduction",
  "Quality-oriented low-bit format", "Mixed precision for conditioning" and
  "Dense fallback is important".
* "VRAM Lab" module page (ComfyUI-MAINodes vram_lab.py): the helpers section
  (`_ranges`, `_norm_rope`, `_blockwise_attention`), the kvi8r section
  (`_hadamard`, `_online_combine`, `_Int8KV`, `_blockwise_attention_q`), the
  precision-probe section (`_fq_int4`, `_fq_int4_had`) and the block section
  (`_phase1_kv`, `_phase2_q_attn`).

Readings where the pages are silent or ambiguous are listed in the design doc and
repeated at each function.  Parity status: every function here is pinned by the
`-m "not gpu"` tests in tests/test_oracle_*.py except `quality_vs_unquantised`,
which is parity unpinned (no page value exists for this format on these inputs).
"""
from .reference import *  # noqa: F401,F403
from .reference import __all__  # noqa: F401
