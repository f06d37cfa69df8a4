"""streamed_qkv_gemm_amd: streamed QKV-quant and packed-K/V attention for MI355X.

The compute lives in libsqg.so (hand-written HIP for gfx950, C ABI in
include/sqg.h).  This package is its Python binding: argument marshalling, torch
tensors for device memory and the current HIP stream.  Build the library with
`python -m streamed_qkv_gemm_amd.build` before use.
"""
from ._binding import (  # noqa: F401
    HEAD_DIM, LIB_PATH, SQG_BF16, SQG_EMIT_KV, SQG_EMIT_Q, SQG_EMIT_QKV, SQG_F16, SQG_F32, SQG_QK_EXACT, SQG_QK_FP8,
    SQG_BF16_ROT, SQG_INT4_ROT, SQG_INT8_ROT, SqgError, alloc_store, chunk_ranges, kv_layout, lib_path, load,
    alloc_staged, kv_block_layout, kv_row_offset, packed_kv_attention, packed_kv_attention_qrecompute,
    packed_kv_attention_staged, qrecompute_workspace_bytes, packed_kv_attention_qrecompute_noalloc,
    noalloc_scratch_bytes, rope_table, staged_sizes,
    streamed_qkv_quant, streamed_qkv_quant_staged, test_fwht_f32, test_quant_pack_f32,
    version,
)
