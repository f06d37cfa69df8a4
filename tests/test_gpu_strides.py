"""GPU checks of row strides at the boundary: x, W_qkv, Q and O may be row slices of
wider buffers (row strides ldx, ldw, ldq, ldo, multiples of 8 elements, 16-byte aligned
bases), and the results must equal those of contiguous buffers bit for bit, since the
kernels' arithmetic does not depend on where a row starts."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_strided_projection_and_attention_match_contiguous(lib):
    N, d = 1100, 512
    ranges = [(0, 128, lib.SQG_INT8_ROT), (128, N, lib.SQG_INT4_ROT)]
    x = synth.make_x(N, d, 0.01, seed=901, device=DEV)
    w = synth.make_w(d, seed=902, device=DEV)
    ref = lib.streamed_qkv_quant(x, w, ranges=ranges, chunk_rows=512)

    # x as columns [64, 64 + d) of a [N, d + 128] buffer, W as columns [8, 8 + 3d) of a
    # [d, 3d + 16] buffer, Q written into columns [32, 32 + d) of a [N, d + 96] buffer
    xw = torch.full((N, d + 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    xw[:, 64:64 + d] = x
    ww = torch.full((d, 3 * d + 16), float("nan"), dtype=torch.bfloat16, device=DEV)
    ww[:, 8:8 + 3 * d] = w
    out = lib.alloc_store(N, d, ranges, device=DEV)
    qw = torch.zeros((N, d + 96), dtype=torch.bfloat16, device=DEV)
    out["q"] = qw[:, 32:32 + d]
    lib.streamed_qkv_quant(xw[:, 64:64 + d], ww[:, 8:8 + 3 * d], ranges=ranges, chunk_rows=512, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out["q"], ref["q"])
    for k in ("kpack", "vpack", "kscale", "vscale"):
        assert torch.equal(out[k], ref[k]), k
    assert bool((qw[:, :32] == 0).all()) and bool((qw[:, 32 + d:] == 0).all())

    # attention from the strided Q into a strided O
    o_ref, l_ref = lib.packed_kv_attention(ref, kv_block=512)
    ow = torch.full((N, d + 64), 7.0, dtype=torch.float32, device=DEV)
    o, l = lib.packed_kv_attention(out, q=out["q"], kv_block=512, o=ow[:, 16:16 + d])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    assert bool((ow[:, :16] == 7.0).all()) and bool((ow[:, 16 + d:] == 7.0).all())
