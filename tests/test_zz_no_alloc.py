"""The allocation-free Q-recompute entry point, through the C ABI, against the
Q-recompute entry point that takes the caller's workspace: two calls in a row on the
same GPU, the second with a smaller input, each equal bit for bit to the existing entry
point and within G3 of the oracle on sampled rows.  The first call spans several chunks
of the device scratch (d_model 7168: 4096-row chunks), the second one chunk."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def host(t):
    return t.detach().cpu().numpy()


def case(lib, N, d, ranges, seed, norm_rope):
    x = synth.make_x(N, d, 0.005, seed=seed, device=DEV)
    w = synth.make_w(d, seed=seed + 1, device=DEV)
    kw = {}
    if norm_rope:
        nw = synth.make_norm_weights(seed + 2)
        kw = dict(q_norm_w=nw[0].to(DEV), k_norm_w=nw[1].to(DEV))
        kw["rope_cos"], kw["rope_sin"] = lib.rope_table(N, 10000.0, device=DEV)
    kv = lib.streamed_qkv_quant(x, w, ranges=ranges, emit=lib.SQG_EMIT_KV, **kw)
    q_kw = {k: v for k, v in kw.items() if k != "k_norm_w"}
    return x, w, kv, q_kw


@pytest.mark.parametrize("N,d,ranges,norm_rope,kv_block", [
    (9000, 7168, [(0, 512, 1), (512, 9000, 0)], True, 4096),   # three scratch chunks
    (1000, 512, None, False, 0),                                # then a smaller call
])
def test_noalloc_qrecompute_equals_workspace_entry(lib, N, d, ranges, norm_rope, kv_block):
    print("[no-alloc] N=%d d=%d" % (N, d), flush=True)
    H = d // 128
    x, w, kv, q_kw = case(lib, N, d, ranges, 900 + N, norm_rope)
    o_ref, l_ref = lib.packed_kv_attention_qrecompute(kv, x, w, kv_block=kv_block, **q_kw)
    o = torch.empty((N, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((H, N), dtype=torch.float32, device=DEV)
    o.fill_(7.0)
    lse.fill_(7.0)
    lib.packed_kv_attention_qrecompute_noalloc(kv, x, w, o, lse, kv_block=kv_block, **q_kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    # and against the oracle on sampled rows (Q rebuilt by the oracle from x, W)
    rows = synth.sample_rows(N, 16, seed=N, must=[N - 1]).numpy()
    segs = oracle.range_segments(N, ranges)
    okw = {}
    if norm_rope:
        nw = synth.make_norm_weights(900 + N + 2)
        okw = dict(q_norm_w=nw[0].numpy(), k_norm_w=nw[1].numpy(), eps=1e-6, rope_theta=10000.0)
    ref = oracle.qkv_quant_rows(synth.bf16_bits(x)[rows], synth.bf16_bits(w), H, rows,
                                oracle.token_formats(N, segs)[rows], **okw)
    layout, _ = oracle.packed_layout(N, H, segs)
    heads = [0, H - 1]
    want, lse_want = oracle.attention_rows_from_store(
        ref["q_bits"], rows, host(kv["kpack"]), host(kv["vpack"]), host(kv["kscale"]),
        host(kv["vscale"]), layout, H, N, kv_block=kv_block, heads=heads)
    got = host(o)[rows]
    for h in heads:
        sl = slice(128 * h, 128 * h + 128)
        err = np.abs(got[:, sl] - want[:, sl])
        rel = np.linalg.norm(got[:, sl] - want[:, sl]) / np.linalg.norm(want[:, sl])
        # the oracle's Q is bf16 of an fp64 sum, the GPU's of an fp32 sum: one bf16 step
        # apart in rare values, within the attention gate
        assert err.max() <= 2e-2 and rel <= 5e-3, (h, err.max(), rel)


def test_noalloc_refuses_chunks_beyond_the_scratch(lib):
    # 70,000 query rows of d_model 512 in one explicit chunk need 68.4 MB, more than the
    # 64 MiB scratch: refused before anything is enqueued (O keeps its contents)
    N, d = 70000, 512
    x, w, kv, q_kw = case(lib, N, d, None, 77, False)
    o = torch.full((N, d), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(lib.SqgError) as e:
        lib.packed_kv_attention_qrecompute_noalloc(kv, x, w, o, q_chunk_rows=131072)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
