"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same chunking, same KV blocking), checked on sampled rows that the
oracle computes one by one: G2 on sampled token rows (including every chunk and
range boundary), G3 on sampled query rows of a few heads against all keys."""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import q_gate, scale_gate

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda"


def host(t):
    return t.detach().cpu().numpy()


def build_inputs(wl):
    x = synth.make_x(wl.n_tokens, wl.d_model, wl.outlier_frac, seed=wl.seed_base + 1, device=DEV,
                     outlier_seed=wl.seed_base + 3)
    w = synth.make_w(wl.d_model, seed=wl.seed_base + 2, device=DEV)
    norm = synth.make_norm_weights(wl.seed_base + 4) if wl.norm_rope else None
    return x, w, norm


@pytest.mark.parametrize("name", ["h3_16k", "h3_64k_mixed", "h3_152k_odd", "h3_217k_normrope"])
def test_fullsize_parity(lib, name):
    wl = synth.WORKLOADS[name]
    N, d, H = wl.n_tokens, wl.d_model, wl.n_heads
    print("[fullsize] %s N=%d d=%d" % (name, N, d), flush=True)
    x, w, norm = build_inputs(wl)
    kw = {}
    if wl.norm_rope:
        kw["q_norm_w"], kw["k_norm_w"] = norm[0].to(DEV), norm[1].to(DEV)
        kw["rope_cos"], kw["rope_sin"] = lib.rope_table(N, 10000.0, device=DEV)
    ranges = wl.ranges
    store = lib.streamed_qkv_quant(x, w, ranges=ranges, chunk_rows=wl.chunk_rows, **kw)
    o, lse = lib.packed_kv_attention(store, kv_block=wl.kv_block)
    torch.cuda.synchronize()

    # ---- G2 on sampled token rows
    extra = [b for (b, _, _) in wl.range_list()[1:]]
    must = synth.boundary_rows(N, wl.chunk_rows, extra)
    rows = synth.sample_rows(N, 48, seed=wl.seed_base + 5, must=must).numpy()
    segs = oracle.range_segments(N, ranges)
    fm = oracle.token_formats(N, segs)[rows]
    xb = synth.bf16_bits(x[torch.from_numpy(rows).to(DEV)])
    okw = {}
    if wl.norm_rope:
        okw = dict(q_norm_w=norm[0].numpy(), k_norm_w=norm[1].numpy(), eps=1e-6, rope_theta=10000.0)
    ref = oracle.qkv_quant_rows(xb, synth.bf16_bits(w), H, rows, fm, **okw)
    layout, _ = oracle.packed_layout(N, H, segs)
    kp, vp = host(store["kpack"]), host(store["vpack"])
    ks, vs = host(store["kscale"]), host(store["vscale"])
    kc, ksc = oracle.gather_packed_rows(kp, ks, layout, H, rows)
    vc, vsc = oracle.gather_packed_rows(vp, vs, layout, H, rows)
    qb = synth.bf16_bits(store["q"])
    for got, want in ((kc, ref["k_codes"]), (vc, ref["v_codes"])):
        dd = np.abs(got.astype(np.int64) - want.astype(np.int64))
        assert dd.max() <= 1 and np.mean(dd == 0) >= 0.999, (name, dd.max(), np.mean(dd == 0))
    scale_gate(ksc, ref["k_scales"], fm)
    scale_gate(vsc, ref["v_scales"], fm)
    q_gate(qb[rows], ref["q_bits"], name)

    # ---- G3 on 32 sampled query rows (the last row and, with a policy, both sides of
    # every range boundary among them) x 8 heads spread over the head range, all keys
    qrows = synth.sample_rows(N, 32, seed=wl.seed_base + 6, must=[N - 1] + extra).numpy()
    heads = sorted(set(np.linspace(0, H - 1, 8).round().astype(int).tolist()))
    o_ref, lse_ref = oracle.attention_rows_from_store(qb[qrows], qrows, kp, vp, ks, vs, layout, H, N,
                                                      kv_block=wl.kv_block, heads=heads)
    og = host(o)[qrows]
    lg = host(lse)[:, qrows]
    for h in heads:
        sl = slice(128 * h, 128 * h + 128)
        err = np.abs(og[:, sl] - o_ref[:, sl])
        rel = np.linalg.norm(og[:, sl] - o_ref[:, sl]) / np.linalg.norm(o_ref[:, sl])
        assert err.max() <= 2e-2 and rel <= 5e-3, (name, h, err.max(), rel)
        assert np.max(np.abs(lg[h] - lse_ref[h])) <= 2e-3


def test_fullsize_variants_217k(lib):
    """The bench's extra measurements at 217,088 tokens x 56 heads, in its launch
    configuration: the fp8 QK^T tier against the fp8 oracle on sampled rows, and the
    Q-recompute and host-staged variants equal to the device path on sampled rows."""
    wl = synth.WORKLOADS["h3_217k_normrope"]
    N, d, H = wl.n_tokens, wl.d_model, wl.n_heads
    print("[fullsize] variants N=%d d=%d" % (N, d), flush=True)
    x, w, norm = build_inputs(wl)
    kw = dict(q_norm_w=norm[0].to(DEV), k_norm_w=norm[1].to(DEV))
    kw["rope_cos"], kw["rope_sin"] = lib.rope_table(N, 10000.0, device=DEV)
    store = lib.streamed_qkv_quant(x, w, ranges=wl.ranges, chunk_rows=wl.chunk_rows, **kw)
    o, lse = lib.packed_kv_attention(store, kv_block=wl.kv_block)
    o8, l8 = lib.packed_kv_attention(store, kv_block=wl.kv_block, qk_mode=lib.SQG_QK_FP8)
    torch.cuda.synchronize()
    qrows = synth.sample_rows(N, 8, seed=wl.seed_base + 7, must=[0, N - 1]).numpy()
    heads = [1, H - 2]
    qb = synth.bf16_bits(store["q"])
    layout, _ = oracle.packed_layout(N, H, oracle.range_segments(N, wl.ranges))
    args = (host(store["kpack"]), host(store["vpack"]), host(store["kscale"]), host(store["vscale"]),
            layout, H, N)
    want, lse_want = oracle.attention_rows_from_store(qb[qrows], qrows, *args, kv_block=wl.kv_block,
                                                      heads=heads, qk="fp8")
    og, lg = host(o8)[qrows], host(l8)[:, qrows]
    for h in heads:
        sl = slice(128 * h, 128 * h + 128)
        err = np.abs(og[:, sl] - want[:, sl])
        rel = np.linalg.norm(og[:, sl] - want[:, sl]) / np.linalg.norm(want[:, sl])
        assert err.max() <= 2e-2 and rel <= 5e-3, ("fp8", h, err.max(), rel)
        assert np.max(np.abs(lg[h] - lse_want[h])) <= 2e-3
    qr = torch.from_numpy(qrows).to(DEV)
    o_ref, l_ref = o[qr].clone(), lse[:, qr].clone()
    del o8, l8, o, lse
    torch.cuda.empty_cache()
    # Q-recompute from a K/V-only store
    kv = lib.streamed_qkv_quant(x, w, ranges=wl.ranges, chunk_rows=wl.chunk_rows, emit=lib.SQG_EMIT_KV, **kw)
    q_kw = {k: v for k, v in kw.items() if k != "k_norm_w"}
    o1, l1 = lib.packed_kv_attention_qrecompute(kv, x, w, kv_block=wl.kv_block, **q_kw)
    torch.cuda.synchronize()
    assert torch.equal(o1[qr], o_ref) and torch.equal(l1[:, qr], l_ref)
    del o1, l1, kv
    torch.cuda.empty_cache()
    # host-staged K/V in blocks of the KV-block size: one launch per block merged through
    # the LSE, against the device path's single walk over the blocks (equal up to
    # rounding), and on its own against the oracle
    st = lib.alloc_staged(N, d, wl.kv_block, wl.ranges, device=DEV)
    lib.streamed_qkv_quant_staged(x, w, st, emit=lib.SQG_EMIT_KV, **kw)
    o2, l2 = lib.packed_kv_attention_staged(st, store["q"])
    torch.cuda.synchronize()
    assert float((o2[qr] - o_ref).abs().max()) <= 2e-3 and float((l2[:, qr] - l_ref).abs().max()) <= 1e-4
    want, lse_want = oracle.attention_rows_from_store(qb[qrows], qrows, *args, kv_block=wl.kv_block,
                                                      heads=heads)
    og, lg = host(o2)[qrows], host(l2)[:, qrows]
    for h in heads:
        sl = slice(128 * h, 128 * h + 128)
        err = np.abs(og[:, sl] - want[:, sl])
        rel = np.linalg.norm(og[:, sl] - want[:, sl]) / np.linalg.norm(want[:, sl])
        assert err.max() <= 2e-2 and rel <= 5e-3, ("staged", h, err.max(), rel)
        assert np.max(np.abs(lg[h] - lse_want[h])) <= 2e-3
