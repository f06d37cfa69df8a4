"""Exact-row routing ([VL] Sol-Attn section, `_exact_av_rows`): the query rows of the
conditioning ranges (text and audio) attend to an exact K/V of every key while the other
rows stay on the low-bit store.  Here the exact store is an all-BF16 store (the rotated
K/V at bf16, [FR] "Mixed precision for conditioning") written beside the INT4 store, and
the routed rows are re-attended through q_begin / q_end into the same O and LSE.  The
combined O and LSE are checked against the oracle row by row (each row against the store
it was routed to), the unrouted rows stay bit-identical to the plain INT4 attention, and
the routed rows come out closer to attention over the unquantised K/V."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import BF16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def host(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("kv_block", [0, 512])
def test_exact_rows_routed_to_a_bf16_store(lib, kv_block):
    N, d = 1500, 512
    H = d // 128
    x = synth.make_x(N, d, 0.01, seed=611, device=DEV)
    w = synth.make_w(d, seed=612, device=DEV)
    low = lib.streamed_qkv_quant(x, w)                                       # all INT4, with Q
    exact = lib.streamed_qkv_quant(x, w, ranges=[(0, N, BF16)], emit=lib.SQG_EMIT_KV)
    routed = [(0, 384), (1024, 1152)]                                        # "text" and "audio" rows
    o, lse = lib.packed_kv_attention(low, kv_block=kv_block)
    o_low, lse_low = o.clone(), lse.clone()
    for a, b in routed:
        lib.packed_kv_attention(exact, q=low["q"], q_begin=a, q_end=b, kv_block=kv_block, o=o, lse=lse)
    torch.cuda.synchronize()

    is_routed = np.zeros(N, bool)
    for a, b in routed:
        is_routed[a:b] = True
    # the unrouted rows are the INT4 attention's, bit for bit
    keep = torch.from_numpy(~is_routed).to(DEV)
    assert torch.equal(o[keep], o_low[keep]) and torch.equal(lse[:, keep], lse_low[:, keep])

    qb = synth.bf16_bits(low["q"])
    rows_r = np.r_[np.arange(0, 384, 5), np.arange(1024, 1152, 3), [383, 1151]]
    rows_l = np.r_[np.arange(384, 1024, 11), np.arange(1152, N, 9), [N - 1]]
    lay_low, _ = oracle.packed_layout(N, H, oracle.range_segments(N, None))
    lay_ex, _ = oracle.packed_layout(N, H, oracle.range_segments(N, [(0, N, BF16)]))
    og, lg = host(o), host(lse)
    for rows, store, lay in ((rows_r, exact, lay_ex), (rows_l, low, lay_low)):
        want, lse_want = oracle.attention_rows_from_store(
            qb[rows], rows, host(store["kpack"]), host(store["vpack"]), host(store["kscale"]),
            host(store["vscale"]), lay, H, N, kv_block=kv_block)
        err = np.abs(og[rows] - want)
        rel = np.linalg.norm(og[rows] - want) / np.linalg.norm(want)
        assert err.max() <= 2e-2 and rel <= 5e-3, (err.max(), rel)
        assert np.max(np.abs(lg[:, rows] - lse_want)) <= 2e-3

    # what the routing is for: the routed rows track attention over the unquantised K/V
    # more closely than the INT4 rows of the same queries do
    ref = oracle.qkv_quant_rows(synth.bf16_bits(x), synth.bf16_bits(w), H, np.arange(N),
                                np.full(N, oracle.INT4))
    o_exact = np.zeros((len(rows_r), d))
    for h in range(H):
        kr = ref["k_rot_f32"][:, h].astype(np.float64)
        vr = ref["v_rot_f32"][:, h].astype(np.float64)
        oh, _ = oracle.attention_rotated_rows(qb[rows_r][:, 128 * h:128 * h + 128], kr, vr, 128 ** -0.5)
        o_exact[:, 128 * h:128 * h + 128] = oh
    e_routed = np.linalg.norm(og[rows_r] - o_exact) / np.linalg.norm(o_exact)
    e_int4 = np.linalg.norm(host(o_low)[rows_r] - o_exact) / np.linalg.norm(o_exact)
    assert e_routed < 0.25 * e_int4, (e_routed, e_int4)
