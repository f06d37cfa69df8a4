"""Benchmark of the streamed QKV-quant + packed-K/V attention hot path on one GPU.

One step = the whole path over one batch of synthetic input already resident in
HBM: streamed_qkv_quant over all row chunks (projection, RMSNorm/RoPE where the
workload has them, Hadamard rotation, quantisation, packing), then
packed_kv_attention over all keys (log-sum-exp merge of the KV blocks where the
workload blocks the keys).  The headline line is the 217,088-token workload; the
four other workloads are measured in the same run at fewer steps and reported
under "configs".  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "packed-KV attention TFLOP/s + streamed QKV-quant tokens/s; peak HBM bytes"
PEAK_TFLOPS_F16 = 2500.0   # MI355X dense bf16 / f16 MFMA (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)
DEFAULT_WORKLOAD = "h3_217k_normrope"

# HBM bytes per launch of the two kernels, from rocprofv3 FETCH_SIZE and WRITE_SIZE
# counters scaled by the same counters on a device copy of known size, keyed by the
# kernel, the SHA-256 of the kernel source they were taken on, and the workload.  A
# changed kernel reports null until the counters are taken again.
MEASURED_TRAFFIC = {
    # profiles/hbm_traffic_h3_217k_normrope.md
    ("packed_attention_kernel", "a2cc8cd6ff8a4470c90c56537c46f5b6fb15d6e5ea8ff575b3631e1ac94f5c30",
     "h3_217k_normrope"): 1.0461e+11,
    ("qkv_quant_kernel", "f13aaa425c9eaeca854aa202c1af9fbb86ec301034ca1be3368906e93aac08bb",
     "h3_217k_normrope"): 7.6023e+09,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--config-steps", type=int, default=3,
                    help="timed steps of each other workload (0 = skip the configs block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=24, help="heads in the oracle's attention sample")
    ap.add_argument("--cpu-query-rows", type=int, default=64, help="query rows in the oracle's attention sample")
    ap.add_argument("--cpu-token-rows", type=int, default=1024, help="token rows in the oracle's QKV-quant sample")
    ap.add_argument("--qrecompute-steps", type=int, default=1,
                    help="steps of the Q-recompute variant timed after the main steps (0 = skip)")
    ap.add_argument("--q-chunk-rows", type=int, default=0, help="query chunk of the Q-recompute variant")
    ap.add_argument("--fp8-steps", type=int, default=1,
                    help="steps of the fp8-QK attention tier timed after the main steps (0 = skip)")
    ap.add_argument("--staged-steps", type=int, default=1,
                    help="steps of the host-staged K/V variant timed after the main steps (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, copy this many MiB device-to-device three times "
                         "(reference dispatches for HBM byte counters)")
    return ap.parse_args()


def kernel_sha(name):
    import hashlib
    with open(os.path.join(ROOT, "streamed_qkv_gemm_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel, source, workload):
    """HBM bytes per launch measured on this exact kernel source, else None."""
    return MEASURED_TRAFFIC.get((kernel, kernel_sha(source), workload))


def make_inputs(wl, dev):
    import torch

    import streamed_qkv_gemm_amd as sqg
    import synth
    x = synth.make_x(wl.n_tokens, wl.d_model, wl.outlier_frac, seed=wl.seed_base + 1, device=dev,
                     outlier_seed=wl.seed_base + 3)
    w = synth.make_w(wl.d_model, seed=wl.seed_base + 2, device=dev)
    kw, norm = {}, None
    if wl.norm_rope:
        norm = synth.make_norm_weights(wl.seed_base + 4)
        kw["q_norm_w"], kw["k_norm_w"] = norm[0].to(dev), norm[1].to(dev)
        kw["rope_cos"], kw["rope_sin"] = sqg.rope_table(wl.n_tokens, 10000.0, device=dev)
    torch.cuda.synchronize()
    return x, w, kw, norm


def run_steps(wl, x, w, kw, steps, warmup, dev):
    """Time `steps` whole-path steps (after `warmup` untimed ones) with HIP events on the
    launch stream; returns the per-step figures and the buffers of the last step."""
    import torch

    import streamed_qkv_gemm_amd as sqg
    N, d, H = wl.n_tokens, wl.d_model, wl.n_heads
    input_bytes = torch.cuda.memory_allocated(dev)
    store = sqg.alloc_store(N, d, wl.ranges, device=dev)
    o = torch.empty((N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        sqg.streamed_qkv_quant(x, w, ranges=wl.ranges, chunk_rows=wl.chunk_rows, out=store, **kw)
        if ev:
            ev[1].record(stream)
        sqg.packed_kv_attention(store, kv_block=wl.kv_block, o=o, lse=lse)
        if ev:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    peak_alloc = torch.cuda.max_memory_allocated(dev)
    qkv_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    att_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    step_list = sorted(e[0].elapsed_time(e[2]) for e in evs)
    step_ms = sum(step_list) / steps

    qkv_flop = 2.0 * N * d * 3 * d
    att_flop = 4.0 * N * N * H * 128
    n_chunks = len(sqg.chunk_ranges(N, wl.chunk_rows, 512))
    L = store["layout"]
    packed_ws = L["q_bytes"] + 2 * L["pack_bytes"] + 2 * L["scale_bytes"]
    att_tflops = att_flop / (att_ms * 1e-3) / 1e12
    qkv_tflops = qkv_flop / (qkv_ms * 1e-3) / 1e12
    # algorithmic HBM bytes per QKV-quant token: x row + Q row + packed K/V rows + scales
    qkv_bytes_per_token = 2 * d + 2 * d + 2 * (L["pack_bytes"] + L["scale_bytes"]) / max(N, 1)
    figures = {
        "ms_per_step": step_ms,
        "ms_per_step_median": step_list[len(step_list) // 2],
        "value": (qkv_flop + att_flop) / (step_ms * 1e-3) / 1e12,
        "attention_tflops": att_tflops,
        "attention_ms": att_ms,
        "attention_mfma_frac": att_tflops / PEAK_TFLOPS_F16,
        "qkv_quant_tokens_per_s": N / (qkv_ms * 1e-3),
        "qkv_quant_tflops": qkv_tflops,
        "qkv_quant_ms": qkv_ms,
        "qkv_quant_mfma_frac": qkv_tflops / PEAK_TFLOPS_F16,
        "qkv_quant_algorithmic_gbs": (N * qkv_bytes_per_token + 2 * d * 3 * d * n_chunks) / (qkv_ms * 1e-3) / 1e9,
        "peak_alloc_bytes": peak_alloc,
        "input_bytes": input_bytes,
        "qkv_working_set_bytes": packed_ws,
        "bf16_qkv_bytes": L["bf16_qkv_bytes"],
        "working_set_ratio": packed_ws / L["bf16_qkv_bytes"],
        "qkv_launches_per_step": n_chunks,
        "wall_s_timed": wall,
    }
    return figures, {"store": store, "o": o, "lse": lse, "qkv_flop": qkv_flop, "att_flop": att_flop}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import streamed_qkv_gemm_amd as sqg
    import synth

    sqg.load()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU: the library has no CPU path")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]
    N, d, H = wl.n_tokens, wl.d_model, wl.n_heads
    print("[bench] workload %s N=%d d=%d steps=%d warmup=%d" % (wl.name, N, d, args.steps, args.warmup),
          file=sys.stderr, flush=True)

    x, w, kw, norm = make_inputs(wl, dev)
    fig, bufs = run_steps(wl, x, w, kw, args.steps, args.warmup, dev)
    store, o, lse = bufs["store"], bufs["o"], bufs["lse"]
    qkv_flop, att_flop = bufs["qkv_flop"], bufs["att_flop"]
    att_ms, qkv_ms = fig["attention_ms"], fig["qkv_quant_ms"]
    L = store["layout"]
    stream = torch.cuda.current_stream(dev)
    print("[bench] main steps done: %.1f ms/step" % fig["ms_per_step"], file=sys.stderr, flush=True)

    # the oracle's timed sample and the parity gates on it, against the O and LSE of the
    # last timed step (before the variants below reuse those buffers)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, x, w, norm, store, o, lse, args.cpu_heads, args.cpu_query_rows,
                           args.cpu_token_rows)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: 3 x %d bytes read + written" % (2 * n), file=sys.stderr)
        del src, dst

    # ---- low-precision QK^T tier: the same attention with scores on block-scaled fp8
    # operands (timed separately, not part of value; its output is compared with the
    # exact tier's O of the last timed step)
    fp8_res = None
    if args.fp8_steps > 0:
        o8 = torch.empty_like(o)
        l8 = torch.empty_like(lse)
        sqg.packed_kv_attention(store, kv_block=wl.kv_block, o=o8, lse=l8, qk_mode=sqg.SQG_QK_FP8)
        torch.cuda.synchronize()
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.fp8_steps)]
        for e0, e1 in fe:
            e0.record(stream)
            sqg.packed_kv_attention(store, kv_block=wl.kv_block, o=o8, lse=l8, qk_mode=sqg.SQG_QK_FP8)
            e1.record(stream)
        torch.cuda.synchronize()
        f_ms = sum(a.elapsed_time(b) for a, b in fe) / args.fp8_steps
        rel = float(torch.linalg.vector_norm(o8 - o) / torch.linalg.vector_norm(o))
        fp8_res = {"steps": args.fp8_steps, "attention_ms": f_ms,
                   "attention_tflops": att_flop / (f_ms * 1e-3) / 1e12,
                   "speedup_vs_exact_tier": att_ms / f_ms, "rel_l2_vs_exact_tier": rel,
                   "dtype": "fp8 e4m3 QK^T (E8M0 per 32 dims), f16 P.V"}
        del o8, l8
        torch.cuda.empty_cache()

    # ---- Q-recompute variant: K/V-only projection, then Q rebuilt per query chunk inside
    # the attention call; no [N, d] Q buffer exists (timed separately, not part of value)
    qrec = None
    if args.qrecompute_steps > 0:
        kv_store = sqg.alloc_store(N, d, wl.ranges, device=dev, emit=sqg.SQG_EMIT_KV)
        ws_bytes = sqg.qrecompute_workspace_bytes(N, d, args.q_chunk_rows)
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
        q_kw = {k: v for k, v in kw.items() if k != "k_norm_w"}

        def qrec_step(ev=None):
            if ev:
                ev[0].record(stream)
            sqg.streamed_qkv_quant(x, w, ranges=wl.ranges, chunk_rows=wl.chunk_rows, out=kv_store,
                                   emit=sqg.SQG_EMIT_KV, **kw)
            if ev:
                ev[1].record(stream)
            sqg.packed_kv_attention_qrecompute(kv_store, x, w, q_chunk_rows=args.q_chunk_rows,
                                               workspace=ws, kv_block=wl.kv_block, o=o, lse=lse, **q_kw)
            if ev:
                ev[2].record(stream)

        qrec_step()
        torch.cuda.synchronize()
        qev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.qrecompute_steps)]
        for i in range(args.qrecompute_steps):
            qrec_step(qev[i])
        torch.cuda.synchronize()
        kv_ms = sum(e[0].elapsed_time(e[1]) for e in qev) / args.qrecompute_steps
        qa_ms = sum(e[1].elapsed_time(e[2]) for e in qev) / args.qrecompute_steps
        qrec_ws = 2 * L["pack_bytes"] + 2 * L["scale_bytes"] + ws_bytes
        qrec = {"steps": args.qrecompute_steps, "ms_per_step": kv_ms + qa_ms,
                "tflops": (qkv_flop + att_flop) / ((kv_ms + qa_ms) * 1e-3) / 1e12,
                "kv_quant_ms": kv_ms, "q_recompute_attention_ms": qa_ms,
                "q_chunk_rows": ws_bytes // (2 * d), "workspace_bytes": ws_bytes,
                "qkv_working_set_bytes": qrec_ws,
                "working_set_ratio": qrec_ws / L["bf16_qkv_bytes"]}
        del kv_store, ws
        torch.cuda.empty_cache()

    # ---- host-staged variant: the packed K/V lives in pinned host memory, one block of
    # kv_block keys at a time on the GPU (timed separately, not part of value)
    staged_res = None
    if args.staged_steps > 0:
        block = wl.kv_block if wl.kv_block > 0 else 16384
        stg = sqg.alloc_staged(N, d, block, wl.ranges, device=dev)
        q_st = torch.empty((N, d), dtype=torch.bfloat16, device=dev)

        def staged_step(ev=None):
            if ev:
                ev[0].record(stream)
            sqg.streamed_qkv_quant_staged(x, w, stg, q=q_st, **kw)
            if ev:
                ev[1].record(stream)
            sqg.packed_kv_attention_staged(stg, q_st, o=o, lse=lse)
            if ev:
                ev[2].record(stream)

        staged_step()
        torch.cuda.synchronize()
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.staged_steps)]
        for i in range(args.staged_steps):
            staged_step(sev[i])
        torch.cuda.synchronize()
        b_ms = sum(e[0].elapsed_time(e[1]) for e in sev) / args.staged_steps
        a_ms = sum(e[1].elapsed_time(e[2]) for e in sev) / args.staged_steps
        (hp, hs, dp, ds), nb = sqg.staged_sizes(N, d, block, wl.ranges)
        staged_res = {"steps": args.staged_steps, "block_rows": block, "n_blocks": nb,
                      "ms_per_step": b_ms + a_ms,
                      "tflops": (qkv_flop + att_flop) / ((b_ms + a_ms) * 1e-3) / 1e12,
                      "qkv_quant_to_host_ms": b_ms, "attention_from_host_ms": a_ms,
                      "host_store_bytes": 2 * (hp + hs), "device_staging_bytes": 4 * (dp + ds),
                      "device_kv_bytes_vs_device_store": 4 * (dp + ds) / (2 * (hp + hs)),
                      "copies": "on a stream of their own, ordered by events against the kernels (overlapped)"}
        del stg, q_st
        torch.cuda.empty_cache()

    # ---- bf16-materialising baseline: x @ W into a bf16 [N, 3d] tensor (library GEMM)
    bf16_base = None
    if not args.no_bf16_baseline:
        try:
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats(dev)
            base0 = torch.cuda.memory_allocated(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            y = torch.matmul(x, w)
            torch.cuda.synchronize()
            e0.record(stream)
            y = torch.matmul(x, w)
            e1.record(stream)
            torch.cuda.synchronize()
            bf16_base = {"extra_peak_bytes": torch.cuda.max_memory_allocated(dev) - base0,
                         "qkv_bytes": y.numel() * 2, "gemm_ms": e0.elapsed_time(e1)}
            del y
        except RuntimeError as exc:  # pragma: no cover - reported, not fatal
            bf16_base = {"error": str(exc)[:200]}
        torch.cuda.empty_cache()

    n_att_launch = 1   # the device path walks every KV block in one launch
    result = {
        "metric": METRIC,
        "value": fig["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fig["ms_per_step"],
        "ms_per_step_median": fig["ms_per_step_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 projection, f16 attention (fp6 score remainder), int4/int8 K/V",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_tokens": N, "d_model": d, "n_heads": H, "head_dim": 128,
                   "ranges": wl.range_list(), "chunk_rows": wl.chunk_rows, "kv_block": wl.kv_block,
                   "norm_rope": wl.norm_rope, "kv_format": "Hadamard-rotated INT4/INT8, group 32, fp16 scales",
                   "parallelism": "none (1 GPU)"},
    }
    result.update({k: v for k, v in fig.items() if k not in ("value", "ms_per_step", "ms_per_step_median")})
    result.update({
        "bf16_materialising_baseline": bf16_base,
        "qrecompute": qrec,
        "fp8_qk_tier": fp8_res,
        "host_staged": staged_res,
        "roofline": {
            "kernel": "packed_attention_kernel",
            "bound": "mfma",
            "achieved": fig["attention_tflops"],
            "peak": PEAK_TFLOPS_F16,
            "unit": "TFLOP/s",
            "frac": fig["attention_tflops"] / PEAK_TFLOPS_F16,
            "traffic": measured_traffic("packed_attention_kernel", "packed_attention.hip", wl.name),
            "launches_per_step": n_att_launch,
            "avg_launch_ms": att_ms / n_att_launch,
            "algorithmic_flop_per_step": att_flop,
            # matrix-core time per algorithmic f16 MFMA: the f16 high part of QK^T and P.V
            # (1 each) plus the fp6 remainder term at four times the f16 rate (1/8)
            "executed_matrix_time_factor": 1.125,
        },
        "qkv_roofline": {
            "kernel": "qkv_quant_kernel", "bound": "mfma", "achieved": fig["qkv_quant_tflops"],
            "peak": PEAK_TFLOPS_F16, "unit": "TFLOP/s", "frac": fig["qkv_quant_tflops"] / PEAK_TFLOPS_F16,
            "traffic": measured_traffic("qkv_quant_kernel", "qkv_quant.hip", wl.name),
            "launches_per_step": fig["qkv_launches_per_step"],
            "avg_launch_ms": qkv_ms / fig["qkv_launches_per_step"],
            "algorithmic_hbm_gbs": fig["qkv_quant_algorithmic_gbs"],
        },
    })

    del x, w, kw, store, o, lse, bufs
    torch.cuda.empty_cache()

    # ---- the other workloads, same path, fewer steps (not part of value)
    configs = {}
    if args.config_steps > 0:
        for name in synth.WORKLOAD_ORDER:
            if name == wl.name:
                continue
            cw = synth.WORKLOADS[name]
            print("[bench] config %s" % name, file=sys.stderr, flush=True)
            cx, cwt, ckw, _ = make_inputs(cw, dev)
            cfig, cbufs = run_steps(cw, cx, cwt, ckw, args.config_steps, 1, dev)
            cfig.update({"n_tokens": cw.n_tokens, "d_model": cw.d_model, "ranges": cw.range_list(),
                         "chunk_rows": cw.chunk_rows, "kv_block": cw.kv_block, "norm_rope": cw.norm_rope,
                         "steps": args.config_steps, "warmup": 1})
            configs[name] = cfig
            del cx, cwt, ckw, cbufs
            torch.cuda.empty_cache()
    result["configs"] = configs
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, w, norm, store, o, lse, n_heads_sample, n_query_rows, n_token_rows):
    """The oracle as it stands, timed on this host's cores on a bounded sample:
    `n_token_rows` token rows of the QKV-quant and `n_query_rows` query rows x
    `n_heads_sample` heads x all keys of the attention (about 10-30 s of host time
    with the defaults).  Reported in the same unit as the GPU figure.  The same rows
    carry the parity gates: G2 (codes of the sampled token rows against the GPU's
    store) and G3 (the GPU's O and LSE of the sampled query rows against the oracle's)."""
    import numpy as np
    import threadpoolctl
    import torch

    import oracle
    import synth

    N, d, H = wl.n_tokens, wl.d_model, wl.n_heads
    dev = x.device
    extra = [b for (b, _, _) in wl.range_list()[1:]]
    rows = synth.sample_rows(N, n_token_rows, seed=wl.seed_base + 5,
                             must=synth.boundary_rows(N, wl.chunk_rows, extra)[:32]).numpy()
    xb = synth.bf16_bits(x[torch.from_numpy(rows).to(dev)])
    wb = synth.bf16_bits(w)
    segs = oracle.range_segments(N, wl.ranges)
    fm = oracle.token_formats(N, segs)[rows]
    okw = {}
    if wl.norm_rope:
        okw = dict(q_norm_w=norm[0].numpy(), k_norm_w=norm[1].numpy(), eps=1e-6, rope_theta=10000.0)
    threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    t0 = time.perf_counter()
    ref = oracle.qkv_quant_rows(xb, wb, H, rows, fm, **okw)
    t_qkv = time.perf_counter() - t0

    layout, _ = oracle.packed_layout(N, H, segs)
    kp, vp = store["kpack"].cpu().numpy(), store["vpack"].cpu().numpy()
    ks, vs = store["kscale"].cpu().numpy(), store["vscale"].cpu().numpy()
    qrows = synth.sample_rows(N, n_query_rows, seed=wl.seed_base + 6).numpy()
    qb = synth.bf16_bits(store["q"])[qrows]
    heads = list(range(0, H, max(1, H // n_heads_sample)))[:n_heads_sample]
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention_rows_from_store(qb, qrows, kp, vp, ks, vs, layout, H, N,
                                                      kv_block=wl.kv_block, heads=heads)
    t_att = time.perf_counter() - t0

    # ---- the gates on the same sample
    g2 = {}
    for t in ("k", "v"):
        codes, _ = oracle.gather_packed_rows(kp if t == "k" else vp, ks if t == "k" else vs, layout, H, rows)
        dd = np.abs(codes.astype(np.int64) - ref[t + "_codes"].astype(np.int64))
        g2[t + "_codes_identical"] = float(np.mean(dd == 0))
        g2[t + "_codes_max_step"] = int(dd.max())
    g2["pass"] = all(g2[t + "_codes_identical"] >= 0.999 and g2[t + "_codes_max_step"] <= 1 for t in ("k", "v"))
    cols = np.concatenate([np.arange(128 * h, 128 * h + 128) for h in heads])
    og = o[torch.from_numpy(qrows).to(dev)].double().cpu().numpy()[:, cols]
    want = o_ref[:, cols]
    lg = lse[:, torch.from_numpy(qrows).to(dev)].double().cpu().numpy()[heads]
    g3 = {"max_abs": float(np.abs(og - want).max()),
          "rel_l2": float(np.linalg.norm(og - want) / np.linalg.norm(want)),
          "lse_max_abs": float(np.abs(lg - lse_ref[heads]).max())}
    g3["pass"] = g3["max_abs"] <= 2e-2 and g3["rel_l2"] <= 5e-3

    qkv_flop = 2.0 * len(rows) * d * 3 * d
    att_flop = 4.0 * len(qrows) * N * len(heads) * 128
    return {
        "value": (qkv_flop + att_flop) / (t_qkv + t_att) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "QKV-quant of %d token rows (%.2f s, %.1f tokens/s) + attention of %d query rows x "
                  "%d heads x all %d keys decoded from the GPU's packed store (%.2f s)"
                  % (len(rows), t_qkv, len(rows) / t_qkv, len(qrows), len(heads), N, t_att),
        "qkv_tokens_per_s": len(rows) / t_qkv,
        "attention_tflops": att_flop / t_att / 1e12,
        "full_problem_s_extrapolated": t_qkv * N / len(rows) + t_att * (N / len(qrows)) * (H / len(heads)),
        "cpu_model": cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "gates_on_sample": {"G2": g2, "G3": g3},
    }


if __name__ == "__main__":
    main()
