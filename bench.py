#!/usr/bin/env python3
"""Benchmark of one Flash-Cache denoising step on one MI355X.

A step is the whole hot path for one layer: fused QKV projection + RoPE +
paged cache write -> bidirectional varlen attention with fused importance ->
top-k reselection, on the batched varlen workload (B=32, LLaDA-8B-shaped layer,
caches of 768..1536 positions, 128 query tokens per sequence). Inputs are seeded
synthetic data already resident in device memory when timing starts. Between
steps a 512 MiB buffer is overwritten so that no step finds the previous step's
weights or cache in the 256 MB Infinity Cache (each layer of a real model has its
own weights).

Prints ONE JSON line (rank 0). Per-kernel times come from HIP events recorded
on the stream the kernels run on.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
# rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch of the C2 step kernels
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c2_step_kernels.pmc_traffic.json")
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--no-flush", action="store_true", help="do not evict the Infinity Cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the Flash-Verify accept-test component")
    ap.add_argument("--calib", action="store_true",
                    help="run one 256 MiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed steps for this many seconds before the warm-up steps, so "
                         "that the GPU clocks reach their sustained state")
    ap.add_argument("--cpu-seqs", type=int, default=32,
                    help="sequences of the batch the CPU oracle baseline runs")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0,
                    help="seconds of CPU work for each oracle baseline leg (all threads, 1 thread)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the timing of the step captured as a HIP graph")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured-peak probes (MFMA rate, KV-cache streaming rate)")
    ap.add_argument("--sweep", choices=("batch", "query"), default=None,
                    help="instead of the benchmark line: step throughput of the C2 layer "
                         "over batch sizes 1..64 (query 64 window + 64 tracked) or over query "
                         "lengths 32..512 per sequence (B=32); one JSON line per point")
    ap.add_argument("--ab-lib", default=None, metavar="PATH",
                    help="A/B in one process: time one entry point (--ab-call) of the C2 step "
                         "(C4 for verify_attention) with another build of libflashcache.so at "
                         "PATH against this tree's build, alternating calls, Infinity Cache "
                         "evicted before each; checks the outputs against each other and exits")
    ap.add_argument("--ab-call", default="attention",
                    choices=("assemble", "qkv", "attention", "topk", "step", "verify_attention"))
    ap.add_argument("--probe-policies", action="store_true",
                    help="time the KV-stream probe on the C2 cache with each cache policy of its "
                         "K-only pass (does a cache serve the second read of K?) and exit")
    ap.add_argument("--only", choices=tuple(COMPONENTS), default=None,
                    help="run only this verify-shaped component and print its JSON object "
                         "(for per-component counter runs; not the benchmark line)")
    return ap.parse_args()


def sweep_main(args):
    """Throughput of the C2-shaped step against batch size or query length (the
    pages' throughput-vs-batch-size and query-size measurements, on synthetic
    inputs of this layer shape)."""
    import dataclasses
    import numpy as np
    import torch
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import workload as W
    from kv_cache_attention_step_amd.runner import StepBuffers

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    if args.sweep == "batch":
        points = [dict(batch=b) for b in (1, 2, 4, 8, 16, 32, 64)]
    else:
        points = [dict(window=q // 2, track=q // 2) for q in (32, 64, 128, 256, 512)]
    for pt in points:
        cfg = dataclasses.replace(CF.C2, **pt)
        inp = W.make_step_inputs(cfg)
        bufs = StepBuffers(inp, device="cuda:0")

        def one_step(ev=None, split=False):
            with torch.cuda.stream(stream):
                flush.fill_(1)
            if ev is not None:
                ev[0].record(stream)
            bufs.assemble(stream)
            bufs.qkv(stream)
            if split:
                ev[1].record(stream)
            bufs.attention(stream)
            if split:
                ev[2].record(stream)
            bufs.topk(stream)
            if ev is not None:
                ev[3].record(stream)

        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            one_step()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            one_step()
        mk = lambda: [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        evs_step, evs = mk(), mk()
        for i in range(args.steps):      # step time: events at the step boundaries only
            one_step(evs_step[i])
        for i in range(args.steps):      # kernel intervals: events between the kernels
            one_step(evs[i], split=True)
        torch.cuda.synchronize()
        el = lambda a, b, e_=None: float(np.mean([e[a].elapsed_time(e[b]) for e in (e_ or evs)]))
        ms = el(0, 3, evs_step)
        print(json.dumps({"sweep": args.sweep, "batch": inp.B, "query_per_seq": cfg.window + cfg.track,
                          "query_tokens": inp.T_q, "cache_tokens": inp.T_k,
                          "ms_per_step": round(ms, 4),
                          "query_tokens_per_s": round(inp.T_q / (ms * 1e-3), 1),
                          "qkv_us": round(el(0, 1) * 1e3, 2), "attention_us": round(el(1, 2) * 1e3, 2),
                          "topk_us": round(el(2, 3) * 1e3, 2)}), flush=True)
        del bufs
        torch.cuda.empty_cache()


def step_work(inp):
    """Algorithmic work per step (one layer)."""
    cfg = inp.cfg
    T_q, T_k, d, H, D = inp.T_q, inp.T_k, cfg.d_model, cfg.n_heads, cfg.head_dim
    esz = 2 if cfg.dtype == "bf16" else 4
    qkv_flops = 2.0 * T_q * (3 * d) * d
    qkv_bytes = (T_q * d + 3 * d * d + 3 * T_q * d) * esz + T_q * 8   # in, W, q/k/v out, pos+slot
    kv_bytes = 2.0 * T_k * H * D * esz                                 # K and V once
    attn_bytes = kv_bytes + 2.0 * T_q * d * esz + H * T_k * 4.0        # + Q + O + importance
    attn_flops = sum(4.0 * (int(inp.cu_seqlens_q[b + 1] - inp.cu_seqlens_q[b])) *
                     int(inp.cu_seqlens_k[b + 1] - inp.cu_seqlens_k[b]) * D * H
                     for b in range(inp.B))
    topk_bytes = H * T_k * 4.0 + T_k
    return dict(qkv_flops=qkv_flops, qkv_bytes=qkv_bytes, attn_bytes=attn_bytes,
                attn_flops=attn_flops, topk_bytes=topk_bytes)


def _oracle_rate(inp, n_seqs, budget_s):
    """Query tokens per second of the untuned oracle over the leading sequences
    of the batch (full step each), stopping once budget_s seconds are spent."""
    from kv_cache_attention_step_amd.workload import sequence_inputs
    from oracle import flashcache_oracle as O
    cfg = inp.cfg
    n = min(n_seqs, inp.B)
    tokens = 0
    positions, _ = O.assemble_batch(inp.tracked, inp.window_start, inp.window_len)
    t0 = time.perf_counter()
    for b in range(n):
        s = sequence_inputs(inp, b, positions)
        O.flash_cache_step(s["hidden"], s["positions"], s["cu_q"], s["cu_k"], inp.w_qkv,
                           cfg.n_heads, cfg.head_dim, cfg.rope_base, s["k_cache"], s["v_cache"],
                           s["block_table"], cfg.page_size, s["cand"], cfg.track, cfg.dtype)
        tokens += s["q1"] - s["q0"]
        if time.perf_counter() - t0 >= budget_s:
            n = b + 1
            break
    dt = time.perf_counter() - t0
    return tokens / dt, n, tokens, dt


def cpu_baseline(inp, n_seqs, budget_s=10.0):
    """The oracle, untuned, on the leading sequences of the same batch, twice:
    with the BLAS thread pool at its default size and with one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    nproc = os.cpu_count() or 1
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    rate, n, tokens, dt = _oracle_rate(inp, n_seqs, budget_s)
    with threadpool_limits(limits=1):
        rate1, n1, tokens1, dt1 = _oracle_rate(inp, n_seqs, budget_s)
    return {"value": round(rate, 1), "unit": "query-tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} of {inp.B} sequences of the same batch ({tokens} query tokens), "
                      f"full step each (fp64 projection, RoPE, cache write, attention, "
                      f"importance, top-k); {dt:.1f} s",
            "host_nproc": nproc, "host_affinity_cpus": affinity,
            "one_thread": {"value": round(rate1, 1), "unit": "query-tokens/s", "cores": 1,
                           "sample": f"{n1} sequences ({tokens1} query tokens); {dt1:.1f} s"}}


def measured_peaks(torch, bufs, flush, stream, reps=20):
    """Rates measured on this device: the sustained bf16 MFMA rate (register
    operands only), and the paged KV cache streamed with the attention
    kernel's access pattern (K and V once; K, then K and V), on the step's own
    cache with the Infinity Cache flushed before every run."""
    import numpy as np
    from kv_cache_attention_step_amd import flashcache as fc
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(max(4 * n_cu, bufs.B * bufs.H), dtype=torch.float32, device="cuda:0")

    def timed(fn, flush_first):
        ts = []
        for i in range(reps + 3):
            if flush_first:
                with torch.cuda.stream(stream):
                    flush.fill_(4)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            if i >= 3:
                ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3

    blocks, iters = 4 * n_cu, 4096
    us = timed(lambda: fc.fc_probe_mfma_bf16(blocks, iters, sink, stream), False)
    mfma_tflops = blocks * 4 * iters * 8 * 32768.0 / (us * 1e-6) / 1e12
    inp = bufs.inp
    kv_bytes = 2.0 * inp.T_k * bufs.H * bufs.D * 2
    stream_us = {}
    for passes in (1, 2):
        stream_us[passes] = timed(lambda: fc.fc_probe_kv_stream(
            bufs.k_cache, bufs.v_cache, bufs.block_table, inp.max_pages, inp.cfg.page_size,
            bufs.cu_k, bufs.B, bufs.H, bufs.D, passes, sink, stream), flush is not None)
    return {"mfma_bf16_tflops": round(mfma_tflops, 1), "mfma_probe_us": round(us, 1),
            "kv_stream_one_pass_us": round(stream_us[1], 2),
            "kv_stream_one_pass_gbs": round(kv_bytes / (stream_us[1] * 1e-6) / 1e9, 1),
            "kv_stream_two_pass_us": round(stream_us[2], 2),
            "kv_stream_two_pass_gbs": round(1.5 * kv_bytes / (stream_us[2] * 1e-6) / 1e9, 1),
            "kv_bytes": kv_bytes}


def probe_policies_main(args):
    """The two-pass K/V stream of the importance path (K, then K and V) on the C2
    cache, with each cache policy on the K-only pass (the K and V pass stays
    nontemporal), against one pass over K and V and one over K alone. If a policy
    let the Infinity Cache or L2 serve the second read of K, the two-pass time would
    fall toward the one-pass time plus a fraction of the K pass."""
    import numpy as np
    import torch
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd import workload as W
    from kv_cache_attention_step_amd.runner import StepBuffers
    torch.cuda.set_device(0)
    inp = W.make_step_inputs(CF.C2)
    bufs = StepBuffers(inp, device="cuda:0")
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(bufs.B * bufs.H, dtype=torch.float32, device="cuda:0")
    kv_bytes = 2.0 * inp.T_k * bufs.H * bufs.D * 2
    cases = [("K and V once, nontemporal", 1, 0, kv_bytes)] + [
        (f"K ({name}), then K and V (nontemporal)", 2, pol, 1.5 * kv_bytes)
        for pol, name in enumerate(("nontemporal", "default", "sc1", "sc0"))]
    run = lambda c: fc.fc_probe_kv_stream(bufs.k_cache, bufs.v_cache, bufs.block_table,
                                          inp.max_pages, inp.cfg.page_size, bufs.cu_k, bufs.B,
                                          bufs.H, bufs.D, c[1], sink, stream, k_policy=c[2])
    for c in cases:   # warm-up, and every case launches
        run(c)
    torch.cuda.synchronize()
    times = {c[0]: [] for c in cases}
    for rep in range(args.steps):   # interleaved, Infinity Cache evicted before each run
        for c in cases:
            flush.fill_(rep & 255)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(c)
            e1.record(stream)
            e1.synchronize()
            times[c[0]].append(e0.elapsed_time(e1) * 1e3)
    for name, passes, pol, nbytes in cases:
        us = float(np.median(times[name]))
        print(json.dumps({"probe": "kv_stream", "case": name, "k_passes": passes, "k_policy": pol,
                          "median_us": round(us, 2), "bytes_requested": nbytes,
                          "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "runs": args.steps}),
              flush=True)


def ab_main(args):
    """A/B timing of one entry point between two builds of the library in one
    process (same inputs, same device state): calls alternate A B / B A, each after
    the Infinity Cache is evicted, HIP events around the call. The outputs of one
    call of each build are compared (bit-identical, or the largest difference of
    the bf16 outputs)."""
    import ctypes
    import numpy as np
    import torch
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd import workload as W
    from kv_cache_attention_step_amd.runner import StepBuffers, VerifyBuffers

    def open_lib(path):
        lib = ctypes.CDLL(os.path.abspath(path))
        for name, (argt, res) in fc._SIGS.items():
            f = getattr(lib, name)
            f.argtypes, f.restype = argt, res
        return lib
    libs = {"A (this tree)": fc.load(), "B (" + args.ab_lib + ")": open_lib(args.ab_lib)}
    torch.cuda.set_device(0)
    if args.ab_call == "verify_attention":
        vb = VerifyBuffers(W.make_verify_inputs(CF.C4, with_logits=False), device="cuda:0")
        vb.qkv()
        fn, outs = vb.attention, lambda: {"attn_out": vb.step.attn_out}
    else:
        b = StepBuffers(W.make_step_inputs(CF.C2), device="cuda:0")
        b.run()
        fn = {"assemble": b.assemble, "qkv": b.qkv, "attention": b.attention, "topk": b.topk,
              "step": b.run}[args.ab_call]
        outs = lambda: {"positions": b.positions, "q_out": b.q_out, "slot_mapping": b.slot_mapping,
                        "attn_out": b.attn_out, "importance": b.importance,
                        "topk_pos": b.topk_pos, "topk_count": b.topk_count}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    got = {}
    for k, lib in libs.items():
        fc._lib = lib
        fn()
        torch.cuda.synchronize()
        got[k] = {n: t.clone() for n, t in outs().items()}
    (ka, ga), (kb, gb) = got.items()
    diffs = {}
    for n in ga:
        if not torch.equal(ga[n], gb[n]):
            a, c = ga[n], gb[n]
            if n in ("q_out", "attn_out"):   # bf16 bits: largest difference of the values
                diffs[n] = float((a.view(torch.bfloat16).float() - c.view(torch.bfloat16).float())
                                 .abs().max())
            elif a.dtype == torch.float32:
                diffs[n] = float((a - c).abs().max())
            else:
                diffs[n] = "differs"
    t0 = time.time()
    while time.time() - t0 < args.settle_s:
        fn()
    torch.cuda.synchronize()
    times = {k: [] for k in libs}
    for r in range(args.steps):
        for k in (list(libs) if r % 2 == 0 else list(libs)[::-1]):
            fc._lib = libs[k]
            flush.fill_(r & 255)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            times[k].append(e0.elapsed_time(e1) * 1e3)
    fc._lib = libs["A (this tree)"]
    print(json.dumps({"ab": args.ab_call, "runs": args.steps,
                      "median_us": {k: round(float(np.median(v)), 2) for k, v in times.items()},
                      "min_us": {k: round(float(np.min(v)), 2) for k, v in times.items()},
                      "outputs_bit_identical": not diffs, "output_differences": diffs}), flush=True)


def _traffic(name):
    """HBM bytes per launch of a kernel from the committed counter runs (None once
    the kernel sources differ from those the counters were taken on)."""
    from kv_cache_attention_step_amd.profiling import load_traffic
    return load_traffic(TRAFFIC_FILE, name)


def verify_component(torch, args):
    """The Flash-Verify accept test at the verify-shaped workload (B=32, 16..128
    verified positions per sequence, two views, vocab 126464): logits drawn on the
    device (values do not change the kernel's work), timed with HIP events."""
    import numpy as np
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import flashcache as fc
    cfg = CF.C4
    from kv_cache_attention_step_amd import workload as W
    rng = W.rng_for(cfg.seed, 0)
    W.draw_lengths(cfg, rng)
    _, _ = W.draw_paging(cfg, np.full(cfg.batch, cfg.cache_len_fixed), rng)
    vlen = rng.integers(cfg.verify_len[0], cfg.verify_len[1] + 1, size=cfg.batch)
    cu_p = torch.tensor(np.concatenate([[0], np.cumsum(vlen)]), dtype=torch.int32, device="cuda:0")
    n_pos = int(vlen.sum())
    R = 2 * n_pos
    gen = torch.Generator(device="cuda:0").manual_seed(cfg.seed)
    logits = (torch.randn((R, cfg.vocab), generator=gen, device="cuda:0") * cfg.logit_std).to(torch.bfloat16)
    draft = torch.randint(0, cfg.vocab, (n_pos,), generator=gen, device="cuda:0", dtype=torch.int32)
    am = torch.empty(R, dtype=torch.int32, device="cuda:0")
    cf = torch.empty(R, dtype=torch.float32, device="cuda:0")
    ar = torch.empty(R, dtype=torch.uint8, device="cuda:0")
    ap = torch.empty(n_pos, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.Stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    ts = []
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s / 2:
        for _ in range(10):
            with torch.cuda.stream(stream):
                flush.fill_(2)
            fc.fv_verify_accept(logits, cfg.vocab, cu_p, cfg.batch, R, draft, cfg.tau, am, cf, ar,
                                ap, stream)
        torch.cuda.synchronize()
    for i in range(args.warmup + args.steps):
        with torch.cuda.stream(stream):
            flush.fill_(2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fc.fv_verify_accept(logits, cfg.vocab, cu_p, cfg.batch, R, draft, cfg.tau, am, cf, ar, ap,
                            stream)
        e1.record(stream)
        if i >= args.warmup:
            ts.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ts])) * 1e3
    nbytes = R * cfg.vocab * 2.0 + R * 9.0 + n_pos * 5.0
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = _verify_oracle_rate(torch, logits, vlen, draft, cfg.tau, budget_s=3.0)
    del logits
    return {"rows": R, "vocab": cfg.vocab, "avg_us": round(us, 2),
            "rows_per_s": round(R / (us * 1e-6), 1),
            "achieved_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic_bytes": _traffic("verify:verify_rows"),
            "cpu_oracle": cpu}


def confidence_component(torch, args):
    """Confidence-aware acceptance (one view, no drafts, the at-least-one rule) at the
    verify-shaped workload: one logit row per verified position (16..128 per sequence,
    B=32, vocab 126464), logits drawn on the device, timed with HIP events after the
    Infinity Cache is evicted."""
    import numpy as np
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd import workload as W
    cfg = CF.C4
    rng = W.rng_for(cfg.seed, 0)
    W.draw_lengths(cfg, rng)
    _, _ = W.draw_paging(cfg, np.full(cfg.batch, cfg.cache_len_fixed), rng)
    vlen = rng.integers(cfg.verify_len[0], cfg.verify_len[1] + 1, size=cfg.batch)
    cu_p = torch.tensor(np.concatenate([[0], np.cumsum(vlen)]), dtype=torch.int32, device="cuda:0")
    n_pos = int(vlen.sum())
    gen = torch.Generator(device="cuda:0").manual_seed(cfg.seed + 1)
    logits = (torch.randn((n_pos, cfg.vocab), generator=gen, device="cuda:0") * cfg.logit_std).to(torch.bfloat16)
    am = torch.empty(n_pos, dtype=torch.int32, device="cuda:0")
    cf = torch.empty(n_pos, dtype=torch.float32, device="cuda:0")
    acc = torch.empty(n_pos, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.Stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    ts = []
    for i in range(args.warmup + args.steps):
        with torch.cuda.stream(stream):
            flush.fill_(2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fc.fv_confidence_accept(logits, cfg.vocab, cu_p, cfg.batch, n_pos, cfg.tau, 1, am, cf, acc,
                                stream)
        e1.record(stream)
        if i >= args.warmup:
            ts.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ts])) * 1e3
    nbytes = n_pos * cfg.vocab * 2.0 + n_pos * 9.0
    del logits
    return {"rows": n_pos, "vocab": cfg.vocab, "avg_us": round(us, 2),
            "rows_per_s": round(n_pos / (us * 1e-6), 1),
            "achieved_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic_bytes": _traffic("confidence:verify_rows")}


def _verify_oracle_rate(torch, logits, vlen, draft, tau, budget_s):
    """Rows per second of the untuned oracle's accept test (argmax, confidence and
    the two-view rule, fp64) on the leading sequences of the same logits, until
    budget_s seconds are spent. numpy's element-wise work runs on one thread."""
    import numpy as np
    from oracle import flashcache_oracle as O
    cu = np.concatenate([[0], np.cumsum(vlen)])
    dr = draft.cpu().numpy()
    rows, spent, b = 0, 0.0, 0
    for b in range(len(vlen)):
        r0, r1 = 2 * int(cu[b]), 2 * int(cu[b + 1])
        bits = logits[r0:r1].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        O.verify_accept(bits, np.array([0, int(vlen[b])]), dr[cu[b]:cu[b + 1]], tau)
        spent += time.perf_counter() - t0
        rows += r1 - r0
        if spent >= budget_s:
            break
    return {"value": round(rows / spent, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} logit rows ({b + 1} of {len(vlen)} sequences, both views), "
                      f"{spent:.1f} s"}


def verify_attention_component(torch, args):
    """Attention of the verify-shaped step (B=32, 4096-key caches): both views of
    each sequence (2 x 16..128 query rows, the same draws as the accept test)
    attend to the sequence's paged cache with a one-pass softmax and no
    importance. Cache, queries and page table are drawn on the device (values do
    not change the kernel's work); timed with HIP events like the accept test."""
    import math
    import numpy as np
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd import workload as W
    cfg = CF.C4
    rng = W.rng_for(cfg.seed, 0)
    W.draw_lengths(cfg, rng)
    L = np.full(cfg.batch, cfg.cache_len_fixed)
    table, num_pages = W.draw_paging(cfg, L, rng)
    vlen = rng.integers(cfg.verify_len[0], cfg.verify_len[1] + 1, size=cfg.batch)
    Qb = 2 * vlen
    dev = "cuda:0"
    B, H, D, ps = cfg.batch, cfg.n_heads, cfg.head_dim, cfg.page_size
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(Qb)]), dtype=torch.int32, device=dev)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(L)]), dtype=torch.int32, device=dev)
    T_q, T_k = int(Qb.sum()), int(L.sum())
    bt = torch.tensor(table, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 1)
    kc = (torch.randn((num_pages, H, ps, D), generator=gen, device=dev) * cfg.kv_std).to(torch.bfloat16)
    vc = (torch.randn((num_pages, H, ps, D), generator=gen, device=dev) * cfg.kv_std).to(torch.bfloat16)
    q = torch.randn((T_q, H, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    wsb = fc.fc_attention_workspace_size(B, T_q, T_k, H, D, 0, int(Qb.max()))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def call():
        fc.fc_varlen_bidir_attention(q, kc, vc, bt, table.shape[1], ps, cu_q, cu_k, B,
                                     int(Qb.max()), T_k, H, D, 1.0 / math.sqrt(D), out, None, 0,
                                     ws, wsb, fc.FC_DTYPE_BF16, stream)
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s / 2:
        for _ in range(10):
            with torch.cuda.stream(stream):
                flush.fill_(3)
            call()
        torch.cuda.synchronize()
    ts = []
    for i in range(args.warmup + args.steps):
        with torch.cuda.stream(stream):
            flush.fill_(3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        if i >= args.warmup:
            ts.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ts])) * 1e3
    nbytes = 2.0 * T_k * H * D * 2 + 2.0 * T_q * H * D * 2
    del kc, vc
    return {"query_rows": T_q, "cache_tokens": T_k, "avg_us": round(us, 2),
            "algorithmic_bytes": nbytes, "achieved_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic_bytes": _traffic("verify_attention:attention_one_pass")}


def _timed(torch, stream, fn, args, flush=None, reps=None):
    """Median of HIP-event intervals of fn on `stream` after a settle phase
    (the Infinity Cache flushed before each call when `flush` is given)."""
    import numpy as np
    reps = reps or args.steps
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s / 2:
        for _ in range(5):
            if flush is not None:
                with torch.cuda.stream(stream):
                    flush.fill_(5)
            fn()
        torch.cuda.synchronize()
    ts = []
    for i in range(args.warmup + reps):
        if flush is not None:
            with torch.cuda.stream(stream):
                flush.fill_(5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        if i >= args.warmup:
            ts.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3


def verify_views_component(torch, args):
    """Flash-Verify's two views with view-private K/V on the verify-shaped
    workload (B=32, 4096-token caches, 16..128 verified positions per sequence,
    the same draws as the accept test): private pages forked, both views
    projected into them, each view attending to its own cache, and the commit
    of a random half of the positions; each stage timed on its own."""
    import numpy as np
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd import workload as W
    cfg = CF.C4
    dev = "cuda:0"
    rng = W.rng_for(cfg.seed, 0)
    W.draw_lengths(cfg, rng)
    L = np.full(cfg.batch, cfg.cache_len_fixed)
    table, num_pages = W.draw_paging(cfg, L, rng)
    n = rng.integers(cfg.verify_len[0], cfg.verify_len[1] + 1, size=cfg.batch)
    B, H, D, ps, d = cfg.batch, cfg.n_heads, cfg.head_dim, cfg.page_size, cfg.d_model
    P = int((n.max() + ps - 1) // ps + 1)
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 2)
    total = num_pages + 2 * B * P
    kc = (torch.randn((total, H, ps, D), generator=gen, device=dev) * cfg.kv_std).to(torch.bfloat16)
    vc = (torch.randn((total, H, ps, D), generator=gen, device=dev) * cfg.kv_std).to(torch.bfloat16)
    t32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device=dev)
    bt, cu_k = t32(table), t32(np.concatenate([[0], np.cumsum(L)]))
    vs = t32(L - n)
    cu_p = t32(np.concatenate([[0], np.cumsum(n)]))
    nv = np.repeat(n, 2)
    cu_q = t32(np.concatenate([[0], np.cumsum(nv)]))
    cu_kv = t32(np.concatenate([[0], np.cumsum(np.repeat(L, 2))]))
    pos = t32(np.concatenate([np.concatenate([np.arange(L[b] - n[b], L[b])] * 2) for b in range(B)]))
    T_q, T_kv = int(nv.sum()), int(2 * L.sum())
    hidden = torch.randn((T_q, d), generator=gen, device=dev).to(torch.bfloat16)
    w = (torch.randn((3 * d, d), generator=gen, device=dev) * cfg.weight_std).to(torch.bfloat16)
    vt = torch.full((2 * B, table.shape[1]), -1, dtype=torch.int32, device=dev)
    q_out = torch.empty((T_q, H, D), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q_out)
    qws = fc.fc_qkv_workspace_size(T_q, d, D, fc.FC_DTYPE_BF16)
    qw = torch.empty(max(qws, 1), dtype=torch.uint8, device=dev)
    aws = fc.fc_attention_workspace_size(2 * B, T_q, T_kv, H, D, 0, int(n.max()))
    aw = torch.empty(max(aws, 1), dtype=torch.uint8, device=dev)
    acc = (torch.rand(int(n.sum()), generator=gen, device=dev) < 0.5).to(torch.uint8)
    stream = torch.cuda.Stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    fork = lambda: fc.fv_fork_view_pages(kc, vc, bt, table.shape[1], ps, cu_k, vs, B, H, D,
                                         num_pages, P, vt, stream)
    proj = lambda: fc.fc_qkv_rope_cache_write(hidden, pos, cu_q, 2 * B, T_q, w, d, H, D,
                                              cfg.rope_base, kc, vc, vt, table.shape[1], ps, q_out,
                                              None, qw, qws, fc.FC_DTYPE_BF16, stream)
    attn = lambda: fc.fc_varlen_bidir_attention(q_out, kc, vc, vt, table.shape[1], ps, cu_q, cu_kv,
                                                2 * B, int(n.max()), T_kv, H, D, 1.0 / D ** 0.5,
                                                out, None, 0, aw, aws, fc.FC_DTYPE_BF16, stream)
    commit = lambda: fc.fv_commit_accepted(kc, vc, bt, vt, table.shape[1], ps, cu_p, vs, B,
                                           int(n.sum()), acc, H, D, stream)
    fork()
    res = {"rows": T_q, "positions": int(n.sum()),
           "fork_us": round(_timed(torch, stream, fork, args, flush), 2),
           "projection_us": round(_timed(torch, stream, proj, args, flush), 2),
           "attention_us": round(_timed(torch, stream, attn, args, flush), 2),
           "commit_us": round(_timed(torch, stream, commit, args, flush), 2)}
    # algorithmic bytes: the pages before a sequence's first private page once, each
    # view's private pages (from that page to the end) once per view, q and out
    first = (L - n) // ps * ps
    uniq = (first.sum() + 2 * (L - first).sum()) * H * D * 2 * 2 + 2.0 * T_q * d * 2
    res["attention_algorithmic_bytes"] = float(uniq)
    res["attention_gbs"] = round(uniq / (res["attention_us"] * 1e-6) / 1e9, 1)
    res["attention_frac_hbm"] = round(uniq / (res["attention_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    res["attention_traffic_bytes"] = _traffic("views:attention_one_pass")
    res["projection_tflops"] = round(2.0 * T_q * 3 * d * d / (res["projection_us"] * 1e-6) / 1e12, 1)
    del kc, vc
    return res


def lmhead_component(torch, args):
    """The LM head with the fused accept test on the verify-shaped rows (4366
    rows of d 4096 against a 126464-token vocabulary); dense bf16 MFMA work
    2 R V d, reported against the MFMA roofline."""
    import numpy as np
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd import workload as W
    cfg = CF.C4
    dev = "cuda:0"
    rng = W.rng_for(cfg.seed, 0)
    W.draw_lengths(cfg, rng)
    W.draw_paging(cfg, np.full(cfg.batch, cfg.cache_len_fixed), rng)
    n = rng.integers(cfg.verify_len[0], cfg.verify_len[1] + 1, size=cfg.batch)
    R = int(2 * n.sum())
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 3)
    h = torch.randn((R, cfg.d_model), generator=gen, device=dev).to(torch.bfloat16)
    w = (torch.randn((cfg.vocab, cfg.d_model), generator=gen, device=dev) * cfg.weight_std).to(torch.bfloat16)
    cu_p = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev)
    draft = torch.randint(0, cfg.vocab, (int(n.sum()),), generator=gen, device=dev, dtype=torch.int32)
    wsb = fc.fv_lmhead_workspace_size(R, cfg.vocab)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    am = torch.empty(R, dtype=torch.int32, device=dev)
    cf = torch.empty(R, dtype=torch.float32, device=dev)
    ar = torch.empty(R, dtype=torch.uint8, device=dev)
    ap = torch.empty(int(n.sum()), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    fn = lambda: fc.fv_lmhead_verify_accept(h, w, cfg.d_model, cfg.vocab, cu_p, cfg.batch, R,
                                            draft, cfg.tau, ws, wsb, am, cf, ar, ap, stream)
    us = _timed(torch, stream, fn, args, None, reps=max(5, args.steps // 5))
    flops = 2.0 * R * cfg.vocab * cfg.d_model
    tf = flops / (us * 1e-6) / 1e12
    del w
    return {"rows": R, "vocab": cfg.vocab, "avg_us": round(us, 1), "achieved_tflops": round(tf, 1),
            "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "logits_bytes_not_written": R * cfg.vocab * 2,
            "traffic_bytes": _traffic("lmhead:lmhead_partials")}


def stack_main(args):
    """Layer-stack workload: 32 layers x 32 block-wise denoising steps of one
    512-token generation (B=32). Prints one JSON line with the time per denoising
    step (all layers) and per generation."""
    import numpy as np
    import torch
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd.runner import LayerStackDriver
    cfg = CF.C3
    torch.cuda.set_device(0)
    drv = LayerStackDriver(cfg, device="cuda:0")
    stream = torch.cuda.Stream()
    # warm-up: one full generation (the cache and tracked sets evolve with it)
    for st in range(cfg.steps):
        drv.run_step(st, stream)
    torch.cuda.synchronize()
    drv = LayerStackDriver(cfg, device="cuda:0")
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(cfg.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        drv.run_step(st, stream)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    q_tokens = sum(x["T_q"] for x in drv.steps)
    out = {"metric": "layer-stack denoising step time (32 layers, B=32)",
           "value": round(float(ms.mean()), 4), "unit": "ms/step", "higher_is_better": False,
           "n_gpus": 1, "steps": cfg.steps, "dtype": cfg.dtype, "data": "synthetic",
           "config": {"workload": "C3: 32 layers x 32 denoising steps, block 16, track 48, "
                                  "B=32, caches 768..1536", "layers": cfg.layers},
           "ms_per_generation": round(float(ms.sum()), 3),
           "query_tokens_per_s": round(q_tokens * cfg.layers / (ms.sum() * 1e-3), 1),
           "step_ms_first_last": [round(float(ms[0]), 4), round(float(ms[-1]), 4)],
           "wall_s": round(wall, 3)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _stack_oracle_rate(cfg, budget_s=args.cpu_budget_s / 2)
    print(json.dumps(out), flush=True)


def _stack_oracle_rate(cfg, budget_s):
    """The untuned oracle on one layer of one denoising step with the full query
    (step 3: 16 window + 48 tracked rows per sequence), one sequence at a time
    (its own pages only) until budget_s seconds are spent: projection, RoPE, cache
    write, attention, importance, top-k and the output projection with residual.
    Extrapolated to all sequences and layers of a denoising step."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import flashcache_oracle as O
    from kv_cache_attention_step_amd import workload as W
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    H, D, ps, st = cfg.n_heads, cfg.head_dim, cfg.page_size, 3
    prompt_len, cache_len, table, num_pages, cu_k = W.multistep_base(cfg)
    kc, vc = W.stack_prefill(cfg, num_pages)
    w_qkv, w_o = W.layer_weights(cfg, 0)
    Q = W.step_query_lens(cfg, st)
    hid = W.step_hidden(cfg, st, cfg.batch * Q)
    cand = W.step_candidates(cfg, st, prompt_len, cu_k)
    spent, n = 0.0, 0
    for b in range(cfg.batch):
        L = int(cache_len[b])
        pages = table[b, :(L + ps - 1) // ps]
        tracked = [np.arange(prompt_len[b], prompt_len[b] + cfg.block_len * st, dtype=np.int64)]
        positions, cu_q = O.assemble_batch(tracked, prompt_len[b:b + 1] + cfg.block_len * st,
                                           cfg.block_len)
        h = hid[b * Q:(b + 1) * Q]
        t0 = time.perf_counter()
        r = O.flash_cache_step(h, positions, cu_q, np.array([0, L], np.int32), w_qkv, H, D,
                               cfg.rope_base, kc[pages], vc[pages],
                               np.arange(len(pages), dtype=np.int32)[None], ps,
                               cand[cu_k[b]:cu_k[b + 1]], cfg.track, cfg.dtype,
                               rms_eps=cfg.rms_eps)
        x = O.f64_to_bf16_bits(O.round_bf16(r["out"].reshape(len(positions), -1)))
        O.linear_residual(x, w_o, h, cfg.dtype)
        spent += time.perf_counter() - t0
        n += 1
        if spent >= budget_s:
            break
    ms_step = spent / n * cfg.batch * cfg.layers * 1e3
    return {"value": round(ms_step, 1), "unit": "ms/step", "cores": int(threads), "kind": "oracle",
            "sample": f"layer 0 of denoising step {st} ({Q} query rows per sequence) for {n} of "
                      f"{cfg.batch} sequences, {spent:.1f} s; x {cfg.batch} sequences / {n} x "
                      f"{cfg.layers} layers"}


def calibration_copy(torch):
    """One 256 MiB device copy and one 512 MiB fill: the references the HBM
    read and write byte counters are scaled by."""
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    fill = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    fill.fill_(1)
    torch.cuda.synchronize()
    del fill


COMPONENTS = {"verify": "verify_component", "confidence": "confidence_component",
              "verify_attention": "verify_attention_component",
              "views": "verify_views_component", "lmhead": "lmhead_component"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.only:
        import torch
        torch.cuda.set_device(0)
        if args.calib:
            calibration_copy(torch)
        res = globals()[COMPONENTS[args.only]](torch, args)
        print(json.dumps({"component": args.only, **res}), flush=True)
        return
    if args.sweep:
        return sweep_main(args)
    if args.probe_policies:
        return probe_policies_main(args)
    if args.ab_lib:
        return ab_main(args)
    if args.config == "C3":
        return stack_main(args)
    import numpy as np
    import torch
    from kv_cache_attention_step_amd import configs as CF
    from kv_cache_attention_step_amd import workload as W
    from kv_cache_attention_step_amd.runner import StepBuffers

    cfg = CF.CONFIGS[args.config]
    inp = W.make_step_inputs(cfg)
    torch.cuda.set_device(0)
    bufs = StepBuffers(inp, device="cuda:0")
    stream = torch.cuda.Stream()
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")

    def one_step(ev=None, split=False):
        """One step; events at its boundaries, and between its kernels when split
        (each event record between two kernels adds a ~5 us gap on the GPU, so
        the step time is taken from steps without them)."""
        if flush is not None:
            with torch.cuda.stream(stream):
                flush.fill_(1)
        if ev is not None:
            ev[0].record(stream)
        bufs.assemble(stream)
        if split:
            ev[1].record(stream)
        bufs.qkv(stream)
        if split:
            ev[2].record(stream)
        bufs.attention(stream)
        if split:
            ev[3].record(stream)
        bufs.topk(stream)
        if ev is not None:
            ev[4].record(stream)

    if args.calib:
        calibration_copy(torch)
    # settle: the clocks swing for the first tens of milliseconds of sustained load
    t_settle = time.perf_counter()
    settle_steps = 0
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(10):
            one_step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    mk = lambda: [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    # the timed steps: events only at each step's boundaries
    evs_step = mk()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(evs_step[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same number of steps again with events between the kernels, for the
    # per-kernel intervals
    evs = mk()
    for i in range(args.steps):
        one_step(evs[i], split=True)
    torch.cuda.synchronize()
    # the same step captured once as a HIP graph and replayed: the kernels are the
    # same, the host enqueues one graph instead of five launches
    graph_ms = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            bufs.assemble(stream)
            bufs.qkv(stream)
            bufs.attention(stream)
            bufs.topk(stream)
        torch.cuda.synchronize()
        gts = []
        for i in range(args.warmup + args.steps):
            if flush is not None:
                with torch.cuda.stream(stream):
                    flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            with torch.cuda.stream(stream):
                graph.replay()
            e1.record(stream)
            if i >= args.warmup:
                gts.append((e0, e1))
        torch.cuda.synchronize()
        graph_ms = round(float(np.median([a.elapsed_time(b) for a, b in gts])), 4)
        del graph
    seg = lambda a, b, e_=None: np.array([e[a].elapsed_time(e[b]) for e in (e_ or evs)]) * 1e3  # us
    k0, k1, k2, k3 = seg(0, 1), seg(1, 2), seg(2, 3), seg(3, 4)
    step_ms = seg(0, 4, evs_step) * 1e-3
    ms_per_step = float(np.median(step_ms))
    work = step_work(inp)
    peaks = None if args.no_probes else measured_peaks(torch, bufs, flush, stream)

    def entry(times, bound, amount, peak, mpeak=None):
        avg = float(times.mean())
        d = {"avg_us": round(avg, 2), "median_us": round(float(np.median(times)), 2),
             "bound": bound}
        rate = amount / (avg * 1e-6) / 1e12   # TFLOP/s or TB/s
        if bound == "mfma":
            d.update(achieved_tflops=round(rate, 1), frac=round(rate / peak, 4))
            if mpeak:
                d["frac_of_measured_mfma"] = round(rate / mpeak, 4)
        else:
            d.update(achieved_gbs=round(rate * 1e3, 1), frac=round(rate * 1e3 / peak, 4))
            if mpeak:
                d["frac_of_measured_stream"] = round(rate * 1e3 / mpeak, 4)
        return d

    mp_mfma = peaks["mfma_bf16_tflops"] if peaks else None
    mp_hbm = peaks["kv_stream_one_pass_gbs"] if peaks else None
    kernels = {
        "assemble_query": {"avg_us": round(float(k0.mean()), 2),
                           "median_us": round(float(np.median(k0)), 2), "bound": "launch"},
        "qkv_rope_cache_write": entry(k1, "mfma", work["qkv_flops"], MFMA_BF16_PEAK_TFLOPS, mp_mfma),
        "varlen_bidir_attention": entry(k2, "hbm", work["attn_bytes"], HBM_PEAK_GBS, mp_hbm),
        "importance_topk": entry(k3, "hbm", work["topk_bytes"], HBM_PEAK_GBS, mp_hbm),
    }
    if peaks:
        # the importance path reads K twice: the two-pass stream of the same
        # cache is that design's memory floor
        kernels["varlen_bidir_attention"]["two_pass_floor_us"] = peaks["kv_stream_two_pass_us"]
    # HBM bytes per launch from the committed counter runs (null once the kernel
    # sources differ from those the counters were taken on)
    from kv_cache_attention_step_amd.profiling import load_traffic
    for name, kd in kernels.items():
        if name != "assemble_query":
            kd["traffic_bytes"] = load_traffic(TRAFFIC_FILE, name)
    dominant = max((k for k in kernels if k != "assemble_query"),
                   key=lambda k: kernels[k]["avg_us"])
    kd = kernels[dominant]
    if kd["bound"] == "mfma":
        roof = {"bound": "mfma", "kernel": dominant, "achieved": kd["achieved_tflops"],
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": kd["frac"],
                "traffic": kd["traffic_bytes"], "measured_peak": mp_mfma,
                "frac_of_measured_peak": kd.get("frac_of_measured_mfma")}
    else:
        roof = {"bound": "hbm", "kernel": dominant, "achieved": kd["achieved_gbs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kd["frac"],
                "traffic": kd["traffic_bytes"], "measured_peak": mp_hbm,
                "frac_of_measured_peak": kd.get("frac_of_measured_stream")}
    verify = None if args.no_verify else verify_component(torch, args)
    confidence = None if args.no_verify else confidence_component(torch, args)
    verify_attn = None if args.no_verify else verify_attention_component(torch, args)
    verify_views = None if args.no_verify else verify_views_component(torch, args)
    lmhead = None if args.no_verify else lmhead_component(torch, args)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seqs, args.cpu_budget_s)
    L = inp.cache_len
    out = {
        "metric": "Flash-Cache step query-tokens/s at B=32 + % of HBM/MFMA roofline (1 GPU)",
        "value": round(inp.T_q / (ms_per_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: seeded N(0,1) hidden states, N(0,0.02) Wqkv, N(0,1.28) stale "
                "KV cache, random page tables; no trained weights or datasets",
        "config": {"workload": f"{cfg.name}: one Flash-Cache step of one layer (QKV+RoPE+paged "
                               f"cache write, bidirectional varlen attention + importance, "
                               f"top-k)",
                   "batch": inp.B, "d_model": cfg.d_model, "heads": cfg.n_heads,
                   "head_dim": cfg.head_dim, "query_tokens": inp.T_q,
                   "query_per_seq": f"{cfg.window} window + {cfg.track} tracked",
                   "cache_tokens": inp.T_k, "cache_len_range": [int(L.min()), int(L.max())],
                   "page_size": cfg.page_size, "infinity_cache_flushed": flush is not None},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "measured_peaks": peaks,
        "timing": {"statistic": "median of the timed steps' HIP-event intervals, events at "
                                "step boundaries only; kernel entries (mean and median) from "
                                "a second run of as many steps with events between kernels",
                   "ms_per_step_mean": round(float(step_ms.mean()), 4),
                   "ms_per_step_with_kernel_events": round(float(np.median(seg(0, 4))) * 1e-3, 4),
                   "ms_per_step_graph_replay": graph_ms},
        "verify_accept_c4": verify,
        "confidence_accept_c4": confidence,
        "verify_attention_c4": verify_attn,
        "verify_two_views_c4": verify_views,
        "lmhead_verify_c4": lmhead,
        "settle": {"seconds": args.settle_s, "steps": settle_steps},
        "step_ms_min": round(float(step_ms.min()), 4),
        "wall_s_timed_loop": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
