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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
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
    ap.add_argument("--sweep", choices=("batch", "query"), default=None,
                    help="instead of the benchmark line: step throughput of the C2 layer "
                         "over batch sizes 1..64 (query 64 window + 64 tracked) or over query "
                         "lengths 32..512 per sequence (B=32); one JSON line per point")
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

        def one_step(ev=None):
            with torch.cuda.stream(stream):
                flush.fill_(1)
            if ev is not None:
                ev[0].record(stream)
            bufs.qkv(stream)
            if ev is not None:
                ev[1].record(stream)
            bufs.attention(stream)
            if ev is not None:
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
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for i in range(args.steps):
            one_step(evs[i])
        torch.cuda.synchronize()
        el = lambda a, b: float(np.mean([e[a].elapsed_time(e[b]) for e in evs]))
        ms = el(0, 3)
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


def cpu_baseline(inp, n_seqs, budget_s=12.0):
    """The oracle, untuned, on the leading sequences of the same batch: at most
    n_seqs of them, stopping once budget_s seconds of CPU work are spent."""
    import numpy as np
    from kv_cache_attention_step_amd.workload import sequence_inputs
    from oracle import flashcache_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = inp.cfg
    n = min(n_seqs, inp.B)
    tokens = 0
    t0 = time.perf_counter()
    for b in range(n):
        s = sequence_inputs(inp, b)
        O.flash_cache_step(s["hidden"], s["positions"], s["cu_q"], s["cu_k"], inp.w_qkv,
                           cfg.n_heads, cfg.head_dim, cfg.rope_base, s["k_cache"], s["v_cache"],
                           s["block_table"], cfg.page_size, s["cand"], cfg.track, cfg.dtype)
        tokens += s["q1"] - s["q0"]
        if time.perf_counter() - t0 >= budget_s:
            n = b + 1
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "query-tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} of {inp.B} sequences of the same batch ({tokens} query tokens), "
                      f"full step each (fp64 projection, RoPE, cache write, attention, "
                      f"importance, top-k); {dt:.1f} s"}


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
    del logits
    return {"rows": R, "vocab": cfg.vocab, "avg_us": round(us, 2),
            "rows_per_s": round(R / (us * 1e-6), 1),
            "achieved_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


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
    wsb = fc.fc_attention_workspace_size(B, T_q, T_k, H, D, 0)
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
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


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
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        return sweep_main(args)
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

    def one_step(ev=None):
        if flush is not None:
            with torch.cuda.stream(stream):
                flush.fill_(1)
        if ev is not None:
            ev[0].record(stream)
        bufs.qkv(stream)
        if ev is not None:
            ev[1].record(stream)
        bufs.attention(stream)
        if ev is not None:
            ev[2].record(stream)
        bufs.topk(stream)
        if ev is not None:
            ev[3].record(stream)

    if args.calib:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k1 = np.array([e[0].elapsed_time(e[1]) for e in evs])
    k2 = np.array([e[1].elapsed_time(e[2]) for e in evs])
    k3 = np.array([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    ms_per_step = float(step_ms.mean())
    work = step_work(inp)
    k1_us, k2_us, k3_us = float(k1.mean()) * 1e3, float(k2.mean()) * 1e3, float(k3.mean()) * 1e3
    kernels = {
        "qkv_rope_cache_write": {
            "avg_us": round(k1_us, 2), "bound": "mfma",
            "achieved_tflops": round(work["qkv_flops"] / (k1_us * 1e-6) / 1e12, 1),
            "frac": round(work["qkv_flops"] / (k1_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "varlen_bidir_attention": {
            "avg_us": round(k2_us, 2), "bound": "hbm",
            "achieved_gbs": round(work["attn_bytes"] / (k2_us * 1e-6) / 1e9, 1),
            "frac": round(work["attn_bytes"] / (k2_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "importance_topk": {
            "avg_us": round(k3_us, 2), "bound": "hbm",
            "achieved_gbs": round(work["topk_bytes"] / (k3_us * 1e-6) / 1e9, 1),
            "frac": round(work["topk_bytes"] / (k3_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    # HBM bytes per launch from the committed counter runs (null once the kernel
    # sources differ from those the counters were taken on)
    from kv_cache_attention_step_amd.profiling import load_traffic
    for name, kd in kernels.items():
        kd["traffic_bytes"] = load_traffic(TRAFFIC_FILE, name)
    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"])
    kd = kernels[dominant]
    if kd["bound"] == "mfma":
        roof = {"bound": "mfma", "kernel": dominant, "achieved": kd["achieved_tflops"],
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": kd["frac"],
                "traffic": kd["traffic_bytes"]}
    else:
        roof = {"bound": "hbm", "kernel": dominant, "achieved": kd["achieved_gbs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kd["frac"],
                "traffic": kd["traffic_bytes"]}
    verify = None if args.no_verify else verify_component(torch, args)
    verify_attn = None if args.no_verify else verify_attention_component(torch, args)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seqs)
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
        "verify_accept_c4": verify,
        "verify_attention_c4": verify_attn,
        "settle": {"seconds": args.settle_s, "steps": settle_steps},
        "step_ms_min": round(float(step_ms.min()), 4),
        "wall_s_timed_loop": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
