"""GPU parity for the layer-stack driver (block-wise denoising through several
layers) and the Flash-Verify-shaped step, against the CPU oracle."""
import dataclasses
import math
import sys
import time

import numpy as np
import pytest

from kv_cache_attention_step_amd import configs as CF
from kv_cache_attention_step_amd import workload as W
from oracle import flashcache_oracle as O
from tests import parity_util as PU

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from kv_cache_attention_step_amd import flashcache as fc
    fc.load()
    return torch


def oracle_stack_chain(cfg, n_layers, n_steps):
    """The oracle's own chain of denoising steps through the layer stack."""
    B, H, D = cfg.batch, cfg.n_heads, cfg.head_dim
    prompt_len, cache_len, table, num_pages, cu_k = W.multistep_base(cfg)
    kc, vc = W.stack_prefill(cfg, num_pages)
    caches = [(kc.copy(), vc.copy()) for _ in range(n_layers)]
    weights = [W.layer_weights(cfg, l) for l in range(n_layers)]
    tracked = [np.zeros(0, np.int64) for _ in range(B)]
    out = []
    for st in range(n_steps):
        Q = W.step_query_lens(cfg, st)
        # the query: tracked positions + block st (the masked window)
        positions, cu_q = O.assemble_batch(tracked, prompt_len + cfg.block_len * st,
                                           cfg.block_len)
        assert np.array_equal(cu_q, (np.arange(B + 1) * Q).astype(np.int32))
        h = O.bf16_to_f64(W.step_hidden(cfg, st, int(cu_q[-1])))
        imp = np.zeros((H, int(cu_k[-1])))
        for l in range(n_layers):
            r = O.flash_cache_step(O.f64_to_bf16_bits(h), positions, cu_q, cu_k, weights[l][0], H, D,
                                   cfg.rope_base, caches[l][0], caches[l][1], table,
                                   cfg.page_size, None, cfg.track, "bf16", rms_eps=cfg.rms_eps)
            caches[l] = (O.f64_to_bf16_bits(r["k_cache"]), O.f64_to_bf16_bits(r["v_cache"]))
            imp += r["importance"]
            x = O.f64_to_bf16_bits(O.round_bf16(r["out"].reshape(len(positions), -1)))
            h_unrounded = O.linear_residual(x, weights[l][1], O.f64_to_bf16_bits(h), "bf16")
            h = O.round_bf16(h_unrounded)
        cand = W.step_candidates(cfg, st + 1, prompt_len, cu_k)
        tp, tc, ts, score = O.importance_topk(imp, cu_k, cand, cfg.track)
        tracked = [tp[b, :tc[b]].astype(np.int64) for b in range(B)]
        out.append(dict(positions=positions, h=h, h_unrounded=h_unrounded, imp=imp, topk_pos=tp,
                        topk_count=tc, score=score, cand=cand, cu_k=cu_k))
    return out


STACK_SMALL = dataclasses.replace(CF.C3, name="C3-small", seed=31, batch=3, d_model=512, n_heads=4,
                                  prompt=(40, 100), gen_len=64, window=16, track=12, layers=3,
                                  steps=4)


def test_layer_stack_chain_small(torch_cuda):
    """Whole denoising chain (4 steps x 3 layers) against the oracle's own chain:
    query positions exact, tracked sets exact outside near-ties, hidden states
    and importance within tolerance."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import LayerStackDriver, to_host
    cfg = STACK_SMALL
    _say("case layer stack small chain")
    drv = LayerStackDriver(cfg)
    ref = oracle_stack_chain(cfg, cfg.layers, cfg.steps)
    snaps = {}

    def on_layer(st, l):
        if l == 0:
            snaps["positions"] = to_host(drv.positions[:drv.steps[st]["T_q"]]).copy()

    for st in range(cfg.steps):
        drv.run_step(st, on_layer=on_layer)
        torch.cuda.synchronize()
        r = ref[st]
        T_q = drv.steps[st]["T_q"]
        assert np.array_equal(snaps["positions"], r["positions"]), f"step {st}: query positions"
        PU.assert_close_chained(O.bf16_to_f64(to_host(drv.h[:T_q])), r["h_unrounded"],
                                f"step {st}: hidden after the stack")
        PU.assert_importance_close(to_host(drv.importance), r["imp"], f"step {st}: importance")
        gpos, gcnt = to_host(drv.topk_pos), to_host(drv.topk_count)
        cu_k = r["cu_k"]
        for b in range(cfg.batch):
            k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
            PU.assert_topk_matches(gpos[b], int(gcnt[b]), r["score"][k0:k1], r["cand"][k0:k1],
                                   cfg.track, f"step {st} seq {b}")
        # the chain only stays comparable while both sides track the same sets
        assert np.array_equal(gpos, r["topk_pos"].astype(np.int32)), \
            f"step {st}: tracked sets differ within the near-tie band; chain diverges"


def _layer_oracle_check(cfg, l, snap, drv, what):
    """One layer of the stack, teacher-forced on the inputs the GPU layer saw,
    every sequence. Projection: the oracle's fp64 q, k, v of the layer's hidden
    state (RMS-normalised) against the GPU's q_out and written cache rows; every
    other cache slot keeps its bytes. Attention and importance, kernel-isolated:
    the oracle attends with the GPU's own q_out and cache (the bytes the kernel
    read). Output projection: h + O Wo^T on the GPU's attention output."""
    H, D = cfg.n_heads, cfg.head_dim
    x = drv.steps[snap["step"]]
    T_q = len(snap["pos"])
    cu_q = np.arange(cfg.batch + 1, dtype=np.int32) * x["Q"]
    wq, wo = W.layer_weights(cfg, l)
    proj = O.qkv_rope_cache_write(snap["h_in"], snap["pos"], cu_q, wq, H, D, cfg.rope_base,
                                  snap["kc"], snap["vc"], drv.table, cfg.page_size, "bf16",
                                  rms_eps=cfg.rms_eps)
    PU.assert_close(O.bf16_to_f64(snap["q"]), proj["q"], "bf16", f"{what}: q")
    slots = proj["slot_mapping"]
    pg, off = slots // cfg.page_size, slots % cfg.page_size
    PU.assert_close(O.bf16_to_f64(snap["kc_after"][pg, :, off, :]), proj["k"], "bf16", f"{what}: K rows")
    PU.assert_close(O.bf16_to_f64(snap["vc_after"][pg, :, off, :]), proj["v"], "bf16", f"{what}: V rows")
    for name in ("kc", "vc"):
        before = snap[name].transpose(0, 2, 1, 3).reshape(-1, H, D).copy()
        after = snap[name + "_after"].transpose(0, 2, 1, 3).reshape(-1, H, D).copy()
        before[slots] = 0
        after[slots] = 0
        assert np.array_equal(before, after), f"{what}: {name} changed outside the written slots"
    out, imp = O.varlen_attention(O.bf16_to_f64(snap["q"]), O.bf16_to_f64(snap["kc_after"]),
                                  O.bf16_to_f64(snap["vc_after"]), drv.table, cfg.page_size, cu_q,
                                  drv.cu_k_np, 1.0 / math.sqrt(D))
    PU.assert_close(O.bf16_to_f64(snap["o"]), out, "bf16", f"{what}: attention out")
    PU.assert_importance_close(snap["imp"], imp, f"{what}: importance")
    for b in range(cfg.batch):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(drv.cu_k_np[b]), int(drv.cu_k_np[b + 1])
        PU.assert_close(O.bf16_to_f64(snap["o"][q0:q1]), out[q0:q1], "bf16",
                        f"{what}: attention out seq {b}")
        PU.assert_importance_close(snap["imp"][:, k0:k1], imp[:, k0:k1],
                                   f"{what}: importance seq {b}")
    # the layer's output is the hidden state carried to the next layer: after 31
    # residual additions |h| exceeds 8, where half a bf16 step (0.031) is above
    # 2e-2, so the carried state's magnitude-scaled bar applies
    ref_h = O.linear_residual(snap["o"].reshape(T_q, -1), wo, snap["h_in"], "bf16")
    PU.assert_close_chained(O.bf16_to_f64(snap["h_out"]), ref_h, f"{what}: h + O Wo^T")


def test_layer_stack_full_size(torch_cuda):
    """The full stack shape (32 layers x 32 steps, B=32, d=4096). Every step:
    invariants (per-head column sums = query rows x layers, top-k counts,
    tracked positions inside the decoded blocks). Against the oracle on every
    sequence: step 0 layer 0 from the seeded inputs alone; the last step at
    layers 0 and 31, teacher-forced on the inputs those layers saw (the caches
    then hold 31 steps of writes and the query holds tracked positions); the
    last step's top-k on the GPU's layer-summed importance."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import LayerStackDriver, to_host
    cfg = CF.C3
    _say("case layer stack full size: generating weights")
    t0 = time.time()
    drv = LayerStackDriver(cfg)
    _say(f"  inputs ready in {time.time() - t0:.1f} s")
    last = cfg.steps - 1
    L_last = cfg.layers - 1
    snaps = {0: dict(step=last), L_last: dict(step=last), "s0": dict(step=0)}
    cache_host = lambda l: (to_host(drv.k_cache[l]).copy(), to_host(drv.v_cache[l]).copy())

    def on_layer(st, l):
        T_q = drv.steps[st]["T_q"]
        if st == 0 and l == 0:
            sn = snaps["s0"]
            sn["q"] = to_host(drv.q_out[:T_q]).copy()
            sn["o"] = to_host(drv.attn_out[:T_q]).copy()
            sn["pos"] = to_host(drv.positions[:T_q]).copy()
        if st == last - 1 and l == L_last:        # caches before the last step's writes
            snaps[0]["kc"], snaps[0]["vc"] = cache_host(0)
            snaps[L_last]["kc"], snaps[L_last]["vc"] = cache_host(L_last)
        if st == last and l == L_last - 1:        # input of the last layer
            snaps[L_last]["h_in"] = to_host(drv.h[:T_q]).copy()
            snaps[L_last]["imp_before"] = to_host(drv.importance).astype(np.float64)
        if st == last and l in (0, L_last):
            sn = snaps[l]
            sn["pos"] = to_host(drv.positions[:T_q]).copy()
            sn["q"] = to_host(drv.q_out[:T_q]).copy()
            sn["o"] = to_host(drv.attn_out[:T_q]).copy()
            sn["h_out"] = to_host(drv.h[:T_q]).copy()
            imp = to_host(drv.importance).astype(np.float64)
            sn["imp"] = imp - sn["imp_before"] if l > 0 else imp
            sn["kc_after"], sn["vc_after"] = cache_host(l)
            if l == 0:
                sn["h_in"] = W.step_hidden(cfg, last, T_q)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for st in range(cfg.steps):
        ev0.record()
        drv.run_step(st, on_layer=on_layer)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1))
        x = drv.steps[st]
        T_q = x["T_q"]
        imp = to_host(drv.importance).astype(np.float64)
        cnt = to_host(drv.topk_count)
        pos = to_host(drv.topk_pos)
        assert np.all(cnt == min(cfg.track, cfg.block_len * (st + 1))), f"step {st} counts"
        for b in range(cfg.batch):
            k0, k1 = int(drv.cu_k_np[b]), int(drv.cu_k_np[b + 1])
            # importance summed over the layers: each head's column sums add up to
            # (query rows) x (layers)
            np.testing.assert_allclose(imp[:, k0:k1].sum(1), x["Q"] * cfg.layers, rtol=2e-4)
            p = pos[b, :cnt[b]]
            assert np.all(np.diff(p) > 0)
            P_b = int(drv.prompt_len[b])
            assert np.all((p >= P_b) & (p < P_b + cfg.block_len * (st + 1)))
        assert np.all(np.isfinite(O.bf16_to_f64(to_host(drv.h[:T_q]))))
        if st == last:
            cand = W.step_candidates(cfg, st + 1, drv.prompt_len, drv.cu_k_np)
            score = imp.sum(0)
            for b in range(cfg.batch):
                k0, k1 = int(drv.cu_k_np[b]), int(drv.cu_k_np[b + 1])
                PU.assert_topk_matches(pos[b], int(cnt[b]), score[k0:k1], cand[k0:k1], cfg.track,
                                       f"last step top-k seq {b}")
    _say(f"  layer stack: {np.mean(times[1:]):.2f} ms per denoising step "
         f"({cfg.layers} layers), {np.sum(times):.1f} ms per {cfg.steps}-step generation")
    # step 0, layer 0 from seeded inputs only: the query is block 0 of each sequence
    wq, _ = W.layer_weights(cfg, 0)
    kc, vc = drv.prefill
    Q0 = drv.steps[0]["Q"]
    sn = snaps["s0"]
    hid = W.step_hidden(cfg, 0, drv.steps[0]["T_q"])
    pos0, cu0 = O.assemble_batch([np.zeros(0, np.int64)] * cfg.batch, drv.prompt_len, Q0)
    np.testing.assert_array_equal(sn["pos"], pos0)
    _say("  oracle: step 0, layer 0, all sequences")
    r = O.flash_cache_step(hid, pos0, cu0, drv.cu_k_np, wq, cfg.n_heads, cfg.head_dim,
                           cfg.rope_base, kc, vc, drv.table, cfg.page_size, None, cfg.track, "bf16",
                           rms_eps=cfg.rms_eps)
    PU.assert_close(O.bf16_to_f64(sn["q"]), r["q"], "bf16", "stack step 0 layer 0 q")
    for b in range(cfg.batch):
        PU.assert_close(O.bf16_to_f64(sn["o"][b * Q0:(b + 1) * Q0]), r["out"][b * Q0:(b + 1) * Q0],
                        "bf16", f"stack step 0 layer 0 attention, seq {b}")
    for l in (0, L_last):
        _say(f"  oracle: step {last}, layer {l}, teacher-forced, all sequences")
        _layer_oracle_check(cfg, l, snaps[l], drv, f"stack step {last} layer {l}")


def test_verify_full_vocab(torch_cuda):
    """Accept test over every row of the verify-shaped workload (vocab 126464)."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import VerifyBuffers
    cfg = CF.C4
    _say("case verify full vocab: drawing logits")
    vi = W.make_verify_inputs(cfg, with_cache=False)
    vb = VerifyBuffers(vi)
    vb.verify()
    torch.cuda.synchronize()
    got = vb.fetch()
    _say("  oracle over all rows")
    am, conf, acc, acc_pos = O.verify_accept(vi.logits, vi.cu_positions, vi.draft, cfg.tau)
    assert np.array_equal(got["argmax"], am)
    np.testing.assert_allclose(got["conf"], conf, rtol=2e-6)
    near = np.abs(conf - cfg.tau) <= 1e-5
    assert np.array_equal(got["accept_row"][~near], acc[~near])
    # per position: exact unless one of its two view rows is near the threshold
    near_pos = np.zeros(len(acc_pos), bool)
    for b in range(cfg.batch):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        n = p1 - p0
        near_pos[p0:p1] = near[2 * p0: 2 * p0 + n] | near[2 * p0 + n: 2 * p0 + 2 * n]
        rows = got["accept_row"]
        assert np.array_equal(got["accept_pos"][p0:p1],
                              rows[2 * p0: 2 * p0 + n] & rows[2 * p0 + n: 2 * p0 + 2 * n])
    assert np.array_equal(got["accept_pos"][~near_pos], acc_pos[~near_pos])
    # the planted rows: argmax is the planted token
    for b in range(cfg.batch):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        n = p1 - p0
        for i in range(n):
            if vi.planted[p0 + i]:
                assert got["argmax"][2 * p0 + i] == vi.target[p0 + i]
                assert got["argmax"][2 * p0 + n + i] == vi.target[p0 + i]
    _say(f"  accepted rows {int(acc.sum())}/{len(acc)}, positions {int(acc_pos.sum())}/{len(acc_pos)}")


def test_verify_step_attention_every_sequence(torch_cuda):
    """Verify-shaped step: Q-only projection of both views and single-pass
    attention over 4096-key caches (up to two row tiles per sequence); every
    sequence against the oracle."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import VerifyBuffers
    cfg = CF.C4
    _say("case verify-shaped attention (all 32 sequences)")
    vi = W.make_verify_inputs(cfg, with_logits=False)
    vb = VerifyBuffers(vi)
    vb.qkv()
    vb.attention()
    torch.cuda.synchronize()
    got = vb.fetch()
    inp = vi.step
    H, D = cfg.n_heads, cfg.head_dim
    for b in range(cfg.batch):
        s = W.sequence_inputs(inp, b)
        proj = O.qkv_rope_cache_write(s["hidden"], s["positions"], s["cu_q"], inp.w_qkv, H, D,
                                      cfg.rope_base, s["k_cache"], s["v_cache"], s["block_table"],
                                      cfg.page_size, "bf16", write_cache=False)
        q0, q1 = s["q0"], s["q1"]
        PU.assert_close(O.bf16_to_f64(got["q_out"][q0:q1]), proj["q"], "bf16", f"verify q seq {b}")
        outr, _ = O.varlen_attention(proj["q_out"], proj["k_cache"], proj["v_cache"],
                                     s["block_table"], cfg.page_size, s["cu_q"], s["cu_k"],
                                     1.0 / math.sqrt(D))
        PU.assert_close(O.bf16_to_f64(got["attn_out"][q0:q1]), outr, "bf16",
                        f"verify attention seq {b}")
