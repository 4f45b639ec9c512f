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
        pos = []
        for b in range(B):
            w0 = int(prompt_len[b]) + cfg.block_len * st
            pos.append(np.concatenate([tracked[b], np.arange(w0, w0 + Q - len(tracked[b]))]))
        positions = np.concatenate(pos).astype(np.int32)
        cu_q = (np.arange(B + 1) * Q).astype(np.int32)
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


def test_layer_stack_full_size(torch_cuda):
    """The full stack shape (32 layers x 32 steps, B=32, d=4096): step 0 layer 0
    against the oracle for two sequences, then invariants over every step."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import LayerStackDriver, to_host
    cfg = CF.C3
    _say("case layer stack full size: generating weights")
    t0 = time.time()
    drv = LayerStackDriver(cfg)
    _say(f"  inputs ready in {time.time() - t0:.1f} s")
    H, D = cfg.n_heads, cfg.head_dim
    snap = {}

    def on_layer(st, l):
        if st == 0 and l == 0:
            T_q = drv.steps[0]["T_q"]
            snap["q"] = to_host(drv.q_out[:T_q]).copy()
            snap["o"] = to_host(drv.attn_out[:T_q]).copy()
            snap["pos"] = to_host(drv.positions[:T_q]).copy()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for st in range(cfg.steps):
        ev0.record()
        drv.run_step(st, on_layer=on_layer if st == 0 else None)
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
    _say(f"  layer stack: {np.mean(times[1:]):.2f} ms per denoising step "
         f"({cfg.layers} layers), {np.sum(times):.1f} ms per {cfg.steps}-step generation")
    # step 0, layer 0 from seeded inputs only: the query is block 0 of each sequence
    wq, _ = W.layer_weights(cfg, 0)
    kc, vc = drv.prefill
    Q0 = drv.steps[0]["Q"]
    hid = W.step_hidden(cfg, 0, drv.steps[0]["T_q"])
    for b in (0, cfg.batch - 1):
        L = int(drv.cache_len[b])
        n_pages = (L + cfg.page_size - 1) // cfg.page_size
        pages = drv.table[b, :n_pages]
        pos_b = snap["pos"][b * Q0:(b + 1) * Q0]
        np.testing.assert_array_equal(pos_b, np.arange(Q0) + int(drv.prompt_len[b]))
        r = O.flash_cache_step(hid[b * Q0:(b + 1) * Q0], pos_b, np.array([0, Q0]),
                               np.array([0, L]), wq, H, D, cfg.rope_base, kc[pages], vc[pages],
                               np.arange(n_pages)[None, :], cfg.page_size, None, cfg.track, "bf16",
                               rms_eps=cfg.rms_eps)
        PU.assert_close(O.bf16_to_f64(snap["q"][b * Q0:(b + 1) * Q0]), r["q"], "bf16",
                        f"stack step 0 layer 0 q, seq {b}")
        PU.assert_close(O.bf16_to_f64(snap["o"][b * Q0:(b + 1) * Q0]), r["out"], "bf16",
                        f"stack step 0 layer 0 attention, seq {b}")


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
    assert np.array_equal(got["accept_pos"], acc_pos) or near.any()
    # the planted rows: argmax is the planted token
    for b in range(cfg.batch):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        n = p1 - p0
        for i in range(n):
            if vi.planted[p0 + i]:
                assert got["argmax"][2 * p0 + i] == vi.target[p0 + i]
                assert got["argmax"][2 * p0 + n + i] == vi.target[p0 + i]
    _say(f"  accepted rows {int(acc.sum())}/{len(acc)}, positions {int(acc_pos.sum())}/{len(acc_pos)}")


def test_verify_step_attention_sampled(torch_cuda):
    """Verify-shaped step: Q-only projection of both views and single-pass
    attention over 4096-key caches (two row tiles per sequence)."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import VerifyBuffers
    cfg = CF.C4
    _say("case verify-shaped attention (sampled sequences)")
    vi = W.make_verify_inputs(cfg, with_logits=False)
    vb = VerifyBuffers(vi)
    vb.qkv()
    vb.attention()
    torch.cuda.synchronize()
    got = vb.fetch()
    inp = vi.step
    H, D = cfg.n_heads, cfg.head_dim
    for b in (0, cfg.batch - 1):
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
