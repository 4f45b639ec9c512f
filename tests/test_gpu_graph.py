"""The step's entry points under HIP graph capture: one Flash-Cache step (query
assembly, projection with cache write, attention with importance, top-k) and
the two-view verify step with its commit, each captured once and replayed
several times, with eager work and synchronisations between the replays; every
replay's outputs must equal the eager run's bit for bit. The library enqueues
only kernels (no memset, no copy, no allocation) when FC_DEBUG is off, so a
captured step is the same work as an eager one."""
import dataclasses
import sys

import numpy as np
import pytest

from kv_cache_attention_step_amd import configs as CF
from kv_cache_attention_step_amd import workload as W

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


def _poison(torch, tensors):
    for t in tensors:
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _replay_and_compare(torch, graph, stream, outputs, expect, fetch, what):
    for r in range(3):
        with torch.cuda.stream(stream):
            _poison(torch, outputs)            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = fetch()
        for key, ref in expect.items():
            assert np.array_equal(got[key], ref, equal_nan=True), f"{what}: replay {r}, {key}"


def test_step_graph_replays_match_eager(torch_cuda):
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import StepBuffers
    cfg = dataclasses.replace(CF.C2, name="C2-B8", seed=61, batch=8)
    _say("case graph capture: one C2-shaped step, B=8")
    inp = W.make_step_inputs(cfg)
    bufs = StepBuffers(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bufs.run()
    torch.cuda.synchronize()
    expect = bufs.fetch()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        bufs.run()
    torch.cuda.synchronize()
    outs = [bufs.positions, bufs.q_out, bufs.attn_out, bufs.slot_mapping, bufs.importance,
            bufs.topk_pos, bufs.topk_count, bufs.topk_score]
    _replay_and_compare(torch, graph, s, outs, expect, bufs.fetch, "step")


def test_two_view_verify_graph_replays_match_eager(torch_cuda):
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import TwoViewVerifyBuffers, to_host
    cfg = dataclasses.replace(CF.C4, name="C4-small", seed=62, batch=5, d_model=512, n_heads=4,
                              page_size=16, cache_len_fixed=300, verify_len=(1, 70))
    _say("case graph capture: two views with private K/V, then the commit")
    vi = W.make_verify_inputs(cfg, with_logits=False)
    tv = TwoViewVerifyBuffers(vi)
    rng = W.rng_for(cfg.seed, 78)
    tv.accept_pos.copy_(torch.from_numpy((rng.random(tv.n_pos) < 0.5).astype(np.uint8)).cuda())
    s = torch.cuda.Stream()

    def step():
        tv.run_views()
        tv.commit()

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()

    def fetch():
        return dict(view_table=to_host(tv.view_table), q_out=to_host(tv.q_out),
                    attn_out=to_host(tv.attn_out), k_cache=to_host(tv.k_cache),
                    v_cache=to_host(tv.v_cache))
    expect = fetch()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    _replay_and_compare(torch, graph, s, [tv.view_table, tv.q_out, tv.attn_out], expect, fetch,
                        "two views")
