"""Debug checks of a step's index inputs (FC_DEBUG and fc_validate_step_inputs)
on device-resident inputs: invalid positions, offsets and page ids are rejected
with FC_ERR_INVALID_VALUE before anything is enqueued (the cache and outputs
stay untouched), valid inputs pass. Every invalid case runs with the checks
on, so no kernel ever sees it."""
import dataclasses
import math
import sys

import numpy as np
import pytest

from kv_cache_attention_step_amd import configs as CF
from kv_cache_attention_step_amd import workload as W
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

SMALL = dataclasses.replace(CF.C2, name="dbg", seed=71, batch=3, d_model=512, n_heads=4,
                            prompt=(40, 120), gen_len=96, window=32, track=24)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd.runner import StepBuffers, to_device, to_host
    fc.load()
    inp = W.make_step_inputs(SMALL)
    pos = PU.oracle_positions(inp)
    num_pages = inp.k_cache.shape[0]
    return dict(torch=torch, fc=fc, inp=inp, pos=pos, num_pages=num_pages, StepBuffers=StepBuffers,
                to_device=to_device, to_host=to_host)


def _expect_invalid(fc, fn, *args, **kw):
    with pytest.raises(fc.FlashCacheError) as ei:
        fn(*args, **kw)
    assert ei.value.status_name == "FC_ERR_INVALID_VALUE", str(ei.value)
    return str(ei.value)


def _validate(e, pos, cu_q, cu_k, table, num_pages=None, T_q=None, T_k=None):
    fc, dev = e["fc"], e["to_device"]
    inp = e["inp"]
    fc.fc_validate_step_inputs(dev(pos) if pos is not None else None, dev(cu_q), dev(cu_k), inp.B,
                               int(cu_q[-1]) if T_q is None else T_q,
                               int(cu_k[-1]) if T_k is None else T_k, dev(table), table.shape[1],
                               SMALL.page_size, e["num_pages"] if num_pages is None else num_pages)


def test_validate_accepts_a_valid_step(env):
    _say("case debug: valid step inputs")
    inp = env["inp"]
    _validate(env, env["pos"], inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table)
    _validate(env, None, inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table)


def test_validate_rejects_each_violation(env):
    _say("case debug: fc_validate_step_inputs violations")
    fc, inp = env["fc"], env["inp"]
    cu_q, cu_k, table = inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table
    q0, q1 = int(cu_q[1]), int(cu_q[2])
    dup = env["pos"].copy()
    dup[q0 + 3] = dup[q0 + 4]                                    # repeated position in sequence 1
    assert "twice" in _expect_invalid(fc, _validate, env, dup, cu_q, cu_k, table)
    far = env["pos"].copy()
    far[q1 - 1] = int(inp.cache_len[1])                          # one past the sequence's end
    assert "outside" in _expect_invalid(fc, _validate, env, far, cu_q, cu_k, table)
    neg = env["pos"].copy()
    neg[0] = -1
    _expect_invalid(fc, _validate, env, neg, cu_q, cu_k, table)
    bad_page = table.copy()
    bad_page[2, 0] = env["num_pages"]                             # page id past the cache
    assert "page id" in _expect_invalid(fc, _validate, env, env["pos"], cu_q, cu_k, bad_page)
    bad_cu = cu_k.copy()
    bad_cu[1], bad_cu[2] = bad_cu[2], bad_cu[1]                  # offsets decrease
    _expect_invalid(fc, _validate, env, env["pos"], cu_q, bad_cu, table)
    _expect_invalid(fc, _validate, env, env["pos"], cu_q, cu_k, table, T_q=int(cu_q[-1]) - 1)


def test_fc_debug_blocks_invalid_calls_before_any_work(env, monkeypatch):
    """With FC_DEBUG=1 each entry point rejects inputs that would make its
    kernels index outside the caller's buffers; the cache and outputs keep their
    bytes (nothing was enqueued). The same calls with valid inputs then run."""
    torch, fc, inp = env["torch"], env["fc"], env["inp"]
    dev, host = env["to_device"], env["to_host"]
    _say("case debug: FC_DEBUG entry-point checks")
    monkeypatch.setenv("FC_DEBUG", "1")
    bufs = env["StepBuffers"](inp)
    bufs.assemble()
    torch.cuda.synchronize()
    assert np.array_equal(host(bufs.positions), env["pos"])
    k_before = host(bufs.k_cache).copy()
    # duplicate position in one sequence: two rows would write one cache slot
    dup = env["pos"].copy()
    q0 = int(inp.cu_seqlens_q[1])
    dup[q0 + 1] = dup[q0]
    bufs.positions.copy_(dev(dup))
    assert "twice" in _expect_invalid(fc, bufs.qkv)
    torch.cuda.synchronize()
    assert np.array_equal(host(bufs.k_cache), k_before), "cache written despite the rejection"
    # a position whose page is outside the sequence's table row
    far = env["pos"].copy()
    far[0] = inp.max_pages * SMALL.page_size
    bufs.positions.copy_(dev(far))
    _expect_invalid(fc, bufs.qkv)
    # negative page-table entry on a page a sequence uses
    bufs.positions.copy_(dev(env["pos"]))
    table = inp.block_table.copy()
    table[1, 0] = -1
    good_table = bufs.block_table.clone()
    bufs.block_table.copy_(dev(table))
    bufs.attn_out.fill_(7)
    _expect_invalid(fc, bufs.attention)
    _expect_invalid(fc, bufs.qkv)
    bufs.block_table.copy_(good_table)
    # more query rows than max_seqlen_q
    bufs.max_seqlen_q -= 1
    assert "max_seqlen_q" in _expect_invalid(fc, bufs.attention)
    bufs.max_seqlen_q += 1
    torch.cuda.synchronize()
    assert np.all(host(bufs.attn_out) == 7), "attention output written despite the rejection"
    # decreasing key offsets for the top-k
    bad = inp.cu_seqlens_k.copy()
    bad[1] = bad[2] + 1
    good_cu = bufs.cu_k.clone()
    bufs.cu_k.copy_(dev(bad))
    _expect_invalid(fc, bufs.topk)
    bufs.cu_k.copy_(good_cu)
    # valid inputs run under the checks
    bufs.run()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(PU.as_f64(host(bufs.attn_out), "bf16")))
