"""The LM head with the fused accept test (fv_lmhead_verify_accept) against the
oracle: every row at a small shape, sampled rows plus every planted row at the
verify-shaped workload (4366 rows, d 4096, vocab 126464)."""
import dataclasses
import sys

import numpy as np
import pytest

from kv_cache_attention_step_amd import configs as CF
from kv_cache_attention_step_amd import workload as W
from oracle import flashcache_oracle as O

pytestmark = pytest.mark.gpu

# fp32 accumulation of 4096 products against the oracle's float64 logits:
# argmax decisions within this logit margin, and accept decisions within this
# confidence band of tau, may go either way
LOGIT_TIE = 1e-4
CONF_BAND = 1e-4


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


def _compare(got, rows, am, conf, acc, top2, what):
    clear = (top2[:, 0] - top2[:, 1]) > LOGIT_TIE
    assert np.array_equal(got["argmax"][rows][clear], am[clear]), what + ": argmax"
    np.testing.assert_allclose(got["conf"][rows], conf, rtol=1e-4, err_msg=what + ": conf")
    decided = clear & (np.abs(conf - 0.9) > CONF_BAND)
    assert np.array_equal(got["accept_row"][rows][decided], acc[decided]), what + ": accept"
    return int((~clear).sum())


def test_lmhead_small_every_row(torch_cuda):
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import LMHeadBuffers
    cfg = dataclasses.replace(CF.C4, name="lm-small", seed=46, batch=5, d_model=512, n_heads=4,
                              vocab=2048, verify_len=(3, 40), cache_len_fixed=64)
    _say("case LM head + accept, small (every row)")
    li = W.make_lmhead_inputs(cfg)
    lb = LMHeadBuffers(li)
    lb.run()
    torch.cuda.synchronize()
    got = lb.fetch()
    vi = li.vi
    am, conf, acc, top2, acc_pos = O.lmhead_verify_accept(li.hidden, li.w_lm, vi.cu_positions,
                                                           vi.draft, cfg.tau)
    _compare(got, np.arange(lb.R), am, conf, acc, top2, "small")
    rows = got["accept_row"]
    for b in range(cfg.batch):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        n = p1 - p0
        assert np.array_equal(got["accept_pos"][p0:p1],
                              rows[2 * p0:2 * p0 + n] & rows[2 * p0 + n:2 * p0 + 2 * n])
    assert acc.sum() > 0 and (acc == 0).sum() > 0


def test_lmhead_verify_shape_sampled(torch_cuda):
    """Full vocabulary: every planted row's argmax is its planted token (its
    softmax probability exceeds 1/2 by construction); 128 sampled rows (the
    first and last sequence, and planted rows elsewhere) against the oracle."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import LMHeadBuffers
    cfg = CF.C4
    _say("case LM head + accept, vocab 126464: drawing inputs")
    li = W.make_lmhead_inputs(cfg)
    vi = li.vi
    lb = LMHeadBuffers(li)
    lb.run()
    torch.cuda.synchronize()
    got = lb.fetch()
    n_pos = int(vi.cu_positions[-1])
    row_pos = np.zeros(lb.R, np.int64)
    for b in range(cfg.batch):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        n = p1 - p0
        row_pos[2 * p0:2 * p0 + n] = np.arange(p0, p1)
        row_pos[2 * p0 + n:2 * p0 + 2 * n] = np.arange(p0, p1)
    planted_rows = np.flatnonzero(vi.planted[row_pos])
    assert np.all(got["argmax"][planted_rows] == vi.target[row_pos[planted_rows]])
    c0 = int(vi.cu_positions[1]) * 2
    cl = int(vi.cu_positions[-2]) * 2
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(0, min(c0, 40)), np.arange(cl, min(lb.R, cl + 40)),
                                     rng.choice(planted_rows, 48, replace=False)]))
    _say(f"  oracle over {len(rows)} sampled rows")
    am, conf, acc, top2 = O.lmhead_verify_accept(li.hidden, li.w_lm, vi.cu_positions, vi.draft,
                                                 cfg.tau, rows=rows)
    _compare(got, rows, am, conf, acc, top2, "verify shape")
    assert got["accept_row"].sum() > 0
