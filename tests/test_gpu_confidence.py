"""Confidence-aware acceptance (fv_confidence_accept) against the oracle: the
hand-worked golden rows, then the [MASK]-view rows of the verify-shaped
workload at its full vocabulary (126464), with and without the
at-least-one-per-sequence rule."""
import json
import os
import sys

import numpy as np
import pytest

from kv_cache_attention_step_amd import configs as CF
from kv_cache_attention_step_amd import workload as W
from oracle import flashcache_oracle as O

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(torch, bits, cu_p, tau, at_least_one):
    from kv_cache_attention_step_amd import flashcache as fc
    R, V = bits.shape
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    lg, cp = t(bits.view(np.int16)), t(np.asarray(cu_p, np.int32))
    am = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    cf = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    ac = torch.full((R,), 7, dtype=torch.uint8, device="cuda")
    fc.fv_confidence_accept(lg, V, cp, len(cu_p) - 1, R, tau, at_least_one, am, cf, ac)
    torch.cuda.synchronize()
    return am.cpu().numpy(), cf.cpu().numpy(), ac.cpu().numpy()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from kv_cache_attention_step_amd import flashcache as fc
    fc.load()
    return torch


def test_confidence_golden_rows(torch_cuda):
    _say("case confidence acceptance: golden rows")
    g = json.load(open(os.path.join(GOLDEN, "confidence_accept.json")))
    bits = W.to_bf16_bits(np.array(g["rows"], np.float32))
    for flag, key in ((0, "expected_accept_threshold_only"), (1, "expected_accept_at_least_one")):
        am, cf, ac = _run(torch_cuda, bits, g["cu_positions"], g["tau"], flag)
        assert np.array_equal(am, g["expected_argmax"])
        np.testing.assert_allclose(cf, g["expected_conf"], rtol=2e-6)
        assert np.array_equal(ac, g[key]), (flag, ac)


def test_confidence_mask_view_full_vocab(torch_cuda):
    """The [MASK]-view rows of the verify-shaped workload (30 % of positions
    carry a planted confident token). Argmax exact, conf to 2e-6 relative,
    accept flags exact except rows whose confidence lies within 1e-5 of tau;
    the fallback row of a sequence with nothing accepted is the oracle's unless
    its two most confident rows are within 1e-5 of each other."""
    cfg = CF.C4
    _say("case confidence acceptance: mask-view rows, vocab 126464")
    vi = W.make_verify_inputs(cfg, with_cache=False)
    cu_p = vi.cu_positions
    rows = []
    for b in range(cfg.batch):
        p0, p1 = int(cu_p[b]), int(cu_p[b + 1])
        n = p1 - p0
        rows.append(vi.logits[2 * p0 + n: 2 * p0 + 2 * n])
    bits = np.ascontiguousarray(np.concatenate(rows))
    _say("  oracle over all rows")
    am_r, cf_r, acc0 = O.confidence_accept(bits, cu_p, cfg.tau, False)
    _, _, acc1 = O.confidence_accept(bits, cu_p, cfg.tau, True)
    near = np.abs(cf_r - cfg.tau) <= 1e-5
    for flag, acc in ((0, acc0), (1, acc1)):
        am, cf, ac = _run(torch_cuda, bits, cu_p, cfg.tau, flag)
        assert np.array_equal(am, am_r)
        np.testing.assert_allclose(cf, cf_r, rtol=2e-6)
        if flag == 0:
            assert np.array_equal(ac[~near], acc[~near])
            continue
        for b in range(cfg.batch):
            p0, p1 = int(cu_p[b]), int(cu_p[b + 1])
            seg_g, seg_o = ac[p0:p1], acc[p0:p1]
            if np.any(near[p0:p1]):
                continue
            if acc0[p0:p1].any():          # threshold decided: identical flags
                assert np.array_equal(seg_g, seg_o), f"sequence {b}"
            else:                           # the fallback row
                assert seg_g.sum() == 1, f"sequence {b}: one fallback row"
                top = np.sort(cf_r[p0:p1])[::-1]
                if len(top) < 2 or top[0] - top[1] > 1e-5 * top[0]:
                    assert np.array_equal(seg_g, seg_o), f"sequence {b}: fallback row"
    assert acc0.sum() > 0 and acc1.sum() > acc0.sum()   # both rules exercised


def test_confidence_at_least_one_with_non_finite_rows(torch_cuda):
    """A sequence whose logits are all NaN next to ordinary sequences: with the
    at-least-one rule it still gets exactly one accepted row when none passed,
    inside its own rows, and the other sequences are unaffected."""
    _say("case confidence acceptance: a sequence of NaN rows")
    rng = np.random.default_rng(5)
    V = 512
    cu = np.array([0, 4, 9, 12], np.int32)
    rows = (rng.standard_normal((int(cu[-1]), V)) * 2).astype(np.float32)
    rows[4:9] = np.nan                       # sequence 1: every logit NaN
    bits = W.to_bf16_bits(rows)
    am, cf, ac = _run(torch_cuda, bits, cu, 0.9, 1)
    assert set(np.unique(ac)) <= {0, 1}
    assert ac[4:9].sum() >= 1, "the NaN sequence accepts at least one row"
    ok = np.r_[0:4, 9:12]
    am_r, cf_r, acc_r = O.confidence_accept(bits[ok], np.array([0, 4, 7], np.int32), 0.9, True)
    assert np.array_equal(am[ok], am_r)
    np.testing.assert_allclose(cf[ok], cf_r, rtol=2e-6)
    assert np.array_equal(ac[ok], acc_r)
