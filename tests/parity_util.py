"""Comparison helpers for GPU-vs-oracle parity (test infrastructure)."""
import numpy as np

from oracle import flashcache_oracle as O

# bf16 interface values against the oracle's unrounded float64 value
BF16_MAX_ABS = 2e-2
BF16_MEAN_REL = 5e-3
# fp32 interface values
F32_MAX_ABS = 1e-4
F32_MEAN_REL = 1e-5
# fp32 importance: relative to the largest entry, and summed relative error
IMP_MAX_REL = 1e-3
IMP_MEAN_REL = 1e-4
# top-k near-tie band, relative to the k-th score
TOPK_TIE_REL = 1e-4


def as_f64(a, dtype):
    return O.as_f64(a, dtype)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = np.abs(got - ref)
    max_abs = float(d.max()) if d.size else 0.0
    denom = float(np.abs(ref).sum())
    mean_rel = float(d.sum() / denom) if denom > 0 else 0.0
    return max_abs, mean_rel


def assert_close(got, ref, dtype, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    max_abs, mean_rel = errors(got, ref)
    if dtype == "bf16":
        tol_abs, tol_rel = BF16_MAX_ABS, BF16_MEAN_REL
    else:
        tol_abs, tol_rel = F32_MAX_ABS, F32_MEAN_REL
    assert max_abs <= tol_abs and mean_rel <= tol_rel, (
        f"{what}: max-abs {max_abs:.3g} (tol {tol_abs}), mean-rel {mean_rel:.3g} (tol {tol_rel})")
    return max_abs, mean_rel


def assert_close_chained(got, ref, what=""):
    """bf16 hidden states carried through several layers. Both sides round the
    state to bf16 after every layer, and where the two pre-rounding values straddle
    a rounding boundary the stored states differ by one bf16 step, which the
    residual path carries forward. One step is 2^-7 relative (0.031 at |x| = 4), so
    the per-element bound scales with magnitude above 1: |g - r| <= 2e-2 max(1, |r|);
    the mean-relative bar stays 5e-3."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    d = np.abs(got - ref)
    worst = float((d / np.maximum(1.0, np.abs(ref))).max())
    mean_rel = float(d.sum() / np.abs(ref).sum())
    assert worst <= BF16_MAX_ABS and mean_rel <= BF16_MEAN_REL, (
        f"{what}: max |g-r|/max(1,|r|) {worst:.3g} (tol {BF16_MAX_ABS}), mean-rel {mean_rel:.3g}")
    return worst, mean_rel


def assert_importance_close(got, ref, what="importance"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    scale = float(np.abs(ref).max()) if ref.size else 1.0
    d = np.abs(got - ref)
    max_rel = float(d.max()) / scale if d.size else 0.0
    mean_rel = float(d.sum() / max(np.abs(ref).sum(), 1e-300))
    assert max_rel <= IMP_MAX_REL and mean_rel <= IMP_MEAN_REL, (
        f"{what}: max-rel {max_rel:.3g} (tol {IMP_MAX_REL}), mean-rel {mean_rel:.3g} "
        f"(tol {IMP_MEAN_REL})")
    return max_rel, mean_rel


def assert_topk_matches(gpu_pos, gpu_cnt, oracle_score, cand, k, what="topk"):
    """One sequence: GPU set vs oracle set, identical outside the near-tie band
    around the oracle's k-th score; same size; GPU positions ascending."""
    local = np.arange(len(oracle_score))
    cands = local[np.asarray(cand) != 0] if cand is not None else local
    kk = min(k, len(cands))
    assert gpu_cnt == kk, f"{what}: count {gpu_cnt} != {kk}"
    g = np.asarray(gpu_pos[:kk], np.int64)
    assert np.all(np.diff(g) > 0), f"{what}: positions not ascending/distinct"
    assert np.all(np.asarray(gpu_pos[kk:]) == -1), f"{what}: padding not -1"
    assert np.all(np.isin(g, cands)), f"{what}: non-candidate chosen"
    if kk == 0:
        return 0
    o, _ = O.topk_select(oracle_score[cands], cands, kk)
    sk = np.sort(oracle_score[cands])[::-1][kk - 1]
    near = set(cands[np.abs(oracle_score[cands] - sk) <= TOPK_TIE_REL * abs(sk)].tolist())
    gs = set(g.tolist()) - near
    os_ = set(o.tolist()) - near
    assert gs == os_, f"{what}: sets differ outside near-ties: gpu-only {sorted(gs - os_)[:10]} " \
                      f"oracle-only {sorted(os_ - gs)[:10]}"
    return len(near)


def compact_sequence(inp, b):
    from kv_cache_attention_step_amd.workload import sequence_inputs
    return sequence_inputs(inp, b)


def oracle_positions(inp):
    """Query positions of a step's inputs as the oracle assembles them (tracked
    positions + masked window per sequence), or the explicit positions the inputs
    carry; checks that the assembled sizes agree with cu_seqlens_q."""
    if inp.positions is not None:
        return np.asarray(inp.positions, np.int32)
    B = inp.B
    rows = [inp.tracked[b, :int(inp.tracked_count[b])] for b in range(B)]
    pos, cu = O.assemble_batch(rows, inp.window_start, inp.window_len)
    assert np.array_equal(cu, inp.cu_seqlens_q), "assembled query sizes != cu_seqlens_q"
    return pos
