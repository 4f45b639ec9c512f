"""Seeded synthetic inputs for the Flash-Cache step.

This module only draws random numbers and lays them out; it performs none of the
step's arithmetic (no projection, rotation, softmax, selection or verification).
Both the HIP path and the CPU oracle are fed from here.

Recipe (the pages give no model weights or data, so everything is synthetic):
  * hidden states ~ N(0, 1); Wqkv and Wo ~ N(0, 0.02) (0.02 is the std);
    values are rounded to bf16 (round-to-nearest-even) for bf16 workloads.
  * the stale KV cache is prefilled with N(0, sqrt(d) * 0.02), the scale a
    projection of the hidden states would have; the same bits go to both sides.
  * paging: page size 16, ceil(L_b / 16) pages per sequence, physical page ids a
    seeded random permutation; unused block-table entries are -1.
  * the masked window is the last `window` positions of the generation; the
    candidates for tracking are the generated positions before it; the initial
    tracked set is a seeded sample of `track` candidates.
  * the query itself (tracked positions plus window, in ascending order) is
    not formed here: the product assembles it on the device
    (fc_assemble_query) and the tests take the oracle's assembly.
All draws use numpy's PCG64 seeded from the config seed (and a stream tag).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import StepConfig


def rng_for(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, *tags]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    nan = np.isnan(x)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = (b[nan] >> np.uint32(16)).astype(np.uint16) | np.uint16(0x40)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return to_bf16_bits(x)
    return x


@dataclass
class StepInputs:
    cfg: StepConfig
    dtype: str
    hidden: np.ndarray          # [T_q, d]   bf16 bits (uint16) or float32
    positions: Optional[np.ndarray]  # [T_q] int32; None: assembled from tracked + window
    cu_seqlens_q: np.ndarray    # [B+1]      int32
    cu_seqlens_k: np.ndarray    # [B+1]      int32
    w_qkv: np.ndarray           # [3d, d]
    k_cache: np.ndarray         # [num_pages, H, page_size, D]
    v_cache: np.ndarray         # [num_pages, H, page_size, D]
    block_table: np.ndarray     # [B, max_pages] int32, -1 padded
    cand_mask: np.ndarray       # [T_k] uint8
    prompt_len: np.ndarray      # [B]
    cache_len: np.ndarray       # [B]
    window_start: np.ndarray    # [B]
    tracked: np.ndarray         # [B, track] int32 ascending
    window_len: int = 0         # masked-window tokens per sequence

    @property
    def tracked_count(self) -> np.ndarray:
        return np.full(self.B, self.tracked.shape[1], dtype=np.int32)

    @property
    def B(self) -> int:
        return int(self.cfg.batch)

    @property
    def T_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def T_k(self) -> int:
        return int(self.cu_seqlens_k[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens_q)))

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def draw_lengths(cfg: StepConfig, rng: np.random.Generator):
    if cfg.cache_len_fixed is not None:
        cache_len = np.full(cfg.batch, cfg.cache_len_fixed, dtype=np.int64)
        prompt_len = cache_len - cfg.gen_len
        return prompt_len, cache_len
    lo, hi = cfg.prompt
    prompt_len = rng.integers(lo, hi + 1, size=cfg.batch) if hi > lo else np.full(cfg.batch, lo)
    prompt_len = prompt_len.astype(np.int64)
    return prompt_len, prompt_len + cfg.gen_len


def draw_paging(cfg: StepConfig, cache_len: np.ndarray, rng: np.random.Generator):
    ps = cfg.page_size
    n_pages = (cache_len + ps - 1) // ps
    total = int(n_pages.sum())
    perm = rng.permutation(total).astype(np.int32)
    max_pages = int(n_pages.max())
    table = np.full((cfg.batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(cfg.batch):
        table[b, : n_pages[b]] = perm[off: off + n_pages[b]]
        off += n_pages[b]
    return table, total


def draw_cache(cfg: StepConfig, num_pages: int, rng: np.random.Generator,
               cache_len: Optional[np.ndarray] = None, block_table: Optional[np.ndarray] = None,
               tail_nan: bool = False):
    shape = (num_pages, cfg.n_heads, cfg.page_size, cfg.head_dim)
    k = _normal(rng, shape, cfg.kv_std, cfg.dtype)
    v = _normal(rng, shape, cfg.kv_std, cfg.dtype)
    if tail_nan:
        # slots past the end of each sequence (inside its last page) hold NaN: they
        # must never be read
        nan = np.uint16(0x7FC0) if cfg.dtype == "bf16" else np.float32(np.nan)
        ps = cfg.page_size
        for b in range(cfg.batch):
            L = int(cache_len[b])
            if L % ps:
                page = block_table[b, L // ps]
                k[page, :, L % ps:, :] = nan
                v[page, :, L % ps:, :] = nan
    return k, v


def make_step_inputs(cfg: StepConfig, tail_nan: bool = False) -> StepInputs:
    """Single-layer Flash-Cache step inputs (C0, C1, C2 and C3's layer shapes)."""
    rng = rng_for(cfg.seed, 0)
    prompt_len, cache_len = draw_lengths(cfg, rng)
    table, num_pages = draw_paging(cfg, cache_len, rng)
    B = cfg.batch
    window_start = cache_len - cfg.window
    tracked = np.zeros((B, cfg.track), dtype=np.int32)
    for b in range(B):
        cands = np.arange(prompt_len[b], window_start[b])
        tracked[b] = np.sort(rng.choice(cands, size=cfg.track, replace=False)) if cfg.track else cands[:0]
    # each query holds its tracked positions and its window, disjoint by construction
    q_lens = np.full(B, cfg.track + cfg.window, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(cache_len)]).astype(np.int32)
    cand = np.zeros(int(cu_k[-1]), dtype=np.uint8)
    for b in range(B):
        cand[cu_k[b] + prompt_len[b]: cu_k[b] + window_start[b]] = 1
    T_q = int(cu_q[-1])
    d = cfg.d_model
    hidden = _normal(rng_for(cfg.seed, 1), (T_q, d), cfg.hidden_std, cfg.dtype)
    w_qkv = _normal(rng_for(cfg.seed, 2), (3 * d, d), cfg.weight_std, cfg.dtype)
    k_cache, v_cache = draw_cache(cfg, num_pages, rng_for(cfg.seed, 3), cache_len, table, tail_nan)
    return StepInputs(cfg=cfg, dtype=cfg.dtype, hidden=hidden, positions=None,
                      cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, w_qkv=w_qkv,
                      k_cache=k_cache, v_cache=v_cache, block_table=table, cand_mask=cand,
                      prompt_len=prompt_len.astype(np.int32), cache_len=cache_len.astype(np.int32),
                      window_start=window_start.astype(np.int32), tracked=tracked,
                      window_len=cfg.window)


# ---------------------------------------------------------------------------
# Multi-layer, multi-step driver inputs (C3): block-wise denoising, block length
# 16; at step s the window is block s and the candidates are the decoded blocks
# [P_b, P_b + 16 s).
# ---------------------------------------------------------------------------

def layer_weights(cfg: StepConfig, layer: int):
    d = cfg.d_model
    w_qkv = _normal(rng_for(cfg.seed, 100, layer), (3 * d, d), cfg.weight_std, cfg.dtype)
    w_o = _normal(rng_for(cfg.seed, 200, layer), (d, d), cfg.weight_std, cfg.dtype)
    return w_qkv, w_o


def multistep_base(cfg: StepConfig, tail_nan: bool = False):
    """Lengths, paging and a per-layer prefilled cache for the multi-step driver."""
    rng = rng_for(cfg.seed, 0)
    prompt_len, cache_len = draw_lengths(cfg, rng)
    table, num_pages = draw_paging(cfg, cache_len, rng)
    cu_k = np.concatenate([[0], np.cumsum(cache_len)]).astype(np.int32)
    return prompt_len.astype(np.int32), cache_len.astype(np.int32), table, num_pages, cu_k


def stack_prefill(cfg: StepConfig, num_pages: int):
    """Stale-cache prefill of the layer stack: one seeded draw, copied into every
    layer's cache (each layer's cache then diverges through its own writes)."""
    return draw_cache(cfg, num_pages, rng_for(cfg.seed, 300))


def step_query_lens(cfg: StepConfig, step: int) -> int:
    """Per-sequence query length at a denoising step: block + tracked (shortfall allowed)."""
    return cfg.block_len + min(cfg.track, cfg.block_len * step)


def step_hidden(cfg: StepConfig, step: int, T_q: int) -> np.ndarray:
    return _normal(rng_for(cfg.seed, 400, step), (T_q, cfg.d_model), cfg.hidden_std, cfg.dtype)


def step_candidates(cfg: StepConfig, step: int, prompt_len, cu_k) -> np.ndarray:
    cand = np.zeros(int(cu_k[-1]), dtype=np.uint8)
    for b in range(cfg.batch):
        cand[cu_k[b] + prompt_len[b]: cu_k[b] + prompt_len[b] + cfg.block_len * step] = 1
    return cand


# ---------------------------------------------------------------------------
# Verify-shaped inputs (C4): two views (draft, [MASK]) of the same verified
# positions; per sequence the query rows are L^v draft-view rows followed by L^v
# mask-view rows; logits are synthetic N(0, logit_std) with a planted argmax.
# ---------------------------------------------------------------------------

@dataclass
class VerifyInputs:
    cfg: StepConfig
    step: StepInputs            # attention-side inputs (query rows = both views)
    verify_len: np.ndarray      # [B] L^v_b
    cu_positions: np.ndarray    # [B+1] prefix sums of L^v_b
    draft: np.ndarray           # [sum L^v] int32
    logits: Optional[np.ndarray]  # [R, V] bf16 bits, R = 2 * sum L^v (None until drawn)
    planted: np.ndarray         # [sum L^v] bool
    target: np.ndarray          # [sum L^v] planted token (or -1)


def make_verify_inputs(cfg: StepConfig, with_logits: bool = True,
                       with_cache: bool = True) -> VerifyInputs:
    rng = rng_for(cfg.seed, 0)
    B = cfg.batch
    prompt_len, cache_len = draw_lengths(cfg, rng)
    table, num_pages = draw_paging(cfg, cache_len, rng)
    lo, hi = cfg.verify_len
    vlen = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    pos_list = []
    for b in range(B):
        blk = np.arange(cache_len[b] - vlen[b], cache_len[b])
        pos_list.append(np.concatenate([blk, blk]))
    positions = np.concatenate(pos_list).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(2 * vlen)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(cache_len)]).astype(np.int32)
    cu_p = np.concatenate([[0], np.cumsum(vlen)]).astype(np.int32)
    T_q = int(cu_q[-1])
    d = cfg.d_model
    hidden = _normal(rng_for(cfg.seed, 1), (T_q, d), cfg.hidden_std, cfg.dtype)
    w_qkv = _normal(rng_for(cfg.seed, 2), (3 * d, d), cfg.weight_std, cfg.dtype)
    if with_cache:
        k_cache, v_cache = draw_cache(cfg, num_pages, rng_for(cfg.seed, 3))
    else:
        k_cache = v_cache = np.zeros((0,), np.uint16)
    step = StepInputs(cfg=cfg, dtype=cfg.dtype, hidden=hidden, positions=positions,
                      cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, w_qkv=w_qkv, k_cache=k_cache,
                      v_cache=v_cache, block_table=table,
                      cand_mask=np.zeros(int(cu_k[-1]), np.uint8),
                      prompt_len=prompt_len.astype(np.int32), cache_len=cache_len.astype(np.int32),
                      window_start=(cache_len - vlen).astype(np.int32),
                      tracked=np.zeros((B, 0), np.int32))
    # planted positions and drafts
    n_pos = int(cu_p[-1])
    V = cfg.vocab
    prng = rng_for(cfg.seed, 5)
    planted = prng.random(n_pos) < cfg.planted_frac
    target = np.where(planted, prng.integers(0, V, size=n_pos), -1).astype(np.int32)
    keep = prng.random(n_pos) < 0.8
    other = prng.integers(0, V - 1, size=n_pos)
    other = np.where(other >= np.maximum(target, 0), other + 1, other)  # any token but the target
    draft = np.where(planted & keep, target, np.where(planted, other, prng.integers(0, V, size=n_pos)))
    draft = draft.astype(np.int32)
    vi = VerifyInputs(cfg=cfg, step=step, verify_len=vlen.astype(np.int32), cu_positions=cu_p,
                      draft=draft, logits=None, planted=planted, target=target)
    if with_logits:
        vi.logits = draw_logits(vi)
    return vi


def planted_logit(c_star: np.ndarray, vocab: int, std: float) -> np.ndarray:
    """Planted logit value for a target confidence c*.

    Only constants are used: the other V-1 logits are N(0, std) draws whose
    exp() has mean exp(std^2 / 2), so their sum is near (V-1) exp(std^2 / 2)
    and the planted value log(c*/(1-c*)) + log(V-1) + std^2/2 lands the
    confidence near c* (the realised value scatters by a few per mille).
    """
    return np.log(c_star / (1.0 - c_star)) + np.log(vocab - 1.0) + 0.5 * std * std


def draw_logits(vi: VerifyInputs, row_block: int = 256) -> np.ndarray:
    cfg = vi.cfg
    V = cfg.vocab
    B = cfg.batch
    R = 2 * int(vi.cu_positions[-1])
    out = np.empty((R, V), dtype=np.uint16)
    # row r -> verified position index
    row_pos = np.empty(R, dtype=np.int64)
    for b in range(B):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        r0 = 2 * p0
        n = p1 - p0
        row_pos[r0: r0 + n] = np.arange(p0, p1)
        row_pos[r0 + n: r0 + 2 * n] = np.arange(p0, p1)
    crng = rng_for(cfg.seed, 6)
    # target confidence per row, uniform on [0.5, 0.99] minus a band around tau
    c = crng.uniform(0.5, 0.99 - 0.04, size=R)
    c = np.where(c >= cfg.tau - 0.02, c + 0.04, c)
    lrng = rng_for(cfg.seed, 7)
    for r0 in range(0, R, row_block):
        r1 = min(R, r0 + row_block)
        x = lrng.standard_normal(size=(r1 - r0, V), dtype=np.float32)
        x *= np.float32(cfg.logit_std)
        for r in range(r0, r1):
            p = row_pos[r]
            if vi.planted[p]:
                x[r - r0, vi.target[p]] = np.float32(planted_logit(c[r], V, cfg.logit_std))
        out[r0:r1] = to_bf16_bits(x)
    return out


def sequence_inputs(inp: StepInputs, b: int, positions: Optional[np.ndarray] = None) -> dict:
    """Sequence b of a batch on its own: its query rows and only its own cache
    pages (page ids renumbered 0..n-1, `pages` maps them back). `positions`: the
    batch's query positions (default: inp.positions)."""
    positions = inp.positions if positions is None else positions
    cfg = inp.cfg
    q0, q1 = int(inp.cu_seqlens_q[b]), int(inp.cu_seqlens_q[b + 1])
    L = int(inp.cache_len[b])
    n_pages = (L + cfg.page_size - 1) // cfg.page_size
    pages = inp.block_table[b, :n_pages]
    return dict(hidden=inp.hidden[q0:q1], positions=positions[q0:q1],
                cu_q=np.array([0, q1 - q0], np.int32), cu_k=np.array([0, L], np.int32),
                k_cache=inp.k_cache[pages], v_cache=inp.v_cache[pages],
                block_table=np.arange(n_pages, dtype=np.int32)[None, :], pages=pages,
                cand=inp.cand_mask[int(inp.cu_seqlens_k[b]): int(inp.cu_seqlens_k[b + 1])],
                q0=q0, q1=q1, L=L)


# ---------------------------------------------------------------------------
# LM-head inputs for the verify-shaped step: the two views' final hidden rows
# and a vocabulary projection W_lm [vocab, d] ~ N(0, weight_std). At a planted
# position both view rows are moved along W_lm[t*] so that their logit for t*
# lands near a target (the same planting recipe as the synthetic logits: the
# other logits have variance |h|^2 weight_std^2).
# ---------------------------------------------------------------------------

@dataclass
class LMHeadInputs:
    vi: VerifyInputs
    hidden: np.ndarray          # [R, d] bf16 bits
    w_lm: np.ndarray            # [V, d] bf16 bits


def make_lmhead_inputs(cfg: StepConfig) -> LMHeadInputs:
    vi = make_verify_inputs(cfg, with_logits=False, with_cache=False)
    V, d = cfg.vocab, cfg.d_model
    w = rng_for(cfg.seed, 8).standard_normal(size=(V, d), dtype=np.float32)
    w *= np.float32(cfg.weight_std)
    w_bits = to_bf16_bits(w)
    del w
    wf = bf16_bits_to_f32(w_bits)
    h = rng_for(cfg.seed, 9).standard_normal(size=(2 * int(vi.cu_positions[-1]), d),
                                             dtype=np.float32)
    crng = rng_for(cfg.seed, 10)
    c = crng.uniform(0.5, 0.99 - 0.04, size=h.shape[0])
    c = np.where(c >= cfg.tau - 0.02, c + 0.04, c)
    sigma2 = d * cfg.weight_std ** 2
    for b in range(cfg.batch):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        n = p1 - p0
        for i in range(n):
            p = p0 + i
            if not vi.planted[p]:
                continue
            wt = wf[vi.target[p]].astype(np.float64)
            for r in (2 * p0 + i, 2 * p0 + n + i):
                lam = planted_logit(c[r], V, np.sqrt(sigma2))
                hr = h[r].astype(np.float64)
                hr += (lam - hr @ wt) * wt / (wt @ wt)
                h[r] = hr.astype(np.float32)
    return LMHeadInputs(vi=vi, hidden=to_bf16_bits(h), w_lm=w_bits)
