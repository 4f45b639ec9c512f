"""CPU oracle for the Flash-Cache denoising step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. The product path never calls it; it shares no code with the
HIP kernels or the C library, and it imports nothing from the product package.

It is plain, slow and written to be checked by eye against the method: numpy in
float64, one sequence and one head at a time, no blocking, fusion or reordering.
Inputs arrive as raw arrays: bf16 values as uint16 bit patterns, fp32 as float32.

Sources (web pages about Flash-dLLM, arXiv 2609.26796):
  [FIG]   signal-papers page on arXiv 2609.26796, figure captions: Fig. 2 says a
          fixed-size query of beta_m tokens (tracked + current masked window)
          attends bidirectionally to the full KV cache via the fused kernel, and
          tracked positions are the top-k decoded tokens by attention importance.
  [NEWS]  infernews post "Flash-dLLM 讓擴散式語言模型解碼更快、更省記憶體":
          paragraph 2 (one fused kernel does QKV projection, RoPE and the cache
          writes; block-scheduled attention handles different query lengths in a
          batch; only new tokens and a few positions chosen by attention
          importance are refreshed), paragraph 3 (Flash-Verify: drafts and [MASK]
          tokens checked through two views, predictions above a confidence
          threshold accepted together).
  [README] zhichai.net forum post quoting the Flash-dLLM README, section 4
          (script defaults: block length 16, confidence threshold 0.9).

Where the pages are silent the oracle takes these readings:
  * Wqkv is [3d, d] (y = x W^T), rows Q | K | V, each head-major, no bias.
  * RoPE is the rotate-half form: pair (e, e + D/2), angle pos * base^(-2e/D),
    applied to Q and K only, positions absolute within the sequence.
  * attention: scale 1/sqrt(D), no mask, no bias, one K/V head per query head;
    the step writes its K/V into the cache first, then attends to all L_b keys.
  * importance of key j = sum over the query rows and heads of the normalised
    softmax probabilities P[i, j]; per-head sums are kept.
  * top-k: larger score first, equal scores -> lower position; result sorted by
    position; fewer candidates than k -> all of them.
  * verify: argmax with the lowest token id on ties; confidence = the largest
    softmax probability; accept a row when argmax == draft and conf >= tau (both
    as float32); a position is accepted when both of its view rows are.
  * confidence-aware acceptance: a position is accepted when its confidence
    alone reaches tau; optionally at least the most confident one per sequence
    (the lowest position among equally confident rows).
  * two views: each view projects its own hidden rows at the verified
    positions; a view attends to the shared cache with its own fresh K/V in
    place of the verified block (nothing of the other view), one-pass softmax.
  * commit: for every accepted position the draft view's K/V (rounded to the
    cache's dtype) replaces the shared cache entry; all else is untouched.
  * LM head: logits = h W_lm^T in float64 from the bf16 operands, never rounded
    to bf16; argmax, confidence and the accept test as for verify.
"""
import math
from itertools import combinations

import numpy as np


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact): a bf16 is the top half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bf16 value (8 significant bits), ties to even.

    x = m * 2**e with 0.5 <= |m| < 1; keeping 8 significant bits means rounding
    m * 256 to an integer (numpy rounds halves to even).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0), e - 8)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit pattern of an already bf16-exact float64 value."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# query assembly ([FIG] Fig. 2: the fixed-size query of a step is the tracked
# positions plus the current masked window)
# ---------------------------------------------------------------------------

def assemble_query(tracked, window_start: int, window_len: int) -> np.ndarray:
    """Query positions of one sequence: the union of its tracked positions and
    the masked window [window_start, window_start + window_len), each position
    once, in ascending order (int64)."""
    window = np.arange(window_start, window_start + window_len, dtype=np.int64)
    return np.union1d(np.asarray(tracked, dtype=np.int64), window)


def assemble_batch(tracked_rows, window_start, window_len):
    """assemble_query per sequence. tracked_rows[b]: that sequence's tracked
    positions; window_len: one length for all sequences or one per sequence.
    Returns (positions [T_q] int32, cu_seqlens_q [B+1] int32)."""
    B = len(tracked_rows)
    wl = np.broadcast_to(np.asarray(window_len, dtype=np.int64), (B,))
    parts = [assemble_query(tracked_rows[b], int(window_start[b]), int(wl[b])) for b in range(B)]
    cu = np.concatenate([[0], np.cumsum([len(p) for p in parts])]).astype(np.int32)
    pos = np.concatenate(parts).astype(np.int32) if B else np.zeros(0, np.int32)
    return pos, cu


# ---------------------------------------------------------------------------
# QKV projection, RoPE, paged cache write ([NEWS] paragraph 2)
# ---------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    e = np.arange(head_dim // 2, dtype=np.float64)
    return base ** (-2.0 * e / head_dim)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE of x[..., T, D] at positions pos[T]: pair (e, e + D/2)
    turns by pos * base^(-2e/D), i.e. (x_e + i x_{e+D/2}) * exp(i theta)."""
    D = x.shape[-1]
    half = D // 2
    theta = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(D, base)[None, :]
    c, s = np.cos(theta), np.sin(theta)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def slot_of(block_table: np.ndarray, b: int, pos: int, page_size: int) -> int:
    page = int(block_table[b, pos // page_size])
    return page * page_size + pos % page_size


def seq_of_rows(cu_seqlens: np.ndarray) -> np.ndarray:
    B = len(cu_seqlens) - 1
    return np.concatenate([np.full(int(cu_seqlens[b + 1] - cu_seqlens[b]), b) for b in range(B)]
                          ).astype(np.int64) if cu_seqlens[-1] > 0 else np.zeros(0, np.int64)


def rms_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """Each row divided by its root mean square: x / sqrt(mean(x^2) + eps) (no
    learned weight). Used for the inputs of a layer stack, where it keeps the
    residual state bounded (a reading: the pages list no normalisation)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def qkv_rope_cache_write(hidden, positions, cu_seqlens_q, w_qkv, n_heads, head_dim, rope_base,
                         k_cache, v_cache, block_table, page_size, dtype, write_cache=True,
                         rms_eps=None):
    """One Flash-Cache projection pass.

    Returns a dict with
      q, k, v      [T_q, H, D] float64, unrounded (q and k after RoPE)
      q_out        q rounded to the interface dtype
      k_cache, v_cache  float64 copies of the caches (values exact in `dtype`)
                   with this step's K/V written at their slots
      slot_mapping [T_q] int64: page * page_size + offset
    """
    x = as_f64(hidden, dtype)
    if rms_eps is not None:
        x = rms_normalize(x, rms_eps)
    w = as_f64(w_qkv, dtype)
    T = x.shape[0]
    H, D = n_heads, head_dim
    d = H * D
    y = x @ w.T                                     # [T, 3d]
    q = y[:, :d].reshape(T, H, D)
    k = y[:, d:2 * d].reshape(T, H, D)
    v = y[:, 2 * d:].reshape(T, H, D)
    pos = np.asarray(positions, dtype=np.int64)
    q = np.stack([rope(q[:, h, :], pos, rope_base) for h in range(H)], axis=1)
    k = np.stack([rope(k[:, h, :], pos, rope_base) for h in range(H)], axis=1)
    kc = as_f64(k_cache, dtype).copy()
    vc = as_f64(v_cache, dtype).copy()
    seq = seq_of_rows(cu_seqlens_q)
    slots = np.zeros(T, dtype=np.int64)
    for t in range(T):
        b = int(seq[t])
        slot = slot_of(block_table, b, int(pos[t]), page_size)
        slots[t] = slot
        if write_cache:
            page, off = divmod(slot, page_size)
            kc[page, :, off, :] = round_to(k[t], dtype)
            vc[page, :, off, :] = round_to(v[t], dtype)
    return dict(q=q, k=k, v=v, q_out=round_to(q, dtype), k_cache=kc, v_cache=vc,
                slot_mapping=slots)


def gather_kv(cache: np.ndarray, block_table: np.ndarray, b: int, length: int, page_size: int):
    """Logical view [L, H, D] of sequence b's cache (positions 0..L-1)."""
    rows = []
    for p in range(length):
        page = int(block_table[b, p // page_size])
        rows.append(cache[page, :, p % page_size, :])
    return np.stack(rows, axis=0)


# ---------------------------------------------------------------------------
# bidirectional attention over the full cache and the per-key
# importance ([FIG] Fig. 2; [NEWS] paragraph 2)
# ---------------------------------------------------------------------------

def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """q [Q, D], k, v [L, D] -> (O [Q, D], P [Q, L], m [Q], l [Q]); exact softmax."""
    s = (q @ k.T) * scale
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    return p @ v, p, m, l


def varlen_attention(q, k_cache, v_cache, block_table, page_size, cu_seqlens_q, cu_seqlens_k,
                     scale, heads=None, seqs=None):
    """q [T_q, H, D] (float64) against each sequence's whole cache.

    Returns O [T_q, H, D] and importance [H, T_k] (column sums of P over the
    sequence's query rows); entries of unselected sequences/heads stay NaN.
    """
    T_q, H, D = q.shape
    B = len(cu_seqlens_q) - 1
    T_k = int(cu_seqlens_k[-1])
    out = np.full((T_q, H, D), np.nan)
    imp = np.full((H, T_k), np.nan)
    heads = range(H) if heads is None else heads
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        L = k1 - k0
        K = gather_kv(k_cache, block_table, b, L, page_size)
        V = gather_kv(v_cache, block_table, b, L, page_size)
        for h in heads:
            if q1 == q0:
                imp[h, k0:k1] = 0.0
                continue
            o, p, _, _ = attention_head(q[q0:q1, h, :], K[:, h, :], V[:, h, :], scale)
            out[q0:q1, h, :] = o
            imp[h, k0:k1] = p.sum(axis=0)
    return out, imp


# ---------------------------------------------------------------------------
# top-k reselection of the tracked positions ([FIG] Fig. 2)
# ---------------------------------------------------------------------------

def head_sum(imp: np.ndarray, as_float32: bool = False) -> np.ndarray:
    """score_j = sum over heads in ascending head order (float64, or float32
    with one rounding per addition)."""
    if not as_float32:
        return imp.sum(axis=0)
    s = np.zeros(imp.shape[1], dtype=np.float32)
    for h in range(imp.shape[0]):
        s = (s + imp[h].astype(np.float32)).astype(np.float32)
    return s


def topk_select(score: np.ndarray, positions: np.ndarray, k: int):
    """Pick min(k, n) entries: larger score first, equal scores -> lower position.
    Returns (positions ascending, their scores)."""
    order = sorted(range(len(score)), key=lambda i: (-float(score[i]), int(positions[i])))
    chosen = sorted(order[:k], key=lambda i: int(positions[i]))
    return (np.array([positions[i] for i in chosen], dtype=np.int64),
            np.array([score[i] for i in chosen], dtype=np.float64))


def importance_topk(imp, cu_seqlens_k, cand_mask, k, score_float32=False):
    """Per sequence: top-k candidate positions by summed importance.

    Returns topk_pos [B, k] (ascending, -1 padded), topk_count [B],
    topk_score [B, k] (NaN padded) and the per-key scores [T_k].
    """
    B = len(cu_seqlens_k) - 1
    score = head_sum(imp, score_float32)
    pos = np.full((B, k), -1, dtype=np.int64)
    sc = np.full((B, k), np.nan)
    cnt = np.zeros(B, dtype=np.int64)
    for b in range(B):
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        local = np.arange(k1 - k0)
        sel = local if cand_mask is None else local[np.asarray(cand_mask[k0:k1]) != 0]
        p, s = topk_select(score[k0 + sel], sel, k)
        cnt[b] = len(p)
        pos[b, :len(p)] = p
        sc[b, :len(p)] = s
    return pos, cnt, sc, score


def topk_exhaustive(score: np.ndarray, positions: np.ndarray, k: int):
    """Brute force over all k-subsets: return the one subset in which every chosen
    entry ranks above every unchosen one under (score desc, position asc)."""
    n = len(score)
    k = min(k, n)
    best = None
    for sub in combinations(range(n), k):
        rest = [i for i in range(n) if i not in sub]
        # a valid top-k set: every chosen entry beats every unchosen one
        ok = all((score[i], -positions[i]) > (score[j], -positions[j]) for i in sub for j in rest)
        if ok:
            assert best is None, "two valid top-k sets"
            best = sub
    return np.array(sorted(positions[i] for i in best), dtype=np.int64)


# ---------------------------------------------------------------------------
# Flash-Verify accept test over the two views ([NEWS] paragraph 3;
# threshold 0.9 from [README] section 4)
# ---------------------------------------------------------------------------

def argmax_conf(row: np.ndarray):
    """Row of logits (float64) -> (lowest index of the maximum, max softmax prob)."""
    mx = row.max()
    a = int(np.flatnonzero(row == mx)[0])
    conf = 1.0 / np.exp(row - mx).sum()
    return a, conf


def verify_accept(logits_bits, cu_positions, draft, tau):
    """logits [R, V] bf16 bits; per sequence L_b draft-view rows then L_b
    mask-view rows. Returns argmax [R], conf [R] (float64), accept_row [R],
    accept_pos [sum L_b]."""
    B = len(cu_positions) - 1
    R = logits_bits.shape[0]
    am = np.zeros(R, dtype=np.int64)
    conf = np.zeros(R, dtype=np.float64)
    acc = np.zeros(R, dtype=np.uint8)
    n_pos = int(cu_positions[-1])
    acc_pos = np.zeros(n_pos, dtype=np.uint8)
    tau32 = np.float32(tau)
    for b in range(B):
        p0, p1 = int(cu_positions[b]), int(cu_positions[b + 1])
        n = p1 - p0
        for i in range(n):
            for view in (0, 1):
                r = 2 * p0 + view * n + i
                a, c = argmax_conf(bf16_to_f64(logits_bits[r]))
                am[r], conf[r] = a, c
                acc[r] = int(a == int(draft[p0 + i]) and np.float32(c) >= tau32)
            acc_pos[p0 + i] = acc[2 * p0 + i] & acc[2 * p0 + n + i]
    return am, conf, acc, acc_pos


def lmhead_verify_accept(hidden_bits, w_lm_bits, cu_positions, draft, tau, rows=None):
    """The LM head followed by the accept test over the two views ([NEWS]
    paragraph 3): logits = hidden . W_lm^T in float64 (no rounding of the
    logits), then per row the lowest argmax, conf = the largest softmax
    probability, accept = (argmax == draft) and conf >= tau (float32), and per
    position the AND of its two view rows. rows: indices of the rows to
    evaluate (default all; accept_pos is returned only then).
    Returns (argmax, conf, accept_row[, accept_pos]) for the rows evaluated,
    plus the top two logits of each (for near-tie bands)."""
    x = bf16_to_f64(hidden_bits)
    w = bf16_to_f64(w_lm_bits)
    R = x.shape[0]
    sel = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    B = len(cu_positions) - 1
    # row -> verified position index
    pos_of = np.zeros(R, dtype=np.int64)
    for b in range(B):
        p0, p1 = int(cu_positions[b]), int(cu_positions[b + 1])
        n = p1 - p0
        pos_of[2 * p0:2 * p0 + n] = np.arange(p0, p1)
        pos_of[2 * p0 + n:2 * p0 + 2 * n] = np.arange(p0, p1)
    am = np.zeros(len(sel), dtype=np.int64)
    conf = np.zeros(len(sel))
    acc = np.zeros(len(sel), dtype=np.uint8)
    top2 = np.zeros((len(sel), 2))
    tau32 = np.float32(tau)
    for j0 in range(0, len(sel), 64):
        blk = sel[j0:j0 + 64]
        logits = x[blk] @ w.T
        for j, r in enumerate(blk):
            a, c = argmax_conf(logits[j])
            am[j0 + j], conf[j0 + j] = a, c
            acc[j0 + j] = int(a == int(draft[pos_of[r]]) and np.float32(c) >= tau32)
            top2[j0 + j] = np.sort(logits[j])[-2:][::-1]
    if rows is not None:
        return am, conf, acc, top2
    acc_pos = np.zeros(int(cu_positions[-1]), dtype=np.uint8)
    for b in range(B):
        p0, p1 = int(cu_positions[b]), int(cu_positions[b + 1])
        n = p1 - p0
        acc_pos[p0:p1] = acc[2 * p0:2 * p0 + n] & acc[2 * p0 + n:2 * p0 + 2 * n]
    return am, conf, acc, top2, acc_pos


def two_view_attention(hidden, w_qkv, n_heads, head_dim, rope_base, k_cache, v_cache,
                       block_table, page_size, cu_positions, verify_start, cache_len, dtype):
    """Flash-Verify's two views with view-private K/V ([NEWS] paragraph 3: drafts
    and [MASK] tokens verified through two views of the same positions).

    Sequence b verifies positions verify_start[b] .. cache_len[b]-1 (n_b of
    them); its hidden rows are n_b draft-view rows then n_b mask-view rows
    (packed by 2 * cu_positions). Each view projects its own rows at those
    positions; its keys and values are the shared cache at the earlier
    positions and its own fresh K/V (rounded to the interface dtype) at the
    verified ones; its rows attend to all L_b keys of that (reading: each view
    sees only its own refreshed entries, as a single Flash-Cache step would).

    Returns dict(out [R, H, D], q [R, H, D] unrounded, k, v [R, H, D] fresh,
    unrounded); rows in the input order.
    """
    x = as_f64(hidden, dtype)
    w = as_f64(w_qkv, dtype)
    kc = as_f64(k_cache, dtype)
    vc = as_f64(v_cache, dtype)
    H, D = n_heads, head_dim
    d = H * D
    R = x.shape[0]
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((R, H, D))
    qa = np.zeros((R, H, D))
    ka = np.zeros((R, H, D))
    va = np.zeros((R, H, D))
    for b in range(len(cu_positions) - 1):
        n = int(cu_positions[b + 1] - cu_positions[b])
        L, vs = int(cache_len[b]), int(verify_start[b])
        assert n == L - vs
        pos = np.arange(vs, L)
        K = gather_kv(kc, block_table, b, L, page_size)
        V = gather_kv(vc, block_table, b, L, page_size)
        for view in (0, 1):
            r0 = 2 * int(cu_positions[b]) + view * n
            y = x[r0:r0 + n] @ w.T
            q = np.stack([rope(y[:, h * D:(h + 1) * D], pos, rope_base) for h in range(H)], axis=1)
            k = np.stack([rope(y[:, d + h * D:d + (h + 1) * D], pos, rope_base) for h in range(H)],
                         axis=1)
            v = y[:, 2 * d:].reshape(n, H, D)
            Kv, Vv = K.copy(), V.copy()
            Kv[vs:] = round_to(k, dtype)
            Vv[vs:] = round_to(v, dtype)
            qr = round_to(q, dtype)
            for h in range(H):
                o, _, _, _ = attention_head(qr[:, h, :], Kv[:, h, :], Vv[:, h, :], scale)
                out[r0:r0 + n, h] = o
            qa[r0:r0 + n], ka[r0:r0 + n], va[r0:r0 + n] = q, k, v
    return dict(out=out, q=qa, k=ka, v=va)


def commit_accepted(k_cache, v_cache, block_table, page_size, cu_positions, verify_start,
                    accept_pos, k_draft, v_draft, dtype):
    """The shared cache after Flash-Verify's commit: every accepted verified
    position takes the draft view's fresh K/V (rounded to the interface dtype);
    every other slot keeps its value. k_draft, v_draft [n_positions, H, D]
    (position order). Returns float64 copies of the caches."""
    kc = as_f64(k_cache, dtype).copy()
    vc = as_f64(v_cache, dtype).copy()
    for b in range(len(cu_positions) - 1):
        for i in range(int(cu_positions[b + 1] - cu_positions[b])):
            p = int(cu_positions[b]) + i
            if accept_pos[p]:
                slot = slot_of(block_table, b, int(verify_start[b]) + i, page_size)
                page, off = divmod(slot, page_size)
                kc[page, :, off, :] = round_to(k_draft[p], dtype)
                vc[page, :, off, :] = round_to(v_draft[p], dtype)
    return kc, vc


def confidence_accept(logits_bits, cu_positions, tau, at_least_one):
    """Confidence-aware acceptance (threshold unmasking, no drafts): one logit
    row per position. Returns argmax [R] (lowest token id on ties), conf [R]
    (float64, the largest softmax probability), accept [R]: conf >= tau, both
    compared as float32. With at_least_one, a sequence with no accepted
    position accepts its most confident one (equal confidences -> the lower
    position), so every step unmasks at least one token per sequence (a
    reading: the pages give no rule for a step where nothing passes)."""
    R = logits_bits.shape[0]
    am = np.zeros(R, dtype=np.int64)
    conf = np.zeros(R, dtype=np.float64)
    acc = np.zeros(R, dtype=np.uint8)
    tau32 = np.float32(tau)
    for r in range(R):
        a, c = argmax_conf(bf16_to_f64(logits_bits[r]))
        am[r], conf[r] = a, c
        acc[r] = int(np.float32(c) >= tau32)
    if at_least_one:
        for b in range(len(cu_positions) - 1):
            p0, p1 = int(cu_positions[b]), int(cu_positions[b + 1])
            if p1 > p0 and not acc[p0:p1].any():
                acc[p0 + int(np.argmax(conf[p0:p1]))] = 1   # first maximum
    return am, conf, acc


# ---------------------------------------------------------------------------
# output projection with residual (multi-layer stack only)
# ---------------------------------------------------------------------------

def linear_residual(x, w, h, dtype):
    """h + x W^T in float64 (x [M, K], W [N, K], h [M, N]); unrounded."""
    return as_f64(h, dtype) + as_f64(x, dtype) @ as_f64(w, dtype).T


# ---------------------------------------------------------------------------
# one Flash-Cache step for one layer ([FIG] Fig. 2): project/rotate/write, then
# attend to the whole cache, then reselect the tracked set
# ---------------------------------------------------------------------------

def flash_cache_step(hidden, positions, cu_seqlens_q, cu_seqlens_k, w_qkv, n_heads, head_dim,
                     rope_base, k_cache, v_cache, block_table, page_size, cand_mask, k, dtype,
                     seqs=None, heads=None, rms_eps=None):
    proj = qkv_rope_cache_write(hidden, positions, cu_seqlens_q, w_qkv, n_heads, head_dim,
                                rope_base, k_cache, v_cache, block_table, page_size, dtype,
                                rms_eps=rms_eps)
    scale = 1.0 / math.sqrt(head_dim)
    out, imp = varlen_attention(proj["q_out"], proj["k_cache"], proj["v_cache"], block_table,
                                page_size, cu_seqlens_q, cu_seqlens_k, scale, heads=heads,
                                seqs=seqs)
    res = dict(proj)
    res.update(out=out, importance=imp)
    if seqs is None and heads is None:
        pos, cnt, sc, score = importance_topk(imp, cu_seqlens_k, cand_mask, k)
        res.update(topk_pos=pos, topk_count=cnt, topk_score=sc, score=score)
    return res
