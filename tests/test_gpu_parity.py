"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs. Run on an MI355X: pytest -m gpu."""
import dataclasses
import math
import sys

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
    fc.load()  # fail loudly when the library is missing
    return torch


def run_gpu_step(inp, torch, keep=False):
    from kv_cache_attention_step_amd.runner import StepBuffers
    bufs = StepBuffers(inp)
    bufs.run()
    torch.cuda.synchronize()
    got = bufs.fetch()
    return (got, bufs) if keep else got


def check_cache(got_cache, in_cache, ref_rows, slots, page_size, H, dtype, what):
    """Written slots against the oracle's unrounded rows, every other slot bit-exact."""
    pages = slots // page_size
    offs = slots % page_size
    written = got_cache[pages, :, offs, :]                        # [T, H, D]
    PU.assert_close(PU.as_f64(written, dtype), ref_rows, dtype, what + " written rows")
    mask = np.ones(got_cache.shape[0] * page_size, bool)
    mask[slots] = False
    g = got_cache.transpose(0, 2, 1, 3).reshape(-1, H, got_cache.shape[-1])
    i = in_cache.transpose(0, 2, 1, 3).reshape(-1, H, in_cache.shape[-1])
    gb = g[mask].view(np.uint32 if g.dtype == np.float32 else np.uint16)
    ib = i[mask].view(np.uint32 if i.dtype == np.float32 else np.uint16)
    assert np.array_equal(gb, ib), f"{what}: untouched slots changed"


def full_parity(inp, got):
    """Every output of one step against the oracle, every sequence and head:
    query positions, slot ids and untouched cache bits exactly; q_out, the
    written K/V rows and the attention output within the bf16 (fp32) bar;
    importance within its bar; top-k sets exactly outside the near-tie band."""
    cfg = inp.cfg
    positions = PU.oracle_positions(inp)
    assert np.array_equal(got["positions"], positions), "query positions (assembly)"
    r = O.flash_cache_step(inp.hidden, positions, inp.cu_seqlens_q, inp.cu_seqlens_k,
                           inp.w_qkv, cfg.n_heads, cfg.head_dim, cfg.rope_base, inp.k_cache,
                           inp.v_cache, inp.block_table, cfg.page_size, inp.cand_mask, cfg.track,
                           cfg.dtype)
    dt = cfg.dtype
    assert np.array_equal(got["slot_mapping"].astype(np.int64), r["slot_mapping"]), "slot mapping"
    PU.assert_close(PU.as_f64(got["q_out"], dt), r["q"], dt, "q_out")
    check_cache(got["k_cache"], inp.k_cache, r["k"], r["slot_mapping"], cfg.page_size,
                cfg.n_heads, dt, "k_cache")
    check_cache(got["v_cache"], inp.v_cache, r["v"], r["slot_mapping"], cfg.page_size,
                cfg.n_heads, dt, "v_cache")
    PU.assert_close(PU.as_f64(got["attn_out"], dt), r["out"], dt, "attention out")
    PU.assert_importance_close(got["importance"], r["importance"])
    for b in range(inp.B):
        q0, q1 = int(inp.cu_seqlens_q[b]), int(inp.cu_seqlens_q[b + 1])
        k0, k1 = int(inp.cu_seqlens_k[b]), int(inp.cu_seqlens_k[b + 1])
        if q1 > q0:
            PU.assert_close(PU.as_f64(got["attn_out"][q0:q1], dt), r["out"][q0:q1], dt,
                            f"attention out seq {b}")
        if k1 > k0 and q1 > q0:
            PU.assert_importance_close(got["importance"][:, k0:k1], r["importance"][:, k0:k1],
                                       f"importance seq {b}")
    score = r["importance"].sum(0)
    n_near = 0
    for b in range(inp.B):
        k0, k1 = int(inp.cu_seqlens_k[b]), int(inp.cu_seqlens_k[b + 1])
        n_near += PU.assert_topk_matches(got["topk_pos"][b], int(got["topk_count"][b]),
                                         score[k0:k1], inp.cand_mask[k0:k1], cfg.track,
                                         f"topk seq {b}")
    return r, n_near


def test_c0_tiny_fp32_step(torch_cuda):
    _say("case C0 tiny fp32 step")
    inp = W.make_step_inputs(CF.C0)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


SMALL_BF16 = dataclasses.replace(CF.C2, name="C2-small", seed=21, batch=3, d_model=512, n_heads=4,
                                 prompt=(40, 300), gen_len=160, window=48, track=40)


def test_small_bf16_varlen_step_with_nan_tails(torch_cuda):
    """Several sequences, ragged key tiles and pages; slots past each sequence end
    hold NaN and must never be read."""
    _say("case C2-small bf16 varlen, NaN tails")
    inp = W.make_step_inputs(SMALL_BF16, tail_nan=True)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


def test_small_page_size_path(torch_cuda):
    """page_size 4 (< 16 keys of a load group span several pages) on the key-split
    path (3 sequences x 4 heads: few (sequence, head) items)."""
    cfg = dataclasses.replace(SMALL_BF16, name="C2-ps4", seed=24, page_size=4)
    _say("case C2-small bf16, page size 4, NaN tails")
    inp = W.make_step_inputs(cfg, tail_nan=True)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


def test_large_page_size_path(torch_cuda):
    """page_size 64: four 16-key load groups share a page; the last page of a
    sequence is partly past its end (NaN tails there must never be read); the
    key-split path (few (sequence, head) items)."""
    cfg = dataclasses.replace(SMALL_BF16, name="C2-ps64", seed=26, page_size=64)
    _say("case C2-small bf16, page size 64, NaN tails")
    inp = W.make_step_inputs(cfg, tail_nan=True)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


WIDE = dataclasses.replace(CF.C2, name="wide", seed=28, batch=9, d_model=2048, n_heads=16,
                           prompt=(40, 300), gen_len=160, window=48, track=40)


@pytest.mark.parametrize("short_q", [False, True])
@pytest.mark.parametrize("ps", [4, 64])
def test_page_sizes_on_the_batched_attention_paths(torch_cuda, ps, short_q):
    """Page sizes 4 and 64 on the paths a full batch takes: 9 sequences x 16
    heads = 144 (sequence, head) items, more than half of 256 CUs, so the
    importance path runs one workgroup per item without a key split; 88 query
    rows per sequence (128-row tiles) or 48 (at most 64 rows: each tile's keys
    are split over the waves). The same device queries and cache then go
    through the one-pass path (no importance). NaN fills the slots past each
    sequence's end."""
    torch = torch_cuda
    w = 24 if short_q else 48
    cfg = dataclasses.replace(WIDE, name=f"wide-ps{ps}-q{2 * w}", seed=28 + ps + w, page_size=ps,
                              window=w, track=w if short_q else 40)
    _say(f"case page size {ps}, {cfg.window + cfg.track} query rows, 144 items")
    inp = W.make_step_inputs(cfg, tail_nan=True)
    assert inp.B * cfg.n_heads * 2 > 256 and (inp.max_seqlen_q <= 64) == short_q
    got, bufs = run_gpu_step(inp, torch, keep=True)
    r, _ = full_parity(inp, got)
    bufs.attention(importance=False)
    torch.cuda.synchronize()
    from kv_cache_attention_step_amd.runner import to_host
    PU.assert_close(PU.as_f64(to_host(bufs.attn_out), "bf16"), r["out"], "bf16",
                    "one-pass attention out")


def test_many_sequences(torch_cuda):
    """70 sequences: more than one wave can rank, so the longest-first order comes
    from the ordering kernel instead of each attention workgroup."""
    cfg = dataclasses.replace(SMALL_BF16, name="C2-many", seed=27, batch=70, prompt=(20, 90),
                              gen_len=48, window=16, track=12)
    _say("case 70 sequences")
    inp = W.make_step_inputs(cfg)
    assert inp.B > 64
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


def test_bf16_query_longer_than_one_row_tile(torch_cuda):
    """Q_b > 128 rows: the importance path loops over row tiles in one workgroup."""
    cfg = dataclasses.replace(SMALL_BF16, name="C2-rows", seed=22, batch=2, prompt=(100, 180),
                              gen_len=300, window=100, track=90)
    _say("case C2-rows bf16 Q_b=190")
    inp = W.make_step_inputs(cfg)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


def test_c1_single_layer_step(torch_cuda):
    _say("case C1 full step")
    inp = W.make_step_inputs(CF.C1)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


def test_c2_full_size_every_sequence(torch_cuda):
    """The batched step at full size (B=32, d=4096, caches 768..1536, 128 query
    rows each) in the launch configuration the benchmark times: every output of
    every sequence against the oracle, plus the column-sum invariant."""
    _say("case C2 full size, all 32 sequences")
    cfg = CF.C2
    inp = W.make_step_inputs(cfg)
    got = run_gpu_step(inp, torch_cuda)
    imp = got["importance"].astype(np.float64)
    assert np.all(np.isfinite(imp)) and np.all(imp >= 0)
    for b in range(inp.B):
        k0, k1 = int(inp.cu_seqlens_k[b]), int(inp.cu_seqlens_k[b + 1])
        qb = int(inp.cu_seqlens_q[b + 1] - inp.cu_seqlens_q[b])
        np.testing.assert_allclose(imp[:, k0:k1].sum(1), qb, rtol=2e-4)
    _say("  oracle over the whole batch")
    full_parity(inp, got)


def test_c2_shaped_ragged_row_tiles(torch_cuda):
    """C2-shaped layers with 9 sequences (1152 query tokens): the projection runs
    256-row tiles (fewer rounds of workgroups than 128-row ones) and the last row
    tile is half empty; every sequence against the oracle."""
    _say("case C2-shaped, 9 sequences (ragged 256-row tiles)")
    cfg = dataclasses.replace(CF.C2, name="C2-9", seed=57, batch=9)
    inp = W.make_step_inputs(cfg)
    assert inp.T_q == 1152
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


@pytest.mark.parametrize("B", [2, 4])
def test_c2_shape_key_split(torch_cuda, B):
    """The C2 layer shape with few sequences: B=4 (128 (sequence, head) items)
    splits each item's keys in S=2 chunks and B=2 (64 items) in S=4 on a
    256-CU device, each chunk several 64-key tiles long; 128 query rows and
    ragged cache lengths per sequence; every output against the oracle."""
    _say(f"case C2 shape, B={B} (attention key split)")
    cfg = dataclasses.replace(CF.C2, name=f"C2-B{B}", seed=60 + B, batch=B)
    inp = W.make_step_inputs(cfg, tail_nan=True)
    assert np.any(inp.cache_len % 64 != 0)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)


def test_c2_deterministic(torch_cuda):
    """Same inputs twice -> bit-identical outputs (no float atomics anywhere)."""
    _say("case C2 determinism")
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import StepBuffers
    inp = W.make_step_inputs(CF.C2)
    bufs = StepBuffers(inp)
    outs = []
    for _ in range(2):
        bufs.run()
        torch.cuda.synchronize()
        f = bufs.fetch()
        outs.append({k: f[k] for k in ("q_out", "attn_out", "importance", "topk_pos",
                                        "topk_score", "slot_mapping")})
    for k in outs[0]:
        assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), k


@pytest.mark.parametrize("H", [8, 32, 43])
def test_topk_kernel_planted_ties(torch_cuda, H):
    """Importance built by the test with many exact ties: the kernel's selection
    must equal the oracle's, both deciding on the same fp32 head-sum. H = 8, 32
    and 43 take the kernel's 8-, 32- and mixed head-load groups."""
    torch = torch_cuda
    from kv_cache_attention_step_amd import flashcache as fc
    _say(f"case topk planted ties H={H}")
    rng = np.random.default_rng(5 + H)
    lens = np.array([1, 7, 64, 300, 1537, 4096, 0, 33])
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T_k = int(cu[-1])
    imp = (rng.integers(0, 6, size=(H, T_k)) / 8.0).astype(np.float32)   # exact, many ties
    cand = (rng.random(T_k) < 0.7).astype(np.uint8)
    for k in (1, 5, 64, 500):
        d_imp = torch.from_numpy(imp).cuda()
        d_cu = torch.from_numpy(cu).cuda()
        d_cand = torch.from_numpy(cand).cuda()
        pos = torch.full((B, k), 77, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
        sc = torch.zeros((B, k), dtype=torch.float32, device="cuda")
        fc.fc_importance_topk(d_imp, d_cu, B, T_k, H, d_cand, k, pos, cnt, sc)
        torch.cuda.synchronize()
        opos, ocnt, osc, _ = O.importance_topk(imp.astype(np.float64), cu, cand, k,
                                                score_float32=True)
        assert np.array_equal(cnt.cpu().numpy(), ocnt), f"k={k} counts"
        assert np.array_equal(pos.cpu().numpy(), opos), f"k={k} positions"
        gsc = sc.cpu().numpy()
        assert np.array_equal(np.nan_to_num(gsc, nan=-1), np.nan_to_num(osc.astype(np.float32),
                                                                        nan=-1)), f"k={k} scores"


def test_topk_length_capacity(torch_cuda):
    """Sequences of exactly FC_TOPK_MAX_LEN keys (scores in LDS), one key more and
    40000 keys (scores recomputed from global memory in every pass) and a short
    one in the same call: every one selected like the oracle, scores bit-exact."""
    torch = torch_cuda
    from kv_cache_attention_step_amd import flashcache as fc
    _say("case topk length capacity")
    rng = np.random.default_rng(11)
    H, k = 32, 48
    lens = np.array([fc.FC_TOPK_MAX_LEN, fc.FC_TOPK_MAX_LEN + 1, 500, 40000])
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T_k = int(cu[-1])
    imp = rng.random((H, T_k)).astype(np.float32)
    cand = (rng.random(T_k) < 0.5).astype(np.uint8)
    pos = torch.full((B, k), 77, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, k), dtype=torch.float32, device="cuda")
    fc.fc_importance_topk(torch.from_numpy(imp).cuda(), torch.from_numpy(cu).cuda(), B, T_k, H,
                          torch.from_numpy(cand).cuda(), k, pos, cnt, sc)
    torch.cuda.synchronize()
    gpos, gcnt, gsc = pos.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()
    opos, ocnt, osc, _ = O.importance_topk(imp.astype(np.float64), cu, cand, k, score_float32=True)
    for b in range(B):
        assert gcnt[b] == ocnt[b] == k and np.array_equal(gpos[b], opos[b]), f"seq {b}"
        assert np.array_equal(gsc[b], osc[b].astype(np.float32)), f"seq {b} scores"


@pytest.mark.parametrize("T,H", [(200, 8), (1300, 8), (3000, 8), (5378, 16)])
def test_qkv_row_scale_every_projection_path(torch_cuda, T, H):
    """Projection of RMS-normalised inputs (the layer stack's use: a per-row scale
    from fc_rms_row_scale, folded into the rotation table for Q and K and applied
    to V) on each projection path of a 256-CU device. At d = 1024 (12 column
    tiles of 256): T=200 (24 tiles of 128 rows: K split in 4, partial products
    then the split epilogue), T=1300 (132 tiles of 128 rows: one pass, 128-row
    tiles), T=3000 (persistent 256-row tiles, the last one partly empty). At
    d = 2048 (24 column tiles): T=5378 (persistent 256-row tiles for 5376 rows,
    whole rounds over the CUs, then the last 2 rows as a launch of 128-row
    tiles). Sampled rows (first, middle and last 16) against the oracle's
    normalised projection, cache slots bit-exact, untouched cache rows
    unchanged."""
    torch = torch_cuda
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd.runner import to_device, to_host
    _say(f"case qkv row scale T={T} H={H}")
    D, ps, eps, base = 128, 16, 1e-5, 5e5
    d = H * D
    rng = W.rng_for(77, T)
    hid = W.to_bf16_bits((rng.standard_normal((T, d)) * 3.0).astype(np.float32))
    w = W.to_bf16_bits((rng.standard_normal((3 * d, d)) * 0.02).astype(np.float32))
    pos = rng.permutation(T + 40)[:T].astype(np.int32)   # distinct positions, one sequence
    cu = np.array([0, T], np.int32)
    maxp = (T + 40 + ps - 1) // ps
    n_pages = maxp + 5
    bt = rng.permutation(n_pages)[:maxp].astype(np.int32)[None, :]
    kc0 = W.to_bf16_bits(rng.standard_normal((n_pages, H, ps, D)).astype(np.float32))
    vc0 = W.to_bf16_bits(rng.standard_normal((n_pages, H, ps, D)).astype(np.float32))
    g_hid, g_w, g_pos, g_cu, g_bt = (to_device(a) for a in (hid, w, pos, cu, bt))
    g_kc, g_vc = to_device(kc0), to_device(vc0)
    g_q = torch.empty((T, H, D), dtype=torch.int16, device="cuda")
    g_sm = torch.empty(T, dtype=torch.int32, device="cuda")
    g_rs = torch.empty(T, dtype=torch.float32, device="cuda")
    wsb = fc.fc_qkv_workspace_size(T, d, D, fc.FC_DTYPE_BF16)
    g_ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    fc.fc_rms_row_scale(g_hid.data_ptr(), T, d, eps, g_rs.data_ptr(), fc.FC_DTYPE_BF16)
    fc.fc_qkv_rope_cache_write(g_hid.data_ptr(), g_pos.data_ptr(), g_cu.data_ptr(), 1, T,
                               g_w.data_ptr(), d, H, D, base, g_kc.data_ptr(), g_vc.data_ptr(),
                               g_bt.data_ptr(), maxp, ps, g_q.data_ptr(), g_sm.data_ptr(),
                               g_ws.data_ptr(), wsb, fc.FC_DTYPE_BF16, row_scale=g_rs.data_ptr())
    torch.cuda.synchronize()
    q_out, sm = to_host(g_q), to_host(g_sm).astype(np.int64)
    kc, vc = to_host(g_kc), to_host(g_vc)
    # slots of every row (bit-exact), and no other cache row touched
    slot_ref = bt[0, pos // ps].astype(np.int64) * ps + pos % ps
    assert np.array_equal(sm, slot_ref), "slot mapping"
    mask = np.ones(n_pages * ps, bool)
    mask[slot_ref] = False
    for got, ref, what in ((kc, kc0, "k"), (vc, vc0, "v")):
        g = got.transpose(0, 2, 1, 3).reshape(-1, H, D)[mask]
        r = ref.transpose(0, 2, 1, 3).reshape(-1, H, D)[mask]
        assert np.array_equal(g, r), f"{what} cache: untouched slots changed"
    # sampled rows (first, middle and last 16) against the oracle
    rows = np.unique(np.concatenate([np.arange(16), T // 2 + np.arange(16), T - 16 + np.arange(16)]))
    r = O.qkv_rope_cache_write(hid[rows], pos[rows], np.array([0, len(rows)]), w, H, D, base,
                               kc0, vc0, bt, ps, "bf16", write_cache=False,
                               rms_eps=eps)
    assert np.array_equal(sm[rows], r["slot_mapping"]), "slot mapping (oracle)"
    PU.assert_close(PU.as_f64(q_out[rows], "bf16"), r["q"], "bf16", "q rows")
    pg, off = slot_ref[rows] // ps, slot_ref[rows] % ps
    PU.assert_close(PU.as_f64(kc[pg, :, off, :], "bf16"), r["k"], "bf16", "k rows")
    PU.assert_close(PU.as_f64(vc[pg, :, off, :], "bf16"), r["v"], "bf16", "v rows")


@pytest.mark.parametrize("M,N,K", [
    (300, 512, 1024),     # 128-row DMA tiles, ragged last row tile
    (1100, 12288, 256),   # 256-row DMA tiles (enough column tiles to fill the CUs)
    (300, 384, 1024),     # width not a multiple of 256: register-staged 128 x 128 tiles
])
def test_linear_residual_bf16(torch_cuda, M, N, K):
    torch = torch_cuda
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd.runner import to_device, to_host
    _say(f"case linear residual bf16 {M}x{N}x{K}")
    rng = W.rng_for(9, 1)
    x = W.to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    w = W.to_bf16_bits((rng.standard_normal((N, K), dtype=np.float32) * 0.02).astype(np.float32))
    h = W.to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
    dx, dw, dh = to_device(x), to_device(w), to_device(h)
    fc.fc_linear_residual(dx, dw, dh, M, N, K, fc.FC_DTYPE_BF16)
    torch.cuda.synchronize()
    ref = O.linear_residual(x, w, h, "bf16")
    PU.assert_close(O.bf16_to_f64(to_host(dh)), ref, "bf16", "h + x W^T")


def test_degenerate_sequences(torch_cuda):
    """A sequence with no query rows, one with a single cached key, and a tracking
    budget larger than the candidate count."""
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import StepBuffers
    _say("case degenerate sequences")
    cfg = dataclasses.replace(SMALL_BF16, name="degenerate", seed=23, batch=3, prompt=(1, 1),
                              gen_len=0, window=0, track=0)
    H, D, ps = cfg.n_heads, cfg.head_dim, cfg.page_size
    rng = W.rng_for(23, 9)
    L = np.array([1, 40, 17], np.int32)
    Q = np.array([1, 0, 5], np.int32)
    table, num_pages = W.draw_paging(cfg, L.astype(np.int64), rng)
    k_cache, v_cache = W.draw_cache(cfg, num_pages, rng)
    pos = np.concatenate([[0], rng.choice(17, 5, replace=False)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(Q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cand = (rng.random(int(cu_k[-1])) < 0.5).astype(np.uint8)
    inp = W.StepInputs(cfg=dataclasses.replace(cfg, track=50), dtype="bf16",
                       hidden=W.to_bf16_bits(rng.standard_normal((6, cfg.d_model),
                                                                 dtype=np.float32)),
                       positions=pos, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                       w_qkv=W.to_bf16_bits((rng.standard_normal((3 * cfg.d_model, cfg.d_model),
                                                                 dtype=np.float32) * 0.02)),
                       k_cache=k_cache, v_cache=v_cache, block_table=table, cand_mask=cand,
                       prompt_len=L, cache_len=L, window_start=L, tracked=np.zeros((3, 0), np.int32))
    got = run_gpu_step(inp, torch)
    r, _ = full_parity(inp, got)
    # no query rows -> zero importance for that sequence
    assert np.all(got["importance"][:, cu_k[1]:cu_k[2]] == 0)


def _attention_direct(torch, q_bits, k_cache, v_cache, table, page_size, cu_q, cu_k, H, D,
                      with_importance, max_seqlen_q):
    """fc_varlen_bidir_attention on device copies of the inputs."""
    from kv_cache_attention_step_amd import flashcache as fc
    dev = "cuda"
    B = len(cu_q) - 1
    T_q, T_k = int(cu_q[-1]), int(cu_k[-1])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q = t(q_bits.view(np.int16))
    kc, vc = t(k_cache.view(np.int16)), t(v_cache.view(np.int16))
    bt, cq, ck = t(table), t(cu_q), t(cu_k)
    out = torch.empty((T_q, H, D), dtype=torch.int16, device=dev)
    imp = torch.full((H, T_k), float("nan"), dtype=torch.float32, device=dev) if with_importance else None
    wsb = fc.fc_attention_workspace_size(B, T_q, T_k, H, D, with_importance, max_seqlen_q)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    fc.fc_varlen_bidir_attention(q, kc, vc, bt, table.shape[1], page_size, cq, ck, B, max_seqlen_q,
                                 T_k, H, D, 1.0 / math.sqrt(D), out, imp, 0, ws, wsb, fc.FC_DTYPE_BF16)
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint16)
    return o, (imp.cpu().numpy() if with_importance else None)


def test_attention_short_query_tiles(torch_cuda):
    """Every sequence has at most 64 query rows (the key-split mode: two waves per
    query half, each on one 32-key block of every tile): a cache shorter than one
    key block, a block holding a single key, ragged last tiles; with and without
    importance."""
    torch = torch_cuda
    _say("case short query tiles (max_seqlen_q <= 64)")
    cfg = dataclasses.replace(SMALL_BF16, name="short-q", seed=24)
    H, D, ps = cfg.n_heads, cfg.head_dim, cfg.page_size
    rng = W.rng_for(24, 1)
    L = np.array([5, 33, 200, 650], np.int64)
    Q = np.array([1, 17, 40, 64], np.int64)
    cfg = dataclasses.replace(cfg, batch=len(L))
    table, num_pages = W.draw_paging(cfg, L, rng)
    k_cache, v_cache = W.draw_cache(cfg, num_pages, rng, cache_len=L, block_table=table,
                                    tail_nan=True)
    cu_q = np.concatenate([[0], np.cumsum(Q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    q_bits = W.to_bf16_bits(rng.standard_normal((int(cu_q[-1]), H, D), dtype=np.float32) * 1.3)
    ref_o, ref_imp = O.varlen_attention(O.bf16_to_f64(q_bits), O.bf16_to_f64(k_cache),
                                        O.bf16_to_f64(v_cache), table, ps, cu_q, cu_k,
                                        1.0 / math.sqrt(D))
    for with_imp in (True, False):
        o, imp = _attention_direct(torch, q_bits, k_cache, v_cache, table, ps, cu_q, cu_k, H, D,
                                   with_imp, int(Q.max()))
        PU.assert_close(O.bf16_to_f64(o), ref_o, "bf16", f"attention out (importance={with_imp})")
        if with_imp:
            PU.assert_importance_close(imp, ref_imp)


@pytest.mark.parametrize("ps", [16, 4])
@pytest.mark.parametrize("accumulate", [0, 1])
def test_attention_long_queries_row_tile_split(torch_cuda, ps, accumulate):
    """Sequences of 0, 100, 129, 300 and 513 query rows (one to five 128-row tiles):
    with importance, every row tile beyond the first runs in its own workgroup and
    its column sums are added to row tile 0's in row-tile order. Attention out and
    importance against the oracle, with importance written (accumulate 0) and added
    to a prefilled buffer (accumulate 1: the zero-row sequence keeps its prefill);
    then the one-pass path on the same inputs (short last tiles in the key-split
    layout)."""
    torch = torch_cuda
    from kv_cache_attention_step_amd import flashcache as fc
    _say(f"case long queries, row-tile split (page size {ps}, accumulate {accumulate})")
    cfg = dataclasses.replace(SMALL_BF16, name="long-q", seed=31, page_size=ps)
    H, D = cfg.n_heads, cfg.head_dim
    rng = W.rng_for(31, ps)
    L = np.array([300, 64, 777, 1500, 900], np.int64)
    Q = np.array([0, 100, 129, 300, 513], np.int64)
    cfg = dataclasses.replace(cfg, batch=len(L))
    table, num_pages = W.draw_paging(cfg, L, rng)
    k_cache, v_cache = W.draw_cache(cfg, num_pages, rng, cache_len=L, block_table=table,
                                    tail_nan=True)
    cu_q = np.concatenate([[0], np.cumsum(Q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    T_q, T_k = int(cu_q[-1]), int(cu_k[-1])
    q_bits = W.to_bf16_bits(rng.standard_normal((T_q, H, D), dtype=np.float32) * 1.3)
    ref_o, ref_imp = O.varlen_attention(O.bf16_to_f64(q_bits), O.bf16_to_f64(k_cache),
                                        O.bf16_to_f64(v_cache), table, ps, cu_q, cu_k,
                                        1.0 / math.sqrt(D))
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    prefill = np.float32(0.25)
    imp = torch.full((H, T_k), float(prefill) if accumulate else float("nan"),
                     dtype=torch.float32, device=dev)
    out = torch.empty((T_q, H, D), dtype=torch.int16, device=dev)
    wsb = fc.fc_attention_workspace_size(len(L), T_q, T_k, H, D, 1, int(Q.max()))
    assert wsb >= 4 * H * T_k * 4      # four levels of column sums past row tile 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    fc.fc_varlen_bidir_attention(t(q_bits.view(np.int16)), t(k_cache.view(np.int16)),
                                 t(v_cache.view(np.int16)), t(table), table.shape[1], ps, t(cu_q),
                                 t(cu_k), len(L), int(Q.max()), T_k, H, D, 1.0 / math.sqrt(D), out,
                                 imp, accumulate, ws, wsb, fc.FC_DTYPE_BF16)
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint16)
    got = imp.cpu().numpy().astype(np.float64)
    PU.assert_close(O.bf16_to_f64(o), ref_o, "bf16", "attention out")
    if accumulate:
        z = slice(int(cu_k[0]), int(cu_k[1]))
        assert np.all(got[:, z] == prefill), "a sequence without query rows kept its prefill"
        got = got - float(prefill)
    PU.assert_importance_close(got, ref_imp)
    # per head, a sequence's column sums add up to its query rows
    for b in range(1, len(L)):
        sums = got[:, cu_k[b]:cu_k[b + 1]].sum(axis=1)
        np.testing.assert_allclose(sums, Q[b], rtol=2e-4)
    if accumulate == 0:
        # the one-pass path on the same inputs: 128-row tiles, the last tile of 129,
        # 300 and 513 rows (1, 44 and 1 rows left) in the key-split layout
        wsb1 = fc.fc_attention_workspace_size(len(L), T_q, T_k, H, D, 0, int(Q.max()))
        ws1 = torch.empty(max(wsb1, 1), dtype=torch.uint8, device=dev)
        out1 = torch.empty((T_q, H, D), dtype=torch.int16, device=dev)
        fc.fc_varlen_bidir_attention(t(q_bits.view(np.int16)), t(k_cache.view(np.int16)),
                                     t(v_cache.view(np.int16)), t(table), table.shape[1], ps,
                                     t(cu_q), t(cu_k), len(L), int(Q.max()), T_k, H, D,
                                     1.0 / math.sqrt(D), out1, None, 0, ws1, wsb1, fc.FC_DTYPE_BF16)
        torch.cuda.synchronize()
        PU.assert_close(O.bf16_to_f64(out1.cpu().numpy().view(np.uint16)), ref_o, "bf16",
                        "one-pass attention out")


def test_verify_small_vocab(torch_cuda):
    torch = torch_cuda
    from kv_cache_attention_step_amd.runner import VerifyBuffers
    _say("case verify small vocab")
    cfg = dataclasses.replace(CF.C4, name="C4-small", seed=41, batch=5, vocab=1000,
                              verify_len=(3, 20), d_model=256, n_heads=2)
    vi = W.make_verify_inputs(cfg, with_cache=False)
    vb = VerifyBuffers(vi)
    vb.verify()
    torch.cuda.synchronize()
    got = vb.fetch()
    am, conf, acc, acc_pos = O.verify_accept(vi.logits, vi.cu_positions, vi.draft, cfg.tau)
    assert np.array_equal(got["argmax"], am)
    np.testing.assert_allclose(got["conf"], conf, rtol=2e-6)
    # rows whose exact confidence sits within 1e-5 of tau may go either way in fp32
    near = np.abs(conf - cfg.tau) <= 1e-5
    assert np.array_equal(got["accept_row"][~near], acc[~near])
    rows = got["accept_row"]
    for b in range(cfg.batch):
        p0, p1 = int(vi.cu_positions[b]), int(vi.cu_positions[b + 1])
        n = p1 - p0
        # accept_pos is the AND of the position's two view rows
        exp = rows[2 * p0: 2 * p0 + n] & rows[2 * p0 + n: 2 * p0 + 2 * n]
        assert np.array_equal(got["accept_pos"][p0:p1], exp)
        near_pos = near[2 * p0: 2 * p0 + n] | near[2 * p0 + n: 2 * p0 + 2 * n]
        assert np.array_equal(got["accept_pos"][p0:p1][~near_pos], acc_pos[p0:p1][~near_pos])
    assert acc.sum() > 0 and (acc == 0).sum() > 0   # both outcomes exercised


def _verify_direct(torch, logits_bits, cu_p, draft, tau):
    """fv_verify_accept on device copies of [R, V] bf16 logit bits."""
    from kv_cache_attention_step_amd import flashcache as fc
    R, V = logits_bits.shape
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    lg, cp, dr = t(logits_bits.view(np.int16)), t(cu_p.astype(np.int32)), t(draft.astype(np.int32))
    am = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    cf = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    ar = torch.full((R,), 7, dtype=torch.uint8, device="cuda")
    ap = torch.full((R // 2,), 7, dtype=torch.uint8, device="cuda")
    fc.fv_verify_accept(lg, V, cp, len(cu_p) - 1, R, dr, tau, am, cf, ar, ap)
    torch.cuda.synchronize()
    return am.cpu().numpy(), cf.cpu().numpy(), ar.cpu().numpy(), ap.cpu().numpy()


def _edge_rows(rng, V):
    """16 logit rows (float64, bf16-exact) that stress the argmax and the sum:
    equal maxima in different lanes, chunks and loop steps, the max at the last
    element, constant rows, masked (-inf) vocabulary, ramps that raise the max
    at every step, and peaked rows (confident predictions)."""
    rnd = lambda: W.bf16_bits_to_f32(W.to_bf16_bits(rng.normal(0.0, 2.0, V))).astype(np.float64)
    rows = [rnd() for _ in range(16)]
    top = 30.0
    rows[1][np.sort(rng.choice(V, size=min(5, V), replace=False))] = top   # scattered ties
    if V >= 8 * 701:
        rows[2][8 * 700 + 2] = top      # later chunk of a lower lane ...
        rows[2][8 * 300 + 5] = top      # ... ties an earlier chunk of a higher lane
        rows[2][8 * 300 + 7] = top
    else:
        rows[2][[V - 1, V // 2, V // 3]] = top
    rows[3][V - 1] = top                # max only at the last element
    rows[4][:] = 0.5                    # constant row: argmax 0, conf 1/V
    rows[5][rng.random(V) < 0.5] = -np.inf
    rows[5][rng.integers(V)] = 1.0      # keep at least one finite logit
    rows[6][:] = -np.inf
    rows[6][V // 2] = -3.0              # one finite logit: conf 1
    rows[7][[0, V - 1]] = top           # tie between the first and last element
    ramp = np.linspace(-60.0, 60.0, V)
    rows[8] = W.bf16_bits_to_f32(W.to_bf16_bits(ramp)).astype(np.float64)
    rows[9] = rows[8][::-1].copy()
    for r in (10, 11, 12, 13):
        rows[r][rng.integers(V)] = 25.0 if r != 13 else 3.0
    return np.stack(rows)


def test_verify_argmax_ties_and_vocab_edges(torch_cuda):
    """Accept test on hand-shaped rows at several vocab sizes: multiples of 8
    (16-byte chunk path, fewer chunks than threads at the small sizes), odd
    sizes (element path), a single logit."""
    torch = torch_cuda
    rng = W.rng_for(53, 0)
    cu_p = np.array([0, 3, 8], np.int32)             # 8 positions, 16 rows
    tau = 0.9
    for V in (126464, 4104, 1000, 1003, 8, 7, 1):
        _say(f"case verify edges vocab={V}")
        x = _edge_rows(rng, V)
        bits = W.to_bf16_bits(x)
        assert np.array_equal(W.bf16_bits_to_f32(bits).astype(np.float64), x)   # bf16-exact
        am_ref = np.array([int(np.flatnonzero(r == r.max())[0]) for r in x])
        # drafts: the row's argmax for positions 0..4 (both views), random else
        draft = rng.integers(0, V, 8).astype(np.int32)
        for b in range(2):
            p0, p1 = int(cu_p[b]), int(cu_p[b + 1])
            n = p1 - p0
            for i in range(n):
                if p0 + i < 5:
                    draft[p0 + i] = am_ref[2 * p0 + i]
        am, conf, acc, acc_pos = O.verify_accept(bits, cu_p, draft, tau)
        got = _verify_direct(torch, bits, cu_p, draft, tau)
        assert np.array_equal(got[0], am), (V, got[0], am)
        np.testing.assert_allclose(got[1], conf, rtol=2e-6, err_msg=f"conf vocab={V}")
        near = np.abs(conf - tau) <= 1e-5
        assert np.array_equal(got[2][~near], acc[~near])
        if not near.any():
            assert np.array_equal(got[3], acc_pos)


@pytest.mark.parametrize("batch,q_per_seq", [(64, 128), (8, 256), (8, 512)])
def test_sweep_shapes(torch_cuda, batch, q_per_seq):
    """The shapes the throughput sweeps add beyond C2: 64 sequences (more than
    one wave of sequences: the longest-first order comes from its own kernel),
    and 256 or 512 query rows per sequence (the importance path walks two or
    four 128-row tiles per (sequence, head)); every output of every sequence
    against the oracle."""
    _say(f"case sweep shape B={batch}, {q_per_seq} query rows per sequence")
    cfg = dataclasses.replace(CF.C2, name=f"sweep-{batch}x{q_per_seq}", seed=90 + batch + q_per_seq,
                              batch=batch, window=q_per_seq // 2, track=q_per_seq // 2)
    inp = W.make_step_inputs(cfg)
    got = run_gpu_step(inp, torch_cuda)
    full_parity(inp, got)
