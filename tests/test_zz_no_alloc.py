"""fc_varlen_bidir_attention_noalloc (the attention without a caller workspace,
its scratch in a static device array) against fc_varlen_bidir_attention with a
workspace, through the C ABI: several calls in a row on one device, each
smaller than the one before, on the paths that use the scratch (key-split
statistics and O partials, the longest-first order of more than 64 sequences)
and the one-pass path. The outputs must be bit-identical (same kernels, same
inputs) and within the bf16 bar of the oracle."""
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


def _case(seed, B, H, L_range, Q_range, ps=16):
    """Attention inputs: bf16 queries, a paged bf16 cache with NaN past every
    sequence's end, ragged lengths."""
    cfg = dataclasses.replace(CF.C2, name=f"noalloc{seed}", seed=seed, batch=B, n_heads=H,
                              d_model=H * 128, page_size=ps)
    rng = W.rng_for(seed, 11)
    L = rng.integers(L_range[0], L_range[1] + 1, size=B).astype(np.int64)
    Q = rng.integers(Q_range[0], Q_range[1] + 1, size=B).astype(np.int64)
    table, num_pages = W.draw_paging(cfg, L, rng)
    kc, vc = W.draw_cache(cfg, num_pages, rng, cache_len=L, block_table=table, tail_nan=True)
    cu_q = np.concatenate([[0], np.cumsum(Q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    q = W.to_bf16_bits(rng.standard_normal((int(cu_q[-1]), H, 128), dtype=np.float32) * 1.3)
    return dict(cfg=cfg, q=q, kc=kc, vc=vc, table=table, cu_q=cu_q, cu_k=cu_k, Q=Q, L=L, H=H, B=B)


def _run(torch, c, with_imp, noalloc):
    from kv_cache_attention_step_amd import flashcache as fc
    from kv_cache_attention_step_amd.runner import to_device, to_host
    B, H = c["B"], c["H"]
    T_q, T_k = int(c["cu_q"][-1]), int(c["cu_k"][-1])
    q, kc, vc = to_device(c["q"]), to_device(c["kc"]), to_device(c["vc"])
    bt, cq, ck = to_device(c["table"]), to_device(c["cu_q"]), to_device(c["cu_k"])
    out = torch.full((T_q, H, 128), 0x7FC0, dtype=torch.int16, device="cuda")
    imp = torch.full((H, T_k), float("nan"), dtype=torch.float32, device="cuda") if with_imp else None
    args = (q, kc, vc, bt, c["table"].shape[1], c["cfg"].page_size, cq, ck, B, int(c["Q"].max()),
            T_k, H, 128, 1.0 / math.sqrt(128), out, imp, 0)
    if noalloc:
        fc.fc_varlen_bidir_attention_noalloc(*args, fc.FC_DTYPE_BF16)
    else:
        wsb = fc.fc_attention_workspace_size(B, T_q, T_k, H, 128, with_imp, int(c["Q"].max()))
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        fc.fc_varlen_bidir_attention(*args, ws, wsb, fc.FC_DTYPE_BF16)
    torch.cuda.synchronize()
    return to_host(out), (to_host(imp) if with_imp else None)


def test_noalloc_attention_matches_workspace_attention():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from kv_cache_attention_step_amd import flashcache as fc
    fc.load()
    cases = [
        ("one sequence, 32 heads: key split in 8 (17 MB of scratch)", _case(81, 1, 32, (700, 900), (128, 128)), True),
        ("3 sequences, 4 heads: key split in 8, smaller", _case(82, 3, 4, (40, 400), (30, 128)), True),
        ("70 sequences: longest-first order from the scratch", _case(83, 70, 4, (20, 150), (5, 40)), True),
        ("2 sequences, one pass (no importance)", _case(84, 2, 4, (30, 200), (3, 20)), False),
    ]
    for what, c, with_imp in cases:
        _say(f"case noalloc: {what}")
        o_ref, i_ref = _run(torch, c, with_imp, noalloc=False)
        o_got, i_got = _run(torch, c, with_imp, noalloc=True)
        assert np.array_equal(o_got, o_ref), f"{what}: attention output differs"
        if with_imp:
            assert np.array_equal(i_got.view(np.uint32), i_ref.view(np.uint32)), f"{what}: importance differs"
        ref_o, ref_imp = O.varlen_attention(O.bf16_to_f64(c["q"]), O.bf16_to_f64(c["kc"]),
                                            O.bf16_to_f64(c["vc"]), c["table"], c["cfg"].page_size,
                                            c["cu_q"], c["cu_k"], 1.0 / math.sqrt(128))
        PU.assert_close(O.bf16_to_f64(o_got), ref_o, "bf16", f"{what}: attention out vs oracle")
        if with_imp:
            PU.assert_importance_close(i_got, ref_imp, f"{what}: importance vs oracle")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """A request whose workspace would exceed the static array is refused before
    anything is enqueued (the pointers are never touched)."""
    from kv_cache_attention_step_amd import flashcache as fc
    fc.load()
    B = 8_000_000            # the longest-first order alone needs 32 MB
    assert fc.fc_attention_workspace_size(B, 0, 0, 32, 128, 1, 128) > fc.FC_ATTN_NOALLOC_SCRATCH_BYTES
    fake = 0x1000
    with pytest.raises(fc.FlashCacheError) as ei:
        fc.fc_varlen_bidir_attention_noalloc(fake, fake, fake, fake, 4, 16, fake, fake, B, 128,
                                             1000, 32, 128, 0.088, fake, fake, 0, fc.FC_DTYPE_BF16,
                                             stream=0)
    assert ei.value.status_name == "FC_ERR_WORKSPACE" and "static scratch" in str(ei.value)
