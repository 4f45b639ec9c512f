"""Device-side drivers for the Flash-Cache step built on the C ABI.

Torch provides device memory and streams only; every step of the path runs in
the library's HIP kernels. Used by the benchmark, the smoke check and the GPU
tests.
"""
import math
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from . import flashcache as fc
from . import workload as W
from .configs import StepConfig
from .workload import StepInputs, VerifyInputs


def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, device="cuda"):
    """numpy -> device tensor; bf16 bit patterns travel as int16."""
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint8:
        pass
    return torch.from_numpy(a).to(device)


def to_host(t, like: Optional[str] = None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def dtype_code(dtype: str) -> int:
    return fc.FC_DTYPE_BF16 if dtype == "bf16" else fc.FC_DTYPE_F32


def elem_dtype(dtype: str):
    torch = _torch()
    return torch.int16 if dtype == "bf16" else torch.float32


class StepBuffers:
    """Device copies of one step's inputs plus its output buffers."""

    def __init__(self, inp: StepInputs, device="cuda"):
        torch = _torch()
        cfg = inp.cfg
        self.inp = inp
        self.cfg = cfg
        self.device = device
        self.B = inp.B
        self.T_q = inp.T_q
        self.T_k = inp.T_k
        self.H, self.D, self.d = cfg.n_heads, cfg.head_dim, cfg.d_model
        self.dtype = dtype_code(inp.dtype)
        self.hidden = to_device(inp.hidden, device)
        self.cu_q = to_device(inp.cu_seqlens_q, device)
        # query positions: given (verify-shaped inputs), or assembled on the device
        # from the tracked positions and the masked window (step S1)
        self.assembled = inp.positions is None
        if self.assembled:
            self.positions = torch.empty(inp.T_q, dtype=torch.int32, device=device)
            self.tracked = to_device(np.ascontiguousarray(inp.tracked, np.int32), device) \
                if inp.tracked.size else None
            self.tracked_count = to_device(inp.tracked_count, device)
            self.window_start = to_device(inp.window_start, device)
        else:
            self.positions = to_device(inp.positions, device)
        self.cu_k = to_device(inp.cu_seqlens_k, device)
        self.w_qkv = to_device(inp.w_qkv, device)
        self.k_cache = to_device(inp.k_cache, device)
        self.v_cache = to_device(inp.v_cache, device)
        self.block_table = to_device(inp.block_table, device)
        self.cand_mask = to_device(inp.cand_mask, device)
        et = elem_dtype(inp.dtype)
        self.q_out = torch.empty((self.T_q, self.H, self.D), dtype=et, device=device)
        self.attn_out = torch.empty((self.T_q, self.H, self.D), dtype=et, device=device)
        self.slot_mapping = torch.empty(self.T_q, dtype=torch.int32, device=device)
        self.importance = torch.empty((self.H, self.T_k), dtype=torch.float32, device=device)
        k = max(1, cfg.track)
        self.k = k
        self.topk_pos = torch.empty((self.B, k), dtype=torch.int32, device=device)
        self.topk_count = torch.empty(self.B, dtype=torch.int32, device=device)
        self.topk_score = torch.empty((self.B, k), dtype=torch.float32, device=device)
        ws = fc.fc_attention_workspace_size(self.B, self.T_q, self.T_k, self.H, self.D, 1,
                                            int(inp.max_seqlen_q))
        self.ws_bytes = ws
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device) if ws else None
        qws = fc.fc_qkv_workspace_size(self.T_q, self.H * self.D, self.D, self.dtype)
        self.qkv_ws_bytes = qws
        self.qkv_workspace = torch.empty(qws, dtype=torch.uint8, device=device) if qws else None
        self.max_seqlen_q = inp.max_seqlen_q
        self.scale = 1.0 / math.sqrt(self.D)

    # the calls of one Flash-Cache step
    def assemble(self, stream=None):
        """Query positions = tracked positions + masked window (nothing to do when
        the inputs carry explicit positions)."""
        if not self.assembled:
            return
        k = self.inp.tracked.shape[1]
        fc.fc_assemble_query(self.tracked, self.tracked_count if k else None, max(k, 1),
                             self.window_start, self.cu_q, self.B, self.positions, stream)

    def qkv(self, stream=None):
        cfg = self.cfg
        fc.fc_qkv_rope_cache_write(self.hidden, self.positions, self.cu_q, self.B, self.T_q,
                                   self.w_qkv, self.d, self.H, self.D, cfg.rope_base, self.k_cache,
                                   self.v_cache, self.block_table, self.inp.max_pages,
                                   cfg.page_size, self.q_out, self.slot_mapping, self.qkv_workspace,
                                   self.qkv_ws_bytes, self.dtype, stream)

    def attention(self, stream=None, importance=True, accumulate=False):
        fc.fc_varlen_bidir_attention(self.q_out, self.k_cache, self.v_cache, self.block_table,
                                     self.inp.max_pages, self.cfg.page_size, self.cu_q, self.cu_k,
                                     self.B, self.max_seqlen_q, self.T_k, self.H, self.D,
                                     self.scale, self.attn_out,
                                     self.importance if importance else None, accumulate,
                                     self.workspace, self.ws_bytes, self.dtype, stream)

    def topk(self, stream=None):
        fc.fc_importance_topk(self.importance, self.cu_k, self.B, self.T_k, self.H, self.cand_mask,
                              self.k, self.topk_pos, self.topk_count, self.topk_score, stream)

    def run(self, stream=None):
        self.assemble(stream)
        self.qkv(stream)
        self.attention(stream)
        self.topk(stream)

    def fetch(self) -> Dict[str, np.ndarray]:
        return dict(positions=to_host(self.positions),
                    q_out=to_host(self.q_out), attn_out=to_host(self.attn_out),
                    slot_mapping=to_host(self.slot_mapping), importance=to_host(self.importance),
                    topk_pos=to_host(self.topk_pos), topk_count=to_host(self.topk_count),
                    topk_score=to_host(self.topk_score), k_cache=to_host(self.k_cache),
                    v_cache=to_host(self.v_cache))


class VerifyBuffers:
    """Flash-Verify-shaped step: Q-only projection of both views, one-pass
    attention over the cache, then the accept test on the logits."""

    def __init__(self, vi: VerifyInputs, device="cuda"):
        torch = _torch()
        self.vi = vi
        self.step = StepBuffers(vi.step, device) if vi.step.k_cache.size else None
        cfg = vi.cfg
        self.V = cfg.vocab
        self.tau = cfg.tau
        self.R = 2 * int(vi.cu_positions[-1])
        self.n_pos = int(vi.cu_positions[-1])
        self.cu_p = to_device(vi.cu_positions, device)
        self.draft = to_device(vi.draft, device)
        self.logits = to_device(vi.logits, device) if vi.logits is not None else None
        self.B = cfg.batch
        self.argmax = torch.empty(self.R, dtype=torch.int32, device=device)
        self.conf = torch.empty(self.R, dtype=torch.float32, device=device)
        self.accept_row = torch.empty(self.R, dtype=torch.uint8, device=device)
        self.accept_pos = torch.empty(self.n_pos, dtype=torch.uint8, device=device)

    def qkv(self, stream=None):
        s = self.step
        fc.fc_qkv_rope_cache_write(s.hidden, s.positions, s.cu_q, s.B, s.T_q, s.w_qkv, s.d, s.H,
                                   s.D, s.cfg.rope_base, None, None, s.block_table,
                                   s.inp.max_pages, s.cfg.page_size, s.q_out, s.slot_mapping,
                                   s.qkv_workspace, s.qkv_ws_bytes, s.dtype, stream)

    def attention(self, stream=None):
        self.step.attention(stream, importance=False)

    def verify(self, stream=None):
        fc.fv_verify_accept(self.logits, self.V, self.cu_p, self.B, self.R, self.draft,
                            self.tau, self.argmax, self.conf, self.accept_row, self.accept_pos,
                            stream)

    def run(self, stream=None):
        self.qkv(stream)
        self.attention(stream)
        self.verify(stream)

    def fetch(self):
        out = dict(argmax=to_host(self.argmax), conf=to_host(self.conf),
                   accept_row=to_host(self.accept_row), accept_pos=to_host(self.accept_pos))
        if self.step is not None:
            out.update(q_out=to_host(self.step.q_out), attn_out=to_host(self.step.attn_out))
        return out


class LayerStackDriver:
    """Block-wise denoising through a stack of layers.

    At denoising step s the query of every sequence is its tracked positions
    followed by block s (block length `block_len`); the tracked positions come
    from the previous step's top-k over the importance summed across all layers
    (none at step 0, fewer than k while few blocks are decoded). Each layer
    projects and rotates the query, writes its own cache, attends to the whole
    cache (importance accumulated over layers) and adds its output projection to
    the hidden states: h <- h + O Wo^T. Each layer's input is RMS-normalised
    (no learned weight) through a per-token row scale applied inside the
    projection; without it the residual state of a deep stack with random
    weights grows without bound. All of it runs through the C ABI.
    """

    def __init__(self, cfg: StepConfig, device="cuda", layers: Optional[int] = None,
                 steps: Optional[int] = None):
        torch = _torch()
        self.cfg = cfg
        self.device = device
        self.n_layers = layers or cfg.layers
        self.n_steps = steps or cfg.steps
        self.B, self.H, self.D, self.d = cfg.batch, cfg.n_heads, cfg.head_dim, cfg.d_model
        self.dtype = dtype_code(cfg.dtype)
        self.k = cfg.track
        prompt_len, cache_len, table, num_pages, cu_k = W.multistep_base(cfg)
        self.prompt_len, self.cache_len, self.table, self.cu_k_np = prompt_len, cache_len, table, cu_k
        self.T_k = int(cu_k[-1])
        self.max_pages = int(table.shape[1])
        self.cu_k = to_device(cu_k, device)
        self.block_table = to_device(table, device)
        kc, vc = W.stack_prefill(cfg, num_pages)
        self.prefill = (kc, vc)
        dk, dv = to_device(kc, device), to_device(vc, device)
        self.k_cache = [dk.clone() for _ in range(self.n_layers)]
        self.v_cache = [dv.clone() for _ in range(self.n_layers)]
        del dk, dv
        self.w_qkv, self.w_o = [], []
        for l in range(self.n_layers):
            wq, wo = W.layer_weights(cfg, l)
            self.w_qkv.append(to_device(wq, device))
            self.w_o.append(to_device(wo, device))
        # per-step host-side inputs (query lengths, windows, candidates, fresh states)
        self.steps = []
        for st in range(self.n_steps):
            q = W.step_query_lens(cfg, st)
            cu_q = np.arange(self.B + 1, dtype=np.int32) * q
            wstart = (prompt_len + cfg.block_len * st).astype(np.int32)
            cand = W.step_candidates(cfg, st + 1, prompt_len, cu_k)
            hid = W.step_hidden(cfg, st, int(cu_q[-1]))
            self.steps.append(dict(Q=q, T_q=int(cu_q[-1]), cu_q=to_device(cu_q, device),
                                   window_start=to_device(wstart, device),
                                   cand=to_device(cand, device), hidden=to_device(hid, device)))
        T_max = max(x["T_q"] for x in self.steps)
        et = elem_dtype(cfg.dtype)
        self.h = torch.empty((T_max, self.d), dtype=et, device=device)
        self.positions = torch.empty(T_max, dtype=torch.int32, device=device)
        self.q_out = torch.empty((T_max, self.H, self.D), dtype=et, device=device)
        self.attn_out = torch.empty((T_max, self.H, self.D), dtype=et, device=device)
        self.importance = torch.empty((self.H, self.T_k), dtype=torch.float32, device=device)
        self.row_scale = torch.empty(T_max, dtype=torch.float32, device=device)
        self.topk_pos = torch.full((self.B, self.k), -1, dtype=torch.int32, device=device)
        self.topk_count = torch.zeros(self.B, dtype=torch.int32, device=device)
        self.topk_score = torch.empty((self.B, self.k), dtype=torch.float32, device=device)
        ws = fc.fc_attention_workspace_size(self.B, T_max, self.T_k, self.H, self.D, 1,
                                            max(x["Q"] for x in self.steps))
        self.ws_bytes = ws
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        qws = fc.fc_qkv_workspace_size(T_max, self.H * self.D, self.D, self.dtype)
        self.qkv_ws_bytes = qws
        self.qkv_workspace = torch.empty(max(qws, 1), dtype=torch.uint8, device=device)
        self.scale = 1.0 / math.sqrt(self.D)

    def run_step(self, st: int, stream=None, on_layer=None):
        cfg = self.cfg
        x = self.steps[st]
        T_q = x["T_q"]
        fc.fc_assemble_query(self.topk_pos if st > 0 else None, self.topk_count if st > 0 else None,
                             self.k, x["window_start"], x["cu_q"], self.B, self.positions, stream)
        if stream is not None:
            with _torch().cuda.stream(stream):
                self.h[:T_q].copy_(x["hidden"])
        else:
            self.h[:T_q].copy_(x["hidden"])
        for l in range(self.n_layers):
            fc.fc_rms_row_scale(self.h, T_q, self.d, cfg.rms_eps, self.row_scale, self.dtype, stream)
            fc.fc_qkv_rope_cache_write(self.h, self.positions, x["cu_q"], self.B, T_q,
                                       self.w_qkv[l], self.d, self.H, self.D, cfg.rope_base,
                                       self.k_cache[l], self.v_cache[l], self.block_table,
                                       self.max_pages, cfg.page_size, self.q_out, None,
                                       self.qkv_workspace, self.qkv_ws_bytes, self.dtype, stream,
                                       row_scale=self.row_scale)
            fc.fc_varlen_bidir_attention(self.q_out, self.k_cache[l], self.v_cache[l],
                                         self.block_table, self.max_pages, cfg.page_size,
                                         x["cu_q"], self.cu_k, self.B, x["Q"], self.T_k, self.H,
                                         self.D, self.scale, self.attn_out, self.importance,
                                         l > 0, self.workspace, self.ws_bytes, self.dtype, stream)
            fc.fc_linear_residual(self.attn_out, self.w_o[l], self.h, T_q, self.d, self.d,
                                  self.dtype, stream)
            if on_layer is not None:
                on_layer(st, l)
        fc.fc_importance_topk(self.importance, self.cu_k, self.B, self.T_k, self.H, x["cand"],
                              self.k, self.topk_pos, self.topk_count, self.topk_score, stream)


class TwoViewVerifyBuffers:
    """Flash-Verify's two views with view-private K/V, then the commit.

    Each sequence b verifies its last n_b positions (verify_start[b] = L_b - n_b)
    through a draft view and a [MASK] view (rows: n_b draft rows, then n_b mask
    rows). The cache arrays get pages_per_view spare pages per (sequence, view)
    after the shared pages; fv_fork_view_pages gives each view a page-table row
    of its own over them; the fused projection writes each view's fresh K/V
    there (2B virtual sequences); the one-pass attention attends each view to
    its own cache; fv_verify_accept decides; fv_commit_accepted copies the
    accepted positions' draft-view K/V into the shared cache.
    """

    def __init__(self, vi: VerifyInputs, device="cuda"):
        torch = _torch()
        inp = vi.step
        cfg = vi.cfg
        self.vi, self.inp, self.cfg, self.device = vi, inp, cfg, device
        B, H, D, ps = cfg.batch, cfg.n_heads, cfg.head_dim, cfg.page_size
        self.B, self.H, self.D, self.d, self.ps = B, H, D, cfg.d_model, ps
        self.dtype = dtype_code(inp.dtype)
        n = vi.verify_len.astype(np.int64)
        L = inp.cache_len.astype(np.int64)
        self.n_pos = int(n.sum())
        self.pages_per_view = int((int(n.max()) + ps - 1) // ps + 1)
        num_pages = inp.k_cache.shape[0]
        self.view_page_base = num_pages
        total = num_pages + 2 * B * self.pages_per_view
        et = elem_dtype(inp.dtype)
        self.k_cache = torch.zeros((total, H, ps, D), dtype=et, device=device)
        self.v_cache = torch.zeros((total, H, ps, D), dtype=et, device=device)
        self.k_cache[:num_pages].copy_(to_device(inp.k_cache, device))
        self.v_cache[:num_pages].copy_(to_device(inp.v_cache, device))
        self.max_pages = inp.max_pages
        self.block_table = to_device(inp.block_table, device)
        self.view_table = torch.full((2 * B, self.max_pages), -1, dtype=torch.int32, device=device)
        self.verify_start_np = (L - n).astype(np.int32)
        self.verify_start = to_device(self.verify_start_np, device)
        self.cu_k = to_device(inp.cu_seqlens_k, device)
        self.cu_p = to_device(vi.cu_positions, device)
        # the 2B virtual sequences: (b, draft), (b, mask), ...
        nv = np.repeat(n, 2)
        self.cu_q_np = np.concatenate([[0], np.cumsum(nv)]).astype(np.int32)
        self.cu_kv_np = np.concatenate([[0], np.cumsum(np.repeat(L, 2))]).astype(np.int32)
        self.cu_q = to_device(self.cu_q_np, device)
        self.cu_kv = to_device(self.cu_kv_np, device)
        self.T_q = int(self.cu_q_np[-1])
        self.T_kv = int(self.cu_kv_np[-1])
        self.max_q = int(n.max())
        self.hidden = to_device(inp.hidden, device)
        self.positions = to_device(inp.positions, device)
        self.w_qkv = to_device(inp.w_qkv, device)
        self.q_out = torch.empty((self.T_q, H, D), dtype=et, device=device)
        self.attn_out = torch.empty((self.T_q, H, D), dtype=et, device=device)
        self.slot_mapping = torch.empty(self.T_q, dtype=torch.int32, device=device)
        qws = fc.fc_qkv_workspace_size(self.T_q, self.d, D, self.dtype)
        self.qkv_ws_bytes = qws
        self.qkv_workspace = torch.empty(max(qws, 1), dtype=torch.uint8, device=device)
        ws = fc.fc_attention_workspace_size(2 * B, self.T_q, self.T_kv, H, D, 0, self.max_q)
        self.ws_bytes = ws
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.accept_pos = torch.zeros(self.n_pos, dtype=torch.uint8, device=device)
        self.scale = 1.0 / math.sqrt(D)

    def fork(self, stream=None):
        fc.fv_fork_view_pages(self.k_cache, self.v_cache, self.block_table, self.max_pages, self.ps,
                              self.cu_k, self.verify_start, self.B, self.H, self.D,
                              self.view_page_base, self.pages_per_view, self.view_table, stream)

    def qkv(self, stream=None):
        fc.fc_qkv_rope_cache_write(self.hidden, self.positions, self.cu_q, 2 * self.B, self.T_q,
                                   self.w_qkv, self.d, self.H, self.D, self.cfg.rope_base,
                                   self.k_cache, self.v_cache, self.view_table, self.max_pages,
                                   self.ps, self.q_out, self.slot_mapping, self.qkv_workspace,
                                   self.qkv_ws_bytes, self.dtype, stream)

    def attention(self, stream=None):
        fc.fc_varlen_bidir_attention(self.q_out, self.k_cache, self.v_cache, self.view_table,
                                     self.max_pages, self.ps, self.cu_q, self.cu_kv, 2 * self.B,
                                     self.max_q, self.T_kv, self.H, self.D, self.scale,
                                     self.attn_out, None, 0, self.workspace, self.ws_bytes,
                                     self.dtype, stream)

    def commit(self, accept_pos=None, stream=None):
        fc.fv_commit_accepted(self.k_cache, self.v_cache, self.block_table, self.view_table,
                              self.max_pages, self.ps, self.cu_p, self.verify_start, self.B,
                              self.n_pos, self.accept_pos if accept_pos is None else accept_pos,
                              self.H, self.D, stream)

    def run_views(self, stream=None):
        self.fork(stream)
        self.qkv(stream)
        self.attention(stream)


class LMHeadBuffers:
    """The LM head with the Flash-Verify accept test fused in: final hidden rows
    of both views times W_lm, reduced per row to argmax and confidence on the
    device (the logits are never written), then the two-view accept test."""

    def __init__(self, li, device="cuda"):
        torch = _torch()
        vi = li.vi
        cfg = vi.cfg
        self.li, self.cfg = li, cfg
        self.R = li.hidden.shape[0]
        self.n_pos = int(vi.cu_positions[-1])
        self.hidden = to_device(li.hidden, device)
        self.w_lm = to_device(li.w_lm, device)
        self.cu_p = to_device(vi.cu_positions, device)
        self.draft = to_device(vi.draft, device)
        ws = fc.fv_lmhead_workspace_size(self.R, cfg.vocab)
        self.ws_bytes = ws
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.argmax = torch.empty(self.R, dtype=torch.int32, device=device)
        self.conf = torch.empty(self.R, dtype=torch.float32, device=device)
        self.accept_row = torch.empty(self.R, dtype=torch.uint8, device=device)
        self.accept_pos = torch.empty(self.n_pos, dtype=torch.uint8, device=device)

    def run(self, stream=None):
        cfg = self.cfg
        fc.fv_lmhead_verify_accept(self.hidden, self.w_lm, cfg.d_model, cfg.vocab, self.cu_p,
                                   cfg.batch, self.R, self.draft, cfg.tau, self.workspace,
                                   self.ws_bytes, self.argmax, self.conf, self.accept_row,
                                   self.accept_pos, stream)

    def fetch(self):
        return dict(argmax=to_host(self.argmax), conf=to_host(self.conf),
                    accept_row=to_host(self.accept_row), accept_pos=to_host(self.accept_pos))
