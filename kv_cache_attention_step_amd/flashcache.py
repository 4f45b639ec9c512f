"""Thin Python binding of libflashcache.so (ctypes).

Argument marshalling only: every function forwards to the C entry point of the
same name. Tensors are passed as raw device pointers (``tensor.data_ptr()``),
``None`` becomes NULL, and the stream defaults to torch's current stream. A
non-zero status raises FlashCacheError with the library's message.

The library must have been built (``__graft_entry__.build()`` or
``python -m kv_cache_attention_step_amd.build_lib``); loading fails loudly
otherwise. There is no fallback implementation.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflashcache.so")

FC_DTYPE_F32 = 0
FC_DTYPE_BF16 = 1
FC_TOPK_MAX_LEN = 16384
FC_ATTN_NOALLOC_SCRATCH_BYTES = 24 << 20

_STATUS = {0: "FC_OK", 1: "FC_ERR_INVALID_VALUE", 2: "FC_ERR_UNSUPPORTED", 3: "FC_ERR_WORKSPACE",
           4: "FC_ERR_HIP"}

EXPORTS = ("fc_status_string", "fc_last_error", "fc_version", "fc_qkv_rope_cache_write",
           "fc_qkv_workspace_size",
           "fc_attention_workspace_size", "fc_varlen_bidir_attention", "fc_importance_topk",
           "fv_verify_accept", "fc_linear_residual", "fc_assemble_query", "fc_rms_row_scale",
           "fc_validate_step_inputs", "fc_varlen_bidir_attention_noalloc",
           "fc_probe_kv_stream", "fc_probe_mfma_bf16", "fv_confidence_accept",
           "fv_fork_view_pages", "fv_commit_accepted", "fv_lmhead_workspace_size",
           "fv_lmhead_verify_accept")


class FlashCacheError(RuntimeError):
    def __init__(self, func, status, message):
        self.status = status
        self.status_name = _STATUS.get(status, str(status))
        super().__init__(f"{func}: {self.status_name}: {message}")


_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32
F32 = ctypes.c_float
SZ = ctypes.c_size_t

_SIGS = {
    "fc_status_string": ([I32], ctypes.c_char_p),
    "fc_last_error": ([], ctypes.c_char_p),
    "fc_version": ([], ctypes.c_char_p),
    "fc_qkv_rope_cache_write": ([P, P, P, I32, I32, P, I32, I32, I32, F32, P, P, P, I32, I32, P, P,
                                 P, P, SZ, I32, P], I32),
    "fc_rms_row_scale": ([P, I32, I32, F32, P, I32, P], I32),
    "fc_qkv_workspace_size": ([I32, I32, I32, I32], SZ),
    "fc_attention_workspace_size": ([I32, I32, I32, I32, I32, I32, I32], SZ),
    "fc_varlen_bidir_attention": ([P, P, P, P, I32, I32, P, P, I32, I32, I32, I32, I32, F32, P, P,
                                   I32, P, SZ, I32, P], I32),
    "fc_importance_topk": ([P, P, I32, I32, I32, P, I32, P, P, P, P], I32),
    "fv_verify_accept": ([P, I32, P, I32, I32, P, F32, P, P, P, P, P], I32),
    "fc_linear_residual": ([P, P, P, I32, I32, I32, I32, P], I32),
    "fc_assemble_query": ([P, P, I32, P, P, I32, P, P], I32),
    "fc_validate_step_inputs": ([P, P, P, I32, I32, I32, P, I32, I32, I32, P], I32),
    "fv_lmhead_workspace_size": ([I32, I32], SZ),
    "fv_lmhead_verify_accept": ([P, P, I32, I32, P, I32, I32, P, F32, P, SZ, P, P, P, P, P], I32),
    "fv_fork_view_pages": ([P, P, P, I32, I32, P, P, I32, I32, I32, I32, I32, P, P], I32),
    "fv_commit_accepted": ([P, P, P, P, I32, I32, P, P, I32, I32, P, I32, I32, P], I32),
    "fv_confidence_accept": ([P, I32, P, I32, I32, F32, I32, P, P, P, P], I32),
    "fc_probe_kv_stream": ([P, P, P, I32, I32, P, I32, I32, I32, I32, I32, P, P], I32),
    "fc_probe_mfma_bf16": ([I32, I32, P, P], I32),
    "fc_varlen_bidir_attention_noalloc": ([P, P, P, P, I32, I32, P, P, I32, I32, I32, I32, I32, F32,
                                           P, P, I32, I32, P], I32),
}


def load(path: str = LIB_PATH):
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libflashcache.so not found at {path}: build it first with "
                           f"`python -m kv_cache_attention_step_amd.build_lib`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(name, status):
    if status != 0:
        msg = load().fc_last_error().decode(errors="replace")
        raise FlashCacheError(name, status, msg)


def fc_version() -> str:
    return load().fc_version().decode()


def fc_status_string(status: int) -> str:
    return load().fc_status_string(status).decode()


def fc_qkv_workspace_size(T_q, d_model, head_dim, dtype) -> int:
    return int(load().fc_qkv_workspace_size(T_q, d_model, head_dim, dtype))


def fc_qkv_rope_cache_write(hidden, positions, cu_seqlens_q, B, T_q, w_qkv, d_model, n_heads,
                            head_dim, rope_base, k_cache, v_cache, block_table, max_pages_per_seq,
                            page_size, q_out, slot_mapping, workspace, workspace_bytes, dtype,
                            stream=None, row_scale=None):
    st = load().fc_qkv_rope_cache_write(
        _p(hidden), _p(positions), _p(cu_seqlens_q), B, T_q, _p(w_qkv), d_model, n_heads,
        head_dim, rope_base, _p(k_cache), _p(v_cache), _p(block_table), max_pages_per_seq,
        page_size, _p(q_out), _p(slot_mapping), _p(row_scale), _p(workspace), workspace_bytes,
        dtype, _stream(stream))
    _check("fc_qkv_rope_cache_write", st)


def fc_rms_row_scale(x, M, N, eps, scale, dtype, stream=None):
    st = load().fc_rms_row_scale(_p(x), M, N, eps, _p(scale), dtype, _stream(stream))
    _check("fc_rms_row_scale", st)


def fc_attention_workspace_size(B, T_q, T_k, n_heads, head_dim, with_importance,
                                max_seqlen_q) -> int:
    return int(load().fc_attention_workspace_size(B, T_q, T_k, n_heads, head_dim,
                                                  int(bool(with_importance)), max_seqlen_q))


def fc_varlen_bidir_attention(q, k_cache, v_cache, block_table, max_pages_per_seq, page_size,
                              cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, T_k, n_heads, head_dim,
                              softmax_scale, out, importance, accumulate, workspace,
                              workspace_bytes, dtype, stream=None):
    st = load().fc_varlen_bidir_attention(
        _p(q), _p(k_cache), _p(v_cache), _p(block_table), max_pages_per_seq, page_size,
        _p(cu_seqlens_q), _p(cu_seqlens_k), B, max_seqlen_q, T_k, n_heads, head_dim,
        softmax_scale, _p(out), _p(importance), int(bool(accumulate)), _p(workspace),
        workspace_bytes, dtype, _stream(stream))
    _check("fc_varlen_bidir_attention", st)


def fc_importance_topk(importance, cu_seqlens_k, B, T_k, n_heads, candidate_mask, k, topk_pos,
                       topk_count, topk_score, stream=None):
    st = load().fc_importance_topk(_p(importance), _p(cu_seqlens_k), B, T_k, n_heads,
                                   _p(candidate_mask), k, _p(topk_pos), _p(topk_count),
                                   _p(topk_score), _stream(stream))
    _check("fc_importance_topk", st)


def fv_verify_accept(logits, vocab, cu_positions, B, R, draft_tokens, tau, argmax, conf,
                     accept_row, accept_pos, stream=None):
    st = load().fv_verify_accept(_p(logits), vocab, _p(cu_positions), B, R, _p(draft_tokens), tau,
                                 _p(argmax), _p(conf), _p(accept_row), _p(accept_pos),
                                 _stream(stream))
    _check("fv_verify_accept", st)


def fc_linear_residual(x, w, h_inout, M, N, K, dtype, stream=None):
    st = load().fc_linear_residual(_p(x), _p(w), _p(h_inout), M, N, K, dtype, _stream(stream))
    _check("fc_linear_residual", st)


def fc_assemble_query(topk_pos, topk_count, k, window_start, cu_seqlens_q, B, positions,
                      stream=None):
    st = load().fc_assemble_query(_p(topk_pos), _p(topk_count), k, _p(window_start),
                                  _p(cu_seqlens_q), B, _p(positions), _stream(stream))
    _check("fc_assemble_query", st)


def fc_validate_step_inputs(positions, cu_seqlens_q, cu_seqlens_k, B, T_q, T_k, block_table,
                            max_pages_per_seq, page_size, num_pages, stream=None):
    st = load().fc_validate_step_inputs(_p(positions), _p(cu_seqlens_q), _p(cu_seqlens_k), B, T_q,
                                        T_k, _p(block_table), max_pages_per_seq, page_size,
                                        num_pages, _stream(stream))
    _check("fc_validate_step_inputs", st)


def fc_varlen_bidir_attention_noalloc(q, k_cache, v_cache, block_table, max_pages_per_seq,
                                      page_size, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, T_k,
                                      n_heads, head_dim, softmax_scale, out, importance,
                                      accumulate, dtype, stream=None):
    st = load().fc_varlen_bidir_attention_noalloc(
        _p(q), _p(k_cache), _p(v_cache), _p(block_table), max_pages_per_seq, page_size,
        _p(cu_seqlens_q), _p(cu_seqlens_k), B, max_seqlen_q, T_k, n_heads, head_dim,
        softmax_scale, _p(out), _p(importance), int(bool(accumulate)), dtype, _stream(stream))
    _check("fc_varlen_bidir_attention_noalloc", st)


def fc_probe_kv_stream(k_cache, v_cache, block_table, max_pages_per_seq, page_size, cu_seqlens_k,
                       B, n_heads, head_dim, k_passes, sink, stream=None, k_policy=0):
    st = load().fc_probe_kv_stream(_p(k_cache), _p(v_cache), _p(block_table), max_pages_per_seq,
                                   page_size, _p(cu_seqlens_k), B, n_heads, head_dim, k_passes,
                                   k_policy, _p(sink), _stream(stream))
    _check("fc_probe_kv_stream", st)


def fc_probe_mfma_bf16(n_blocks, iters, sink, stream=None):
    st = load().fc_probe_mfma_bf16(n_blocks, iters, _p(sink), _stream(stream))
    _check("fc_probe_mfma_bf16", st)


def fv_confidence_accept(logits, vocab, cu_positions, B, R, tau, at_least_one, argmax, conf,
                         accept, stream=None):
    st = load().fv_confidence_accept(_p(logits), vocab, _p(cu_positions), B, R, tau,
                                     int(bool(at_least_one)), _p(argmax), _p(conf), _p(accept),
                                     _stream(stream))
    _check("fv_confidence_accept", st)


def fv_fork_view_pages(k_cache, v_cache, block_table, max_pages_per_seq, page_size, cu_seqlens_k,
                       verify_start, B, n_heads, head_dim, view_page_base, pages_per_view,
                       view_block_table, stream=None):
    st = load().fv_fork_view_pages(_p(k_cache), _p(v_cache), _p(block_table), max_pages_per_seq,
                                   page_size, _p(cu_seqlens_k), _p(verify_start), B, n_heads,
                                   head_dim, view_page_base, pages_per_view,
                                   _p(view_block_table), _stream(stream))
    _check("fv_fork_view_pages", st)


def fv_commit_accepted(k_cache, v_cache, block_table, view_block_table, max_pages_per_seq,
                       page_size, cu_positions, verify_start, B, n_positions, accept_pos, n_heads,
                       head_dim, stream=None):
    st = load().fv_commit_accepted(_p(k_cache), _p(v_cache), _p(block_table),
                                   _p(view_block_table), max_pages_per_seq, page_size,
                                   _p(cu_positions), _p(verify_start), B, n_positions,
                                   _p(accept_pos), n_heads, head_dim, _stream(stream))
    _check("fv_commit_accepted", st)


def fv_lmhead_workspace_size(R, vocab) -> int:
    return int(load().fv_lmhead_workspace_size(R, vocab))


def fv_lmhead_verify_accept(hidden, w_lm, d_model, vocab, cu_positions, B, R, draft_tokens, tau,
                            workspace, workspace_bytes, argmax, conf, accept_row, accept_pos,
                            stream=None):
    st = load().fv_lmhead_verify_accept(_p(hidden), _p(w_lm), d_model, vocab, _p(cu_positions), B,
                                        R, _p(draft_tokens), tau, _p(workspace), workspace_bytes,
                                        _p(argmax), _p(conf), _p(accept_row), _p(accept_pos),
                                        _stream(stream))
    _check("fv_lmhead_verify_accept", st)
