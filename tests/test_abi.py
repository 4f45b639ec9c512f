"""C ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host (nothing is enqueued)."""
import ctypes
import os
import re

import pytest

from kv_cache_attention_step_amd import flashcache as fc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashcache.h")


def _lib():
    if not os.path.exists(fc.LIB_PATH):
        pytest.skip("libflashcache.so not built (run __graft_entry__.build())")
    return fc.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:fc|fv)_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_step_calls():
    names = declared_functions()
    for n in ("fc_qkv_rope_cache_write", "fc_varlen_bidir_attention", "fc_importance_topk",
              "fv_verify_accept"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in flashcache.h but not exported"
    assert set(declared_functions()) == set(fc.EXPORTS)
    assert fc.fc_version().startswith("flashcache-gfx950")


def test_status_strings_are_never_null():
    _lib()
    for st in range(0, 6):
        assert isinstance(fc.fc_status_string(st), str) and fc.fc_status_string(st)


FAKE = 0x1000  # a non-null pointer value that is never dereferenced by a rejected call


def _expect(status_name, fn, *args):
    with pytest.raises(fc.FlashCacheError) as ei:
        fn(*args, stream=0)
    assert ei.value.status_name == status_name, str(ei.value)
    assert str(ei.value)


def test_qkv_argument_checks():
    _lib()
    base = dict(hidden=FAKE, positions=FAKE, cu_seqlens_q=FAKE, B=1, T_q=4, w_qkv=FAKE,
                d_model=256, n_heads=2, head_dim=128, rope_base=1e4, k_cache=FAKE, v_cache=FAKE,
                block_table=FAKE, max_pages_per_seq=4, page_size=16, q_out=FAKE,
                slot_mapping=None, workspace=FAKE, workspace_bytes=1 << 20,
                dtype=fc.FC_DTYPE_BF16, row_scale=None)

    def call(**over):
        a = dict(base)
        a.update(over)
        return lambda stream: fc.fc_qkv_rope_cache_write(**a, stream=stream)

    def expect(name, **over):
        with pytest.raises(fc.FlashCacheError) as ei:
            call(**over)(0)
        assert ei.value.status_name == name, str(ei.value)

    expect("FC_ERR_INVALID_VALUE", B=0)
    expect("FC_ERR_INVALID_VALUE", d_model=255)
    expect("FC_ERR_INVALID_VALUE", dtype=7)
    expect("FC_ERR_INVALID_VALUE", hidden=None)
    expect("FC_ERR_INVALID_VALUE", k_cache=None)            # only one of the two caches
    expect("FC_ERR_INVALID_VALUE", page_size=12)
    expect("FC_ERR_INVALID_VALUE", block_table=None)        # cache write needs the table
    expect("FC_ERR_INVALID_VALUE", rope_base=1.0)
    expect("FC_ERR_UNSUPPORTED", n_heads=4, head_dim=64)    # bf16 supports D = 128 only
    expect("FC_ERR_UNSUPPORTED", n_heads=3, d_model=384)    # d % 256 != 0
    expect("FC_ERR_UNSUPPORTED", dtype=fc.FC_DTYPE_F32, n_heads=8, head_dim=32)
    need = fc.fc_qkv_workspace_size(4, 256, 128, fc.FC_DTYPE_BF16)
    assert need >= 4 * 64 * 8
    expect("FC_ERR_WORKSPACE", workspace_bytes=need - 1)
    expect("FC_ERR_WORKSPACE", workspace=None)
    for name in ("hidden", "w_qkv", "q_out", "k_cache", "workspace"):   # 16-byte rows
        over = {name: FAKE + 8}
        if name == "k_cache":
            over["v_cache"] = FAKE + 8
        expect("FC_ERR_INVALID_VALUE", **over)
    assert fc.fc_qkv_workspace_size(4, 256, 64, fc.FC_DTYPE_F32) == 0
    # nothing to do is not an error
    call(T_q=0)(0)


def test_attention_argument_checks():
    _lib()
    base = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, block_table=FAKE, max_pages_per_seq=4,
                page_size=16, cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, B=2, max_seqlen_q=8, T_k=64,
                n_heads=2, head_dim=128, softmax_scale=0.088, out=FAKE, importance=FAKE,
                accumulate=0, workspace=FAKE, workspace_bytes=1 << 26, dtype=fc.FC_DTYPE_BF16)

    def expect(name, **over):
        a = dict(base)
        a.update(over)
        with pytest.raises(fc.FlashCacheError) as ei:
            fc.fc_varlen_bidir_attention(**a, stream=0)
        assert ei.value.status_name == name, str(ei.value)

    expect("FC_ERR_INVALID_VALUE", B=0)
    expect("FC_ERR_INVALID_VALUE", q=None)
    expect("FC_ERR_INVALID_VALUE", page_size=0)
    expect("FC_ERR_INVALID_VALUE", softmax_scale=0.0)
    expect("FC_ERR_INVALID_VALUE", dtype=3)
    expect("FC_ERR_UNSUPPORTED", head_dim=64)
    need = fc.fc_attention_workspace_size(2, 8, 64, 2, 128, 1)
    assert need >= 2 * 4
    expect("FC_ERR_WORKSPACE", workspace_bytes=need - 1)
    expect("FC_ERR_WORKSPACE", workspace=None)
    a = dict(base)
    a.update(max_seqlen_q=0)
    fc.fc_varlen_bidir_attention(**a, stream=0)   # empty query: returns OK, enqueues nothing


def test_topk_verify_linear_assemble_argument_checks():
    _lib()
    with pytest.raises(fc.FlashCacheError) as ei:
        fc.fc_importance_topk(FAKE, FAKE, 1, 10, 2, None, 0, FAKE, FAKE, None, stream=0)
    assert ei.value.status_name == "FC_ERR_INVALID_VALUE"
    with pytest.raises(fc.FlashCacheError) as ei:
        fc.fc_importance_topk(FAKE, None, 1, 10, 2, None, 4, FAKE, FAKE, None, stream=0)
    assert ei.value.status_name == "FC_ERR_INVALID_VALUE"
    for tau in (0.0, 1.5, -0.1):
        with pytest.raises(fc.FlashCacheError) as ei:
            fc.fv_verify_accept(FAKE, 100, FAKE, 1, 4, FAKE, tau, FAKE, FAKE, FAKE, None, stream=0)
        assert ei.value.status_name == "FC_ERR_INVALID_VALUE"
    with pytest.raises(fc.FlashCacheError) as ei:
        fc.fv_verify_accept(FAKE, 100, FAKE, 1, 3, FAKE, 0.9, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status_name == "FC_ERR_INVALID_VALUE"      # odd row count
    fc.fv_verify_accept(None, 100, FAKE, 1, 0, None, 0.9, None, None, None, None, stream=0)
    with pytest.raises(fc.FlashCacheError) as ei:
        fc.fc_linear_residual(FAKE, FAKE, FAKE, 4, 100, 64, fc.FC_DTYPE_BF16, stream=0)
    assert ei.value.status_name == "FC_ERR_UNSUPPORTED"
    with pytest.raises(fc.FlashCacheError) as ei:
        fc.fc_linear_residual(None, FAKE, FAKE, 4, 128, 64, fc.FC_DTYPE_BF16, stream=0)
    assert ei.value.status_name == "FC_ERR_INVALID_VALUE"
    with pytest.raises(fc.FlashCacheError) as ei:
        fc.fc_assemble_query(None, FAKE, 4, FAKE, FAKE, 2, FAKE, stream=0)
    assert ei.value.status_name == "FC_ERR_INVALID_VALUE"
    for args in ((FAKE, 4, 0, 1e-5, FAKE), (FAKE, 4, 16, -1.0, FAKE), (None, 4, 16, 1e-5, FAKE)):
        with pytest.raises(fc.FlashCacheError) as ei:
            fc.fc_rms_row_scale(*args, fc.FC_DTYPE_BF16, stream=0)
        assert ei.value.status_name == "FC_ERR_INVALID_VALUE"


def test_last_error_message_names_the_call():
    lib = _lib()
    st = lib.fc_importance_topk(None, None, 0, 0, 0, None, 0, None, None, None, None)
    assert st == 1
    assert b"fc_importance_topk" in lib.fc_last_error()
