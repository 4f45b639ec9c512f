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
    need = fc.fc_attention_workspace_size(2, 8, 64, 2, 128, 1, 8)
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


def _rejects(status_name, fn, *args, **kw):
    with pytest.raises(fc.FlashCacheError) as ei:
        fn(*args, stream=0, **kw)
    assert ei.value.status_name == status_name, str(ei.value)


def test_verify_side_argument_checks():
    """Host checks of the two-view, commit, LM-head and confidence entry points:
    rejected before anything is enqueued (the pointers are never touched)."""
    _lib()
    F = FAKE
    # confidence-aware acceptance
    _rejects("FC_ERR_INVALID_VALUE", fc.fv_confidence_accept, F, 100, F, 0, 4, 0.9, 1, F, F, F)
    _rejects("FC_ERR_INVALID_VALUE", fc.fv_confidence_accept, F, 100, F, 1, 4, 0.0, 1, F, F, F)
    _rejects("FC_ERR_INVALID_VALUE", fc.fv_confidence_accept, None, 100, F, 1, 4, 0.9, 1, F, F, F)
    fc.fv_confidence_accept(None, 100, F, 1, 0, 0.9, 1, None, None, None, stream=0)  # no rows
    # fork of view-private pages
    fork = lambda **kw: dict(dict(k_cache=F, v_cache=F, block_table=F, max_pages_per_seq=8,
                                  page_size=16, cu_seqlens_k=F, verify_start=F, B=2, n_heads=4,
                                  head_dim=128, view_page_base=100, pages_per_view=3,
                                  view_block_table=F), **kw)
    for kw, st in ((dict(B=0), "FC_ERR_INVALID_VALUE"), (dict(head_dim=64), "FC_ERR_UNSUPPORTED"),
                   (dict(page_size=12), "FC_ERR_INVALID_VALUE"), (dict(pages_per_view=0), "FC_ERR_INVALID_VALUE"),
                   (dict(verify_start=None), "FC_ERR_INVALID_VALUE"),
                   (dict(view_page_base=2 ** 31 - 10), "FC_ERR_INVALID_VALUE")):
        with pytest.raises(fc.FlashCacheError) as ei:
            fc.fv_fork_view_pages(**fork(**kw), stream=0)
        assert ei.value.status_name == st, (kw, str(ei.value))
    # commit
    commit = lambda **kw: dict(dict(k_cache=F, v_cache=F, block_table=F, view_block_table=F,
                                    max_pages_per_seq=8, page_size=16, cu_positions=F,
                                    verify_start=F, B=2, n_positions=10, accept_pos=F, n_heads=4,
                                    head_dim=128), **kw)
    for kw, st in ((dict(n_heads=0), "FC_ERR_INVALID_VALUE"), (dict(head_dim=96), "FC_ERR_UNSUPPORTED"),
                   (dict(accept_pos=None), "FC_ERR_INVALID_VALUE"), (dict(page_size=3), "FC_ERR_INVALID_VALUE")):
        with pytest.raises(fc.FlashCacheError) as ei:
            fc.fv_commit_accepted(**commit(**kw), stream=0)
        assert ei.value.status_name == st, (kw, str(ei.value))
    fc.fv_commit_accepted(**commit(n_positions=0), stream=0)   # nothing to commit
    # LM head: vocabulary and width the tile pipeline does not take, odd row count,
    # small workspace
    lm = lambda **kw: dict(dict(hidden=F, w_lm=F, d_model=512, vocab=2048, cu_positions=F, B=2,
                                R=8, draft_tokens=F, tau=0.9, workspace=F,
                                workspace_bytes=fc.fv_lmhead_workspace_size(8, 2048), argmax=F,
                                conf=F, accept_row=F, accept_pos=F), **kw)
    for kw, st in ((dict(vocab=2000), "FC_ERR_UNSUPPORTED"), (dict(d_model=500), "FC_ERR_UNSUPPORTED"),
                   (dict(R=7), "FC_ERR_INVALID_VALUE"), (dict(tau=1.5), "FC_ERR_INVALID_VALUE"),
                   (dict(workspace_bytes=16), "FC_ERR_WORKSPACE"), (dict(hidden=None), "FC_ERR_INVALID_VALUE")):
        with pytest.raises(fc.FlashCacheError) as ei:
            fc.fv_lmhead_verify_accept(**lm(**kw), stream=0)
        assert ei.value.status_name == st, (kw, str(ei.value))
    assert fc.fv_lmhead_workspace_size(8, 2048) == 8 * 16 * 12
    assert fc.fv_lmhead_workspace_size(0, 2048) == 0
    # measurement probes
    _rejects("FC_ERR_INVALID_VALUE", fc.fc_probe_kv_stream, F, F, F, 8, 16, F, 2, 4, 128, 3, F)
    _rejects("FC_ERR_UNSUPPORTED", fc.fc_probe_kv_stream, F, F, F, 8, 16, F, 2, 4, 64, 1, F)
    _rejects("FC_ERR_INVALID_VALUE", fc.fc_probe_kv_stream, F, F, F, 8, 12, F, 2, 4, 128, 1, F)
    # cache policy of the K pass: 0..3, only with two passes, pages of 16 keys or more
    _rejects("FC_ERR_INVALID_VALUE", fc.fc_probe_kv_stream, F, F, F, 8, 16, F, 2, 4, 128, 2, F,
             k_policy=4)
    _rejects("FC_ERR_INVALID_VALUE", fc.fc_probe_kv_stream, F, F, F, 8, 16, F, 2, 4, 128, 1, F,
             k_policy=1)
    _rejects("FC_ERR_UNSUPPORTED", fc.fc_probe_kv_stream, F, F, F, 8, 4, F, 2, 4, 128, 2, F,
             k_policy=1)
    _rejects("FC_ERR_INVALID_VALUE", fc.fc_probe_mfma_bf16, 0, 10, F)
    _rejects("FC_ERR_INVALID_VALUE", fc.fc_probe_mfma_bf16, 4, 10, None)


def test_last_error_message_names_the_call():
    lib = _lib()
    st = lib.fc_importance_topk(None, None, 0, 0, 0, None, 0, None, None, None, None)
    assert st == 1
    assert b"fc_importance_topk" in lib.fc_last_error()


def test_last_error_is_per_thread():
    """Two host threads each make a rejected call, then (after both have) read the
    message: each sees its own call's message, not the other thread's."""
    import threading
    lib = _lib()
    barrier = threading.Barrier(2)
    seen = {}

    def topk_thread():
        st = lib.fc_importance_topk(None, None, 0, 0, 0, None, 0, None, None, None, None)
        barrier.wait()
        seen["topk"] = (st, lib.fc_last_error())

    def linear_thread():
        st = lib.fc_linear_residual(None, None, None, 0, 0, 0, 0, None)
        barrier.wait()
        seen["linear"] = (st, lib.fc_last_error())

    threads = [threading.Thread(target=topk_thread), threading.Thread(target=linear_thread)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=30)
    assert seen["topk"][0] != 0 and b"fc_importance_topk" in seen["topk"][1]
    assert seen["linear"][0] != 0 and b"fc_linear_residual" in seen["linear"][1]
    assert b"fc_linear_residual" not in seen["topk"][1]


def _sanitized_build(tmp):
    """Library sources with AddressSanitizer and UndefinedBehaviorSanitizer on
    their host code (device code unchanged), linked with the C harness into one
    executable."""
    import subprocess
    from concurrent.futures import ThreadPoolExecutor
    from kv_cache_attention_step_amd import build_lib as BL
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
        cmd = [BL.hipcc(), "-x", "hip", f"--offload-arch={BL.ARCH}", "-O2", "-g", "-std=c++17",
               "-fPIC", "-c", os.path.join(BL.CSRC, src), "-o", obj] + san + BL.DEVICE_FLAGS
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}: {r.stderr[-3000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, BL.SOURCES))
    harness = os.path.join(tmp, "abi_host_checks.o")
    r = subprocess.run([clang, "-std=c11", "-g", "-O1", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "abi_host_checks.c"), "-o", harness],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(tmp, "abi_host_checks")
    r = subprocess.run([clang + "++", "-fsanitize=address,undefined", "-o", exe, harness] + objs +
                       ["-L" + os.path.join(rocm, "lib"), "-lamdhip64",
                        "-Wl,-rpath," + os.path.join(rocm, "lib")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.slow
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """Every entry point's argument checks, size queries at edge values and
    status strings, run from C against the library's host code built with ASan
    and UBSan: any out-of-bounds access, use after free, signed overflow or
    other undefined behaviour on the host side aborts the run."""
    import shutil
    import subprocess
    from kv_cache_attention_step_amd import build_lib as BL
    try:
        BL.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = _sanitized_build(str(tmp_path))
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.pop("FC_DEBUG", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "abi host checks ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
    shutil.rmtree(str(tmp_path), ignore_errors=True)
