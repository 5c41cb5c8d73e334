"""The C ABI without a GPU: the built library loads and exports every function
that include/sspec.h declares, the Python binding covers the same set, and
the host-side workspace sizing follows the header's rules (sizes grow with
the problem, invalid arguments give 0).  No kernel is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sspec.h")
LIB = os.path.join(ROOT, "sparse_self_speculative_amd", "libsspec.so")
I32 = ctypes.c_int32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)   # comments mention names too
    return sorted(set(re.findall(r"\b(?:const\s+char\s*\*|int|size_t)\s+(sspec_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):   # nothing built yet: build it (hipcc cross-compiles without a GPU)
        import sys
        sys.path.insert(0, ROOT)
        import __graft_entry__
        __graft_entry__.build()
    return ctypes.CDLL(LIB)


def sized(lib, name, nargs):
    f = getattr(lib, name)
    f.restype = ctypes.c_size_t
    f.argtypes = [I32] * nargs
    return f


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("sspec_verify_attn", "sspec_pillar_topk", "sspec_sparse_draft_attn", "sspec_unified_attn",
              "sspec_verify_workspace_size", "sspec_pillar_topk_workspace_size", "sspec_draft_workspace_size",
              "sspec_unified_workspace_size", "sspec_workspace_init", "sspec_read_device_error",
              "sspec_last_error"):
        assert n in names, n


def test_library_exports_every_declared_function(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared in sspec.h but not exported: {missing}"


def test_binding_covers_the_header():
    from sparse_self_speculative_amd import sspec as S
    assert sorted(S.EXPORTED) == declared_functions()
    for py in ("verify_attn", "pillar_topk", "sparse_draft_attn", "unified_attn", "verify_workspace_size",
               "pillar_topk_workspace_size", "draft_workspace_size", "unified_workspace_size", "workspace",
               "read_device_error"):
        assert callable(getattr(S, py)), py


def test_last_error_is_a_string(lib):
    f = lib.sspec_last_error
    f.restype = ctypes.c_char_p
    assert isinstance(f(), bytes)


def test_workspace_sizes(lib):
    uni = sized(lib, "sspec_unified_workspace_size", 6)   # num_seqs, max_verify, max_ctx, hq, hkv, k
    base = uni(128, 16, 32776, 32, 8, 8)
    assert base > 0
    assert uni(128, 16, 65536, 32, 8, 8) > base           # longer contexts
    assert uni(256, 32, 32776, 32, 8, 8) > base           # more requests
    assert uni(128, 16, 32776, 32, 8, 16) > base          # more verify queries
    for bad in ((0, 16, 32776, 32, 8, 8), (128, -1, 32776, 32, 8, 8), (128, 16, 0, 32, 8, 8),
                (128, 16, 32776, 4, 8, 8), (128, 16, 32776, 32, 0, 8), (128, 16, 32776, 32, 8, -1)):
        assert uni(*bad) == 0, bad

    ver = sized(lib, "sspec_verify_workspace_size", 5)    # n, max_ctx, hq, hkv, k
    assert ver(16, 4096, 32, 8, 8) > ver(8, 4096, 32, 8, 8) > 0
    assert ver(-1, 4096, 32, 8, 8) == 0 and ver(8, 0, 32, 8, 8) == 0 and ver(8, 4096, 32, 8, -1) == 0

    top = sized(lib, "sspec_pillar_topk_workspace_size", 3)   # n, max_ctx, hkv
    assert top(16, 4096, 8) > top(8, 4096, 8) > 0
    assert top(8, 0, 8) == 0 and top(8, 4096, 0) == 0

    dra = sized(lib, "sspec_draft_workspace_size", 4)   # n, max_ctx, hq, hkv
    assert dra(16, 4096, 32, 8) >= dra(8, 4096, 32, 8) > 0
    assert dra(8, 4096, 4, 8) == 0 and dra(-1, 4096, 32, 8) == 0
