"""CPU-only checks of the C-ABI library: it loads and exports every entry
point the header declares; host-side helpers behave. No compute calls."""
import ctypes
import os
import re

import pytest

from block_sparse_cross_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "splitkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(splitkv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from block_sparse_cross_amd import build
        build.build()
    return binding.lib()


def test_header_declares_the_four_calls():
    fns = declared_functions()
    for name in ("splitkv_plan", "splitkv_attn_fwd", "splitkv_attn_bwd", "splitkv_lse_merge"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(binding.EXPORTED) == set(declared_functions())


def test_status_strings(lib):
    assert binding.status_str(0) == "ok"
    assert "invalid" in binding.status_str(-1)
    assert "unsupported" in binding.status_str(-2)
    assert "workspace" in binding.status_str(-3)
    assert "HIP" in binding.status_str(-4)
    assert "unknown" in binding.status_str(7)


def test_workspace_sizes_are_host_arithmetic(lib):
    an = binding.Anchors(None, None, 512, 16)
    hd = binding.Heads(32, 8, 128, binding.SPLITKV_BF16, 128 ** -0.5)
    fwd = binding.splitkv_workspace_bytes(binding.SPLITKV_OP_FWD, an, hd, None)
    bwd = binding.splitkv_workspace_bytes(binding.SPLITKV_OP_BWD, an, hd, None)
    assert fwd >= 512 * 8 and fwd % 256 == 0
    assert bwd >= fwd + (512 * 16 * 4 // 32) * 8 and bwd % 256 == 0
    assert binding.splitkv_workspace_bytes(binding.SPLITKV_OP_MERGE) == 0
    assert binding.splitkv_workspace_bytes(binding.SPLITKV_OP_PLAN) == 0


def test_library_has_no_oracle_symbols(lib):
    # the product library must not contain the oracle
    for name in ("oracle_lpt", "oracle_partial_attn", "oracle_merge"):
        with pytest.raises(AttributeError):
            getattr(lib, name)


def test_ceiling_library_exports_its_loop(lib):
    """The matrix-core ceiling loop bench.py reports beside the attention rates
    is a library of its own, built with the main one; it rejects bad arguments
    on the host (no launch)."""
    from block_sparse_cross_amd import build
    if not os.path.exists(build.CEILING_LIB):
        build.build()
    c = ctypes.CDLL(build.CEILING_LIB)
    fn = c.splitkv_ceiling_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_void_p]
    assert fn(None, 1, 1, None, None) == -1
    assert fn(ctypes.c_void_p(16), -1, 1, ctypes.c_void_p(16), None) == -1
    assert fn(ctypes.c_void_p(16), 1, 0, ctypes.c_void_p(16), None) == -1
    assert fn(ctypes.c_void_p(17), 1, 1, ctypes.c_void_p(16), None) == -1
