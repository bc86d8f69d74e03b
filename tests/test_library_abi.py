"""The C-ABI library on the CPU: it loads, exports every symbol include/tgs.h
declares, sizes workspaces, and rejects bad arguments before touching the GPU."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgs.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
LIB = os.path.join(ROOT, "top_gradient_sparsification_amd", "libtgs.so")


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tgs_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libtgs.so is not built (run __graft_entry__.build())")
    import top_gradient_sparsification_amd as tgs
    return tgs.library()


def test_header_declares_the_three_operations():
    names = declared_functions()
    for f in ("tgs_topk_ef_step", "tgs_threshold_ef_step", "tgs_gtopk_merge", "tgs_topk_workspace_bytes",
              "tgs_threshold_workspace_bytes", "tgs_gtopk_workspace_bytes", "tgs_status_string",
              "tgs_last_error", "tgs_check_device_error"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (tgs_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        getattr(lib, f)  # resolvable through ctypes too


def test_header_compiles_as_c():
    src = '#include "tgs.h"\n#include "tgs_testing.h"\nint main(void){ return (int)sizeof(tgs_status); }\n'
    proc = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only", "-I", os.path.dirname(HEADER),
                           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-"], input=src,
                          capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr


def test_workspace_queries(lib):
    import top_gradient_sparsification_amd as tgs
    assert tgs.topk_workspace_bytes(25_600_000, 25_600) > 0
    assert tgs.topk_workspace_bytes(10, 11) == 0          # k > n
    assert tgs.topk_workspace_bytes(-1, 0) == 0
    assert tgs.topk_workspace_bytes(2**31, 1) == 0       # n beyond int32 indices
    assert tgs.topk_workspace_bytes(0, 0) > 0
    # the selected entries are staged twice (8 bytes each) in the workspace
    assert tgs.topk_workspace_bytes(1 << 20, 100_000) >= 16 * 100_000
    assert tgs.threshold_workspace_bytes(1_500_000_000) > 0
    assert tgs.threshold_workspace_bytes(-5) == 0
    assert tgs.gtopk_workspace_bytes(32, 25_600, 25_600_000) > 0
    assert tgs.gtopk_workspace_bytes(0, 1, 10) == 0
    assert tgs.gtopk_workspace_bytes(2, 11, 10) == 0


def test_invalid_arguments_fail_before_any_launch(lib):
    vp = ctypes.c_void_p
    dummy = vp(0x10000)  # never dereferenced: validation fails first
    i64 = ctypes.c_int64
    # n < 0
    st = lib.tgs_topk_ef_step(dummy, dummy, i64(-1), i64(0), None, None, dummy, 1 << 30, None)
    assert st == -1 and b"n=" in lib.tgs_last_error()
    # k > n
    st = lib.tgs_topk_ef_step(dummy, vp(0x20000), i64(10), i64(11), vp(0x30000), vp(0x40000), dummy, 1 << 30, None)
    assert st == -1
    # overlapping grad / residual
    st = lib.tgs_topk_ef_step(vp(0x100000), vp(0x100010), i64(64), i64(1), vp(0x900000), vp(0xA00000),
                              vp(0xB00000), 1 << 30, None)
    assert st == -1 and b"overlap" in lib.tgs_last_error()
    # misaligned pointer
    st = lib.tgs_topk_ef_step(vp(0x100002), vp(0x200000), i64(64), i64(1), vp(0x900000), vp(0xA00000),
                              vp(0xB00000), 1 << 30, None)
    assert st == -1
    # workspace too small
    st = lib.tgs_topk_ef_step(vp(0x100000), vp(0x200000), i64(64), i64(1), vp(0x900000), vp(0xA00000),
                              vp(0xB00000), 16, None)
    assert st == -2 and b"workspace" in lib.tgs_last_error()
    # lambda NaN / negative
    for lam in (float("nan"), -1.0):
        st = lib.tgs_threshold_ef_step(vp(0x100000), vp(0x200000), i64(64), ctypes.c_float(lam), vp(0x900000),
                                       vp(0xA00000), i64(8), vp(0xC00000), vp(0xB00000), 1 << 30, None)
        assert st == -1
    # P < 1, k > n
    st = lib.tgs_gtopk_merge(vp(0x100000), vp(0x200000), 0, i64(1), i64(10), vp(0x900000), vp(0xA00000),
                             vp(0xC00000), vp(0xB00000), 1 << 30, None)
    assert st == -1
    st = lib.tgs_gtopk_merge(vp(0x100000), vp(0x200000), 2, i64(11), i64(10), vp(0x900000), vp(0xA00000),
                             vp(0xC00000), vp(0xB00000), 1 << 30, None)
    assert st == -1
    assert lib.tgs_status_string(-2).startswith(b"TGS_EWORKSPACE")
    assert lib.tgs_set_option(1, 15) == -1
    assert lib.tgs_set_option(99, 0) == -1


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The binding and the library never import, load or run the oracle."""
    pkg = os.path.join(ROOT, "top_gradient_sparsification_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f


def test_segmented_table_checks_before_any_launch(lib):
    """The layer-wise step validates its host segment table (and the
    workspace size) before it enqueues anything: fake device pointers are
    never touched."""
    import numpy as np
    import top_gradient_sparsification_amd as tgs
    assert tgs.topk_segmented_workspace_bytes([0, 10, 300_000, 300_100], [1, 300, 0]) > 0
    assert tgs.topk_segmented_workspace_bytes([0], []) > 0
    for offs, ks in (([0, 10, 5], [1, 1]),          # offsets decrease
                     ([1, 10], [1]),                 # offsets[0] != 0
                     ([0, 10], [11]),                # k above the segment length
                     ([0, 10], [-1]),
                     ([0, 2**31], [1])):             # beyond int32 indices
        assert tgs.topk_segmented_workspace_bytes(offs, ks) == 0, (offs, ks)
        o = np.asarray(offs, np.int64)
        k = np.asarray(ks, np.int64)
        st = lib.tgs_topk_ef_step_segmented(ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), k.size,
                                            o.ctypes.data, k.ctypes.data, ctypes.c_void_p(0x300000),
                                            ctypes.c_void_p(0x400000), ctypes.c_void_p(0x500000), 1 << 30, None)
        assert st == -1, (offs, ks)
    o = np.asarray([0, 1000, 400_000], np.int64)
    k = np.asarray([3, 400], np.int64)
    need = tgs.topk_segmented_workspace_bytes(o, k)
    st = lib.tgs_topk_ef_step_segmented(ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000), 2, o.ctypes.data,
                                        k.ctypes.data, ctypes.c_void_p(0x30000000), ctypes.c_void_p(0x40000000),
                                        ctypes.c_void_p(0x50000000), need - 1, None)
    assert st == -2
