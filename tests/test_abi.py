"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from tenant_composite_lora_amd import tclora

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tcl.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tcl_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return tclora.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(tclora.EXPORTS) == names


def test_version(L):
    assert b"gfx950" in L.tcl_version()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"(TCL_E[A-Z]+|TCL_OK)\s*=\s*(-?\d+)", text))
    assert int(consts["TCL_OK"]) == tclora.OK
    assert int(consts["TCL_EINVAL"]) == tclora.EINVAL
    assert int(consts["TCL_EALIGN"]) == tclora.EALIGN
    assert int(consts["TCL_ENOSPC"]) == tclora.ENOSPC
    assert int(consts["TCL_EUNSUPPORTED"]) == tclora.EUNSUPPORTED
    assert int(consts["TCL_EHIP"]) == tclora.EHIP
    assert f"TCL_MAX_RANK {tclora.MAX_RANK}" in text
    assert f"TCL_MAX_PAIRS_PER_GROUP {tclora.MAX_PAIRS_PER_GROUP}" in text


def test_status_codes_match_oracle():
    import oracle as O
    assert (O.OK, O.EINVAL, O.ENOSPC, O.EUNSUPPORTED) == (
        tclora.OK, tclora.EINVAL, tclora.ENOSPC, tclora.EUNSUPPORTED)


def test_plan_bytes(L):
    out = ctypes.c_size_t(0)
    assert L.tcl_plan_bytes(32, 32, 96, 64, 96, ctypes.byref(out)) == 0
    small = out.value
    assert small > 0 and small % 256 == 0
    assert L.tcl_plan_bytes(4224, 4224, 10600, 256, 10600, ctypes.byref(out)) == 0
    assert out.value > small
    assert L.tcl_plan_bytes(0, 0, 0, 1, 0, ctypes.byref(out)) == 0
    for args in [(-1, 1, 1, 1, 1), (1, -1, 1, 1, 1), (1, 1, -1, 1, 1), (1, 1, 1, 0, 1),
                 (1, 1, 1, 1, -1), (1 << 25, 1, 1, 1, 1)]:
        assert L.tcl_plan_bytes(*args, ctypes.byref(out)) == tclora.EINVAL, args
        assert len(L.tcl_last_error()) > 0
    assert L.tcl_plan_bytes(1, 1, 1, 1, 1, None) == tclora.EINVAL


def _comp(T=3, G=2, NP=3, N=4, cap=4, ptr=0x1000):
    return tclora.Composites(T, G, NP, N, cap, ptr, ptr, ptr, ptr)


def test_plan_map_host_errors(L):
    h = ctypes.c_void_p(0)
    need = tclora.plan_bytes(3, 2, 3, 4, 4)
    # null composites / out
    assert L.tcl_plan_map(None, 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    c = _comp()
    assert L.tcl_plan_map(ctypes.byref(c), 0x10000, need, None, None) == tclora.EINVAL
    # null arrays
    c0 = tclora.Composites(3, 2, 3, 4, 4, None, 0x1000, 0x1000, 0x1000)
    assert L.tcl_plan_map(ctypes.byref(c0), 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    c1 = tclora.Composites(3, 2, 3, 4, 4, 0x1000, 0x1000, None, 0x1000)
    assert L.tcl_plan_map(ctypes.byref(c1), 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    # sizes
    cbad = _comp(N=0)
    assert L.tcl_plan_map(ctypes.byref(cbad), 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    # buffer
    assert L.tcl_plan_map(ctypes.byref(c), None, need, None, ctypes.byref(h)) == tclora.EINVAL
    assert L.tcl_plan_map(ctypes.byref(c), 0x10010, need, None, ctypes.byref(h)) == tclora.EALIGN
    assert L.tcl_plan_map(ctypes.byref(c), 0x10000, need - 1, None, ctypes.byref(h)) == tclora.ENOSPC
    assert b"needs" in L.tcl_last_error()
    assert h.value is None


def test_null_plan_rejected(L):
    m = tclora.ModuleDesc(4, 16, 16, 4, tclora.BF16, 0x1000, 0x2000, None)
    out = ctypes.c_size_t(0)
    assert L.tcl_workspace_bytes(None, ctypes.byref(m), 1, ctypes.byref(out)) == tclora.EINVAL
    assert L.tcl_shrink(None, ctypes.byref(m), 0x1000, 16, 0, 0x1000, None) == tclora.EINVAL
    assert L.tcl_expand(None, ctypes.byref(m), 0x1000, 0x1000, 16, 1, None) == tclora.EINVAL
    assert L.tcl_plan_status(None, None, None, None) == tclora.EINVAL
    c = tclora.Composites(4, 4, 4, 4, 4, 0x1000, 0x2000, 0x3000, 0x4000)
    ptrs = (ctypes.c_void_p * 1)(0x1000)
    lds = (ctypes.c_int64 * 1)(16)
    assert L.tcl_remap_apply(None, ctypes.byref(c), ctypes.byref(m), 1, ptrs, lds, 0, ptrs,
                             lds, 1, 0x1000, 1 << 20, None) == tclora.EINVAL
    assert L.tcl_remap_shrink(None, ctypes.byref(c), ctypes.byref(m), 1, ptrs, lds, 0, 0x1000,
                              1 << 20, None) == tclora.EINVAL
    assert L.tcl_plan_copy_out(None, *([None] * 9)) == tclora.EINVAL
    L.tcl_plan_free(None)


def test_load_ranks_host_errors(L):
    m = tclora.ModuleDesc(4, 16, 16, 8, tclora.BF16, 0x1000, 0x2000, None)
    k = np.array([0, 8, 9, 1], np.int32)          # 9 > r_max
    rc = L.tcl_module_load_ranks(ctypes.byref(m), k.ctypes.data_as(ctypes.c_void_p), 0x3000,
                                 None)
    assert rc == tclora.EINVAL and b"k[2]" in L.tcl_last_error()
    k = np.array([0, -1, 2, 1], np.int32)
    rc = L.tcl_module_load_ranks(ctypes.byref(m), k.ctypes.data_as(ctypes.c_void_p), 0x3000,
                                 None)
    assert rc == tclora.EINVAL
    assert L.tcl_module_load_ranks(ctypes.byref(m), None, 0x3000, None) == tclora.EINVAL


def test_gate_host_errors(L):
    """tcl_gate_topk rejects bad sizes and pointers on the host (no GPU)."""
    P = 0x1000

    def call(T=4, C=8, k=2, ldl=8, ldc=8, lg=P, cd=P, out=P):
        return L.tcl_gate_topk(lg, ldl, cd, ldc, T, C, k, out, out, out, out, None)

    assert call(T=-1) == tclora.EINVAL
    assert call(C=0) == tclora.EINVAL
    assert call(C=65, ldl=65, ldc=65) == tclora.EINVAL
    assert call(k=0) == tclora.EINVAL
    assert call(k=9) == tclora.EINVAL              # k > n_candidates
    assert call(ldl=7) == tclora.EINVAL
    assert call(ldc=7) == tclora.EINVAL
    assert call(lg=None) == tclora.EINVAL
    assert call(cd=None) == tclora.EINVAL
    assert call(out=None) == tclora.EINVAL
    assert call(T=1 << 30, k=4, C=8) == tclora.EINVAL  # T * k beyond 32-bit indexing
    assert call(lg=P + 2) == tclora.EALIGN
    assert b"gate" in L.tcl_last_error()
