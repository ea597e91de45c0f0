"""Host-side checks of the C ABI (CPU only, no kernel launches).

The shared library must load, export every function that include/dcp_mla.h
declares, and reject bad arguments on the host with the documented negative
status before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcp_mla.h")


@pytest.fixture(scope="module")
def lib():
    from kv_sharded_mla_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from kv_sharded_mla_amd.build import build
        build()
    return _binding.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b((?:dcp|mla)_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"dcp_alloc_virtual", "dcp_kv_write", "mla_decode_partial", "dcp_lse_merge",
            "mla_decode_workspace_size", "dcp_status_string", "dcp_pool_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    from kv_sharded_mla_amd import dcp_status_string
    assert dcp_status_string(0) == "ok"
    assert "out of pages" in dcp_status_string(1)
    assert "aligned" in dcp_status_string(-3)
    assert dcp_status_string(12345) == "unknown status"


def _layout(c=4, page=16, num_pages=10, kv=0, interleave=1):
    from kv_sharded_mla_amd import make_layout
    return make_layout(c, page, num_pages, kv, interleave)


def test_pool_bytes(lib):
    from kv_sharded_mla_amd import dcp_pool_bytes
    assert dcp_pool_bytes(_layout(4, 16, 10, 0)) == 10 * 16 * 1152
    assert dcp_pool_bytes(_layout(4, 16, 10, 1)) == 10 * 16 * 576
    assert dcp_pool_bytes(_layout(0, 16, 10, 0)) == -1
    assert dcp_pool_bytes(_layout(4, 16, 10, 7)) == -1
    # interleave size: a divisor of the page size; 0 reads as 1
    assert dcp_pool_bytes(_layout(4, 16, 10, 0, 8)) == 10 * 16 * 1152
    assert dcp_pool_bytes(_layout(4, 16, 10, 0, 16)) == 10 * 16 * 1152
    assert dcp_pool_bytes(_layout(4, 16, 10, 0, 0)) == 10 * 16 * 1152
    assert dcp_pool_bytes(_layout(4, 16, 10, 0, 3)) == -1
    assert dcp_pool_bytes(_layout(4, 16, 10, 0, 32)) == -1
    assert dcp_pool_bytes(_layout(4, 16, 10, 0, -2)) == -1


def test_host_argument_errors(lib):
    L = _layout()
    ref = ctypes.byref(L)
    # merge: bad c, bad base, null pointers, misalignment
    assert lib.dcp_lse_merge(0, 4, 16, 16, 0, 16, 16, None) == -1
    assert lib.dcp_lse_merge(2, 4, 16, 16, 5, 16, 16, None) == -1
    assert lib.dcp_lse_merge(2, 4, None, 16, 0, 16, 16, None) == -1
    assert lib.dcp_lse_merge(2, 4, 8, 16, 0, 16, 16, None) == -3
    assert lib.dcp_lse_merge(2, 0, None, None, 0, None, None, None) == 0   # nothing to do
    # decode: unsupported heads / q_len, bad rank range, missing workspace
    args = dict(pools=16, scales=None, rb=0, rc=4, q=16, B=1, q_len=1, H=16, bt=16, bts=4, sl=16, maxl=64,
                scale=0.1, base=0, causal=1, o=16, lse=16, ws=None, wsb=0, st=None, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.mla_decode_partial(ref, a["pools"], a["scales"], a["rb"], a["rc"], a["q"], a["B"], a["q_len"],
                                      a["H"], a["bt"], a["bts"], a["sl"], a["maxl"], a["scale"], a["base"],
                                      a["causal"], a["o"], a["lse"], a["ws"], a["wsb"], a["st"], a["stream"])
    assert call(H=24) == -2
    assert call(q_len=9) == -2
    assert call(rb=2, rc=3) == -1
    assert call(scale=float("inf")) == -1
    assert call(q=8) == -3
    assert call(base=3) == -1
    assert call(maxl=2**31) == -2
    assert call(B=0) == 0
    # every call needs its workspace (the work plan lives there): none given
    assert call(maxl=1 << 20, B=1) == -4
    assert call() == -4
    # kv write / alloc
    assert lib.dcp_kv_write(ref, 16, None, 16, 4, 16, 16, 1, 4, 8, None, None, None, None) == -3
    assert lib.dcp_kv_write(ctypes.byref(_layout(kv=1)), 16, None, 16, 4, 16, 16, 1, 4, 16, None, None, None,
                            None) == -1
    assert lib.dcp_alloc_virtual(ref, 16, None, 16, 16, 1, 16, 4, None, None) == -1
    assert lib.dcp_alloc_virtual(ref, 16, 16, 16, 16, -1, 16, 4, None, None) == -1


def test_workspace_size_covers_the_work_plan(lib):
    from kv_sharded_mla_amd import mla_decode_workspace_size
    # every call plans its work items in the workspace, so the size is never 0 for valid
    # arguments; it holds at least one partial (512 outputs + lse, fp32) per unit and row
    units, rows = 8 * 64, 16
    n = mla_decode_workspace_size(_layout(8, 64, 100, 0), 8, 64, 1, 16, 32768)
    assert n >= units * rows * 513 * 4
    # a longer context can only need more items
    assert mla_decode_workspace_size(_layout(8, 64, 100, 0), 8, 64, 1, 16, 1 << 20) >= n
    # small pages bound an item's length (its page ids fit the LDS table), so more items
    assert mla_decode_workspace_size(_layout(8, 1, 100, 0), 8, 64, 1, 16, 1 << 20) > \
        mla_decode_workspace_size(_layout(8, 64, 100, 0), 8, 64, 1, 16, 1 << 20)
    assert mla_decode_workspace_size(_layout(8, 64, 100, 0), 8, 4, 9, 64, 1000) == 0  # invalid -> 0
    # runs of I positions per owner can only raise one rank's share of a request
    for L in (100, 1000, 1 << 20):
        assert mla_decode_workspace_size(_layout(8, 64, 100, 0, 64), 8, 64, 1, 16, L) >= \
            mla_decode_workspace_size(_layout(8, 64, 100, 0), 8, 64, 1, 16, L)
    assert mla_decode_workspace_size(_layout(8, 64, 100, 0, 48), 8, 64, 1, 16, 1000) == 0


def test_layout_copy_argument_errors(lib):
    """dcp_kv_read / dcp_kv_relayout reject bad arguments on the host (nothing enqueued)."""
    L = _layout()
    ref = ctypes.byref(L)

    def read(**kw):
        a = dict(pools=16, ps=None, bt=16, bts=4, sl=16, cu=16, B=2, n=8, out=16, osc=None, st=None, stream=None)
        a.update(kw)
        return lib.dcp_kv_read(ref if "lay" not in kw else kw["lay"], a["pools"], a["ps"], a["bt"], a["bts"], a["sl"],
                               a["cu"], a["B"], a["n"], a["out"], a["osc"], a["st"], a["stream"])
    assert read(B=0) == 0                      # nothing to do
    assert read(B=-1) == -1 and read(B=65537) == -1 and read(n=-1) == -1 and read(bts=0) == -1
    assert read(pools=None) == -1 and read(cu=None) == -1 and read(out=None) == -1
    assert read(out=8) == -3                   # rows_out not 16-byte aligned
    assert read(lay=ctypes.byref(_layout(kv=1))) == -1          # e4m3 needs the scale arrays
    assert read(lay=ctypes.byref(_layout(c=1 << 16, page=1 << 15, num_pages=1))) == -2   # page * c > 2^30

    def relayout(**kw):
        a = dict(src=16, ssc=None, snp=4, sbt=16, sbts=4, sl=16, B=2, rb=0, rc=4, pools=16, ps=None, bt=16, bts=4,
                 st=None, stream=None)
        a.update(kw)
        return lib.dcp_kv_relayout(ref, a["src"], a["ssc"], a["snp"], a["sbt"], a["sbts"], a["sl"], a["B"], a["rb"],
                                   a["rc"], a["pools"], a["ps"], a["bt"], a["bts"], a["st"], a["stream"])
    assert relayout(B=0) == 0
    assert relayout(rb=-1) == -1 and relayout(rc=0) == -1 and relayout(rb=2, rc=3) == -1   # ranks within [0, c)
    assert relayout(snp=-1) == -1 and relayout(sbts=0) == -1 and relayout(bts=0) == -1
    assert relayout(src=None) == -1 and relayout(sbt=None) == -1 and relayout(pools=None) == -1
    assert relayout(src=8) == -3 and relayout(pools=24) == -3
