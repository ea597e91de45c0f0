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
    assert "partner" in dcp_status_string(5)
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
    # every call needs its workspace (the work plan lives there, or at least a
    # token buffer when no request can be split): none given
    assert call(maxl=1 << 20, B=1) == -4
    assert call() == -4
    assert call(ws=256, wsb=255) == -4
    # kv write / alloc
    assert lib.dcp_kv_write(ref, 16, None, 16, 4, 16, 16, 1, 4, 8, None, None, None, None) == -3
    assert lib.dcp_kv_write(ctypes.byref(_layout(kv=1)), 16, None, 16, 4, 16, 16, 1, 4, 16, None, None, None,
                            None) == -1
    assert lib.dcp_alloc_virtual(ref, 16, None, 16, 16, 1, 16, 4, None, None) == -1
    assert lib.dcp_alloc_virtual(ref, 16, 16, 16, 16, -1, 16, 4, None, None) == -1


def test_workspace_size_covers_the_work_plan(lib):
    from kv_sharded_mla_amd import mla_decode_workspace_size
    # with at most 256 tokens per rank no (rank, request) is split: one launch, no work
    # plan, and a token size that does not grow with the batch
    for B in (1, 64, 4096):
        for maxl in (1, 1000, 8 * 256):
            assert mla_decode_workspace_size(_layout(8, 64, 100, 0), 8, B, 4, 128, maxl) == 256
    assert mla_decode_workspace_size(_layout(8, 64, 100, 0), 8, 64, 4, 128, 8 * 256 + 1) > 256
    # longer calls plan their work items in the workspace; it holds at least one
    # partial (512 outputs + lse, fp32) per unit and row
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


def test_binding_rejects_short_buffers(lib):
    """The Python binding checks buffer sizes before any pointer reaches a kernel: a
    flattened payload, a short slot or scale array, or a block table with fewer rows
    than requests is a ValueError (CPU tensors: the size check comes first)."""
    import torch
    import kv_sharded_mla_amd as K
    lay = _layout(2, 16, 4, K.KV_BF16)
    lay8 = _layout(2, 16, 4, K.KV_FP8_E4M3)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    bt, sl, cu = i32(3, 2), i32(3), i32(4)
    rows = torch.zeros(5, 1152, dtype=torch.uint8)
    # rows flattened to 1-D bytes: the row count would be the byte count
    with pytest.raises(ValueError, match="rows"):
        K.dcp_kv_write(lay, None, None, bt, sl, cu, rows.reshape(-1), None, torch.zeros(5 * 1152, dtype=torch.int64))
    with pytest.raises(ValueError, match="rows"):
        K.dcp_kv_write(lay8, None, None, bt, sl, cu, rows)                   # 1152-byte rows for e4m3
    with pytest.raises(ValueError, match="slot_out"):
        K.dcp_kv_write(lay, None, None, bt, sl, cu, rows, None, torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError, match="row_scales"):
        K.dcp_kv_write(lay8, None, None, bt, sl, cu, torch.zeros(5, 576, dtype=torch.uint8), torch.zeros(4))
    with pytest.raises(ValueError, match="block_table"):
        K.dcp_kv_write(lay, None, None, i32(2, 2), sl, cu, rows)
    with pytest.raises(ValueError, match="cu_new"):
        K.dcp_kv_write(lay, None, None, bt, sl, i32(3), rows)
    with pytest.raises(ValueError, match="block_table"):
        K.dcp_alloc_virtual(lay, i32(4), i32(1), sl, sl, i32(2, 2))
    with pytest.raises(ValueError, match="new_len"):
        K.dcp_alloc_virtual(lay, i32(4), i32(1), sl, i32(2), bt)
    with pytest.raises(ValueError, match="rows_out"):
        K.dcp_kv_read(lay, None, None, bt, sl, cu, torch.zeros(7, 100, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales_out"):
        K.dcp_kv_read(lay8, None, None, bt, sl, cu, torch.zeros(7, 576, dtype=torch.uint8), torch.zeros(6))
    # decode: pools shorter than rank_count pools, missing e4m3 scales, short table
    q = torch.zeros(3, 1, 16, 576, dtype=torch.bfloat16)
    pb = K.dcp_pool_bytes(lay)
    o = torch.zeros(2 * 3 * 16 * 512)
    lse = torch.zeros(2 * 3 * 16)
    with pytest.raises(ValueError, match="pools"):
        K.mla_decode_partial(lay, torch.zeros(pb, dtype=torch.uint8), None, 0, 2, q, bt, sl, 64, 0.1, 0, True, o, lse)
    with pytest.raises(ValueError, match="pool_scales"):
        K.mla_decode_partial(lay8, torch.zeros(2 * K.dcp_pool_bytes(lay8), dtype=torch.uint8), torch.zeros(64), 0, 2,
                             q, bt, sl, 64, 0.1, 0, True, o, lse)
    with pytest.raises(ValueError, match="block_table"):
        K.mla_decode_partial(lay, torch.zeros(2 * pb, dtype=torch.uint8), None, 0, 2, q, i32(2, 2), sl, 64, 0.1, 0,
                             True, o, lse)
    with pytest.raises(ValueError, match="ranks"):
        K.mla_decode_partial(lay, torch.zeros(2 * pb, dtype=torch.uint8), None, 1, 2, q, bt, sl, 64, 0.1, 0, True, o,
                             lse)
    with pytest.raises(ValueError, match="pools"):
        K.dcp_kv_relayout(lay, torch.zeros(16 * 1152, dtype=torch.uint8), None, i32(3, 2), sl, 0, 2,
                          torch.zeros(pb, dtype=torch.uint8), None, bt)
