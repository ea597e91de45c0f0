"""ctypes binding of libdcpmla.so: argument marshalling only.

Every function here has the name of a C entry point in include/dcp_mla.h,
checks that the torch tensors it is handed have the dtype, device and
contiguity that entry point expects, and passes their device pointers and the
current HIP stream through.  All computation happens in the HIP kernels; if
the shared library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdcpmla.so")

KV_BF16 = 0
KV_FP8_E4M3 = 1
LSE_BASE_E = 0
LSE_BASE_2 = 1
D_QK = 576
D_V = 512
MAX_Q_LEN = 8

DEV_OK = 0
DEV_OUT_OF_PAGES = 1
DEV_BAD_LENGTH = 2
DEV_TABLE_OVERFLOW = 3
DEV_BAD_PAGE = 4
DEV_DECODE_STALLED = 5


class DcpError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status} ({text})")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("c", ctypes.c_int32), ("page", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("interleave", ctypes.c_int32)]

    def __repr__(self):
        return (f"Layout(c={self.c}, page={self.page}, num_pages={self.num_pages}, kv_dtype={self.kv_dtype}, "
                f"interleave={self.interleave})")


_lib = None
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PL = ctypes.POINTER(Layout)

_SIGS = {
    "dcp_pool_bytes": (_I64, [_PL]),
    "dcp_alloc_virtual": (ctypes.c_int, [_PL, _VP, _VP, _VP, _VP, _I32, _VP, _I32, _VP, _VP]),
    "dcp_kv_write": (ctypes.c_int, [_PL, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I64, _VP, _VP, _VP, _VP, _VP]),
    "dcp_kv_read": (ctypes.c_int, [_PL, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I64, _VP, _VP, _VP, _VP]),
    "dcp_kv_relayout": (ctypes.c_int, [_PL, _VP, _VP, _I32, _VP, _I32, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _I32,
                                       _VP, _VP]),
    "mla_decode_workspace_size": (ctypes.c_size_t, [_PL, _I32, _I32, _I32, _I32, _I64]),
    "mla_decode_partial": (ctypes.c_int, [_PL, _VP, _VP, _I32, _I32, _VP, _I32, _I32, _I32, _VP, _I32, _VP,
                                          _I64, ctypes.c_float, _I32, _I32, _VP, _VP, _VP, ctypes.c_size_t,
                                          _VP, _VP]),
    "mla_decode_partial_noalloc": (ctypes.c_int, [_PL, _VP, _VP, _I32, _I32, _VP, _I32, _I32, _I32, _VP, _I32,
                                                  _VP, _I64, ctypes.c_float, _I32, _I32, _VP, _VP, _VP, _VP]),
    "mla_decode_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "dcp_lse_merge": (ctypes.c_int, [_I32, _I64, _VP, _VP, _I32, _VP, _VP, _VP]),
    "dcp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


def load_library(path: str = LIB_PATH):
    """Load (once) and return the shared library; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first (python -m kv_sharded_mla_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def dcp_status_string(status: int) -> str:
    return load_library().dcp_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise DcpError(fn, status, dcp_status_string(status))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel=None) -> int:
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return int(t.data_ptr())


def _bytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _need(cond: bool, msg: str):
    """Size check before any pointer leaves Python: a short buffer would let a kernel
    write past its end."""
    if not cond:
        raise ValueError(msg)


def _row_bytes(layout: Layout) -> int:
    return D_QK if layout.kv_dtype == KV_FP8_E4M3 else 2 * D_QK


def _rows_of(t: torch.Tensor, layout: Layout, name: str) -> int:
    """Number of latent rows in a [n][576] payload tensor (any element type)."""
    if t.dim() < 1:
        raise ValueError(f"{name} must be [n_rows][...]")
    n = t.shape[0]
    _need(_bytes(t) == n * _row_bytes(layout), f"{name} must hold {n} rows of {_row_bytes(layout)} bytes")
    return n


def _table_rows(block_table: torch.Tensor, batch: int, name: str = "block_table"):
    _need(block_table.dim() == 2 and block_table.shape[0] >= batch, f"{name} must be [>= {batch}][stride]")


def _pool_check(layout: Layout, pools, pool_scales, ranks: int):
    pb = dcp_pool_bytes(layout)
    _need(_bytes(pools) >= ranks * pb, f"pools must hold {ranks} pools of {pb} bytes")
    if layout.kv_dtype == KV_FP8_E4M3:
        cap = layout.num_pages * layout.page
        _need(pool_scales is not None and pool_scales.numel() >= ranks * cap,
              f"pool_scales must hold {ranks} x {cap} scales")


def make_layout(c: int, page: int, num_pages: int, kv_dtype: int = KV_BF16, interleave: int = 1) -> Layout:
    return Layout(int(c), int(page), int(num_pages), int(kv_dtype), int(interleave))


def dcp_pool_bytes(layout: Layout) -> int:
    return int(load_library().dcp_pool_bytes(ctypes.byref(layout)))


def dcp_alloc_virtual(layout: Layout, free_stack, free_top, old_len, new_len, block_table,
                      dev_status=None, stream=None):
    B = old_len.numel()
    _need(new_len.numel() >= B, "new_len must hold one length per request")
    _table_rows(block_table, B)
    lib = load_library()
    st = lib.dcp_alloc_virtual(
        ctypes.byref(layout), _ptr(free_stack, "free_stack", torch.int32), _ptr(free_top, "free_top", torch.int32, 1),
        _ptr(old_len, "old_len", torch.int32), _ptr(new_len, "new_len", torch.int32, B), B,
        _ptr(block_table, "block_table", torch.int32), block_table.shape[-1],
        _ptr(dev_status, "dev_status", torch.int32, 1), _stream(stream))
    _check("dcp_alloc_virtual", st)


def dcp_kv_write(layout: Layout, pools, pool_scales, block_table, seq_len, cu_new, rows, row_scales=None,
                 slot_out=None, dev_status=None, stream=None):
    B = seq_len.numel()
    n_rows = _rows_of(rows, layout, "rows")
    _table_rows(block_table, B)
    _need(cu_new.numel() >= B + 1, "cu_new must hold batch + 1 offsets")
    _need(row_scales is None or row_scales.numel() >= n_rows, "row_scales must hold one scale per row")
    _need(slot_out is None or slot_out.numel() >= n_rows, "slot_out must hold one slot per row")
    lib = load_library()
    st = lib.dcp_kv_write(
        ctypes.byref(layout), _ptr(pools, "pools", (torch.uint8, torch.int16, torch.bfloat16)),
        _ptr(pool_scales, "pool_scales", torch.float32), _ptr(block_table, "block_table", torch.int32),
        block_table.shape[-1], _ptr(seq_len, "seq_len", torch.int32), _ptr(cu_new, "cu_new", torch.int32, B + 1),
        B, n_rows, _ptr(rows, "rows", (torch.uint8, torch.int16, torch.bfloat16)),
        _ptr(row_scales, "row_scales", torch.float32), _ptr(slot_out, "slot_out", torch.int64),
        _ptr(dev_status, "dev_status", torch.int32, 1), _stream(stream))
    _check("dcp_kv_write", st)


def dcp_kv_read(layout: Layout, pools, pool_scales, block_table, seq_len, cu_out, rows_out, scales_out=None,
                dev_status=None, stream=None):
    """Gather positions 0 .. seq_len[b]-1 of every request into rows_out[cu_out[b] + p] (token order)."""
    B = seq_len.numel()
    payload = (torch.uint8, torch.int16, torch.bfloat16)
    n_rows = _rows_of(rows_out, layout, "rows_out")
    _table_rows(block_table, B)
    _need(cu_out.numel() >= B + 1, "cu_out must hold batch + 1 offsets")
    _need(scales_out is None or scales_out.numel() >= n_rows, "scales_out must hold one scale per row")
    st = load_library().dcp_kv_read(
        ctypes.byref(layout), _ptr(pools, "pools", payload), _ptr(pool_scales, "pool_scales", torch.float32),
        _ptr(block_table, "block_table", torch.int32), block_table.shape[-1], _ptr(seq_len, "seq_len", torch.int32),
        _ptr(cu_out, "cu_out", torch.int32, B + 1), B, n_rows, _ptr(rows_out, "rows_out", payload),
        _ptr(scales_out, "scales_out", torch.float32), _ptr(dev_status, "dev_status", torch.int32, 1),
        _stream(stream))
    _check("dcp_kv_read", st)


def dcp_kv_relayout(layout: Layout, src_pool, src_scales, src_block_table, seq_len, rank_begin: int,
                    rank_count: int, pools, pool_scales, block_table, dev_status=None, stream=None):
    """Copy the rows of ranks [rank_begin, rank_begin + rank_count) from a dense paged pool
    (pages of layout.page tokens) into their owner pools (those ranks' pools, back to back)."""
    B = seq_len.numel()
    payload = (torch.uint8, torch.int16, torch.bfloat16)
    row_bytes = _row_bytes(layout)
    src_pages = src_pool.numel() * src_pool.element_size() // (row_bytes * layout.page)
    _need(0 <= rank_begin and rank_count >= 1 and rank_begin + rank_count <= layout.c, "ranks outside the group")
    _pool_check(layout, pools, pool_scales, rank_count)
    _table_rows(block_table, B)
    _table_rows(src_block_table, B, "src_block_table")
    _need(src_scales is None or src_scales.numel() >= src_pages * layout.page,
          "src_scales must hold one scale per source slot")
    st = load_library().dcp_kv_relayout(
        ctypes.byref(layout), _ptr(src_pool, "src_pool", payload), _ptr(src_scales, "src_scales", torch.float32),
        src_pages, _ptr(src_block_table, "src_block_table", torch.int32), src_block_table.shape[-1],
        _ptr(seq_len, "seq_len", torch.int32), B, int(rank_begin), int(rank_count), _ptr(pools, "pools", payload),
        _ptr(pool_scales, "pool_scales", torch.float32), _ptr(block_table, "block_table", torch.int32),
        block_table.shape[-1], _ptr(dev_status, "dev_status", torch.int32, 1), _stream(stream))
    _check("dcp_kv_relayout", st)


def mla_decode_workspace_size(layout: Layout, rank_count: int, batch: int, q_len: int, heads: int,
                              max_seq_len: int) -> int:
    return int(load_library().mla_decode_workspace_size(ctypes.byref(layout), rank_count, batch, q_len, heads,
                                                        int(max_seq_len)))


def mla_decode_partial(layout: Layout, pools, pool_scales, rank_begin: int, rank_count: int, q, block_table,
                       seq_len, max_seq_len: int, sm_scale: float, lse_base: int, causal: bool, o_part, lse_part,
                       workspace=None, dev_status=None, stream=None):
    """q: bf16 (or int16 payload) [batch][q_len][heads][576]."""
    batch, q_len, heads, d = q.shape
    if d != D_QK:
        raise ValueError("q must be [batch][q_len][heads][576]")
    rows = batch * q_len * heads
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _need(0 <= rank_begin and rank_count >= 1 and rank_begin + rank_count <= layout.c, "ranks outside the group")
    _pool_check(layout, pools, pool_scales, rank_count)
    _table_rows(block_table, batch)
    lib = load_library()
    st = lib.mla_decode_partial(
        ctypes.byref(layout), _ptr(pools, "pools", (torch.uint8, torch.int16, torch.bfloat16)),
        _ptr(pool_scales, "pool_scales", torch.float32), rank_begin, rank_count,
        _ptr(q, "q", (torch.bfloat16, torch.int16)), batch, q_len, heads,
        _ptr(block_table, "block_table", torch.int32), block_table.shape[-1],
        _ptr(seq_len, "seq_len", torch.int32, batch), int(max_seq_len), float(sm_scale), int(lse_base),
        1 if causal else 0, _ptr(o_part, "o_part", torch.float32, rank_count * rows * D_V),
        _ptr(lse_part, "lse_part", torch.float32, rank_count * rows), _ptr(workspace, "workspace"), ws_bytes,
        _ptr(dev_status, "dev_status", torch.int32, 1), _stream(stream))
    _check("mla_decode_partial", st)


def mla_decode_partial_noalloc(layout: Layout, pools, pool_scales, rank_begin: int, rank_count: int, q,
                               block_table, seq_len, max_seq_len: int, sm_scale: float, lse_base: int, causal: bool,
                               o_part, lse_part, dev_status=None, stream=None):
    """mla_decode_partial with the library's own scratch in place of a workspace."""
    batch, q_len, heads, d = q.shape
    if d != D_QK:
        raise ValueError("q must be [batch][q_len][heads][576]")
    rows = batch * q_len * heads
    _need(0 <= rank_begin and rank_count >= 1 and rank_begin + rank_count <= layout.c, "ranks outside the group")
    _pool_check(layout, pools, pool_scales, rank_count)
    _table_rows(block_table, batch)
    st = load_library().mla_decode_partial_noalloc(
        ctypes.byref(layout), _ptr(pools, "pools", (torch.uint8, torch.int16, torch.bfloat16)),
        _ptr(pool_scales, "pool_scales", torch.float32), rank_begin, rank_count,
        _ptr(q, "q", (torch.bfloat16, torch.int16)), batch, q_len, heads,
        _ptr(block_table, "block_table", torch.int32), block_table.shape[-1],
        _ptr(seq_len, "seq_len", torch.int32, batch), int(max_seq_len), float(sm_scale), int(lse_base),
        1 if causal else 0, _ptr(o_part, "o_part", torch.float32, rank_count * rows * D_V),
        _ptr(lse_part, "lse_part", torch.float32, rank_count * rows), _ptr(dev_status, "dev_status", torch.int32, 1),
        _stream(stream))
    _check("mla_decode_partial_noalloc", st)


def mla_decode_noalloc_scratch_bytes() -> int:
    return int(load_library().mla_decode_noalloc_scratch_bytes())


def dcp_lse_merge(c: int, o_part, lse_part, lse_base: int, o_out, lse_out, stream=None):
    rows = lse_out.numel()
    lib = load_library()
    st = lib.dcp_lse_merge(
        int(c), rows, _ptr(o_part, "o_part", torch.float32, c * rows * D_V),
        _ptr(lse_part, "lse_part", torch.float32, c * rows), int(lse_base),
        _ptr(o_out, "o_out", (torch.bfloat16, torch.int16), rows * D_V), _ptr(lse_out, "lse_out", torch.float32),
        _stream(stream))
    _check("dcp_lse_merge", st)
