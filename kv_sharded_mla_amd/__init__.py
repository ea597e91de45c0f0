"""MI355X-native decode-context-parallel absorbed-MLA hot path.

The work happens in ``libdcpmla.so`` (HIP kernels for gfx950 behind the C ABI
of include/dcp_mla.h).  This package is its thin Python binding: the
functions below carry the C entry points' names and only marshal torch
tensors (device memory) and the current HIP stream.
"""
from ._binding import (  # noqa: F401
    D_QK, D_V, DEV_BAD_LENGTH, DEV_BAD_PAGE, DEV_DECODE_STALLED, DEV_OK, DEV_OUT_OF_PAGES, DEV_TABLE_OVERFLOW, KV_BF16, KV_FP8_E4M3,
    LIB_PATH, LSE_BASE_2, LSE_BASE_E, MAX_Q_LEN, DcpError, Layout, dcp_alloc_virtual, dcp_kv_read, dcp_kv_relayout,
    dcp_kv_write, dcp_lse_merge,
    dcp_pool_bytes, dcp_status_string, load_library, make_layout, mla_decode_noalloc_scratch_bytes, mla_decode_partial,
    mla_decode_partial_noalloc, mla_decode_workspace_size)


def build(verbose: bool = False) -> str:
    """Compile the HIP library for gfx950 (always recompiles)."""
    from .build import build as _build
    return _build(verbose=verbose)
