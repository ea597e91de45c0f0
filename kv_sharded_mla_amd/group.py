"""An emulated DCP group on one GPU: c owner pools back to back in HBM.

Holds the device buffers one layer of a DCP group needs (pools, shared block
table, free stack, lengths) and drives the C entry points in the order a
decode step uses them: allocate virtual pages, scatter the new rows into
their owner pools, attend every rank's shard, merge the partials.  Buffer
management only; every step runs in the HIP library.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import _binding as B


class DcpGroup:
    def __init__(self, c: int, page: int, num_pages: int, kv_dtype: int, batch: int, bt_stride: int,
                 free_stack: Optional[np.ndarray] = None, device: str = "cuda", sentinel: Optional[int] = None,
                 interleave: int = 1):
        self.layout = B.make_layout(c, page, num_pages, kv_dtype, interleave)
        self.interleave = interleave
        self.c, self.page, self.num_pages, self.batch = c, page, num_pages, batch
        self.fp8 = kv_dtype == B.KV_FP8_E4M3
        self.device = torch.device(device)
        self.row_bytes = B.D_QK if self.fp8 else 2 * B.D_QK
        pool_bytes = B.dcp_pool_bytes(self.layout)
        if sentinel is None:
            self.pools = torch.empty(c * pool_bytes, dtype=torch.uint8, device=self.device)
        else:
            self.pools = torch.full((c * pool_bytes,), sentinel, dtype=torch.uint8, device=self.device)
        self.pool_scales = (torch.full((c * num_pages * page,), float("nan") if sentinel is not None else 0.0,
                                       dtype=torch.float32, device=self.device) if self.fp8 else None)
        self.block_table = torch.full((batch, bt_stride), -1, dtype=torch.int32, device=self.device)
        fs = np.arange(num_pages, dtype=np.int32) if free_stack is None else np.asarray(free_stack, np.int32)
        self.free_stack = torch.from_numpy(fs.copy()).to(self.device)
        self.free_top = torch.tensor([num_pages], dtype=torch.int32, device=self.device)
        self.seq_len = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.max_seq_len = 0

    # ---- cache growth -------------------------------------------------
    def append(self, counts: Sequence[int], rows: torch.Tensor, row_scales: Optional[torch.Tensor] = None,
               slot_out: Optional[torch.Tensor] = None):
        """Append counts[b] new latent rows to request b (rows in request order)."""
        counts = np.asarray(counts, dtype=np.int64)
        cu = np.zeros(self.batch + 1, dtype=np.int64)
        cu[1:] = np.cumsum(counts)
        new_len = self.seq_len + torch.from_numpy(counts.astype(np.int32)).to(self.device)
        B.dcp_alloc_virtual(self.layout, self.free_stack, self.free_top, self.seq_len, new_len, self.block_table,
                            self.dev_status)
        cu_t = torch.from_numpy(cu.astype(np.int32)).to(self.device)
        B.dcp_kv_write(self.layout, self.pools, self.pool_scales, self.block_table, new_len, cu_t, rows, row_scales,
                       slot_out, self.dev_status)
        self.seq_len = new_len
        self.max_seq_len = max(self.max_seq_len, int(new_len.max().item()) if self.batch else 0)

    def status(self) -> int:
        return int(self.dev_status.item())

    # ---- attention ----------------------------------------------------
    def workspace_for(self, q_len: int, heads: int, rank_count: Optional[int] = None) -> Optional[torch.Tensor]:
        n = B.mla_decode_workspace_size(self.layout, rank_count or self.c, self.batch, q_len, heads,
                                        self.max_seq_len)
        if n == 0:
            return None
        return torch.empty((n + 15) // 16 * 4, dtype=torch.float32, device=self.device)

    def decode(self, q: torch.Tensor, sm_scale: float, lse_base: int, causal: bool = True,
               rank_begin: int = 0, rank_count: Optional[int] = None, workspace=None, out=None):
        """Per-rank partials: o_part [ranks][B][q_len][H][512] fp32, lse_part [ranks][B][q_len][H]."""
        rc = self.c if rank_count is None else rank_count
        batch, q_len, heads, _ = q.shape
        if out is None:
            o_part = torch.empty((rc, batch, q_len, heads, B.D_V), dtype=torch.float32, device=self.device)
            lse_part = torch.empty((rc, batch, q_len, heads), dtype=torch.float32, device=self.device)
        else:
            o_part, lse_part = out
        if workspace is None:
            workspace = self.workspace_for(q_len, heads, rc)
        pools = self.pools[rank_begin * B.dcp_pool_bytes(self.layout):]
        scales = None
        if self.fp8:
            scales = self.pool_scales[rank_begin * self.num_pages * self.page:]
        B.mla_decode_partial(self.layout, pools, scales, rank_begin, rc, q, self.block_table, self.seq_len,
                             self.max_seq_len, sm_scale, lse_base, causal, o_part, lse_part, workspace,
                             self.dev_status)
        return o_part, lse_part

    @staticmethod
    def merge(o_part: torch.Tensor, lse_part: torch.Tensor, lse_base: int, out=None):
        """Exact merge over the leading rank axis: o bf16 [...][512], lse fp32 [...]."""
        c = o_part.shape[0]
        if out is None:
            o = torch.empty(o_part.shape[1:], dtype=torch.bfloat16, device=o_part.device)
            lse = torch.empty(lse_part.shape[1:], dtype=torch.float32, device=o_part.device)
        else:
            o, lse = out
        B.dcp_lse_merge(c, o_part, lse_part, lse_base, o, lse)
        return o, lse
