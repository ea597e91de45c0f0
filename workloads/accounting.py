"""Algorithmic bytes and FLOPs of one DCP MLA-decode layer-step.

The counting rules follow the vLLM GLM-5.3 blog post (section "Why the
numbers add up"): each (KV row, query head) pair costs 2*576 FLOPs for QK and
2*512 for PV, 2176 in all, softmax not counted; bf16 query and output add
2*576 + 2*512 = 2176 bytes per head; each KV row is read once for all heads.
Those footnote figures are reproduced in the tests to pin these functions.
"""
from __future__ import annotations

import numpy as np

from .configs import D_QK, D_V, Workload


def flops_per_score(d_qk: int = D_QK, d_v: int = D_V) -> int:
    return 2 * d_qk + 2 * d_v


def query_output_bytes_per_head(d_qk: int = D_QK, d_v: int = D_V, elem_bytes: int = 2) -> int:
    return elem_bytes * (d_qk + d_v)


def kv_bytes_per_token(w: Workload) -> int:
    """Bytes of one stored latent row: 576 bf16, or 576 e4m3 codes + one fp32 scale."""
    return 2 * D_QK if w.kv_dtype == "bf16" else D_QK + 4


def visible_scores(w: Workload, lens) -> int:
    """Sum over requests and query rows of the positions each row attends to."""
    tot = 0
    for L in np.asarray(lens, dtype=np.int64):
        for i in range(w.q_len):
            vis = int(L) - w.q_len + i + 1 if w.causal else int(L)
            tot += max(vis, 0) * w.H
    return tot


def layer_step(w: Workload, lens) -> dict:
    """Algorithmic work of one layer-step of the whole emulated c-rank group."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * kv_bytes_per_token(w)
    flops = visible_scores(w, lens) * flops_per_score()
    rows = w.B * w.q_len * w.H
    q_bytes = rows * D_QK * 2
    part_bytes = w.c * rows * (D_V + 1) * 4            # fp32 o_r and lse_r
    final_bytes = rows * (D_V * 2 + 4)                 # bf16 o and fp32 lse
    return dict(kv_bytes=kv, flops=flops, rows=rows, q_bytes=q_bytes,
                partial_bytes=part_bytes, final_bytes=final_bytes,
                decode_bytes=kv + w.c * q_bytes + part_bytes,
                merge_bytes=part_bytes + final_bytes,
                intensity=flops / kv if kv else 0.0)


def owned_tokens(L: int, c: int, r: int, I: int = 1) -> int:
    """Positions below L that rank r owns when runs of I positions go to the ranks in turn."""
    full = L // (I * c)
    return full * I + min(max(L - full * I * c - r * I, 0), I)


def visible_scores_rank(w: Workload, lens, r: int) -> int:
    """visible_scores restricted to the positions rank r owns."""
    tot = 0
    for L in np.asarray(lens, dtype=np.int64):
        for i in range(w.q_len):
            lim = int(L) - w.q_len + i + 1 if w.causal else int(L)
            tot += owned_tokens(max(min(lim, int(L)), 0), w.c, r, w.interleave) * w.H
    return tot


def rank_share(w: Workload, lens, r: int = 0) -> dict:
    """Algorithmic work of one rank's decode call (rank_begin = r, rank_count = 1):
    the rank's KV rows read once, q read once, its partials written."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = sum(owned_tokens(int(L), w.c, r, w.interleave) for L in lens) * kv_bytes_per_token(w)
    rows = w.B * w.q_len * w.H
    return dict(kv_bytes=kv, flops=visible_scores_rank(w, lens, r) * flops_per_score(),
                decode_bytes=kv + rows * D_QK * 2 + rows * (D_V + 1) * 4)
