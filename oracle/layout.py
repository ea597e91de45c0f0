"""Integer model of the DCP shared virtual KV layout (oracle; test infrastructure only).

Follows the SGLang page "Decode Context Parallelism", section "Virtual KV
layout": each rank has physical capacity C tokens in pages of P tokens; the
group exposes one shared virtual allocator with capacity C*c and page size
P*c; a virtual slot v belongs to rank owner(v) = v mod c and sits there at
physical slot physical(v) = floor(v / c).  Every rank sees the same
request-to-token map; on a write each rank keeps the positions it owns and
compacts them into its own pool.  The vLLM page "Context Parallel Deployment"
(section "Decode Context Parallel") gives the user-visible block size as the
physical block times the DCP size (16 tokens at DCP 4 cover 64 tokens).

Readings where the pages are silent (the allocator's policy and the call
contract are not on the pages; these fix the one exact answer the bit-exact
checks compare against):

* A virtual page id is a page index shared by all owner pools: virtual page
  g covers virtual slots [g*P*c, (g+1)*P*c) and, on every rank, physical
  slots [g*P, (g+1)*P).
* Pages are popped from the top of a caller-supplied free stack, in
  (request, logical page) order; a call that cannot be satisfied takes no
  page at all (all-or-nothing).
* New rows of request b occupy the last n_b positions before seq_len[b].
* Interleave size I (the vLLM study page "vLLM Decode Context Parallelism",
  section on operation, configuration example: a KV interleave size, one
  token by default, larger chunks for less sorting work at some imbalance):
  consecutive chunks of I positions go to the ranks in turn, owner(p) =
  floor(p / I) mod c, and I divides P so that every virtual page still gives
  each rank exactly P positions.  In virtual-slot terms owner(v) =
  floor(v / I) mod c and physical(v) = floor(v / (I c)) I + v mod I, which
  are the pages' v mod c and floor(v / c) at I = 1.  Rank r's j-th position
  is then p = floor(j / I) I c + r I + j mod I, and its page is floor(j / P),
  so the shared block table is still the rank-local page table.

Status codes mirror the library's documented device status values; they are
restated here rather than imported.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

OK = 0
OUT_OF_PAGES = 1
BAD_LENGTH = 2
TABLE_OVERFLOW = 3
BAD_PAGE = 4


def owner(v: int, c: int, I: int = 1) -> int:
    return (v // I) % c


def physical(v: int, c: int, I: int = 1) -> int:
    return (v // (I * c)) * I + v % I


def virtual_page_size(P: int, c: int) -> int:
    return P * c


def virtual_capacity(C: int, c: int) -> int:
    return C * c


def pages_for(length: int, P: int, c: int) -> int:
    """Virtual pages that hold ``length`` tokens (ceil(length / (P*c)))."""
    vp = P * c
    return (length + vp - 1) // vp


def virtual_slot(bt_row: Sequence[int], p: int, P: int, c: int) -> int:
    """Virtual slot of logical position p of a request whose pages are bt_row."""
    vp = P * c
    return int(bt_row[p // vp]) * vp + p % vp


def slot_of(bt_row: Sequence[int], p: int, P: int, c: int, I: int = 1) -> Tuple[int, int]:
    """(owner rank, physical slot in that rank's pool) of logical position p."""
    v = virtual_slot(bt_row, p, P, c)
    return owner(v, c, I), physical(v, c, I)


def alloc_virtual(free_stack: np.ndarray, free_top: int, old_len: Sequence[int],
                  new_len: Sequence[int], block_table: np.ndarray, P: int, c: int):
    """Grow every request from old_len to new_len tokens.

    Returns ``(status, free_top, block_table)``; on any error nothing changes.
    """
    bt = np.array(block_table, copy=True)
    stride = bt.shape[1]
    B = len(old_len)
    for b in range(B):
        if old_len[b] < 0 or new_len[b] < old_len[b]:
            return BAD_LENGTH, free_top, np.array(block_table, copy=True)
    for b in range(B):
        if pages_for(int(new_len[b]), P, c) > stride:
            return TABLE_OVERFLOW, free_top, np.array(block_table, copy=True)
    need = [pages_for(int(new_len[b]), P, c) - pages_for(int(old_len[b]), P, c) for b in range(B)]
    if sum(need) > free_top:
        return OUT_OF_PAGES, free_top, np.array(block_table, copy=True)
    top = free_top
    for b in range(B):
        first = pages_for(int(old_len[b]), P, c)
        for i in range(need[b]):
            top -= 1
            bt[b, first + i] = free_stack[top]
    return OK, top, bt


def write_slots(block_table: np.ndarray, seq_len: Sequence[int], cu_new: Sequence[int],
                P: int, c: int, num_pages: int, I: int = 1, n_rows: int = None):
    """Destination of every new row: (status, owner[N], phys[N]); -1 where skipped.

    Rows cu_new[b] .. cu_new[b+1]-1 belong to request b.  ``n_rows`` (default
    cu_new[B]) is the number of rows handed over; a row that belongs to no
    request (below cu_new[0] or at or past cu_new[B]) is skipped with
    BAD_LENGTH.
    """
    B = len(seq_len)
    N = int(cu_new[B]) if n_rows is None else int(n_rows)
    own = np.full(N, -1, dtype=np.int64)
    phys = np.full(N, -1, dtype=np.int64)
    status = OK
    if N > 0 and (B == 0 or int(cu_new[0]) > 0 or int(cu_new[B]) < N):
        status = BAD_LENGTH
    stride = block_table.shape[1]
    for b in range(B):
        n_b = int(cu_new[b + 1]) - int(cu_new[b])
        first = int(seq_len[b]) - n_b
        for k in range(max(n_b, 0)):
            row = int(cu_new[b]) + k
            if row >= N:
                break
            p = first + k
            if first < 0:
                status = max(status, BAD_LENGTH)
                continue
            if p // (P * c) >= stride:
                status = max(status, TABLE_OVERFLOW)
                continue
            page = int(block_table[b, p // (P * c)])
            if page < 0 or page >= num_pages:
                status = max(status, BAD_PAGE)
                continue
            r, s = slot_of(block_table[b], p, P, c, I)
            own[row], phys[row] = r, s
    return status, own, phys


def pool_image(pools: np.ndarray, block_table: np.ndarray, seq_len, cu_new, rows: np.ndarray,
               P: int, c: int, scales: np.ndarray = None, pool_scales: np.ndarray = None, I: int = 1):
    """Expected pool bytes after scattering ``rows`` into a copy of ``pools``.

    ``pools`` is [c][num_pages*P][row elements] in the stored dtype; every row
    of ``rows`` is handed over (see :func:`write_slots`).
    """
    out = np.array(pools, copy=True)
    outs = None if pool_scales is None else np.array(pool_scales, copy=True)
    num_pages = out.shape[1] // P
    status, own, phys = write_slots(block_table, seq_len, cu_new, P, c, num_pages, I, n_rows=len(rows))
    for n in range(len(own)):
        if own[n] >= 0:
            out[own[n], phys[n]] = rows[n]
            if outs is not None:
                outs[own[n], phys[n]] = scales[n]
    return status, own, phys, out, outs


def owned_positions(length: int, c: int, r: int, I: int = 1) -> np.ndarray:
    """Logical positions of a request of ``length`` tokens that rank r owns, ascending."""
    return np.array([p for p in range(length) if owner(p, c, I) == r], dtype=np.int64)


def owned_count(length: int, c: int, r: int, I: int = 1) -> int:
    return sum(1 for p in range(length) if (p // I) % c == r)


def rank_local_slots(block_table_row: Sequence[int], length: int, P: int, c: int, r: int,
                     I: int = 1) -> List[int]:
    """Physical slots, in rank r's pool, of the positions r owns, in position order."""
    return [slot_of(block_table_row, int(p), P, c, I)[1] for p in owned_positions(length, c, r, I)]


# ---- extend and prefill->decode relayout ------------------------------------
#
# SGLang page "Decode Context Parallelism": the section on the decode cost
# model says an extend step may gather the cached prefix shards back into
# token order before appending new tokens; the section "DCP x PD
# disaggregation" says dense prefill pages cannot be copied into striped decode
# storage as they are, that a DCP1 prefill feeding a DCP-c decode relays the
# tokens out, selecting and packing the rows each decode rank owns, and that
# the plan carries the exact token count so that no stale row of a partly
# filled last page is transferred.


def read_rows(pools: np.ndarray, block_table: np.ndarray, seq_len: Sequence[int], cu_out: Sequence[int],
              P: int, c: int, I: int = 1, pool_scales: np.ndarray = None, out: np.ndarray = None,
              out_scales: np.ndarray = None):
    """Rows of positions 0 .. seq_len[b]-1 of every request, in token order.

    Row p of request b goes to ``out[cu_out[b] + p]``.  ``pools`` is
    [c][num_pages*P][row elements].  A request with seq_len < 0, with
    cu_out[b+1] - cu_out[b] != seq_len[b], or whose span [cu_out[b],
    cu_out[b+1]) leaves the output rows is skipped (BAD_LENGTH), one that
    needs more virtual pages than a table row holds is skipped
    (TABLE_OVERFLOW), and a position on a page id outside the pools is skipped
    (BAD_PAGE).  Skipped rows of ``out`` keep their contents.  Returns
    ``(status, out, out_scales)``.
    """
    B = len(seq_len)
    num_pages = pools.shape[1] // P
    n_out = int(cu_out[B]) if out is None else out.shape[0]
    if out is None:
        out = np.zeros((n_out,) + pools.shape[2:], dtype=pools.dtype)
    else:
        out = np.array(out, copy=True)
    if pool_scales is not None:
        out_scales = np.zeros(n_out, np.float32) if out_scales is None else np.array(out_scales, copy=True)
    stride = block_table.shape[1]
    status = OK
    for b in range(B):
        L = int(seq_len[b])
        if L < 0 or int(cu_out[b]) < 0 or int(cu_out[b + 1]) > n_out or int(cu_out[b + 1]) - int(cu_out[b]) != L:
            status = max(status, BAD_LENGTH)
            continue
        if pages_for(L, P, c) > stride:
            status = max(status, TABLE_OVERFLOW)
            continue
        for p in range(L):
            page = int(block_table[b, p // (P * c)])
            if page < 0 or page >= num_pages:
                status = max(status, BAD_PAGE)
                continue
            r, s = slot_of(block_table[b], p, P, c, I)
            out[int(cu_out[b]) + p] = pools[r, s]
            if pool_scales is not None:
                out_scales[int(cu_out[b]) + p] = pool_scales[r, s]
    return status, out, out_scales


def relayout_dense(src_pool: np.ndarray, src_table: np.ndarray, seq_len: Sequence[int], P: int, c: int,
                   dst_pools: np.ndarray, dst_table: np.ndarray, rank_begin: int, rank_count: int,
                   I: int = 1, src_scales: np.ndarray = None, dst_scales: np.ndarray = None):
    """Copy every request's rows from a dense (DCP1) paged pool into the owner pools.

    The dense pool is [num_src_pages*P][row elements]; position p of request b
    sits there at slot src_table[b][p // P] * P + p % P.  Exactly the
    positions p < seq_len[b] whose owner is in [rank_begin, rank_begin +
    rank_count) are written, at the slot the shared virtual table dst_table
    gives them; nothing else in ``dst_pools`` changes.  Requests or positions
    that fail a check are skipped as in :func:`read_rows` (a page id of
    either table outside its pool: BAD_PAGE).  Returns ``(status, dst_pools,
    dst_scales)``.
    """
    out = np.array(dst_pools, copy=True)
    outs = None if dst_scales is None else np.array(dst_scales, copy=True)
    n_src_pages = src_pool.shape[0] // P
    num_pages = out.shape[1] // P
    status = OK
    for b in range(len(seq_len)):
        L = int(seq_len[b])
        if L < 0:
            status = max(status, BAD_LENGTH)
            continue
        if (L + P - 1) // P > src_table.shape[1] or pages_for(L, P, c) > dst_table.shape[1]:
            status = max(status, TABLE_OVERFLOW)
            continue
        for p in range(L):
            # the owner does not depend on the page ids (I divides P): ranks
            # outside the range neither read nor check anything
            if not rank_begin <= owner(p, c, I) < rank_begin + rank_count:
                continue
            sp = int(src_table[b, p // P])
            vpg = int(dst_table[b, p // (P * c)])
            if sp < 0 or sp >= n_src_pages or vpg < 0 or vpg >= num_pages:
                status = max(status, BAD_PAGE)
                continue
            r, s = slot_of(dst_table[b], p, P, c, I)
            out[r, s] = src_pool[sp * P + p % P]
            if outs is not None:
                outs[r, s] = src_scales[sp * P + p % P]
    return status, out, outs
