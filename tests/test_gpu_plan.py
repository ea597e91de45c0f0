"""GPU check of the decode's work plan: integer index work, compared bit for bit.

The work plan is no part of the method's arithmetic (it only decides which
workgroup decodes which rank-local token range), so the oracle has nothing to
say about it; the attention parity tests catch a plan that drops or repeats a
token only through the outputs.  Here the plan that decode_plan_kernel writes
into the caller's workspace is read back and compared with a restatement of
its rules in Python:

* a unit (rank r, request b) holds ceil(n / stage) stages, n the rank's
  tokens of request b (the oracle's owned_count; stages of 32 bf16 or 64
  e4m3 tokens);
* the total W is cut into items of T = clamp(ceil(W / target), t_min, t_max)
  stages, target = 2 x CUs / row blocks, halved when the longest unit is at
  most 1.25 x the mean; a unit of s stages gets ceil(s / T) items: equal
  ones for such equal-length batches, else items of T stages and one shorter
  last item;
* slots: the items of units with several items first (unit order), then
  the single-item units;
* dispatch order (ragged batches of at most 1024 units): every T-stage item
  first, unit by unit, then the shorter last items longest first (ties by
  unit); otherwise the slot order;
* one record per dispatch position (slot, unit, first and end token,
  request length, single-item flag), slot -1 past the last item.

It also checks what the rules imply: every unit's items tile its tokens
exactly once, the positions are a permutation of the slots.
"""
import math

import numpy as np
import pytest
import torch

from oracle import layout as OL
from parity import Case, log
from workloads import configs as C

pytestmark = pytest.mark.gpu

MAX_TAB, ITEM_MIN_STAGES, ITEMS_PER_CU = 512, 8, 2


def W(**kw):
    base = dict(name="t", index=110, B=1, H=16, q_len=1, c=4, P=16, kv_dtype="bf16", lse_base="e", fixed_len=64)
    base.update(kw)
    return C.Workload(**base)


def _ragged(n, seed, long):
    lens = [int(x) for x in np.random.default_rng(seed).integers(0, 400, n)]
    for b, L in long.items():
        lens[b] = L
    return lens


def _al(x):
    return (x + 255) // 256 * 256


def expected_plan(w, lens, max_seq_len, cus):
    """The plan's rules restated: (layout sizes, records, n_items, unit_first, unit_count, split_units)."""
    rows = w.q_len * w.H
    rg = 4 if rows % 64 == 0 else (2 if rows % 32 == 0 else 1)
    nrb = rows // (16 * rg)
    stok = 64 if w.kv_dtype == "fp8" else 32
    units = w.c * w.B
    cyc = w.interleave * w.c
    stages_max = -(-(-(-max_seq_len // cyc) * w.interleave) // stok)
    t_max = min(1 << 27, max(1, (MAX_TAB - 1) * w.P // stok))
    t_min = min(max(1, ITEM_MIN_STAGES * 32 // stok), t_max)
    target = max(1, ITEMS_PER_CU * cus // nrb)
    assert stages_max > t_min, "a case for the plan must need one"
    max_items = units + max(target, units * -(-stages_max // t_max))
    st = [-(-OL.owned_count(int(lens[u % w.B]), w.c, u // w.B, w.interleave) // stok) for u in range(units)]
    W_, smax = sum(st), max(st)
    uniform = smax * units * 4 <= W_ * 5
    if uniform:
        target = max(1, target // 2)
    T = min(max(-(-W_ // target), t_min), t_max)

    def plan_of(s):
        if s == 0:
            return 1, 0
        items = -(-s // T)
        if not uniform:
            return items, T
        ln = -(-s // items)
        return -(-s // ln), ln

    plans = [plan_of(s) for s in st]
    split = [u for u in range(units) if plans[u][0] > 1]
    first, nxt = {}, 0
    for u in split:
        first[u] = nxt
        nxt += plans[u][0]
    for u in range(units):
        if plans[u][0] == 1:
            first[u] = nxt
            nxt += 1
    n_total = nxt
    lpt = not uniform and units <= 1024
    pos = {}
    if lpt:
        full = [(s // ln if s > 0 else 0) for s, (_, ln) in zip(st, plans)]
        before = np.concatenate([[0], np.cumsum(full)])
        rest = [(u, st[u] - full[u] * plans[u][1]) for u in range(units) if full[u] < plans[u][0]]
        order = sorted(rest, key=lambda t: (-min(t[1], (1 << 20) - 1), t[0]))
        rank = {u: i for i, (u, _) in enumerate(order)}
        for u in range(units):
            for k in range(plans[u][0]):
                pos[(u, k)] = int(before[u]) + k if k < full[u] else int(before[-1]) + rank[u]
    else:
        for u in range(units):
            for k in range(plans[u][0]):
                pos[(u, k)] = first[u] + k
    n_pos = (max_items + 7) // 8 * 8
    recs = np.zeros((n_pos, 8), dtype=np.int64)
    recs[:, 0] = -1
    for u in range(units):
        items, ln = plans[u]
        L = int(lens[u % w.B])
        for k in range(items):
            recs[pos[(u, k)]] = [first[u] + k, u, k * ln * stok, min((k + 1) * ln, st[u]) * stok, L,
                                 1 if items == 1 else 0, 0, 0]
    items_max = plan_of(smax)[0]
    sizes = dict(rows=rows, max_items=max_items, units=units, n_pos=n_pos, stok=stok)
    return (sizes, recs, [n_total, len(split), items_max], [first[u] for u in range(units)],
            [plans[u][0] for u in range(units)], split, st)


CASES = [
    ("ragged_16_units_h16", W(index=110, H=16, c=4, P=16, B=4), _ragged(4, 21, {1: 9000})),
    ("ragged_64_units", W(index=111, H=16, c=4, P=16, B=16), _ragged(16, 22, {3: 6000, 9: 2500})),
    ("ragged_h128_two_blocks", W(index=112, H=128, c=4, P=64, B=8), _ragged(8, 23, {0: 30000, 5: 7000})),
    ("ragged_verify_q4", W(index=113, H=16, q_len=4, c=4, P=64, B=4), _ragged(4, 24, {2: 12000})),
    ("ragged_interleave_16", W(index=114, H=16, c=4, P=64, B=6, interleave=16), _ragged(6, 25, {4: 20000})),
    ("ragged_257_units", W(index=115, H=16, c=1, P=16, B=257), _ragged(257, 26, {100: 7000})),
    ("equal_lengths", W(index=116, H=64, c=2, P=64, fixed_len=20000, B=3), None),
    ("e4m3_equal_lengths", W(index=117, H=64, c=8, P=64, fixed_len=30000, B=2, kv_dtype="fp8"), None),
    ("units_over_1024", W(index=118, H=16, c=4, P=16, B=260), _ragged(260, 27, {3: 12000, 259: 12000})),
]


@pytest.mark.parametrize("name,w,lens", CASES, ids=[c[0] for c in CASES])
def test_plan_records_match_the_rules(name, w, lens):
    log(f"plan case {name}: {w}")
    case = Case(w, lens=lens)
    g = case.group
    ws = g.workspace_for(w.q_len, w.H)
    assert ws is not None
    from kv_sharded_mla_amd import LSE_BASE_2, LSE_BASE_E
    g.decode(case.q, w.sm_scale, LSE_BASE_2 if w.lse_base == "2" else LSE_BASE_E, w.causal, workspace=ws)
    torch.cuda.synchronize()
    assert g.status() == 0
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sizes, recs, n_items, unit_first, unit_count, split, st = expected_plan(w, case.lens, g.max_seq_len, cus)
    # workspace: partial o, partial lse, then the plan's int32 arrays (each section 256-byte aligned)
    off_ints = _al(sizes["max_items"] * sizes["rows"] * 512 * 4) + _al(sizes["max_items"] * sizes["rows"] * 4)
    ints = ws.view(torch.int32).cpu().numpy()[off_ints // 4:]
    n_pos, units = sizes["n_pos"], sizes["units"]
    got_recs = ints[:8 * n_pos].reshape(n_pos, 8).astype(np.int64)
    rest = ints[8 * n_pos:]
    got_n_items = rest[:3].tolist()
    got_first = rest[3:3 + units].tolist()
    got_count = rest[3 + units:3 + 2 * units].tolist()
    got_split = rest[3 + 2 * units:3 + 2 * units + len(split)].tolist()
    assert got_n_items == n_items, (got_n_items, n_items)
    assert got_first == unit_first and got_count == unit_count
    assert got_split == split
    n_total = n_items[0]
    # past the last item only the slot field is written (-1)
    assert np.array_equal(got_recs[n_total:, 0], recs[n_total:, 0])
    assert np.array_equal(got_recs[:n_total], recs[:n_total]), \
        np.argwhere(got_recs[:n_total] != recs[:n_total])[:5]
    # what the rules imply: the positions hold every slot once, and each unit's
    # items tile its visible tokens (whole stages, the last one clipped at the end)
    assert sorted(got_recs[:n_total, 0].tolist()) == list(range(n_total))
    for u in range(units):
        mine = sorted((r[2], r[3]) for r in got_recs[:n_total] if r[1] == u)
        assert mine[0][0] == 0 and all(a[1] == b[0] for a, b in zip(mine, mine[1:]))
        assert mine[-1][1] == st[u] * sizes["stok"]
    log(f"{name}: {n_total} items, {len(split)} split units, records identical")
