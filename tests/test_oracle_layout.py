"""Pins for the oracle's integer layout model (CPU only).

Literal vectors come from the pages (tests/golden/stripes.json, each with its
citation); the rest is brute-force enumeration of small groups against the
closed forms owner(v) = v mod c, physical(v) = floor(v/c), plus the balance
property that one widened virtual page maps to one physical page on every rank.
"""
import json
import os

import numpy as np
import pytest

from oracle import layout

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_dcp4_diagram_vectors():
    g = _gold("stripes.json")["dcp4_diagram"]
    for r, want in enumerate(g["owned"]):
        assert list(layout.owned_positions(g["tokens"], g["c"], r)) == want


def test_dcp4_4096_prefix_and_share():
    g = _gold("stripes.json")["dcp4_4096_prefix"]
    for r, want in enumerate(g["owned_prefix"]):
        got = layout.owned_positions(g["tokens"], g["c"], r)
        assert list(got[:3]) == want
        assert len(got) == g["owned_count"]


def test_effective_block_size():
    g = _gold("stripes.json")["effective_block"]
    assert layout.virtual_page_size(g["P"], g["c"]) == g["virtual_page"]


def test_allocator_hand_worked_example():
    # P=2, c=2 -> virtual page of 4 tokens.  Request 0 grows 0 -> 5 tokens (2 pages),
    # request 1 grows 3 -> 9 tokens (from 1 page to 3).  Pops come off the top of the
    # stack in (request, page) order: 8, 6 for request 0, then 4, 2 for request 1.
    stack = np.array([5, 3, 9, 1, 7, 0, 2, 4, 6, 8], dtype=np.int32)
    bt = np.full((2, 4), -1, dtype=np.int32)
    bt[1, 0] = 11
    st, top, out = layout.alloc_virtual(stack, 10, [0, 3], [5, 9], bt, P=2, c=2)
    assert st == layout.OK and top == 6
    assert out.tolist() == [[8, 6, -1, -1], [11, 4, 2, -1]]


@pytest.mark.parametrize("old,new,top,stride,want", [
    ([0, 0], [9, 9], 4, 4, layout.OUT_OF_PAGES),       # needs 3 + 3 > 4
    ([4, 0], [3, 1], 10, 4, layout.BAD_LENGTH),         # shrinking
    ([0, 0], [17, 1], 10, 4, layout.TABLE_OVERFLOW),    # 5 pages > stride 4
])
def test_allocator_errors_change_nothing(old, new, top, stride, want):
    stack = np.arange(10, dtype=np.int32)
    bt = np.full((2, stride), -7, dtype=np.int32)
    st, t2, out = layout.alloc_virtual(stack, top, old, new, bt, P=2, c=2)
    assert st == want and t2 == top and np.array_equal(out, bt)


def _grow(rng, c, P, lens_final, steps):
    """Grow a batch step by step through the allocator; returns block table and stack."""
    B = len(lens_final)
    vp = P * c
    num_pages = sum((L + vp - 1) // vp for L in lens_final) + 2
    stack = rng.permutation(num_pages).astype(np.int32)
    top = num_pages
    stride = max((L + vp - 1) // vp for L in lens_final) + 1
    bt = np.full((B, stride), -1, dtype=np.int32)
    cur = [0] * B
    for s in range(1, steps + 1):
        new = [min(L, (L * s) // steps) for L in lens_final]
        st, top, bt = layout.alloc_virtual(stack, top, cur, new, bt, P, c)
        assert st == layout.OK
        cur = new
    return bt, num_pages


@pytest.mark.parametrize("seed", range(12))
def test_slot_map_brute_force(seed):
    rng = np.random.default_rng(seed)
    c = int(rng.integers(1, 9))
    P = int(rng.integers(1, 5))
    B = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(0, 200, size=B)]
    bt, num_pages = _grow(rng, c, P, lens, steps=int(rng.integers(1, 6)))
    C = num_pages * P
    seen = set()
    for b, L in enumerate(lens):
        for p in range(L):
            r, s = layout.slot_of(bt[b], p, P, c)
            assert r == p % c                       # interleave of one token
            assert 0 <= s < C
            assert (r, s) not in seen               # no two tokens share a slot
            seen.add((r, s))
        # the rank-local walk over owned positions uses the shared table directly:
        # the j-th owned position of rank r sits at bt[j // P] * P + j % P
        for r in range(c):
            want = [int(bt[b, j // P]) * P + j % P for j in range(layout.owned_count(L, c, r))]
            assert layout.rank_local_slots(bt[b], L, P, c, r) == want


@pytest.mark.parametrize("c,P", [(1, 4), (2, 3), (4, 16), (8, 2), (5, 7)])
def test_balance_within_one_token(c, P):
    for L in range(0, 300):
        counts = [layout.owned_count(L, c, r) for r in range(c)]
        assert max(counts) - min(counts) <= 1
        assert sum(counts) == L
    # one widened virtual page is one physical page on every rank: each rank stores its
    # share in (a prefix of) the request's own virtual pages, in the same page ids, and
    # page counts differ by at most one (only the partial last page can be missing)
    rng = np.random.default_rng(c * 10 + P)
    for L in [1, P * c - 1, P * c, P * c + 1, 5 * P * c + 3]:
        bt, _ = _grow(rng, c, P, [L], steps=3)
        vpages = [int(x) for x in bt[0, :layout.pages_for(L, P, c)]]
        for r in range(c):
            pg = []
            for s in layout.rank_local_slots(bt[0], L, P, c, r):
                if not pg or pg[-1] != s // P:
                    pg.append(s // P)
            assert pg == vpages[:len(pg)]
            assert len(vpages) - len(pg) <= 1


def test_write_slots_positions_and_errors():
    c, P = 2, 2
    bt = np.array([[3, 1, -1], [0, 9, -1]], dtype=np.int32)
    # request 0 appends 3 rows ending at length 6 (positions 3,4,5); request 1 appends 1 row at 5
    st, own, phys = layout.write_slots(bt, [6, 5], [0, 3, 4], P, c, num_pages=4)
    assert st == layout.BAD_PAGE                         # page 9 >= 4 pages
    assert own.tolist() == [1, 0, 1, -1]
    # position 3: v = 3*4 + 3 = 15 -> owner 1, phys 7 ; position 4: v = 1*4 + 0 -> owner 0, phys 2
    assert phys.tolist() == [7, 2, 2, -1]
    st, _, _ = layout.write_slots(bt, [2, 0], [0, 3, 3], P, c, num_pages=4)
    assert st == layout.BAD_LENGTH


def test_pool_image_sentinel_untouched():
    c, P = 2, 2
    bt = np.array([[1, 0]], dtype=np.int32)
    pools = np.full((c, 2 * P, 3), 0xEE, dtype=np.uint8)
    rows = np.arange(15, dtype=np.uint8).reshape(5, 3)
    st, own, phys, out, _ = layout.pool_image(pools, bt, [5], [0, 5], rows, P, c)
    assert st == layout.OK
    written = {(int(o), int(s)) for o, s in zip(own, phys)}
    for r in range(c):
        for s in range(2 * P):
            if (r, s) not in written:
                assert (out[r, s] == 0xEE).all()      # a partial last page leaks nothing
    assert len(written) == 5


# ---- interleave size I > 1 -------------------------------------------------
# Pinned against a constructive model written without the closed forms: each
# virtual page of P*c positions is dealt to the ranks in chunks of I
# consecutive positions, rank after rank, and every rank appends what it is
# dealt to its own physical page in arrival order.

def _dealt(P, c, I, n_pages):
    """position -> (rank, physical slot) for pages 0..n_pages-1 with identity page ids."""
    out = {}
    for g in range(n_pages):
        fill = [0] * c
        pos = g * P * c
        rank = 0
        while pos < (g + 1) * P * c:
            for _ in range(I):
                out[pos] = (rank, g * P + fill[rank])
                fill[rank] += 1
                pos += 1
            rank = (rank + 1) % c
    return out


@pytest.mark.parametrize("c,P,I", [(2, 4, 2), (3, 6, 3), (4, 8, 2), (4, 16, 16), (8, 16, 4), (1, 8, 4), (3, 4, 1)])
def test_interleaved_slots_match_dealing(c, P, I):
    n_pages = 5
    want = _dealt(P, c, I, n_pages)
    bt = list(range(n_pages))
    for p, (r, s) in want.items():
        assert layout.slot_of(bt, p, P, c, I) == (r, s), (p, r, s)
    # each (rank, slot) of a virtual page is used exactly once
    assert len(set(want.values())) == len(want)


@pytest.mark.parametrize("c,I", [(2, 2), (3, 4), (4, 16), (8, 8), (5, 3)])
def test_interleaved_ownership_and_balance(c, I):
    for L in range(0, 3 * I * c + 5):
        counts = [layout.owned_count(L, c, r, I) for r in range(c)]
        assert sum(counts) == L
        assert max(counts) - min(counts) <= I
        for r in range(c):
            pos = layout.owned_positions(L, c, r, I)
            assert len(pos) == counts[r]
            # rank r's j-th position in closed form
            j = np.arange(len(pos))
            assert np.array_equal(pos, (j // I) * I * c + r * I + j % I)


@pytest.mark.parametrize("c,P,I", [(2, 4, 2), (4, 16, 4), (3, 12, 6)])
def test_interleaved_rank_local_page_table_is_the_block_table(c, P, I):
    rng = np.random.default_rng(7)
    bt = rng.permutation(40)[:8]
    for L in (1, P * c - 1, P * c, 3 * P * c + 5, 8 * P * c):
        for r in range(c):
            n = layout.owned_count(L, c, r, I)
            want = [int(bt[j // P]) * P + j % P for j in range(n)]
            assert layout.rank_local_slots(bt, L, P, c, r, I) == want


def test_interleave_one_is_the_token_cycle():
    for v in range(200):
        for c in (1, 2, 3, 8):
            assert layout.owner(v, c, 1) == v % c and layout.physical(v, c, 1) == v // c


# ---- extend gather (striped -> token order) and DCP1 -> DCP c relayout -------
# Expected pools are built with the dealing model above (chunks of I positions
# dealt rank after rank onto each rank's own page of the virtual page), with
# page ids taken from the request's table; no closed form of the oracle is used.

def _dealt_request(bt_row, L, P, c, I):
    """position -> (rank, physical slot) of one request whose virtual pages are bt_row."""
    out = {}
    for g in range((L + P * c - 1) // (P * c)):
        fill = [0] * c
        pos, rank = g * P * c, 0
        while pos < (g + 1) * P * c:
            for _ in range(I):
                if pos < L:
                    out[pos] = (rank, int(bt_row[g]) * P + fill[rank])
                fill[rank] += 1
                pos += 1
            rank = (rank + 1) % c
    return out


def _row(b, p, width=5):
    return np.array([(b * 131 + p * 7 + k * 3) % 65521 for k in range(width)], dtype=np.uint16)


def _striped_case(seed, c, P, I, lens):
    rng = np.random.default_rng(seed)
    vp = P * c
    stride = max(1, max((L + vp - 1) // vp for L in lens))
    num_pages = sum((L + vp - 1) // vp for L in lens) + 2
    ids = rng.permutation(num_pages)
    bt = np.full((len(lens), stride), -1, np.int32)
    k = 0
    for b, L in enumerate(lens):
        for g in range((L + vp - 1) // vp):
            bt[b, g] = ids[k]
            k += 1
    return bt, num_pages


@pytest.mark.parametrize("c,P,I,lens", [
    (4, 2, 1, [22, 0, 9]), (2, 4, 2, [17, 8]), (3, 6, 3, [40, 1, 18]), (8, 16, 4, [300]), (1, 4, 1, [13, 4]),
    (4, 8, 8, [70, 33]),
])
def test_read_rows_restores_token_order(c, P, I, lens):
    bt, num_pages = _striped_case(len(lens) + c, c, P, I, lens)
    pools = np.full((c, num_pages * P, 5), 0xBEEF, np.uint16)
    for b, L in enumerate(lens):
        for p, (r, s) in _dealt_request(bt[b], L, P, c, I).items():
            pools[r, s] = _row(b, p)
    cu = np.concatenate([[0], np.cumsum(lens)])
    st, out, _ = layout.read_rows(pools, bt, lens, cu, P, c, I)
    assert st == layout.OK
    want = np.array([_row(b, p) for b, L in enumerate(lens) for p in range(L)], dtype=np.uint16).reshape(-1, 5)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("seed", range(6))
def test_read_rows_inverts_the_scatter(seed):
    rng = np.random.default_rng(seed)
    c = int(rng.integers(1, 6))
    P = int(rng.choice([1, 4, 6, 16]))
    I = int(rng.choice([d for d in range(1, P + 1) if P % d == 0]))
    lens = [int(x) for x in rng.integers(0, 90, size=int(rng.integers(1, 5)))]
    bt, num_pages = _striped_case(seed, c, P, I, lens)
    rows = rng.integers(0, 65536, size=(sum(lens), 7)).astype(np.uint16)
    scales = rng.standard_normal(sum(lens)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pools = np.zeros((c, num_pages * P, 7), np.uint16)
    pscales = np.zeros((c, num_pages * P), np.float32)
    st, _, _, pools, pscales = layout.pool_image(pools, bt, lens, cu, rows, P, c, scales, pscales, I)
    assert st == layout.OK
    st, out, out_sc = layout.read_rows(pools, bt, lens, cu, P, c, I, pool_scales=pscales)
    assert st == layout.OK
    assert np.array_equal(out, rows) and np.array_equal(out_sc, scales)


def test_read_rows_errors_skip_and_keep():
    c, P = 2, 2
    bt = np.array([[0, 1], [1, -1], [5, 0]], np.int32)
    pools = np.arange(c * 2 * P * 3, dtype=np.uint16).reshape(c, 2 * P, 3)
    sentinel = np.full((9, 3), 0xEEEE, np.uint16)
    # request 0 fine (5 tokens), request 1 has a length that disagrees with cu_out
    st, out, _ = layout.read_rows(pools, bt, [5, 2, 0], [0, 5, 8, 8], P, c, out=sentinel[:8])
    assert st == layout.BAD_LENGTH and (out[5:8] == 0xEEEE).all() and not (out[:5] == 0xEEEE).any()
    # 9 tokens need 3 virtual pages of 4 > stride 2
    st, out, _ = layout.read_rows(pools, bt, [9, 0, 0], [0, 9, 9, 9], P, c, out=sentinel)
    assert st == layout.TABLE_OVERFLOW and (out == 0xEEEE).all()
    # page id 5 is outside a 2-page pool: the 4 positions of that virtual page are skipped
    st, out, _ = layout.read_rows(pools, bt, [0, 0, 6], [0, 0, 0, 6], P, c, out=sentinel[:6])
    assert st == layout.BAD_PAGE and (out[:4] == 0xEEEE).all() and not (out[4:6] == 0xEEEE).any()


def _dense_case(seed, c, P, I, lens):
    """A DCP1 pool (pages of P in a shuffled order) holding _row(b, p), its table, and the
    striped side's virtual table."""
    rng = np.random.default_rng(seed)
    n_src = sum((L + P - 1) // P for L in lens) + 1
    sids = rng.permutation(n_src)
    s_stride = max(1, max((L + P - 1) // P for L in lens))
    src_bt = np.full((len(lens), s_stride), -1, np.int32)
    src = np.full((n_src * P, 5), 0xDDDD, np.uint16)
    k = 0
    for b, L in enumerate(lens):
        for q in range((L + P - 1) // P):
            src_bt[b, q] = sids[k]
            k += 1
        for p in range(L):
            src[src_bt[b, p // P] * P + p % P] = _row(b, p)
    bt, num_pages = _striped_case(seed + 100, c, P, I, lens)
    return src, src_bt, bt, num_pages


@pytest.mark.parametrize("c,P,I,lens", [
    (4, 2, 1, [22, 0, 9]), (2, 4, 2, [17, 8]), (3, 6, 3, [40, 1, 18]), (8, 16, 16, [300, 5]), (1, 4, 1, [13, 4]),
])
def test_relayout_places_exactly_the_owned_rows(c, P, I, lens):
    src, src_bt, bt, num_pages = _dense_case(c * 10 + P, c, P, I, lens)
    dst = np.full((c, num_pages * P, 5), 0xEEEE, np.uint16)
    st, out, _ = layout.relayout_dense(src, src_bt, lens, P, c, dst, bt, 0, c, I)
    assert st == layout.OK
    written = set()
    for b, L in enumerate(lens):
        for p, (r, s) in _dealt_request(bt[b], L, P, c, I).items():
            assert np.array_equal(out[r, s], _row(b, p)), (b, p)
            written.add((r, s))
    # the exact token count: every other slot, including the rest of a partly
    # filled last page, keeps what it held
    for r in range(c):
        for s in range(num_pages * P):
            if (r, s) not in written:
                assert (out[r, s] == 0xEEEE).all()
        got = sum(1 for (rr, _) in written if rr == r)
        assert got == sum(layout.owned_count(L, c, r, I) for L in lens)


def test_relayout_rank_ranges_compose():
    c, P, I, lens = 4, 4, 2, [37, 12]
    src, src_bt, bt, num_pages = _dense_case(3, c, P, I, lens)
    dst = np.full((c, num_pages * P, 5), 0xEEEE, np.uint16)
    _, whole, _ = layout.relayout_dense(src, src_bt, lens, P, c, dst, bt, 0, c, I)
    part = dst
    for r in range(c):
        st, part, _ = layout.relayout_dense(src, src_bt, lens, P, c, part, bt, r, 1, I)
        assert st == layout.OK
        # one decode rank's call writes its own pool only
        _, alone, _ = layout.relayout_dense(src, src_bt, lens, P, c, dst, bt, r, 1, I)
        for o in range(c):
            assert np.array_equal(alone[o], whole[o] if o == r else dst[o])
    assert np.array_equal(part, whole)


def test_relayout_to_one_rank_is_the_page_copy():
    # equal DCP sizes (1 and 1) take the existing page path: with the same table the
    # destination pages are the source pages, row for row, over each request's length
    P, lens = 4, [10, 3]
    src, src_bt, _, _ = _dense_case(5, 1, P, 1, lens)
    dst = np.full((1,) + src.shape, 0xEEEE, np.uint16)
    st, out, _ = layout.relayout_dense(src, src_bt, lens, P, 1, dst, src_bt, 0, 1, 1)
    assert st == layout.OK
    for b, L in enumerate(lens):
        for p in range(L):
            slot = src_bt[b, p // P] * P + p % P
            assert np.array_equal(out[0, slot], src[slot])


def test_relayout_errors():
    c, P, I, lens = 2, 4, 4, [16]
    src, src_bt, bt, num_pages = _dense_case(9, c, P, I, lens)
    dst = np.full((c, num_pages * P, 5), 0xEEEE, np.uint16)
    st, out, _ = layout.relayout_dense(src, src_bt, [-1], P, c, dst, bt, 0, c, I)
    assert st == layout.BAD_LENGTH and np.array_equal(out, dst)
    st, out, _ = layout.relayout_dense(src, src_bt[:, :2], [16], P, c, dst, bt, 0, c, I)
    assert st == layout.TABLE_OVERFLOW and np.array_equal(out, dst)
    # with I = P each source page belongs to one rank: a bad page of rank 1 is an error
    # for a call that covers rank 1 and invisible to one that covers rank 0 only
    bad = src_bt.copy()
    bad[0, 1] = 99          # positions 4..7, owned by rank 1
    st, out, _ = layout.relayout_dense(src, bad, [16], P, c, dst, bt, 0, c, I)
    assert st == layout.BAD_PAGE
    st, out0, _ = layout.relayout_dense(src, bad, [16], P, c, dst, bt, 0, 1, I)
    assert st == layout.OK and np.array_equal(out0[1], dst[1])


def test_read_rows_span_outside_the_output_is_skipped():
    c, P = 2, 2
    bt = np.array([[0, 1]], np.int32)
    pools = np.arange(c * 2 * P * 3, dtype=np.uint16).reshape(c, 2 * P, 3)
    sentinel = np.full((4, 3), 0xEEEE, np.uint16)
    st, out, _ = layout.read_rows(pools, bt, [3], [2, 5], P, c, out=sentinel)
    assert st == layout.BAD_LENGTH and (out == 0xEEEE).all()
    st, out, _ = layout.read_rows(pools, bt, [3], [1, 4], P, c, out=sentinel)
    assert st == layout.OK and (out[0] == 0xEEEE).all() and not (out[1:] == 0xEEEE).any()


# ---- planted mistakes in the gather and the relayout -------------------------
# A copy of read_rows or relayout_dense with one plausible bug (made by editing
# its source text) replaces the oracle function while the pins above run: at
# least one pin must fail for every mutant.

_READ_PINS = [
    lambda: [test_read_rows_restores_token_order(*a) for a in [
        (4, 2, 1, [22, 0, 9]), (2, 4, 2, [17, 8]), (3, 6, 3, [40, 1, 18]), (8, 16, 4, [300]), (1, 4, 1, [13, 4]),
        (4, 8, 8, [70, 33])]],
    lambda: [test_read_rows_inverts_the_scatter(s) for s in range(6)],
    lambda: test_read_rows_errors_skip_and_keep(),
    lambda: test_read_rows_span_outside_the_output_is_skipped(),
]
_RELAYOUT_PINS = [
    lambda: [test_relayout_places_exactly_the_owned_rows(*a) for a in [
        (4, 2, 1, [22, 0, 9]), (2, 4, 2, [17, 8]), (3, 6, 3, [40, 1, 18]), (8, 16, 16, [300, 5]),
        (1, 4, 1, [13, 4])]],
    lambda: test_relayout_rank_ranges_compose(),
    lambda: test_relayout_to_one_rank_is_the_page_copy(),
    lambda: test_relayout_errors(),
]

_MUTANTS = {
    # the interleave size ignored when locating a position
    "read_interleave_ignored": ("read_rows", "r, s = slot_of(block_table[b], p, P, c, I)",
                                "r, s = slot_of(block_table[b], p, P, c, 1)"),
    # the output span no longer checked against the output rows
    "read_span_check_dropped": ("read_rows",
                                "if L < 0 or int(cu_out[b]) < 0 or int(cu_out[b + 1]) > n_out or int(cu_out[b + 1]) - int(cu_out[b]) != L:",
                                "if L < 0 or int(cu_out[b + 1]) - int(cu_out[b]) != L:"),
    # the source slot one position off inside its page
    "relayout_shifted_source_slot": ("relayout_dense", "out[r, s] = src_pool[sp * P + p % P]",
                                     "out[r, s] = src_pool[sp * P + (p + 1) % P]"),
    # the rank filter of a partial call taken with interleave 1
    "relayout_rank_filter_token_cycle": ("relayout_dense",
                                         "if not rank_begin <= owner(p, c, I) < rank_begin + rank_count:",
                                         "if not rank_begin <= owner(p, c, 1) < rank_begin + rank_count:"),
    # one row past the exact token count (a stale row of a partial last page)
    "relayout_one_extra_row": ("relayout_dense", "        for p in range(L):\n            # the owner",
                               "        for p in range(L + 1):\n            # the owner"),
}


@pytest.mark.parametrize("kind", sorted(_MUTANTS))
def test_planted_gather_and_relayout_mistakes_fail_a_pin(kind, monkeypatch):
    import inspect
    import textwrap
    fn, old, new = _MUTANTS[kind]
    src = textwrap.dedent(inspect.getsource(getattr(layout, fn)))
    assert src.count(old) == 1, (kind, "mutation does not apply")
    ns = dict(vars(layout))
    exec(compile(src.replace(old, new), f"<mutant {kind}>", "exec"), ns)
    monkeypatch.setattr(layout, fn, ns[fn])
    failed = 0
    for pin in (_READ_PINS if fn == "read_rows" else _RELAYOUT_PINS):
        try:
            pin()
        except Exception:      # an assertion, or an index past the output the real code never writes
            failed += 1
    assert failed >= 1, kind
