"""GPU parity of mla_decode_partial (+ dcp_lse_merge) against the float64 oracle.

Small cases span several LDS stages, ragged tails, empty shards (L < c),
zero-length requests, every row-block shape (16/32/64 rows per workgroup and
several blocks), q_len 4 causal verification, non-causal multi-row queries,
base-2 LSE, pages that do not align with a stage, KV splits with their
combine, the e4m3 format, interleave sizes I > 1 (runs of I positions
per owner, including runs that leave whole ranks empty), and the limits:
q_len 8, 256 heads, 16 owner pools, 256-token pages, more than 1024 units
(rank, request) in one call, unit counts on both sides of each size of the
work plan's workgroup (64 / 65, 256 / 257), and verification rows
whose causal limit falls before position 0 (they see nothing: lse = -inf,
o = 0, on every rank and after the merge); a zero and a negative softmax
scale; e4m3 with base-2 LSE.  Sixty-four seeded random shapes draw heads,
query rows, group size, page size, interleave, dtype, LSE base, causality
and ragged lengths together.  Each compares every request's merged output
and every rank's partial with the oracle at the stated tolerances.  Repeated
calls are bitwise stable, two calls in flight on two streams at once give
what they give alone, and lengths, table sizes and page ids that only the
device can see to be wrong are reported with their codes while the other
requests stay right.
"""
import numpy as np
import pytest
import torch

from parity import Case, check_case, log
from workloads import configs as C

pytestmark = pytest.mark.gpu


def W(**kw):
    base = dict(name="t", index=50, B=1, H=16, q_len=1, c=4, P=16, kv_dtype="bf16", lse_base="e", fixed_len=64)
    base.update(kw)
    return C.Workload(**base)


def _ragged(n, seed, long):
    """n short request lengths in [0, 400) (seeded) with a few long ones."""
    lens = [int(x) for x in np.random.default_rng(seed).integers(0, 400, n)]
    for b, L in long.items():
        lens[b] = L
    return lens


CASES = [
    ("tiny", C.TINY, None),
    ("c1_ragged_tail", W(index=51, c=1, P=16, fixed_len=100), None),
    ("empty_shards", W(index=52, c=8, P=16, fixed_len=5), None),
    ("zero_len_request", W(index=53, B=3, c=4, P=64), [0, 77, 300]),
    ("h32", W(index=54, H=32, c=2, P=64, fixed_len=500), None),
    ("h64", W(index=55, H=64, c=4, P=64, fixed_len=777), None),
    ("h128_two_blocks", W(index=56, H=128, c=2, P=64, fixed_len=300, B=2), None),
    # 64-row bf16 blocks (16 waves) on pages a stage can straddle, with a split unit
    ("h128_page16_splits", W(index=76, H=128, c=2, P=16, B=2), [20000, 333]),
    ("verify_h16_q4", W(index=57, H=16, q_len=4, c=4, P=64, fixed_len=203, B=2), None),
    ("verify_h128_q4", W(index=58, H=128, q_len=4, c=4, P=64, fixed_len=130), None),
    ("noncausal_q2", W(index=59, H=32, q_len=2, c=3, P=32, fixed_len=90, causal=False), None),
    ("base2", W(index=60, H=16, c=8, P=64, fixed_len=1000, lse_base="2", B=2), None),
    ("page_not_stage_aligned", W(index=61, H=16, c=3, P=48, fixed_len=700), None),
    ("page_1", W(index=62, H=16, c=2, P=1, fixed_len=70), None),
    ("splits_long", W(index=63, H=16, c=1, P=64, fixed_len=20000), None),
    ("splits_ragged_batch", W(index=64, H=64, c=2, P=64, B=3), [9000, 1, 4444]),
    ("fp8_h64", W(index=65, H=64, c=8, P=64, fixed_len=3000, kv_dtype="fp8"), None),
    ("fp8_h16_unaligned", W(index=66, H=16, c=2, P=16, fixed_len=333, kv_dtype="fp8"), None),
    ("fp8_verify", W(index=67, H=32, q_len=4, c=4, P=64, fixed_len=1500, kv_dtype="fp8", B=2), None),
    ("fp8_splits", W(index=68, H=64, c=1, P=64, fixed_len=40000, kv_dtype="fp8"), None),
    ("fp8_one_to_four_stages", W(index=72, H=32, c=1, P=64, B=5, kv_dtype="fp8"), [1, 40, 70, 100, 128]),
    ("fp8_empty_shards", W(index=73, H=64, c=8, P=16, fixed_len=5, kv_dtype="fp8"), None),
    # the largest verification step (q_len 8), many heads, a wide group, large pages
    ("verify_q8_h32", W(index=91, H=32, q_len=8, c=4, P=64, fixed_len=1000, B=2), None),
    ("fp8_verify_q8_h16", W(index=92, H=16, q_len=8, c=2, P=32, fixed_len=333, kv_dtype="fp8"), None),
    ("h256_q1", W(index=93, H=256, c=2, P=64, fixed_len=900), None),
    ("c16_wide_group", W(index=94, H=16, c=16, P=16, fixed_len=1500, B=2), None),
    ("page_256", W(index=95, H=64, c=4, P=256, fixed_len=3000), None),
    ("verify_q8_shorter_than_q_len", W(index=96, H=16, q_len=8, c=4, P=16, B=3), [1, 5, 8]),
    # degenerate scales: a zero scale gives uniform weights (o = mean of the
    # visible V rows, lse = ln n), a negative one favours the lowest scores
    ("zero_scale", W(index=97, H=32, q_len=2, c=4, P=16, fixed_len=500, sm_scale=0.0), None),
    ("negative_scale", W(index=98, H=16, c=3, P=32, fixed_len=400, sm_scale=-C.SM_SCALE), None),
    ("fp8_base2", W(index=99, H=64, c=4, P=64, fixed_len=2000, kv_dtype="fp8", lse_base="2"), None),
    # interleave size I > 1: owners take runs of I consecutive positions
    ("il16_h64", W(index=80, H=64, c=4, P=64, fixed_len=777, interleave=16), None),
    ("il64_two_owners_of_eight", W(index=81, H=32, c=8, P=64, fixed_len=100, interleave=64), None),
    ("il8_verify_q4", W(index=82, H=16, q_len=4, c=3, P=32, fixed_len=203, B=2, interleave=8), None),
    ("il4_noncausal_q2", W(index=83, H=32, q_len=2, c=3, P=32, fixed_len=90, causal=False, interleave=4), None),
    ("il32_splits", W(index=84, H=16, c=2, P=64, fixed_len=20000, interleave=32), None),
    ("il8_ragged_batch", W(index=85, H=64, c=4, P=16, B=4, interleave=8), [1, 9, 500, 3001]),
    ("il3_page48", W(index=86, H=16, c=3, P=48, fixed_len=700, interleave=3), None),
    ("il16_h128_two_blocks", W(index=90, H=128, c=2, P=64, fixed_len=300, B=2, interleave=16), None),
    ("fp8_il16", W(index=87, H=64, c=8, P=64, fixed_len=3000, kv_dtype="fp8", interleave=16), None),
    ("fp8_il64_verify", W(index=88, H=32, q_len=4, c=4, P=64, fixed_len=1500, kv_dtype="fp8", B=2,
                          interleave=64), None),
    ("fp8_il8_short", W(index=89, H=16, c=8, P=16, fixed_len=37, kv_dtype="fp8", interleave=8), None),
    # the work plan over more than 1024 units (several 1024-unit chunks, split
    # units in both) and at exactly 1024 ragged units (longest-first order of
    # the single-item units)
    ("units_over_1024", W(index=74, H=16, c=4, P=16, B=260), _ragged(260, 7, {3: 12000, 130: 8000, 259: 12000})),
    ("units_1024_ragged", W(index=75, H=16, c=8, P=16, B=128), _ragged(128, 8, {0: 30000, 77: 9000})),
    # the plan's workgroup is sized to the units (64, 256 or 1024 threads):
    # ragged batches on both sides of each size, one of them with 64-row blocks
    ("plan_64_units", W(index=101, H=16, c=4, P=16, B=16), _ragged(16, 9, {2: 6000})),
    ("plan_65_units", W(index=102, H=16, c=5, P=16, B=13), _ragged(13, 10, {0: 5000})),
    ("plan_65_units_h128", W(index=105, H=128, c=5, P=64, B=13), _ragged(13, 13, {4: 4000})),
    ("plan_256_units", W(index=103, H=16, c=8, P=16, B=32), _ragged(32, 11, {5: 9000, 31: 4000})),
    ("plan_257_units", W(index=104, H=16, c=1, P=16, B=257), _ragged(257, 12, {100: 7000})),
]


@pytest.mark.parametrize("name,w,lens", CASES, ids=[c[0] for c in CASES])
def test_decode_parity_small(name, w, lens):
    log(f"case {name}: {w}")
    case = Case(w, lens=lens)
    check_case(case)


def test_needles_dominate():
    # planted keys aligned with a head's query make a few weights O(1): the output is
    # far from the Gaussian limit and still matches the oracle
    from workloads import gen
    w = W(index=69, H=64, c=4, P=64, fixed_len=4000, B=2)
    q = gen.q_bits(w)
    needles = {b: gen.needle_rows(w, q, b, 4000, count=4, gain=0.6) for b in range(w.B)}
    case = Case(w, needles=needles)
    o_part, lse_part, o, lse = check_case(case)
    assert np.abs(o).max() > 0.5


def test_repeat_runs_bitwise_stable():
    w = W(index=70, H=64, c=4, P=64, fixed_len=2000, B=2)
    case = Case(w)
    a = case.run()
    b = case.run()
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("kv,H", [("bf16", 16), ("bf16", 64), ("fp8", 64)])
def test_decode_pages_beyond_4gib(kv, H):
    # Regression: the 64-bit page base of the direct-to-LDS loads once picked up a
    # sign-extended low word.  Four owner pools of about 1.25 GiB each, with an identity
    # free stack handing out the highest page ids first, put the pages in use about
    # 1.25 GiB apart across 5 GiB: whatever the allocation base, some of them have bit
    # 31 of the low address word set.
    row = 1152 if kv == "bf16" else 576
    pages = (5 << 30) // (64 * row * 4) + 1
    w = W(index=71, H=H, c=4, P=64, fixed_len=3000, B=2, kv_dtype=kv)
    case = Case(w, seed_free_stack=False, num_pages=pages)
    bt = case.group.block_table.cpu().numpy()
    assert bt[bt >= 0].min() * 64 * row > (1 << 30)
    check_case(case)


def _scale_q_rows(case, exps):
    """Multiply each query row r by 2**exps[r % len(exps)] (exact in bf16)."""
    qb = case.q_bits
    f = (qb.astype(np.uint32) << 16).view(np.float32).reshape(qb.shape)
    rows = f.reshape(f.shape[0], -1, f.shape[-1])
    for r in range(rows.shape[1]):
        rows[:, r, :] *= np.float32(2.0 ** exps[r % len(exps)])
    case.q_bits = (rows.reshape(qb.shape).view(np.uint32) >> 16).astype(np.uint16)
    assert np.isfinite(rows).all()
    case.q = __import__("torch").from_numpy(case.q_bits.view(np.int16)).to("cuda")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("k", [-40, 40])
def test_query_magnitudes_far_from_one(kv, k):
    # a q 2^k times larger, with a softmax scale 2^-k times smaller, is the
    # same attention; scores and the running maximum must not lose it
    w = W(index=74, H=64, c=4, P=64, fixed_len=700, B=2, kv_dtype=kv, sm_scale=C.SM_SCALE * 2.0 ** (-k))
    case = Case(w)
    _scale_q_rows(case, [k])
    log(f"{kv}: q scaled by 2^{k}")
    check_case(case)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_query_rows_of_different_magnitudes(kv):
    # rows 2^-4 .. 2^4 apart in one 16-row block (sharp and flat softmax side
    # by side).  The score arithmetic is held to the stated lse tolerance.  A
    # sharp row makes o close to a single V row (|o| up to ~4 here).  bf16
    # rounding to nearest even has a relative error of at most 2^-8, and o
    # goes through one such rounding in the fp32 partials (the bf16 P of the
    # PV product: at most 2^-8 sum_j p_j |v_j| / l, which is |o| for a sharp
    # row) and a second one in the merged bf16 output.  Either can exceed the
    # absolute 1e-2, so o is held to max(stated tolerance, 2^-8 max|o|) in the
    # partials and max(stated tolerance, 2^-7 max|o|) after the merge.
    from parity import TOL
    w = W(index=75, H=64, c=2, P=64, fixed_len=500, B=2, kv_dtype=kv)
    case = Case(w)
    _scale_q_rows(case, [-4, -3, -2, -1, 0, 1, 2, 3, 4])
    o_part, lse_part, o, lse = case.run()
    to, tl = TOL[kv]
    for b in range(w.B):
        ro, rl, rop, rlp = case.oracle(b)
        for name, got_o, got_l, ref_o, ref_l in (("merged", o[b], lse[b], ro, rl), ("partials", o_part[:, b], lse_part[:, b], rop, rlp)):
            fin = ~np.isneginf(ref_l)
            assert np.array_equal(fin, ~np.isneginf(got_l)), name
            dl = float(np.abs(got_l[fin] - ref_l[fin]).max())
            do = float(np.abs(got_o - ref_o).max())
            bound = max(to, 2.0 ** (-7 if name == "merged" else -8) * float(np.abs(ref_o).max()))
            log(f"{kv} b={b} {name}: max|do|={do:.3e} (bound {bound:.3e}) max|dlse|={dl:.3e} (tol {tl})")
            assert dl <= tl and do <= bound, (name, do, bound, dl)


# One real rank's call: rank_begin = r, rank_count = 1 on that rank's own pool (and
# sub-ranges of the emulated group).  The kernel judges visibility with the global
# rank r but reads pool, scales and outputs at the local index; every rank's
# partial must still be the oracle's striped partial of rank r (SGLang page,
# "MLA decode dataflow": each rank returns its own o_r, lse_r).
RANK_CASES = [
    # name, workload, lengths, short (single launch, no work plan)
    ("bf16_direct", W(index=100, H=64, c=4, P=64, fixed_len=900, B=3), None, True),
    ("bf16_split", W(index=101, H=64, c=8, P=64, fixed_len=30000, B=2), None, False),
    ("fp8_direct", W(index=102, H=64, c=8, P=64, fixed_len=1500, kv_dtype="fp8", B=2), None, True),
    ("fp8_split", W(index=103, H=64, c=4, P=64, fixed_len=40000, kv_dtype="fp8"), None, False),
    ("il16_verify_q4", W(index=104, H=16, q_len=4, c=8, P=64, fixed_len=1777, B=2, interleave=16), None, True),
    ("il16_verify_q4_split", W(index=105, H=16, q_len=4, c=8, P=64, fixed_len=25000, interleave=16), None, False),
    ("h128_verify_ragged", W(index=106, H=128, q_len=4, c=6, P=32, B=3), [700, 9000, 5], False),
]


@pytest.mark.parametrize("name,w,lens,short", RANK_CASES, ids=[c[0] for c in RANK_CASES])
def test_rank_subset_calls(name, w, lens, short):
    from kv_sharded_mla_amd import LSE_BASE_2, LSE_BASE_E
    from parity import compare
    case = Case(w, lens=lens)
    o_full, l_full, _, _ = case.run()
    base = LSE_BASE_2 if w.lse_base == "2" else LSE_BASE_E
    ranges = [(1, 1), (w.c - 1, 1), (0, 1)] + ([(2, 3)] if w.c >= 5 else [])
    refs = [case.oracle(b) for b in range(w.B)]
    for rb, rc in ranges:
        o_p, l_p = case.group.decode(case.q, w.sm_scale, base, w.causal, rank_begin=rb, rank_count=rc)
        import torch
        torch.cuda.synchronize()
        assert case.group.status() == 0
        o_p, l_p = o_p.cpu().numpy(), l_p.cpu().numpy()
        assert o_p.shape[0] == rc
        for b in range(w.B):
            _, _, rop, rlp = refs[b]
            compare(f"{name} ranks [{rb}, {rb + rc}) b={b}", o_p[:, b], l_p[:, b], rop[rb:rb + rc], rlp[rb:rb + rc],
                    w.kv_dtype, partial=True)
        if short:
            # without a work plan every (rank, request) is one workgroup doing the same
            # arithmetic in either call: bit for bit
            assert np.array_equal(o_p.view(np.uint32), o_full[rb:rb + rc].view(np.uint32))
            assert np.array_equal(l_p.view(np.uint32), l_full[rb:rb + rc].view(np.uint32))


@pytest.mark.parametrize("fill", ["all_bits_set", "random_bytes"])
def test_workspace_contents_do_not_matter(fill):
    # Every call writes the workspace parts it reads (work plan, split
    # partials): a workspace left full of other data (every bit set, or random
    # bytes) gives the outputs of a zeroed one, bit for bit, on each of several
    # calls in a row, and those match the oracle.  Ragged lengths (split and
    # single-item units, an empty rank) and 64-row blocks (two per request)
    # on bf16 and e4m3.
    import torch
    from kv_sharded_mla_amd import LSE_BASE_E
    for kv in ("bf16", "fp8"):
        w = W(index=110, H=128, c=4, P=64, B=3, kv_dtype=kv)
        case = Case(w, lens=[30000, 9000, 3])
        ws0 = case.group.workspace_for(w.q_len, w.H)
        ws0.zero_()
        ref_o, ref_l = case.group.decode(case.q, w.sm_scale, LSE_BASE_E, w.causal, workspace=ws0)
        ref_o, ref_l = ref_o.clone(), ref_l.clone()
        ws = torch.empty_like(ws0)
        if fill == "all_bits_set":
            ws.view(torch.int32).fill_(-1)
        else:
            g = torch.Generator(device="cuda").manual_seed(7)
            ws.view(torch.int32).copy_(torch.randint(-2**31, 2**31 - 1, ws.shape, generator=g, device="cuda",
                                                     dtype=torch.int64).to(torch.int32))
        for k in range(3):
            o, l = case.group.decode(case.q, w.sm_scale, LSE_BASE_E, w.causal, workspace=ws)
            torch.cuda.synchronize()
            log(f"{kv} {fill} call {k}: identical={bool(torch.equal(o, ref_o) and torch.equal(l, ref_l))}")
            assert torch.equal(o, ref_o) and torch.equal(l, ref_l), (kv, fill, k)
        assert case.group.status() == 0
        check_case(case)


def _random_case(seed):
    """A seeded random decode shape: heads, query rows, group size, page size,
    interleave, dtype, LSE base, causality and ragged lengths (some long enough
    to split) drawn together, the oracle's work kept to a few seconds."""
    rng = np.random.default_rng(1000 + seed)
    H = int(rng.choice([16, 32, 64, 128]))
    q_len = int(rng.choice([1, 1, 2, 4]))
    c = int(rng.choice([1, 2, 3, 4, 8]))
    P = int(rng.choice([1, 16, 32, 48, 64]))
    il = int(rng.choice([d for d in (1, 1, 2, 4, 8, 16) if P % d == 0]))
    kv = str(rng.choice(["bf16", "fp8"]))
    B = int(rng.integers(1, 4))
    budget = 3_000_000 // (H * q_len)          # sum of lengths the oracle does in seconds
    lens = [int(x) for x in rng.integers(0, max(2, min(3000, budget // B)), B)]
    if rng.random() < 0.5:                     # one request long enough for a split
        lens[int(rng.integers(0, B))] = int(min(budget, rng.integers(6000, 12000)))
    w = W(index=200 + seed, B=B, H=H, q_len=q_len, c=c, P=P, kv_dtype=kv, interleave=il,
          lse_base=str(rng.choice(["e", "2"])), causal=bool(rng.random() < 0.8), fixed_len=None)
    return w, lens


@pytest.mark.parametrize("seed", range(64))
def test_decode_random_shapes(seed):
    w, lens = _random_case(seed)
    log(f"random case {seed}: {w} lens {lens}")
    check_case(Case(w, lens=lens))


def test_two_streams_at_once():
    # two calls with their own workspaces in flight on two streams at once give
    # what they give alone: no state is shared between calls beyond their arguments
    from kv_sharded_mla_amd import LSE_BASE_E
    cases = [Case(W(index=126, H=128, c=4, P=64, B=3), lens=[20000, 300, 7000]),
             Case(W(index=127, H=64, c=8, P=64, B=2, kv_dtype="fp8"), lens=[30000, 5000])]
    alone = []
    for case in cases:
        o, l = case.group.decode(case.q, case.w.sm_scale, LSE_BASE_E, case.w.causal)
        torch.cuda.synchronize()
        alone.append((o.cpu().numpy(), l.cpu().numpy()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    for case, s in zip(cases, streams):
        with torch.cuda.stream(s):
            ws = case.group.workspace_for(case.w.q_len, case.w.H)
            outs.append(case.group.decode(case.q, case.w.sm_scale, LSE_BASE_E, case.w.causal, workspace=ws))
    torch.cuda.synchronize()
    for case, (o, l), (ro, rl) in zip(cases, outs, alone):
        assert np.array_equal(o.cpu().numpy().view(np.uint32), ro.view(np.uint32)), case.w
        assert np.array_equal(l.cpu().numpy().view(np.uint32), rl.view(np.uint32)), case.w
        assert case.group.status() == 0
    log("two streams at once: both calls bit-identical to their calls alone")


def _decode_raw(case, seq_len, max_seq_len, block_table):
    """One call with the given lengths, bound and table; returns outputs and the status code."""
    import kv_sharded_mla_amd as K
    w, g = case.w, case.group
    o = torch.full((w.c, w.B, w.q_len, w.H, K.D_V), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.c, w.B, w.q_len, w.H), float("nan"), dtype=torch.float32, device="cuda")
    n = K.mla_decode_workspace_size(g.layout, w.c, w.B, w.q_len, w.H, max_seq_len)
    ws = torch.empty(max(n // 4, 4), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.mla_decode_partial(g.layout, g.pools, g.pool_scales, 0, w.c, case.q, block_table, seq_len, max_seq_len,
                         w.sm_scale, K.LSE_BASE_E, w.causal, o, lse, ws, status)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("kind", ["bad_length", "table_overflow", "bad_page"])
def test_decode_reports_bad_arguments_on_the_device(kind):
    # Conditions only the device can see, forced from the host: a request longer
    # than max_seq_len, one that needs more block-table columns than bt_stride,
    # a block-table entry outside the pool.  The call reports the documented
    # code; a request whose length it cannot take decodes as empty (lse = -inf,
    # o = 0 on every rank), a bad page id reads page 0 instead (values
    # unspecified, no access outside the pool), and the other requests are
    # still right.
    from parity import compare
    import kv_sharded_mla_amd as K
    w = W(index=128, H=16, c=4, P=16, B=3)
    lens = [500, 300, 2000]
    case = Case(w, lens=lens)
    g = case.group
    seq = g.seq_len.clone()
    bt = g.block_table.clone()
    max_len = g.max_seq_len
    bad = 2
    if kind == "bad_length":
        max_len = 600                       # request 2 (2000) exceeds the bound
        want = K.DEV_BAD_LENGTH
    elif kind == "table_overflow":
        bt = bt[:, :10].contiguous()        # 10 virtual pages of 64: 640 tokens; request 2 needs 32
        want = K.DEV_TABLE_OVERFLOW
    else:
        bt[bad, 3] = g.num_pages + 5        # one page of request 2 outside the pool
        want = K.DEV_BAD_PAGE
    o, lse, st = _decode_raw(case, seq, max_len, bt)
    assert st == want, (kind, st)
    for b in range(w.B):
        if b == bad and kind != "bad_page":
            assert np.isneginf(lse[:, b]).all() and not o[:, b].any(), kind
            continue
        if b == bad:
            continue
        _, _, rop, rlp = case.oracle(b)
        compare(f"{kind} b={b}", o[:, b], lse[:, b], rop, rlp, w.kv_dtype, partial=True)
    log(f"{kind}: status {st}, the other requests right")
