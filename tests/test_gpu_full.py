"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Every workload's whole batch is written by one dcp_alloc_virtual +
dcp_kv_write call and decoded by one mla_decode_partial call over all c
emulated ranks (the same work plan and kernels as the benchmark), then merged
by dcp_lse_merge.  Checked against the oracle on the generator's host rows:

* the integer path: the block table and every row's slot bit-exact against
  the layout model, every row's bytes (and e4m3 scale) at its slot, and every
  other slot still holding the sentinel;
* every (request, rank) partial against the oracle's attention over that
  rank's striped positions;
* every merged row against the oracle's merge of its partials, which equals
  full attention over the request (pinned on the CPU for every c);
* full attention computed directly over the whole request for sampled
  requests, one of the 1,048,576-token requests included;
* one real rank's call (rank_begin = r, rank_count = 1) for the first and the
  last rank against the same oracle partials.

With ``needles`` the sampled requests carry a few planted keys aligned with one
head's query, so that some outputs are O(1) instead of near the Gaussian limit
sm_scale * q[:512].
"""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import layout as OL
from parity import Case, compare, log
from workloads import configs as C
from workloads import gen

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5
# workload -> requests whose full attention is also computed directly
DIRECT = {"tiny": "0", "tplocal": "0,31,63", "replq": "longest,shortest", "verify": "0,15", "long": "2"}


def _pick(spec, lens):
    out = []
    for tok in spec.split(","):
        out.append(int(np.argmax(lens)) if tok == "longest" else int(np.argmin(lens)) if tok == "shortest"
                   else int(tok))
    return out


def _check_layout(case):
    """Block table, slots and pool bytes of the bulk write against the layout model."""
    w, g = case.w, case.group
    vp = w.P * w.c
    B = w.B
    stack = gen.free_stack(w, case.num_pages)
    st, top, bt = OL.alloc_virtual(stack, case.num_pages, [0] * B, case.lens,
                                   np.full((B, case.bt_stride), -1, np.int32), w.P, w.c)
    assert st == OL.OK
    assert np.array_equal(g.block_table.cpu().numpy(), bt)
    assert int(g.free_top.item()) == top
    cu = np.concatenate([[0], np.cumsum(case.lens)])
    st, own, phys = OL.write_slots(bt, case.lens, cu, w.P, w.c, case.num_pages, w.interleave)
    assert st == OL.OK
    cap = case.num_pages * w.P
    assert np.array_equal(case.slots.cpu().numpy(), own * cap + phys)
    data, scale = case.rows
    rb = g.row_bytes
    pools = g.pools.view(w.c * cap, rb)
    flat = torch.from_numpy(own * cap + phys).to("cuda")
    host = data.view(np.uint8).reshape(len(data), rb)
    step = 1 << 20
    for a in range(0, len(flat), step):
        got = pools[flat[a:a + step]].cpu().numpy()
        assert np.array_equal(got, host[a:a + step]), f"row bytes differ in rows {a}..{a + step}"
        if scale is not None:
            gs = g.pool_scales[flat[a:a + step]].cpu().numpy()
            assert np.array_equal(gs.view(np.uint32), scale[a:a + step].view(np.uint32))
    # nothing else written: every other slot keeps the sentinel (a random row equal to
    # the sentinel in every byte has probability 2^-4608)
    touched = 0
    for a in range(0, w.c * cap, step):
        touched += int((pools[a:a + step] != SENTINEL).any(dim=1).sum().item())
    assert touched == len(flat)
    if scale is not None:
        assert int(torch.isnan(g.pool_scales).logical_not().sum().item()) == len(flat)
    log(f"{w.name}: block table, {len(flat)} slots and row bytes exact; other slots untouched")


@pytest.mark.parametrize("name", ["tiny", "tplocal", "replq", "verify", "long"])
def test_full_size_every_request_and_rank(name):
    from kv_sharded_mla_amd import LSE_BASE_2, LSE_BASE_E
    w = C.BY_NAME[name]
    log(f"full-size {name}: B={w.B} H={w.H} q_len={w.q_len} c={w.c} kv={w.kv_dtype}")
    case = Case(w, keep_rows=True, keep_slots=True, sentinel=SENTINEL)
    _check_layout(case)
    o_part, lse_part, o, lse = case.run()
    log(f"{name}: decoded {int(case.lens.sum())} tokens")
    base = LSE_BASE_2 if w.lse_base == "2" else LSE_BASE_E
    share = {}
    for r in sorted({0, w.c - 1}):
        op, lp = case.group.decode(case.q, w.sm_scale, base, w.causal, rank_begin=r, rank_count=1)
        share[r] = (op.cpu().numpy()[0], lp.cpu().numpy()[0])
    torch.cuda.synchronize()
    assert case.group.status() == 0
    direct = _pick(DIRECT[name], case.lens)
    for b in range(w.B):
        L = int(case.lens[b])
        kv = case.kv_host(b)
        rop, rlp = OA.rank_partials(case.q_bits[b], kv, L, w.sm_scale, w.c, w.causal, w.lse_base, I=w.interleave)
        compare(f"{name} b={b} (L={L}) partials of all {w.c} ranks", o_part[:, b], lse_part[:, b], rop, rlp,
                w.kv_dtype, partial=True)
        for r, (op, lp) in share.items():
            compare(f"{name} b={b} rank {r} alone", op[b], lp[b], rop[r], rlp[r], w.kv_dtype, partial=True)
        ro, rl = OA.merge(rop, rlp, w.lse_base)
        compare(f"{name} b={b} merged vs merge of the oracle partials", o[b], lse[b], ro, rl, w.kv_dtype)
        if b in direct:
            fo, fl = OA.decode_attention(case.q_bits[b], kv, L, w.sm_scale, w.causal, w.lse_base)
            compare(f"{name} b={b} merged vs full attention", o[b], lse[b], fo, fl, w.kv_dtype)


@pytest.mark.parametrize("name", ["tplocal", "replq", "verify", "long"])
def test_full_size_needles(name):
    w = C.BY_NAME[name]
    lens = gen.lengths(w)
    qb = gen.q_bits(w)
    picked = _pick(DIRECT[name], lens)
    planted = {b: gen.needle_rows(w, qb, b, int(lens[b]), count=4, gain=0.6) for b in picked}
    log(f"full-size {name} with needles in requests {picked}")
    case = Case(w, keep_rows=True, needles=planted)
    o_part, lse_part, o, lse = case.run()
    for b in picked:
        assert np.abs(o[b]).max() > 0.5, (b, float(np.abs(o[b]).max()))
        L = int(case.lens[b])
        kv = case.kv_host(b)
        rop, rlp = OA.rank_partials(case.q_bits[b], kv, L, w.sm_scale, w.c, w.causal, w.lse_base, I=w.interleave)
        compare(f"{name} b={b} needles: partials", o_part[:, b], lse_part[:, b], rop, rlp, w.kv_dtype, partial=True)
        ro, rl = OA.merge(rop, rlp, w.lse_base)
        compare(f"{name} b={b} needles: merged", o[b], lse[b], ro, rl, w.kv_dtype)
