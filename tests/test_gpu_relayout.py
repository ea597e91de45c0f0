"""GPU parity of the extend gather (dcp_kv_read) and the DCP1 -> DCP c relayout
(dcp_kv_relayout), bit-exact.

Expected bytes come from oracle.layout.read_rows / relayout_dense on the same
seeded inputs; the full-size case checks a round trip (relayout, then gather
back to token order) on the 16-head workload's shape and samples positions
against the oracle's slot map.
"""
import numpy as np
import pytest
import torch

from oracle import layout as OL
from parity import log

pytestmark = pytest.mark.gpu


def _lib():
    import kv_sharded_mla_amd as K
    K.load_library()
    return K


def _t(a, dtype=torch.int32):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype)


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to("cuda")


def _striped(rng, interleaved, kv, max_len=900):
    c = int(rng.integers(1, 9))
    P = int(rng.choice([4, 12, 16, 64] if interleaved else [1, 3, 16, 64]))
    I = int(rng.choice([d for d in range(2, P + 1) if P % d == 0])) if interleaved else 1
    B = int(rng.integers(1, 7))
    lens = rng.integers(0, max_len, size=B)
    if B > 2:
        lens[1] = 0
    vp = P * c
    num_pages = int(sum((L + vp - 1) // vp for L in lens)) + 2
    stride = int(max((L + vp - 1) // vp for L in lens)) + 1
    st, _, bt = OL.alloc_virtual(rng.permutation(num_pages).astype(np.int32), num_pages, np.zeros(B, np.int64),
                                 lens, np.full((B, stride), -1, np.int32), P, c)
    assert st == OL.OK
    row_bytes = 576 if kv == "fp8" else 1152
    return c, P, I, lens, num_pages, bt, row_bytes


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("interleaved", [False, True])
def test_kv_read_token_order_exact(kv, seed, interleaved):
    K = _lib()
    rng = np.random.default_rng(300 + seed + 50 * interleaved)
    c, P, I, lens, num_pages, bt, rb = _striped(rng, interleaved, kv)
    fp8 = kv == "fp8"
    pools = rng.integers(0, 256, size=(c, num_pages * P, rb), dtype=np.uint8)
    pscales = rng.standard_normal((c, num_pages * P)).astype(np.float32) if fp8 else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n_rows = int(cu[-1]) + 3                      # rows past the last request stay untouched
    out0 = np.full((n_rows, rb), 0xEE, np.uint8)
    sc0 = np.full(n_rows, -7.0, np.float32) if fp8 else None
    st, want, want_sc = OL.read_rows(pools, bt, lens, cu, P, c, I, pool_scales=pscales, out=out0, out_scales=sc0)
    assert st == OL.OK
    layout = K.make_layout(c, P, num_pages, K.KV_FP8_E4M3 if fp8 else K.KV_BF16, I)
    d_out = _u8(out0).view(n_rows, rb)
    d_sc = _t(sc0, torch.float32) if fp8 else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.dcp_kv_read(layout, _u8(pools), _t(pscales, torch.float32) if fp8 else None, _t(bt), _t(lens), _t(cu),
                  d_out, d_sc, status)
    assert int(status.item()) == 0
    assert np.array_equal(d_out.cpu().numpy(), want)
    if fp8:
        assert np.array_equal(d_sc.cpu().numpy().view(np.uint32), want_sc.view(np.uint32))
    log(f"kv_read {kv} seed={seed} c={c} P={P} I={I} lens={list(lens)} ok")


def test_kv_read_errors_skip_and_report():
    K = _lib()
    c, P = 2, 2
    bt = np.array([[0, 1, -1], [1, -1, -1], [5, 0, -1]], np.int32)
    pools = np.arange(c * 2 * P * 1152, dtype=np.uint32).astype(np.uint8).reshape(c, 2 * P, 1152)
    layout = K.make_layout(c, P, 2, K.KV_BF16)
    for lens, cu, n_rows in [([5, 2, 0], [0, 5, 8, 8], 8),       # span of request 1 != its length
                             ([5, 2, 0], [0, 5, 7, 7], 6),       # span of request 1 leaves the output
                             ([13, 0, 0], [0, 13, 13, 13], 13),  # 13 tokens need 4 virtual pages > 3
                             ([0, 0, 6], [0, 0, 0, 6], 6)]:      # page id 5 is outside a 2-page pool
        out0 = np.full((n_rows, 1152), 0xEE, np.uint8)
        st, want, _ = OL.read_rows(pools, bt, lens, cu, P, c, out=out0)
        assert st != OL.OK
        d_out = _u8(out0).view(n_rows, 1152)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        K.dcp_kv_read(layout, _u8(pools), None, _t(bt), _t(lens), _t(cu), d_out, None, status)
        assert int(status.item()) == st, (lens, cu)
        assert np.array_equal(d_out.cpu().numpy(), want)


def _dense(rng, lens, P, rb, fp8):
    n_src = int(sum((L + P - 1) // P for L in lens)) + 1
    s_stride = max(1, int(max((L + P - 1) // P for L in lens)))
    src_bt = np.full((len(lens), s_stride), -1, np.int32)
    ids = rng.permutation(n_src)
    k = 0
    for b, L in enumerate(lens):
        for q in range((L + P - 1) // P):
            src_bt[b, q] = ids[k]
            k += 1
    src = rng.integers(0, 256, size=(n_src * P, rb), dtype=np.uint8)
    ssc = rng.standard_normal(n_src * P).astype(np.float32) if fp8 else None
    return src, ssc, src_bt


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("interleaved", [False, True])
def test_kv_relayout_exact(kv, seed, interleaved):
    K = _lib()
    rng = np.random.default_rng(400 + seed + 50 * interleaved)
    c, P, I, lens, num_pages, bt, rb = _striped(rng, interleaved, kv)
    fp8 = kv == "fp8"
    src, ssc, src_bt = _dense(rng, lens, P, rb, fp8)
    dst0 = rng.integers(0, 256, size=(c, num_pages * P, rb), dtype=np.uint8)   # old bytes must survive
    dsc0 = rng.standard_normal((c, num_pages * P)).astype(np.float32) if fp8 else None
    layout = K.make_layout(c, P, num_pages, K.KV_FP8_E4M3 if fp8 else K.KV_BF16, I)
    pool_bytes = num_pages * P * rb
    r1 = int(rng.integers(0, c))
    for rank_begin, rank_count in [(0, c), (r1, 1)]:
        st, want, want_sc = OL.relayout_dense(src, src_bt, lens, P, c, dst0, bt, rank_begin, rank_count, I,
                                              src_scales=ssc, dst_scales=dsc0)
        assert st == OL.OK
        d_pools = _u8(dst0)
        d_psc = _t(dsc0, torch.float32).reshape(-1) if fp8 else None
        sl = slice(rank_begin * pool_bytes, (rank_begin + rank_count) * pool_bytes)
        ssl = slice(rank_begin * num_pages * P, (rank_begin + rank_count) * num_pages * P)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        K.dcp_kv_relayout(layout, _u8(src), _t(ssc, torch.float32) if fp8 else None, _t(src_bt), _t(lens),
                          rank_begin, rank_count, d_pools[sl], d_psc[ssl] if fp8 else None, _t(bt), status)
        assert int(status.item()) == 0
        assert np.array_equal(d_pools.cpu().numpy().reshape(c, num_pages * P, rb), want)
        if fp8:
            assert np.array_equal(d_psc.cpu().numpy().reshape(c, -1).view(np.uint32), want_sc.view(np.uint32))
    log(f"kv_relayout {kv} seed={seed} c={c} P={P} I={I} lens={list(lens)} ranks (0,{c}) and ({r1},1) ok")


def test_kv_relayout_errors_skip_and_report():
    K = _lib()
    c, P, I = 2, 4, 4
    lens = np.array([16])
    rng = np.random.default_rng(5)
    src, _, src_bt = _dense(rng, lens, P, 1152, False)
    bt = np.array([[0, 1]], np.int32)
    dst0 = np.full((c, 2 * P, 1152), 0xEE, np.uint8)
    layout = K.make_layout(c, P, 2, K.KV_BF16, I)
    bad = src_bt.copy()
    bad[0, 1] = 99                      # positions 4..7, owned by rank 1 at I = P
    cases = [(np.array([-1]), src_bt, bt, 0, c), (lens, src_bt[:, :2], bt, 0, c), (lens, src_bt, bt[:, :1], 0, c),
             (lens, bad, bt, 0, c), (lens, bad, bt, 0, 1), (lens, src_bt, np.array([[0, 7]], np.int32), 0, c)]
    for ln, sbt, dbt, r0, rc in cases:
        st, want, _ = OL.relayout_dense(src, sbt, ln, P, c, dst0, dbt, r0, rc, I)
        d_pools = _u8(dst0)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        pb = 2 * P * 1152
        K.dcp_kv_relayout(layout, _u8(src), None, _t(sbt), _t(ln), r0, rc, d_pools[r0 * pb:(r0 + rc) * pb], None,
                          _t(dbt), status)
        assert int(status.item()) == st, (ln, r0, rc)
        assert np.array_equal(d_pools.cpu().numpy().reshape(c, 2 * P, 1152), want)


@pytest.mark.parametrize("name", ["tplocal", "long"])
def test_relayout_then_read_round_trip_full_size(name):
    """Full workload shapes: 64 requests of 32768 tokens (c = 8, P = 64, bf16 rows) and 4
    requests of 1,048,576 tokens (c = 8, P = 64, e4m3 rows with their scales)."""
    K = _lib()
    from workloads import configs as C, gen
    w = C.BY_NAME[name]
    fp8 = w.kv_dtype == "fp8"
    rb = 576 if fp8 else 1152
    lens = gen.lengths(w)
    B, P, c = w.B, w.P, w.c
    rng = np.random.default_rng(11)
    src_pages = int(sum((L + P - 1) // P for L in lens))
    s_stride = int(max((L + P - 1) // P for L in lens))
    ids = rng.permutation(src_pages).astype(np.int32)
    src_bt = np.full((B, s_stride), -1, np.int32)
    k = 0
    for b, L in enumerate(lens):
        n = (int(L) + P - 1) // P
        src_bt[b, :n] = ids[k:k + n]
        k += n
    g = torch.Generator(device="cuda").manual_seed(3)
    src = torch.randint(0, 256, (src_pages * P, rb), dtype=torch.uint8, device="cuda", generator=g)
    ssc = torch.rand(src_pages * P, device="cuda", generator=g) if fp8 else None
    num_pages = gen.pool_pages(w, lens)
    vp = P * c
    stride = int(max((int(L) + vp - 1) // vp for L in lens))
    st, _, bt = OL.alloc_virtual(gen.free_stack(w, num_pages), num_pages, np.zeros(B, np.int64), lens,
                                 np.full((B, stride), -1, np.int32), P, c)
    assert st == OL.OK
    layout = K.make_layout(c, P, num_pages, K.KV_FP8_E4M3 if fp8 else K.KV_BF16)
    pools = torch.zeros(c * num_pages * P * rb, dtype=torch.uint8, device="cuda")
    pscales = torch.zeros(c * num_pages * P, dtype=torch.float32, device="cuda") if fp8 else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_bt, d_lens = _t(bt), _t(lens)
    K.dcp_kv_relayout(layout, src, ssc, _t(src_bt), d_lens, 0, c, pools, pscales, d_bt, status)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out = torch.empty((int(cu[-1]), rb), dtype=torch.uint8, device="cuda")
    out_sc = torch.empty(int(cu[-1]), dtype=torch.float32, device="cuda") if fp8 else None
    K.dcp_kv_read(layout, pools, pscales, d_bt, d_lens, _t(cu), out, out_sc, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # token order of the dense pool: row p of request b is at src_bt[b][p // P] * P + p % P
    pos = np.concatenate([np.arange(int(L)) for L in lens])
    req = np.repeat(np.arange(B), lens)
    idx = torch.from_numpy(src_bt[req, pos // P].astype(np.int64) * P + pos % P).cuda()
    assert torch.equal(out, src.index_select(0, idx))
    if fp8:
        assert torch.equal(out_sc.view(torch.int32), ssc.index_select(0, idx).view(torch.int32))
    # sampled positions against the oracle's slot map, straight from the striped pools
    pv = pools.view(c, num_pages * P, rb)
    for _ in range(256):
        b = int(rng.integers(0, B))
        p = int(rng.integers(0, int(lens[b])))
        r, s = OL.slot_of(bt[b], p, P, c)
        srow = int(src_bt[b, p // P]) * P + p % P
        assert torch.equal(pv[r, s], src[srow])
        if fp8:
            assert float(pscales[r * num_pages * P + s]) == float(ssc[srow])
    log(f"{name}: relayout + read round trip of {int(cu[-1])} rows of {rb} B ok")
