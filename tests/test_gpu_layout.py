"""GPU parity of the integer path: dcp_alloc_virtual and dcp_kv_write, bit-exact.

Expected block tables, free-stack tops, slots and pool bytes come from the
oracle's integer layout model (oracle.layout) on the same seeded inputs.
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


@pytest.mark.parametrize("seed,B", [(s, None) for s in range(6)] + [(6, 65), (7, 1000), (8, 1025), (9, 4097)])
def test_alloc_matches_oracle_over_growth(seed, B):
    """Block table and free-stack top bit-exact over four growth steps.  Batches of
    65 and 1000 requests span several waves of the allocator's scan (the carry over
    the wave totals); 1025 and 4097 give every thread several requests."""
    K = _lib()
    rng = np.random.default_rng(seed)
    c = int(rng.integers(1, 9))
    P = int(rng.choice([1, 2, 16, 64]))
    B = int(rng.integers(1, 40)) if B is None else B
    final = rng.integers(0, 5000, size=B)
    vp = P * c
    num_pages = int(sum((L + vp - 1) // vp for L in final)) + 3
    stride = int(max((L + vp - 1) // vp for L in final)) + 1
    stack = rng.permutation(num_pages).astype(np.int32)
    layout = K.make_layout(c, P, num_pages, K.KV_BF16)
    d_stack, d_top = _t(stack), _t([num_pages])
    d_bt = _t(np.full((B, stride), -1, np.int32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    h_bt = np.full((B, stride), -1, np.int32)
    h_top = num_pages
    cur = np.zeros(B, np.int64)
    for step in range(1, 5):
        new = (final * step) // 4
        K.dcp_alloc_virtual(layout, d_stack, d_top, _t(cur), _t(new), d_bt, status)
        st, h_top, h_bt = OL.alloc_virtual(stack, h_top, cur, new, h_bt, P, c)
        assert st == OL.OK
        assert int(status.item()) == 0
        assert int(d_top.item()) == h_top
        assert np.array_equal(d_bt.cpu().numpy(), h_bt)
        cur = new
    log(f"alloc seed={seed} c={c} P={P} B={B} pages={num_pages} ok")


@pytest.mark.parametrize("old,new,top,stride,code", [
    ([0, 0], [9, 9], 4, 4, OL.OUT_OF_PAGES),
    ([4, 0], [3, 1], 10, 4, OL.BAD_LENGTH),
    ([0, 0], [17, 1], 10, 4, OL.TABLE_OVERFLOW),
])
def test_alloc_errors_leave_state(old, new, top, stride, code):
    K = _lib()
    layout = K.make_layout(2, 2, 10, K.KV_BF16)
    d_stack = _t(np.arange(10, dtype=np.int32))
    d_top = _t([top])
    d_bt = _t(np.full((2, stride), -7, np.int32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.dcp_alloc_virtual(layout, d_stack, d_top, _t(old), _t(new), d_bt, status)
    assert int(status.item()) == code
    assert int(d_top.item()) == top
    assert (d_bt.cpu().numpy() == -7).all()


@pytest.mark.parametrize("B,needy", [(1025, 1020), (4097, 3000), (200, 130)])
def test_alloc_out_of_pages_in_a_later_wave(B, needy):
    # only one request, owned by a thread beyond the first wave, needs pages, and
    # one more than the stack holds: all or nothing, nothing changes
    K = _lib()
    c, P = 2, 4
    old = np.full(B, 8, np.int64)
    new = old.copy()
    new[needy] = 8 + 5 * P * c          # five more virtual pages
    top = 4
    layout = K.make_layout(c, P, 10, K.KV_BF16)
    d_top = _t([top])
    d_bt = _t(np.full((B, 8), -7, np.int32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.dcp_alloc_virtual(layout, _t(np.arange(10, dtype=np.int32)), d_top, _t(old), _t(new), d_bt, status)
    st, h_top, h_bt = OL.alloc_virtual(np.arange(10, dtype=np.int32), top, old, new, np.full((B, 8), -7, np.int32),
                                       P, c)
    assert st == OL.OUT_OF_PAGES and int(status.item()) == OL.OUT_OF_PAGES
    assert int(d_top.item()) == h_top == top
    assert np.array_equal(d_bt.cpu().numpy(), h_bt) and (h_bt == -7).all()
    # with one more page on the stack the same call succeeds and takes exactly those five
    d_top = _t([5])
    status.zero_()
    K.dcp_alloc_virtual(layout, _t(np.arange(10, dtype=np.int32)), d_top, _t(old), _t(new), d_bt, status)
    st, h_top, h_bt = OL.alloc_virtual(np.arange(10, dtype=np.int32), 5, old, new, np.full((B, 8), -7, np.int32),
                                       P, c)
    assert st == OL.OK and int(status.item()) == 0 and int(d_top.item()) == h_top == 0
    assert np.array_equal(d_bt.cpu().numpy(), h_bt)


def test_kv_write_rows_below_the_first_offset_belong_to_no_request():
    # cu_new[0] > 0: rows 0 .. cu_new[0]-1 belong to no request; they are skipped
    # with BAD_LENGTH and slot -1 (never written over a cached token of request 0)
    K = _lib()
    c, P = 2, 4
    lens = np.array([12, 7])
    vp = P * c
    bt = np.array([[2, 0], [1, -1]], np.int32)
    cu = np.array([3, 6, 8])            # request 0 appends rows 3..5, request 1 rows 6..7
    N = 8
    rng = np.random.default_rng(9)
    rows = rng.integers(0, 65536, size=(N, 576)).astype(np.uint16)
    pools = np.full((c, 3 * P, 576), 0x5A5A, np.uint16)
    est, own, phys, want, _ = OL.pool_image(pools, bt, lens, cu, rows, P, c)
    assert est == OL.BAD_LENGTH and (own[:3] == -1).all() and (own[3:] >= 0).all()
    layout = K.make_layout(c, P, 3, K.KV_BF16)
    d_pools = torch.from_numpy(pools.view(np.uint8).reshape(-1).copy()).to("cuda")
    slot = torch.full((N,), -99, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.dcp_kv_write(layout, d_pools, None, _t(bt), _t(lens), _t(cu),
                   torch.from_numpy(rows.view(np.uint8).copy()).to("cuda"), None, slot, status)
    assert int(status.item()) == OL.BAD_LENGTH
    assert np.array_equal(d_pools.cpu().numpy().view(np.uint16).reshape(c, -1, 576), want)
    s = slot.cpu().numpy()
    cap = 3 * P
    assert (s[:3] == -1).all() and np.array_equal(s[3:], own[3:] * cap + phys[3:])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("interleaved", [False, True])
def test_kv_write_pool_bytes_exact(kv, seed, interleaved):
    """Pool bytes and slots of dcp_kv_write equal the layout model's, round robin
    (I = 1) and with runs of I positions per owner (I a divisor of P)."""
    K = _lib()
    rng = np.random.default_rng(100 + seed + 50 * interleaved)
    c = int(rng.integers(1, 9))
    P = int(rng.choice([4, 12, 16, 64] if interleaved else [1, 3, 16, 64]))
    I = int(rng.choice([d for d in range(2, P + 1) if P % d == 0])) if interleaved else 1
    B = int(rng.integers(1, 12))
    lens = rng.integers(0, 700, size=B)
    vp = P * c
    num_pages = int(sum((L + vp - 1) // vp for L in lens)) + 2
    stride = int(max((L + vp - 1) // vp for L in lens)) + 1
    stack = rng.permutation(num_pages).astype(np.int32)
    st, top, bt = OL.alloc_virtual(stack, num_pages, np.zeros(B, np.int64), lens,
                                   np.full((B, stride), -1, np.int32), P, c)
    assert st == OL.OK
    N = int(lens.sum())
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    fp8 = kv == "fp8"
    elems = 576
    row_dtype = np.uint8 if fp8 else np.uint16
    rows = rng.integers(0, 256 if fp8 else 65536, size=(N, elems)).astype(row_dtype)
    scales = rng.standard_normal(N).astype(np.float32) if fp8 else None
    pools = np.full((c, num_pages * P, elems), 0xEE if fp8 else 0xEEEE, dtype=row_dtype)
    pscales = np.full((c, num_pages * P), -1.5, np.float32) if fp8 else None
    est, own, phys, want, want_sc = OL.pool_image(pools, bt, lens, cu, rows, P, c, scales, pscales, I)
    assert est == OL.OK
    layout = K.make_layout(c, P, num_pages, K.KV_FP8_E4M3 if fp8 else K.KV_BF16, I)
    d_pools = torch.from_numpy(pools.view(np.uint8).reshape(-1).copy()).to("cuda")
    d_psc = _t(pscales.reshape(-1), torch.float32) if fp8 else None
    d_rows = torch.from_numpy(rows.view(np.uint8).reshape(N, -1).copy()).to("cuda")
    d_sc = _t(scales, torch.float32) if fp8 else None
    slot = torch.full((N,), -99, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.dcp_kv_write(layout, d_pools, d_psc, _t(bt), _t(lens), _t(cu), d_rows, d_sc, slot, status)
    assert int(status.item()) == 0
    got = d_pools.cpu().numpy().view(row_dtype).reshape(c, num_pages * P, elems)
    assert np.array_equal(got, want)
    cap = num_pages * P
    assert np.array_equal(slot.cpu().numpy(), own * cap + phys)
    if fp8:
        assert np.array_equal(d_psc.cpu().numpy().reshape(c, -1).view(np.uint32), want_sc.view(np.uint32))
    log(f"kv_write {kv} seed={seed} c={c} P={P} B={B} rows={N} ok")


def test_kv_write_skips_bad_rows_and_reports():
    K = _lib()
    c, P = 2, 2
    bt = np.array([[3, 1, -1], [0, 9, -1]], dtype=np.int32)
    lens = np.array([6, 5])
    cu = np.array([0, 3, 4])
    rows = np.arange(4 * 576, dtype=np.uint16).reshape(4, 576)
    pools = np.full((c, 4 * P, 576), 0x1234, dtype=np.uint16)
    est, own, phys, want, _ = OL.pool_image(pools, bt, lens, cu, rows, P, c)
    assert est == OL.BAD_PAGE
    layout = K.make_layout(c, P, 4, K.KV_BF16)
    d_pools = torch.from_numpy(pools.view(np.uint8).reshape(-1).copy()).to("cuda")
    slot = torch.zeros(4, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.dcp_kv_write(layout, d_pools, None, _t(bt), _t(lens), _t(cu),
                   torch.from_numpy(rows.view(np.uint8).copy()).to("cuda"), None, slot, status)
    assert int(status.item()) == OL.BAD_PAGE
    assert np.array_equal(d_pools.cpu().numpy().view(np.uint16).reshape(c, -1, 576), want)
    s = slot.cpu().numpy()
    assert s[3] == -1 and np.array_equal(s[:3], own[:3] * 4 * P + phys[:3])
