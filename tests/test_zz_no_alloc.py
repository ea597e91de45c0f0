"""The allocation-free decode entry point (mla_decode_partial_noalloc) through the C ABI.

It must give the same outputs as mla_decode_partial with a caller workspace,
bit for bit (same work plan and kernels; only the scratch address differs), on
two calls in a row with the second one smaller (the scratch keeps the first
call's contents, which the second must not depend on), on the single-launch
path and on the planned split path, and match the oracle; a call whose
workspace would exceed the scratch is refused on the host; and one call
captured in a HIP graph, replayed after seq_len changes, equals the eager
call with the same lengths.
"""
import numpy as np
import pytest
import torch

from parity import Case, compare, log
from workloads import configs as C

pytestmark = pytest.mark.gpu


def W(**kw):
    base = dict(name="na", index=120, B=1, H=16, q_len=1, c=4, P=64, kv_dtype="bf16", lse_base="e", fixed_len=64)
    base.update(kw)
    return C.Workload(**base)


def _both(case):
    import kv_sharded_mla_amd as K
    w, g = case.w, case.group
    base = K.LSE_BASE_2 if w.lse_base == "2" else K.LSE_BASE_E
    ref_o, ref_l = g.decode(case.q, w.sm_scale, base, w.causal)
    o = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    K.mla_decode_partial_noalloc(g.layout, g.pools, g.pool_scales, 0, w.c, case.q, g.block_table, g.seq_len,
                                 g.max_seq_len, w.sm_scale, base, w.causal, o, lse, g.dev_status)
    torch.cuda.synchronize()
    assert g.status() == 0
    return ref_o.cpu().numpy(), ref_l.cpu().numpy(), o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    # split path (work plan, partials in the scratch, combine) then a smaller split call
    (W(index=121, H=128, c=4, B=3, fixed_len=20000), W(index=122, H=64, c=2, B=2, fixed_len=9000, kv_dtype="fp8")),
    # split path, then the single-launch path (no plan) of a small call
    (W(index=123, H=64, q_len=4, c=8, B=2, fixed_len=30000, kv_dtype="fp8"), W(index=124, H=16, c=4, fixed_len=300)),
])
def test_noalloc_matches_workspace_call(first, second):
    import kv_sharded_mla_amd as K
    assert K.mla_decode_noalloc_scratch_bytes() == 256 << 20
    for w in (first, second):
        case = Case(w)
        need = K.mla_decode_workspace_size(case.group.layout, w.c, w.B, w.q_len, w.H, case.group.max_seq_len)
        log(f"no-alloc {w}: workspace {need} bytes")
        assert need <= K.mla_decode_noalloc_scratch_bytes()
        ref_o, ref_l, o, lse = _both(case)
        assert np.array_equal(o.view(np.uint32), ref_o.view(np.uint32))
        assert np.array_equal(lse.view(np.uint32), ref_l.view(np.uint32))
        for b in range(w.B):
            _, _, rop, rlp = case.oracle(b)
            compare(f"no-alloc {w.name} b={b}", o[:, b], lse[:, b], rop, rlp, w.kv_dtype, partial=True)
        del case
        torch.cuda.empty_cache()


def test_noalloc_refuses_a_call_beyond_the_scratch():
    import kv_sharded_mla_amd as K
    B, H, c = 256, 128, 8
    layout = K.make_layout(c, 64, 2, K.KV_BF16)
    need = K.mla_decode_workspace_size(layout, c, B, 1, H, 1 << 20)
    assert need > K.mla_decode_noalloc_scratch_bytes()
    pools = torch.zeros(c * K.dcp_pool_bytes(layout), dtype=torch.uint8, device="cuda")
    q = torch.zeros((B, 1, H, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    o = torch.zeros((c, B, 1, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.zeros((c, B, 1, H), dtype=torch.float32, device="cuda")
    with pytest.raises(K.DcpError) as e:
        K.mla_decode_partial_noalloc(layout, pools, None, 0, c, q, bt, sl, 1 << 20, 0.1, 0, True, o, lse)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert not o.any() and not lse.any()      # nothing was enqueued


def test_noalloc_call_in_a_graph_follows_new_lengths():
    # the callers this entry point is for capture it in graphs: one captured call
    # replayed after seq_len changes equals the eager call with the same lengths
    import kv_sharded_mla_amd as K
    w = W(index=125, H=128, c=4, B=4)
    lens = [9000, 300, 5000, 17]
    case = Case(w, lens=lens)
    g = case.group
    shape = (w.c, w.B, w.q_len, w.H, 512)
    o_cap = torch.empty(shape, dtype=torch.float32, device="cuda")
    l_cap = torch.empty(shape[:-1], dtype=torch.float32, device="cuda")

    def call(o, lse):
        K.mla_decode_partial_noalloc(g.layout, g.pools, g.pool_scales, 0, w.c, case.q, g.block_table, g.seq_len,
                                     g.max_seq_len, w.sm_scale, K.LSE_BASE_E, w.causal, o, lse, g.dev_status)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(o_cap, l_cap)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o_cap, l_cap)
    torch.cuda.synchronize()
    full = g.seq_len.clone()
    for i, ls in enumerate([lens, [4000, 300, 100, 17], [9000, 0, 700, 17]]):
        g.seq_len.copy_(torch.tensor(ls, dtype=torch.int32, device="cuda"))
        ref_o = torch.full_like(o_cap, float("nan"))
        ref_l = torch.full_like(l_cap, float("nan"))
        call(ref_o, ref_l)
        torch.cuda.synchronize()
        o_cap.fill_(float("nan"))
        l_cap.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(o_cap.cpu().numpy().view(np.uint32), ref_o.cpu().numpy().view(np.uint32)), (i, ls)
        assert np.array_equal(l_cap.cpu().numpy().view(np.uint32), ref_l.cpu().numpy().view(np.uint32)), (i, ls)
        log(f"no-alloc graph replay {i} lengths {ls}: bit-identical to the eager call")
    g.seq_len.copy_(full)
    assert g.status() == 0
