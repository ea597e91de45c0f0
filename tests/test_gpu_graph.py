"""mla_decode_partial captured in a HIP graph and replayed with new lengths.

The work plan is made on the device from seq_len at every call, so one
captured call (plan, decode, split combine) stays right when the lengths
change between replays: each replay must equal, bit for bit, an eager call
with the same lengths.  The replays are interleaved with eager calls and
synchronisations, and every replay is checked, not only the first.  The
first replay is also compared with the oracle.
"""
import numpy as np
import pytest
import torch

from parity import Case, compare, log
from workloads import configs as C

pytestmark = pytest.mark.gpu


def W(**kw):
    base = dict(name="t", index=120, B=4, H=64, q_len=1, c=4, P=64, kv_dtype="bf16", lse_base="e", fixed_len=64)
    base.update(kw)
    return C.Workload(**base)


@pytest.mark.parametrize("kv,H", [("bf16", 64), ("bf16", 128), ("fp8", 64)])
def test_graph_replays_follow_new_lengths(kv, H):
    w = W(index=120 if kv == "bf16" else 121, H=H, kv_dtype=kv)
    lens = [9000, 300, 5000, 17]
    case = Case(w, lens=lens)
    g = case.group
    from kv_sharded_mla_amd import LSE_BASE_E
    ws = g.workspace_for(w.q_len, w.H)
    shape = (w.c, w.B, w.q_len, w.H, 512)
    o_cap = torch.empty(shape, dtype=torch.float32, device="cuda")
    l_cap = torch.empty(shape[:-1], dtype=torch.float32, device="cuda")
    full = g.seq_len.clone()

    def eager():
        o, l = g.decode(case.q, w.sm_scale, LSE_BASE_E, w.causal, workspace=ws)
        torch.cuda.synchronize()
        return o.cpu().numpy(), l.cpu().numpy()

    # warm the entry point on a side stream before capture, as torch asks
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.decode(case.q, w.sm_scale, LSE_BASE_E, w.causal, workspace=ws, out=(o_cap, l_cap))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.decode(case.q, w.sm_scale, LSE_BASE_E, w.causal, workspace=ws, out=(o_cap, l_cap))
    torch.cuda.synchronize()

    # length sets at most the captured ones (the cache holds their rows): the
    # full lengths, a split unit cut short, every request short, one emptied
    sets = [lens, [4000, 300, 5000, 17], [100, 64, 33, 17], [9000, 0, 700, 17], lens]
    for i, ls in enumerate(sets):
        g.seq_len.copy_(torch.tensor(ls, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        ref_o, ref_l = eager()          # eager work between the replays
        o_cap.fill_(float("nan"))
        l_cap.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = o_cap.cpu().numpy(), l_cap.cpu().numpy()
        assert np.array_equal(got_o.view(np.uint32), ref_o.view(np.uint32)), (i, ls)
        assert np.array_equal(got_l.view(np.uint32), ref_l.view(np.uint32)), (i, ls)
        log(f"{kv} H={H} replay {i} lengths {ls}: bit-identical to the eager call")
        if i == 0:
            for b in range(w.B):
                _, _, rop, rlp = case.oracle(b)
                compare(f"graph replay b={b}", got_o[:, b], got_l[:, b], rop, rlp, kv, partial=True)
    g.seq_len.copy_(full)
    assert g.status() == 0


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_layer_step_graph_matches_eager(kv):
    # One whole layer-step (page-stack restore, allocation of the new tokens'
    # pages, scatter of their rows, decode, merge) captured once and replayed,
    # as a serving loop that captures its decode step runs it.  The last token
    # of request 2 (position 256) opens a virtual page, so every step pops a
    # page; each replay restores the stack top first and must pop the same one.
    import kv_sharded_mla_amd as K
    w = W(index=122 if kv == "bf16" else 123, kv_dtype=kv)
    lens = np.array([3000, 700, 257, 64])
    case = Case(w, lens=lens, keep_rows=True)
    g = case.group
    data, scale = case.rows
    last = np.asarray(case.cu[1:]) - 1                      # each request's newest row
    new_rows = torch.from_numpy(data.view(np.uint8).reshape(len(data), -1)[last]).to("cuda")
    new_sc = torch.from_numpy(scale[last]).to("cuda") if scale is not None else None
    old_len = torch.tensor(lens - 1, dtype=torch.int32, device="cuda")
    new_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cu_new = torch.arange(w.B + 1, dtype=torch.int32, device="cuda")
    saved_top = g.free_top.clone()
    ws = g.workspace_for(w.q_len, w.H)
    o_part = torch.empty((w.c, w.B, w.q_len, w.H, 512), dtype=torch.float32, device="cuda")
    lse_part = torch.empty(o_part.shape[:-1], dtype=torch.float32, device="cuda")
    o = torch.empty((w.B, w.q_len, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.q_len, w.H), dtype=torch.float32, device="cuda")

    def step():
        g.free_top.copy_(saved_top)
        K.dcp_alloc_virtual(g.layout, g.free_stack, g.free_top, old_len, new_len, g.block_table, g.dev_status)
        K.dcp_kv_write(g.layout, g.pools, g.pool_scales, g.block_table, new_len, cu_new, new_rows, new_sc, None,
                       g.dev_status)
        g.decode(case.q, w.sm_scale, K.LSE_BASE_E, w.causal, workspace=ws, out=(o_part, lse_part))
        g.merge(o_part, lse_part, K.LSE_BASE_E, out=(o, lse))

    def outputs():
        torch.cuda.synchronize()
        return [t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()
                for t in (o_part, lse_part, o, lse, g.block_table)]

    step()
    ref = outputs()
    assert g.status() == 0, g.status()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        step()                                   # eager work between the replays
        assert all(np.array_equal(a, b) for a, b in zip(outputs(), ref)), i
        for t in (o_part, lse_part, lse):
            t.fill_(float("nan"))
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = outputs()
        for name, a, b in zip(("o_part", "lse_part", "o", "lse", "block_table"), got, ref):
            assert np.array_equal(a, b), (i, name)
        log(f"{kv} layer-step replay {i}: bit-identical to the eager step")
    assert g.status() == 0, g.status()
    # and the step's outputs are the oracle's
    o_f = o.float().cpu().numpy()
    l_f = lse.cpu().numpy()
    for b in range(w.B):
        ro, rl, rop, rlp = case.oracle(b)
        compare(f"layer-step graph b={b} merged", o_f[b], l_f[b], ro, rl, kv)
        compare(f"layer-step graph b={b} partials", o_part[:, b].cpu().numpy(), lse_part[:, b].cpu().numpy(), rop, rlp,
                kv, partial=True)
