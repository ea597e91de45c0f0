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
