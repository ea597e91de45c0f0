"""GPU parity of dcp_lse_merge against the oracle's float64 merge."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from parity import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("c,rows,base", [(1, 5, "e"), (2, 64, "2"), (4, 1000, "e"), (8, 257, "2"), (3, 3, "e")])
def test_merge_matches_oracle(c, rows, base):
    import kv_sharded_mla_amd as K
    rng = np.random.default_rng(c * 100 + rows)
    o = rng.standard_normal((c, rows, 512)).astype(np.float32)
    lse = (rng.standard_normal((c, rows)) * 4 + 10).astype(np.float32)
    # empty partials: some single ranks, and (if c allows) a whole row
    drop = rng.random((c, rows)) < 0.2
    lse[drop] = -np.inf
    o[drop] = 0
    lse[:, rows // 2] = -np.inf
    o[:, rows // 2] = 0
    ref_o, ref_l = OA.merge(o.astype(np.float64), lse.astype(np.float64), base)
    d_o = torch.from_numpy(o).cuda()
    d_l = torch.from_numpy(lse).cuda()
    out_o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty(rows, dtype=torch.float32, device="cuda")
    K.dcp_lse_merge(c, d_o, d_l, K.LSE_BASE_2 if base == "2" else K.LSE_BASE_E, out_o, out_l)
    go = out_o.float().cpu().numpy()
    gl = out_l.cpu().numpy()
    inf = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(gl), inf)
    assert not go[inf].any()
    do = np.abs(go - ref_o).max()
    # bf16 output: half an ulp of |o| plus fp32 arithmetic
    bound = np.abs(ref_o) * 2.0 ** -8 + 1e-5
    assert (np.abs(go - ref_o) <= bound).all(), do
    dl = np.abs(gl[~inf] - ref_l[~inf]).max()
    assert dl < 2e-5, dl
    log(f"merge c={c} rows={rows} base={base}: max|do|={do:.2e} max|dlse|={dl:.2e}")


def test_merge_output_is_round_to_nearest_even():
    import kv_sharded_mla_amd as K
    # c = 1 with lse finite passes o through: the bf16 result must be torch's RNE cast
    rng = np.random.default_rng(5)
    o = rng.standard_normal((1, 64, 512)).astype(np.float32)
    lse = np.zeros((1, 64), np.float32)
    out_o = torch.empty((64, 512), dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty(64, dtype=torch.float32, device="cuda")
    K.dcp_lse_merge(1, torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(), K.LSE_BASE_E, out_o, out_l)
    want = torch.from_numpy(o[0]).to(torch.bfloat16)
    assert torch.equal(out_o.cpu().view(torch.int16), want.view(torch.int16))
