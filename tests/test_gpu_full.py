"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole batch is decoded by one mla_decode_partial call over all c emulated
ranks (the same work plan and kernel as the benchmark) and merged by
dcp_lse_merge.  The oracle cannot attend every request of a multi-gigabyte
batch in seconds, so it checks samples and properties:

* the merge: the oracle's float64 merge of the GPU partials of every request
  equals the GPU's merged output (holds at any size);
* sampled requests: the GPU partials of sampled ranks equal the oracle's
  attention over those ranks' positions, and (where the oracle finishes in a
  few seconds) the merged output equals full attention over the request.

Inputs are the seeded generator's rows, kept on the host for the oracle.
"""
import numpy as np
import pytest

from oracle import attention as OA
from parity import Case, compare, log
from workloads import configs as C

pytestmark = pytest.mark.gpu

# workload -> (requests, ranks, full attention for those requests?)
SAMPLES = {
    "tplocal": ("0,31,63", "all", True),
    "replq": ("longest,shortest,20", "0,7", True),
    "verify": ("0,15", "all", True),
    "long": ("2", "0,7", False),
}


def _pick(spec, lens, n):
    out = []
    for tok in spec.split(","):
        if tok == "longest":
            out.append(int(np.argmax(lens)))
        elif tok == "shortest":
            out.append(int(np.argmin(lens)))
        elif tok == "all":
            return list(range(n))
        else:
            out.append(int(tok))
    return out


@pytest.mark.parametrize("needles", [False, True], ids=["plain", "needles"])
@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_sampled(name, needles):
    """With ``needles`` the sampled requests carry a few planted keys aligned with
    one head's query, so that some outputs are O(1) instead of near the Gaussian
    limit sm_scale * q[:512]."""
    from workloads import gen
    w = C.BY_NAME[name]
    log(f"full-size {name}{' with needles' if needles else ''}: B={w.B} H={w.H} q_len={w.q_len} c={w.c} "
        f"kv={w.kv_dtype}")
    lens = gen.lengths(w)
    planted = None
    if needles:
        qb = gen.q_bits(w)
        planted = {b: gen.needle_rows(w, qb, b, int(lens[b]), count=4, gain=0.6)
                   for b in _pick(SAMPLES[name][0], lens, w.B)}
    case = Case(w, keep_rows=True, needles=planted)
    o_part, lse_part, o, lse = case.run()
    if needles:
        for b in planted:
            assert np.abs(o[b]).max() > 0.5, (b, float(np.abs(o[b]).max()))
    log(f"{name}: decoded {int(case.lens.sum())} tokens")
    for b in range(w.B):
        ro, rl = OA.merge(o_part[:, b], lse_part[:, b], w.lse_base)
        compare(f"{name} b={b} merge of the GPU partials", o[b], lse[b], ro, rl, w.kv_dtype)
    reqs_spec, ranks_spec, full = SAMPLES[name]
    for b in _pick(reqs_spec, case.lens, w.B):
        L = int(case.lens[b])
        kv = case.kv_host(b)
        for r in _pick(ranks_spec, case.lens, w.c):
            ro, rl = OA.decode_attention(case.q_bits[b], kv, L, w.sm_scale, w.causal, w.lse_base, c=w.c, r=r,
                                         I=w.interleave)
            compare(f"{name} b={b} (L={L}) rank {r} partial", o_part[r, b], lse_part[r, b], ro, rl, w.kv_dtype,
                    partial=True)
        if full:
            ro, rl = OA.decode_attention(case.q_bits[b], kv, L, w.sm_scale, w.causal, w.lse_base)
            compare(f"{name} b={b} (L={L}) merged vs full attention", o[b], lse[b], ro, rl, w.kv_dtype)
