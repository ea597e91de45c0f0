"""Shared helpers of the GPU parity tests.

Inputs come from the seeded generators in ``workloads.gen``; the expected
values come from ``oracle`` on the host copies of those inputs.  Nothing the
oracle sees is read back from the GPU.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

from oracle import attention as OA
from workloads import gen
from workloads.configs import Workload

TOL = {"bf16": (1e-2, 1e-3), "fp8": (3e-2, 1e-3)}   # (max |do|, max |dlse|)


def log(msg):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


class Case:
    """One workload's inputs on host and device, and its emulated group."""

    def __init__(self, w: Workload, lens=None, needles=None, seed_free_stack=True, sentinel=None,
                 num_pages=None, keep_rows=False, keep_slots=False):
        from kv_sharded_mla_amd import KV_BF16, KV_FP8_E4M3
        from kv_sharded_mla_amd.group import DcpGroup
        self.w = w
        self.lens = gen.lengths(w) if lens is None else np.asarray(lens, dtype=np.int64)
        self.q_bits = gen.q_bits(w)
        self.needles = needles
        self.num_pages = gen.pool_pages(w, self.lens) if num_pages is None else int(num_pages)
        vp = w.P * w.c
        self.bt_stride = max(1, max((int(L) + vp - 1) // vp for L in self.lens))
        fs = gen.free_stack(w, self.num_pages) if seed_free_stack else None
        self.group = DcpGroup(w.c, w.P, self.num_pages, KV_FP8_E4M3 if w.kv_dtype == "fp8" else KV_BF16,
                              w.B, self.bt_stride, free_stack=fs, sentinel=sentinel,
                              interleave=w.interleave)
        data, scale, cu = gen.batch_rows(w, self.lens, needles=needles)
        self.cu = cu
        # the generator's host rows, kept for the oracle when regenerating them per
        # request would be slow (full-size workloads)
        self.rows = (data, scale) if keep_rows else None
        rows = torch.from_numpy(data.view(np.uint8).reshape(len(data), -1)).to("cuda")
        sc = torch.from_numpy(scale).to("cuda") if scale is not None else None
        # slot_out of the bulk write (owner * capacity + physical slot), kept on request
        self.slots = torch.empty(len(data), dtype=torch.int64, device="cuda") if keep_slots else None
        self.group.append([int(L) for L in self.lens], rows, sc, self.slots)
        del rows, sc
        torch.cuda.synchronize()
        assert self.group.status() == 0, self.group.status()
        self.q = torch.from_numpy(self.q_bits.view(np.int16)).to("cuda")

    def kv_host(self, b):
        L = int(self.lens[b])
        if self.rows is not None:
            data, scale = self.rows
            a = int(self.cu[b])
            return data[a:a + L], None if scale is None else scale[a:a + L]
        return gen.kv_rows(self.w, b, L, needles=(self.needles or {}).get(b))

    def run(self):
        from kv_sharded_mla_amd import LSE_BASE_2, LSE_BASE_E
        base = LSE_BASE_2 if self.w.lse_base == "2" else LSE_BASE_E
        o_part, lse_part = self.group.decode(self.q, self.w.sm_scale, base, self.w.causal)
        o, lse = self.group.merge(o_part, lse_part, base)
        torch.cuda.synchronize()
        assert self.group.status() == 0, self.group.status()
        return (o_part.cpu().numpy(), lse_part.cpu().numpy(), o.float().cpu().numpy(), lse.cpu().numpy())

    def oracle(self, b, partials=True):
        w = self.w
        kv = self.kv_host(b)
        L = int(self.lens[b])
        o, lse = OA.decode_attention(self.q_bits[b], kv, L, w.sm_scale, w.causal, w.lse_base)
        if not partials:
            return o, lse, None, None
        op, lp = OA.rank_partials(self.q_bits[b], kv, L, w.sm_scale, w.c, w.causal, w.lse_base, I=w.interleave)
        return o, lse, op, lp


def compare(name, got_o, got_lse, ref_o, ref_lse, kind, partial=False):
    """Assert the stated tolerances; -inf lse must match exactly (empty shards).

    The stated o bound assumes |o| of order 1.  A near one-hot row makes |o|
    reach a few units, and then each bf16 rounding on the way (relative error
    at most 2^-8 with 8 significant bits) can exceed it on its own: the fp32
    partials take one (the bf16 P of the PV product), the merged bf16 output
    a second.  o is held to max(stated bound, 2^-8 max|o|) in the partials and
    max(stated bound, 2^-7 max|o|) after the merge; lse keeps its bound.
    """
    to, tl = TOL[kind]
    if ref_o.size:
        to = max(to, 2.0 ** (-8 if partial else -7) * float(np.abs(ref_o).max()))
    ref_inf = np.isneginf(ref_lse)
    got_inf = np.isneginf(got_lse)
    assert np.array_equal(ref_inf, got_inf), f"{name}: empty-shard pattern differs"
    fin = ~ref_inf
    do = float(np.abs(got_o - ref_o).max()) if got_o.size else 0.0
    dl = float(np.abs(got_lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    if ref_inf.any():
        assert not got_o[ref_inf].any(), f"{name}: empty shard must give o = 0"
    rms = float(np.sqrt((ref_o ** 2).mean())) if ref_o.size else 0.0
    log(f"{name}: max|do|={do:.3e} (tol {to}) max|dlse|={dl:.3e} (tol {tl}) rel={do / max(rms, 1e-30):.3e}")
    assert do <= to, f"{name}: max |do| = {do} > {to}"
    assert dl <= tl, f"{name}: max |dlse| = {dl} > {tl}"
    assert math.isfinite(do) and math.isfinite(dl)
    return do, dl


def check_case(case: Case, requests=None, partials=True):
    o_part, lse_part, o, lse = case.run()
    reqs = range(case.w.B) if requests is None else requests
    for b in reqs:
        ro, rl, rop, rlp = case.oracle(b, partials)
        compare(f"{case.w.name} b={b} merged", o[b], lse[b], ro, rl, case.w.kv_dtype)
        if partials:
            compare(f"{case.w.name} b={b} partials", o_part[:, b], lse_part[:, b], rop, rlp, case.w.kv_dtype,
                    partial=True)
    return o_part, lse_part, o, lse
