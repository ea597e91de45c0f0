"""The five synthetic DCP MLA-decode workloads, as shapes only.

Nothing here computes attention, a page map or a merge: these are the sizes
that the seeded generators in ``workloads.gen`` draw inputs for, and that the
tests and the benchmark iterate over.

Shapes follow the latent-KV description of absorbed MLA on the SGLang page
"Decode Context Parallelism" (section "Why decode context parallelism?": one
latent KV shared by every query head) and the vLLM GLM-5.3 blog post
("Why the numbers add up": QK over 576 dims, PV over 512 dims).  The ragged
length mix of the replicated-q workload follows the agentic length
distribution of the llm-wiki article "vLLM Decode Context Parallelism"
(section "Why focus on decode": about 53% of contexts at or above 64K tokens,
up to 1M, the rest below 64K).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

D_QK = 576  # 512 latent + 64 rope
D_V = 512   # V is the first 512 columns of the latent row
SM_SCALE = 1.0 / math.sqrt(192.0)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the workload list; seeds derive from it
    B: int                # requests in the batch
    H: int                # query heads that share one latent row
    q_len: int            # query rows per request (1 = decode, >1 = verify)
    c: int                # DCP group size (owner pools)
    P: int                # physical page size in tokens
    kv_dtype: str         # "bf16" or "fp8"
    lse_base: str         # "e" or "2"
    fixed_len: Optional[int] = None            # every request has this global KV length
    ragged: Optional[Tuple[Tuple[int, int, int], ...]] = None  # (count, lo, hi) log-uniform groups
    causal: bool = True
    sm_scale: float = SM_SCALE
    interleave: int = 1   # KV interleave size I: runs of I consecutive positions per owner
    description: str = ""

    @property
    def virtual_page(self) -> int:
        return self.P * self.c

    @property
    def rows(self) -> int:
        """Query rows per request (q_len * H)."""
        return self.q_len * self.H

    @property
    def kv_row_bytes(self) -> int:
        return 2 * D_QK if self.kv_dtype == "bf16" else D_QK  # fp8 scale stored apart


TINY = Workload(
    name="tiny", index=0, B=1, H=16, q_len=1, c=4, P=16, kv_dtype="bf16", lse_base="e",
    fixed_len=1024,
    description="batch 1, 16 heads, context 1024, c=4, P=16 (virtual page 64), q_len 1, base-e LSE")

TP_LOCAL = Workload(
    name="tplocal", index=1, B=64, H=16, q_len=1, c=8, P=64, kv_dtype="bf16", lse_base="2",
    fixed_len=32768,
    description="TP-local 16 heads, batch 64, context 32768, c=8 (4096 tokens per owner), P=64, q_len 1, base-2 LSE")

REPL_Q = Workload(
    name="replq", index=2, B=32, H=128, q_len=1, c=8, P=64, kv_dtype="bf16", lse_base="e",
    ragged=((17, 65536, 262144), (15, 2048, 65536)),
    description="replicated-q 128 heads, batch 32, ragged contexts (17 log-uniform in [64K,256K], "
                "15 log-uniform in [2K,64K)), c=8, P=64, q_len 1")

VERIFY = Workload(
    name="verify", index=3, B=16, H=128, q_len=4, c=4, P=64, kv_dtype="bf16", lse_base="e",
    fixed_len=65536,
    description="static target verification: 128 heads, batch 16, context 65536, q_len 4 causal, c=4, P=64")

LONG_FP8 = Workload(
    name="long", index=4, B=4, H=64, q_len=1, c=8, P=64, kv_dtype="fp8", lse_base="e",
    fixed_len=1 << 20,
    description="long context: 64 heads, batch 4, context 1048576, c=8, P=64, e4m3 KV + fp32 per-token scale")

ALL = (TINY, TP_LOCAL, REPL_Q, VERIFY, LONG_FP8)
BY_NAME = {w.name: w for w in ALL}


def scaled(w: Workload, *, B=None, H=None, q_len=None, c=None, P=None, length=None,
           kv_dtype=None, lse_base=None, causal=None, interleave=None, name=None) -> Workload:
    """A copy of ``w`` with some sizes replaced (used for small parity cases)."""
    kw = dict(w.__dict__)
    for k, v in dict(B=B, H=H, q_len=q_len, c=c, P=P, kv_dtype=kv_dtype, lse_base=lse_base,
                     causal=causal, interleave=interleave).items():
        if v is not None:
            kw[k] = v
    if length is not None:
        kw["fixed_len"] = length
        kw["ragged"] = None
    kw["name"] = name or (w.name + "-scaled")
    return Workload(**kw)
