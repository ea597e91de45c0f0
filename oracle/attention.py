"""Full-context absorbed-MLA decode attention in float64, its striped partials, and
the exact LSE merge (oracle; test infrastructure only).

Absorbed MLA: every query head attends over one shared latent row per token
(SGLang page "Decode Context Parallelism", section "Why decode context
parallelism?").  The latent row is 576 wide, 512 latent columns then 64 rope
columns; scores use all 576 columns and the value is the first 512 columns of
the same row (vLLM GLM-5.3 blog post, section "Why the numbers add up": QK
over 576 dims, PV over 512 dims).

Per query row (request b, query index i, head h) the plain definition is

    s_p = sm_scale * <q, K_p>           for visible positions p
    lse = log sum_p exp(s_p)            (base e; base 2 is lse * log2(e))
    o   = sum_p exp(s_p - lse) * K_p[0:512]

Visibility: with q_len query rows the i-th sits at global position
L - q_len + i and sees positions p <= L - q_len + i when causal (the verify
contract of the SGLang page, section "DCP x speculative decoding": the kernel
is told the group size, its rank and the global KV length so causality still
sees the whole sequence); when not causal every query row sees all L tokens.

A rank r of a DCP group of size c owns the positions p with p mod c = r
(SGLang page, introduction) and returns its locally normalised o_r and lse_r
over those positions; an empty set gives lse_r = -inf and o_r = 0.  The merge
(SGLang page, section "MLA decode dataflow") is lse = logsumexp_r lse_r and
o = sum_r exp(lse_r - lse) * o_r, in the base the attention used; it is exact
up to floating-point reduction order.

Evaluation is two-pass (row maximum first, then the exponentials); large
contexts are processed in chunks of positions, which only regroups the sums.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Tuple

import numpy as np

from .codecs import bf16_to_f64, decode_rows

D_QK = 576
D_V = 512
LOG2E = 1.0 / math.log(2.0)
CHUNK = 65536


def _limits(L: int, q_len: int, causal: bool) -> np.ndarray:
    """Largest visible position for each query row index i."""
    if causal:
        return np.array([L - q_len + i for i in range(q_len)], dtype=np.int64)
    return np.full(q_len, L - 1, dtype=np.int64)


def attend(q: np.ndarray, fetch: Callable[[int, int], Tuple[np.ndarray, np.ndarray]],
           n: int, limit: np.ndarray, sm_scale: float, chunk: int = CHUNK):
    """Softmax attention of query rows over ``n`` latent rows fetched in chunks.

    q      float64 [R][576]
    fetch  (start, stop) -> (rows float64 [m][576], positions int64 [m])
    limit  int64 [R]: row r sees positions <= limit[r]
    Returns (o float64 [R][512], lse_e float64 [R]); rows that see nothing get
    o = 0 and lse = -inf.
    """
    R = q.shape[0]
    m = np.full(R, -np.inf)
    # pass 1: row maxima of the visible scores
    for a in range(0, n, chunk):
        rows, pos = fetch(a, min(n, a + chunk))
        s = sm_scale * (q @ rows.T)
        s = np.where(pos[None, :] <= limit[:, None], s, -np.inf)
        m = np.maximum(m, s.max(axis=1))
    # pass 2: normaliser and weighted values
    ell = np.zeros(R)
    acc = np.zeros((R, D_V))
    safe_m = np.where(np.isfinite(m), m, 0.0)
    for a in range(0, n, chunk):
        rows, pos = fetch(a, min(n, a + chunk))
        s = sm_scale * (q @ rows.T)
        vis = pos[None, :] <= limit[:, None]
        e = np.exp(np.where(vis, s - safe_m[:, None], -np.inf))
        ell += e.sum(axis=1)
        acc += e @ rows[:, :D_V]
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(ell[:, None] > 0, acc / np.where(ell > 0, ell, 1.0)[:, None], 0.0)
        lse = np.where(ell > 0, m + np.log(np.where(ell > 0, ell, 1.0)), -np.inf)
    return o, lse


def to_base(lse_e: np.ndarray, base: str) -> np.ndarray:
    return lse_e * LOG2E if base == "2" else lse_e


def decode_attention(q_bits: np.ndarray, kv, L: int, sm_scale: float, causal: bool = True,
                     base: str = "e", c: int = 1, r: Optional[int] = None, chunk: int = CHUNK,
                     I: int = 1):
    """Attention of one request's query rows over its KV (or rank r's share of it).

    q_bits  uint16 [q_len][H][576] bf16 payloads
    kv      (data, scale): logical rows in position order, data uint16 [L][576]
            (bf16) or uint8 [L][576] (e4m3) with float32 scale [L]
    r       None: all positions; else only the positions rank r owns, p with
            floor(p / I) mod c == r (interleave I; I = 1: p mod c == r)
    Returns o float64 [q_len][H][512] and lse float64 [q_len][H] in ``base``.
    """
    q_len, H, _ = q_bits.shape
    q = bf16_to_f64(q_bits).reshape(q_len * H, D_QK)
    lim = np.repeat(_limits(L, q_len, causal), H)
    data, scale = kv
    if r is None:
        n = L

        def fetch(a, z):
            return decode_rows(data[a:z], None if scale is None else scale[a:z]), np.arange(a, z)
    else:
        # rank r's j-th position is floor(j / I) I c + r I + j mod I
        full = L // (I * c)
        n = full * I + min(max(L - full * I * c - r * I, 0), I)

        def fetch(a, z):
            j = np.arange(a, z)
            pos = (j // I) * I * c + r * I + j % I
            return decode_rows(data[pos], None if scale is None else scale[pos]), pos
    o, lse = attend(q, fetch, n, lim, sm_scale, chunk)
    return o.reshape(q_len, H, D_V), to_base(lse, base).reshape(q_len, H)


def merge(o_parts: np.ndarray, lse_parts: np.ndarray, base: str = "e"):
    """Exact LSE merge of c partials along axis 0.

    o_parts [c][...][512], lse_parts [c][...] (same base).  Partials with
    lse = -inf get weight 0; if all are -inf the result is o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if base == "2":
        ln = lse_parts / LOG2E
    else:
        ln = lse_parts
    M = ln.max(axis=0)
    safe = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(ln - safe[None])                     # exp(-inf) = 0 for empty partials
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse_ln = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    wn = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, to_base(lse_ln, base)


def rank_partials(q_bits, kv, L, sm_scale, c, causal=True, base="e", I=1):
    """(o_r, lse_r) for every rank r of a c-way striped group: [c][q_len][H][512], [c][q_len][H]."""
    outs = [decode_attention(q_bits, kv, L, sm_scale, causal, base, c=c, r=r, I=I) for r in range(c)]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])
