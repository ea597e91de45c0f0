"""Seeded synthetic inputs for the DCP MLA-decode workloads.

This module draws numbers and stores them in the formats the kernels read; it
holds none of the method's arithmetic (no attention, no page map, no merge).
Both the oracle-side tests and the GPU side receive its outputs as inputs.

Streams (one ``numpy.random.SeedSequence`` entropy tuple each, so any piece can
be regenerated alone):

* lengths      (1000 + workload index, 0)
* free stack   (1000 + workload index, 1)
* q            (1000 + workload index, 2)
* KV rows      (1000 + workload index, 3, request, chunk), chunks of 65536 rows

Value recipe: q and latent KV are N(0, 1) drawn in float32 and rounded to
bfloat16 (round to nearest even).  For the e4m3 KV format each token row gets
one float32 scale = max|row| / 448 (1.0 for an all-zero row); the row is
divided by it, clamped to +-448 and rounded to the nearest e4m3fn code.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Tuple

import numpy as np
import torch

from .configs import D_QK, Workload

CHUNK = 65536
E4M3_MAX = 448.0


def _ss(*entropy) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(entropy)))


def lengths(w: Workload) -> np.ndarray:
    """Global KV length of every request (int64 [B])."""
    if w.fixed_len is not None:
        return np.full(w.B, w.fixed_len, dtype=np.int64)
    rng = _ss(1000 + w.index, 0)
    out = []
    for count, lo, hi in w.ragged:
        u = rng.uniform(math.log(lo), math.log(hi), size=count)
        out.append(np.floor(np.exp(u)).astype(np.int64))
    lens = np.concatenate(out)
    lens = np.clip(lens, 1, None)
    rng.shuffle(lens)
    assert lens.shape[0] == w.B
    return lens


def pool_pages(w: Workload, lens: np.ndarray, spare: int = 1) -> int:
    """Physical pages per owner pool: enough for every request plus ``spare``."""
    vp = w.P * w.c
    return int(sum((int(L) + vp - 1) // vp for L in lens)) + spare


def free_stack(w: Workload, num_pages: int) -> np.ndarray:
    """Initial free stack of page ids (int32 [num_pages]), a seeded permutation."""
    rng = _ss(1000 + w.index, 1)
    return rng.permutation(num_pages).astype(np.int32)


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def q_bits(w: Workload) -> np.ndarray:
    """Query rows as bf16 bits, uint16 [B][q_len][H][576]."""
    rng = _ss(1000 + w.index, 2)
    x = rng.standard_normal((w.B, w.q_len, w.H, D_QK), dtype=np.float32)
    return _to_bf16_bits(x)


def _kv_chunk_f32(w: Workload, b: int, chunk: int, n: int) -> np.ndarray:
    rng = _ss(1000 + w.index, 3, b, chunk)
    return rng.standard_normal((n, D_QK), dtype=np.float32)


def encode_fp8(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row scale and e4m3fn codes (uint8 [n][576], float32 [n])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[:, None], -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def kv_rows(w: Workload, b: int, L: int, start: int = 0, stop: Optional[int] = None,
            needles: Optional[dict] = None):
    """Logical latent rows [start, stop) of request ``b`` (global positions).

    Returns ``(data, scale)``: bf16 bits uint16 [n][576] and None, or e4m3
    codes uint8 [n][576] and float32 scales [n].  ``needles`` maps a position
    to a float32 [576] row that replaces the drawn one (planted keys).
    """
    stop = L if stop is None else stop
    parts = []
    c0 = start // CHUNK
    c1 = (stop + CHUNK - 1) // CHUNK
    for ch in range(c0, c1):
        lo, hi = ch * CHUNK, min((ch + 1) * CHUNK, L)
        x = _kv_chunk_f32(w, b, ch, hi - lo)
        a, z = max(lo, start), min(hi, stop)
        parts.append(x[a - lo:z - lo])
    x = np.concatenate(parts) if parts else np.zeros((0, D_QK), np.float32)
    if needles:
        for p, row in needles.items():
            if start <= p < stop:
                x[p - start] = row
    if w.kv_dtype == "bf16":
        return _to_bf16_bits(x), None
    return encode_fp8(x)


def needle_rows(w: Workload, qbits: np.ndarray, b: int, L: int, count: int = 3, gain: float = 0.5):
    """Planted keys: rows aligned with one head's query so a few scores are O(10).

    Returns {position: float32 row}.  Positions are spread over the context and
    deterministic in (workload, request).
    """
    rng = _ss(1000 + w.index, 4, b)
    q32 = (qbits[b, -1].astype(np.uint32) << 16).view(np.float32)  # last query row, [H][576]
    out = {}
    for k in range(count):
        p = int(rng.integers(0, L))
        h = int(rng.integers(0, w.H))
        out[p] = (gain * q32[h]).astype(np.float32)
    return out


def batch_rows(w: Workload, lens: np.ndarray, threads: Optional[int] = None, needles=None):
    """All logical rows of the batch in (request, position) order.

    Returns ``(data, scale, cu)`` with ``cu`` int32 [B+1] the row offsets.
    ``needles`` is an optional {request: {position: row}}.
    """
    B = len(lens)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    fp8 = w.kv_dtype == "fp8"
    data = np.empty((total, D_QK), dtype=np.uint8 if fp8 else np.uint16)
    scale = np.empty(total, dtype=np.float32) if fp8 else None
    jobs = []
    for b in range(B):
        L = int(lens[b])
        for s in range(0, L, CHUNK):
            jobs.append((b, s, min(L, s + CHUNK)))

    def run(job):
        b, s, e = job
        d, sc = kv_rows(w, b, int(lens[b]), s, e, needles=(needles or {}).get(b))
        o = int(cu[b])
        data[o + s:o + e] = d
        if fp8:
            scale[o + s:o + e] = sc

    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(run, jobs))
    return data, scale, cu.astype(np.int32) if total < 2**31 else cu
