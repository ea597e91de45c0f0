"""Benchmark of the DCP MLA decode hot path on one MI355X.

One step = one layer-step of an emulated c-rank DCP group: allocate virtual
pages for the q_len new tokens of every request, scatter their latent rows
into the owner pools, attend every rank's striped shard (partials), and merge
the partials.  The context (L - q_len tokens per request) is written before
timing and stays resident in HBM; two identical copies of the pools are used
in alternation so consecutive steps never find the previous step's KV in the
256 MB MALL.

Prints one JSON line (rank 0).  Progress goes to stderr.

    python bench.py [--config replq] [--extras tiny,tplocal,verify,long] [--steps K] [--warmup W] [--gpus 1]

The headline line is the replicated-q workload (128 heads, 32 ragged requests
up to 256K tokens, the largest of the five that one GPU holds); the same run
times the other workloads and reports each under "workloads": decode time,
roofline fractions and the one-rank share.

With --op read or --op relayout it times instead the extend gather
(dcp_kv_read: all cached rows of the workload back to token order) or the
DCP1 -> DCP c relayout (dcp_kv_relayout: a dense paged pool of the
workload's context into the c owner pools), both byte copies bound by HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("mla_decode.hip", "dcp_common.hpp"):
        with open(os.path.join(ROOT, "kv_sharded_mla_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_copy_traffic(op: str, cfg_name: str):
    """HBM traffic per layout-copy launch from a committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"kv_{op}_{cfg_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "kv_sharded_mla_amd", "csrc", "kv_layout.hip"), "rb") as fh:
        h.update(fh.read())
    if t.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    return t.get("hbm_bytes_per_launch")


def load_traffic(cfg_name: str):
    """HBM traffic per decode launch from a committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"mla_decode_{cfg_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def host_info():
    """CPU model and BLAS library the oracle runs on (for the baseline's record)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return model, blas


def cpu_baseline(w, lens, budget_s: float):
    """The oracle as it stands (rank partials + merge), timed on a sample of requests."""
    import numpy as np
    from oracle import attention as OA
    from workloads import accounting, gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = os.cpu_count() or 1
    q_bits = gen.q_bits(w)
    done_bytes = 0
    t_total = 0.0
    n = 0
    for b in range(w.B):
        L = int(lens[b])
        kv = gen.kv_rows(w, b, L)           # stored-format bytes (generation not timed)
        t0 = time.perf_counter()
        op, lp = OA.rank_partials(q_bits[b], kv, L, w.sm_scale, w.c, w.causal, w.lse_base, I=w.interleave)
        OA.merge(op, lp, w.lse_base)
        t_total += time.perf_counter() - t0
        done_bytes += L * accounting.kv_bytes_per_token(w)
        n += 1
        if t_total >= budget_s:
            break
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"requests 0..{n - 1} of {w.name} ({n}/{w.B}), all {w.H} heads x q_len {w.q_len}, "
                      f"{w.c} rank partials + merge in float64, {t_total:.1f} s",
            "seconds": round(t_total, 2), "cpu_model": host_info()[0], "blas": host_info()[1]}


HEADLINE = "replq"        # the largest single-GPU workload: 128 heads, ragged contexts up to 256K
EXTRAS = ("tiny", "tplocal", "verify", "long")


def roofline_of(w, flops, nbytes, t_ms):
    """Fractions of the MI355X peaks for one launch of t_ms: HBM GB/s and bf16 MFMA TFLOP/s;
    the 128-head workloads are judged on MFMA, the others on HBM."""
    gbps = nbytes / (t_ms * 1e-3) / 1e9
    tflops = flops / (t_ms * 1e-3) / 1e12
    mfma_bound = w.H * w.q_len >= 128
    return dict(bound="mfma" if mfma_bound else "hbm", gbps=gbps, tflops=tflops,
                hbm_frac=gbps / HBM_PEAK_GBPS, mfma_frac=tflops / MFMA_BF16_PEAK_TFLOPS,
                frac=(tflops / MFMA_BF16_PEAK_TFLOPS) if mfma_bound else (gbps / HBM_PEAK_GBPS))


def time_workload(w, steps, warmup, copies=2, share=True, decode_only=0, calib_copy_mib=0, graph=True):
    """Time `steps` layer-steps of workload w on resident pools; returns the measurements."""
    import numpy as np
    import torch

    import kv_sharded_mla_amd as K
    from kv_sharded_mla_amd.group import DcpGroup
    from workloads import accounting, gen

    dev = torch.device("cuda:0")
    lens = gen.lengths(w)
    ctx = np.maximum(lens - w.q_len, 0)           # resident context before the step's new tokens
    num_pages = gen.pool_pages(w, lens)
    vp = w.P * w.c
    stride = int(max((int(L) + vp - 1) // vp for L in lens))
    kv_kind = K.KV_FP8_E4M3 if w.kv_dtype == "fp8" else K.KV_BF16
    base = K.LSE_BASE_2 if w.lse_base == "2" else K.LSE_BASE_E

    log(f"workload {w.name}: B={w.B} H={w.H} q_len={w.q_len} c={w.c} P={w.P} kv={w.kv_dtype} "
        f"sum(L)={int(lens.sum())}; generating inputs")
    t0 = time.time()
    data, scale, cu = gen.batch_rows(w, lens)
    log(f"generated {data.nbytes / 2**30:.2f} GiB of latent rows in {time.time() - t0:.1f} s")
    # split every request's rows into resident context and the step's new rows
    ctx_idx = np.concatenate([np.arange(cu[b], cu[b] + ctx[b]) for b in range(w.B)]).astype(np.int64)
    new_idx = np.concatenate([np.arange(cu[b] + ctx[b], cu[b + 1]) for b in range(w.B)]).astype(np.int64)
    row_u8 = data.view(np.uint8).reshape(len(data), -1)
    new_rows = torch.from_numpy(row_u8[new_idx]).to(dev)
    new_sc = torch.from_numpy(scale[new_idx]).to(dev) if scale is not None else None
    stack = gen.free_stack(w, num_pages)
    groups = []
    ctx_rows = torch.from_numpy(row_u8[ctx_idx]).to(dev)
    ctx_sc = torch.from_numpy(scale[ctx_idx]).to(dev) if scale is not None else None
    del data, scale, row_u8
    for k in range(copies):
        g = DcpGroup(w.c, w.P, num_pages, kv_kind, w.B, stride, free_stack=stack, device="cuda:0",
                     interleave=w.interleave)
        g.append([int(x) for x in ctx], ctx_rows, ctx_sc)
        groups.append(g)
    del ctx_rows, ctx_sc
    torch.cuda.synchronize()
    assert all(g.status() == 0 for g in groups)
    log(f"{copies} resident pool copies written ({groups[0].pools.numel() * copies / 2**30:.2f} GiB)")

    q = torch.from_numpy(gen.q_bits(w).view(np.int16)).to(dev)
    old_len = torch.from_numpy(ctx.astype(np.int32)).to(dev)
    new_len = torch.from_numpy(lens.astype(np.int32)).to(dev)
    cu_new = torch.from_numpy(np.concatenate([[0], np.cumsum(lens - ctx)]).astype(np.int32)).to(dev)
    max_len = int(lens.max())
    for g in groups:
        g.max_seq_len = max_len
    ws_bytes = K.mla_decode_workspace_size(groups[0].layout, w.c, w.B, w.q_len, w.H, max_len)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=dev)
    o_part = torch.empty((w.c, w.B, w.q_len, w.H, K.D_V), dtype=torch.float32, device=dev)
    lse_part = torch.empty((w.c, w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.q_len, w.H, K.D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # If a new token opens a virtual page, every step pops the same pages again from the
    # same stack top: restore the top first so repeated steps stay identical.
    need_pages = int(sum((int(L) + vp - 1) // vp - (int(x) + vp - 1) // vp for L, x in zip(lens, ctx)))
    saved_top = [g.free_top.clone() for g in groups]

    def step(gi, ev=None):
        g = groups[gi]
        if ev is not None:
            ev[0].record(stream)
        if need_pages:
            g.free_top.copy_(saved_top[gi])
        K.dcp_alloc_virtual(g.layout, g.free_stack, g.free_top, old_len, new_len, g.block_table, g.dev_status)
        K.dcp_kv_write(g.layout, g.pools, g.pool_scales, g.block_table, new_len, cu_new, new_rows, new_sc, None,
                       g.dev_status)
        if ev is not None:
            ev[1].record(stream)
        K.mla_decode_partial(g.layout, g.pools, g.pool_scales, 0, w.c, q, g.block_table, new_len, max_len,
                             w.sm_scale, base, w.causal, o_part, lse_part, ws, g.dev_status)
        if ev is not None:
            ev[2].record(stream)
        K.dcp_lse_merge(w.c, o_part, lse_part, base, o, lse)
        if ev is not None:
            ev[3].record(stream)

    for i in range(warmup):
        step(i % len(groups))
    torch.cuda.synchronize()
    assert all(g.status() == 0 for g in groups), [g.status() for g in groups]
    for g in groups:
        g.seq_len = new_len.clone()
    log(f"warmup {warmup} steps done; timing {steps} steps")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(i % len(groups), evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert all(g.status() == 0 for g in groups), [g.status() for g in groups]
    r = dict(lens=lens, max_len=max_len, wall_ms=wall * 1e3 / steps)
    r["t_write"] = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    r["t_dec"] = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    r["t_merge"] = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    r["t_step"] = evs[0][0].elapsed_time(evs[-1][3]) / steps
    dec_each = sorted(e[1].elapsed_time(e[2]) for e in evs)
    r["dec_med"] = dec_each[len(dec_each) // 2]
    r["dec_p90"] = dec_each[min(len(dec_each) - 1, (9 * len(dec_each)) // 10)]
    log(f"per step: wall {r['wall_ms'] * 1e3:.1f} us; events: write {r['t_write'] * 1e3:.1f} us, decode "
        f"{r['t_dec'] * 1e3:.1f} us, merge {r['t_merge'] * 1e3:.1f} us, step {r['t_step'] * 1e3:.1f} us")
    # one real rank's share: rank 0's pool alone (rank_begin 0, rank_count 1), as one GPU
    # of a c-GPU group would run it (its own, smaller work plan)
    r["t_share"] = None
    if share:
        g = groups[0]
        ws1 = torch.empty(max(K.mla_decode_workspace_size(g.layout, 1, w.B, w.q_len, w.H, max_len) // 4, 4),
                          dtype=torch.float32, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for k in range(-2, len(ev)):
            if k >= 0:
                ev[k][0].record(stream)
            K.mla_decode_partial(g.layout, g.pools, g.pool_scales, 0, 1, q, g.block_table, new_len, max_len,
                                 w.sm_scale, base, w.causal, o_part[:1], lse_part[:1], ws1, g.dev_status)
            if k >= 0:
                ev[k][1].record(stream)
        torch.cuda.synchronize()
        assert g.status() == 0, g.status()
        r["t_share"] = sorted(a.elapsed_time(b) for a, b in ev)[len(ev) // 2]
    log(f"decode median {r['dec_med'] * 1e3:.1f} us, p90 {r['dec_p90'] * 1e3:.1f} us"
        + ("" if r["t_share"] is None else f"; one rank's share {r['t_share'] * 1e3:.1f} us"))
    # The same layer-step captured in a HIP graph (one per pool copy) and replayed, as a serving
    # loop that captures its decode step runs it: the host's per-call launch cost (ctypes and the
    # binding's checks, four entry points per step) leaves the step.  Every replay does the whole
    # step (page restore, allocation, scatter, decode with its device-side plan, merge); the
    # outputs of the last replay must equal the eager step's bit for bit.
    r["t_step_graph"] = None
    if graph:
        ref_o, ref_lse = o.clone(), lse.clone()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)  # warm the entry points on a side stream before capture, as torch asks
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for gi in range(len(groups)):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(gi)
            graphs.append(gr)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        r["t_step_graph"] = e0.elapsed_time(e1) / steps
        assert all(g.status() == 0 for g in groups), [g.status() for g in groups]
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), "graph replay output differs from eager"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "graph replay lse differs from eager"
        del graphs, ref_o, ref_lse
        log(f"graph-replayed layer-step {r['t_step_graph'] * 1e3:.1f} us (outputs identical to the eager step)")
    for i in range(decode_only):
        g = groups[i % len(groups)]
        K.mla_decode_partial(g.layout, g.pools, g.pool_scales, 0, w.c, q, g.block_table, new_len, max_len,
                             w.sm_scale, base, w.causal, o_part, lse_part, ws, g.dev_status)
    if calib_copy_mib:
        n = calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    del groups, o_part, lse_part, o, lse, ws, q
    torch.cuda.empty_cache()
    r["acct"] = accounting.layer_step(w, lens)
    r["share_acct"] = accounting.rank_share(w, lens, 0)
    return r


def summary_of(w, r):
    """Per-workload figures of the JSON line (decode us, roofline fractions, one rank's share)."""
    acct, sh = r["acct"], r["share_acct"]
    roof = roofline_of(w, acct["flops"], acct["decode_bytes"], r["t_dec"])
    out = {"workload": w.name, "decode_us": round(r["t_dec"] * 1e3, 2),
           "decode_median_us": round(r["dec_med"] * 1e3, 2), "decode_p90_us": round(r["dec_p90"] * 1e3, 2),
           "us_per_layer_step": round(r["wall_ms"] * 1e3, 2),
           "us_per_layer_step_graph": None if r["t_step_graph"] is None else round(r["t_step_graph"] * 1e3, 2),
           "bound": roof["bound"], "frac": round(roof["frac"], 4),
           "hbm_frac": round(roof["hbm_frac"], 4), "mfma_frac": round(roof["mfma_frac"], 4),
           "decode_gbps": round(roof["gbps"], 1), "decode_tflops": round(roof["tflops"], 2)}
    if r["t_share"] is not None:
        sr = roofline_of(w, sh["flops"], sh["decode_bytes"], r["t_share"])
        out.update({"one_rank_share_us": round(r["t_share"] * 1e3, 2), "one_rank_share_frac": round(sr["frac"], 4),
                    "one_rank_share_hbm_frac": round(sr["hbm_frac"], 4)})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=HEADLINE, help="workload of the headline line")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="other workloads timed in the same run and reported under 'workloads' ('' for none)")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--copies", type=int, default=2, help="pool copies used in rotation")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--interleave", type=int, default=None,
                    help="KV interleave size I (a divisor of the page size; the workload's own by default)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB once (HBM counter calibration)")
    ap.add_argument("--no-share", action="store_true",
                    help="skip timing one rank's share (profiling runs that should hold only group launches)")
    ap.add_argument("--op", choices=("step", "read", "relayout"), default="step",
                    help="what to time: the decode layer-step (default) or one of the layout copies")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed layer-step timing (profiling runs)")
    ap.add_argument("--decode-only", type=int, default=0,
                    help="after the timed steps, launch the decode entry point this many more times (profiling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; the c-rank DCP group is emulated on that GPU "
              "(--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_sharded_mla_amd as K
    from workloads import configs

    w = configs.BY_NAME[args.config]
    if args.interleave is not None:
        w = configs.scaled(w, interleave=args.interleave, name=w.name)
    if args.op != "step":
        return bench_copy(args, w)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    K.load_library()
    torch.cuda.set_device(0)

    r = time_workload(w, args.steps, args.warmup, args.copies, not args.no_share, args.decode_only,
                      args.calib_copy_mib, not args.no_graph)
    acct = r["acct"]
    lens, max_len = r["lens"], r["max_len"]
    ms_per_step = r["wall_ms"]
    kv_gbps = acct["kv_bytes"] / (ms_per_step * 1e-3) / 1e9
    tflops = acct["flops"] / (ms_per_step * 1e-3) / 1e12
    rf = roofline_of(w, acct["flops"], acct["decode_bytes"], r["t_dec"])
    if rf["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": round(rf["tflops"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(rf["frac"], 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(rf["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(rf["frac"], 4)}
    roof["traffic"] = load_traffic(w.name)
    roof["kernel"] = "mla_decode_partial (decode kernel + work plan and split combine when units split)"
    roof["algorithmic_bytes_per_launch"] = acct["decode_bytes"]
    roof["flops_per_launch"] = acct["flops"]
    roof["hbm_frac"] = round(rf["hbm_frac"], 4)
    roof["mfma_frac"] = round(rf["mfma_frac"], 4)
    roof["launch_us"] = round(r["t_dec"] * 1e3, 2)

    out = {
        "metric": "DCP MLA decode: achieved KV GB/s & % roofline; TFLOP/s; us per layer-step",
        "value": round(kv_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q and latent KV" + (", e4m3 + fp32 per-token scale" if w.kv_dtype == "fp8"
                                                              else ", bf16") + ")",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "q_len": w.q_len, "dcp": w.c, "page": w.P,
                   "interleave": w.interleave, "kv": w.kv_dtype, "context_tokens": int(lens.sum()), "max_len": max_len,
                   "lse_base": w.lse_base, "emulated_ranks_on_one_gpu": w.c},
        "us_per_layer_step": round(ms_per_step * 1e3, 2),
        "us_per_layer_step_graph": None if r["t_step_graph"] is None else round(r["t_step_graph"] * 1e3, 2),
        "tflops": round(tflops, 2),
        "kernel_us": {"alloc+kv_write": round(r["t_write"] * 1e3, 2), "mla_decode_partial": round(r["t_dec"] * 1e3, 2),
                      "dcp_lse_merge": round(r["t_merge"] * 1e3, 2),
                      "mla_decode_partial_median": round(r["dec_med"] * 1e3, 2),
                      "mla_decode_partial_p90": round(r["dec_p90"] * 1e3, 2),
                      "one_rank_share_decode": None if r["t_share"] is None else round(r["t_share"] * 1e3, 2)},
        "roofline": roof,
    }
    if r["t_share"] is not None:
        out["one_rank_share"] = {k: v for k, v in summary_of(w, r).items() if k.startswith("one_rank")}
    extras = [x for x in args.extras.split(",") if x and x != w.name]
    if extras:
        out["workloads"] = {}
        for name in extras:
            we = configs.BY_NAME[name]
            re_ = time_workload(we, args.extra_steps, min(args.warmup, 5), args.copies, not args.no_share,
                                graph=not args.no_graph)
            out["workloads"][name] = summary_of(we, re_)
    if not args.no_cpu_baseline:
        log(f"timing the oracle on the host for about {args.cpu_budget:.0f} s")
        out["cpu_baseline"] = cpu_baseline(w, lens, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def copy_cpu_baseline(op, w, lens, budget_s: float):
    """The oracle's read_rows / relayout_dense timed on whole requests of the workload."""
    import numpy as np
    from oracle import layout as OL
    from workloads import accounting
    rb = accounting.kv_bytes_per_token(w) - (4 if w.kv_dtype == "fp8" else 0)
    P, c = w.P, w.c
    t_total, done, n = 0.0, 0, 0
    rng = np.random.default_rng(0)
    for b in range(w.B):
        L = int(lens[b])
        vp = P * c
        nv = (L + vp - 1) // vp
        bt = np.arange(nv, dtype=np.int32)[None, :]
        pools = rng.integers(0, 256, size=(c, nv * P, rb), dtype=np.uint8)
        t0 = time.perf_counter()
        if op == "read":
            OL.read_rows(pools, bt, [L], [0, L], P, c, w.interleave)
        else:
            src = rng.integers(0, 256, size=(((L + P - 1) // P) * P, rb), dtype=np.uint8)
            sbt = np.arange((L + P - 1) // P, dtype=np.int32)[None, :]
            OL.relayout_dense(src, sbt, [L], P, c, pools, bt, 0, c, w.interleave)
        t_total += time.perf_counter() - t0
        done += 2 * L * accounting.kv_bytes_per_token(w)
        n += 1
        if t_total >= budget_s:
            break
    return {"value": round(done / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"requests 0..{n - 1} of {w.name} ({n}/{w.B}), {op} of every row in a Python loop, "
                      f"{t_total:.1f} s", "seconds": round(t_total, 2)}


def bench_copy(args, w):
    """Time dcp_kv_read or dcp_kv_relayout over the workload's whole context."""
    import numpy as np
    import torch

    import kv_sharded_mla_amd as K
    from kv_sharded_mla_amd.group import DcpGroup
    from workloads import accounting, gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    K.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lens = gen.lengths(w)
    P, c = w.P, w.c
    fp8 = w.kv_dtype == "fp8"
    rb = accounting.kv_bytes_per_token(w) - (4 if fp8 else 0)
    n_tok = int(lens.sum())
    log(f"{args.op} on {w.name}: B={w.B} c={c} P={P} I={w.interleave} kv={w.kv_dtype} sum(L)={n_tok}")
    # dense DCP1 pool with shuffled page ids, random bytes
    rng = np.random.default_rng(17)
    npg = [(int(L) + P - 1) // P for L in lens]
    ids = rng.permutation(sum(npg)).astype(np.int32)
    src_bt = np.full((w.B, max(npg)), -1, np.int32)
    k = 0
    for b, n in enumerate(npg):
        src_bt[b, :n] = ids[k:k + n]
        k += n
    gcpu = torch.Generator(device="cuda").manual_seed(5)
    src = torch.randint(0, 256, (sum(npg) * P * rb,), dtype=torch.uint8, device=dev, generator=gcpu)
    ssc = torch.rand(sum(npg) * P, device=dev, generator=gcpu) if fp8 else None
    num_pages = gen.pool_pages(w, lens)
    vp = P * c
    stride = int(max((int(L) + vp - 1) // vp for L in lens))
    g = DcpGroup(c, P, num_pages, K.KV_FP8_E4M3 if fp8 else K.KV_BF16, w.B, stride,
                 free_stack=gen.free_stack(w, num_pages), device="cuda:0", interleave=w.interleave)
    d_lens = torch.from_numpy(lens.astype(np.int32)).to(dev)
    K.dcp_alloc_virtual(g.layout, g.free_stack, g.free_top, torch.zeros_like(d_lens), d_lens, g.block_table,
                        g.dev_status)
    d_sbt = torch.from_numpy(src_bt).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    out = torch.empty((n_tok, rb), dtype=torch.uint8, device=dev)
    out_sc = torch.empty(n_tok, dtype=torch.float32, device=dev) if fp8 else None

    def launch():
        if args.op == "relayout":
            K.dcp_kv_relayout(g.layout, src, ssc, d_sbt, d_lens, 0, c, g.pools, g.pool_scales, g.block_table,
                              g.dev_status)
        else:
            K.dcp_kv_read(g.layout, g.pools, g.pool_scales, g.block_table, d_lens, cu, out, out_sc, g.dev_status)

    K.dcp_kv_relayout(g.layout, src, ssc, d_sbt, d_lens, 0, c, g.pools, g.pool_scales, g.block_table, g.dev_status)
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    assert g.status() == 0, g.status()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        launch()
        e[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert g.status() == 0, g.status()
    if args.calib_copy_mib:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
        del a
    t_launch = sum(a.elapsed_time(b) for a, b in evs) / args.steps       # ms
    moved = 2 * n_tok * accounting.kv_bytes_per_token(w)                  # read + write, rows and scales
    gbps = moved / (t_launch * 1e-3) / 1e9
    log(f"{args.op}: {t_launch * 1e3:.1f} us per launch, {gbps:.0f} GB/s")
    name = "dcp_kv_read (extend gather to token order)" if args.op == "read" else \
        "dcp_kv_relayout (DCP1 paged pool -> c owner pools)"
    out_json = {
        "metric": f"DCP KV {args.op}: achieved HBM GB/s (bytes read + written per launch)",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8",
        "data": "synthetic (random bytes in the " + ("e4m3 row + fp32 scale" if fp8 else "bf16 row") + " layout)",
        "config": {"workload": w.name, "op": args.op, "batch": w.B, "dcp": c, "page": P, "interleave": w.interleave,
                   "kv": w.kv_dtype, "context_tokens": n_tok, "emulated_ranks_on_one_gpu": c},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": load_copy_traffic(args.op, w.name),
                     "kernel": name,
                     "algorithmic_bytes_per_launch": moved, "launch_us": round(t_launch * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        log(f"timing the oracle on the host for about {args.cpu_budget:.0f} s")
        out_json["cpu_baseline"] = copy_cpu_baseline(args.op, w, lens, args.cpu_budget)
    else:
        out_json["cpu_baseline"] = None
    print(json.dumps(out_json), flush=True)


if __name__ == "__main__":
    main()
