"""Pins for the bytes/FLOPs accounting against the pages' footnote arithmetic.

The figures live in tests/golden/footnotes.json with their citation (vLLM
GLM-5.3 blog post, section "Why the numbers add up").
"""
import json
import os

import numpy as np

from workloads import accounting, configs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "footnotes.json")


def _g():
    with open(GOLD) as f:
        return json.load(f)


def test_flops_and_qo_bytes_per_head():
    g = _g()
    assert accounting.flops_per_score(g["qk_dims"], g["pv_dims"]) == g["flops_per_row_per_head"]
    assert accounting.query_output_bytes_per_head(g["qk_dims"], g["pv_dims"]) == g["qo_bytes_per_head"]
    assert g["row_bytes_kv"] + g["row_bytes_index"] == g["row_bytes_fp8_ds_mla"]


def test_sparse_mla_intensity_by_head_count():
    g = _g()
    rows_bytes = g["sparse_rows"] * g["row_bytes_fp8_ds_mla"]
    assert round(rows_bytes / 1e6, 2) == g["bytes_per_query_MB"]
    for key in ("heads_8", "heads_64"):
        h = g[key]["heads"]
        flops = h * g["sparse_rows"] * accounting.flops_per_score()
        nbytes = rows_bytes + h * accounting.query_output_bytes_per_head()
        assert round(flops / 1e6, 1) == round(g[key]["MFLOP"], 1) or round(flops / 1e6) == g[key]["MFLOP"]
        assert round(nbytes / 1e6, 2) == g[key]["MB"]
        assert round(flops / nbytes) == g[key]["flop_per_byte"]
    assert round(g["h200"]["dense_bf16_tflops"] / g["h200"]["hbm_tb_s"]) == g["h200"]["ridge_flop_per_byte"]


def test_million_token_kv_sizing():
    g = _g()
    t = g["per_token"]
    per_tok = t["mla_layers"] * t["mla_bytes"] + t["indexer_layers"] * t["indexer_bytes"] + t["mtp_bytes"]
    assert per_tok == t["total_bytes"]
    total = per_tok * g["tokens"]
    assert round(total / 2**30, 1) == g["total_GiB"]
    assert round(total / 2**30 / g["dcp"], 1) == g["per_gpu_GiB"]


def test_workload_intensities():
    # 16 heads of bf16 latent rows: 16*2176/1152 ~ 30 FLOP/B; 128 heads ~ 242; fp8 64 heads ~ 240
    st = accounting.layer_step(configs.TP_LOCAL, [32768] * 64)
    assert st["kv_bytes"] == 64 * 32768 * 1152
    assert abs(st["intensity"] - 16 * 2176 / 1152) < 1e-9
    st = accounting.layer_step(configs.LONG_FP8, [1 << 20] * 4)
    assert st["kv_bytes"] == 4 * (1 << 20) * 580
    v = accounting.layer_step(configs.VERIFY, [65536] * 16)
    # q_len 4 causal: rows see L-3, L-2, L-1, L positions
    assert v["flops"] == 16 * 128 * 2176 * (4 * 65536 - 6)
    assert np.isclose(v["intensity"], 128 * 2176 * (4 * 65536 - 6) / (65536 * 1152))


def test_rank_shares_add_up_to_the_group():
    # every position has exactly one owner, so the ranks' KV bytes and scores sum to
    # the group's, for any interleave size
    from workloads import configs as C
    for w in C.ALL:
        for I in (1, 16):
            wi = C.scaled(w, interleave=I) if w.P % I == 0 else w
            lens = np.array([1, 5, 777, 4096, 33333][: wi.B] + [100] * max(0, wi.B - 5))
            tot = accounting.layer_step(wi, lens)
            kv = sum(accounting.rank_share(wi, lens, r)["kv_bytes"] for r in range(wi.c))
            fl = sum(accounting.rank_share(wi, lens, r)["flops"] for r in range(wi.c))
            assert kv == tot["kv_bytes"] and fl == tot["flops"], (w.name, I)
