"""Host logic of bench.py (CPU only): metric names, roofline choice, work counts, the CPU
baseline's fields."""
import importlib.util
import os

import numpy as np

from mla_latent_kv_lat_amd import configs, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(spec)
spec.loader.exec_module(bench)


def test_metric_names_follow_the_workload():
    assert bench.metric_name(configs.V2_DECODE) == \
        "MLA decode latent-cache GB/s + TFLOP/s and % roofline (bf16, B=32, T=4096)"
    assert "paged" in bench.metric_name(configs.PAGED_VARLEN)
    assert "s_q=4" in bench.metric_name(configs.SPEC_FP8) and "fp8" in bench.metric_name(configs.SPEC_FP8)


def test_roofline_bound_follows_the_arithmetic_intensity():
    # 1 query token: 2176 flop per token and head over 1152 bytes per token (ridge 314.6)
    # is memory-bound; 4 query tokens over an fp8 cache (644 bytes per token) are not.
    for cfg, bound in ((configs.V2_DECODE, "hbm"), (configs.LONG_CONTEXT, "hbm"), (configs.SPEC_FP8, "mfma")):
        lens = np.full(cfg.batch, cfg.seq_len)
        wc = bench.work_counts(cfg, lens)
        roof = bench.decode_roofline(cfg, wc, 1.0)
        assert roof["bound"] == bound, cfg.name
        if bound == "hbm":
            assert abs(roof["achieved"] - wc["decode_bytes"] / 1e-3 / 1e9) < 0.1
        else:
            assert abs(roof["achieved"] - wc["attn_flops"] / 1e-3 / 1e12) < 0.1
        assert 0 < roof["frac"] == round(roof["achieved"] / roof["peak"], 4)


def test_work_counts_of_the_headline():
    cfg = configs.V2_DECODE
    wc = bench.work_counts(cfg, np.full(cfg.batch, cfg.seq_len))
    assert wc["cache_bytes"] == 32 * 4096 * (512 * 2 + 64 * 2)
    assert wc["attn_flops"] == 128 * 32 * 4096 * (2 * 576 + 2 * 512)


def test_cpu_baseline_reports_cores_and_single_core():
    inp = synth.make_inputs(configs.TINY, 0)
    res = bench.cpu_baseline(inp, 0.05, 0.05)
    assert res["kind"] == "oracle" and res["value"] > 0
    assert 1 <= res["cores"] <= bench.host_cores()
    assert res["single_core"]["cores"] == 1 and res["single_core"]["value"] > 0
