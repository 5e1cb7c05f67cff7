"""Shared fixtures and glue for the test suite.

Markers:
  gpu -- needs an MI355X (gfx950) and the built libmla.so; run with ``-m gpu``.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU and the built HIP library")


def decoded(inp):
    """Float64 view of a synthetic workload, decoded by the oracle's own codecs.

    Returns a dict with q_nope, q_rope, w_uk, w_uv and the contiguous caches c_kv
    [B,T,d_c] and k_rope [B,T,d_r] (paged pools are gathered through the block table;
    fp8 latents are dequantized with their per-token scale).
    """
    from oracle import mla_oracle as O
    cfg = inp.cfg
    act = cfg.act_dtype
    d = {
        "q_nope": O.decode(inp.q_nope, act),
        "q_rope": O.decode(inp.q_rope, act),
        "w_uk": O.decode(inp.w_uk, act),
        "w_uv": O.decode(inp.w_uv, act),
    }
    if cfg.kv_dtype == "fp8":
        lat = O.dequantize_cache(inp.c_kv, inp.kv_scale)
    else:
        lat = O.decode(inp.c_kv, cfg.kv_dtype)
    rope = O.decode(inp.k_rope, act)
    if cfg.paged:
        lat = O.gather_pages(lat, inp.block_table, inp.seq_lens, cfg.seq_len)
        rope = O.gather_pages(rope, inp.block_table, inp.seq_lens, cfg.seq_len)
    d["c_kv"] = lat
    d["k_rope"] = rope
    d["seq_lens"] = inp.seq_lens
    d["scale"] = cfg.softmax_scale
    return d


def max_rel_err(got, ref):
    """max |got - ref| / max |ref| over one output tensor (finite reference entries)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.isfinite(ref)
    denom = np.max(np.abs(ref[m])) if m.any() else 0.0
    if denom == 0:
        return float(np.max(np.abs(got[m]))) if m.any() else 0.0
    return float(np.max(np.abs(got[m] - ref[m])) / denom)


def max_abs_err(got, ref):
    """max |got - ref| over the finite reference entries (used for log-sum-exp values,
    whose size, about ln T, would make a relative bar loose)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.isfinite(ref)
    return float(np.max(np.abs(got[m] - ref[m]))) if m.any() else 0.0
