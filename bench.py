#!/usr/bin/env python3
"""Benchmark of one weight-absorbed MLA decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--replicas R]

A step is the whole hot path over one batch: mla_absorb_q -> mla_decode (split-K decode
kernel + combine) -> mla_absorb_out, on synthetic inputs already resident in HBM.  The
timed loop cycles over R copies of the cache and weights at distinct addresses so that
the 151 MB bf16 cache of the headline workload cannot be served from the 256 MB
last-level (Infinity) cache between steps.

Prints one JSON line:
  value        latent-cache GB/s of the whole step (cache bytes / step time)
  roofline     the decode call (its kernels) against the 8 TB/s HBM peak, timed with HIP
               events around each call inside the timed loop
  configs      the decode call alone on the other full-size workloads (paged variable-length,
               long context, speculative fp8), each with its own roofline (the fp8 one also
               with both products on the fp8 matrix instruction, labelled), plus the headline's
               decode call with its cache left warm in the last-level cache (labelled)
  cpu_baseline the CPU oracle (fp64 numpy, absorbed form) on a bounded sample of the
               same workload, on this host's cores, and on one core
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 flop / clk / CU
FP8_MFMA_PEAK_TFS = 5033.2   # twice the bf16 rate (dense fp8)


def bytes_of(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "fp8": 1}[dtype]


def work_counts(cfg, seq_lens) -> dict:
    """Algorithmic work of one step: every cache byte read once, q in / o out once."""
    L = np.asarray(seq_lens, np.int64)
    kvb, ab = bytes_of(cfg.kv_dtype), bytes_of(cfg.act_dtype)
    per_token = cfg.d_latent * kvb + cfg.d_rope * ab + (4 if cfg.kv_dtype == "fp8" else 0)
    cache = int(L.sum()) * per_token
    rows = cfg.batch * cfg.q_len * cfg.n_heads
    qo = rows * ((cfg.d_latent + cfg.d_rope) * ab + cfg.d_latent * ab + 4)
    vis = sum(max(0, min(int(l) - cfg.q_len + i + 1, int(l))) for l in L for i in range(cfg.q_len))
    attn_flops = cfg.n_heads * vis * (2 * (cfg.d_latent + cfg.d_rope) + 2 * cfg.d_latent)
    absorb_flops = 2 * rows * cfg.d_head * cfg.d_latent
    weight_bytes = 2 * cfg.n_heads * cfg.d_head * cfg.d_latent * ab
    return {"cache_bytes": cache, "qo_bytes": qo, "attn_flops": attn_flops,
            "absorb_flops_each": absorb_flops, "weight_bytes": weight_bytes,
            "decode_bytes": cache + qo}


def decode_sources_sha256() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mla_latent_kv_lat_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith(("decode_", "device_common", "mfma_common", "mla_internal")):
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed rocprofv3 counter summary, if it was
    taken on the current decode sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"decode_sources_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"hbm_bytes_per_decode_call:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_val) or m_sha.group(1) != decode_sources_sha256():
        return None
    return float(m_val.group(1))


def metric_name(cfg) -> str:
    lens = f"T={cfg.seq_len}" if not cfg.paged else f"T<={cfg.seq_len}, paged"
    sq = f", s_q={cfg.q_len}" if cfg.q_len > 1 else ""
    return f"MLA decode latent-cache GB/s + TFLOP/s and % roofline ({cfg.kv_dtype}, B={cfg.batch}, {lens}{sq})"


def decode_roofline(cfg, wc, call_ms: float) -> dict:
    """The decode call against HBM for the streaming workloads, against the bf16 matrix peak
    where the arithmetic intensity is past the ridge (speculative multi-token fp8).  `traffic`
    is the call's measured HBM bytes either way."""
    mfma_bound = wc["attn_flops"] / wc["decode_bytes"] > BF16_MFMA_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved = wc["attn_flops"] / (call_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFS, 4),
                "traffic": measured_traffic(cfg.name)}
    achieved = wc["decode_bytes"] / (call_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name)}


def time_decode_calls(w, calls: int, warmup: int, ramp_ms: float = 200.0) -> list:
    """Milliseconds of each of `calls` decode calls (HIP events on the stream the library
    launches on), cycling over the workload's cache replicas, after `ramp_ms` of untimed
    calls (the clock drops while the host prepares inputs) and `warmup` more."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ramp_ms:
        for k in range(10):
            w.decode(w.caches[k % len(w.caches)])
        torch.cuda.synchronize()
    for k in range(warmup):
        w.decode(w.caches[k % len(w.caches)])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for k in range(calls):
        ev[k][0].record()
        w.decode(w.caches[k % len(w.caches)])
        ev[k][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def side_workload(cfg, calls: int, warmup: int) -> dict:
    """The decode call alone on one full-size workload (queries absorbed once beforehand),
    its cache bigger than the last-level cache, so every call streams it from HBM."""
    import torch
    from mla_latent_kv_lat_amd import synth
    from mla_latent_kv_lat_amd.runner import DeviceWorkload
    t0 = time.perf_counter()
    inp = synth.make_inputs(cfg, 0)
    wc = work_counts(cfg, inp.seq_lens)
    w = DeviceWorkload(inp, replicas=1)
    w.absorb_q()
    gen_s = time.perf_counter() - t0
    ms = time_decode_calls(w, calls, warmup)
    avg = float(np.mean(ms))
    out = {"metric": metric_name(cfg), "workload": cfg.name, "decode_call_us": round(avg * 1e3, 2),
           "decode_call_us_p10_p90": [round(float(np.percentile(ms, 10)) * 1e3, 2),
                                      round(float(np.percentile(ms, 90)) * 1e3, 2)],
           "value": round(wc["cache_bytes"] / (avg * 1e-3) / 1e9, 2), "unit": "GB/s",
           "tflops": round(wc["attn_flops"] / (avg * 1e-3) / 1e12, 2),
           "decode_tokens_per_s": round(cfg.batch * cfg.q_len / (avg * 1e-3), 1),
           "dtype": cfg.kv_dtype, "cache_bytes": wc["cache_bytes"], "splits": w.plan[0], "calls": calls,
           "roofline": decode_roofline(cfg, wc, avg)}
    print(f"[bench] {cfg.name}: decode call {avg * 1e3:.1f} us over {calls} calls (inputs {gen_s:.1f} s)",
          file=sys.stderr, flush=True)
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cfg.kv_dtype == "fp8":
        # The opt-in approximation with both products on the fp8 matrix instruction
        # (dims.fp8_scores = 2): same inputs, its own rounding of the query and of P.
        w8 = DeviceWorkload(inp, replicas=1, fp8_scores=2)
        w8.absorb_q()
        ms8 = time_decode_calls(w8, calls, warmup)
        avg8 = float(np.mean(ms8))
        tf8 = wc["attn_flops"] / (avg8 * 1e-3) / 1e12
        roof8 = decode_roofline(cfg, wc, avg8)
        roof8["traffic"] = measured_traffic(cfg.name + "_fp8products")
        roof8["fp8_peak_frac"] = round(tf8 / FP8_MFMA_PEAK_TFS, 4)
        out["fp8_products"] = {
            "note": "dims.fp8_scores = 2: query and probabilities rounded to e4m3, both products on the fp8 "
                    "matrix instruction (an approximation, not the exact path above)",
            "decode_call_us": round(avg8 * 1e3, 2), "tflops": round(tf8, 2),
            "decode_tokens_per_s": round(cfg.batch * cfg.q_len / (avg8 * 1e-3), 1), "roofline": roof8}
        print(f"[bench] {cfg.name} fp8 products: decode call {avg8 * 1e3:.1f} us", file=sys.stderr, flush=True)
        del w8
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity), not the machine's count."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(inp, budget_s: float, single_core_budget_s: float = 0.0) -> dict:
    """Time the CPU oracle's absorbed form on whole sequences until the time budget is spent
    (cycling over the batch again when it is done sooner); then, with a budget, the same on
    one core (its BLAS limited to one thread)."""
    from oracle import mla_oracle as O
    cfg = inp.cfg
    act = cfg.act_dtype

    def dec_seq(b_list):
        q_nope = O.decode(inp.q_nope[b_list], act)
        q_rope = O.decode(inp.q_rope[b_list], act)
        if cfg.paged:
            lat = O.decode(inp.c_kv, cfg.kv_dtype)
            rope = O.decode(inp.k_rope, act)
            lat = O.gather_pages(lat, inp.block_table[b_list], inp.seq_lens[b_list], cfg.seq_len)
            rope = O.gather_pages(rope, inp.block_table[b_list], inp.seq_lens[b_list], cfg.seq_len)
        elif cfg.kv_dtype == "fp8":
            lat = O.dequantize_cache(inp.c_kv[b_list], inp.kv_scale[b_list])
            rope = O.decode(inp.k_rope[b_list], act)
        else:
            lat = O.decode(inp.c_kv[b_list], cfg.kv_dtype)
            rope = O.decode(inp.k_rope[b_list], act)
        return q_nope, q_rope, lat, rope

    w_uk, w_uv = O.decode(inp.w_uk, act), O.decode(inp.w_uv, act)

    def run(budget):
        done, secs = [], 0.0
        b = 0
        while secs < budget:
            # Grow the sample in whole sequences until the time budget is spent.
            q_nope, q_rope, lat, rope = dec_seq([b])
            t0 = time.perf_counter()
            O.mla_absorbed(q_nope, q_rope, lat, rope, w_uk, w_uv, inp.seq_lens[[b]], cfg.softmax_scale)
            secs += time.perf_counter() - t0
            done.append(b)
            b = (b + 1) % cfg.batch
        return done, secs

    def sample(done, secs):
        return (f"{len(done)} sequence passes over the {cfg.batch} sequences of {cfg.name}, whole absorbed "
                f"decode (q absorption, attention, output absorption) in fp64, {secs:.2f} s wall")

    done, secs = run(budget_s)
    wc = work_counts(cfg, inp.seq_lens[done])
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    res = {"value": wc["cache_bytes"] / secs / 1e9, "unit": "GB/s", "cores": int(min(threads, host_cores())),
           "kind": "oracle", "sample": sample(done, secs)}
    if single_core_budget_s > 0:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            done1, secs1 = run(single_core_budget_s)
        res["single_core"] = {"value": work_counts(cfg, inp.seq_lens[done1])["cache_bytes"] / secs1 / 1e9,
                              "unit": "GB/s", "cores": 1, "sample": sample(done1, secs1)}
    return res


def bench_cache_append(args, cfg) -> int:
    """Time mla_cache_append alone: the new tokens' projection onto W_DKV / W_KR, rotation
    and scatter into a paged pool.  HBM-bound on the two weight matrices."""
    import torch
    from mla_latent_kv_lat_amd import capi, synth
    from mla_latent_kv_lat_amd.runner import to_device
    dm = args.d_model
    inp = synth.make_append_inputs(cfg, dm, 0)
    act, kv = cfg.act_dtype, cfg.kv_dtype
    dc, dr, bs, M = cfg.d_latent, cfg.d_rope, cfg.block_size, cfg.batch * cfg.q_len
    ab = 4 if act == "f32" else 2
    kb = {"f32": 4, "bf16": 2, "fp8": 1}[kv]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    x = to_device(inp.x, act, "cuda")
    reps = []
    for _ in range(max(1, args.replicas)):  # weight replicas, cycled: streamed from HBM each call
        reps.append((to_device(inp.w_dkv, act, "cuda"), to_device(inp.w_kr, act, "cuda")))
    c_pool = torch.zeros((inp.n_blocks, bs, dc), dtype=tdt[kv], device="cuda")
    r_pool = torch.zeros((inp.n_blocks, bs, dr), dtype=tdt[act], device="cuda")
    s_pool = torch.zeros((inp.n_blocks, bs), dtype=torch.float32, device="cuda") if kv == "fp8" else None
    table = to_device(inp.block_table, "i32", "cuda")
    lens = to_device(inp.seq_lens, "i32", "cuda")
    d = capi.dims_from_config(cfg)
    ws = torch.empty(capi.mla_cache_append_workspace_bytes(d, dm), dtype=torch.uint8, device="cuda")

    def call(k):
        wd, wk = reps[k % len(reps)]
        capi.mla_cache_append(d, x, wd, wk, c_pool, r_pool, table, lens, ws, kv_scale_pool=s_pool,
                              kv_dtype=capi.DTYPE_CODES[kv])

    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < args.ramp_ms:
        for _ in range(20):
            call(n)
            n += 1
        torch.cuda.synchronize()
    for k in range(args.warmup):
        call(k)
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(K):
        ev[k][0].record()
        call(k)
        ev[k][1].record()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / K
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    weight_bytes = dm * (dc + dr) * ab
    alg_bytes = weight_bytes + M * dm * ab + M * (dc * kb + dr * ab + (4 if kv == "fp8" else 0))
    flops = 2.0 * M * dm * (dc + dr)
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    print(f"[bench] cache_append {cfg.name} d_model={dm}: {call_ms * 1e3:.2f} us/call", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "MLA cache append (new-token latent + rotated RoPE key into the paged pool) GB/s",
        "value": round(alg_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "clock_ramp": {"ms": args.ramp_ms, "steps": n},
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if act == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian hidden states and random-init projections)",
        "config": {"workload": f"cache_append_{cfg.name}_dmodel{dm}", "batch": cfg.batch, "q_len": cfg.q_len,
                   "d_model": dm, "d_latent": dc, "d_rope": dr, "kv_dtype": kv, "block_size": bs,
                   "weight_replicas": len(reps)},
        "call_us": round(call_ms * 1e3, 3), "tflops": round(flops / (call_ms * 1e-3) / 1e12, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }), flush=True)
    return 0


def bench_prefill(args, cfg) -> int:
    """Time mla_prefill alone: B prompts of T tokens, every token a query (explicit form:
    decompression of K and V per head, then causal attention).  Bound by the matrix cores."""
    import torch
    from mla_latent_kv_lat_amd import capi, synth
    from mla_latent_kv_lat_amd.runner import to_device
    B, T = args.prefill_batch, args.prefill_len
    pc = cfg.with_(batch=B, q_len=T, seq_len=T, cfg_id=50, paged=False, kv_dtype="bf16")
    print(f"[bench] prefill B={B} T={T} n_h={pc.n_heads}: generating inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(pc, 0, lengths=np.full(B, T, np.int32))
    dev = lambda a, k="bf16": to_device(a, k, "cuda")
    q_nope, q_rope, c_kv, k_rope = dev(inp.q_nope), dev(inp.q_rope), dev(inp.c_kv), dev(inp.k_rope)
    w_uk, w_uv, lens = dev(inp.w_uk), dev(inp.w_uv), dev(inp.seq_lens, "i32")
    H, dh = pc.n_heads, pc.d_head
    out = torch.empty(B, T, H, dh, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, T, H, dtype=torch.float32, device="cuda")
    d = capi.dims_from_config(pc)
    ws = torch.empty(capi.mla_prefill_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")

    def call():
        capi.mla_prefill(d, q_nope, q_rope, c_kv, k_rope, T, lens, w_uk, w_uv, out, lse, ws)

    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < args.ramp_ms:
        call()
        n += 1
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / K
    decomp = 2.0 * B * T * pc.d_latent * H * 2 * dh
    attn = 2.0 * H * B * (T * (T + 1) / 2) * (dh + pc.d_rope + dh)
    tf = (decomp + attn) / (ms * 1e-3) / 1e12
    print(f"[bench] prefill: {ms * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "MLA prefill (explicit form) TFLOP/s", "value": round(tf, 1), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "clock_ramp": {"ms": args.ramp_ms, "steps": n},
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian prompts, cache and random-init weights)",
        "config": {"workload": f"prefill_bf16_b{B}_t{T}_h{H}", "batch": B, "seq_len": T, "n_heads": H,
                   "d_head": dh, "d_latent": pc.d_latent, "d_rope": pc.d_rope},
        "gflop": {"decompression": round(decomp / 1e9, 1), "attention": round(attn / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tf / BF16_MFMA_PEAK_TFS, 4), "traffic": None},
    }), flush=True)
    return 0


def bench_projections(args, cfg) -> int:
    """Time the weight-streaming steps around the attention at DeepSeek-V2 widths for the
    batch's new tokens: the query path from hidden states, unfolded (c_q = x W_DQ, the
    content and RoPE up-projections, key absorption) and folded (c_q, the RoPE
    up-projection, c_q W_UQK), and the output path (value absorption, O W_O).  Each is
    bound by its weight bytes, streamed from HBM (replicas cycled)."""
    import torch
    from mla_latent_kv_lat_amd import capi
    M, dm, dcq, H, dh, dr, dc = cfg.batch * cfg.q_len, args.d_model, args.d_cq, cfg.n_heads, cfg.d_head, cfg.d_rope, cfg.d_latent
    g = torch.Generator(device="cpu").manual_seed(0)
    rnd = lambda *shape, std=1.0: (torch.randn(*shape, generator=g) * std).to(torch.bfloat16).cuda()
    x = rnd(M, dm)
    reps = []
    for _ in range(max(1, args.replicas)):
        w = {"dq": rnd(dm, dcq, std=dm ** -0.5), "uq": rnd(dcq, H * dh, std=dcq ** -0.5),
             "qr": rnd(dcq, H * dr, std=dcq ** -0.5), "uk": rnd(H, dh, dc, std=dc ** -0.5),
             "uv": rnd(H, dc, dh, std=dc ** -0.5), "o": rnd(H * dh, dm, std=(H * dh) ** -0.5)}
        w["uqk"] = torch.empty(dcq, H * dc, dtype=torch.bfloat16, device="cuda")
        capi.mla_absorb_q(capi.dims(dcq, 1, H, dh, dc, dr, 1.0), w["uq"].view(dcq, 1, H, dh), w["uk"], w["uqk"])
        w["uvo"] = torch.empty(H * dc, dm, dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        t_f = time.perf_counter()
        capi.mla_fold_output_weights(w["uv"], w["o"], w["uvo"])
        torch.cuda.synchronize()
        fold_ms = (time.perf_counter() - t_f) * 1e3
        reps.append(w)
    c_q = torch.empty(M, dcq, dtype=torch.bfloat16, device="cuda")
    q_nope = torch.empty(M, H * dh, dtype=torch.bfloat16, device="cuda")
    q_rope = torch.empty(M, H * dr, dtype=torch.bfloat16, device="cuda")
    q_lat = torch.empty(M, H * dc, dtype=torch.bfloat16, device="cuda")
    o_lat = rnd(M, H * dc)
    heads = torch.empty(M, H * dh, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(M, dm, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(capi.mla_linear_workspace_bytes(M, K, N) for K, N in
                         ((dm, dcq), (dcq, H * dh), (dcq, H * dr), (dcq, H * dc), (H * dh, dm), (H * dc, dm))),
                     dtype=torch.uint8, device="cuda")
    dq = capi.dims(M, 1, H, dh, dc, dr, 1.0)

    def query_unfolded(w):
        capi.mla_linear(x, w["dq"], c_q, ws)
        capi.mla_linear(c_q, w["uq"], q_nope, ws)
        capi.mla_linear(c_q, w["qr"], q_rope, ws)
        capi.mla_absorb_q(dq, q_nope.view(M, 1, H, dh), w["uk"], q_lat.view(M, 1, H, dc))

    def query_folded(w):
        capi.mla_linear(x, w["dq"], c_q, ws)
        capi.mla_linear(c_q, w["qr"], q_rope, ws)
        capi.mla_linear(c_q, w["uqk"], q_lat, ws)

    def output(w):
        capi.mla_absorb_out(dq, o_lat.view(M, 1, H, dc), w["uv"], heads.view(M, 1, H, dh))
        capi.mla_linear(heads, w["o"], y, ws)

    def output_folded(w):
        capi.mla_linear(o_lat, w["uvo"], y, ws)

    def timed(fn):
        for k in range(args.warmup):
            fn(reps[k % len(reps)])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(args.steps):
            fn(reps[k % len(reps)])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.ramp_ms:
        query_unfolded(reps[0])
        torch.cuda.synchronize()
    ms_u, ms_f, ms_o, ms_of = timed(query_unfolded), timed(query_folded), timed(output), timed(output_folded)
    b = lambda n: 2 * n
    bytes_u = b(dm * dcq + dcq * H * dh + dcq * H * dr + H * dh * dc)
    bytes_f = b(dm * dcq + dcq * H * dr + dcq * H * dc)
    bytes_o = b(H * dc * dh + H * dh * dm)
    bytes_of = b(H * dc * dm)
    gbs = lambda nb, ms: nb / (ms * 1e-3) / 1e9
    print(f"[bench] query unfolded {ms_u * 1e3:.1f} us, folded {ms_f * 1e3:.1f} us, output {ms_o * 1e3:.1f} us, "
          f"output folded {ms_of * 1e3:.1f} us (fold {fold_ms:.2f} ms, once per weight set)", file=sys.stderr, flush=True)
    ach = gbs(bytes_u, ms_u)
    print(json.dumps({
        "metric": "MLA query path from hidden states (unfolded), weight GB/s", "value": round(ach, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_u, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian hidden states and random-init weights)",
        "config": {"workload": f"projections_m{M}_dmodel{dm}_dcq{dcq}_h{H}", "tokens": M, "d_model": dm,
                   "d_cq": dcq, "n_heads": H, "d_head": dh, "d_rope": dr, "d_latent": dc,
                   "weight_replicas": len(reps)},
        "query_unfolded_us": round(ms_u * 1e3, 2), "query_unfolded_weight_MB": round(bytes_u / 1e6, 1),
        "query_folded_us": round(ms_f * 1e3, 2), "query_folded_weight_MB": round(bytes_f / 1e6, 1),
        "output_us": round(ms_o * 1e3, 2), "output_weight_MB": round(bytes_o / 1e6, 1),
        "output_GBs": round(gbs(bytes_o, ms_o), 1), "query_folded_GBs": round(gbs(bytes_f, ms_f), 1),
        "output_folded_us": round(ms_of * 1e3, 2), "output_folded_weight_MB": round(bytes_of / 1e6, 1),
        "output_folded_GBs": round(gbs(bytes_of, ms_of), 1), "output_fold_ms_once": round(fold_ms, 3),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None},
    }), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--ramp-ms", type=float, default=300.0,
                    help="untimed steps run for this long before the warmup steps, so the GPU "
                         "clocks have left their idle state (input generation leaves it idle)")
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--fp8-scores", type=int, choices=(0, 1, 2), default=0,
                    help="1: latent score term as an fp8 matrix product (fp8-cache workloads)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--cpu-single-core-budget", type=float, default=8.0,
                    help="seconds of the oracle on one core (0: skip)")
    ap.add_argument("--side-workloads", default="paged_varlen_bf16_b64,long_bf16_b4_t131072,spec4_fp8_b128_t8192",
                    help="comma-separated workloads whose decode call is also timed (empty: none)")
    ap.add_argument("--side-calls", type=int, default=40, help="timed decode calls per side workload")
    ap.add_argument("--warm-calls", type=int, default=100,
                    help="decode calls timed with the cache left in the last-level cache (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter calibration)")
    ap.add_argument("--prefill-batch", type=int, default=1, help="prompts for --stage prefill")
    ap.add_argument("--prefill-len", type=int, default=4096, help="prompt length for --stage prefill")
    ap.add_argument("--d-cq", type=int, default=1536, help="query latent width for --stage projections")
    ap.add_argument("--stage", choices=("step", "cache_append", "prefill", "projections"), default="step",
                    help="step: absorb_q + decode + absorb_out (the headline); cache_append: the "
                         "cache write of the new tokens alone; prefill: mla_prefill of whole prompts; "
                         "projections: query path from hidden states (unfolded and folded) and output path")
    ap.add_argument("--d-model", type=int, default=5120, help="hidden width for --stage cache_append")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path is "
              "not sharded across GPUs.", file=sys.stderr)
        return 2

    import torch
    from mla_latent_kv_lat_amd import configs, synth
    from mla_latent_kv_lat_amd.runner import DeviceWorkload

    cfg = configs.BY_NAME[args.workload] if args.workload else configs.HEADLINE
    if args.stage == "cache_append":
        return bench_cache_append(args, cfg)
    if args.stage == "prefill":
        return bench_prefill(args, cfg)
    if args.stage == "projections":
        return bench_projections(args, cfg)
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg, 0)
    wc = work_counts(cfg, inp.seq_lens)
    w = DeviceWorkload(inp, split_tokens=args.split_tokens, replicas=args.replicas,
                       fp8_scores=args.fp8_scores)
    print(f"[bench] plan (splits, tokens/split) = {w.plan}; workspace {w.ws_bytes} B",
          file=sys.stderr, flush=True)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t_ramp = time.perf_counter()
    ramp_steps = 0
    while (time.perf_counter() - t_ramp) * 1e3 < args.ramp_ms:
        for _ in range(20):
            w.step()
        ramp_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    K = args.steps
    # The K timed steps, with nothing but the library's kernels on the stream: `value`.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(K):
        c = w.caches[k % len(w.caches)]
        w.absorb_q(c)
        w.decode(c)
        w.absorb_out(c)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / K
    # A second pass of K steps with events around each decode call (on the stream the
    # library launches on): the decode call's time for the roofline.  The events are kept
    # out of the first pass because each one adds a marker to the stream between kernels.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    evs, eve = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    evs.record()
    for k in range(K):
        c = w.caches[k % len(w.caches)]
        w.absorb_q(c)
        ev[k][0].record()
        w.decode(c)
        ev[k][1].record()
        w.absorb_out(c)
    eve.record()
    torch.cuda.synchronize()
    ms_step_ev = evs.elapsed_time(eve) / K
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    dec_avg = float(np.mean(dec_ms))
    print(f"[bench] timed {K} steps: {ms_step * 1e3:.1f} us/step ({ms_step_ev * 1e3:.1f} with events around "
          f"each decode call), decode call {dec_avg * 1e3:.1f} us "
          f"(p10 {np.percentile(dec_ms, 10) * 1e3:.1f}, p90 {np.percentile(dec_ms, 90) * 1e3:.1f})",
          file=sys.stderr, flush=True)

    roof = decode_roofline(cfg, wc, dec_avg)

    # The same decode call with one cache copy, called back to back: the 151 MB cache stays in
    # the 256 MB last-level cache between calls (not a cold-HBM figure; labelled as such).
    side = {}
    if args.warm_calls > 0:
        w1 = DeviceWorkload(inp, split_tokens=args.split_tokens, replicas=1, fp8_scores=args.fp8_scores)
        w1.absorb_q()
        warm_ms = time_decode_calls(w1, args.warm_calls, 20)
        warm_avg = float(np.mean(warm_ms))
        del w1
        side["last_level_cache_warm"] = {
            "workload": cfg.name, "note": "one cache copy, calls back to back: served largely from the 256 MB "
                                          "last-level cache, not from HBM",
            "decode_call_us": round(warm_avg * 1e3, 2),
            "value": round(wc["cache_bytes"] / (warm_avg * 1e-3) / 1e9, 2), "unit": "GB/s"}
    plan, n_replicas = w.plan, len(w.caches)
    names = [n for n in args.side_workloads.split(",") if n and n != cfg.name]
    if names:
        del w
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        for n in names:
            side[n] = side_workload(configs.BY_NAME[n], args.side_calls, 5)
    result = {
        "metric": metric_name(cfg),
        "value": round(wc["cache_bytes"] / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "clock_ramp": {"ms": args.ramp_ms, "steps": ramp_steps},
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act_dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian latent cache, queries and random-init weights)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "q_len": cfg.q_len,
                   "n_heads": cfg.n_heads, "d_head": cfg.d_head, "d_latent": cfg.d_latent,
                   "d_rope": cfg.d_rope, "seq_len": cfg.seq_len, "kv_dtype": cfg.kv_dtype,
                   "paged": cfg.paged, "splits": plan[0], "split_tokens": plan[1],
                   "fp8_scores": args.fp8_scores,
                   "cache_replicas": n_replicas},
        "tflops": round(wc["attn_flops"] / (ms_step * 1e-3) / 1e12, 2),
        "decode_tokens_per_s": round(cfg.batch * cfg.q_len / (ms_step * 1e-3), 1),
        "decode_call_us": round(dec_avg * 1e3, 2),
        "ms_per_step_with_call_events": round(ms_step_ev, 5),
        "decode_call_tflops": round(wc["attn_flops"] / (dec_avg * 1e-3) / 1e12, 2),
        "decode_call_mfma_frac": round(wc["attn_flops"] / (dec_avg * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFS, 4),
        "roofline": roof,
        "configs": side,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, args.cpu_single_core_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
