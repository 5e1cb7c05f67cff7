"""GPU parity of the explicit-form prefill (mla_prefill) against the oracle's
decompress-then-attend form, through the C ABI.

Bar: bf16, max |gpu - ref| / max |ref| <= 2e-2 for the output and the log-sum-exp.  Cache
rows past each sequence's length are NaN-poisoned, so any read of them shows up.  The
decompressed keys and values that the library leaves in its workspace are also checked
against the oracle's own decompression (same bar), so a failure names its stage.

Every case prints its name and shape before touching the GPU.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import capi, configs, synth
from mla_latent_kv_lat_amd.runner import to_device, to_host_f64
from conftest import decoded, max_abs_err, max_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()
    return "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def run_prefill(cfg, lengths, seed=0, pass_lengths=True):
    inp = synth.make_inputs(cfg, seed, lengths=np.asarray(lengths, np.int32), poison_tail=True)
    B, S, H, T = cfg.batch, cfg.q_len, cfg.n_heads, cfg.seq_len
    dev = lambda a, k="bf16": to_device(a, k, "cuda")
    d = capi.dims_from_config(cfg)
    ws_bytes = capi.mla_prefill_workspace_bytes(d, T)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, S, H, cfg.d_head, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, S, H, dtype=torch.float32, device="cuda")
    lens = dev(inp.seq_lens, "i32") if pass_lengths else None
    capi.mla_prefill(d, dev(inp.q_nope), dev(inp.q_rope), dev(inp.c_kv), dev(inp.k_rope), T, lens,
                     dev(inp.w_uk), dev(inp.w_uv), out, lse, ws)
    torch.cuda.synchronize()
    # Decompressed [B * T, H, 256] (key then value) after the concatenated weights.
    wbytes = (H * 256 * 512 * 2 + 255) // 256 * 256
    kv = ws[wbytes:wbytes + B * T * H * 256 * 2].view(torch.bfloat16).view(B, T, H, 256)
    return inp, to_host_f64(out), to_host_f64(lse), to_host_f64(kv)


def check(cfg, lengths, rows=None, pass_lengths=True):
    inp, out, lse, kv = run_prefill(cfg, lengths, pass_lengths=pass_lengths)
    d = decoded(inp)
    # Stage 1: decompression of the rows each sequence owns.
    uk, uv = O.to_page_layout(d["w_uk"], d["w_uv"])
    H, dh = cfg.n_heads, cfg.d_head
    errs = []
    for b in range(cfg.batch):
        L = int(inp.seq_lens[b])
        K = (d["c_kv"][b, :L] @ uk).reshape(L, H, dh)
        V = (d["c_kv"][b, :L] @ uv).reshape(L, H, dh)
        errs.append(max(max_rel_err(kv[b, :L, :, :dh], K), max_rel_err(kv[b, :L, :, dh:], V)))
    e_kv = max(errs)
    # Stage 2: attention (the oracle's explicit form, optionally on sampled rows).
    ref_o, ref_l = O.mla_explicit(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                                  inp.seq_lens, cfg.softmax_scale, rows=rows)
    done = ~np.isnan(ref_l)
    fin = done & np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(lse[done]), np.isneginf(ref_l[done]))
    e_o = max_rel_err(out[done], ref_o[done])
    e_l = max_abs_err(lse[fin], ref_l[fin])
    print(f"  kv {e_kv:.2e}  out {e_o:.2e}  lse {e_l:.2e}", flush=True)
    assert e_kv <= TOL and e_o <= TOL and e_l <= TOL


def prefill_cfg(**kw):
    return configs.V2_DECODE.with_(cfg_id=40, **kw)


def test_prefill_full_prompts_ragged_tiles():
    # T not a multiple of the 64-key tile nor of the 128-query block
    cfg = prefill_cfg(batch=2, q_len=300, seq_len=300, n_heads=8)
    say("prefill full prompts", cfg.batch, cfg.q_len, cfg.seq_len, cfg.n_heads)
    check(cfg, [300, 300])


def test_prefill_suffix_queries_ragged_lengths():
    # the queries are the last S rows of sequences of different lengths
    cfg = prefill_cfg(batch=3, q_len=150, seq_len=400, n_heads=4)
    say("prefill suffix queries", cfg.batch, cfg.q_len, cfg.seq_len, cfg.n_heads)
    check(cfg, [400, 211, 150])


def test_prefill_without_lengths():
    cfg = prefill_cfg(batch=1, q_len=256, seq_len=256, n_heads=8)
    say("prefill, seq_lens NULL", cfg.q_len, cfg.seq_len)
    check(cfg, [256], pass_lengths=False)


def test_prefill_few_queries():
    # s_q = 3 against 700 rows: the decode-like end of the range
    cfg = prefill_cfg(batch=2, q_len=3, seq_len=700, n_heads=16)
    say("prefill few queries", cfg.q_len, cfg.seq_len, cfg.n_heads)
    check(cfg, [700, 64])


def test_prefill_all_heads_sampled():
    # the DeepSeek-V2 head count; the oracle checks a seeded sample of (b, i, h) rows
    cfg = prefill_cfg(batch=1, q_len=512, seq_len=512, n_heads=128)
    say("prefill 128 heads", cfg.q_len, cfg.seq_len)
    rng = np.random.default_rng(3)
    rows = sorted({(0, int(i), int(h)) for i, h in zip(rng.integers(0, 512, 200), rng.integers(0, 128, 200))}
                  | {(0, 0, 0), (0, 511, 127), (0, 127, 5), (0, 128, 5)})
    check(cfg, [512], rows=rows)


def test_prefill_bench_size_sampled():
    """The size the prefill bench times (one 4096-token prompt, every token a query, 128
    heads): a seeded sample of (query, head) outputs and log-sum-exps, edges included, and
    the decompressed keys and values of three heads over every row (the full oracle would
    take minutes)."""
    T, H = 4096, 128
    cfg = prefill_cfg(batch=1, q_len=T, seq_len=T, n_heads=H)
    say("prefill bench size, sampled", T, H)
    inp = synth.make_inputs(cfg, 5, lengths=np.array([T], np.int32))
    dev = lambda a, k="bf16": to_device(a, k, "cuda")
    d = capi.dims_from_config(cfg)
    ws = torch.empty(capi.mla_prefill_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    out = torch.empty(1, T, H, cfg.d_head, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, T, H, dtype=torch.float32, device="cuda")
    capi.mla_prefill(d, dev(inp.q_nope), dev(inp.q_rope), dev(inp.c_kv), dev(inp.k_rope), T,
                     dev(inp.seq_lens, "i32"), dev(inp.w_uk), dev(inp.w_uv), out, lse, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = sorted({(0, int(i), int(h)) for i, h in zip(rng.integers(0, T, 96), rng.integers(0, H, 96))}
                  | {(0, 0, 0), (0, T - 1, H - 1), (0, 255, 64), (0, 256, 64), (0, 63, 1), (0, 64, 1)})
    ii = torch.tensor([r[1] for r in rows], device="cuda")
    hh = torch.tensor([r[2] for r in rows], device="cuda")
    got_o = to_host_f64(out[0, ii, hh])
    got_l = to_host_f64(lse[0, ii, hh])
    dd = decoded(inp)
    ref_o, ref_l = O.mla_explicit(dd["q_nope"], dd["q_rope"], dd["c_kv"], dd["k_rope"], dd["w_uk"], dd["w_uv"],
                                  inp.seq_lens, cfg.softmax_scale, rows=rows)
    ref_o = np.stack([ref_o[r] for r in rows])
    ref_l = np.array([ref_l[r] for r in rows])
    e_o, e_l = max_rel_err(got_o, ref_o), max_rel_err(got_l, ref_l)
    # decompressed key and value of three heads, every row (workspace: weights, then kv)
    wbytes = (H * 256 * 512 * 2 + 255) // 256 * 256
    kv = ws[wbytes:wbytes + T * H * 256 * 2].view(torch.bfloat16).view(T, H, 256)
    uk, uv = O.to_page_layout(dd["w_uk"], dd["w_uv"])
    e_kv = 0.0
    for h in (0, 77, H - 1):
        cols = slice(h * cfg.d_head, (h + 1) * cfg.d_head)
        got = to_host_f64(kv[:, h])
        e_kv = max(e_kv, max_rel_err(got[:, :cfg.d_head], dd["c_kv"][0] @ uk[:, cols]),
                   max_rel_err(got[:, cfg.d_head:], dd["c_kv"][0] @ uv[:, cols]))
    print(f"  {len(rows)} rows: out {e_o:.2e}  lse {e_l:.2e}  kv (3 heads) {e_kv:.2e}", flush=True)
    assert e_o <= TOL and e_l <= TOL and e_kv <= TOL
