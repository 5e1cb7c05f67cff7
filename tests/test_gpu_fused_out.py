"""mla_decode_absorb_out (latent attention and output absorption in one call) against the
two separate calls, bit for bit, and against the oracle.

The fused path merges the sequences cut by range boundaries inside the output absorption;
its arithmetic is that of the separate merge and absorption kernels, so o_lat, lse and out
must be identical.  Cases cover every kind of row the merge sees (a sequence without tiles,
one wholly inside a range, one cut into at most 4 pieces, one cut into more), both bf16
matrix-core kernels, a row count that is not a multiple of the 16-row groups, and the plans
that fall back to the two calls (fixed splits, the general kernel, fp32).
Every case prints its name and shape first.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import capi, configs, synth
from mla_latent_kv_lat_amd.runner import DeviceWorkload, to_host_f64
from conftest import decoded, max_rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()
    return "cuda"


CASES = {
    # name: (config, overrides, lengths, split_tokens, row block)
    "ragged_rows64": (configs.V2_DECODE, dict(batch=8, seq_len=1000), [1000, 0, 333, 1, 999, 512, 64, 700], 0, "64"),
    "ragged_rows128": (configs.V2_DECODE, dict(batch=8, seq_len=1000), [1000, 0, 333, 1, 999, 512, 64, 700], 0, "128"),
    "many_short_whole": (configs.V2_DECODE, dict(batch=200, seq_len=64), None, 0, "64"),
    "one_long_many_pieces": (configs.V2_DECODE, dict(batch=40, seq_len=4000), [4000] + [50] * 39, 0, "64"),
    "rows_not_multiple_of_16": (configs.V2_DECODE, dict(batch=3, seq_len=700), [700, 10, 333], 0, "128"),
    "fixed_splits_fallback": (configs.V2_DECODE, dict(batch=3, seq_len=700), [700, 10, 333], 256, "64"),
    "general_kernel_fallback": (configs.V2_DECODE, dict(batch=3, seq_len=300, n_heads=8), [300, 1, 77], 0, None),
    "fp32_fallback": (configs.TINY, dict(batch=2, seq_len=128), [128, 40], 0, None),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fused_equals_separate_calls(case, monkeypatch):
    base, kw, lengths, split_tokens, rb = CASES[case]
    if rb:
        monkeypatch.setenv("MLA_DECODE_ROW_BLOCK", rb)
    else:
        monkeypatch.delenv("MLA_DECODE_ROW_BLOCK", raising=False)
    cfg = base.with_(cfg_id=70, **kw)
    print(f"[case] fused decode + absorb_out {case}: B={cfg.batch} T={cfg.seq_len} heads={cfg.n_heads} "
          f"split_tokens={split_tokens}", flush=True)
    if lengths is None:
        lengths = np.random.default_rng(5).integers(0, cfg.seq_len + 1, size=cfg.batch)
    inp = synth.make_inputs(cfg, 0, lengths=np.array(lengths, np.int32))
    w = DeviceWorkload(inp, split_tokens=split_tokens)
    w.absorb_q()
    w.decode()
    w.absorb_out()
    torch.cuda.synchronize()
    sep = {k: to_host_f64(t).copy() for k, t in (("o_lat", w.o_lat), ("lse", w.lse), ("out", w.out))}
    for t in (w.o_lat, w.lse, w.out):
        t.fill_(float("nan"))
    w.decode_absorb_out()
    torch.cuda.synchronize()
    fused = {k: to_host_f64(t) for k, t in (("o_lat", w.o_lat), ("lse", w.lse), ("out", w.out))}
    for k in sep:
        assert np.array_equal(sep[k], fused[k], equal_nan=True), k
    # And the oracle: out = (attention over the latent) . W_UV per head.
    d = decoded(inp)
    q_lat = O.absorb_query(d["q_nope"], d["w_uk"])
    q_dec = O.decode(synth.store(q_lat.astype(np.float32), cfg.act_dtype), cfg.act_dtype)
    o_ref, _ = O.latent_attention(q_dec, d["q_rope"], d["c_kv"], d["k_rope"], d["seq_lens"], d["scale"])
    out_ref = O.absorb_output(O.decode(synth.store(o_ref.astype(np.float32), cfg.act_dtype), cfg.act_dtype), d["w_uv"])
    e = max_rel_err(fused["out"], out_ref)
    print(f"  fused == separate bitwise; out vs oracle {e:.2e}", flush=True)
    assert e <= TOL[cfg.act_dtype]
