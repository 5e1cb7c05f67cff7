"""mla_decode_noalloc (partial results in the library's static device array) against
mla_decode with a caller workspace: the same plan and kernels, so the outputs must be
equal bit for bit.  Two calls in a row, the second on a smaller batch, so a result left in
the shared array by the first call would show in the second."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import capi, configs, synth
from mla_latent_kv_lat_amd.runner import DeviceWorkload, to_device, to_host_f64
from conftest import decoded, max_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()
    return "cuda"


def one_call(cfg, seed, lengths, fp8_scores=0):
    inp = synth.make_inputs(cfg, seed, lengths=np.array(lengths, np.int32), poison_tail=True)
    d = decoded(inp)
    q_bits = synth.store(O.absorb_query(d["q_nope"], d["w_uk"]).astype(np.float32), cfg.act_dtype)
    w = DeviceWorkload(inp, fp8_scores=fp8_scores)
    q_lat = to_device(q_bits, cfg.act_dtype, "cuda")
    w.decode(q_lat=q_lat)
    torch.cuda.synchronize()
    o_ws, l_ws = to_host_f64(w.o_lat), to_host_f64(w.lse)
    # The same call without a workspace, into freshly poisoned outputs.
    w.o_lat.fill_(float("nan"))
    w.lse.fill_(float("nan"))
    c = w.caches[0]
    capi.mla_decode_noalloc(w.dims, q_lat, w.q_rope, c["c_kv"], c["k_rope"], cfg.seq_len, w.seq_lens,
                            w.o_lat, w.lse, kv_scale=c["kv_scale"])
    torch.cuda.synchronize()
    o_na, l_na = to_host_f64(w.o_lat), to_host_f64(w.lse)
    assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na)
    q_dec = O.decode(q_bits, cfg.act_dtype)
    if fp8_scores == 0:
        o_ref, _ = O.latent_attention(q_dec, d["q_rope"], d["c_kv"], d["k_rope"], d["seq_lens"], d["scale"])
    elif fp8_scores == 1:
        o_ref, _ = O.latent_attention_fp8_query(q_dec, d["q_rope"], d["c_kv"], d["k_rope"], d["seq_lens"],
                                                d["scale"])
    else:
        o_ref, _ = O.latent_attention_fp8(q_dec, d["q_rope"], inp.c_kv, inp.kv_scale, d["k_rope"],
                                          d["seq_lens"], d["scale"])
    e = max_rel_err(o_na, o_ref)
    print(f"  noalloc == workspace bitwise; o_lat vs the oracle's definition {e:.2e}", flush=True)
    # the fp8 cache's kernel bar (fp8_scores 1 and 2 against their own definitions)
    assert e <= 2e-2
    return w.ws_bytes


@pytest.mark.parametrize("kv,rows,fp8_scores", [("bf16", "128", 0), ("bf16", "64", 0), ("fp8", None, 0),
                                               ("fp8", None, 1), ("fp8", None, 2)])
def test_noalloc_equals_workspace_call_twice(kv, rows, fp8_scores, monkeypatch):
    # A bf16 cache runs on either matrix-core kernel (row blocks of 128 or 64 query rows).
    if rows:
        monkeypatch.setenv("MLA_DECODE_ROW_BLOCK", rows)
    base = configs.V2_DECODE if kv == "bf16" else configs.SPEC_FP8
    big = base.with_(batch=9, seq_len=1500, cfg_id=60)
    print(f"[case] noalloc {kv} fp8_scores={fp8_scores} first call {big.batch}x{big.seq_len}", flush=True)
    ws1 = one_call(big, 0, np.random.default_rng(1).integers(1, 1501, size=9), fp8_scores)
    small = base.with_(batch=2, seq_len=300, cfg_id=61)
    print(f"[case] noalloc {kv} fp8_scores={fp8_scores} second call {small.batch}x{small.seq_len}", flush=True)
    ws2 = one_call(small, 1, [300, 17], fp8_scores)
    assert 0 < ws2 <= ws1 <= capi.NOALLOC_SCRATCH_BYTES
