"""GPU parity of the projections around the attention (mla_linear), of the query path from
hidden states (query compression, then either the unfolded up-projection and key
absorption or the folded W_UQ W_UK product), and of the output projection, against the
oracle.

Bar: bf16, max |gpu - ref| / max |ref| <= 2e-2.  Every case prints its name and shape first.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import capi, synth
from mla_latent_kv_lat_amd.runner import to_device, to_host_f64
from conftest import max_rel_err

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


def bf16(a):
    """Round to bf16 storage (the tensors the GPU sees) and back to float64."""
    return O.decode(synth.store(np.asarray(a, np.float32), "bf16"), "bf16")


def dev(a):
    """A float64 array whose values are bf16-exact, as a device bf16 tensor."""
    return to_device(synth.store(np.asarray(a, np.float32), "bf16"), "bf16", "cuda")


def gaussian(seed, shape, std=1.0):
    return (np.random.default_rng(seed).normal(size=shape) * std).astype(np.float32)


def linear(x, w):
    """mla_linear on device tensors; returns the bf16 result tensor."""
    M, K = x.shape
    N = w.shape[1]
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(capi.mla_linear_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
    capi.mla_linear(x, w, y, ws)
    return y


@pytest.mark.parametrize("M,K,N", [(32, 5120, 1536), (33, 512, 192), (5, 256, 64), (32, 1536, 8192)])
def test_linear(M, K, N):
    say("linear", M, K, N)
    x = bf16(gaussian(1, (M, K)))
    w = bf16(gaussian(2, (K, N), K ** -0.5))
    y = linear(dev(x), dev(w))
    torch.cuda.synchronize()
    err = max_rel_err(to_host_f64(y), x @ w)
    print(f"  max rel err {err:.2e}", flush=True)
    assert err <= TOL


DS = dict(M=32, d_model=5120, d_cq=1536, n_h=128, d_h=128, d_r=64, d_c=512)


def query_inputs(seed=0):
    s = DS
    x = bf16(gaussian(seed, (s["M"], s["d_model"])))
    w_dq = bf16(gaussian(seed + 1, (s["d_model"], s["d_cq"]), s["d_model"] ** -0.5))
    w_uq = bf16(gaussian(seed + 2, (s["d_cq"], s["n_h"], s["d_h"]), s["d_cq"] ** -0.5))
    w_qr = bf16(gaussian(seed + 3, (s["d_cq"], s["n_h"], s["d_r"]), s["d_cq"] ** -0.5))
    w_uk = bf16(gaussian(seed + 4, (s["n_h"], s["d_h"], s["d_c"]), s["d_c"] ** -0.5))
    return x, w_dq, w_uq, w_qr, w_uk


def test_query_path_unfolded_and_folded():
    """x -> c_q -> (q_nope, q_rope) -> q_lat, and x -> c_q -> q_lat through the folded
    W_UQ W_UK (the fold itself formed on the device by the key absorption of W_UQ)."""
    s = DS
    say("query path", s)
    x, w_dq, w_uq, w_qr, w_uk = query_inputs()
    M, d_cq, n_h, d_h, d_r, d_c = s["M"], s["d_cq"], s["n_h"], s["d_h"], s["d_r"], s["d_c"]
    c_q = linear(dev(x), dev(w_dq))
    q_nope = linear(c_q, dev(w_uq.reshape(d_cq, n_h * d_h)))
    q_rope = linear(c_q, dev(w_qr.reshape(d_cq, n_h * d_r)))
    q_lat = torch.empty(M, n_h, d_c, dtype=torch.bfloat16, device="cuda")
    dq = capi.dims(M, 1, n_h, d_h, d_c, d_r, 1.0)
    capi.mla_absorb_q(dq, q_nope.view(M, 1, n_h, d_h), dev(w_uk), q_lat)
    # fold: W_UQK[k, h, :] = W_UQ[k, h, :] W_UK[h], i.e. the key absorption with d_cq rows
    w_uqk = torch.empty(d_cq, n_h, d_c, dtype=torch.bfloat16, device="cuda")
    capi.mla_absorb_q(capi.dims(d_cq, 1, n_h, d_h, d_c, d_r, 1.0), dev(w_uq).view(d_cq, 1, n_h, d_h),
                      dev(w_uk), w_uqk)
    q_lat_f = linear(c_q, w_uqk.view(d_cq, n_h * d_c))
    torch.cuda.synchronize()

    ref_nope, ref_rope = O.query_from_hidden(x, w_dq, w_uq, w_qr)
    ref_lat = O.absorb_query(ref_nope[:, None], w_uk)[:, 0]
    hs = [0, 77, 127]  # the fold is checked on sampled heads (the oracle's product is slow)
    ref_fold = O.fold_query_weights(w_uq[:, hs], w_uk[hs])
    errs = {
        "c_q": max_rel_err(to_host_f64(c_q), x @ w_dq),
        "q_nope": max_rel_err(to_host_f64(q_nope).reshape(M, n_h, d_h), ref_nope),
        "q_rope": max_rel_err(to_host_f64(q_rope).reshape(M, n_h, d_r), ref_rope),
        "q_lat": max_rel_err(to_host_f64(q_lat), ref_lat),
        "w_uqk": max_rel_err(to_host_f64(w_uqk)[:, hs], ref_fold),
        "q_lat_folded": max_rel_err(to_host_f64(q_lat_f).reshape(M, n_h, d_c), ref_lat),
    }
    print("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL, k


def test_output_projection():
    """o_lat -> per-head outputs (value absorption) -> O W_O."""
    s = DS
    say("output projection", s)
    M, n_h, d_h, d_c, d_model = s["M"], s["n_h"], s["d_h"], s["d_c"], s["d_model"]
    o_lat = bf16(gaussian(10, (M, n_h, d_c)))
    w_uv = bf16(gaussian(11, (n_h, d_c, d_h), d_c ** -0.5))
    w_o = bf16(gaussian(12, (n_h * d_h, d_model), (n_h * d_h) ** -0.5))
    heads = torch.empty(M, 1, n_h, d_h, dtype=torch.bfloat16, device="cuda")
    capi.mla_absorb_out(capi.dims(M, 1, n_h, d_h, d_c, 64, 1.0), dev(o_lat).view(M, 1, n_h, d_c), dev(w_uv), heads)
    y = linear(heads.view(M, n_h * d_h), dev(w_o))
    torch.cuda.synchronize()
    ref = O.output_projection(bf16(O.absorb_output(o_lat[:, None], w_uv)[:, 0]), w_o)
    err = max_rel_err(to_host_f64(y), ref)
    print(f"  max rel err {err:.2e}", flush=True)
    assert err <= TOL


def test_output_path_folded():
    """out = o_lat (viewed as [M, n_h d_c]) . W_UVO, where W_UVO[h] = W_UV[h] . W_O[h d_h :
    (h + 1) d_h] is formed on the device by mla_fold_output_weights: the fold against the
    oracle's (sampled heads), and the folded output path against the oracle's unfolded
    one (value absorption, then O W_O, in fp64)."""
    s = DS
    say("output path, folded", s)
    M, n_h, d_h, d_c, d_model = s["M"], s["n_h"], s["d_h"], s["d_c"], s["d_model"]
    o_lat = bf16(gaussian(10, (M, n_h, d_c)))
    w_uv = bf16(gaussian(11, (n_h, d_c, d_h), d_c ** -0.5))
    w_o = bf16(gaussian(12, (n_h * d_h, d_model), (n_h * d_h) ** -0.5))
    w_uvo = torch.empty(n_h, d_c, d_model, dtype=torch.bfloat16, device="cuda")
    capi.mla_fold_output_weights(dev(w_uv), dev(w_o), w_uvo)
    y = linear(dev(o_lat).view(M, n_h * d_c), w_uvo.view(n_h * d_c, d_model))
    torch.cuda.synchronize()
    hs = [0, 77, 127]  # the fold is checked on sampled heads (the oracle's product is slow)
    ref_fold = O.fold_output_weights(w_uv[hs], w_o.reshape(n_h, d_h, d_model)[hs].reshape(-1, d_model))
    errs = {"w_uvo": max_rel_err(to_host_f64(w_uvo[hs]), ref_fold),
            "out": max_rel_err(to_host_f64(y), O.output_projection(O.absorb_output(o_lat[:, None], w_uv)[:, 0], w_o))}
    print("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL, k
