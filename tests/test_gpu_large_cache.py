"""GPU parity on caches larger than 4 GiB: every byte offset into the cache past 2^32 and
every element index past 2^31 must be formed in 64-bit arithmetic.

Each case places a small seeded workload at the far end of a large cache: the contiguous
cases as the last sequences of a batch whose earlier sequences are empty (length 0, so the
kernels read none of their rows), the paged cases as the last blocks of a large pool reached
through the block table.  Every unused cache row holds NaN (bf16) or the e4m3fn NaN code, so
a read of a wrong row shows in the outputs.  The reference is the oracle's latent attention
on the small workload; the empty sequences must give o_lat 0 and lse -inf.  Bars as in the
other decode parity tests: bf16 2e-2 (o_lat relative, lse absolute), fp8 cache 2e-2 against
the oracle on the dequantized cache.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import capi, configs, synth
from mla_latent_kv_lat_amd.runner import to_device, to_host_f64
from conftest import decoded, max_abs_err, max_rel_err
from test_gpu_parity import KERNELS, TOL, say, use_kernel

pytestmark = pytest.mark.gpu

BIG_T = 131072  # tokens per sequence slot of the large contiguous caches
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()
    yield "cuda"
    torch.cuda.empty_cache()


def nan_filled(shape, kind):
    if kind == "bf16":
        return torch.full(shape, BF16_NAN, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if kind == "fp8":
        return torch.full(shape, E4M3_NAN, dtype=torch.uint8, device="cuda")
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def small_case(cfg, lengths):
    """The small workload, its stored q_lat (the oracle's, rounded to the stored dtype) and
    the oracle's attention outputs."""
    inp = synth.make_inputs(cfg, 0, lengths=np.array(lengths, np.int32), poison_tail=True)
    d = decoded(inp)
    q_bits = synth.store(O.absorb_query(d["q_nope"], d["w_uk"]).astype(np.float32), cfg.act_dtype)
    q_dec = O.decode(q_bits, cfg.act_dtype)
    o_ref, lse_ref = O.latent_attention(q_dec, d["q_rope"], d["c_kv"], d["k_rope"], d["seq_lens"], d["scale"])
    return inp, q_bits, o_ref, lse_ref


def check(o, lse, o_ref, lse_ref, tol, what):
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), what
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(lse[fin], lse_ref[fin])
    print(f"  {what}: o_lat {e_o:.2e} lse {e_l:.2e}", flush=True)
    assert e_o <= tol and e_l <= tol, (what, e_o, e_l)


def contiguous_case(cfg, lengths, big_b):
    """cfg's sequences become sequences big_b - len(lengths) .. big_b - 1 of a [big_b, BIG_T]
    cache; returns (o_lat, lse) of the whole batch and the small reference."""
    inp, q_bits, o_ref, lse_ref = small_case(cfg, lengths)
    nb, T = cfg.batch, cfg.seq_len
    first = big_b - nb
    big = cfg.with_(batch=big_b, seq_len=BIG_T)
    kv, act = cfg.kv_dtype, cfg.act_dtype
    c_kv = nan_filled((big_b, BIG_T, cfg.d_latent), kv)
    k_rope = nan_filled((big_b, BIG_T, cfg.d_rope), act)
    c_kv[first:, :T] = to_device(inp.c_kv, kv, "cuda")
    k_rope[first:, :T] = to_device(inp.k_rope, act, "cuda")
    kv_scale = None
    if kv == "fp8":
        kv_scale = nan_filled((big_b, BIG_T), "f32")
        kv_scale[first:, :T] = to_device(inp.kv_scale, "f32", "cuda")
    rows = (cfg.q_len, cfg.n_heads)
    q_lat = torch.zeros((big_b, *rows, cfg.d_latent), dtype=torch.bfloat16, device="cuda")
    q_rope = torch.zeros((big_b, *rows, cfg.d_rope), dtype=torch.bfloat16, device="cuda")
    q_lat[first:] = to_device(q_bits, act, "cuda")
    q_rope[first:] = to_device(inp.q_rope, act, "cuda")
    seq_lens = torch.zeros(big_b, dtype=torch.int32, device="cuda")
    seq_lens[first:] = to_device(inp.seq_lens, "i32", "cuda")
    o_lat = torch.empty_like(q_lat)
    lse = torch.empty((big_b, *rows), dtype=torch.float32, device="cuda")
    dims = capi.dims_from_config(big)
    ws_bytes = capi.mla_decode_workspace_bytes(dims, capi.DTYPE_CODES[kv], BIG_T)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    assert c_kv.numel() * c_kv.element_size() > 2 ** 32 and c_kv.numel() > 2 ** 31
    capi.mla_decode(dims, q_lat, q_rope, c_kv, k_rope, BIG_T, seq_lens, o_lat, lse, ws, ws_bytes,
                    kv_scale=kv_scale, kv_dtype=capi.DTYPE_CODES[kv])
    torch.cuda.synchronize()
    o, l = to_host_f64(o_lat), to_host_f64(lse)
    del c_kv, k_rope, kv_scale
    assert np.all(o[:first] == 0) and np.all(np.isneginf(l[:first]))
    return o[first:], l[first:], o_ref, lse_ref


@pytest.mark.parametrize("kern", list(KERNELS))
def test_contiguous_bf16_cache_past_4gib(kern, monkeypatch):
    n_heads = use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=2, seq_len=2500, cfg_id=38, n_heads=n_heads)
    big_b = 34  # 34 x 131072 rows of 1 KB: 4.56 GB
    say("large contiguous bf16 cache", kern, "batch", big_b, "T", BIG_T, cfg)
    o, l, o_ref, l_ref = contiguous_case(cfg, [2500, 777], big_b)
    check(o, l, o_ref, l_ref, TOL["bf16"], f"bf16 {kern}")


def test_contiguous_fp8_cache_past_4gib():
    cfg = configs.SPEC_FP8.with_(batch=2, seq_len=1500, cfg_id=39)
    big_b = 66  # 66 x 131072 rows of 512 codes: 4.43 GB
    say("large contiguous fp8 cache", "batch", big_b, "T", BIG_T, cfg)
    o, l, o_ref, l_ref = contiguous_case(cfg, [1500, 333], big_b)
    check(o, l, o_ref, l_ref, TOL["fp8"], "fp8")


@pytest.mark.parametrize("kern", ["rows128", "pair", "rows64"])
@pytest.mark.parametrize("block_size", [64, 48])
def test_paged_bf16_pool_past_4gib(block_size, kern, monkeypatch):
    use_kernel(kern, monkeypatch)
    cfg = configs.PAGED_VARLEN.with_(batch=2, seq_len=1500, len_min=1, block_size=block_size, cfg_id=40)
    say("large paged bf16 pool", kern, "block size", block_size, cfg)
    inp, q_bits, o_ref, lse_ref = small_case(cfg, [1500, 640])
    n_small = inp.c_kv.shape[0]
    n_big = (34 * BIG_T) // block_size  # 4.56 GB of latent rows
    shift = n_big - n_small  # the workload's blocks become the pool's last ones
    c_kv = nan_filled((n_big, block_size, cfg.d_latent), "bf16")
    k_rope = nan_filled((n_big, block_size, cfg.d_rope), "bf16")
    c_kv[shift:] = to_device(inp.c_kv, "bf16", "cuda")
    k_rope[shift:] = to_device(inp.k_rope, "bf16", "cuda")
    table = np.where(inp.block_table >= 0, inp.block_table + shift, -1).astype(np.int32)
    assert int(table.max()) * block_size * cfg.d_latent * 2 > 2 ** 32
    q_lat = to_device(q_bits, "bf16", "cuda")
    q_rope = to_device(inp.q_rope, "bf16", "cuda")
    o_lat = torch.empty_like(q_lat)
    lse = torch.empty(q_lat.shape[:-1], dtype=torch.float32, device="cuda")
    dims = capi.dims_from_config(cfg)
    ws_bytes = capi.mla_decode_workspace_bytes(dims, capi.MLA_BF16, cfg.seq_len)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    capi.mla_decode_paged(dims, q_lat, q_rope, c_kv, k_rope, to_device(table, "i32", "cuda"),
                          to_device(inp.seq_lens, "i32", "cuda"), cfg.seq_len, o_lat, lse, ws, ws_bytes)
    torch.cuda.synchronize()
    del c_kv, k_rope
    check(to_host_f64(o_lat), to_host_f64(lse), o_ref, lse_ref, TOL["bf16"], f"paged {kern} bs {block_size}")
