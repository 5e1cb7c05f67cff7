"""GPU parity of the cache-write step and the query rotation, through the C ABI, against
the CPU oracle.

Bars: bf16 outputs 2e-2 and fp32 outputs 1e-4 (max |gpu - ref| / max |ref|); the fp8
latent 6e-2 against the oracle's latent before quantization, with at least 99% of the
codes equal to the oracle's (the rest one code step away: the kernel decides each code
from its fp32 sum, the oracle from the fp64 one) and the per-token scale within 1e-5.
Pool rows are bit-exact where integer work decides them: the rows of the new tokens are
written at exactly the block-table positions, and every other pool byte is untouched.

Every case prints its name, seed and shape before touching the GPU.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import capi, configs, synth
from mla_latent_kv_lat_amd.runner import to_device, to_host_f64
from conftest import max_rel_err

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A  # every pool byte before the call


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()
    return "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def decode_store(arr, kind):
    return O.decode(arr, kind)


def run_append(cfg, d_model, pairing, base=10000.0, seed=0):
    inp = synth.make_append_inputs(cfg, d_model, seed)
    B, sq, dc, dr, bs = cfg.batch, cfg.q_len, cfg.d_latent, cfg.d_rope, cfg.block_size
    act, kv = cfg.act_dtype, cfg.kv_dtype
    say(f"cache_append {cfg.name} d_model={d_model} pairing={pairing} B={B} s_q={sq} kv={kv} seed={seed}")
    x = to_device(inp.x, act, "cuda")
    w_dkv = to_device(inp.w_dkv, act, "cuda")
    w_kr = to_device(inp.w_kr, act, "cuda")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    elt = {"f32": 4, "bf16": 2, "fp8": 1}
    c_pool = torch.full((inp.n_blocks, bs, dc * elt[kv]), SENTINEL, dtype=torch.uint8, device="cuda")
    r_pool = torch.full((inp.n_blocks, bs, dr * elt[act]), SENTINEL, dtype=torch.uint8, device="cuda")
    s_pool = torch.full((inp.n_blocks, bs), -7.0, dtype=torch.float32, device="cuda") if kv == "fp8" else None
    table = to_device(inp.block_table, "i32", "cuda")
    lens = to_device(inp.seq_lens, "i32", "cuda")
    d = capi.dims_from_config(cfg)
    ws_bytes = capi.mla_cache_append_workspace_bytes(d, d_model)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    c_view = c_pool if kv == "fp8" else c_pool.view(tdt[kv])
    capi.mla_cache_append(d, x, w_dkv, w_kr, c_view, r_pool.view(tdt[act]), table, lens, ws,
                          rope_base=base, pairing=pairing, kv_scale_pool=s_pool,
                          x_dtype=capi.DTYPE_CODES[act], kv_dtype=capi.DTYPE_CODES[kv])
    torch.cuda.synchronize()
    return inp, c_pool.cpu().numpy(), r_pool.cpu().numpy(), (None if s_pool is None else s_pool.cpu().numpy())


def check_append(cfg, d_model, pairing, base=10000.0, seed=0):
    inp, c_pool, r_pool, s_pool = run_append(cfg, d_model, pairing, base, seed)
    act, kv = cfg.act_dtype, cfg.kv_dtype
    dc, dr, bs = cfg.d_latent, cfg.d_rope, cfg.block_size
    c_ref, k_ref, pos = O.cache_append_rows(O.decode(inp.x, act), O.decode(inp.w_dkv, act),
                                            O.decode(inp.w_kr, act), inp.seq_lens, cfg.q_len, base, pairing)
    rows = inp.block_table[np.arange(cfg.batch)[:, None], pos // bs] * bs + pos % bs  # [B, s_q]
    flat_rows = rows.reshape(-1)
    assert len(set(flat_rows.tolist())) == flat_rows.size
    c_flat = c_pool.reshape(-1, c_pool.shape[-1])
    r_flat = r_pool.reshape(-1, r_pool.shape[-1])
    # untouched rows keep the sentinel, bit for bit
    mask = np.ones(c_flat.shape[0], bool)
    mask[flat_rows] = False
    assert np.all(c_flat[mask] == SENTINEL) and np.all(r_flat[mask] == SENTINEL)
    # rope key
    k_store = r_flat[flat_rows].view(np.uint16 if act == "bf16" else np.float32)
    k_got = O.decode(k_store, act).reshape(k_ref.shape)
    tol = 2e-2 if act == "bf16" else 1e-4
    ek = max_rel_err(k_got, k_ref)
    # latent
    c_ref_f = c_ref.reshape(-1, dc)
    if kv == "fp8":
        codes = c_flat[flat_rows]
        scale = s_pool.reshape(-1)[flat_rows].astype(np.float64)
        ref_codes, ref_scale = O.quantize_e4m3fn_rows(c_ref_f)
        np.testing.assert_allclose(scale, ref_scale, rtol=1e-5)
        same = np.mean(codes == ref_codes)
        deq = O.decode_e4m3fn(codes) * scale[:, None]
        ec = max_rel_err(deq, c_ref_f)
        near = np.abs(O.decode_e4m3fn(codes) - O.decode_e4m3fn(ref_codes)) <= \
            np.maximum(np.abs(O.decode_e4m3fn(ref_codes)) * 0.125, 2.0 ** -9)
        print(f"  codes equal {same:.5f}, latent max rel err {ec:.2e}, rope {ek:.2e}", flush=True)
        assert same >= 0.99 and np.all(near)
        assert ec <= 6e-2
    else:
        c_store = c_flat[flat_rows].view(np.uint16 if kv == "bf16" else np.float32)
        ec = max_rel_err(O.decode(c_store, kv), c_ref_f)
        print(f"  latent max rel err {ec:.2e}, rope {ek:.2e}", flush=True)
        assert ec <= tol
    assert ek <= tol


TINY_APPEND = configs.TINY.with_(batch=3, q_len=2, seq_len=100, len_min=3, paged=True, block_size=16)


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_cache_append_tiny_f32(pairing):
    check_append(TINY_APPEND, 96, pairing)


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_cache_append_v2_bf16(pairing):
    check_append(configs.V2_DECODE.with_(batch=8), 5120, pairing)


def test_cache_append_paged_varlen_ragged_d_model():
    # d_model not a multiple of the split-K chunk, block size not a multiple of anything
    check_append(configs.PAGED_VARLEN.with_(batch=6, block_size=7, seq_len=300, len_min=1), 1000, "half")


def test_cache_append_fp8_speculative():
    check_append(configs.SPEC_FP8.with_(batch=8, seq_len=1000), 5120, "interleaved", base=500000.0)


def test_cache_append_long_positions():
    # positions near 131072: the rotation angle must be formed in double precision
    check_append(configs.LONG_CONTEXT, 2048, "interleaved")


@pytest.mark.parametrize("cfg,pairing", [(configs.TINY.with_(q_len=3, seq_len=40), "interleaved"),
                                         (configs.SPEC_FP8.with_(batch=4), "half"),
                                         (configs.LONG_CONTEXT, "interleaved")])
def test_rope_query(cfg, pairing):
    say(f"rope_query {cfg.name} pairing={pairing}")
    inp = synth.make_inputs(cfg, 1)
    act = cfg.act_dtype
    q = to_device(inp.q_rope, act, "cuda")
    lens = to_device(inp.seq_lens, "i32", "cuda")
    capi.mla_rope_query(capi.dims_from_config(cfg), q, lens, rope_base=10000.0, pairing=pairing)
    torch.cuda.synchronize()
    got = to_host_f64(q)
    pos = O.new_token_positions(inp.seq_lens, cfg.q_len)  # [B, s_q]
    ref = O.rope_rotate(O.decode(inp.q_rope, act), pos[:, :, None], 10000.0, pairing)
    err = max_rel_err(got, ref)
    print(f"  max rel err {err:.2e}", flush=True)
    assert err <= (2e-2 if act == "bf16" else 1e-4)


def test_append_then_decode_matches_oracle():
    """The cache written by mla_cache_append is the cache mla_decode_paged reads."""
    cfg = configs.PAGED_VARLEN.with_(batch=4, seq_len=700, len_min=100)
    d_model = 1024
    inp_a = synth.make_append_inputs(cfg, d_model, 2)
    say(f"append+decode {cfg.name} B={cfg.batch}")
    # the pool of the decode inputs (same layout: same seed and lengths)
    lens = inp_a.seq_lens
    base = synth.make_inputs(cfg, 2, lengths=lens)
    assert np.array_equal(base.block_table, inp_a.block_table)
    act = cfg.act_dtype
    c_pool = to_device(base.c_kv, cfg.kv_dtype, "cuda")
    r_pool = to_device(base.k_rope, act, "cuda")
    table = to_device(base.block_table, "i32", "cuda")
    dlen = to_device(lens, "i32", "cuda")
    d = capi.dims_from_config(cfg)
    ws = torch.empty(capi.mla_cache_append_workspace_bytes(d, d_model), dtype=torch.uint8, device="cuda")
    capi.mla_cache_append(d, to_device(inp_a.x, act, "cuda"), to_device(inp_a.w_dkv, act, "cuda"),
                          to_device(inp_a.w_kr, act, "cuda"), c_pool, r_pool, table, dlen, ws)
    # decode over the updated pool
    q_lat = to_device(synth.make_stage_input(cfg, 2, "q_lat", (cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_latent)), act, "cuda")
    q_rope = to_device(base.q_rope, act, "cuda")
    o_lat = torch.empty_like(q_lat)
    lse = torch.empty(cfg.batch, cfg.q_len, cfg.n_heads, dtype=torch.float32, device="cuda")
    dws = torch.empty(max(1, capi.mla_decode_workspace_bytes(d, capi.DTYPE_CODES[cfg.kv_dtype], cfg.seq_len)),
                      dtype=torch.uint8, device="cuda")
    capi.mla_decode_paged(d, q_lat, q_rope, c_pool, r_pool, table, dlen, cfg.seq_len, o_lat, lse, dws)
    torch.cuda.synchronize()
    # oracle: the pool with the new rows written by the oracle's own cache write
    c_ref, k_ref, pos = O.cache_append_rows(O.decode(inp_a.x, act), O.decode(inp_a.w_dkv, act),
                                            O.decode(inp_a.w_kr, act), lens, cfg.q_len, 10000.0, "interleaved")
    lat = O.decode(base.c_kv, cfg.kv_dtype).copy()
    rope = O.decode(base.k_rope, act).copy()
    bs = cfg.block_size
    for b in range(cfg.batch):
        for i in range(cfg.q_len):
            p = int(pos[b, i])
            lat[base.block_table[b, p // bs], p % bs] = c_ref[b, i]
            rope[base.block_table[b, p // bs], p % bs] = k_ref[b, i]
    lat_c = O.gather_pages(lat, base.block_table, lens, cfg.seq_len)
    rope_c = O.gather_pages(rope, base.block_table, lens, cfg.seq_len)
    ql = O.decode(synth.make_stage_input(cfg, 2, "q_lat", (cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_latent)), act)
    o_ref, lse_ref = O.latent_attention(ql, O.decode(base.q_rope, act), lat_c, rope_c, lens, cfg.softmax_scale)
    err = max_rel_err(to_host_f64(o_lat), o_ref)
    print(f"  o_lat max rel err {err:.2e}", flush=True)
    assert err <= 2e-2
