"""GPU parity of the decode with both products in fp8 (dims.fp8_scores = 2) through the C ABI.

Its reference is the oracle's plain definition of that approximation, latent_attention_fp8:
the query rounded per 128-column slice as for the fp8 score product, and each softmax weight
times its token's scale rounded to e4m3 precision for the product with the stored codes
(the normaliser from the unrounded weights).  Bar: the fp8 cache's kernel bar, 2e-2
(o_lat: max |gpu - ref| / max |ref|; lse: absolute).  How far the approximation is from
exact attention on the dequantized cache, and from the latent before quantization, is
printed as a measurement.

Rounding a weight is an integer decision taken in floating point: the kernel takes it on a
float32 logit (matrix-core accumulation), the oracle on a float64 one, and the two differ
by about 1e-4 in base-2 units, so a weight whose scaled value lies that close to a
midpoint between two e4m3 values may round the other way on the two sides.  Either choice
is correct.  Element by element, o_lat may therefore also move by what all such ambiguous
weights can change it (one step of 4 significant bits each, times |code| / normaliser),
computed from the definition with a relative window of 2e-3 around each midpoint (ten
times the logit difference).

Every case prints its name, seed and shape before touching the GPU.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import capi, configs, synth
from mla_latent_kv_lat_amd.runner import DeviceWorkload, to_device, to_host_f64
from conftest import decoded, max_abs_err, max_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()  # fails loudly when libmla.so is missing
    return "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def contiguous_codes(inp, batches=None):
    """The stored e4m3 codes [B, T, d_c] and token scales [B, T] of the (sampled) sequences,
    gathered through the block table for a paged pool."""
    codes, ts = inp.c_kv, inp.kv_scale
    if inp.cfg.paged:
        codes = O.gather_pages(codes, inp.block_table, inp.seq_lens, inp.cfg.seq_len)
        ts = O.gather_pages(ts, inp.block_table, inp.seq_lens, inp.cfg.seq_len)
    if batches is not None:
        codes, ts = codes[batches], ts[batches]
    return codes, ts


def stored_query(inp):
    """The oracle's q_lat rounded to the stored activation dtype (both sides read these bits)."""
    d = decoded(inp)
    q_lat = O.absorb_query(d["q_nope"], d["w_uk"])
    return synth.store(q_lat.astype(np.float32), inp.cfg.act_dtype), d


def run_decode(inp, q_bits, split_tokens=0):
    w = DeviceWorkload(inp, split_tokens=split_tokens, fp8_scores=2)
    w.decode(q_lat=to_device(q_bits, inp.cfg.act_dtype, "cuda"))
    torch.cuda.synchronize()
    return to_host_f64(w.o_lat), to_host_f64(w.lse), w


def reference(inp, q_bits, d, batches=None):
    sl = slice(None) if batches is None else batches
    codes, ts = contiguous_codes(inp, batches)
    q_dec = O.decode(q_bits[sl], inp.cfg.act_dtype)
    return O.latent_attention_fp8(q_dec, d["q_rope"][sl], codes, ts, d["k_rope"][sl], d["seq_lens"][sl],
                                  d["scale"])


def flip_allowance(inp, q_bits, d, batches=None, eps=2e-3):
    """Per o_lat element: the sum over weights whose scaled value w_t ts_t lies within a
    relative eps of a rounding midpoint (4 significant bits) of one rounding step times
    |code_t| / sum_t w_t.  Weights and logits as latent_attention_fp8 defines them."""
    sl = slice(None) if batches is None else batches
    codes, ts = contiguous_codes(inp, batches)
    q = O.round_query_slices_e4m3(O.decode(q_bits[sl], inp.cfg.act_dtype), 128)
    q_rope, k_rope, lens = d["q_rope"][sl], d["k_rope"][sl], d["seq_lens"][sl]
    B, sq, n_h, d_c = q.shape
    allow = np.zeros((B, sq, n_h, d_c))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        C = O.decode_e4m3fn(codes[b, :L])
        t_s = np.asarray(ts[b, :L], np.float64)
        x = (d["scale"] * ((q[b] @ C.T) * t_s + q_rope[b] @ k_rope[b, :L].T) * np.log2(np.e)).reshape(sq * n_h, L)
        n_vis = np.repeat([O.visible_keys(L, sq, i) for i in range(sq)], n_h)
        vis = np.arange(L)[None, :] < n_vis[:, None]
        x = np.where(vis, x, -np.inf)
        top = np.max(x, axis=1, initial=-np.inf)
        k = np.where(np.isfinite(top), np.ceil(top), 0.0)
        w = np.where(vis, np.exp2(x - k[:, None]), 0.0)
        tot = w.sum(axis=1)
        v = w * t_s[None, :]
        m, e = np.frexp(v)
        pos = m * 16.0                       # position on the grid of 4 significant bits
        amb = vis & (np.abs(pos - np.floor(pos) - 0.5) < eps * pos)
        step = np.where(amb, np.ldexp(1.0, e - 4), 0.0)
        with np.errstate(divide="ignore", invalid="ignore"):
            a = np.where(tot[:, None] > 0, (step @ np.abs(C)) / tot[:, None], 0.0)
        allow[b] = a.reshape(sq, n_h, d_c)
    return allow


def measure_vs_exact(o, l, inp, q_bits, d, batches=None):
    sl = slice(None) if batches is None else batches
    q_dec = O.decode(q_bits[sl], inp.cfg.act_dtype)
    o_x, l_x = O.latent_attention(q_dec, d["q_rope"][sl], d["c_kv"][sl], d["k_rope"][sl], d["seq_lens"][sl],
                                  d["scale"])
    fin = np.isfinite(l_x)
    msg = f"o_lat {max_rel_err(o, o_x):.2e} lse {max_abs_err(l[fin], l_x[fin]):.2e} (dequantized cache)"
    if inp.c_kv_prequant is not None and not inp.cfg.paged:
        pre = np.where(np.isfinite(inp.c_kv_prequant[sl]), inp.c_kv_prequant[sl], 0).astype(np.float64)
        o_p, _ = O.latent_attention(q_dec, d["q_rope"][sl], pre, d["k_rope"][sl], d["seq_lens"][sl], d["scale"])
        msg += f", o_lat {max_rel_err(o, o_p):.2e} (pre-quantization)"
    print("  measured distance from exact attention: " + msg, flush=True)


def check(o, l, o_ref, l_ref, allow, what):
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref)), what
    fin = np.isfinite(l_ref)
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l[fin], l_ref[fin])
    scale = max(np.max(np.abs(o_ref)), 1e-300)
    beyond = np.max(np.maximum(np.abs(o - o_ref) - allow, 0.0)) / scale
    print(f"  {what}: against the fp8 definition o_lat {e_o:.2e} ({beyond:.2e} beyond the allowance for "
          f"ambiguous roundings, largest allowance {np.max(allow) / scale:.2e}) lse {e_l:.2e}", flush=True)
    assert beyond <= TOL and e_l <= TOL, (what, e_o, beyond, e_l)


# Ragged lengths with an empty sequence, one shorter than s_q = 4 (some queries see nothing)
# and lengths that end inside a 32-token half; balanced ranges, static splits of 64 and 192
# tokens (many partial pieces), a split of 1024 (one piece per sequence: the 700-token one
# runs 11 steps, so the loads of a step are issued during the products of the step three
# before it, the steady state of long sequences), and 4x larger logits (peaked attention).
CASES = [(0, 1.0), (64, 1.0), (192, 1.0), (1024, 1.0), (0, 4.0)]


@pytest.mark.parametrize("split_tokens,q_gain", CASES, ids=["balanced", "split64", "split192", "whole", "peaked"])
def test_decode_fp8_values(split_tokens, q_gain):
    cfg = configs.SPEC_FP8.with_(batch=5, seq_len=700, cfg_id=41)
    lengths = [700, 0, 2, 333, 97]
    say("decode fp8 values", split_tokens, q_gain, lengths, cfg)
    inp = synth.make_inputs(cfg, 0, lengths=np.array(lengths, np.int32), poison_tail=True, q_gain=q_gain)
    q_bits, d = stored_query(inp)
    o, l, w = run_decode(inp, q_bits, split_tokens)
    del w
    o_ref, l_ref = reference(inp, q_bits, d)
    empty = np.asarray(lengths) == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(l[empty]))
    check(o, l, o_ref, l_ref, flip_allowance(inp, q_bits, d), f"split {split_tokens} gain {q_gain}")
    measure_vs_exact(o, l, inp, q_bits, d)


def test_decode_fp8_values_deterministic():
    """The same plan and inputs give the same bits run to run."""
    cfg = configs.SPEC_FP8.with_(batch=3, seq_len=900, cfg_id=42)
    say("decode fp8 values determinism", cfg)
    inp = synth.make_inputs(cfg, 1, poison_tail=True)
    q_bits, _ = stored_query(inp)
    o1, l1, w = run_decode(inp, q_bits)
    w.decode(q_lat=to_device(q_bits, cfg.act_dtype, "cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(o1, to_host_f64(w.o_lat)) and np.array_equal(l1, to_host_f64(w.lse), equal_nan=True)


# Paged pools: block sizes 64 and 32 take one table entry per 32-token half (32: every step
# spans two blocks), 48 the token-by-token lookup.  Each must give the contiguous layout's
# bits, with NaN-poisoned rows outside every sequence.
@pytest.mark.parametrize("block_size", [64, 32, 48])
def test_paged_equals_contiguous_bitwise(block_size):
    cfg = configs.SPEC_FP8.with_(batch=5, seq_len=700, len_min=1, paged=True, block_size=block_size, cfg_id=43)
    say("fp8 values paged vs contiguous", block_size, cfg)
    inp = synth.make_inputs(cfg, 0, poison_tail=True)
    q_bits, d = stored_query(inp)
    o_p, l_p, w = run_decode(inp, q_bits)
    del w
    flat = synth.Inputs(**{**inp.__dict__})
    flat.cfg = cfg.with_(paged=False)
    flat.c_kv = O.gather_pages(inp.c_kv, inp.block_table, inp.seq_lens, cfg.seq_len, fill=synth.E4M3_NAN_CODE)
    flat.k_rope = O.gather_pages(inp.k_rope, inp.block_table, inp.seq_lens, cfg.seq_len, fill=synth.BF16_NAN_BITS)
    flat.kv_scale = O.gather_pages(inp.kv_scale, inp.block_table, inp.seq_lens, cfg.seq_len, fill=np.nan)
    flat.block_table = None
    o_c, l_c, w = run_decode(flat, q_bits)
    del w
    assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c, equal_nan=True)
    o_ref, l_ref = reference(inp, q_bits, d)
    check(o_p, l_p, o_ref, l_ref, flip_allowance(inp, q_bits, d), f"paged bs={block_size}")


def test_full_size_sampled_fp8_values():
    """The speculative fp8 workload at full size (the launch the benchmark times) on sampled
    sequences against the definition, then the whole step's distance from exact attention."""
    cfg = configs.SPEC_FP8
    say("full size fp8 values", cfg.name)
    inp = synth.make_inputs(cfg, 0)
    q_lat = O.absorb_query(O.decode(inp.q_nope, cfg.act_dtype), O.decode(inp.w_uk, cfg.act_dtype))
    q_bits = synth.store(q_lat.astype(np.float32), cfg.act_dtype)
    del q_lat
    w = DeviceWorkload(inp, fp8_scores=2)
    w.decode(q_lat=to_device(q_bits, cfg.act_dtype, "cuda"))
    torch.cuda.synchronize()
    o, l = to_host_f64(w.o_lat), to_host_f64(w.lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    batches = [5, 127]
    sub = synth.Inputs(**{**inp.__dict__})
    sub.q_nope, sub.q_rope, sub.seq_lens = inp.q_nope[batches], inp.q_rope[batches], inp.seq_lens[batches]
    sub.c_kv, sub.k_rope, sub.kv_scale = inp.c_kv[batches], inp.k_rope[batches], inp.kv_scale[batches]
    sub.c_kv_prequant = inp.c_kv_prequant[batches] if inp.c_kv_prequant is not None else None
    d = decoded(sub)
    o_ref, l_ref = reference(sub, q_bits[batches], d)
    check(o[batches], l[batches], o_ref, l_ref, flip_allowance(sub, q_bits[batches], d), "full size")
    measure_vs_exact(o[batches], l[batches], sub, q_bits[batches], d)
    del w


@pytest.mark.parametrize("fp8_scores", [1, 2])
def test_fused_absorb_out_equals_separate_calls(fp8_scores):
    """mla_decode_absorb_out with an fp8 product mode: o_lat, lse and out bit for bit those of
    mla_decode followed by mla_absorb_out (the same decode kernel; the range merge inside the
    absorption does the separate merge's arithmetic)."""
    cfg = configs.SPEC_FP8.with_(batch=6, seq_len=900, cfg_id=44)
    lengths = [900, 0, 3, 517, 64, 899]
    say("fused decode + absorb_out, fp8_scores", fp8_scores, lengths, cfg)
    inp = synth.make_inputs(cfg, 2, lengths=np.array(lengths, np.int32), poison_tail=True)
    w = DeviceWorkload(inp, fp8_scores=fp8_scores)
    w.absorb_q()
    w.decode()
    w.absorb_out()
    torch.cuda.synchronize()
    sep = {k: to_host_f64(t).copy() for k, t in (("o_lat", w.o_lat), ("lse", w.lse), ("out", w.out))}
    for t in (w.o_lat, w.lse, w.out):
        t.fill_(float("nan"))
    w.decode_absorb_out()
    torch.cuda.synchronize()
    for k, t in (("o_lat", w.o_lat), ("lse", w.lse), ("out", w.out)):
        assert np.array_equal(sep[k], to_host_f64(t), equal_nan=True), k
    assert np.all(np.isfinite(sep["out"]))
    del w
