"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (max |gpu - ref| / max |ref| per output tensor; the log-sum-exp, whose size is about
ln T, is held to the same number as an ABSOLUTE bar, max |gpu - ref|):
  fp32 workloads 1e-4; bf16 2e-2; fp8 cache 2e-2 against the oracle on the dequantized
  cache and 6e-2 against the oracle on the latent before quantization.
Integer work (block-table lookup, fp8 code table) is bit-exact.

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

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 2e-2}
TOL_FP8_PREQUANT = 6e-2


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()  # fails loudly when libmla.so is missing
    return "cuda"


def say(*a):
    print("[case]", *a, flush=True)


# The bf16 decode has three matrix-core kernels (row blocks of 128 query rows; of 64 rows
# with two score waves per row block; of 64 rows with loader, score and output roles) and a
# general one (any head count).  The plan picks by sequence length; the environment
# variables MLA_DECODE_ROW_BLOCK (128 or 64) and MLA_DECODE_PAIR ("0": the role kernel for
# 64-row blocks) force one of the first three, so every small case below runs on each.
KERNELS = {"rows128": (128, "128", None), "pair": (128, "64", None), "rows64": (128, "64", "0"),
           "general": (8, None, None)}


def use_kernel(kern, monkeypatch):
    n_heads, env, pair = KERNELS[kern]
    if env is None:
        monkeypatch.delenv("MLA_DECODE_ROW_BLOCK", raising=False)
    else:
        monkeypatch.setenv("MLA_DECODE_ROW_BLOCK", env)
    if pair is None:
        monkeypatch.delenv("MLA_DECODE_PAIR", raising=False)
    else:
        monkeypatch.setenv("MLA_DECODE_PAIR", pair)
    return n_heads


def run(inp, split_tokens=0, stages=True, fp8_scores=0):
    """Run the three calls; return host float64 arrays of every output."""
    w = DeviceWorkload(inp, split_tokens=split_tokens, fp8_scores=fp8_scores)
    w.step()
    torch.cuda.synchronize()
    res = {"q_lat": to_host_f64(w.q_lat), "o_lat": to_host_f64(w.o_lat),
           "lse": to_host_f64(w.lse), "out": to_host_f64(w.out), "plan": w.plan}
    return res, w


def oracle_full(d, batches=None):
    sl = slice(None) if batches is None else batches
    return O.mla_absorbed(d["q_nope"][sl], d["q_rope"][sl], d["c_kv"][sl], d["k_rope"][sl],
                          d["w_uk"], d["w_uv"], d["seq_lens"][sl], d["scale"])


def check_all(res, ref, tol, batches=None, what=""):
    sl = slice(None) if batches is None else batches
    errs = {k: max_rel_err(res[k][sl], ref[k]) for k in ("q_lat", "o_lat", "out")}
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isneginf(res["lse"][sl]), np.isneginf(ref["lse"])), what
    errs["lse"] = max_abs_err(res["lse"][sl][fin], ref["lse"][fin]) if fin.any() else 0.0
    print(f"  {what} max rel err (lse: abs): " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= tol, (what, k, v)
    return errs


# ------------------------------------------------------------------ utilities ----

def test_fp8_code_table_matches_format_definition():
    """Both device conversions (general kernels: to fp32; matrix-core kernels: to bf16)
    decode every e4m3fn code exactly as the format defines it."""
    say("fp8 table")
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    capi.mla_fp8_e4m3_table(out)
    ref = O.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    for half in (0, 1):
        got = out[256 * half:256 * (half + 1)].cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), half
        ok = ~np.isnan(ref)
        assert np.array_equal(got[ok], ref[ok]), half


@pytest.mark.parametrize("block_size", [64, 16, 7])
def test_gather_pages_bit_exact(block_size):
    cfg = configs.PAGED_VARLEN.with_(batch=5, seq_len=700, len_min=1, block_size=block_size, cfg_id=20)
    say("gather", block_size, cfg)
    inp = synth.make_inputs(cfg, 3)
    pool = to_device(inp.c_kv, "bf16", "cuda")
    table = to_device(inp.block_table, "i32", "cuda")
    lens = to_device(inp.seq_lens, "i32", "cuda")
    dst = torch.zeros(cfg.batch, cfg.seq_len, cfg.d_latent, dtype=torch.bfloat16, device="cuda")
    capi.mla_gather_pages(pool, table, lens, cfg.seq_len, dst)
    torch.cuda.synchronize()
    got = dst.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = O.gather_pages(inp.c_kv, inp.block_table, inp.seq_lens, cfg.seq_len, fill=0)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------- tiny (fp32) ----

def test_tiny_config_end_to_end():
    cfg = configs.TINY
    say("tiny", cfg)
    inp = synth.make_inputs(cfg, 0)
    d = decoded(inp)
    res, _ = run(inp)
    ref = oracle_full(d)
    check_all(res, ref, TOL["f32"], what="tiny")
    ex, _ = O.mla_explicit(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                           d["seq_lens"], d["scale"])
    assert max_rel_err(res["out"], ex) <= TOL["f32"]


@pytest.mark.parametrize("split_tokens", [0, 32, 100])
def test_tiny_config_splits_and_ragged(split_tokens):
    cfg = configs.TINY.with_(batch=3, q_len=2, cfg_id=21)
    say("tiny ragged", split_tokens, cfg)
    inp = synth.make_inputs(cfg, 1, lengths=np.array([128, 37, 2], np.int32), poison_tail=True)
    d = decoded(inp)
    res, _ = run(inp, split_tokens=split_tokens)
    check_all(res, oracle_full(d), TOL["f32"], what=f"tiny split={split_tokens}")


# ------------------------------------------------------- stage-by-stage bf16 ----

def test_absorb_q_and_out_v2_shapes():
    cfg = configs.V2_DECODE
    say("absorb stages", cfg)
    inp = synth.make_inputs(cfg.with_(seq_len=64), 0)
    d = decoded(inp)
    w = DeviceWorkload(inp)
    w.absorb_q()
    # Output side on its own: a latent output drawn as a stand-alone stored input.
    o_lat_bits = synth.make_stage_input(cfg, 0, "o_lat", (cfg.batch, 1, cfg.n_heads, cfg.d_latent), 0.1)
    o_lat = to_device(o_lat_bits, "bf16", "cuda")
    w.absorb_out(o_lat=o_lat)
    torch.cuda.synchronize()
    ref_q = O.absorb_query(d["q_nope"], d["w_uk"])
    e_q = max_rel_err(to_host_f64(w.q_lat), ref_q)
    ref_o = O.absorb_output(O.decode_bf16(o_lat_bits), d["w_uv"])
    e_o = max_rel_err(to_host_f64(w.out), ref_o)
    print(f"  absorb_q {e_q:.2e} absorb_out {e_o:.2e}")
    assert e_q <= TOL["bf16"] and e_o <= TOL["bf16"]


def decode_stage_case(cfg, seed, lengths, split_tokens, poison=True, q_gain=1.0, fp8_scores=0, edit=None):
    """mla_decode alone: both sides read the same stored q_lat (the oracle's q_lat rounded
    to the stored dtype), so only the attention stage is compared.  edit(inp), if given,
    changes the stored inputs before either side reads them."""
    inp = synth.make_inputs(cfg, seed, lengths=np.array(lengths, np.int32), poison_tail=poison,
                            q_gain=q_gain)
    if edit is not None:
        edit(inp)
    d = decoded(inp)
    q_lat = O.absorb_query(d["q_nope"], d["w_uk"])
    q_bits = synth.store(q_lat.astype(np.float32), cfg.act_dtype)
    q_dec = O.decode(q_bits, cfg.act_dtype)
    w = DeviceWorkload(inp, split_tokens=split_tokens, fp8_scores=fp8_scores)
    w.decode(q_lat=to_device(q_bits, cfg.act_dtype, "cuda"))
    torch.cuda.synchronize()
    o_ref, lse_ref = O.latent_attention(q_dec, d["q_rope"], d["c_kv"], d["k_rope"], d["seq_lens"],
                                        d["scale"])
    o_got, lse_got = to_host_f64(w.o_lat), to_host_f64(w.lse)
    return o_got, lse_got, o_ref, lse_ref, inp, d, w


@pytest.mark.parametrize("kern", list(KERNELS))
@pytest.mark.parametrize("split_tokens", [0, 64, 192, 512])
def test_decode_stage_bf16_ragged(split_tokens, kern, monkeypatch):
    n_heads = use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=3, seq_len=1000, cfg_id=22, n_heads=n_heads)
    say("decode bf16 ragged", split_tokens, cfg)
    o, l, o_ref, l_ref, *_ = decode_stage_case(cfg, 0, [1000, 77, 1], split_tokens)
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l, l_ref)
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= TOL["bf16"] and e_l <= TOL["bf16"]


@pytest.mark.parametrize("kern", ["rows128", "pair", "rows64"])
def test_decode_stage_peaked_scores(kern, monkeypatch):
    use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=2, seq_len=700, cfg_id=23)
    say("decode peaked", cfg)
    o, l, o_ref, l_ref, *_ = decode_stage_case(cfg, 0, [700, 333], 128, q_gain=4.0)
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l, l_ref)
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= TOL["bf16"] and e_l <= TOL["bf16"]


@pytest.mark.parametrize("kern", list(KERNELS))
@pytest.mark.parametrize("split_tokens", [0, 2048])
@pytest.mark.parametrize("gain", [8.0, 24.0])
def test_decode_rising_scores(gain, split_tokens, kern, monkeypatch):
    """Latent rows scaled up along the sequence (x1 at token 0 to x gain at the last), so
    every row's scores rise far above the max of its first tile.  The 128-row kernel fixes
    each row's reference at its first visible tile and reruns a piece against the true
    maxima once a score rises more than 64 (base 2) above it: gain 24 takes that second
    pass (rises of 49 to 125 on the single-piece split), gain 8 stays in the first pass with
    probabilities up to 2^40.  Both must match the oracle."""
    n_heads = use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=2, seq_len=1500, cfg_id=31, n_heads=n_heads)
    lengths = [1500, 900]

    def scale_up(inp):
        g = 1.0 + (gain - 1.0) * np.arange(cfg.seq_len) / (cfg.seq_len - 1)
        inp.c_kv = synth.store((O.decode(inp.c_kv, "bf16") * g[None, :, None]).astype(np.float32), "bf16")

    say("decode rising scores", gain, split_tokens, cfg)
    o, l, o_ref, l_ref, inp, d, _ = decode_stage_case(cfg, 0, lengths, split_tokens, edit=scale_up)
    # The rise the case is built for (first sequence, whole-sequence piece), in base 2.
    q = O.absorb_query(d["q_nope"], d["w_uk"])[0].reshape(-1, cfg.d_latent)
    s = (q @ d["c_kv"][0].T + d["q_rope"][0].reshape(-1, cfg.d_rope) @ d["k_rope"][0].T) * d["scale"] / np.log(2)
    rise = (s.max(1) - s[:, :32].max(1)).max()
    print(f"  largest rise above the first tile: {rise:.1f} (base 2)")
    assert (rise > 64) == (gain > 10)
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l, l_ref)
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= TOL["bf16"] and e_l <= TOL["bf16"]


@pytest.mark.parametrize("kern", list(KERNELS))
@pytest.mark.parametrize("split_tokens", [0, 128])
def test_decode_stage_bf16_causal(split_tokens, kern, monkeypatch):
    """Four query tokens per sequence, causal among them, on a bf16 cache, on every bf16
    kernel: query i of a sequence of L rows sees rows t <= L - 4 + i.  A sequence of 3 rows
    leaves its query 0 with no visible key: o_lat 0 and lse -inf."""
    n_heads = use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=3, q_len=4, seq_len=700, cfg_id=36, n_heads=n_heads)
    say("decode bf16 causal", split_tokens, cfg)
    o, l, o_ref, l_ref, *_ = decode_stage_case(cfg, 0, [700, 130, 3], split_tokens)
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l, l_ref)
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= TOL["bf16"] and e_l <= TOL["bf16"]
    none = ~np.isfinite(l_ref)
    assert none.sum() == n_heads  # query 0 of the 3-row sequence, every head
    assert np.all(l[none] == -np.inf) and np.all(o[none] == 0)


@pytest.mark.parametrize("kern", ["rows128", "pair", "rows64"])
def test_decode_stage_bf16_odd_row_blocks(kern, monkeypatch):
    """64 heads and 3 query tokens: 192 query rows per sequence, three 64-row blocks (the
    128-row kernel's second block half empty), causal, ragged lengths."""
    use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=3, q_len=3, n_heads=64, seq_len=900, cfg_id=37)
    say("decode bf16 192 rows", cfg)
    o, l, o_ref, l_ref, *_ = decode_stage_case(cfg, 0, [900, 250, 33], 0)
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l, l_ref)
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= TOL["bf16"] and e_l <= TOL["bf16"]


@pytest.mark.parametrize("n_heads", [128, 8], ids=["mfma", "general"])
@pytest.mark.parametrize("split_tokens", [0, 128])
def test_decode_stage_fp8_causal(split_tokens, n_heads):
    cfg = configs.SPEC_FP8.with_(batch=3, seq_len=700, cfg_id=24, n_heads=n_heads)
    say("decode fp8 causal", split_tokens, cfg)
    o, l, o_ref, l_ref, inp, d, _ = decode_stage_case(cfg, 0, [700, 130, 4], split_tokens)
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l, l_ref)
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e} (dequantized cache)")
    assert e_o <= TOL["fp8"] and e_l <= TOL["fp8"]
    # Against the latent before quantization (kernel + quantization error).
    pre = np.where(np.isfinite(inp.c_kv_prequant), inp.c_kv_prequant, 0).astype(np.float64)
    q_dec = O.decode(synth.store(O.absorb_query(d["q_nope"], d["w_uk"]).astype(np.float32), "bf16"), "bf16")
    o_pre, _ = O.latent_attention(q_dec, d["q_rope"], pre, d["k_rope"], d["seq_lens"], d["scale"])
    e_pre = max_rel_err(o, o_pre)
    print(f"  o_lat vs pre-quantization latent {e_pre:.2e}")
    assert e_pre <= TOL_FP8_PREQUANT


def test_causal_equals_independent_single_query_decodes():
    cfg = configs.SPEC_FP8.with_(batch=2, seq_len=300, cfg_id=25)
    say("causal vs single", cfg)
    lengths = np.array([300, 41], np.int32)
    inp = synth.make_inputs(cfg, 0, lengths=lengths)
    res, _ = run(inp, split_tokens=64)
    for i in range(cfg.q_len):
        one = synth.make_inputs(cfg.with_(q_len=1), 0, lengths=lengths - cfg.q_len + 1 + i)
        # Same cache and weights; the single query is query i of the causal block.
        one.q_nope = np.ascontiguousarray(inp.q_nope[:, i:i + 1])
        one.q_rope = np.ascontiguousarray(inp.q_rope[:, i:i + 1])
        one.c_kv, one.k_rope, one.kv_scale = inp.c_kv, inp.k_rope, inp.kv_scale
        one.w_uk, one.w_uv = inp.w_uk, inp.w_uv
        r1, _ = run(one, split_tokens=64)
        e = max_rel_err(r1["out"][:, 0], res["out"][:, i])
        print(f"  query {i}: {e:.2e}")
        assert e <= 1e-2


# -------------------------------------------------------------- paged cache ----

@pytest.mark.parametrize("kern", ["rows128", "pair", "rows64"])
def test_paged_equals_contiguous_bitwise(kern, monkeypatch):
    use_kernel(kern, monkeypatch)
    cfg = configs.PAGED_VARLEN.with_(batch=6, seq_len=1500, len_min=1, cfg_id=26)
    say("paged vs contiguous", cfg)
    inp = synth.make_inputs(cfg, 0, poison_tail=True)
    res_p, wp = run(inp, split_tokens=256)
    # Contiguous copy of the same rows (gathered on the host from the stored pool).
    flat = synth.Inputs(**{**inp.__dict__})
    flat.cfg = cfg.with_(paged=False)
    flat.c_kv = O.gather_pages(inp.c_kv, inp.block_table, inp.seq_lens, cfg.seq_len, fill=synth.BF16_NAN_BITS)
    flat.k_rope = O.gather_pages(inp.k_rope, inp.block_table, inp.seq_lens, cfg.seq_len, fill=synth.BF16_NAN_BITS)
    flat.block_table = None
    res_c, _ = run(flat, split_tokens=256)
    for k in ("o_lat", "lse", "out"):
        assert np.array_equal(res_p[k], res_c[k], equal_nan=True), k
    d = decoded(inp)
    check_all(res_p, oracle_full(d), TOL["bf16"], what="paged")


# Every paged layout of the decode kernel against the contiguous one, bit for bit, for bf16
# and fp8 caches: blocks of 64 tokens (each 32-token tile inside one block, one table entry
# per tile) and of 48 and 16 tokens (rows looked up token by token).  Rows a sequence does not
# own hold NaN in both layouts, so reading one would show.
# The fp8 score product ("fp8s": the loaders also stage the stored codes) is checked the same
# way for the tile-per-block and the token-by-token layouts.
PAGED_LAYOUT_CASES = [(kv, bs, 0) for kv in ("bf16", "fp8") for bs in (64, 48, 16)] + \
    [("fp8", 64, 1), ("fp8", 48, 1)]


@pytest.mark.parametrize("kv,block_size,fp8_scores", PAGED_LAYOUT_CASES,
                         ids=[f"{k}-{b}" + ("-fp8s" if f else "") for k, b, f in PAGED_LAYOUT_CASES])
@pytest.mark.parametrize("kern", ["rows128", "pair", "rows64"])
def test_paged_layouts_equal_contiguous_bitwise(kv, block_size, fp8_scores, kern, monkeypatch):
    if kv != "bf16" and kern == "rows128":
        pytest.skip("the 128-row kernel reads bf16 caches only")
    use_kernel(kern, monkeypatch)
    base = configs.PAGED_VARLEN if kv == "bf16" else configs.SPEC_FP8
    cfg = base.with_(batch=5, seq_len=700, len_min=1, paged=True, block_size=block_size, cfg_id=27)
    say("paged layout vs contiguous", kv, block_size, "fp8_scores", fp8_scores, cfg)
    inp = synth.make_inputs(cfg, 0, poison_tail=True)
    res_p, _ = run(inp, fp8_scores=fp8_scores)
    flat = synth.Inputs(**{**inp.__dict__})
    flat.cfg = cfg.with_(paged=False)
    lat_fill = synth.BF16_NAN_BITS if kv == "bf16" else synth.E4M3_NAN_CODE
    flat.c_kv = O.gather_pages(inp.c_kv, inp.block_table, inp.seq_lens, cfg.seq_len, fill=lat_fill)
    flat.k_rope = O.gather_pages(inp.k_rope, inp.block_table, inp.seq_lens, cfg.seq_len, fill=synth.BF16_NAN_BITS)
    if kv == "fp8":
        flat.kv_scale = O.gather_pages(inp.kv_scale, inp.block_table, inp.seq_lens, cfg.seq_len, fill=np.nan)
    flat.block_table = None
    res_c, _ = run(flat, fp8_scores=fp8_scores)
    for k in ("o_lat", "lse", "out"):
        assert np.array_equal(res_p[k], res_c[k], equal_nan=True), k
    check_all(res_p, oracle_full(decoded(inp)), TOL_FP8_PREQUANT if fp8_scores else TOL[kv],
              what=f"paged {kv} bs={block_size} fp8_scores={fp8_scores}")


# ------------------------------------------------ full-size, sampled oracle ----

FULL = [configs.TINY, configs.V2_DECODE, configs.PAGED_VARLEN, configs.LONG_CONTEXT, configs.SPEC_FP8]
SAMPLE = {configs.V2_DECODE.name: [0, 17, 31], configs.PAGED_VARLEN.name: [0, 33, 63],
          configs.LONG_CONTEXT.name: [2], configs.SPEC_FP8.name: [5, 127]}


# Each workload at full size with the plan's own kernel choice, plus the bf16 decode and the
# paged workload forced onto the other matrix-core kernels.
FULL_CASES = [(c, None) for c in FULL] + [(configs.V2_DECODE, "rows128"), (configs.V2_DECODE, "rows64"),
                                          (configs.PAGED_VARLEN, "pair"), (configs.PAGED_VARLEN, "rows64")]


@pytest.mark.parametrize("cfg,kern", FULL_CASES, ids=[c.name + (f"-{k}" if k else "") for c, k in FULL_CASES])
def test_full_size_sampled(cfg, kern, monkeypatch):
    if kern is not None:
        use_kernel(kern, monkeypatch)
    say("full size", cfg.name, kern or "planned kernel")
    inp = synth.make_inputs(cfg, 0)
    res, w = run(inp)
    print(f"  plan (splits, tokens) = {res['plan']}", flush=True)
    for k in ("o_lat", "out", "lse"):
        assert np.all(np.isfinite(res[k])), k
    batches = SAMPLE.get(cfg.name)
    d = decoded_batches(inp, batches)
    ref = oracle_full(d)
    sl = slice(None) if batches is None else batches
    errs = check_all(res, ref, TOL[cfg.kv_dtype], batches=sl, what=cfg.name)
    if cfg.kv_dtype == "fp8":
        # Kernel + quantization error: the same sampled sequences against the oracle on the
        # latent before quantization.
        pre_ref = oracle_prequant(inp, batches)
        e_pre = {k: max_rel_err(res[k][sl], pre_ref[k]) for k in ("o_lat", "out")}
        fin = np.isfinite(pre_ref["lse"])
        e_pre["lse"] = max_abs_err(res["lse"][sl][fin], pre_ref["lse"][fin])
        print("  against the pre-quantization latent: " + ", ".join(f"{k}={v:.2e}" for k, v in e_pre.items()),
              flush=True)
        for k, v in e_pre.items():
            assert v <= TOL_FP8_PREQUANT, (k, v)
    del w


def oracle_prequant(inp, batches):
    """The oracle's whole absorbed step on the float32 latent before fp8 encoding, for the
    sampled sequences of a contiguous fp8 workload."""
    sub = synth.Inputs(**{**inp.__dict__})
    sub.q_nope, sub.q_rope = inp.q_nope[batches], inp.q_rope[batches]
    sub.seq_lens = inp.seq_lens[batches]
    sub.c_kv, sub.k_rope, sub.kv_scale = inp.c_kv[batches], inp.k_rope[batches], inp.kv_scale[batches]
    d = decoded(sub)
    d["c_kv"] = np.where(np.isfinite(inp.c_kv_prequant[batches]), inp.c_kv_prequant[batches], 0).astype(np.float64)
    return oracle_full(d)


def decoded_batches(inp, batches):
    """Decode only the sampled sequences (keeps the oracle's work and memory small)."""
    if batches is None:
        return decoded(inp)
    sub = synth.Inputs(**{**inp.__dict__})
    sub.q_nope, sub.q_rope = inp.q_nope[batches], inp.q_rope[batches]
    sub.seq_lens = inp.seq_lens[batches]
    if inp.cfg.paged:
        sub.block_table = inp.block_table[batches]
    else:
        sub.c_kv, sub.k_rope = inp.c_kv[batches], inp.k_rope[batches]
        if inp.kv_scale is not None:
            sub.kv_scale = inp.kv_scale[batches]
    return decoded(sub)


@pytest.mark.parametrize("kern", ["rows128", "pair", "rows64"])
def test_run_to_run_bitwise_deterministic(kern, monkeypatch):
    use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=4, seq_len=2048, cfg_id=27)
    say("determinism", cfg)
    inp = synth.make_inputs(cfg, 0)
    r1, w = run(inp, split_tokens=256)
    w.step()
    torch.cuda.synchronize()
    for k, t in (("o_lat", w.o_lat), ("lse", w.lse), ("out", w.out)):
        assert np.array_equal(r1[k], to_host_f64(t)), k


@pytest.mark.parametrize("kern", list(KERNELS))
def test_lengths_above_T_are_clamped(kern, monkeypatch):
    """Every kernel of the call clamps seq_lens[b] to [0, T]: lengths above T give the
    result of length T (and read no row past T)."""
    n_heads = use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=3, seq_len=256, cfg_id=29, n_heads=n_heads)
    say("lengths above T", cfg)
    o_t, l_t, o_ref, _, inp, _, w = decode_stage_case(cfg, 0, [256, 256, 100], 64)
    # The same workload on the device, with the first two stored lengths past T.
    w.seq_lens.copy_(torch.tensor([256 + 37, 256 + 1, 100], dtype=torch.int32))
    q_bits = synth.store(O.absorb_query(O.decode(inp.q_nope, "bf16"), O.decode(inp.w_uk, "bf16"))
                         .astype(np.float32), "bf16")
    w.decode(q_lat=to_device(q_bits, "bf16", "cuda"))
    torch.cuda.synchronize()
    o_x, l_x = to_host_f64(w.o_lat), to_host_f64(w.lse)
    assert np.array_equal(o_t, o_x) and np.array_equal(l_t, l_x)
    assert max_rel_err(o_x, o_ref) <= TOL["bf16"]


@pytest.mark.parametrize("kern", list(KERNELS))
def test_empty_and_short_sequences(kern, monkeypatch):
    n_heads = use_kernel(kern, monkeypatch)
    cfg = configs.V2_DECODE.with_(batch=3, seq_len=256, cfg_id=28, n_heads=n_heads)
    say("empty sequence", cfg)
    o, l, o_ref, l_ref, *_ = decode_stage_case(cfg, 0, [0, 1, 256], 64)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert max_rel_err(o, o_ref) <= TOL["bf16"]


# Balanced ranges (the default plan of the matrix-core path): the batch's tiles are cut into
# equal ranges on the device, so sequences are split at data-dependent places, several
# whole sequences can share a workgroup, ranges can be empty (fewer tiles than ranges), and
# batches above 1024 sequences take the separate prefix kernel.  Up to 64 sequences each
# wave scans the lengths on its own (one lane per sequence); 65 takes the workgroup scan.
_LENS_64 = [int(x) for x in np.random.default_rng(11).integers(0, 301, size=64)]
_LENS_64[0] = _LENS_64[63] = 0  # empty first and last sequences
BALANCED_CASES = {
    "many_short": (dict(batch=200, seq_len=200, n_heads=128), None),
    "wave_scan_64": (dict(batch=64, seq_len=300, n_heads=128), _LENS_64),
    "workgroup_scan_65": (dict(batch=65, seq_len=300, n_heads=128), _LENS_64 + [300]),
    "fewer_tiles_than_ranges": (dict(batch=2, seq_len=40, n_heads=128), [1, 40]),
    "empty_sequences": (dict(batch=5, seq_len=300, n_heads=128), [0, 300, 0, 1, 65]),
    "prefix_kernel_batch": (dict(batch=1100, seq_len=64, n_heads=64), None),
}


@pytest.mark.parametrize("kern", ["rows128", "pair", "rows64"])
@pytest.mark.parametrize("case", list(BALANCED_CASES))
def test_decode_balanced_ranges(case, kern, monkeypatch):
    use_kernel(kern, monkeypatch)
    kw, lengths = BALANCED_CASES[case]
    cfg = configs.V2_DECODE.with_(cfg_id=30, **kw)
    if lengths is None:
        lengths = np.random.default_rng(7).integers(1, cfg.seq_len + 1, size=cfg.batch)
    say("decode balanced", case, cfg.batch, cfg.n_heads, cfg.seq_len)
    o, l, o_ref, l_ref, inp, d, w = decode_stage_case(cfg, 0, lengths, 0)
    assert w.plan[1] == 0, w.plan  # balanced ranges
    empty = np.asarray(lengths) == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(l[empty]))
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref))
    e_o, e_l = max_rel_err(o, o_ref), max_abs_err(l[fin], l_ref[fin])
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e}", flush=True)
    assert e_o <= TOL["bf16"] and e_l <= TOL["bf16"]


# fp8 score product (dims.fp8_scores = 1): the kernel rounds each row's 128-column query
# slices to e4m3 and multiplies them with the stored codes.  Its parity reference is the
# oracle's plain definition of that approximation (latent_attention_fp8_query: the same
# rounding of the query, then exact attention), held to the fp8 cache's kernel bar 2e-2
# (lse: absolute).  How far the approximation itself is from exact attention is printed as a
# measurement: the e4m3 query rounding moves each logit by about 2^-4 of its size, so on a
# sequence of a few tokens the log-sum-exp moves by several 1e-2, and at 4x larger logits
# (peaked attention) the output by several percent.
# A split of 1024 keeps each sequence in one piece (11 steps for 700 tokens: the steady state
# of long sequences, where a step's loads are issued among earlier products).
@pytest.mark.parametrize("split_tokens,q_gain", [(0, 1.0), (128, 1.0), (1024, 1.0), (0, 4.0)],
                         ids=["balanced", "split128", "whole", "peaked"])
def test_decode_fp8_scores(split_tokens, q_gain):
    cfg = configs.SPEC_FP8.with_(batch=3, seq_len=700, cfg_id=31)
    say("decode fp8 scores", split_tokens, q_gain, cfg)
    o, l, o_ref, l_ref, inp, d, _ = decode_stage_case(cfg, 0, [700, 130, 4], split_tokens,
                                                      q_gain=q_gain, fp8_scores=1)
    q_dec = O.decode(synth.store(O.absorb_query(d["q_nope"], d["w_uk"]).astype(np.float32), "bf16"), "bf16")
    o_apx, l_apx = O.latent_attention_fp8_query(q_dec, d["q_rope"], d["c_kv"], d["k_rope"], d["seq_lens"],
                                                d["scale"])
    e_o, e_l = max_rel_err(o, o_apx), max_abs_err(l, l_apx)
    assert np.array_equal(np.isneginf(l), np.isneginf(l_apx))
    pre = np.where(np.isfinite(inp.c_kv_prequant), inp.c_kv_prequant, 0).astype(np.float64)
    o_pre, _ = O.latent_attention(q_dec, d["q_rope"], pre, d["k_rope"], d["seq_lens"], d["scale"])
    print(f"  against the fp8-query definition: o_lat {e_o:.2e} lse {e_l:.2e}; measured distance from "
          f"exact attention: o_lat {max_rel_err(o, o_ref):.2e} lse {max_abs_err(l, l_ref):.2e} "
          f"(dequantized cache), o_lat {max_rel_err(o, o_pre):.2e} (pre-quantization)", flush=True)
    assert e_o <= TOL["fp8"] and e_l <= TOL["fp8"]


def test_full_size_sampled_fp8_scores():
    """The speculative fp8 workload at full size with the fp8 score product: the decode call
    on the oracle's q_lat (stored as bf16, so both sides round the same query) against the
    fp8-query definition on sampled sequences; then the whole step, whose distance from
    exact attention is printed as a measurement."""
    cfg = configs.SPEC_FP8
    say("full size fp8 scores", cfg.name)
    inp = synth.make_inputs(cfg, 0)
    q_lat = O.absorb_query(O.decode(inp.q_nope, cfg.act_dtype), O.decode(inp.w_uk, cfg.act_dtype))
    q_bits = synth.store(q_lat.astype(np.float32), cfg.act_dtype)
    del q_lat
    w = DeviceWorkload(inp, fp8_scores=1)
    w.decode(q_lat=to_device(q_bits, cfg.act_dtype, "cuda"))
    torch.cuda.synchronize()
    o, l = to_host_f64(w.o_lat), to_host_f64(w.lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    batches = SAMPLE[cfg.name]
    d = decoded_batches(inp, batches)
    o_apx, l_apx = O.latent_attention_fp8_query(O.decode(q_bits[batches], cfg.act_dtype), d["q_rope"], d["c_kv"],
                                                d["k_rope"], d["seq_lens"], d["scale"])
    e_o, e_l = max_rel_err(o[batches], o_apx), max_abs_err(l[batches], l_apx)
    print(f"  decode vs fp8-query definition: o_lat {e_o:.2e} lse {e_l:.2e}", flush=True)
    assert e_o <= TOL["fp8"] and e_l <= TOL["fp8"]
    w.step()
    torch.cuda.synchronize()
    ref = oracle_full(d)
    print(f"  whole step, measured distance from exact attention: out "
          f"{max_rel_err(to_host_f64(w.out)[batches], ref['out']):.2e}", flush=True)
    del w


def test_binding_rejects_strided_views():
    """A transposed or sliced view would be read as a dense array at its address; the
    binding refuses it (a dense copy is accepted)."""
    say("binding strided view")
    cfg = configs.V2_DECODE.with_(batch=2, seq_len=64, cfg_id=34)
    d = capi.dims_from_config(cfg)
    q = torch.zeros(2, 1, 128, 256, dtype=torch.bfloat16, device="cuda")[..., :128]
    w_uk = torch.zeros(128, 128, 512, dtype=torch.bfloat16, device="cuda")
    q_lat = torch.empty(2, 1, 128, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="contiguous"):
        capi.mla_absorb_q(d, q, w_uk, q_lat)
    capi.mla_absorb_q(d, q.contiguous(), w_uk, q_lat)
    torch.cuda.synchronize()
    assert int(q_lat.count_nonzero()) == 0
