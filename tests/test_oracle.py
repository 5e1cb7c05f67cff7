"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each pin is a plain function so that tests/test_oracle_mutations.py can plant a
mistake in the oracle and check that some pin fails.

What pins what:
* codecs -- torch's CPU casts (all 256 e4m3fn codes; bf16 bit patterns);
* cache arithmetic -- the numbers "Operator Notes (1): MLA" prints (tests/golden);
* explicit form -- torch scaled_dot_product_attention (fp64, CPU, explicit scale and
  boolean mask built from token positions) and pure-Python loops on tiny inputs;
* absorbed form -- equals the explicit form (associativity, which the pages state);
* softmax -- rows sum to one, no negative weights;
* closed forms -- one visible token, zero query, identical tokens, a constant added
  to every logit, token permutation, identity weights (MQA over the latent);
* split/merge -- any partition of the tokens merges back to the single pass;
* paging -- gather through a block table inverts a scatter with a known permutation;
* fp8 encoding -- round trip within the format's half-ulp bound.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_lat_amd import configs, synth
from conftest import decoded

HERE = os.path.dirname(os.path.abspath(__file__))

SMALL = configs.MLAConfig(
    name="small_f32", cfg_id=100, batch=2, q_len=3, n_heads=4, d_head=8, d_latent=16,
    d_rope=4, seq_len=20, kv_dtype="f32", act_dtype="f32")


def small_inputs(seed=0, lengths=(20, 7), cfg=SMALL, **kw):
    return decoded(synth.make_inputs(cfg, seed, lengths=np.array(lengths, np.int32), **kw))


# ------------------------------------------------------------------------ pins ----

def pin_e4m3_table():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_bf16_decode():
    bits = np.random.default_rng(1).integers(0, 1 << 16, size=4096).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x7F7F], np.uint16)])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_cache_arithmetic():
    g = json.load(open(os.path.join(HERE, "golden", "cache_arithmetic.json")))
    mha = O.mha_cache_numbers_per_token(g["n_heads"], g["d_head"])
    mla = O.mla_cache_numbers_per_token(g["d_latent"])
    assert mha == g["mha_numbers_per_token"]
    assert mla == g["mla_numbers_per_token"]
    assert round(mha * g["context_tokens"] / 1e9, 2) == g["mha_numbers_at_context_billion"]
    assert round(mla * g["context_tokens"] / 1e9, 2) == g["mla_numbers_at_context_billion"]
    assert round(mha / mla) == g["shrink_factor_approx"]
    assert round(100 * (1 - mla / mha), 1) == g["reduction_percent_approx"]


def _positions_mask(L, sq, T):
    """Query i sits at absolute position L - sq + i and may see positions <= its own."""
    qpos = (L - sq + np.arange(sq))[:, None]
    kpos = np.arange(T)[None, :]
    return (kpos <= qpos) & (kpos < L)


def sdpa_reference(d):
    """Explicit attention through torch's library routine, per (b, h), fp64 on CPU."""
    q_nope, q_rope, c, r = d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"]
    B, sq, n_h, d_h = q_nope.shape
    T = c.shape[1]
    out = np.zeros((B, sq, n_h, d_h))
    for b in range(B):
        L = int(d["seq_lens"][b])
        mask = torch.from_numpy(_positions_mask(L, sq, T))
        for h in range(n_h):
            K = c[b] @ d["w_uk"][h].T                   # [T, d_h]
            V = c[b] @ d["w_uv"][h]                     # [T, d_h]
            q = np.concatenate([q_nope[b, :, h], q_rope[b, :, h]], axis=-1)
            k = np.concatenate([K, r[b]], axis=-1)
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(V)[None],
                attn_mask=mask[None], scale=d["scale"])
            out[b, :, h] = o[0].numpy()
    return out


def pin_explicit_vs_sdpa(d):
    ref = sdpa_reference(d)
    got, _ = O.mla_explicit(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"],
                            d["w_uv"], d["seq_lens"], d["scale"])
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-12), np.max(np.abs(got - ref))


def brute_force(d):
    """Pure-Python loops, one (b, i, h) row at a time, straight from the definition."""
    q_nope, q_rope, c, r = d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"]
    wk, wv = d["w_uk"], d["w_uv"]
    B, sq, n_h, d_h = q_nope.shape
    d_c, d_r = c.shape[2], r.shape[2]
    out = np.zeros((B, sq, n_h, d_h))
    for b in range(B):
        L = int(d["seq_lens"][b])
        for i in range(sq):
            last = L - sq + i
            for h in range(n_h):
                scores = []
                for t in range(L):
                    if t > last:
                        continue
                    dot = 0.0
                    for j in range(d_h):
                        k_tj = sum(c[b, t, cc] * wk[h, j, cc] for cc in range(d_c))
                        dot += q_nope[b, i, h, j] * k_tj
                    for rr in range(d_r):
                        dot += q_rope[b, i, h, rr] * r[b, t, rr]
                    scores.append((t, d["scale"] * dot))
                if not scores:
                    continue
                mx = max(s for _, s in scores)
                ws = [(t, math.exp(s - mx)) for t, s in scores]
                tot = sum(w for _, w in ws)
                for j in range(d_h):
                    acc = 0.0
                    for t, w in ws:
                        v_tj = sum(c[b, t, cc] * wv[h, cc, j] for cc in range(d_c))
                        acc += (w / tot) * v_tj
                    out[b, i, h, j] = acc
    return out


def pin_explicit_vs_brute(d):
    ref = brute_force(d)
    got, _ = O.mla_explicit(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"],
                            d["w_uv"], d["seq_lens"], d["scale"])
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12), np.max(np.abs(got - ref))


def pin_absorbed_vs_explicit(d, rows=None, tol=1e-10):
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"],
                         d["w_uv"], d["seq_lens"], d["scale"])
    ex, ex_lse = O.mla_explicit(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"],
                                d["w_uv"], d["seq_lens"], d["scale"], rows=rows)
    m = ~np.isnan(ex)
    err = np.max(np.abs(res["out"][m] - ex[m])) / np.max(np.abs(ex[m]))
    assert err <= tol, err
    ml = ~np.isnan(ex_lse)
    assert np.allclose(res["lse"][ml], ex_lse[ml], rtol=0, atol=1e-10)


def pin_softmax_rows():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((9, 33)) * 5
    n_vis = np.array([33, 1, 0, 5, 33, 2, 17, 32, 8])
    p, lse = O._softmax_rows(s, n_vis)
    assert np.all(p >= 0)
    assert np.allclose(p.sum(axis=1)[n_vis > 0], 1.0, atol=1e-12)
    assert np.all(p[n_vis == 0] == 0) and np.all(np.isneginf(lse[n_vis == 0]))
    for r in range(9):
        assert np.all(p[r, n_vis[r]:] == 0)
        if n_vis[r]:
            ref = np.log(np.sum(np.exp(s[r, :n_vis[r]])))
            assert abs(lse[r] - ref) < 1e-12


def pin_split_merge(d, n_splits):
    q_lat = O.absorb_query(d["q_nope"], d["w_uk"])
    full_o, full_lse = O.latent_attention(q_lat, d["q_rope"], d["c_kv"], d["k_rope"],
                                          d["seq_lens"], d["scale"])
    B, sq = q_lat.shape[:2]
    T = d["c_kv"].shape[1]
    bounds = np.linspace(0, T, n_splits + 1).round().astype(int)
    parts_o, parts_l = [], []
    for s in range(n_splits):
        lo, hi = bounds[s], bounds[s + 1]
        # The subset [lo, hi): run attention on those rows only, with the causal limit of
        # each query expressed through a per-query visible count inside the subset.
        o = np.zeros_like(full_o)
        l = np.full(full_lse.shape, -np.inf)
        for b in range(B):
            L = int(d["seq_lens"][b])
            for i in range(sq):
                vis_hi = min(hi, O.visible_keys(L, sq, i))
                n = max(vis_hi - lo, 0)
                if n == 0:
                    continue
                oo, ll = O.latent_attention(q_lat[b:b + 1, i:i + 1], d["q_rope"][b:b + 1, i:i + 1],
                                            d["c_kv"][b:b + 1, lo:lo + n], d["k_rope"][b:b + 1, lo:lo + n],
                                            np.array([n]), d["scale"])
                o[b, i], l[b, i] = oo[0, 0], ll[0, 0]
        parts_o.append(o)
        parts_l.append(l)
    mo, ml = O.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.allclose(mo, full_o, rtol=0, atol=1e-12), np.max(np.abs(mo - full_o))
    fin = np.isfinite(full_lse)
    assert np.allclose(ml[fin], full_lse[fin], atol=1e-12)
    assert np.array_equal(np.isneginf(ml), np.isneginf(full_lse))


# ----------------------------------------------------------------------- tests ----

def test_e4m3_table():
    pin_e4m3_table()


def test_bf16_decode():
    pin_bf16_decode()


def test_cache_arithmetic_matches_page():
    pin_cache_arithmetic()
    # With the decoupled RoPE key of width 64 the MLA cache is 576 numbers per token.
    assert O.mla_cache_numbers_per_token(512, 64) == 576


@pytest.mark.parametrize("lengths", [(20, 7), (3, 20), (20, 20)])
def test_explicit_matches_torch_sdpa(lengths):
    pin_explicit_vs_sdpa(small_inputs(lengths=lengths))


def test_explicit_matches_sdpa_single_query():
    cfg = SMALL.with_(q_len=1, cfg_id=101)
    pin_explicit_vs_sdpa(small_inputs(cfg=cfg, lengths=(20, 9)))


def test_explicit_matches_brute_force():
    tiny = configs.MLAConfig(name="bf", cfg_id=102, batch=2, q_len=2, n_heads=2, d_head=3,
                             d_latent=5, d_rope=2, seq_len=6, kv_dtype="f32", act_dtype="f32")
    pin_explicit_vs_brute(small_inputs(cfg=tiny, lengths=(6, 3)))


def test_absorbed_equals_explicit_small():
    pin_absorbed_vs_explicit(small_inputs())


def test_absorbed_equals_explicit_tiny_config():
    d = decoded(synth.make_inputs(configs.TINY, 0))
    pin_absorbed_vs_explicit(d)


def test_absorbed_equals_explicit_v2_shapes_sampled():
    """Full DeepSeek-V2 widths (n_h=d_h=128, d_c=512, d_r=64) on a short context."""
    cfg = configs.V2_DECODE.with_(batch=2, seq_len=256)
    d = decoded(synth.make_inputs(cfg, 0))
    rows = [(0, 0, 0), (0, 0, 77), (1, 0, 127), (1, 0, 5)]
    pin_absorbed_vs_explicit(d, rows=rows)


def test_absorbed_equals_explicit_causal_fp8():
    cfg = configs.SPEC_FP8.with_(batch=2, seq_len=64, n_heads=8)
    d = decoded(synth.make_inputs(cfg, 0))
    pin_absorbed_vs_explicit(d)


def test_softmax_rows():
    pin_softmax_rows()


def test_single_visible_token_closed_form():
    d = small_inputs(lengths=(1, 1), cfg=SMALL.with_(q_len=1, cfg_id=103))
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                         d["seq_lens"], d["scale"])
    for b in range(2):
        for h in range(SMALL.n_heads):
            assert np.allclose(res["o_lat"][b, 0, h], d["c_kv"][b, 0], atol=1e-14)
            assert np.allclose(res["out"][b, 0, h], d["c_kv"][b, 0] @ d["w_uv"][h], atol=1e-12)


def test_zero_query_gives_mean_of_visible_latents():
    d = small_inputs()
    d["q_nope"][:] = 0
    d["q_rope"][:] = 0
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                         d["seq_lens"], d["scale"])
    for b in range(2):
        L = int(d["seq_lens"][b])
        for i in range(SMALL.q_len):
            n = O.visible_keys(L, SMALL.q_len, i)
            assert np.allclose(res["o_lat"][b, i], d["c_kv"][b, :n].mean(axis=0)[None], atol=1e-13)
            assert np.allclose(res["lse"][b, i], math.log(n), atol=1e-13)


def test_identical_tokens_give_that_token():
    d = small_inputs()
    d["c_kv"][:] = d["c_kv"][:, :1]
    d["k_rope"][:] = d["k_rope"][:, :1]
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                         d["seq_lens"], d["scale"])
    for b in range(2):
        assert np.allclose(res["o_lat"][b], np.broadcast_to(d["c_kv"][b, 0], res["o_lat"][b].shape),
                           atol=1e-13)


def test_constant_logit_shift_leaves_output_unchanged():
    """An extra RoPE channel whose key is 1 for every token adds scale*a to every logit
    of a row whose query component is a: outputs stay, lse moves by exactly that."""
    d = small_inputs()
    base = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                          d["seq_lens"], d["scale"])
    a = np.random.default_rng(5).standard_normal(d["q_rope"].shape[:3]) * 3
    q_rope = np.concatenate([d["q_rope"], a[..., None]], axis=-1)
    k_rope = np.concatenate([d["k_rope"], np.ones(d["k_rope"].shape[:2] + (1,))], axis=-1)
    sh = O.mla_absorbed(d["q_nope"], q_rope, d["c_kv"], k_rope, d["w_uk"], d["w_uv"],
                        d["seq_lens"], d["scale"])
    assert np.allclose(sh["out"], base["out"], atol=1e-12)
    assert np.allclose(sh["lse"], base["lse"] + d["scale"] * a, atol=1e-12)


def test_token_permutation_invariance():
    cfg = SMALL.with_(q_len=1, cfg_id=104)
    d = small_inputs(cfg=cfg, lengths=(20, 20))
    base = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                          d["seq_lens"], d["scale"])
    perm = np.random.default_rng(9).permutation(20)
    pm = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"][:, perm], d["k_rope"][:, perm],
                        d["w_uk"], d["w_uv"], d["seq_lens"], d["scale"])
    assert np.allclose(pm["out"], base["out"], atol=1e-12)
    assert np.allclose(pm["lse"], base["lse"], atol=1e-12)


def test_identity_weights_reduce_to_mqa_over_latent():
    """d_h = d_c and W_UK[h] = W_UV[h] = I: every head attends over the latent itself,
    i.e. multi-query attention with one shared key/value head."""
    cfg = SMALL.with_(d_head=16, d_latent=16, cfg_id=105)
    d = small_inputs(cfg=cfg)
    eye = np.broadcast_to(np.eye(16), (cfg.n_heads, 16, 16)).copy()
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], eye, eye,
                         d["seq_lens"], d["scale"])
    B, sq, n_h = cfg.batch, cfg.q_len, cfg.n_heads
    for b in range(B):
        L = int(d["seq_lens"][b])
        mask = torch.from_numpy(_positions_mask(L, sq, cfg.seq_len))
        q = np.concatenate([d["q_nope"][b], d["q_rope"][b]], -1).transpose(1, 0, 2)  # [n_h, sq, D]
        k = np.concatenate([d["c_kv"][b], d["k_rope"][b]], -1)
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(np.broadcast_to(k, (n_h,) + k.shape).copy()),
            torch.from_numpy(np.broadcast_to(d["c_kv"][b], (n_h,) + d["c_kv"][b].shape).copy()),
            attn_mask=mask[None], scale=d["scale"]).numpy()
        assert np.allclose(res["out"][b], o.transpose(1, 0, 2), atol=1e-12)


@pytest.mark.parametrize("n_splits", [1, 2, 7, 20])
def test_split_merge_equals_single_pass(n_splits):
    pin_split_merge(small_inputs(), n_splits)


def test_causal_equals_independent_single_query_decodes():
    d = small_inputs()
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                         d["seq_lens"], d["scale"])
    sq = SMALL.q_len
    for i in range(sq):
        lens = np.array([L - sq + i + 1 for L in d["seq_lens"]])
        one = O.mla_absorbed(d["q_nope"][:, i:i + 1], d["q_rope"][:, i:i + 1], d["c_kv"], d["k_rope"],
                             d["w_uk"], d["w_uv"], lens, d["scale"])
        assert np.allclose(one["out"][:, 0], res["out"][:, i], atol=1e-13)


def test_no_visible_key_gives_zero_and_neg_inf():
    d = small_inputs(lengths=(0, 2))
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                         d["seq_lens"], d["scale"])
    assert np.all(res["out"][0] == 0) and np.all(np.isneginf(res["lse"][0]))
    # sequence 1 has 2 rows and 3 queries: query 0 sees nothing, queries 1, 2 see 1, 2 rows.
    assert np.all(res["out"][1, 0] == 0) and np.all(np.isneginf(res["lse"][1, 0]))
    assert np.all(np.isfinite(res["lse"][1, 1:]))


def test_gather_pages_inverts_scatter():
    rng = np.random.default_rng(11)
    B, T, bs, dd = 3, 50, 8, 5
    lens = np.array([50, 17, 8])
    cont = rng.standard_normal((B, T, dd))
    nb = (lens + bs - 1) // bs
    perm = rng.permutation(int(nb.sum()))
    table = np.full((B, (T + bs - 1) // bs), -1)
    pool = np.full((int(nb.sum()), bs, dd), np.nan)
    off = 0
    for b in range(B):
        table[b, :nb[b]] = perm[off:off + nb[b]]
        off += nb[b]
        for k in range(nb[b]):
            rows = cont[b, k * bs:(k + 1) * bs]
            pool[table[b, k], :len(rows)] = rows
    got = O.gather_pages(pool, table, lens, T)
    for b in range(B):
        assert np.array_equal(got[b, :lens[b]], cont[b, :lens[b]])
        assert np.all(got[b, lens[b]:] == 0)


def test_fp8_round_trip_within_half_ulp():
    cfg = configs.SPEC_FP8.with_(batch=2, seq_len=32, n_heads=2)
    inp = synth.make_inputs(cfg, 0)
    deq = O.dequantize_cache(inp.c_kv, inp.kv_scale)
    x = inp.c_kv_prequant.astype(np.float64)
    s = inp.kv_scale.astype(np.float64)[..., None]
    y = x / s
    # e4m3: 3 mantissa bits -> half ulp is 2^-4 relative for normals (|y| >= 2^-6),
    # and 2^-10 absolute in the subnormal range.
    bound = np.where(np.abs(y) >= 2.0 ** -6, np.abs(y) * 2.0 ** -4, 2.0 ** -10) * s
    assert np.all(np.abs(deq - x) <= bound * (1 + 1e-6))
    # The per-token scale maps the row maximum onto the largest code, 448.
    assert np.allclose(np.max(np.abs(deq), axis=-1), np.max(np.abs(x), axis=-1), rtol=2 ** -4)


def test_poisoned_tails_do_not_reach_the_oracle():
    inp = synth.make_inputs(SMALL, 0, lengths=np.array([20, 7], np.int32), poison_tail=True)
    d = decoded(inp)
    assert np.isnan(d["c_kv"][1, 7:]).all()
    res = O.mla_absorbed(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["w_uk"], d["w_uv"],
                         d["seq_lens"], d["scale"])
    assert np.all(np.isfinite(res["out"]))
