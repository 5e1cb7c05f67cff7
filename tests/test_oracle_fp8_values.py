"""Pins of the oracle's fp8 value product (round_significand, latent_attention_fp8).

* round_significand against torch's own e4m3fn cast (a library routine) over the format's
  normal range, its commuting with powers of two, and hand-worked ties;
* latent_attention_fp8 on a hand-worked case (every weight equal, every token scale 0.7,
  which rounds to 0.6875), against a brute-force loop that rounds each weight through
  torch's e4m3fn cast, and within the rounding bound of latent_attention_fp8_query (the
  same scores with an exact value product), whose lse it shares."""
import math

import numpy as np
import torch

from oracle import mla_oracle as O


def _torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float64)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_round_significand_vs_torch():
    r = np.random.default_rng(11)
    # magnitudes spread over the normal range [2^-6, 448], both signs
    x = np.exp2(r.uniform(-6, np.log2(448), 20000)) * np.where(r.random(20000) < 0.5, -1, 1)
    assert np.array_equal(O.round_significand(x), _torch_e4m3(x))
    for k in (-40, -7, 13):
        assert np.array_equal(O.round_significand(x * 2.0 ** k), O.round_significand(x) * 2.0 ** k)
    # hand-worked: 0.7 = 1.0110011..b * 2^-1 -> 1.011b * 2^-1; ties go to the even mantissa
    assert O.round_significand(0.7) == 0.6875
    assert O.round_significand(1.0625) == 1.0 and O.round_significand(1.1875) == 1.25
    assert O.round_significand(0.0) == 0.0 and O.round_significand(-3.0) == -3.0


def small_case(seed=5, B=2, sq=2, n_h=3, d_c=256, d_r=8, T=11):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 0x7F, size=(B, T, d_c)).astype(np.uint8)  # finite codes, either sign
    codes |= np.where(r.random((B, T, d_c)) < 0.5, 0x80, 0).astype(np.uint8)
    return dict(q_lat=r.standard_normal((B, sq, n_h, d_c)) * 0.02, q_rope=r.standard_normal((B, sq, n_h, d_r)),
                codes=codes, kv_scale=r.uniform(0.005, 0.02, (B, T)), k_rope=r.standard_normal((B, T, d_r)),
                seq_lens=np.array([T, 5]), scale=0.3)


def pin_fp8_values_hand_case():
    """Zero queries: every visible weight is 1; with every token scale 0.7 each weight times
    its scale rounds to 0.6875, so o_lat = 0.6875 * (mean of the visible decoded codes) and
    lse = ln(visible tokens)."""
    c = small_case()
    c["q_lat"][:] = 0.0
    c["q_rope"][:] = 0.0
    c["kv_scale"][:] = 0.7
    o, l = O.latent_attention_fp8(c["q_lat"], c["q_rope"], c["codes"], c["kv_scale"], c["k_rope"],
                                  c["seq_lens"], c["scale"])
    B, sq, n_h, _ = o.shape
    for b in range(B):
        L = int(c["seq_lens"][b])
        for i in range(sq):
            vis = O.visible_keys(L, sq, i)
            mean = O.decode_e4m3fn(c["codes"][b, :vis]).mean(axis=0)
            for h in range(n_h):
                assert np.allclose(o[b, i, h], 0.6875 * mean, rtol=1e-14, atol=1e-14)
                assert abs(l[b, i, h] - math.log(vis)) <= 1e-14


def pin_fp8_values_brute_force():
    """Loops over rows and tokens.  Scores from the rounded query (round_query_slices_e4m3,
    pinned on its own) and the decoded codes; each weight 2^(x_t - K), K the ceiling of the
    row's largest base-2 logit, times the token's scale, is rounded by torch's e4m3fn cast
    after scaling by the power of two that puts it in [128, 256)."""
    c = small_case()
    qr = O.round_query_slices_e4m3(c["q_lat"], 128)
    B, sq, n_h, d_c = qr.shape
    o_ref = np.zeros_like(qr)
    l_ref = np.full((B, sq, n_h), -np.inf)
    for b in range(B):
        L = int(c["seq_lens"][b])
        C = O.decode_e4m3fn(c["codes"][b])
        for i in range(sq):
            vis = max(0, min(L - sq + i + 1, L))
            for h in range(n_h):
                if vis == 0:
                    continue
                xs = [c["scale"] * (float(qr[b, i, h] @ C[t]) * c["kv_scale"][b, t]
                                    + float(c["q_rope"][b, i, h] @ c["k_rope"][b, t])) / math.log(2.0)
                      for t in range(vis)]
                K = math.ceil(max(xs))
                w = [2.0 ** (x - K) for x in xs]
                acc = np.zeros(d_c)
                for t in range(vis):
                    v = w[t] * c["kv_scale"][b, t]
                    e = math.floor(math.log2(v)) - 7
                    acc += float(_torch_e4m3(v * 2.0 ** -e)) * 2.0 ** e * C[t]
                o_ref[b, i, h] = acc / sum(w)
                l_ref[b, i, h] = (K + math.log2(sum(w))) * math.log(2.0)
    o, l = O.latent_attention_fp8(c["q_lat"], c["q_rope"], c["codes"], c["kv_scale"], c["k_rope"],
                                  c["seq_lens"], c["scale"])
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * max(1.0, np.max(np.abs(o_ref)))
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(l[fin] - l_ref[fin])) <= 1e-12


def pin_fp8_values_bound():
    """Against the exact value product on the same scores: each rounded weight is within 2^-4
    of its value, so |o - o_exact| <= 2^-4 sum_t w_t ts_t |code_t| / sum_t w_t per column; the
    lse is the same."""
    c = small_case(seed=9)
    c["q_lat"] *= 30.0  # spread the weights over many binades
    o, l = O.latent_attention_fp8(c["q_lat"], c["q_rope"], c["codes"], c["kv_scale"], c["k_rope"],
                                  c["seq_lens"], c["scale"])
    deq = O.dequantize_cache(c["codes"], c["kv_scale"])
    o_x, l_x = O.latent_attention_fp8_query(c["q_lat"], c["q_rope"], deq, c["k_rope"], c["seq_lens"], c["scale"])
    assert np.array_equal(np.isneginf(l), np.isneginf(l_x))
    fin = np.isfinite(l_x)
    assert np.max(np.abs(l[fin] - l_x[fin])) <= 1e-12
    B, sq, n_h, _ = o.shape
    for b in range(B):
        L = int(c["seq_lens"][b])
        for i in range(sq):
            vis = O.visible_keys(L, sq, i)
            if vis == 0:
                continue
            absv = np.abs(deq[b, :vis])
            for h in range(n_h):
                # exact softmax probabilities of the shared scores
                qr = O.round_query_slices_e4m3(c["q_lat"][b, i, h][None], 128)[0]
                s = c["scale"] * (deq[b, :vis] @ qr + c["k_rope"][b, :vis] @ c["q_rope"][b, i, h])
                p = np.exp(s - s.max())
                p /= p.sum()
                bound = 2.0 ** -4 * (p @ absv) * (1 + 1e-9) + 1e-15
                assert np.all(np.abs(o[b, i, h] - o_x[b, i, h]) <= bound)
    assert np.max(np.abs(o - o_x)) > 0  # the rounding is not a no-op on this case


def test_round_significand_vs_torch():
    pin_round_significand_vs_torch()


def test_fp8_values_hand_case():
    pin_fp8_values_hand_case()


def test_fp8_values_brute_force():
    pin_fp8_values_brute_force()


def test_fp8_values_bound():
    pin_fp8_values_bound()
