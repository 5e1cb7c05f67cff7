"""Pins of the oracle's fp8-query approximation (round_query_slices_e4m3,
latent_attention_fp8_query): exactly representable slices are left unchanged, the rounding
stays within the e4m3 format's half-step, and the attention on the rounded query matches a
brute-force loop that takes its codes from torch's own e4m3fn cast."""
import numpy as np
import torch

from oracle import mla_oracle as O

# Every finite positive normal e4m3fn code below 448 (exponent field 1..15, NaN excluded).
_NORMAL_CODES = np.array([c for c in range(0x08, 0x7E)], np.uint8)


def exact_slices(rows=6, d_c=512, width=128, seed=0):
    """q [rows, d_c] whose 128-column slices are e4m3 values times a power of two per slice,
    each slice holding one +-448 * 2^k element, so each slice's fp8 encoding is exact."""
    r = np.random.default_rng(seed)
    q = np.empty((rows, d_c))
    ks = [0, -8, 5, -3, 2, -6]
    for i in range(rows):
        for j in range(d_c // width):
            k = ks[(i + j) % len(ks)]
            codes = r.choice(_NORMAL_CODES, size=width)
            vals = O.decode_e4m3fn(codes) * np.where(r.random(width) < 0.5, -1.0, 1.0)
            vals[r.integers(width)] = 448.0 * (1 if r.random() < 0.5 else -1)
            q[i, j * width:(j + 1) * width] = vals * 2.0 ** k
    return q


def pin_round_query_exact_slices():
    q = exact_slices()
    got = O.round_query_slices_e4m3(q, 128)
    assert np.array_equal(got, q)


def pin_round_query_bound():
    q = np.random.default_rng(1).standard_normal((5, 512)) * np.exp(np.random.default_rng(2).normal(size=(5, 1)))
    got = O.round_query_slices_e4m3(q, 128)
    qs, gs = q.reshape(5, 4, 128), got.reshape(5, 4, 128)
    scale = np.max(np.abs(qs), axis=-1, keepdims=True) / 448.0
    y = np.abs(qs) / scale
    err = np.abs(gs - qs)
    normal = y >= 2.0 ** -6
    # nearest e4m3 value: half a step of 2^-3 relative in the normal range, half the
    # subnormal step 2^-9 (times the slice scale) below it; the float32 reading of the query
    # and of the scale adds a few 2^-24 relative
    slack = 1 + 2.0 ** -18
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(qs[normal]) * slack)
    assert np.all(err[~normal] <= 2.0 ** -10 * np.broadcast_to(scale, qs.shape)[~normal] * slack)
    # each slice's largest element encodes as +-448 times the slice scale
    idx = np.argmax(np.abs(qs), axis=-1)[..., None]
    assert np.allclose(np.take_along_axis(gs, idx, -1), np.take_along_axis(qs, idx, -1), rtol=2.0 ** -21, atol=0)


def small_case(seed=3, B=2, sq=2, n_h=3, d_c=256, d_r=8, T=9):
    r = np.random.default_rng(seed)
    return dict(q_lat=r.standard_normal((B, sq, n_h, d_c)), q_rope=r.standard_normal((B, sq, n_h, d_r)),
                c_kv=r.standard_normal((B, T, d_c)), k_rope=r.standard_normal((B, T, d_r)),
                seq_lens=np.array([T, 4]), scale=0.11)


def pin_fp8_query_attention_identity():
    """With exactly representable query slices the approximation is the exact attention
    (the RoPE query, left unrounded, is Gaussian)."""
    c = small_case()
    B, sq, n_h, d_c = c["q_lat"].shape
    c["q_lat"] = exact_slices(B * sq * n_h, d_c, 128, seed=4).reshape(B, sq, n_h, d_c)
    o1, l1 = O.latent_attention_fp8_query(c["q_lat"], c["q_rope"], c["c_kv"], c["k_rope"], c["seq_lens"],
                                          c["scale"])
    o2, l2 = O.latent_attention(c["q_lat"], c["q_rope"], c["c_kv"], c["k_rope"], c["seq_lens"], c["scale"])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_fp8_query_brute_force():
    """Loops over rows and tokens; the query codes come from torch's e4m3fn cast (a library
    routine) of the float32 y = q * (448 / max|slice|), the softmax from its definition."""
    c = small_case()
    q, qr, C, R, lens, sc = c["q_lat"], c["q_rope"], c["c_kv"], c["k_rope"], c["seq_lens"], c["scale"]
    B, sq, n_h, d_c = q.shape
    o_ref = np.zeros_like(q)
    l_ref = np.full((B, sq, n_h), -np.inf)
    for b in range(B):
        L = int(lens[b])
        for i in range(sq):
            vis = max(0, min(L - sq + i + 1, L))
            for h in range(n_h):
                qh = np.empty(d_c)
                for j in range(d_c // 128):
                    sl = q[b, i, h, j * 128:(j + 1) * 128].astype(np.float32)
                    amax = np.max(np.abs(sl))
                    y = sl * (np.float32(448) / amax)  # the float32 decision of the definition
                    codes = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn)
                    qh[j * 128:(j + 1) * 128] = codes.to(torch.float64).numpy() * float(amax * np.float32(1 / 448))
                if vis == 0:
                    continue
                logits = [sc * (qh @ C[b, t] + qr[b, i, h] @ R[b, t]) for t in range(vis)]
                m = max(logits)
                e = [np.exp(x - m) for x in logits]
                tot = sum(e)
                o_ref[b, i, h] = sum(e[t] / tot * C[b, t] for t in range(vis))
                l_ref[b, i, h] = m + np.log(tot)
    o, l = O.latent_attention_fp8_query(q, qr, C, R, lens, sc)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 and np.array_equal(np.isneginf(l), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(l[fin] - l_ref[fin])) <= 1e-12


def test_round_query_exact_slices():
    pin_round_query_exact_slices()


def test_round_query_bound():
    pin_round_query_bound()


def test_fp8_query_attention_identity():
    pin_fp8_query_attention_identity()


def test_fp8_query_brute_force():
    pin_fp8_query_brute_force()
