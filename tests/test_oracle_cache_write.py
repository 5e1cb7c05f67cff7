"""Pins of the oracle's cache-write step (new-token latent, rotated RoPE key, fp8 encoding).

Every pin checks the oracle against something other than itself: closed forms of the
rotary embedding worked out by hand, invariants any rotation satisfies, torch's own e4m3
cast, and brute-force loops for the projections.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O

PAIRINGS = ("interleaved", "half")


def pin_rope_hand_example():
    # d_r = 4, base 100: pair 0 turns by p, pair 1 by p * 100^(-1/2) = p / 10.
    x = np.array([[1.0, 0.0, 0.0, 1.0]])
    got_i = O.rope_rotate(x, np.array([1.0]), 100.0, "interleaved")[0]
    # interleaved pairs (x0, x1), (x2, x3)
    want_i = [math.cos(1), math.sin(1), -math.sin(0.1), math.cos(0.1)]
    np.testing.assert_allclose(got_i, want_i, rtol=0, atol=1e-14)
    got_h = O.rope_rotate(x, np.array([1.0]), 100.0, "half")[0]
    # half pairs (x0, x2), (x1, x3)
    want_h = [math.cos(1), -math.sin(0.1), math.sin(1), math.cos(0.1)]
    np.testing.assert_allclose(got_h, want_h, rtol=0, atol=1e-14)


def pin_rope_invariants():
    rng = np.random.default_rng(3)
    for pairing in PAIRINGS:
        q = rng.normal(size=(5, 64))
        k = rng.normal(size=(5, 64))
        m = rng.integers(0, 5000, size=5).astype(np.float64)
        n = rng.integers(0, 5000, size=5).astype(np.float64)
        # position 0 is the identity
        np.testing.assert_allclose(O.rope_rotate(q, np.zeros(5), 10000.0, pairing), q, rtol=0, atol=0)
        # each pair keeps its length
        r = O.rope_rotate(q, m, 10000.0, pairing)
        if pairing == "interleaved":
            na, nb = q[:, 0::2] ** 2 + q[:, 1::2] ** 2, r[:, 0::2] ** 2 + r[:, 1::2] ** 2
        else:
            na, nb = q[:, :32] ** 2 + q[:, 32:] ** 2, r[:, :32] ** 2 + r[:, 32:] ** 2
        np.testing.assert_allclose(nb, na, rtol=1e-12)
        # rotations compose
        np.testing.assert_allclose(O.rope_rotate(O.rope_rotate(q, m, 10000.0, pairing), n, 10000.0, pairing),
                                   O.rope_rotate(q, m + n, 10000.0, pairing), rtol=0, atol=1e-9)
        # the dot product of two rotated vectors depends on the position difference only
        lhs = np.sum(O.rope_rotate(q, m, 10000.0, pairing) * O.rope_rotate(k, n, 10000.0, pairing), axis=-1)
        rhs = np.sum(O.rope_rotate(q, m - n, 10000.0, pairing) * k, axis=-1)
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-9)


def pin_quantize_vs_torch():
    rng = np.random.default_rng(4)
    c = rng.normal(size=(64, 512)) * rng.uniform(0.01, 100.0, size=(64, 1))
    c[5] = 0.0
    codes, scale = O.quantize_e4m3fn_rows(c)
    assert scale[5] == 1.0 and np.all(codes[5] == 0)
    y = torch.from_numpy(c / scale[:, None]).to(torch.float32)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    amax = np.abs(c).max(axis=1)
    assert np.array_equal(scale, np.where(amax > 0, amax / 448.0, 1.0))


def pin_quantize_special():
    # amax -> +-448 (codes 0x7E, 0xFE); exact ties between neighbours go to the even code:
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39); 1.1875 between 1.125 and 1.25 (0x3A).
    codes, scale = O.quantize_e4m3fn_rows(np.array([[448.0, 1.0625, 1.1875, -448.0, 0.0, -1e-9]]))
    assert scale[0] == 1.0
    # ... and a negative value too small for the format becomes -0 (0x80)
    assert codes[0].tolist() == [0x7E, 0x38, 0x3A, 0xFE, 0x00, 0x80]


def pin_cache_append_brute():
    rng = np.random.default_rng(5)
    B, sq, dm, dc, dr = 2, 3, 8, 4, 4
    x = rng.normal(size=(B, sq, dm))
    w_dkv = rng.normal(size=(dm, dc))
    w_kr = rng.normal(size=(dm, dr))
    seq_lens = np.array([3, 10])
    c, k, pos = O.cache_append_rows(x, w_dkv, w_kr, seq_lens, sq, 10000.0, "interleaved")
    for b in range(B):
        for i in range(sq):
            assert pos[b, i] == seq_lens[b] - sq + i
            for j in range(dc):
                assert abs(c[b, i, j] - sum(x[b, i, t] * w_dkv[t, j] for t in range(dm))) < 1e-12
            kraw = [sum(x[b, i, t] * w_kr[t, j] for t in range(dm)) for j in range(dr)]
            want = O.rope_rotate(np.array([kraw]), np.array([float(pos[b, i])]), 10000.0, "interleaved")[0]
            np.testing.assert_allclose(k[b, i], want, rtol=0, atol=1e-12)


def test_rope_hand_example():
    pin_rope_hand_example()


def test_rope_invariants():
    pin_rope_invariants()


def test_quantize_matches_torch_e4m3_cast():
    pin_quantize_vs_torch()


def test_quantize_special_values_and_ties():
    pin_quantize_special()


def test_cache_append_rows_brute_force():
    pin_cache_append_brute()
