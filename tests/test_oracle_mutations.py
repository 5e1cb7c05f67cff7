"""Plant one plausible mistake at a time in the oracle and check a pin catches it.

The mistakes are planted in the oracle module (on the CPU, through monkeypatch) and
never touch the GPU path.  Each case names the pin expected to fail.
"""
import numpy as np
import pytest

from oracle import mla_oracle as O
import test_oracle as P
import test_oracle_cache_write as PC
import test_oracle_query as PQ
import test_oracle_fp8_query as PF
import test_oracle_fp8_values as PV

_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _latent_attention_no_rope(q_lat, q_rope, c_kv, k_rope, seq_lens, scale):
    return _orig["latent_attention"](q_lat, 0 * q_rope, c_kv, k_rope, seq_lens, scale)


def _explicit_no_rope(q_nope, q_rope, *a, **k):
    return _orig["mla_explicit"](q_nope, 0 * q_rope, *a, **k)


def _softmax_wrong_sign(s, n_vis):
    return _orig["_softmax_rows"](-s, n_vis)


def _visible_off_by_one(seq_len, q_len, i):
    return int(min(max(seq_len - q_len + i, 0), seq_len))


def _absorb_query_wrong_head(q_nope, w_uk):
    return _orig["absorb_query"](q_nope, np.roll(w_uk, 1, axis=0))


def _absorb_output_wrong_head(o_lat, w_uv):
    return _orig["absorb_output"](o_lat, np.roll(w_uv, 1, axis=0))


def _page_layout_transposed(w_uk, w_uv):
    n_h, d_h, d_c = w_uk.shape
    uk = np.transpose(w_uk, (2, 1, 0)).reshape(d_c, n_h * d_h)
    uv = np.transpose(w_uv, (1, 2, 0)).reshape(d_c, n_h * d_h)
    return uk, uv


def _merge_inverted_weights(o_parts, lse_parts):
    return _orig["merge_partials"](o_parts, -np.asarray(lse_parts))


def _e4m3_wrong_bias(codes):
    return _orig["decode_e4m3fn"](codes) * 2.0


def _bf16_low_half(bits):
    return np.asarray(bits, np.uint16).astype(np.float64)


def _latent_attention_scale_on_latent_only(q_lat, q_rope, c_kv, k_rope, seq_lens, scale):
    return _orig["latent_attention"](q_lat, q_rope / scale, c_kv, k_rope, seq_lens, scale)


def _mha_count_wrong(n_heads, d_head):
    return n_heads * d_head


def _rope_sin_sign(x, positions, base, pairing):
    return _orig["rope_rotate"](x, -np.asarray(positions, np.float64), base, pairing)


def _rope_wrong_frequency(x, positions, base, pairing):
    return _orig["rope_rotate"](x, positions, np.sqrt(base), pairing)


def _rope_swapped_pairing(x, positions, base, pairing):
    return _orig["rope_rotate"](x, positions, base, "half" if pairing == "interleaved" else "interleaved")


def _positions_off_by_one(seq_lens, q_len):
    return _orig["new_token_positions"](seq_lens, q_len) + 1


def _quantize_half_scale(c):
    # the stored scale is amax / 224: dequantised values come out twice too large
    codes, scale = _orig["quantize_e4m3fn_rows"](c)
    return codes, scale * 2.0


def _quantize_ties_up(c):
    codes, scale = _orig["quantize_e4m3fn_rows"](np.nextafter(np.asarray(c, np.float64), np.inf))
    return codes, scale


def _fold_query_head_swapped(w_uq, w_uk):
    return np.einsum("khj,hjc->khc", np.asarray(w_uq, np.float64), np.asarray(w_uk, np.float64)[::-1])


def _query_rope_from_content_matrix(x, w_dq, w_uq, w_qr):
    c_q = np.asarray(x, np.float64) @ np.asarray(w_dq, np.float64)
    return np.einsum("mk,khj->mhj", c_q, w_uq), np.einsum("mk,khj->mhj", c_q, w_uq)[..., :w_qr.shape[2]]


def _output_transposed_heads(out_heads, w_o):
    o = np.asarray(out_heads, np.float64)
    return o.transpose(0, 2, 1).reshape(o.shape[0], -1) @ np.asarray(w_o, np.float64)


def _fold_output_wrong_slice(w_uv, w_o):
    w_uv = np.asarray(w_uv, np.float64)
    n_h, d_c, d_h = w_uv.shape
    w_o = np.asarray(w_o, np.float64).reshape(d_h, n_h, -1).transpose(1, 0, 2)
    return np.einsum("hcj,hjd->hcd", w_uv, w_o)


def _round_query_one_scale_per_row(q_lat, slice_width=128):
    return _orig["round_query_slices_e4m3"](q_lat, np.asarray(q_lat).shape[-1])


def _fp8_query_unrounded(q_lat, q_rope, c_kv, k_rope, seq_lens, scale, slice_width=128):
    return _orig["latent_attention"](q_lat, q_rope, c_kv, k_rope, seq_lens, scale)


def _fp8_query_rounds_rope_too(q_lat, q_rope, c_kv, k_rope, seq_lens, scale, slice_width=128):
    q_rope = np.asarray(q_rope, np.float64)
    pad = (-q_rope.shape[-1]) % slice_width
    r = _orig["round_query_slices_e4m3"](np.concatenate([q_rope, np.zeros(q_rope.shape[:-1] + (pad,))], -1),
                                         slice_width)[..., :q_rope.shape[-1]]
    return _orig["latent_attention_fp8_query"](q_lat, r, c_kv, k_rope, seq_lens, scale, slice_width)


def _round_significand_truncates(x, bits=4):
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.trunc(m * 2.0 ** bits), e - bits)


def _fp8_values_with(**change):
    """latent_attention_fp8 with one step changed (its own code, re-written per mutation)."""
    def f(q_lat, q_rope, codes, kv_scale, k_rope, seq_lens, scale, slice_width=128):
        q = O.round_query_slices_e4m3(q_lat, slice_width)
        B, sq, n_h, d_c = q.shape
        o_lat = np.zeros((B, sq, n_h, d_c))
        lse = np.full((B, sq, n_h), -np.inf)
        for b in range(B):
            L = int(seq_lens[b])
            C = O.decode_e4m3fn(np.asarray(codes)[b, :L])
            ts = np.asarray(kv_scale, np.float64)[b, :L]
            s = scale * ((q[b] @ C.T) * ts + np.asarray(q_rope)[b] @ np.asarray(k_rope)[b, :L].T)
            x = (s * np.log2(np.e)).reshape(sq * n_h, L)
            n_vis = np.repeat([O.visible_keys(L, sq, i) for i in range(sq)], n_h)
            vis = np.arange(L)[None, :] < n_vis[:, None]
            x = np.where(vis, x, -np.inf)
            top = np.max(x, axis=1, initial=-np.inf)
            k = np.where(np.isfinite(top), top if change.get("real_reference") else np.ceil(top), 0.0)
            w = np.where(vis, np.exp2(x - k[:, None]), 0.0)
            if change.get("round_before_scale"):
                pw = O.round_significand(w) * ts[None, :]
            else:
                pw = O.round_significand(w * ts[None, :])
            tot = (pw / ts[None, :]).sum(axis=1) if change.get("rounded_normaliser") else w.sum(axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                o = np.where(tot[:, None] > 0, (pw @ C) / tot[:, None], 0.0)
                l = np.where(tot > 0, (k + np.log2(tot)) * np.log(2.0), -np.inf)
            o_lat[b] = o.reshape(sq, n_h, d_c)
            lse[b] = l.reshape(sq, n_h)
        return o_lat, lse
    return f


def _fp8_values_unrounded(q_lat, q_rope, codes, kv_scale, k_rope, seq_lens, scale, slice_width=128):
    return _orig["latent_attention_fp8_query"](q_lat, q_rope, O.dequantize_cache(codes, kv_scale), k_rope,
                                               seq_lens, scale, slice_width)


CASES = [
    ("latent_attention", _latent_attention_no_rope, lambda: P.pin_absorbed_vs_explicit(P.small_inputs())),
    ("latent_attention", _latent_attention_scale_on_latent_only,
     lambda: P.pin_absorbed_vs_explicit(P.small_inputs())),
    ("mla_explicit", _explicit_no_rope, lambda: P.pin_explicit_vs_sdpa(P.small_inputs())),
    ("_softmax_rows", _softmax_wrong_sign, lambda: P.pin_explicit_vs_sdpa(P.small_inputs())),
    ("_softmax_rows", _softmax_wrong_sign, P.pin_softmax_rows),
    ("visible_keys", _visible_off_by_one, lambda: P.pin_explicit_vs_sdpa(P.small_inputs())),
    ("absorb_query", _absorb_query_wrong_head, lambda: P.pin_absorbed_vs_explicit(P.small_inputs())),
    ("absorb_output", _absorb_output_wrong_head, lambda: P.pin_absorbed_vs_explicit(P.small_inputs())),
    ("to_page_layout", _page_layout_transposed, lambda: P.pin_explicit_vs_sdpa(P.small_inputs())),
    ("merge_partials", _merge_inverted_weights, lambda: P.pin_split_merge(P.small_inputs(), 3)),
    ("decode_e4m3fn", _e4m3_wrong_bias, P.pin_e4m3_table),
    ("decode_bf16", _bf16_low_half, P.pin_bf16_decode),
    ("mha_cache_numbers_per_token", _mha_count_wrong, P.pin_cache_arithmetic),
    ("rope_rotate", _rope_sin_sign, PC.pin_rope_hand_example),
    ("rope_rotate", _rope_wrong_frequency, PC.pin_rope_hand_example),
    ("rope_rotate", _rope_swapped_pairing, PC.pin_rope_hand_example),
    ("new_token_positions", _positions_off_by_one, PC.pin_cache_append_brute),
    ("quantize_e4m3fn_rows", _quantize_half_scale, PC.pin_quantize_special),
    ("quantize_e4m3fn_rows", _quantize_ties_up, PC.pin_quantize_special),
    ("fold_query_weights", _fold_query_head_swapped, PQ.pin_fold_query_selection),
    ("query_from_hidden", _query_rope_from_content_matrix, PQ.pin_query_brute_force),
    ("output_projection", _output_transposed_heads, PQ.pin_output_identity_and_brute_force),
    ("fold_output_weights", _fold_output_wrong_slice, PQ.pin_fold_output_brute_force),
    ("round_query_slices_e4m3", _round_query_one_scale_per_row, PF.pin_round_query_exact_slices),
    ("latent_attention_fp8_query", _fp8_query_unrounded, PF.pin_fp8_query_brute_force),
    ("latent_attention_fp8_query", _fp8_query_rounds_rope_too, PF.pin_fp8_query_attention_identity),
    ("round_significand", _round_significand_truncates, PV.pin_round_significand_vs_torch),
    ("latent_attention_fp8", _fp8_values_with(real_reference=True), PV.pin_fp8_values_brute_force),
    ("latent_attention_fp8", _fp8_values_with(round_before_scale=True), PV.pin_fp8_values_brute_force),
    ("latent_attention_fp8", _fp8_values_with(rounded_normaliser=True), PV.pin_fp8_values_brute_force),
    ("latent_attention_fp8", _fp8_values_unrounded, PV.pin_fp8_values_bound),
    ("latent_attention_fp8", _fp8_values_unrounded, PV.pin_fp8_values_hand_case),
]


@pytest.mark.parametrize("name,mutant,pin", CASES, ids=[f"{c[0]}-{c[1].__name__}" for c in CASES])
def test_pin_catches_planted_mistake(monkeypatch, name, mutant, pin):
    pin()  # the unmutated oracle passes the pin
    monkeypatch.setattr(O, name, mutant)
    with pytest.raises((AssertionError, ValueError)):
        pin()
