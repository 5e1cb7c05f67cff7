"""CPU oracle for weight-absorbed Multi-head Latent Attention (MLA) decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module: only
the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
no code with the HIP library (no kernels, headers, helpers or tables); it reads the
same stored input bytes and decodes them itself.

Everything is float64 numpy.  Each function follows one passage of the source pages,
named by page title and section:

* "Operator Notes (1): MLA — Multi-head Latent Attention at the Operator Level"
  (section 2, the operator pseudocode and shapes; sections 1 and 3, cache sizes);
* "multi-head latent attention" glossary entry (the paragraph on the decoupled RoPE
  key, which also states that the up-projections can be absorbed into the query
  and output projections);
* "Multi-Head Latent Attention and the compression of the KV cache" dispatch (the
  paragraph on mathematical equivalence through associativity);
* the same Operator Notes page, section 4 (query compression).

Readings of points the pages leave open (stated once here, used throughout):

* Softmax scale: the caller passes it; the workloads use 1/sqrt(d_h + d_r), the width
  of the concatenated [content | RoPE] key, for the whole dot product.
* Weight layout: ``w_uk[h, j, c]`` and ``w_uv[h, c, j]`` hold the page's
  ``W_UK[c, h*d_h + j]`` and ``W_UV[c, h*d_h + j]`` (a pure permutation;
  ``to_page_layout`` converts).
* The RoPE key ``k_rope[t, :]`` is one d_r-wide vector per token shared by all heads;
  ``q_rope`` is per head.  Both arrive already rotated.
* ``seq_lens[b]`` counts cache rows including the s_q new tokens; query i of a
  sequence of length L sees rows t <= L - s_q + i (causal among the new tokens).
* A query row that sees no key returns zeros and lse = -inf.

Parity pins for every function live in tests/test_oracle*.py.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------------
# Stored-number decoding (from the formats' definitions, not from any library)
# ---------------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper 16 bits of an IEEE-754 binary32; decoding is exact."""
    b32 = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16))
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns stay NaN
        return b32.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": finite, no infinities).

    Bit layout S EEEE MMM, exponent bias 7.  Exponent field 0 encodes subnormals
    (M/8) * 2^-6; other fields encode (1 + M/8) * 2^(E-7).  The two codes with
    E = 15 and M = 7 are NaN; every other code is finite (largest 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * np.exp2(-6.0)
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, val)


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "fp8":
        return decode_e4m3fn(arr)
    raise ValueError(dtype)


def dequantize_cache(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp8 latent with one float32 scale per token: value = e4m3(code) * scale[token]."""
    return decode_e4m3fn(codes) * np.asarray(scale, np.float64)[..., None]


# ---------------------------------------------------------------------------------
# Cache arithmetic ("Operator Notes (1): MLA", sections 1 and 3)
# ---------------------------------------------------------------------------------


def mha_cache_numbers_per_token(n_heads: int, d_head: int) -> int:
    """Full K and V for every head are cached: two n_h*d_h-wide vectors per token."""
    return 2 * n_heads * d_head


def mla_cache_numbers_per_token(d_latent: int, d_rope: int = 0) -> int:
    """Only the latent (plus, with decoupled RoPE, the shared rotary key) is cached."""
    return d_latent + d_rope


# ---------------------------------------------------------------------------------
# Weight layouts
# ---------------------------------------------------------------------------------


def to_page_layout(w_uk: np.ndarray, w_uv: np.ndarray):
    """Per-head stored weights -> the page's [d_c, n_h*d_h] matrices.

    ``W_UK_page[c, h*d_h + j] = w_uk[h, j, c]`` and ``W_UV_page[c, h*d_h + j] = w_uv[h, c, j]``
    ("Operator Notes (1): MLA", section 2: both up-projections map the d_c-wide latent
    to all heads' keys / values at once).
    """
    n_h, d_h, d_c = w_uk.shape
    uk = np.transpose(w_uk, (2, 0, 1)).reshape(d_c, n_h * d_h)
    uv = np.transpose(w_uv, (1, 0, 2)).reshape(d_c, n_h * d_h)
    return uk, uv


# ---------------------------------------------------------------------------------
# Masking (causal among the s_q new tokens)
# ---------------------------------------------------------------------------------


def visible_keys(seq_len: int, q_len: int, i: int) -> int:
    """Number of cache rows query i sees: rows 0 .. L - s_q + i (clamped to [0, L])."""
    return int(min(max(seq_len - q_len + i + 1, 0), seq_len))


def _softmax_rows(s: np.ndarray, n_vis: np.ndarray):
    """Row softmax of scores s[r, t] over the first n_vis[r] columns.

    Returns (p, lse): p is zero outside the visible prefix, lse = log sum_t exp(s).
    A row with nothing visible gets p = 0 and lse = -inf.
    """
    R, L = s.shape
    vis = np.arange(L)[None, :] < n_vis[:, None]
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    denom = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(denom[:, None] > 0, e / denom[:, None], 0.0)
        lse = np.where(denom > 0, m_safe + np.log(denom), -np.inf)
    return p, lse


# ---------------------------------------------------------------------------------
# Explicit form: decompress K and V from the latent, then attend.
# ("Operator Notes (1): MLA", section 2; plus the decoupled RoPE key of the glossary
# entry's paragraph on rotary position.)  This is the authority.
# ---------------------------------------------------------------------------------


def mla_explicit(q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, seq_lens, scale, rows=None):
    """Decompress-then-attend MLA decode.

    q_nope [B,s_q,n_h,d_h], q_rope [B,s_q,n_h,d_r], c_kv [B,T,d_c], k_rope [B,T,d_r],
    w_uk [n_h,d_h,d_c], w_uv [n_h,d_c,d_h] (float64).  ``rows`` optionally restricts
    the work to a list of (b, i, h) triples.

    Per head h: K_h = c_kv W_UK (the head's d_h columns), V_h = c_kv W_UV (likewise);
    the score of token t is scale * (q_nope . K_h[t] + q_rope . k_rope[t]); softmax over
    the visible tokens; the output is the probability-weighted sum of V_h rows.
    Returns out[B,s_q,n_h,d_h] (NaN where not computed) and lse[B,s_q,n_h].
    """
    B, sq, n_h, d_h = q_nope.shape
    uk_page, uv_page = to_page_layout(w_uk, w_uv)
    out = np.full((B, sq, n_h, d_h), np.nan)
    lse = np.full((B, sq, n_h), np.nan)
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(sq) for h in range(n_h)]
    by_bh = {}
    for (b, i, h) in rows:
        by_bh.setdefault((b, h), []).append(i)
    for (b, h), qs in sorted(by_bh.items()):
        L = int(seq_lens[b])
        cols = slice(h * d_h, (h + 1) * d_h)
        K = c_kv[b, :L] @ uk_page[:, cols]              # [L, d_h]
        V = c_kv[b, :L] @ uv_page[:, cols]              # [L, d_h]
        for i in qs:
            s = scale * (K @ q_nope[b, i, h] + k_rope[b, :L] @ q_rope[b, i, h])
            p, l = _softmax_rows(s[None, :], np.array([visible_keys(L, sq, i)]))
            out[b, i, h] = p[0] @ V
            lse[b, i, h] = l[0]
    return out, lse


# ---------------------------------------------------------------------------------
# Absorbed form (glossary entry, paragraph on the decoupled RoPE key: W_UK folds into
# the query side and W_UV into the output side; the dispatch's associativity paragraph
# states that this gives the same result).  Three stages, one per library call.
# ---------------------------------------------------------------------------------


def absorb_query(q_nope, w_uk):
    """q_lat[b,i,h,c] = sum_j q_nope[b,i,h,j] * w_uk[h,j,c]: the query expressed against
    the latent, so that q_nope . (c_kv W_UK_h)[t] = q_lat . c_kv[t]."""
    B, sq, n_h, _ = q_nope.shape
    q_lat = np.empty((B, sq, n_h, w_uk.shape[2]))
    for h in range(n_h):
        q_lat[:, :, h, :] = q_nope[:, :, h, :] @ w_uk[h]
    return q_lat


def latent_attention(q_lat, q_rope, c_kv, k_rope, seq_lens, scale):
    """Attention of every head directly over the cached latent.

    score[t] = scale * (q_lat . c_kv[t] + q_rope . k_rope[t]); softmax over visible t;
    o_lat = sum_t p[t] * c_kv[t] (the latent is both key and value).
    Returns o_lat [B,s_q,n_h,d_c] and lse [B,s_q,n_h] (natural log).
    """
    B, sq, n_h, d_c = q_lat.shape
    o_lat = np.zeros((B, sq, n_h, d_c))
    lse = np.full((B, sq, n_h), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        C = c_kv[b, :L]
        R = k_rope[b, :L]
        s = scale * (q_lat[b] @ C.T + q_rope[b] @ R.T)          # [s_q, n_h, L]
        n_vis = np.repeat([visible_keys(L, sq, i) for i in range(sq)], n_h)
        p, l = _softmax_rows(s.reshape(sq * n_h, L), n_vis)
        o_lat[b] = (p @ C).reshape(sq, n_h, d_c)
        lse[b] = l.reshape(sq, n_h)
    return o_lat, lse


def absorb_output(o_lat, w_uv):
    """out[b,i,h,j] = sum_c o_lat[b,i,h,c] * w_uv[h,c,j]: the per-head value projection
    applied once to the attended latent instead of to every cached token."""
    B, sq, n_h, _ = o_lat.shape
    out = np.empty((B, sq, n_h, w_uv.shape[2]))
    for h in range(n_h):
        out[:, :, h, :] = o_lat[:, :, h, :] @ w_uv[h]
    return out


def mla_absorbed(q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, seq_lens, scale):
    """The whole absorbed decode. Returns dict(out, o_lat, lse, q_lat)."""
    q_lat = absorb_query(q_nope, w_uk)
    o_lat, lse = latent_attention(q_lat, q_rope, c_kv, k_rope, seq_lens, scale)
    return {"q_lat": q_lat, "o_lat": o_lat, "lse": lse, "out": absorb_output(o_lat, w_uv)}


# ---------------------------------------------------------------------------------
# Splitting the token axis and merging (log-sum-exp combine)
# ---------------------------------------------------------------------------------


def merge_partials(o_parts, lse_parts):
    """Merge attention results computed over disjoint token subsets.

    o_parts [S, ..., d] are each subset's normalised outputs, lse_parts [S, ...] their
    log-sum-exp.  Since exp(lse_s) is each subset's softmax denominator, the full output
    is the exp(lse_s)-weighted mean of the o_s, and the full lse is log sum_s exp(lse_s).
    Subsets with lse = -inf (nothing visible) carry zero weight.
    """
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    M = np.max(lse_parts, axis=0)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - M_safe), 0.0)
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(tot[..., None] > 0, np.einsum("s...,s...d->...d", w, o_parts) / tot[..., None], 0.0)
        lse = np.where(tot > 0, M_safe + np.log(tot), -np.inf)
    return o, lse


# ---------------------------------------------------------------------------------
# Paged cache: block-table lookup
# ---------------------------------------------------------------------------------


def gather_pages(pool, block_table, seq_lens, seq_len_max, fill=0.0):
    """Rebuild contiguous per-sequence rows from a block pool.

    Logical row t of sequence b lives in pool block ``block_table[b, t // bs]`` at offset
    ``t % bs``.  Rows at or past seq_lens[b] are set to ``fill``.
    pool [N_blk, bs, ...] -> [B, seq_len_max, ...].
    """
    bs = pool.shape[1]
    B = block_table.shape[0]
    out = np.full((B, seq_len_max) + pool.shape[2:], fill, dtype=pool.dtype)
    for b in range(B):
        for t in range(int(seq_lens[b])):
            out[b, t] = pool[block_table[b, t // bs], t % bs]
    return out


# ---------------------------------------------------------------------------------
# Cache write of the new tokens ("Operator Notes (1): MLA", section 2: the latent is the
# only KV state cached; "multi-head latent attention" glossary entry, paragraph on the
# decoupled RoPE key: a small separate rotated key is cached next to the latent)
# ---------------------------------------------------------------------------------
#
# Readings (the pages name these steps but print no formula):
# * the decoupled key is projected from the same hidden state by its own matrix W_KR
#   [d_model, d_r] and rotated by its position;
# * the rotation is the standard rotary position embedding: dims are paired, pair j is
#   rotated by the angle  position * base^(-2j / d_r);  the pairing is a parameter,
#   "interleaved" (2j, 2j + 1) or "half" (j, j + d_r / 2);
# * new token i of a sequence whose length (counting the new tokens) is L sits at position
#   L - s_q + i, the same convention the decode's causal mask uses;
# * an fp8 cache stores per token scale = max|c| / 448 (1 for an all-zero row) and the
#   e4m3 code nearest to c / scale (ties to the even code).


def rope_rotate(x, positions, base: float, pairing: str):
    """Rotary position embedding of the last axis of x (even width d_r).

    positions broadcasts against x.shape[:-1].  Pair j = (x_a, x_b) becomes
    (x_a cos t - x_b sin t, x_a sin t + x_b cos t) with t = position * base^(-2j / d_r).
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = np.asarray(base, np.float64) ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(positions, np.float64)[..., None] * inv
    cos, sin = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    if pairing == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * cos - b * sin
        out[..., 1::2] = a * sin + b * cos
    elif pairing == "half":
        a, b = x[..., :half], x[..., half:]
        out[..., :half] = a * cos - b * sin
        out[..., half:] = a * sin + b * cos
    else:
        raise ValueError(pairing)
    return out


def new_token_positions(seq_lens, q_len: int):
    """Position of new token i of sequence b: seq_lens[b] - q_len + i."""
    return np.asarray(seq_lens, np.int64)[:, None] - q_len + np.arange(q_len)[None, :]


def cache_append_rows(x, w_dkv, w_kr, seq_lens, q_len: int, base: float, pairing: str):
    """Latent and rotated RoPE key of every new token.

    x [B, s_q, d_model], w_dkv [d_model, d_c], w_kr [d_model, d_r] ->
    (c [B, s_q, d_c], k_rope [B, s_q, d_r], positions [B, s_q]).
    """
    x = np.asarray(x, np.float64)
    c = x @ np.asarray(w_dkv, np.float64)
    k = x @ np.asarray(w_kr, np.float64)
    pos = new_token_positions(seq_lens, q_len)
    return c, rope_rotate(k, pos, base, pairing), pos


_E4M3_MAGNITUDES = None


def _nearest_e4m3fn_codes(y):
    """e4m3fn code of sign(y) and of the finite magnitude nearest to |y| (|y| <= 448; ties
    to the magnitude whose code has an even mantissa), as a sign-magnitude format rounds."""
    global _E4M3_MAGNITUDES
    if _E4M3_MAGNITUDES is None:
        codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: +0 .. 448 (0x7F is NaN)
        _E4M3_MAGNITUDES = (codes, decode_e4m3fn(codes))
    cand_codes, cand_vals = _E4M3_MAGNITUDES
    y = np.asarray(y, np.float64)
    d = np.abs(np.abs(y)[..., None] - cand_vals)              # [..., n, 127]
    best = d.min(axis=-1, keepdims=True)
    # among the nearest magnitudes prefer an even mantissa (code bit 0 clear)
    pref = np.where(d <= best, (cand_codes & 1).astype(np.int64), 2)
    mag = cand_codes[np.argmin(pref * 1e9 + d, axis=-1)]
    sign = np.where(np.signbit(y), 0x80, 0x00).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def quantize_e4m3fn_rows(c):
    """Per-row fp8 encoding: scale = max|row| / 448 (1 if the row is zero) and, for every
    element y = c / scale, the nearest e4m3fn code (_nearest_e4m3fn_codes).
    Returns (codes uint8, scale float64)."""
    c = np.asarray(c, np.float64)
    amax = np.max(np.abs(c), axis=-1)
    scale = np.where(amax > 0, amax / 448.0, 1.0)
    return _nearest_e4m3fn_codes(c / scale[..., None]), scale


def round_query_slices_e4m3(q_lat, slice_width: int = 128):
    """The query as an fp8 score product sees it: every row of q_lat cut into slices of
    ``slice_width`` columns, each slice replaced by its fp8 encoding decoded back.  The
    encoding is the per-slice one of quantize_e4m3fn_rows (scale max|slice| / 448, nearest
    e4m3fn code), with its decisions taken in float32, the precision of the kernel that
    makes them (which code a value gets is an integer decided by floating point): the
    query is read as float32, y = q * (448 / max|slice|) with the quotient and the product
    rounded to float32 and clamped to +-448, and the slice scale is max|slice| * (1 / 448)
    in float32."""
    q = np.asarray(q_lat, np.float64)
    *lead, d_c = q.shape
    if d_c % slice_width:
        raise ValueError("d_c must be a multiple of the slice width")
    q32 = q.reshape(*lead, d_c // slice_width, slice_width).astype(np.float32)
    amax = np.max(np.abs(q32), axis=-1, keepdims=True)
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1))
    inv = np.where(pos, np.float32(448) / safe, np.float32(1)).astype(np.float32)
    y = np.clip(q32 * inv, np.float32(-448), np.float32(448)).astype(np.float32)
    scale = np.where(pos, amax * np.float32(1.0 / 448.0), np.float32(1)).astype(np.float32)
    return (decode_e4m3fn(_nearest_e4m3fn_codes(y)) * scale.astype(np.float64)).reshape(q.shape)


def latent_attention_fp8_query(q_lat, q_rope, c_kv, k_rope, seq_lens, scale, slice_width: int = 128):
    """An approximation of latent_attention that lets the latent part of the score run as an
    fp8 matrix product against a quantized (fp8) cache, the quantized-cache direction of
    "Multi-Head Latent Attention (MLA) Explained", section "Which Models Use MLA and What Is
    Next": the latent score term uses the rounded query of round_query_slices_e4m3; the RoPE
    term and the product with the latent (the value) are exact.  Returns (o_lat, lse)."""
    return latent_attention(round_query_slices_e4m3(q_lat, slice_width), q_rope, c_kv, k_rope, seq_lens,
                            scale)


def round_significand(x, bits: int = 4):
    """x rounded to ``bits`` significant binary digits, ties to the even one.  With bits = 4
    this is the precision of an e4m3 number in its normal range (an implicit leading one and
    three stored mantissa bits), without the format's bounds on the exponent."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)  # x = m * 2^e with 0.5 <= |m| < 1 (m = 0 for x = 0)
    return np.ldexp(np.round(m * 2.0 ** bits), e - bits)


def latent_attention_fp8(q_lat, q_rope, codes, kv_scale, k_rope, seq_lens, scale, slice_width: int = 128):
    """Both products of the absorbed decode on fp8 operands (the quantized-cache direction
    of "Multi-Head Latent Attention (MLA) Explained", section "Which Models Use MLA and What
    Is Next").  The score is latent_attention_fp8_query's: the latent query rounded slice by
    slice (round_query_slices_e4m3), times the stored codes (decode_e4m3fn) and the token's
    scale, plus the exact RoPE term.  The softmax weights are exact; the value product runs on
    the stored codes, with each weight times its token's scale rounded to e4m3 precision
    (round_significand).  The normaliser sums the unrounded weights.

    Reading: the weight of token t is taken as 2^(x_t - k), with x_t the base-2 logit
    (scale * log2(e) * score) and k an integer (here the ceiling of the row's largest logit);
    since rounding to a number of significant bits commutes with multiplying by a power of
    two, the rounded products do not depend on which integer it is.

    codes [B, T, d_c] uint8 e4m3fn, kv_scale [B, T]; the rest as latent_attention.
    Returns (o_lat, lse), lse in natural-log units."""
    q = round_query_slices_e4m3(q_lat, slice_width)
    q_rope = np.asarray(q_rope, np.float64)
    k_rope = np.asarray(k_rope, np.float64)
    B, sq, n_h, d_c = q.shape
    o_lat = np.zeros((B, sq, n_h, d_c))
    lse = np.full((B, sq, n_h), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        C = decode_e4m3fn(np.asarray(codes)[b, :L])
        ts = np.asarray(kv_scale, np.float64)[b, :L]
        s = scale * ((q[b] @ C.T) * ts + q_rope[b] @ k_rope[b, :L].T)     # [s_q, n_h, L]
        x = (s * np.log2(np.e)).reshape(sq * n_h, L)
        n_vis = np.repeat([visible_keys(L, sq, i) for i in range(sq)], n_h)
        vis = np.arange(L)[None, :] < n_vis[:, None]
        x = np.where(vis, x, -np.inf)
        top = np.max(x, axis=1, initial=-np.inf)
        k = np.where(np.isfinite(top), np.ceil(top), 0.0)
        w = np.where(vis, np.exp2(x - k[:, None]), 0.0)
        tot = w.sum(axis=1)
        pw = round_significand(w * ts[None, :])
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(tot[:, None] > 0, (pw @ C) / tot[:, None], 0.0)
            l = np.where(tot > 0, (k + np.log2(tot)) * np.log(2.0), -np.inf)
        o_lat[b] = o.reshape(sq, n_h, d_c)
        lse[b] = l.reshape(sq, n_h)
    return o_lat, lse


# ---------------------------------------------------------------------------------
# Query compression and the output projection ("Operator Notes (1): MLA", section 4: the
# query is compressed too, c_q = x W_DQ and Q = c_q W_UQ; section 2: out = O W_O), and the
# folds of the glossary entry's paragraph on the decoupled RoPE key (W_UK absorbed into
# the query side, W_UV into the output side).
# ---------------------------------------------------------------------------------
#
# Readings: the query latent width d_cq is a parameter (the page writes "d_c dim"); the
# up-projection of the query yields, per head, the d_h content part followed by the d_r
# RoPE part, kept as two matrices w_uq [d_cq, n_h, d_h] and w_qr [d_cq, n_h, d_r]; no
# normalisation sits between the two projections (the pages show none).


def query_from_hidden(x, w_dq, w_uq, w_qr):
    """x [M, d_model] -> (q_nope [M, n_h, d_h], q_rope [M, n_h, d_r]) through c_q = x W_DQ."""
    c_q = np.asarray(x, np.float64) @ np.asarray(w_dq, np.float64)
    w_uq = np.asarray(w_uq, np.float64)
    w_qr = np.asarray(w_qr, np.float64)
    q_nope = np.einsum("mk,khj->mhj", c_q, w_uq, optimize=True)
    q_rope = np.einsum("mk,khj->mhj", c_q, w_qr, optimize=True)
    return q_nope, q_rope


def fold_query_weights(w_uq, w_uk):
    """W_UQK[k, h, c] = sum_j w_uq[k, h, j] w_uk[h, j, c]: the query up-projection
    followed by the key absorption, as one matrix from c_q to the latent query."""
    return np.einsum("khj,hjc->khc", np.asarray(w_uq, np.float64), np.asarray(w_uk, np.float64), optimize=True)


def output_projection(out_heads, w_o):
    """out_heads [M, n_h, d_h] (the concatenated head outputs O) -> O W_O [M, d_model]."""
    o = np.asarray(out_heads, np.float64)
    return o.reshape(o.shape[0], -1) @ np.asarray(w_o, np.float64)


def fold_output_weights(w_uv, w_o):
    """W_UVO[h, c, :] = sum_j w_uv[h, c, j] w_o[h d_h + j, :]: the value up-projection
    followed by the output projection, per head, so that out = sum_h o_lat[h] W_UVO[h]."""
    w_uv = np.asarray(w_uv, np.float64)
    n_h, d_c, d_h = w_uv.shape
    w_o = np.asarray(w_o, np.float64).reshape(n_h, d_h, -1)
    return np.einsum("hcj,hjd->hcd", w_uv, w_o, optimize=True)
