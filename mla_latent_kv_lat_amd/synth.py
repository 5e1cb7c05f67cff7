"""Seeded synthetic inputs for MLA decode workloads.

This module is shared by the GPU path's tests and benchmark and by the CPU oracle's
tests.  It draws random numbers and encodes them into the storage formats the
library consumes; it does no attention arithmetic at all (no projection, no score,
no softmax, no weighted sum).

Recipe (one generator per tensor, so that each tensor is reproducible alone):

* ``numpy.random.default_rng(SeedSequence([seed, cfg_id, tensor_id]))`` with the
  tensor ids in ``TENSOR_IDS``.
* Activations (``c_kv``, ``k_rope``, ``q_nope``, ``q_rope``) are N(0, 1).
* Up-projection weights ``W_UK[n_h, d_h, d_c]`` and ``W_UV[n_h, d_c, d_h]`` are
  N(0, 1) / sqrt(d_c): both read the d_c-wide latent, so d_c is their fan-in.
* Values are drawn in float32 and then stored:
  - ``f32``  as is;
  - ``bf16`` rounded to nearest-even (torch's CPU cast), kept as raw uint16 bits;
  - ``fp8``  (latent only) per token: scale = max|row| / 448 (1 for an all-zero row),
    code = e4m3fn(round-to-nearest-even(row / scale)) via torch's CPU cast, kept as
    raw uint8 codes next to a float32 scale per token.
* Variable lengths are uniform integers in [len_min, T] (both ends included).
* A paged cache is a pool of ``N_blk = sum_b ceil(L_b / bs)`` blocks; a seeded
  permutation of the pool indices is dealt out in order, ceil(L_b / bs) entries per
  sequence; unused block-table slots hold -1.
* ``poison_tail=True`` fills every cache row a sequence does not own (rows at or past
  its length) with NaN, so that a kernel which reads masked rows into its sums fails.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import MLAConfig

TENSOR_IDS = {
    "c_kv": 0, "k_rope": 1, "q_nope": 2, "q_rope": 3, "w_uk": 4, "w_uv": 5,
    "lengths": 6, "perm": 7, "q_lat": 8, "o_lat": 9, "x": 10, "w_dkv": 11, "w_kr": 12,
}

E4M3_MAX = 448.0
BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F


def rng_for(seed: int, cfg_id: int, tensor: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg_id, TENSOR_IDS[tensor]]))


def normal_f32(seed: int, cfg_id: int, tensor: str, shape, std: float = 1.0) -> np.ndarray:
    x = rng_for(seed, cfg_id, tensor).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the raw 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Encode float32 values (already within +-448) as OCP e4m3fn bytes, nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def quantize_rows_e4m3(x: np.ndarray):
    """Per-row (last axis) scaled e4m3fn encoding: returns (codes uint8, scale float32)."""
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    y = np.clip(x / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return f32_to_e4m3_codes(y), scale


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"no plain storage for dtype {dtype!r}")


@dataclass
class Inputs:
    """Stored (raw) tensors of one decode workload, as numpy arrays.

    bf16 tensors are uint16 bit patterns, fp8 tensors uint8 codes, f32 tensors float32.
    Contiguous caches are [B, T, .]; paged caches are pools [N_blk, bs, .] plus a
    block table [B, max_blocks] (int32, -1 where unused).
    """
    cfg: MLAConfig
    seed: int
    q_nope: np.ndarray
    q_rope: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    c_kv: np.ndarray                  # [B,T,d_c] or pool [N_blk,bs,d_c]
    k_rope: np.ndarray                # [B,T,d_r] or pool [N_blk,bs,d_r]
    kv_scale: Optional[np.ndarray]    # fp8 only: [B,T] or pool [N_blk,bs] float32
    seq_lens: np.ndarray              # [B] int32
    block_table: Optional[np.ndarray] = None   # paged only
    c_kv_prequant: Optional[np.ndarray] = None  # fp8 only: the float32 latent before encoding

    @property
    def n_blocks(self) -> int:
        return int(self.c_kv.shape[0]) if self.cfg.paged else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1]) if self.block_table is not None else 0


def draw_lengths(cfg: MLAConfig, seed: int) -> np.ndarray:
    if cfg.len_min is None:
        return np.full(cfg.batch, cfg.seq_len, dtype=np.int32)
    r = rng_for(seed, cfg.cfg_id, "lengths")
    return r.integers(cfg.len_min, cfg.seq_len, size=cfg.batch, endpoint=True).astype(np.int32)


def paged_layout(cfg: MLAConfig, seed: int, seq_lens: np.ndarray):
    """Block table of a shared pool: N_blk = sum_b ceil(L_b / bs) blocks, a seeded
    permutation of the pool dealt out in order; unused slots hold -1.  Returns (table, N_blk)."""
    bs = cfg.block_size
    nblk_per = (seq_lens.astype(np.int64) + bs - 1) // bs
    n_blk = int(nblk_per.sum())
    max_blocks = (cfg.seq_len + bs - 1) // bs
    perm = rng_for(seed, cfg.cfg_id, "perm").permutation(n_blk).astype(np.int32)
    table = np.full((cfg.batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(cfg.batch):
        n = int(nblk_per[b])
        table[b, :n] = perm[off:off + n]
        off += n
    return table, n_blk


def make_inputs(cfg: MLAConfig, seed: int = 0, *, poison_tail: bool = False,
                q_gain: float = 1.0, lengths: Optional[np.ndarray] = None) -> Inputs:
    B, sq, H = cfg.batch, cfg.q_len, cfg.n_heads
    dh, dc, dr, T = cfg.d_head, cfg.d_latent, cfg.d_rope, cfg.seq_len
    cid = cfg.cfg_id
    act = cfg.act_dtype

    q_nope = normal_f32(seed, cid, "q_nope", (B, sq, H, dh))
    q_rope = normal_f32(seed, cid, "q_rope", (B, sq, H, dr))
    if q_gain != 1.0:
        q_nope *= np.float32(q_gain)
        q_rope *= np.float32(q_gain)
    w_std = 1.0 / float(dc) ** 0.5
    w_uk = normal_f32(seed, cid, "w_uk", (H, dh, dc), w_std)
    w_uv = normal_f32(seed, cid, "w_uv", (H, dc, dh), w_std)

    seq_lens = draw_lengths(cfg, seed) if lengths is None else np.asarray(lengths, np.int32)
    if seq_lens.shape != (B,) or seq_lens.min() < 0 or seq_lens.max() > T:
        raise ValueError("lengths must be [B] integers in [0, T]")

    if cfg.paged:
        bs = cfg.block_size
        table, n_blk = paged_layout(cfg, seed, seq_lens)
        lat_shape, rope_shape = (n_blk, bs, dc), (n_blk, bs, dr)
    else:
        table = None
        lat_shape, rope_shape = (B, T, dc), (B, T, dr)

    c_lat = normal_f32(seed, cid, "c_kv", lat_shape)
    c_rope = normal_f32(seed, cid, "k_rope", rope_shape)

    # Rows each sequence does not own: [L_b, T) of a contiguous cache, and the tail of
    # the last block of each sequence in a pool (whole blocks are all owned).
    if poison_tail:
        if cfg.paged:
            for b in range(B):
                L = int(seq_lens[b])
                if L % cfg.block_size:
                    blk = table[b, L // cfg.block_size]
                    c_lat[blk, L % cfg.block_size:] = np.nan
                    c_rope[blk, L % cfg.block_size:] = np.nan
        else:
            for b in range(B):
                L = int(seq_lens[b])
                c_lat[b, L:] = np.nan
                c_rope[b, L:] = np.nan

    kv_scale = None
    prequant = None
    if cfg.kv_dtype == "fp8":
        prequant = c_lat
        finite = np.where(np.isfinite(c_lat), c_lat, np.float32(0))
        codes, kv_scale = quantize_rows_e4m3(finite)
        if poison_tail:
            codes[~np.isfinite(c_lat)] = E4M3_NAN_CODE
        c_store = codes
    else:
        c_store = store(c_lat, cfg.kv_dtype)

    return Inputs(
        cfg=cfg, seed=seed,
        q_nope=store(q_nope, act), q_rope=store(q_rope, act),
        w_uk=store(w_uk, act), w_uv=store(w_uv, act),
        c_kv=c_store, k_rope=store(c_rope, act), kv_scale=kv_scale,
        seq_lens=seq_lens, block_table=table, c_kv_prequant=prequant,
    )


def make_stage_input(cfg: MLAConfig, seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    """A stand-alone stored activation (e.g. a latent query or a latent output), for
    testing one entry point on its own."""
    return store(normal_f32(seed, cfg.cfg_id, name, shape, std), cfg.act_dtype)


@dataclass
class AppendInputs:
    """Inputs of the cache-write step: hidden states of the s_q new tokens of every
    sequence, the down-projection W_DKV [d_model, d_c] and the RoPE-key projection
    W_KR [d_model, d_r] (both N(0,1) / sqrt(d_model): d_model is their fan-in), and a pool
    layout in which the new tokens are the last s_q rows of each sequence."""
    cfg: MLAConfig
    d_model: int
    x: np.ndarray          # [B, s_q, d_model] stored
    w_dkv: np.ndarray      # [d_model, d_c] stored
    w_kr: np.ndarray       # [d_model, d_r] stored
    seq_lens: np.ndarray   # [B] int32, counting the new tokens
    block_table: np.ndarray
    n_blocks: int


def make_append_inputs(cfg: MLAConfig, d_model: int, seed: int = 0) -> AppendInputs:
    B, sq, dc, dr = cfg.batch, cfg.q_len, cfg.d_latent, cfg.d_rope
    cid = cfg.cfg_id
    w_std = 1.0 / float(d_model) ** 0.5
    x = normal_f32(seed, cid, "x", (B, sq, d_model))
    w_dkv = normal_f32(seed, cid, "w_dkv", (d_model, dc), w_std)
    w_kr = normal_f32(seed, cid, "w_kr", (d_model, dr), w_std)
    seq_lens = np.maximum(draw_lengths(cfg, seed), sq).astype(np.int32)
    table, n_blk = paged_layout(cfg, seed, seq_lens)
    act = cfg.act_dtype
    return AppendInputs(cfg=cfg, d_model=d_model, x=store(x, act), w_dkv=store(w_dkv, act),
                        w_kr=store(w_kr, act), seq_lens=seq_lens, block_table=table, n_blocks=n_blk)
