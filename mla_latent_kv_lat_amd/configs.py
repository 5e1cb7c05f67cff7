"""Workload shapes for weight-absorbed MLA decode.

The DeepSeek-V2-style dimensions (n_h = d_h = 128, d_c = 512) are the ones the
"Operator Notes (1): MLA" page uses in its section 1 (MHA cache size) and section 3
(cache-shrink table).  The decoupled RoPE key width d_r and the batch / context
mixes are workload choices of this project, stated here once so that the tests,
the benchmark and the oracle all read the same numbers.

Every field is a plain integer or string; nothing here computes attention.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class MLAConfig:
    name: str
    cfg_id: int                 # feeds the seed sequence of every tensor of this workload
    batch: int                  # B: number of sequences
    q_len: int                  # s_q: new query tokens per sequence (causal among them)
    n_heads: int                # n_h
    d_head: int                 # d_h
    d_latent: int               # d_c
    d_rope: int                 # d_r: width of the decoupled RoPE key
    seq_len: int                # T: context length (upper bound when lengths vary)
    kv_dtype: str               # storage of c_kv: "f32" | "bf16" | "fp8"
    act_dtype: str              # storage of q_nope, q_rope, k_rope, W_UK, W_UV, q_lat, o_lat, out
    paged: bool = False
    block_size: int = 64
    len_min: Optional[int] = None   # variable lengths: uniform integers in [len_min, seq_len]
    description: str = ""

    @property
    def rows(self) -> int:
        """Query rows per sequence: every (query token, head) pair."""
        return self.q_len * self.n_heads

    @property
    def softmax_scale(self) -> float:
        """1/sqrt(d_h + d_r): the width of the concatenated [content | rope] key."""
        return 1.0 / float(self.d_head + self.d_rope) ** 0.5

    def with_(self, **kw) -> "MLAConfig":
        return replace(self, **kw)


TINY = MLAConfig(
    name="tiny_f32", cfg_id=0, batch=1, q_len=1, n_heads=8, d_head=32, d_latent=64,
    d_rope=16, seq_len=128, kv_dtype="f32", act_dtype="f32",
    description="batch 1, 1 query token, n_h=8, d_h=32, d_c=64, d_r=16, T=128, fp32",
)

V2_DECODE = MLAConfig(
    name="v2_decode_bf16_b32_t4096", cfg_id=1, batch=32, q_len=1, n_heads=128, d_head=128,
    d_latent=512, d_rope=64, seq_len=4096, kv_dtype="bf16", act_dtype="bf16",
    description="DeepSeek-V2-shaped decode: B=32, s_q=1, n_h=128, d_h=128, d_c=512, d_r=64, "
                "T=4096, bf16 cache and weights, fp32 accumulate",
)

PAGED_VARLEN = MLAConfig(
    name="paged_varlen_bf16_b64", cfg_id=2, batch=64, q_len=1, n_heads=128, d_head=128,
    d_latent=512, d_rope=64, seq_len=16384, len_min=512, kv_dtype="bf16", act_dtype="bf16",
    paged=True, block_size=64,
    description="64 sequences, lengths uniform in [512, 16384], bf16 latent cache in 64-token "
                "blocks, block table a seeded permutation of a shared pool",
)

LONG_CONTEXT = MLAConfig(
    name="long_bf16_b4_t131072", cfg_id=3, batch=4, q_len=1, n_heads=128, d_head=128,
    d_latent=512, d_rope=64, seq_len=131072, kv_dtype="bf16", act_dtype="bf16",
    description="B=4, T=131072 per sequence, bf16 contiguous cache",
)

SPEC_FP8 = MLAConfig(
    name="spec4_fp8_b128_t8192", cfg_id=4, batch=128, q_len=4, n_heads=128, d_head=128,
    d_latent=512, d_rope=64, seq_len=8192, kv_dtype="fp8", act_dtype="bf16",
    description="B=128, 4 query tokens causal among themselves, T=8192, c_kv fp8 e4m3 with a "
                "per-token fp32 scale, k_rope bf16",
)

ALL = (TINY, V2_DECODE, PAGED_VARLEN, LONG_CONTEXT, SPEC_FP8)
BY_NAME = {c.name: c for c in ALL}

# The workload the benchmark line is quoted on.
HEADLINE = V2_DECODE
