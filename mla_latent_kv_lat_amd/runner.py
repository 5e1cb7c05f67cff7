"""Device plumbing around libmla: upload a workload, allocate outputs, run one decode step.

A step is the three library calls of weight-absorbed MLA decode:
  mla_absorb_q -> mla_decode (or mla_decode_paged) -> mla_absorb_out.
torch only provides device memory and the stream; all arithmetic runs in libmla.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import capi as libmla
from .synth import Inputs

TORCH_OF = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(arr: np.ndarray, kind: str, device) -> torch.Tensor:
    """Raw stored array -> device tensor of the matching torch dtype (bits unchanged)."""
    if kind == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, np.float32))
    elif kind == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif kind == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(arr, np.uint8))
    elif kind == "i32":
        t = torch.from_numpy(np.ascontiguousarray(arr, np.int32))
    else:
        raise ValueError(kind)
    return t.to(device)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


class DeviceWorkload:
    """One workload resident in device memory, with its outputs and workspace."""

    def __init__(self, inp: Inputs, device="cuda", split_tokens: int = 0, replicas: int = 1,
                 fp8_scores: int = 0):
        cfg = inp.cfg
        self.cfg, self.inp, self.device = cfg, inp, device
        act, kvk = cfg.act_dtype, cfg.kv_dtype
        self.dims = libmla.dims_from_config(cfg, split_tokens, fp8_scores)
        self.q_nope = to_device(inp.q_nope, act, device)
        self.q_rope = to_device(inp.q_rope, act, device)
        self.seq_lens = to_device(inp.seq_lens, "i32", device)
        # `replicas` copies of the cache and weights at distinct addresses, cycled by step(),
        # so that a timed loop streams from HBM rather than from the last-level cache.
        self.caches = []
        for _ in range(max(1, replicas)):
            c = {
                "c_kv": to_device(inp.c_kv, kvk, device),
                "k_rope": to_device(inp.k_rope, act, device),
                "kv_scale": None if inp.kv_scale is None else to_device(inp.kv_scale, "f32", device),
                "w_uk": to_device(inp.w_uk, act, device),
                "w_uv": to_device(inp.w_uv, act, device),
            }
            self.caches.append(c)
        self.block_table = None if inp.block_table is None else to_device(inp.block_table, "i32", device)
        B, sq, H = cfg.batch, cfg.q_len, cfg.n_heads
        dt = TORCH_OF[act]
        self.q_lat = torch.empty(B, sq, H, cfg.d_latent, dtype=dt, device=device)
        self.o_lat = torch.empty(B, sq, H, cfg.d_latent, dtype=dt, device=device)
        self.out = torch.empty(B, sq, H, cfg.d_head, dtype=dt, device=device)
        self.lse = torch.empty(B, sq, H, dtype=torch.float32, device=device)
        kv_code = libmla.DTYPE_CODES[kvk]
        self.ws_bytes = libmla.mla_decode_workspace_bytes(self.dims, kv_code, cfg.seq_len)
        self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
                          if self.ws_bytes else None)
        self.plan = libmla.mla_decode_plan(self.dims, kv_code, cfg.seq_len)
        self._k = 0

    def absorb_q(self, c: Optional[dict] = None):
        c = c or self.caches[0]
        libmla.mla_absorb_q(self.dims, self.q_nope, c["w_uk"], self.q_lat)

    def decode(self, c: Optional[dict] = None, q_lat=None):
        c = c or self.caches[0]
        q_lat = self.q_lat if q_lat is None else q_lat
        cfg = self.cfg
        if cfg.paged:
            libmla.mla_decode_paged(self.dims, q_lat, self.q_rope, c["c_kv"], c["k_rope"],
                                    self.block_table, self.seq_lens, cfg.seq_len, self.o_lat,
                                    self.lse, self.workspace, kv_scale_pool=c["kv_scale"],
                                    block_size=cfg.block_size)
        else:
            libmla.mla_decode(self.dims, q_lat, self.q_rope, c["c_kv"], c["k_rope"], cfg.seq_len,
                              self.seq_lens, self.o_lat, self.lse, self.workspace,
                              kv_scale=c["kv_scale"])

    def absorb_out(self, c: Optional[dict] = None, o_lat=None):
        c = c or self.caches[0]
        libmla.mla_absorb_out(self.dims, self.o_lat if o_lat is None else o_lat, c["w_uv"], self.out)

    def decode_absorb_out(self, c: Optional[dict] = None, q_lat=None):
        """Latent attention and output absorption in one library call (contiguous caches;
        a paged cache takes the two calls)."""
        c = c or self.caches[0]
        q_lat = self.q_lat if q_lat is None else q_lat
        cfg = self.cfg
        if cfg.paged:
            self.decode(c, q_lat)
            self.absorb_out(c)
            return
        libmla.mla_decode_absorb_out(self.dims, q_lat, self.q_rope, c["c_kv"], c["k_rope"], cfg.seq_len,
                                     self.seq_lens, c["w_uv"], self.o_lat, self.lse, self.out, self.workspace,
                                     kv_scale=c["kv_scale"])

    def step(self):
        """One whole decode step over the next replica."""
        c = self.caches[self._k % len(self.caches)]
        self._k += 1
        self.absorb_q(c)
        self.decode(c)
        self.absorb_out(c)
