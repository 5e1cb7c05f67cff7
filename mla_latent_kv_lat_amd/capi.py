"""Thin ctypes binding of libmla (include/mla.h).

Argument marshalling only: every function here passes device pointers, sizes and the
current HIP stream to the C entry point of the same name and raises ``MLAError`` on a
non-OK status (or returns the status with ``check=False``).  No computation happens in
Python, and nothing falls back to another implementation: if libmla.so is missing the
import of this module's functions fails loudly.

Tensor arguments are torch tensors (their ``data_ptr()`` is passed) or, for tests of the
validation paths, plain integers taken as raw addresses.  Dtypes are inferred from the
tensors: float32 -> MLA_F32, bfloat16 -> MLA_BF16, uint8 / float8_e4m3fn -> MLA_FP8_E4M3.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
MLA_F32, MLA_BF16, MLA_FP8_E4M3 = range(3)

DTYPE_CODES = {"f32": MLA_F32, "bf16": MLA_BF16, "fp8": MLA_FP8_E4M3}

EXPORTED = (
    "mla_absorb_q", "mla_decode", "mla_decode_paged", "mla_decode_workspace_bytes",
    "mla_decode_plan", "mla_absorb_out", "mla_gather_pages", "mla_fp8_e4m3_table",
    "mla_status_str", "mla_last_hip_error", "mla_version", "mla_cache_append_workspace_bytes",
    "mla_cache_append", "mla_rope_query", "mla_prefill_workspace_bytes", "mla_prefill",
    "mla_linear_workspace_bytes", "mla_linear", "mla_decode_noalloc", "mla_fold_output_weights",
    "mla_decode_absorb_out",
)

# Size of the static device array mla_decode_noalloc keeps its partial results in.
NOALLOC_SCRATCH_BYTES = 80 << 20


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().mla_status_str(status).decode()
        if status == MLA_ERR_HIP:
            msg += f" (hipError_t {_lib().mla_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


class MlaDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("d_head", ctypes.c_int32), ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("split_tokens", ctypes.c_int32),
        ("fp8_scores", ctypes.c_int32),
    ]


def dims(batch, q_len, n_heads, d_head, d_latent, d_rope, softmax_scale, split_tokens=0,
         fp8_scores=0) -> MlaDims:
    return MlaDims(batch, q_len, n_heads, d_head, d_latent, d_rope, softmax_scale, split_tokens,
                   fp8_scores)


def dims_from_config(cfg, split_tokens: int = 0, fp8_scores: int = 0) -> MlaDims:
    return dims(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_head, cfg.d_latent, cfg.d_rope,
                cfg.softmax_scale, split_tokens, fp8_scores)


_LIB: Optional[ctypes.CDLL] = None

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_dims_p = ctypes.POINTER(MlaDims)
_SIGNATURES = {
    "mla_absorb_q": [_dims_p, _vp, _i32, _vp, _i32, _vp, _i32, _vp],
    "mla_absorb_out": [_dims_p, _vp, _i32, _vp, _i32, _vp, _i32, _vp],
    "mla_decode": [_dims_p, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _vp,
                   _vp, _sz, _vp],
    "mla_decode_paged": [_dims_p, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _i32,
                         _vp, _i32, _vp, _i32, _vp, _vp, _sz, _vp],
    "mla_decode_noalloc": [_dims_p, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _vp,
                           _vp],
    "mla_decode_workspace_bytes": [_dims_p, _i32, _i32],
    "mla_decode_plan": [_dims_p, _i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)],
    "mla_gather_pages": [_vp, _i32, _i32, _i64, _vp, _i32, _i32, _vp, _i32, _vp, _vp],
    "mla_fp8_e4m3_table": [_vp, _vp],
    "mla_cache_append_workspace_bytes": [_dims_p, _i32],
    "mla_cache_append": [_dims_p, _i32, _vp, _vp, _vp, _i32, ctypes.c_float, _i32, _vp, _i32, _vp, _vp,
                         _i32, _i32, _vp, _i32, _vp, _vp, _sz, _vp],
    "mla_rope_query": [_dims_p, _vp, _i32, _vp, ctypes.c_float, _i32, _vp],
    "mla_prefill_workspace_bytes": [_dims_p, _i32],
    "mla_linear_workspace_bytes": [_i32, _i32, _i32],
    "mla_linear": [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp],
    "mla_fold_output_weights": [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp],
    "mla_decode_absorb_out": [_dims_p, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                              _vp, _sz, _vp],
    "mla_prefill": [_dims_p, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp],
    "mla_status_str": [_i32],
    "mla_last_hip_error": [],
    "mla_version": [],
}


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmla.so not built ({LIB_PATH}); run "
                              "`python -m mla_latent_kv_lat_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _i32
        lib.mla_decode_workspace_bytes.restype = _sz
        lib.mla_cache_append_workspace_bytes.restype = _sz
        lib.mla_prefill_workspace_bytes.restype = _sz
        lib.mla_linear_workspace_bytes.restype = _sz
        lib.mla_status_str.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def library() -> ctypes.CDLL:
    """The loaded libmla.so (raises ImportError if it was not built)."""
    return _lib()


def _ptr(x):
    """Device address of a tensor argument (or a raw integer address, passed through).
    Tensors must be dense and on the GPU: the library reads them as contiguous row-major
    arrays at that address, so a strided view or a host tensor would be misread."""
    if x is None:
        return None
    if isinstance(x, int):
        return _vp(x)
    if not x.is_cuda:
        raise ValueError(f"libmla needs device tensors, got one on {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"libmla needs contiguous tensors, got strides {tuple(x.stride())} "
                         f"for shape {tuple(x.shape)}")
    return _vp(x.data_ptr())


def _dt(x, explicit=None) -> int:
    if explicit is not None:
        return DTYPE_CODES[explicit] if isinstance(explicit, str) else int(explicit)
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.float32:
            return MLA_F32
        if x.dtype == torch.bfloat16:
            return MLA_BF16
        if x.dtype in (torch.uint8, torch.float8_e4m3fn):
            return MLA_FP8_E4M3
        raise TypeError(f"unsupported tensor dtype {x.dtype}")
    raise TypeError("dtype must be given for raw pointers")


def _stream(stream):
    if stream is not None:
        return _vp(stream if isinstance(stream, int) else stream.cuda_stream)
    if torch.cuda.is_available() and torch.cuda.is_initialized():
        return _vp(torch.cuda.current_stream().cuda_stream)
    return None


def _done(status: int, where: str, check: bool) -> int:
    if check and status != MLA_OK:
        raise MLAError(status, where)
    return status


def mla_absorb_q(d: MlaDims, q_nope, w_uk, q_lat, *, dtype=None, stream=None, check=True) -> int:
    dt = _dt(q_nope, dtype)
    st = _lib().mla_absorb_q(ctypes.byref(d), _ptr(q_nope), dt, _ptr(w_uk), _dt(w_uk, dtype),
                             _ptr(q_lat), _dt(q_lat, dtype), _stream(stream))
    return _done(st, "mla_absorb_q", check)


def mla_absorb_out(d: MlaDims, o_lat, w_uv, out, *, dtype=None, stream=None, check=True) -> int:
    st = _lib().mla_absorb_out(ctypes.byref(d), _ptr(o_lat), _dt(o_lat, dtype), _ptr(w_uv),
                               _dt(w_uv, dtype), _ptr(out), _dt(out, dtype), _stream(stream))
    return _done(st, "mla_absorb_out", check)


def mla_decode_workspace_bytes(d: MlaDims, kv_dtype, max_seq_len: int) -> int:
    return int(_lib().mla_decode_workspace_bytes(ctypes.byref(d), _dt(None, kv_dtype), max_seq_len))


def mla_decode_plan(d: MlaDims, kv_dtype, max_seq_len: int, *, check=True):
    n, tok = _i32(0), _i32(0)
    st = _lib().mla_decode_plan(ctypes.byref(d), _dt(None, kv_dtype), max_seq_len,
                                ctypes.byref(n), ctypes.byref(tok))
    if not check:
        return st, n.value, tok.value
    _done(st, "mla_decode_plan", True)
    return n.value, tok.value


def mla_decode(d: MlaDims, q_lat, q_rope, c_kv, k_rope, T: int, seq_lens, o_lat, lse, workspace,
               workspace_bytes: Optional[int] = None, *, kv_scale=None, q_dtype=None,
               kv_dtype=None, stream=None, check=True) -> int:
    qdt = _dt(q_lat, q_dtype)
    kvdt = _dt(c_kv, kv_dtype)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib().mla_decode(ctypes.byref(d), _ptr(q_lat), _ptr(q_rope), qdt, _ptr(c_kv), kvdt,
                           _ptr(kv_scale), _ptr(k_rope), qdt if k_rope is None else _dt(k_rope, q_dtype),
                           T, _ptr(seq_lens), _ptr(o_lat), qdt if o_lat is None else _dt(o_lat, q_dtype),
                           _ptr(lse), _ptr(workspace), workspace_bytes, _stream(stream))
    return _done(st, "mla_decode", check)


def mla_decode_absorb_out(d: MlaDims, q_lat, q_rope, c_kv, k_rope, T: int, seq_lens, w_uv, o_lat, lse, out,
                          workspace, workspace_bytes: Optional[int] = None, *, kv_scale=None, q_dtype=None,
                          kv_dtype=None, stream=None, check=True) -> int:
    """mla_decode followed by mla_absorb_out in one call (argument marshalling only)."""
    qdt = _dt(q_lat, q_dtype)
    kvdt = _dt(c_kv, kv_dtype)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib().mla_decode_absorb_out(ctypes.byref(d), _ptr(q_lat), _ptr(q_rope), qdt, _ptr(c_kv), kvdt,
                                      _ptr(kv_scale), _ptr(k_rope), qdt if k_rope is None else _dt(k_rope, q_dtype),
                                      T, _ptr(seq_lens), _ptr(w_uv), _ptr(o_lat), _ptr(lse), _ptr(out),
                                      _ptr(workspace), workspace_bytes, _stream(stream))
    return _done(st, "mla_decode_absorb_out", check)


def mla_decode_noalloc(d: MlaDims, q_lat, q_rope, c_kv, k_rope, T: int, seq_lens, o_lat, lse, *,
                       kv_scale=None, q_dtype=None, kv_dtype=None, stream=None, check=True) -> int:
    """mla_decode with its partial results in the library's static device array (no
    workspace argument; argument marshalling only)."""
    qdt = _dt(q_lat, q_dtype)
    kvdt = _dt(c_kv, kv_dtype)
    st = _lib().mla_decode_noalloc(ctypes.byref(d), _ptr(q_lat), _ptr(q_rope), qdt, _ptr(c_kv), kvdt,
                                   _ptr(kv_scale), _ptr(k_rope), qdt if k_rope is None else _dt(k_rope, q_dtype),
                                   T, _ptr(seq_lens), _ptr(o_lat), qdt if o_lat is None else _dt(o_lat, q_dtype),
                                   _ptr(lse), _stream(stream))
    return _done(st, "mla_decode_noalloc", check)


def mla_decode_paged(d: MlaDims, q_lat, q_rope, c_kv_pool, k_rope_pool, block_table, seq_lens,
                     max_seq_len: int, o_lat, lse, workspace, workspace_bytes: Optional[int] = None,
                     *, kv_scale_pool=None, block_size: Optional[int] = None,
                     n_blocks: Optional[int] = None, max_blocks_per_seq: Optional[int] = None,
                     q_dtype=None, kv_dtype=None, stream=None, check=True) -> int:
    qdt = _dt(q_lat, q_dtype)
    kvdt = _dt(c_kv_pool, kv_dtype)
    if block_size is None:
        block_size = c_kv_pool.shape[1]
    if n_blocks is None:
        n_blocks = c_kv_pool.shape[0]
    if max_blocks_per_seq is None:
        max_blocks_per_seq = block_table.shape[1]
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib().mla_decode_paged(
        ctypes.byref(d), _ptr(q_lat), _ptr(q_rope), qdt, _ptr(c_kv_pool), kvdt, _ptr(kv_scale_pool),
        _ptr(k_rope_pool), qdt if k_rope_pool is None else _dt(k_rope_pool, q_dtype), n_blocks,
        block_size, _ptr(block_table), max_blocks_per_seq, _ptr(seq_lens), max_seq_len, _ptr(o_lat),
        qdt if o_lat is None else _dt(o_lat, q_dtype), _ptr(lse), _ptr(workspace), workspace_bytes,
        _stream(stream))
    return _done(st, "mla_decode_paged", check)


def mla_gather_pages(pool, block_table, seq_lens, max_seq_len: int, dst, *, block_size=None,
                     n_blocks=None, row_bytes=None, batch=None, max_blocks_per_seq=None,
                     stream=None, check=True) -> int:
    if block_size is None:
        block_size = pool.shape[1]
    if n_blocks is None:
        n_blocks = pool.shape[0]
    if row_bytes is None:
        row_bytes = pool[0, 0].numel() * pool.element_size()
    if batch is None:
        batch = block_table.shape[0]
    if max_blocks_per_seq is None:
        max_blocks_per_seq = block_table.shape[1]
    st = _lib().mla_gather_pages(_ptr(pool), n_blocks, block_size, row_bytes, _ptr(block_table), batch,
                                 max_blocks_per_seq, _ptr(seq_lens), max_seq_len, _ptr(dst),
                                 _stream(stream))
    return _done(st, "mla_gather_pages", check)


ROPE_PAIRING = {"interleaved": 0, "half": 1}


def mla_cache_append_workspace_bytes(d: MlaDims, d_model: int) -> int:
    return int(_lib().mla_cache_append_workspace_bytes(ctypes.byref(d), d_model))


def mla_cache_append(d: MlaDims, x, w_dkv, w_kr, c_kv_pool, k_rope_pool, block_table, seq_lens, workspace,
                     *, rope_base: float = 10000.0, pairing: str = "interleaved", kv_scale_pool=None,
                     workspace_bytes: Optional[int] = None, d_model: Optional[int] = None,
                     block_size: Optional[int] = None, n_blocks: Optional[int] = None,
                     max_blocks_per_seq: Optional[int] = None, x_dtype=None, kv_dtype=None,
                     stream=None, check=True) -> int:
    if d_model is None:
        d_model = x.shape[-1]
    if block_size is None:
        block_size = c_kv_pool.shape[1]
    if n_blocks is None:
        n_blocks = c_kv_pool.shape[0]
    if max_blocks_per_seq is None:
        max_blocks_per_seq = block_table.shape[1]
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib().mla_cache_append(
        ctypes.byref(d), d_model, _ptr(x), _ptr(w_dkv), _ptr(w_kr), _dt(x, x_dtype), rope_base,
        ROPE_PAIRING[pairing], _ptr(c_kv_pool), _dt(c_kv_pool, kv_dtype), _ptr(kv_scale_pool),
        _ptr(k_rope_pool), n_blocks, block_size, _ptr(block_table), max_blocks_per_seq, _ptr(seq_lens),
        _ptr(workspace), workspace_bytes, _stream(stream))
    return _done(st, "mla_cache_append", check)


def mla_rope_query(d: MlaDims, q_rope, seq_lens, *, rope_base: float = 10000.0, pairing: str = "interleaved",
                   dtype=None, stream=None, check=True) -> int:
    st = _lib().mla_rope_query(ctypes.byref(d), _ptr(q_rope), _dt(q_rope, dtype), _ptr(seq_lens), rope_base,
                               ROPE_PAIRING[pairing], _stream(stream))
    return _done(st, "mla_rope_query", check)


def mla_prefill_workspace_bytes(d: MlaDims, T: int) -> int:
    return int(_lib().mla_prefill_workspace_bytes(ctypes.byref(d), T))


def mla_prefill(d: MlaDims, q_nope, q_rope, c_kv, k_rope, T: int, seq_lens, w_uk, w_uv, out, lse,
                workspace, *, workspace_bytes=None, dtype=None, stream=None, check=True) -> int:
    """Explicit-form causal prefill (argument marshalling only)."""
    wsb = workspace_bytes
    if wsb is None:
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib().mla_prefill(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(c_kv), _ptr(k_rope), T,
                            _ptr(seq_lens), _ptr(w_uk), _ptr(w_uv), _dt(q_nope, dtype), _ptr(out), _ptr(lse),
                            _ptr(workspace), wsb, _stream(stream))
    return _done(st, "mla_prefill", check)


def mla_linear_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(_lib().mla_linear_workspace_bytes(M, K, N))


def mla_linear(x, w, y, workspace, *, M=None, K=None, N=None, workspace_bytes=None, dtype=None,
               stream=None, check=True) -> int:
    """y = x . w for row-major x [M, K], w [K, N], y [M, N] (argument marshalling only)."""
    if M is None:
        M = y.shape[0]
    if K is None:
        K = w.shape[0]
    if N is None:
        N = w.shape[1]
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib().mla_linear(_ptr(x), _ptr(w), _ptr(y), M, K, N, _dt(x, dtype), _ptr(workspace),
                           workspace_bytes, _stream(stream))
    return _done(st, "mla_linear", check)


def mla_fold_output_weights(w_uv, w_o, w_uvo, *, n_h=None, d_c=None, d_h=None, d_model=None, dtype=None,
                            stream=None, check=True) -> int:
    """w_uvo[h] = w_uv[h] . w_o[h d_h : (h + 1) d_h] for w_uv [n_h, d_c, d_h], w_o [n_h d_h,
    d_model], w_uvo [n_h, d_c, d_model] (argument marshalling only)."""
    if n_h is None:
        n_h, d_c, d_h = w_uv.shape
    if d_model is None:
        d_model = w_o.shape[1]
    st = _lib().mla_fold_output_weights(_ptr(w_uv), _ptr(w_o), _ptr(w_uvo), n_h, d_c, d_h, d_model,
                                        _dt(w_uv, dtype), _stream(stream))
    return _done(st, "mla_fold_output_weights", check)


def mla_fp8_e4m3_table(out, *, stream=None, check=True) -> int:
    return _done(_lib().mla_fp8_e4m3_table(_ptr(out), _stream(stream)), "mla_fp8_e4m3_table", check)


def mla_status_str(status: int) -> str:
    return _lib().mla_status_str(status).decode()


def mla_last_hip_error() -> int:
    return int(_lib().mla_last_hip_error())


def mla_version() -> int:
    return int(_lib().mla_version())
