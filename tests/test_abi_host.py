"""Host-side checks of the C ABI: no GPU needed, no kernel is ever launched.

Every call below fails validation (or is host-only planning), so it returns before the
library makes any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from mla_latent_kv_lat_amd import build, capi as L, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

A = 1 << 20  # a fake, 16-byte aligned "device address": never dereferenced on these paths


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(L.LIB_PATH):
        build.build()
    return L.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def test_status_strings_and_version():
    for s in range(5):
        assert L.mla_status_str(s).startswith("MLA_")
    assert "unknown" in L.mla_status_str(99)
    assert L.mla_version() >= 100
    assert L.mla_last_hip_error() == 0


def v2(**kw):
    c = configs.V2_DECODE
    base = dict(batch=c.batch, q_len=c.q_len, n_heads=c.n_heads, d_head=c.d_head,
                d_latent=c.d_latent, d_rope=c.d_rope, softmax_scale=c.softmax_scale)
    base.update(kw)
    return L.dims(**base)


BAD_DIMS = [dict(batch=0), dict(q_len=0), dict(q_len=9), dict(n_heads=0), dict(d_head=0),
            dict(d_latent=0), dict(d_rope=-1), dict(softmax_scale=0.0),
            dict(softmax_scale=float("nan")), dict(softmax_scale=float("inf")),
            dict(softmax_scale=-1.0), dict(split_tokens=-5)]


@pytest.mark.parametrize("bad", BAD_DIMS)
def test_bad_dims_rejected_everywhere(bad):
    d = v2(**bad)
    bf = "bf16"
    assert L.mla_absorb_q(d, A, A, A, dtype=bf, check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_absorb_out(d, A, A, A, dtype=bf, check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_decode(d, A, A, A, A, 4096, None, A, None, A, 1 << 30, q_dtype=bf, kv_dtype=bf,
                        check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_decode_paged(d, A, A, A, A, A, A, 4096, A, None, A, 1 << 30, block_size=64,
                              n_blocks=64, max_blocks_per_seq=64, q_dtype=bf, kv_dtype=bf,
                              check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_decode_workspace_bytes(d, "bf16", 4096) == 0
    assert L.mla_decode_plan(d, "bf16", 4096, check=False)[0] == L.MLA_ERR_INVALID_ARG


def test_null_dims_pointer(lib):
    f = lib.mla_absorb_q
    assert f(None, A, 1, A, 1, A, 1, None) == L.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_workspace_bytes(None, 1, 4096) == 0


def test_absorb_argument_errors():
    d = v2()
    assert L.mla_absorb_q(d, 0, A, A, dtype="bf16", check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_absorb_q(d, A, 0, A, dtype="bf16", check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_absorb_q(d, A, A, 0, dtype="bf16", check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_absorb_q(d, A + 2, A, A, dtype="bf16", check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_absorb_out(d, A, A + 8, A, dtype="bf16", check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_absorb_q(d, A, A, A, dtype="fp8", check=False) == L.MLA_ERR_UNSUPPORTED
    assert L.mla_absorb_q(d, A, A, A, dtype=7, check=False) == L.MLA_ERR_INVALID_ARG
    # mixed dtypes
    lib = L.library()
    st = lib.mla_absorb_q(ctypes.byref(d), ctypes.c_void_p(A), L.MLA_BF16, ctypes.c_void_p(A),
                          L.MLA_F32, ctypes.c_void_p(A), L.MLA_BF16, None)
    assert st == L.MLA_ERR_UNSUPPORTED


def _decode(d, **kw):
    args = dict(q_lat=A, q_rope=A, c_kv=A, k_rope=A, T=4096, seq_lens=None, o_lat=A, lse=None,
                workspace=A, workspace_bytes=1 << 30, q_dtype="bf16", kv_dtype="bf16")
    args.update(kw)
    return L.mla_decode(d, args.pop("q_lat"), args.pop("q_rope"), args.pop("c_kv"), args.pop("k_rope"),
                        args.pop("T"), args.pop("seq_lens"), args.pop("o_lat"), args.pop("lse"),
                        args.pop("workspace"), args.pop("workspace_bytes"), check=False, **args)


def test_decode_argument_errors():
    d = v2(split_tokens=512)
    E, U, W = L.MLA_ERR_INVALID_ARG, L.MLA_ERR_UNSUPPORTED, L.MLA_ERR_WORKSPACE
    assert _decode(d, q_lat=0) == E
    assert _decode(d, c_kv=0) == E
    assert _decode(d, o_lat=0) == E
    assert _decode(d, q_rope=0) == E          # d_r > 0 needs the RoPE query
    assert _decode(d, k_rope=0) == E
    assert _decode(d, T=0) == E
    assert _decode(d, c_kv=A + 4) == E        # misaligned
    assert _decode(d, lse=A + 2) == E
    assert _decode(d, seq_lens=A + 1) == E
    assert _decode(d, kv_dtype="fp8") == E    # fp8 cache without its scale
    assert _decode(d, kv_scale=A) == E        # scale given for a bf16 cache
    assert _decode(d, q_dtype="fp8", kv_dtype="fp8", kv_scale=A) == U
    assert _decode(d, q_dtype="f32", kv_dtype="bf16") == U
    assert _decode(d, q_dtype="bf16", kv_dtype="f32") == U
    assert _decode(v2(d_latent=4096)) == U
    need = L.mla_decode_workspace_bytes(d, "bf16", 4096)
    assert need > 0
    assert _decode(d, workspace=None, workspace_bytes=0) == W
    assert _decode(d, workspace_bytes=need - 1) == W
    assert _decode(d, workspace=A + 16, workspace_bytes=need) == W   # not 256-byte aligned


def test_decode_without_rope_needs_no_rope_pointers():
    d = v2(d_rope=0, split_tokens=512)
    # Passes validation up to the workspace check, which fails on purpose (a split plan
    # needs a workspace), so nothing is launched.
    assert L.mla_decode_workspace_bytes(d, "bf16", 4096) > 0
    assert _decode(d, q_rope=0, k_rope=0, workspace=None, workspace_bytes=0) == L.MLA_ERR_WORKSPACE


def test_paged_argument_errors():
    d = v2(split_tokens=1024)
    need = L.mla_decode_workspace_bytes(d, "bf16", 16384)

    def call(**kw):
        a = dict(block_table=A, seq_lens=A, max_seq_len=16384, block_size=64, n_blocks=100,
                 max_blocks_per_seq=256, workspace=A, workspace_bytes=need)
        a.update(kw)
        return L.mla_decode_paged(d, A, A, A, A, a.pop("block_table"), a.pop("seq_lens"),
                                  a.pop("max_seq_len"), A, None, a.pop("workspace"),
                                  a.pop("workspace_bytes"), q_dtype="bf16", kv_dtype="bf16",
                                  check=False, **a)

    E = L.MLA_ERR_INVALID_ARG
    assert call(block_table=0) == E
    assert call(seq_lens=0) == E
    assert call(block_size=0) == E
    assert call(n_blocks=0) == E
    assert call(max_blocks_per_seq=0) == E
    assert call(max_seq_len=0) == E
    assert call(max_blocks_per_seq=255) == E  # 64 * 255 < 16384
    assert call(block_table=A + 2) == E
    assert call(workspace_bytes=need - 256) == L.MLA_ERR_WORKSPACE


def test_utility_argument_errors():
    E = L.MLA_ERR_INVALID_ARG
    g = L.mla_gather_pages
    kw = dict(block_size=64, n_blocks=10, row_bytes=1152, batch=2, max_blocks_per_seq=4, check=False)
    assert g(0, A, A, 256, A, **kw) == E
    assert g(A, A, A, 256, 0, **kw) == E
    assert g(A, A, A, 256, A, **{**kw, "row_bytes": 6}) == E
    assert g(A, A, A, 300, A, **kw) == E      # 64 * 4 < 300
    assert L.mla_fp8_e4m3_table(0, check=False) == E


@pytest.mark.parametrize("cfg", configs.ALL, ids=lambda c: c.name)
def test_plan_covers_the_context(cfg):
    d = L.dims_from_config(cfg)
    n, tok = L.mla_decode_plan(d, cfg.kv_dtype, cfg.seq_len)
    ws = L.mla_decode_workspace_bytes(d, cfg.kv_dtype, cfg.seq_len)
    rows = cfg.q_len * cfg.n_heads
    r = lambda x: (x + 255) // 256 * 256
    # The matrix-core paths (bf16 queries, d_c 512, d_r 64) balance the batch's tiles over n
    # ranges on the device (tok = 0): one range per compute unit and row block (128 query
    # rows for a bf16 cache of sequences up to at least 8192 tokens, or with rows a
    # multiple of 32 but not of 64; otherwise 64, which needs rows a multiple of 64; 256
    # compute units planned for when no device is present), two bf16 partial slots per
    # range, plus the [B + 1] int64 tile prefix.
    mfma = cfg.act_dtype == "bf16" and cfg.d_latent == 512 and cfg.d_rope == 64 and (
        (cfg.kv_dtype == "bf16" and rows % 32 == 0) or (cfg.kv_dtype == "fp8" and rows % 64 == 0))
    if mfma:
        row_block = 128 if cfg.kv_dtype == "bf16" and (cfg.seq_len >= 8192 or rows % 64) else 64
        assert tok == 0 and n == max(1, 256 // ((rows + row_block - 1) // row_block))
        assert ws == r((cfg.batch + 1) * 8) + r(n * 2 * rows * cfg.d_latent * 2) + r(n * 2 * rows * 4)
        return
    assert n >= 1 and tok >= 1
    assert (n - 1) * tok < cfg.seq_len <= n * tok
    if n == 1:
        assert ws == 0
    else:
        po = cfg.batch * n * rows * cfg.d_latent * 4
        pl = cfg.batch * n * rows * 4
        assert ws == r(po) + r(pl)


def test_plan_honours_split_tokens():
    cfg = configs.LONG_CONTEXT
    for st in (1, 100, 4096, 200000):
        d = L.dims_from_config(cfg, split_tokens=st)
        n, tok = L.mla_decode_plan(d, "bf16", cfg.seq_len)
        assert tok >= st and (n - 1) * tok < cfg.seq_len <= n * tok


# ---- cache write and query rotation: argument checks (no launch) ----------------------

def append_call(d=None, **kw):
    """mla_cache_append with fake device addresses; every case below fails validation."""
    args = dict(d_model=5120, x=A, w_dkv=A, w_kr=A, x_dt=L.MLA_BF16, base=10000.0, pairing=0,
                c_pool=A, kv_dt=L.MLA_BF16, scale_pool=None, rope_pool=A, n_blocks=100, bs=64,
                table=A, max_blocks=64, seq_lens=A, ws=None, ws_bytes=0)
    args.update(kw)
    d = d or v2()
    return L.library().mla_cache_append(
        ctypes.byref(d), args["d_model"], args["x"], args["w_dkv"], args["w_kr"], args["x_dt"],
        args["base"], args["pairing"], args["c_pool"], args["kv_dt"], args["scale_pool"],
        args["rope_pool"], args["n_blocks"], args["bs"], args["table"], args["max_blocks"],
        args["seq_lens"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=0), L.MLA_ERR_INVALID_ARG),
    (dict(pairing=2), L.MLA_ERR_INVALID_ARG),
    (dict(base=1.0), L.MLA_ERR_INVALID_ARG),
    (dict(base=float("nan")), L.MLA_ERR_INVALID_ARG),
    (dict(x=None), L.MLA_ERR_INVALID_ARG),
    (dict(w_kr=None), L.MLA_ERR_INVALID_ARG),
    (dict(table=None), L.MLA_ERR_INVALID_ARG),
    (dict(bs=0), L.MLA_ERR_INVALID_ARG),
    (dict(x=A + 8), L.MLA_ERR_INVALID_ARG),
    (dict(x_dt=L.MLA_FP8_E4M3), L.MLA_ERR_UNSUPPORTED),
    (dict(x_dt=L.MLA_F32), L.MLA_ERR_UNSUPPORTED),          # f32 activations need an f32 cache
    (dict(kv_dt=L.MLA_F32), L.MLA_ERR_UNSUPPORTED),         # bf16 activations, f32 cache
    (dict(kv_dt=L.MLA_FP8_E4M3), L.MLA_ERR_INVALID_ARG),    # fp8 needs the scale pool
    (dict(), L.MLA_ERR_WORKSPACE),                          # no workspace
    (dict(ws=A, ws_bytes=16), L.MLA_ERR_WORKSPACE),         # too small
])
def test_cache_append_argument_errors(kw, status):
    assert append_call(**kw) == status


def test_cache_append_odd_rope_width_rejected():
    assert append_call(d=v2(d_rope=63)) == L.MLA_ERR_INVALID_ARG


def test_cache_append_workspace_formula():
    d = v2()
    # split-K chunks of 256 over d_model, fp32 partial rows of d_c + d_r per new token
    assert L.mla_cache_append_workspace_bytes(d, 5120) == 20 * 32 * 1 * 576 * 4
    assert L.mla_cache_append_workspace_bytes(d, 100) == 1 * 32 * 576 * 4
    assert L.mla_cache_append_workspace_bytes(d, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), L.MLA_ERR_INVALID_ARG),
    (dict(seq_lens=None), L.MLA_ERR_INVALID_ARG),
    (dict(pairing=5), L.MLA_ERR_INVALID_ARG),
    (dict(base=0.5), L.MLA_ERR_INVALID_ARG),
    (dict(dt=L.MLA_FP8_E4M3), L.MLA_ERR_UNSUPPORTED),
    (dict(q=A + 4), L.MLA_ERR_INVALID_ARG),
])
def test_rope_query_argument_errors(kw, status):
    args = dict(q=A, dt=L.MLA_BF16, seq_lens=A, base=10000.0, pairing=0)
    args.update(kw)
    d = v2()
    st = L.library().mla_rope_query(ctypes.byref(d), args["q"], args["dt"], args["seq_lens"], args["base"],
                                    args["pairing"], None)
    assert st == status


def test_fp8_scores_argument():
    """fp8_scores must be 0, 1 or 2, and 1 and 2 need the fp8 cache on the matrix-core kernel
    (same plan as without)."""
    cfg = configs.SPEC_FP8
    for bad in (3, -1):
        assert L.mla_decode_plan(L.dims_from_config(cfg, fp8_scores=bad), "fp8", cfg.seq_len,
                                 check=False)[0] == L.MLA_ERR_INVALID_ARG
    for mode in (1, 2):
        assert L.mla_decode_plan(L.dims_from_config(cfg, fp8_scores=mode), "fp8", cfg.seq_len) == \
            L.mla_decode_plan(L.dims_from_config(cfg), "fp8", cfg.seq_len)
        v2 = configs.V2_DECODE
        assert L.mla_decode_plan(L.dims_from_config(v2, fp8_scores=mode), "bf16", v2.seq_len,
                                 check=False)[0] == L.MLA_ERR_UNSUPPORTED
        small = cfg.with_(n_heads=8)  # general kernel
        assert L.mla_decode_plan(L.dims_from_config(small, fp8_scores=mode), "fp8", small.seq_len,
                                 check=False)[0] == L.MLA_ERR_UNSUPPORTED


def test_prefill_workspace_and_argument_errors():
    """mla_prefill: workspace formula, and every rejected argument returns before a launch."""
    r = lambda x: (x + 255) // 256 * 256
    d = v2(batch=2, q_len=300, n_heads=8)
    assert L.mla_prefill_workspace_bytes(d, 300) == r(8 * 256 * 512 * 2) + r(2 * 300 * 8 * 256 * 2)
    assert L.mla_prefill_workspace_bytes(d, 299) == 0            # q_len > T
    assert L.mla_prefill_workspace_bytes(v2(d_head=64), 300) == 0  # no kernel for d_h = 64

    def call(dims=d, T=300, dtype="bf16", ws=A, ws_bytes=1 << 40, **ptrs):
        p = dict(q_nope=A, q_rope=A, c_kv=A, k_rope=A, seq_lens=A, w_uk=A, w_uv=A, out=A, lse=A)
        p.update(ptrs)
        return L.mla_prefill(dims, p["q_nope"], p["q_rope"], p["c_kv"], p["k_rope"], T, p["seq_lens"],
                             p["w_uk"], p["w_uv"], p["out"], p["lse"], ws, workspace_bytes=ws_bytes,
                             dtype=dtype, check=False)

    E, U, W = L.MLA_ERR_INVALID_ARG, L.MLA_ERR_UNSUPPORTED, L.MLA_ERR_WORKSPACE
    assert L.library().mla_prefill_workspace_bytes(None, 300) == 0
    assert call(T=0) == E
    assert call(T=299) == E                      # more queries than rows
    assert call(dims=v2(batch=0)) == E
    assert call(dims=v2(softmax_scale=0.0)) == E
    assert call(dtype="f32") == U
    assert call(dims=v2(d_latent=256)) == U
    assert call(dims=v2(d_rope=32)) == U
    assert call(dims=v2(fp8_scores=1)) == U
    assert call(dims=v2(n_heads=40000)) == U      # 2 n_h column tiles exceed a grid dimension
    # 65536 query blocks of 256 exceed a grid dimension (65535 blocks still fit)
    assert call(dims=v2(batch=1, q_len=65536 * 256, n_heads=1), T=65536 * 256) == U
    assert call(dims=v2(batch=1, q_len=65535 * 256, n_heads=1), T=65535 * 256, ws=None) == W
    for k in ("q_nope", "q_rope", "c_kv", "k_rope", "w_uk", "w_uv", "out"):
        assert call(**{k: None}) == E, k
        assert call(**{k: A + 8}) == E, k         # not 16-byte aligned
    assert call(seq_lens=A + 2) == E
    assert call(lse=A + 2) == E
    need = L.mla_prefill_workspace_bytes(d, 300)
    assert call(ws=None) == W
    assert call(ws_bytes=need - 1) == W
    assert call(ws=A + 16, ws_bytes=need) == W     # not 256-byte aligned


def test_linear_workspace_and_argument_errors():
    assert L.mla_linear_workspace_bytes(32, 5120, 1536) == 32 * 20 * 1536 * 4
    assert L.mla_linear_workspace_bytes(32, 5000, 1536) == 0     # K not a multiple of 256
    assert L.mla_linear_workspace_bytes(32, 5120, 100) == 0      # N not a multiple of 64
    assert L.mla_linear_workspace_bytes(0, 5120, 1536) == 0

    def call(x=A, w=A, y=A, M=32, K=512, N=128, dtype="bf16", ws=A, ws_bytes=1 << 30):
        return L.mla_linear(x, w, y, ws, M=M, K=K, N=N, workspace_bytes=ws_bytes, dtype=dtype, check=False)

    E, U, W = L.MLA_ERR_INVALID_ARG, L.MLA_ERR_UNSUPPORTED, L.MLA_ERR_WORKSPACE
    assert call(M=0) == E and call(K=0) == E and call(N=-64) == E
    assert call(K=300) == U and call(N=100) == U and call(dtype="f32") == U
    assert call(M=32 * 65535 + 1) == U
    for k in ("x", "w", "y"):
        assert call(**{k: None}) == E, k
        assert call(**{k: A + 8}) == E, k
    need = L.mla_linear_workspace_bytes(32, 512, 128)
    assert call(ws=None) == W and call(ws_bytes=need - 1) == W and call(ws=A + 4, ws_bytes=need) == W


def test_binding_rejects_host_tensors():
    # The binding passes tensor addresses to the device code: host tensors are refused
    # before any call into the library.
    import torch
    d = v2()
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="device tensors"):
        L.mla_absorb_q(d, x, A, A, dtype="bf16")
    with pytest.raises(ValueError, match="device tensors"):
        L.mla_linear(A, x, A, A, M=32, K=256, N=64, workspace_bytes=1 << 20, dtype="bf16")


def test_noalloc_decode_validates_before_any_hip_call():
    """mla_decode_noalloc shares mla_decode's checks, and refuses plans whose partial
    results exceed its static array, all before touching the device."""
    bf = "bf16"
    assert L.mla_decode_noalloc(v2(batch=0), A, A, A, A, 4096, None, A, None, q_dtype=bf, kv_dtype=bf,
                                check=False) == L.MLA_ERR_INVALID_ARG
    assert L.mla_decode_noalloc(v2(), A, A, A, A, 0, None, A, None, q_dtype=bf, kv_dtype=bf,
                                check=False) == L.MLA_ERR_INVALID_ARG
    # fp32 caches run the general kernel with fixed splits: 1024 sequences x 32 splits of
    # 64 rows of 512 fp32 partials need 4 GiB of workspace.
    d = L.dims(1024, 1, 64, 128, 512, 64, 0.07, split_tokens=256)
    need = L.mla_decode_workspace_bytes(d, "f32", 8192)
    assert need > L.NOALLOC_SCRATCH_BYTES
    assert L.mla_decode_noalloc(d, A, A, A, A, 8192, None, A, None, q_dtype="f32", kv_dtype="f32",
                                check=False) == L.MLA_ERR_WORKSPACE


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+MLA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("rows", ["128", "64", None])
def test_noalloc_scratch_holds_every_full_size_plan(rows, monkeypatch):
    """The static array of mla_decode_noalloc holds the workspace of every full-size
    workload's plan, on either bf16 matrix-core kernel."""
    if rows:
        monkeypatch.setenv("MLA_DECODE_ROW_BLOCK", rows)
    else:
        monkeypatch.delenv("MLA_DECODE_ROW_BLOCK", raising=False)
    for cfg in (configs.V2_DECODE, configs.PAGED_VARLEN, configs.LONG_CONTEXT, configs.SPEC_FP8):
        ws = L.mla_decode_workspace_bytes(L.dims_from_config(cfg), cfg.kv_dtype, cfg.seq_len)
        assert 0 < ws <= L.NOALLOC_SCRATCH_BYTES, (cfg.name, rows, ws)


@pytest.mark.parametrize("pair", ["0", "1"])
def test_bf16_64_row_kernels_share_the_plan(pair, monkeypatch):
    """Both bf16 kernels with 64-row blocks (paired score waves, or loader/score/output
    roles: MLA_DECODE_PAIR=0) take the same balanced ranges and the same workspace, so the
    combine and the fused output absorption read their partials alike."""
    monkeypatch.setenv("MLA_DECODE_ROW_BLOCK", "64")
    monkeypatch.setenv("MLA_DECODE_PAIR", pair)
    d = L.dims_from_config(configs.V2_DECODE)
    plan = L.mla_decode_plan(d, "bf16", configs.V2_DECODE.seq_len)
    ws = L.mla_decode_workspace_bytes(d, "bf16", configs.V2_DECODE.seq_len)
    monkeypatch.delenv("MLA_DECODE_PAIR")
    assert plan == L.mla_decode_plan(d, "bf16", configs.V2_DECODE.seq_len)
    assert ws == L.mla_decode_workspace_bytes(d, "bf16", configs.V2_DECODE.seq_len)
    assert plan[0] == 256 // 2  # ranges: compute units / row blocks of the 128 heads


def test_fold_output_weights_validates_before_any_hip_call():
    """mla_fold_output_weights rejects unsupported shapes and dtypes, null and misaligned
    pointers without touching the device."""
    f = L._lib().mla_fold_output_weights
    bf, f32 = L.MLA_BF16, L.MLA_F32
    assert f(A, A, A, 128, 512, 128, 5120, f32, None) == L.MLA_ERR_UNSUPPORTED
    assert f(A, A, A, 128, 512, 64, 5120, bf, None) == L.MLA_ERR_UNSUPPORTED   # d_h not 128 / 512
    assert f(A, A, A, 128, 512, 128, 5000, bf, None) == L.MLA_ERR_UNSUPPORTED  # d_model % 64
    assert f(None, A, A, 128, 512, 128, 5120, bf, None) == L.MLA_ERR_INVALID_ARG
    assert f(A + 2, A, A, 128, 512, 128, 5120, bf, None) == L.MLA_ERR_INVALID_ARG
    assert f(A, A, A, 0, 512, 128, 5120, bf, None) == L.MLA_ERR_INVALID_ARG


def test_decode_absorb_out_validates_before_any_hip_call():
    """mla_decode_absorb_out shares mla_decode's checks and rejects a NULL or misaligned
    w_uv or out, all before touching the device."""
    f = L._lib().mla_decode_absorb_out
    bf = L.MLA_BF16
    d = v2()
    ws = 1 << 30

    def call(w_uv=A, out=A, dims=d):
        return f(ctypes.byref(dims), A, A, bf, A, bf, None, A, bf, 4096, None, w_uv, A, None, out, A, ws, None)
    assert call(w_uv=None) == L.MLA_ERR_INVALID_ARG
    assert call(out=None) == L.MLA_ERR_INVALID_ARG
    assert call(w_uv=A + 2) == L.MLA_ERR_INVALID_ARG
    assert call(out=A + 8) == L.MLA_ERR_INVALID_ARG
    assert call(dims=v2(batch=0)) == L.MLA_ERR_INVALID_ARG
