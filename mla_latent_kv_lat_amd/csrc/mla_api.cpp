// C ABI of libmla: argument validation, split-K planning and kernel dispatch.
//
// Validation and planning are pure host logic and run before any HIP call, so every
// error path can be exercised on a machine without a GPU.  Launch failures surface as
// MLA_ERR_HIP with the hipError_t kept per thread.
#include <cstdlib>
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxLatent = 2048;      // general-kernel limits (query rows are staged in LDS)
constexpr int kMaxRope = 512;
constexpr int kMaxQLen = 8;
constexpr int kMaxRows = 1 << 16;
constexpr int kMaxGridDim = 65535;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(mla_dtype t) {
  switch (t) {
    case MLA_F32: return 4;
    case MLA_BF16: return 2;
    case MLA_FP8_E4M3: return 1;
  }
  return 0;
}

bool valid_dtype(mla_dtype t) { return t == MLA_F32 || t == MLA_BF16 || t == MLA_FP8_E4M3; }

mla_status hip_status(int err) {
  if (err == 0) return MLA_OK;
  g_last_hip_error = err;
  return MLA_ERR_HIP;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shared argument checks of mla_decode and mla_decode_paged.
mla_status check_decode_common(const mla_dims* d, const void* q_lat, const void* q_rope,
                               mla_dtype q_dt, const void* kv, mla_dtype kv_dt,
                               const float* kv_scale, const void* k_rope, mla_dtype rope_dt,
                               const void* o_lat, mla_dtype o_dt, const float* lse) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!valid_dtype(q_dt) || !valid_dtype(kv_dt) || !valid_dtype(rope_dt) || !valid_dtype(o_dt))
    return MLA_ERR_INVALID_ARG;
  if (!q_lat || !kv || !o_lat) return MLA_ERR_INVALID_ARG;
  if (d->d_rope > 0 && (!q_rope || !k_rope)) return MLA_ERR_INVALID_ARG;
  if ((kv_dt == MLA_FP8_E4M3) != (kv_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (!aligned(q_lat, 16) || !aligned(kv, 16) || !aligned(o_lat, 16)) return MLA_ERR_INVALID_ARG;
  if (q_rope && !aligned(q_rope, 16)) return MLA_ERR_INVALID_ARG;
  if (k_rope && !aligned(k_rope, 16)) return MLA_ERR_INVALID_ARG;
  if (kv_scale && !aligned(kv_scale, 4)) return MLA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return MLA_ERR_INVALID_ARG;
  // Supported dtype sets.
  if (q_dt == MLA_FP8_E4M3 || rope_dt != q_dt || o_dt != q_dt) return MLA_ERR_UNSUPPORTED;
  if (q_dt == MLA_F32 && kv_dt != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (q_dt == MLA_BF16 && kv_dt == MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (d->d_latent > kMaxLatent || d->d_rope > kMaxRope) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

void fill_common(DecodeArgs* a, const mla_dims* d, const void* q_lat, const void* q_rope,
                 mla_dtype q_dt, const void* kv, mla_dtype kv_dt, const float* kv_scale,
                 const void* k_rope, void* o_lat, float* lse) {
  a->B = d->batch;
  a->sq = d->q_len;
  a->H = d->n_heads;
  a->dc = d->d_latent;
  a->dr = d->d_rope;
  a->scale_log2 = d->softmax_scale * 1.4426950408889634f;
  a->q_lat = q_lat;
  a->q_rope = q_rope;
  a->q_dt = q_dt;
  a->c_kv = kv;
  a->kv_dt = kv_dt;
  a->kv_scale = kv_scale;
  a->k_rope = k_rope;
  a->o_lat = o_lat;
  a->lse = lse;
  a->paged = false;
  a->block_size = 0;
  a->block_table = nullptr;
  a->max_blocks = 0;
  a->part_o = nullptr;
  a->part_bf16 = false;
  a->part_lse = nullptr;
  a->prefix = nullptr;
  a->prefix_here = false;
  a->fp8_scores = d->fp8_scores;
}

}  // namespace

mla_status attach_workspace(DecodeArgs* a, const DecodePlan& p, void* ws, size_t ws_bytes) {
  if (p.workspace == 0) return MLA_OK;
  if (!ws || ws_bytes < p.workspace || !aligned(ws, 256)) return MLA_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  size_t o_bytes;
  if (p.balanced) {
    a->prefix = reinterpret_cast<const int64_t*>(w);
    a->prefix_here = a->B <= p.max_prefix_here;
    w += align_up(size_t(a->B + 1) * 8, 256);
    o_bytes = align_up(size_t(p.num_splits) * 2 * p.rows * a->dc * 2, 256);
  } else {
    o_bytes = align_up(size_t(a->B) * p.num_splits * p.rows * a->dc * (p.part_bf16 ? 2 : 4), 256);
  }
  a->part_o = w;
  a->part_bf16 = p.part_bf16;
  a->part_lse = reinterpret_cast<float*>(w + o_bytes);
  return MLA_OK;
}

mla_status run_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t s, bool combine) {
  if (p.balanced && !a.prefix_here) {
    const int err = launch_tile_prefix(a, s);
    if (err) return hip_status(err);
  }
  int err = p.kernel == DecodeKernel::kLatent ? launch_decode_latent(a, p, s)
            : p.kernel == DecodeKernel::kPair   ? launch_decode_pair(a, p, s)
            : p.kernel == DecodeKernel::kMfma   ? (a.fp8_scores ? launch_decode_fp8(a, p, s)
                                                                : launch_decode_mfma(a, p, s))
                                                : launch_decode_general(a, p, s);
  if (err) return hip_status(err);
  if (combine && (p.balanced || p.num_splits > 1)) return hip_status(launch_combine(a, p, s));
  return MLA_OK;
}

mla_status hip_error_status(int err) { return hip_status(err); }

mla_status prepare_decode(const mla_dims* d, const void* q_lat, const void* q_rope, mla_dtype q_dt,
                          const void* c_kv, mla_dtype kv_dt, const float* kv_scale, const void* k_rope,
                          mla_dtype rope_dt, int32_t T, const int32_t* seq_lens, void* o_lat,
                          mla_dtype o_dt, float* lse, DecodeArgs* a, DecodePlan* p) {
  mla_status st = check_decode_common(d, q_lat, q_rope, q_dt, c_kv, kv_dt, kv_scale, k_rope,
                                       rope_dt, o_lat, o_dt, lse);
  if (st != MLA_OK) return st;
  if (T < 1) return MLA_ERR_INVALID_ARG;
  if (seq_lens && !aligned(seq_lens, 4)) return MLA_ERR_INVALID_ARG;
  st = plan_decode(d, q_dt, kv_dt, T, p);
  if (st != MLA_OK) return st;
  fill_common(a, d, q_lat, q_rope, q_dt, c_kv, kv_dt, kv_scale, k_rope, o_lat, lse);
  a->T = T;
  a->seq_lens = seq_lens;
  return MLA_OK;
}

mla_status check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->batch < 1 || d->q_len < 1 || d->q_len > kMaxQLen || d->n_heads < 1 || d->d_head < 1 ||
      d->d_latent < 1 || d->d_rope < 0 || d->split_tokens < 0 || d->fp8_scores < 0 ||
      d->fp8_scores > 2)
    return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (int64_t(d->q_len) * d->n_heads > kMaxRows) return MLA_ERR_UNSUPPORTED;
  // Batch and heads index grid dimensions that hold at most 65535 workgroups.
  if (d->batch > kMaxGridDim || d->n_heads > kMaxGridDim) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

bool latent_decode_eligible(const mla_dims* d, mla_dtype q_dt, mla_dtype kv_dt, int32_t max_seq_len) {
  // 32-bit byte offsets within one sequence's rows, as for the 64-row kernel.
  const int64_t seq_bytes = int64_t(max_seq_len) * 512 * 2;
  return q_dt == MLA_BF16 && kv_dt == MLA_BF16 && d->fp8_scores == 0 && d->d_latent == 512 && d->d_rope == 64 &&
         (d->q_len * d->n_heads) % 32 == 0 && seq_bytes < (int64_t(1) << 31);
}

bool mfma_decode_eligible(const mla_dims* d, mla_dtype q_dt, mla_dtype kv_dt, int32_t max_seq_len) {
  // The matrix-core kernel addresses one sequence's cache rows with 32-bit byte offsets.
  const int64_t seq_bytes = int64_t(max_seq_len) * 512 * (kv_dt == MLA_FP8_E4M3 ? 1 : 2);
  return q_dt == MLA_BF16 && (kv_dt == MLA_BF16 || kv_dt == MLA_FP8_E4M3) && d->d_latent == 512 &&
         d->d_rope == 64 && (d->q_len * d->n_heads) % 64 == 0 && seq_bytes < (int64_t(1) << 31);
}

// The 64-row bf16 decode runs on the paired-score-wave kernel unless the environment
// variable MLA_DECODE_PAIR is "0" (then on the kernel with loader, score and output roles).
static bool pair_enabled() {
  const char* env = std::getenv("MLA_DECODE_PAIR");
  return !(env && env[0] == '0' && env[1] == 0);
}

mla_status plan_decode(const mla_dims* d, mla_dtype q_dt, mla_dtype kv_dt, int32_t max_seq_len,
                       DecodePlan* plan) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (max_seq_len < 1) return MLA_ERR_INVALID_ARG;
  DecodePlan p{};
  p.rows = d->q_len * d->n_heads;
  int num_cus = kDefaultCUs, n_xcd = kDefaultXcds;
  device_topology(&num_cus, &n_xcd);
  p.n_xcd = n_xcd;
  int tile, min_chunk;
  // Kernel choice for bf16 caches: the 128-row kernel halves how often a cache row is
  // read per sequence but splits each sequence into twice as many ranges, whose merge
  // costs a fixed few microseconds; it wins once sequences are long.  MLA_DECODE_ROW_BLOCK
  // (64 or 128) overrides the length rule.
  const char* rb_env = std::getenv("MLA_DECODE_ROW_BLOCK");
  const int rb_force = rb_env ? std::atoi(rb_env) : 0;
  const bool old_ok = mfma_decode_eligible(d, q_dt, kv_dt, max_seq_len);
  const bool want_latent =
      rb_force == 128 || (rb_force != 64 && (max_seq_len >= kLatentMinSeqLen || !old_ok));
  if (want_latent && latent_decode_eligible(d, q_dt, kv_dt, max_seq_len)) {
    p.kernel = DecodeKernel::kLatent;
    p.row_block = 128;
    p.max_prefix_here = 64;
    tile = 64;
    min_chunk = 512;
  } else if (old_ok && kv_dt == MLA_BF16 && d->fp8_scores == 0 && pair_enabled()) {
    // bf16 caches: the 64-row kernel with two score waves per row block (it computes the
    // tile prefix itself for up to 64 sequences).
    p.kernel = DecodeKernel::kPair;
    p.row_block = 64;
    p.max_prefix_here = 64;
    tile = 64;
    min_chunk = 512;
  } else if (old_ok) {
    p.kernel = DecodeKernel::kMfma;
    p.row_block = 64;
    p.max_prefix_here = kMaxInKernelPrefixBatch;
    tile = 64;
    min_chunk = 512;
  } else {
    p.kernel = DecodeKernel::kGeneral;
    p.row_block = 4;
    tile = 256;
    min_chunk = 256;
  }
  if (d->fp8_scores && (p.kernel != DecodeKernel::kMfma || kv_dt != MLA_FP8_E4M3))
    return MLA_ERR_UNSUPPORTED;
  const int64_t units = int64_t(d->batch) * ceil_div(p.rows, p.row_block);
  // The matrix-core paths store their normalised partial outputs as bf16: they are combined
  // into a bf16 output, and halving them halves the extra traffic of splitting.
  p.part_bf16 = p.kernel != DecodeKernel::kGeneral;
  if (d->split_tokens == 0 && p.kernel != DecodeKernel::kGeneral) {
    // Balanced ranges: the 32-token tiles of the whole batch (per row block) are divided
    // into num_splits contiguous ranges of equal size on the device, from the actual
    // sequence lengths, so that ragged batches keep every compute unit busy.  Each range
    // runs on one workgroup per row block; a sequence cut by range boundaries is merged
    // afterwards.
    const int64_t rblocks = ceil_div(p.rows, p.row_block);
    const int64_t ranges = std::max<int64_t>(1, num_cus / rblocks);
    p.balanced = true;
    p.num_splits = int32_t(ranges);
    p.split_tokens = 0;
    p.workspace = align_up(size_t(d->batch + 1) * 8, 256) +
                  align_up(size_t(ranges) * 2 * p.rows * d->d_latent * 2, 256) +
                  align_up(size_t(ranges) * 2 * p.rows * 4, 256);
    *plan = p;
    return MLA_OK;
  }
  int64_t chunk;
  if (d->split_tokens > 0) {
    chunk = ceil_div(d->split_tokens, tile) * tile;
  } else {
    // Enough workgroups to give every compute unit at least one, without making a split
    // so short that its partial result costs more traffic than its share of the cache.
    const int64_t want_splits = ceil_div(num_cus, units);
    chunk = ceil_div(ceil_div(max_seq_len, want_splits), tile) * tile;
    if (chunk < min_chunk) chunk = min_chunk;
  }
  const int64_t splits = ceil_div(max_seq_len, chunk);
  if (splits > 8192 || chunk > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  p.num_splits = int32_t(splits);
  p.split_tokens = int32_t(chunk);
  if (p.num_splits > 1) {
    p.workspace = align_up(size_t(d->batch) * splits * p.rows * d->d_latent * (p.part_bf16 ? 2 : 4), 256) +
                  align_up(size_t(d->batch) * splits * p.rows * 4, 256);
  }
  *plan = p;
  return MLA_OK;
}

}  // namespace mla

using namespace mla;

extern "C" {

mla_status mla_absorb_q(const mla_dims* d, const void* q_nope, mla_dtype q_dt, const void* w_uk,
                        mla_dtype w_dt, void* q_lat, mla_dtype out_dt, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!valid_dtype(q_dt) || !valid_dtype(w_dt) || !valid_dtype(out_dt)) return MLA_ERR_INVALID_ARG;
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_INVALID_ARG;
  if (!aligned(q_nope, 16) || !aligned(w_uk, 16) || !aligned(q_lat, 16)) return MLA_ERR_INVALID_ARG;
  if (q_dt != w_dt || q_dt != out_dt || q_dt == MLA_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  return hip_status(launch_absorb(q_nope, w_uk, q_lat, q_dt, d->batch * d->q_len, d->n_heads,
                                  d->d_head, d->d_latent, static_cast<hipStream_t>(stream)));
}

mla_status mla_absorb_out(const mla_dims* d, const void* o_lat, mla_dtype in_dt, const void* w_uv,
                          mla_dtype w_dt, void* out, mla_dtype out_dt, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!valid_dtype(in_dt) || !valid_dtype(w_dt) || !valid_dtype(out_dt)) return MLA_ERR_INVALID_ARG;
  if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned(o_lat, 16) || !aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_INVALID_ARG;
  if (in_dt != w_dt || in_dt != out_dt || in_dt == MLA_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  return hip_status(launch_absorb(o_lat, w_uv, out, in_dt, d->batch * d->q_len, d->n_heads,
                                  d->d_latent, d->d_head, static_cast<hipStream_t>(stream)));
}

size_t mla_cache_append_workspace_bytes(const mla_dims* d, int32_t d_model) {
  if (check_dims(d) != MLA_OK || d_model < 1) return 0;
  return size_t(cache_append_chunks(d_model)) * size_t(d->batch) * d->q_len *
         (size_t(d->d_latent) + d->d_rope) * sizeof(float);
}

mla_status mla_cache_append(const mla_dims* d, int32_t d_model, const void* x, const void* w_dkv,
                            const void* w_kr, mla_dtype x_dt, float rope_base, mla_rope_pairing pairing,
                            void* c_kv_pool, mla_dtype kv_dt, float* kv_scale_pool, void* k_rope_pool,
                            int32_t n_blocks, int32_t block_size, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, void* workspace,
                            size_t workspace_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d_model < 1 || !valid_dtype(x_dt) || !valid_dtype(kv_dt)) return MLA_ERR_INVALID_ARG;
  if (pairing != MLA_ROPE_INTERLEAVED && pairing != MLA_ROPE_HALF) return MLA_ERR_INVALID_ARG;
  if (d->d_rope % 2 != 0) return MLA_ERR_INVALID_ARG;
  if (d->d_rope > 0 && (!(rope_base > 1.f) || !std::isfinite(rope_base))) return MLA_ERR_INVALID_ARG;
  if (!x || !w_dkv || !c_kv_pool || !block_table || !seq_lens) return MLA_ERR_INVALID_ARG;
  if (d->d_rope > 0 && (!w_kr || !k_rope_pool)) return MLA_ERR_INVALID_ARG;
  if (n_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_dkv, 16) || (w_kr && !aligned(w_kr, 16)) || !aligned(c_kv_pool, 16) ||
      (k_rope_pool && !aligned(k_rope_pool, 16)) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return MLA_ERR_INVALID_ARG;
  if (x_dt == MLA_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (x_dt == MLA_F32 ? kv_dt != MLA_F32 : kv_dt == MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (kv_dt == MLA_FP8_E4M3 && (!kv_scale_pool || !aligned(kv_scale_pool, 4))) return MLA_ERR_INVALID_ARG;
  const int64_t M = int64_t(d->batch) * d->q_len;
  if ((M + 31) / 32 > kMaxGridDim || cache_append_chunks(d_model) > kMaxGridDim) return MLA_ERR_UNSUPPORTED;
  const size_t need = mla_cache_append_workspace_bytes(d, d_model);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return MLA_ERR_WORKSPACE;
  CacheAppendArgs a;
  a.M = int32_t(M);
  a.sq = d->q_len;
  a.d_model = d_model;
  a.dc = d->d_latent;
  a.dr = d->d_rope;
  a.x = x;
  a.w_dkv = w_dkv;
  a.w_kr = w_kr;
  a.x_dt = x_dt;
  a.kv_dt = kv_dt;
  a.base = rope_base;
  a.pairing = int32_t(pairing);
  a.c_pool = c_kv_pool;
  a.scale_pool = kv_scale_pool;
  a.rope_pool = k_rope_pool;
  a.bs = block_size;
  a.table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.part = static_cast<float*>(workspace);
  return hip_status(launch_cache_append(a, static_cast<hipStream_t>(stream)));
}

mla_status mla_rope_query(const mla_dims* d, void* q_rope, mla_dtype q_dt, const int32_t* seq_lens,
                          float rope_base, mla_rope_pairing pairing, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!valid_dtype(q_dt) || !q_rope || !seq_lens) return MLA_ERR_INVALID_ARG;
  if (pairing != MLA_ROPE_INTERLEAVED && pairing != MLA_ROPE_HALF) return MLA_ERR_INVALID_ARG;
  if (d->d_rope < 2 || d->d_rope % 2 != 0 || !(rope_base > 1.f) || !std::isfinite(rope_base))
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q_rope, 16) || !aligned(seq_lens, 4)) return MLA_ERR_INVALID_ARG;
  if (q_dt == MLA_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (int64_t(d->batch) * d->q_len * d->n_heads > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  return hip_status(launch_rope_query(q_rope, q_dt, d->batch, d->q_len, d->n_heads, d->d_rope, rope_base,
                                      int32_t(pairing), seq_lens, static_cast<hipStream_t>(stream)));
}

// Prefill shapes: every dimension but the latent-attention ones as in check_dims, any
// q_len up to T.
static mla_status check_prefill(const mla_dims* d, int32_t T, mla_dtype dt) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->batch < 1 || d->q_len < 1 || d->n_heads < 1 || d->d_head < 1 || d->d_latent < 1 ||
      d->d_rope < 0 || d->split_tokens < 0 || d->fp8_scores < 0 || d->fp8_scores > 2 || T < 1 ||
      d->q_len > T)
    return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (!valid_dtype(dt)) return MLA_ERR_INVALID_ARG;
  if (dt != MLA_BF16 || d->d_head != 128 || d->d_latent != 512 || d->d_rope != 64 || d->fp8_scores)
    return MLA_ERR_UNSUPPORTED;
  // Grid limits: the decompression has 2 n_h column tiles, the attention ceil(s_q / 256)
  // query blocks and B sequences in dimensions of at most 65535 workgroups.
  if (d->batch > kMaxGridDim || 2 * int64_t(d->n_heads) > kMaxGridDim ||
      (int64_t(d->q_len) + 255) / 256 > kMaxGridDim || int64_t(d->batch) * T > INT32_MAX)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// Projections: bf16, K a multiple of 256, N a multiple of 64, M in [1, 32 * 65535].
static mla_status check_linear(int32_t M, int32_t K, int32_t N, mla_dtype dt) {
  if (M < 1 || K < 1 || N < 1 || !valid_dtype(dt)) return MLA_ERR_INVALID_ARG;
  if (dt != MLA_BF16 || K % 256 != 0 || N % 64 != 0 || int64_t(M) > 32 * int64_t(kMaxGridDim) ||
      K / 256 > kMaxGridDim || N / 64 > kMaxGridDim || int64_t(M) * N / 8 > int64_t(INT32_MAX) * 256)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

size_t mla_linear_workspace_bytes(int32_t M, int32_t K, int32_t N) {
  if (check_linear(M, K, N, MLA_BF16) != MLA_OK) return 0;
  return size_t(M) * (K / 256) * N * 4;
}

mla_status mla_linear(const void* x, const void* w, void* y, int32_t M, int32_t K, int32_t N, mla_dtype dt,
                      void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_linear(M, K, N, dt);
  if (st != MLA_OK) return st;
  if (!x || !w || !y) return MLA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return MLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < size_t(M) * (K / 256) * N * 4 || !aligned(workspace, 16))
    return MLA_ERR_WORKSPACE;
  return hip_status(launch_linear(x, w, y, M, K, N, static_cast<float*>(workspace),
                                  static_cast<hipStream_t>(stream)));
}

mla_status mla_fold_output_weights(const void* w_uv, const void* w_o, void* w_uvo, int32_t n_h, int32_t d_c,
                                   int32_t d_h, int32_t d_model, mla_dtype dt, void* stream) {
  if (n_h < 1 || d_c < 1 || d_h < 1 || d_model < 1) return MLA_ERR_INVALID_ARG;
  if (dt != MLA_BF16 || !absorb_mfma_supported(dt, d_c, d_h, d_model)) return MLA_ERR_UNSUPPORTED;
  if (!w_uv || !w_o || !w_uvo) return MLA_ERR_INVALID_ARG;
  if (!aligned(w_uv, 16) || !aligned(w_o, 16) || !aligned(w_uvo, 16)) return MLA_ERR_INVALID_ARG;
  return hip_status(launch_fold_output(w_uv, w_o, w_uvo, n_h, d_c, d_h, d_model, static_cast<hipStream_t>(stream)));
}

size_t mla_prefill_workspace_bytes(const mla_dims* d, int32_t T) {
  if (check_prefill(d, T, MLA_BF16) != MLA_OK) return 0;
  return prefill_workspace_bytes(d->batch, T, d->n_heads);
}

mla_status mla_prefill(const mla_dims* d, const void* q_nope, const void* q_rope, const void* c_kv,
                       const void* k_rope, int32_t T, const int32_t* seq_lens, const void* w_uk,
                       const void* w_uv, mla_dtype dt, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  mla_status st = check_prefill(d, T, dt);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_rope || !c_kv || !k_rope || !w_uk || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  for (const void* p : {q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, static_cast<const void*>(out)})
    if (!aligned(p, 16)) return MLA_ERR_INVALID_ARG;
  if ((seq_lens && !aligned(seq_lens, 4)) || (lse && !aligned(lse, 4))) return MLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < prefill_workspace_bytes(d->batch, T, d->n_heads) ||
      !aligned(workspace, 256))
    return MLA_ERR_WORKSPACE;
  PrefillArgs a{};
  a.B = d->batch;
  a.S = d->q_len;
  a.H = d->n_heads;
  a.T = T;
  a.scale_log2 = d->softmax_scale * 1.4426950408889634f;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.seq_lens = seq_lens;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.lse = lse;
  return hip_status(launch_prefill(a, workspace, static_cast<hipStream_t>(stream)));
}

size_t mla_decode_workspace_bytes(const mla_dims* d, mla_dtype kv_dt, int32_t max_seq_len) {
  DecodePlan p;
  mla_dtype q_dt = kv_dt == MLA_F32 ? MLA_F32 : MLA_BF16;
  if (plan_decode(d, q_dt, kv_dt, max_seq_len, &p) != MLA_OK) return 0;
  return p.workspace;
}

mla_status mla_decode_plan(const mla_dims* d, mla_dtype kv_dt, int32_t max_seq_len,
                           int32_t* num_splits, int32_t* split_tokens) {
  if (!valid_dtype(kv_dt)) return MLA_ERR_INVALID_ARG;
  DecodePlan p;
  mla_dtype q_dt = kv_dt == MLA_F32 ? MLA_F32 : MLA_BF16;
  mla_status st = plan_decode(d, q_dt, kv_dt, max_seq_len, &p);
  if (st != MLA_OK) return st;
  if (num_splits) *num_splits = p.num_splits;
  if (split_tokens) *split_tokens = p.split_tokens;
  return MLA_OK;
}

mla_status mla_decode(const mla_dims* d, const void* q_lat, const void* q_rope, mla_dtype q_dt,
                      const void* c_kv, mla_dtype kv_dt, const float* kv_scale, const void* k_rope,
                      mla_dtype rope_dt, int32_t T, const int32_t* seq_lens, void* o_lat,
                      mla_dtype o_dt, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  DecodeArgs a;
  DecodePlan p;
  mla_status st = prepare_decode(d, q_lat, q_rope, q_dt, c_kv, kv_dt, kv_scale, k_rope, rope_dt, T,
                                 seq_lens, o_lat, o_dt, lse, &a, &p);
  if (st != MLA_OK) return st;
  st = attach_workspace(&a, p, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  return run_decode(a, p, static_cast<hipStream_t>(stream));
}

mla_status mla_decode_absorb_out(const mla_dims* d, const void* q_lat, const void* q_rope, mla_dtype q_dt,
                                 const void* c_kv, mla_dtype kv_dt, const float* kv_scale, const void* k_rope,
                                 mla_dtype rope_dt, int32_t T, const int32_t* seq_lens, const void* w_uv,
                                 void* o_lat, float* lse, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  DecodeArgs a;
  DecodePlan p;
  mla_status st = prepare_decode(d, q_lat, q_rope, q_dt, c_kv, kv_dt, kv_scale, k_rope, rope_dt, T, seq_lens,
                                 o_lat, q_dt, lse, &a, &p);
  if (st != MLA_OK) return st;
  if (!w_uv || !out || !aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_INVALID_ARG;
  st = attach_workspace(&a, p, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  const auto s = static_cast<hipStream_t>(stream);
  if (merge_absorb_fits(a, p, d->d_head)) {
    st = run_decode(a, p, s, false);
    if (st != MLA_OK) return st;
    return hip_status(launch_merge_absorb(a, p, w_uv, out, d->d_head, s));
  }
  st = run_decode(a, p, s, true);
  if (st != MLA_OK) return st;
  return mla_absorb_out(d, o_lat, q_dt, w_uv, q_dt, out, q_dt, stream);
}

mla_status mla_decode_paged(const mla_dims* d, const void* q_lat, const void* q_rope,
                            mla_dtype q_dt, const void* c_kv_pool, mla_dtype kv_dt,
                            const float* kv_scale_pool, const void* k_rope_pool, mla_dtype rope_dt,
                            int32_t n_blocks, int32_t block_size, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t max_seq_len, void* o_lat, mla_dtype o_dt, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_decode_common(d, q_lat, q_rope, q_dt, c_kv_pool, kv_dt, kv_scale_pool,
                                       k_rope_pool, rope_dt, o_lat, o_dt, lse);
  if (st != MLA_OK) return st;
  if (n_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1 || max_seq_len < 1)
    return MLA_ERR_INVALID_ARG;
  if (!block_table || !seq_lens || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return MLA_ERR_INVALID_ARG;
  if (int64_t(block_size) * max_blocks_per_seq < max_seq_len) return MLA_ERR_INVALID_ARG;
  DecodePlan p;
  st = plan_decode(d, q_dt, kv_dt, max_seq_len, &p);
  if (st != MLA_OK) return st;
  DecodeArgs a;
  fill_common(&a, d, q_lat, q_rope, q_dt, c_kv_pool, kv_dt, kv_scale_pool, k_rope_pool, o_lat, lse);
  a.T = max_seq_len;
  a.seq_lens = seq_lens;
  a.paged = true;
  a.block_size = block_size;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  st = attach_workspace(&a, p, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  return run_decode(a, p, static_cast<hipStream_t>(stream));
}

mla_status mla_gather_pages(const void* pool, int32_t n_blocks, int32_t block_size, int64_t row_bytes,
                            const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t max_seq_len, void* dst, void* stream) {
  if (!pool || !block_table || !seq_lens || !dst) return MLA_ERR_INVALID_ARG;
  if (n_blocks < 1 || block_size < 1 || row_bytes < 4 || row_bytes % 4 || batch < 1 ||
      max_blocks_per_seq < 1 || max_seq_len < 1)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(pool, 4) || !aligned(dst, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return MLA_ERR_INVALID_ARG;
  if (int64_t(block_size) * max_blocks_per_seq < max_seq_len) return MLA_ERR_INVALID_ARG;
  return hip_status(launch_gather_pages(pool, block_size, row_bytes, block_table, batch,
                                        max_blocks_per_seq, seq_lens, max_seq_len, dst,
                                        static_cast<hipStream_t>(stream)));
}

mla_status mla_fp8_e4m3_table(float* out, void* stream) {
  if (!out || !aligned(out, 4)) return MLA_ERR_INVALID_ARG;
  return hip_status(launch_fp8_table(out, static_cast<hipStream_t>(stream)));
}

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for this dtype/shape";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP launch failed";
  }
  return "unknown mla_status";
}

int mla_last_hip_error(void) { return g_last_hip_error; }

int mla_version(void) { return 100; }

}  // extern "C"
