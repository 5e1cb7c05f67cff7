// Internal host-side interface between the C ABI (mla_api.cpp) and the kernel launchers.
// No device code here, so the validation and planning logic builds as plain C++ too.
#pragma once

#include <cstddef>
#include <cstdint>

#include "mla.h"

typedef struct ihipStream_t* hipStream_t;

namespace mla {

// Which decode kernel family runs a call.
enum class DecodeKernel : int {
  kGeneral = 0,  // VALU kernel for any supported shape (one workgroup per 4 query rows)
  kMfma = 1,     // matrix-core kernel (64 query rows per workgroup): fp8 caches
  kLatent = 2,   // matrix-core kernel (128 query rows per workgroup): bf16 caches
  kPair = 3,     // matrix-core kernel (64 query rows, two score waves per row block): bf16 caches
};

// Split-K plan of one decode call.
struct DecodePlan {
  DecodeKernel kernel;
  int32_t rows;          // s_q * n_h query rows per sequence
  int32_t row_block;     // query rows per workgroup
  int32_t num_splits;    // context splits per sequence (grid dimension)
  int32_t split_tokens;  // tokens per split (multiple of the token tile); 0 when balanced
  bool balanced;         // num_splits ranges of equal work over the whole batch (see below)
  bool part_bf16;        // partial outputs stored as bf16 (else fp32)
  size_t workspace;      // bytes of partial results (0 when num_splits == 1)
  int32_t n_xcd;         // XCDs of the device (work units are spread in contiguous runs)
  int32_t max_prefix_here;  // balanced ranges: largest batch whose tile prefix the decode kernel computes
};

// Topology the plan is made for: the current device's compute units and XCDs (queried once
// per device), or these defaults when no device is present.
constexpr int kDefaultCUs = 256;
constexpr int kDefaultXcds = 8;
constexpr int kLatentMinSeqLen = 8192;  // shortest longest-sequence for the 128-row kernel
void device_topology(int* cus, int* xcds);

// Everything a decode kernel reads or writes.  Pointers are device pointers.
struct DecodeArgs {
  int32_t B, sq, H, dc, dr;
  float scale_log2;      // softmax_scale * log2(e): scores are kept in base-2 units
  const void* q_lat;     // [B, sq, H, dc]
  const void* q_rope;    // [B, sq, H, dr]
  mla_dtype q_dt;
  const void* c_kv;      // [B, T, dc] or pool [n_blocks, block_size, dc]
  mla_dtype kv_dt;
  const float* kv_scale; // [B, T] or pool [n_blocks, block_size] (fp8 only)
  const void* k_rope;    // [B, T, dr] or pool
  int64_t T;             // rows per sequence of a contiguous cache
  const int32_t* seq_lens;  // [B] or nullptr (every sequence has T rows)
  bool paged;
  int32_t block_size;
  const int32_t* block_table;  // [B, max_blocks]
  int32_t max_blocks;
  void* o_lat;           // [B, sq, H, dc], dtype q_dt
  float* lse;            // [B, sq, H] or nullptr
  // Static splits: part_o [B, S, rows, dc], part_lse [B, S, rows].  Balanced ranges:
  // part_o [R, 2, rows, dc], part_lse [R, 2, rows] (a range's first and last piece).
  void* part_o;          // normalised partial outputs, fp32 or bf16
  bool part_bf16;        // element type of part_o
  const int64_t* prefix; // balanced ranges: [B + 1] exclusive prefix sum of 32-token tiles per
                         // sequence (lengths clamped to [0, T]); nullptr for static splits
  bool prefix_here;      // the decode kernel computes and stores prefix itself (small batches)
  int32_t fp8_scores;    // fp8 cache, matrix-core kernel: 1 = latent score term as an fp8
                         // product; 2 = both products fp8 (decode_fp8.hip)
  float* part_lse;       // [B, S, rows] base-2 log-sum-exp of each split (S > 1)
};

// Everything the prefill kernels read or write.  Pointers are device pointers; the shapes
// are d_h = 128, d_c = 512, d_r = 64, bf16.
struct PrefillArgs {
  int32_t B, S, H, T;    // S queries per sequence: the last S of its L rows
  float scale_log2;      // softmax_scale * log2(e)
  const void* q_nope;    // [B, S, H, 128]
  const void* q_rope;    // [B, S, H, 64]
  const void* c_kv;      // [B, T, 512]
  const void* k_rope;    // [B, T, 64]
  const int32_t* seq_lens;  // [B] or nullptr (every sequence has T rows)
  const void* w_uk;      // [H, 128, 512]
  const void* w_uv;      // [H, 512, 128]
  void* out;             // [B, S, H, 128]
  float* lse;            // [B, S, H] or nullptr
  const void* kv;        // set by the launcher: decompressed [B * T, H, 256] in the workspace
};

// Everything the cache-write kernels read or write.  Pointers are device pointers.
struct CacheAppendArgs {
  int32_t M, sq, d_model, dc, dr;   // M = B * s_q new tokens
  const void* x;                    // [M, d_model]
  const void* w_dkv;                // [d_model, dc]
  const void* w_kr;                 // [d_model, dr]
  mla_dtype x_dt, kv_dt;
  float base;
  int32_t pairing;
  void* c_pool;                     // [n_blocks * bs, dc]
  float* scale_pool;                // [n_blocks * bs] (fp8 only)
  void* rope_pool;                  // [n_blocks * bs, dr]
  int32_t bs;
  const int32_t* table;             // [B, max_blocks]
  int32_t max_blocks;
  const int32_t* seq_lens;          // [B]
  float* part;                      // workspace: [M, chunks, dc] then [M, chunks, dr] fp32
};

// Host-only validation and planning (mla_api.cpp).
mla_status check_dims(const mla_dims* d);
// mla_decode's argument checks and plan, and the args of its kernels without a workspace.
mla_status prepare_decode(const mla_dims* d, const void* q_lat, const void* q_rope, mla_dtype q_dt,
                          const void* c_kv, mla_dtype kv_dt, const float* kv_scale, const void* k_rope,
                          mla_dtype rope_dt, int32_t T, const int32_t* seq_lens, void* o_lat,
                          mla_dtype o_dt, float* lse, DecodeArgs* a, DecodePlan* p);
// Points the kernels' partial results at a workspace of ws_bytes bytes (MLA_ERR_WORKSPACE
// when it is missing, too small or not 256-byte aligned).
mla_status attach_workspace(DecodeArgs* a, const DecodePlan& p, void* ws, size_t ws_bytes);
// Enqueues the planned kernels of one decode call on stream s.
mla_status run_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t s, bool combine = true);
// MLA_OK for 0, else MLA_ERR_HIP with the hipError_t kept for mla_last_hip_error().
mla_status hip_error_status(int err);
mla_status plan_decode(const mla_dims* d, mla_dtype q_dt, mla_dtype kv_dt, int32_t max_seq_len,
                       DecodePlan* plan);
bool mfma_decode_eligible(const mla_dims* d, mla_dtype q_dt, mla_dtype kv_dt, int32_t max_seq_len);
bool latent_decode_eligible(const mla_dims* d, mla_dtype q_dt, mla_dtype kv_dt, int32_t max_seq_len);

// Launchers (one per kernel file).  Return the hipError_t of the launch as int.
int launch_decode_general(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
int launch_decode_fp8(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
int launch_decode_latent(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
int launch_decode_pair(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
int launch_combine(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
// The balanced ranges' merge inside the output absorption (decode_general.hip).
bool merge_absorb_fits(const DecodeArgs& a, const DecodePlan& p, int32_t d_h);
int launch_merge_absorb(const DecodeArgs& a, const DecodePlan& p, const void* w_uv, void* out, int32_t d_h,
                        hipStream_t s);
int launch_tile_prefix(const DecodeArgs& a, hipStream_t s);
constexpr int kMaxInKernelPrefixBatch = 1024;  // batches up to this size skip the prefix kernel
int launch_absorb(const void* x, const void* w, void* y, mla_dtype dt, int32_t M, int32_t H,
                  int32_t K, int32_t N, hipStream_t s);
bool absorb_mfma_supported(mla_dtype dt, int32_t M, int32_t K, int32_t N);
int launch_fold_output(const void* w_uv, const void* w_o, void* w_uvo, int32_t n_h, int32_t d_c, int32_t d_h,
                       int32_t d_model, hipStream_t s);
int launch_absorb_mfma(const void* x, const void* w, void* y, int32_t M, int32_t H, int32_t K,
                       int32_t N, hipStream_t s);
int launch_gather_pages(const void* pool, int32_t block_size, int64_t row_bytes,
                        const int32_t* table, int32_t B, int32_t max_blocks, const int32_t* seq_lens,
                        int32_t max_seq_len, void* dst, hipStream_t s);
int launch_fp8_table(float* out, hipStream_t s);
int64_t cache_append_chunks(int32_t d_model);  // split-K chunks of the projection
bool proj_mfma_supported(int32_t M, int32_t K_total, int32_t N, int32_t kchunk);
int launch_proj_mfma(const void* x, const void* w, float* part, int32_t N, const void* w2, float* part2,
                     int32_t N2, int32_t M, int32_t K_total, int32_t kchunk, hipStream_t s);
int launch_cache_append(const CacheAppendArgs& a, hipStream_t s);
int launch_rope_query(void* q, mla_dtype dt, int32_t B, int32_t sq, int32_t H, int32_t dr, float base,
                      int32_t pairing, const int32_t* seq_lens, hipStream_t s);
int launch_fp8_bf16_table(float* out, hipStream_t s);
size_t prefill_workspace_bytes(int32_t B, int32_t T, int32_t H);
int launch_linear(const void* x, const void* w, void* y, int32_t M, int32_t K, int32_t N, float* part,
                  hipStream_t s);
int launch_prefill(PrefillArgs a, void* ws, hipStream_t s);

}  // namespace mla
