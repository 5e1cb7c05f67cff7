// Cache write of the new tokens and the query's rotary embedding.
//
// The latent is the only KV state an MLA layer caches ("Operator Notes (1): MLA",
// section 2, c_kv = x . W_DKV); next to it sits the small decoupled key that carries the
// rotary position ("multi-head latent attention" glossary entry, paragraph on the
// decoupled RoPE key).  Per new token: c = x . W_DKV, kr = RoPE(x . W_KR, position), both
// stored at the token's row of the paged pool (fp8 caches store per-token scaled e4m3
// codes of c).
//
// A split-K projection (the few rows of a decode step against the two weight matrices,
// fp32 partial sums per 256-wide K chunk, so that many workgroups stream the weights), then
// a finalize kernel per row that sums the partials, rotates the key, encodes and scatters.
// bf16 projections with d_model a multiple of 256 and d_c, d_r multiples of 64 run on the
// matrix-core per-head kernel (the K chunks as heads); the rest on a VALU kernel (one lane
// per output column, 8 rows per wave).  Partials: [M, chunks, d_c] then [M, chunks, d_r].
#include <algorithm>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kPN = 64;   // output columns per projection workgroup (one per lane)
constexpr int kPM = 32;   // rows per projection workgroup (8 per wave)
constexpr int kPK = 256;  // K per projection workgroup (one split-K chunk)

// part_c[m][kc][n] (n < dc) and part_r[m][kc][n - dc] = sum_{k in chunk kc} x[m][k] * W[k][n],
// W = [w_dkv | w_kr].
template <typename S>
__global__ __launch_bounds__(256) void proj_partial_kernel(const typename S::raw* __restrict__ x,
                                                           const typename S::raw* __restrict__ w_dkv,
                                                           const typename S::raw* __restrict__ w_kr,
                                                           int M, int K, int dc, int dr,
                                                           float* __restrict__ part_c, float* __restrict__ part_r) {
  const int N = dc + dr;
  const int KC = gridDim.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = blockIdx.x * kPN + lane;
  const int nc = min(n, N - 1);  // lanes past the last column read a valid one, store nothing
  const int kc = blockIdx.y, k0 = kc * kPK, k1 = min(K, k0 + kPK);
  const int m0 = blockIdx.z * kPM + 8 * wv;
  const typename S::raw* wcol = nc < dc ? w_dkv + nc : w_kr + (nc - dc);
  const int ws = nc < dc ? dc : dr;
  int64_t xrow[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) xrow[r] = int64_t(min(m0 + r, M - 1)) * K;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int k = k0; k < k1; ++k) {
    const float wk = load_as_f32<S>(wcol, int64_t(k) * ws);
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = fmaf(load_as_f32<S>(x, xrow[r] + k), wk, acc[r]);
  }
  if (n < N) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (m0 + r < M) {
        if (n < dc) part_c[(int64_t(m0 + r) * KC + kc) * dc + n] = acc[r];
        else part_r[(int64_t(m0 + r) * KC + kc) * dr + (n - dc)] = acc[r];
      }
  }
}

// cos / sin of position * base^(-2j / d_r) for rotation pair j, in double precision:
// positions reach 10^5 and more, where a float angle would be off by several milliradians.
__device__ __forceinline__ void rope_angle(int pos, int j, int dr, float base, float& c, float& s) {
  const double inv = exp2(-2.0 * double(j) / double(dr) * log2(double(base)));
  double sd, cd;
  sincos(double(pos) * inv, &sd, &cd);
  c = float(cd);
  s = float(sd);
}

// Element indices of rotation pair j.
__device__ __forceinline__ void rope_pair(int j, int dr, int pairing, int& ia, int& ib) {
  if (pairing == MLA_ROPE_INTERLEAVED) {
    ia = 2 * j;
    ib = 2 * j + 1;
  } else {
    ia = j;
    ib = j + dr / 2;
  }
}

// Two workgroups per new token (grid y): y = 0 sums the latent's split-K partials (one
// thread per column, every chunk's load in flight at once), encodes the row and writes it
// to the token's pool row; y = 1 does the same for the RoPE key and rotates it, its angle
// (double-precision arithmetic) computed while its partial loads are in flight.
constexpr int kFinBatch = 32;  // split-K chunks summed per batch of loads (d_model 5120: 20 chunks)

__device__ __forceinline__ float sum_chunks(const float* src, int stride, int KC) {
  float s = 0.f;
  for (int k0 = 0; k0 < KC; k0 += kFinBatch) {
    float v[kFinBatch];
#pragma unroll
    for (int k = 0; k < kFinBatch; ++k) v[k] = k0 + k < KC ? src[int64_t(k0 + k) * stride] : 0.f;
#pragma unroll
    for (int k = 0; k < kFinBatch; ++k) s += v[k];
  }
  return s;
}

template <typename XS, typename KVS>
__global__ __launch_bounds__(1024) void append_finalize_kernel(const float* __restrict__ part_c,
                                                               const float* __restrict__ part_r, int KC, int M,
                                                               int sq, int dc, int dr, float base, int pairing,
                                                               void* c_pool, float* scale_pool, void* rope_pool,
                                                               int bs, const int32_t* __restrict__ table,
                                                               int max_blocks, const int32_t* __restrict__ seq_lens) {
  extern __shared__ float rowv[];  // latent: one slot per wave for the max; key: its d_r sums
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int b = m / sq, i = m - b * sq;
  // The token's pool row (a length load, then a block-table load) is looked up while the
  // partial sums' loads are in flight; a sequence shorter than its new tokens (pos < 0) is
  // skipped after them (uniform per workgroup, before any barrier or store).
  auto pool_row = [&](int& pos) {
    pos = seq_lens[b] - sq + i;
    return pos < 0 ? int64_t(-1) : int64_t(table[int64_t(b) * max_blocks + pos / bs]) * bs + pos % bs;
  };
  if (blockIdx.y == 1) {
    // RoPE key: thread n owns column n (threads past d_r only take part in the barrier).
    const bool own = tid < dr;
    const int n = own ? tid : 0;
    float c = 1.f, sn = 0.f;
    int partner = n;
    bool first = true;
    const float* src = part_r + int64_t(m) * KC * dr + n;
    float v[kFinBatch];
    const bool one_batch = KC <= kFinBatch;
    if (one_batch) {
#pragma unroll
      for (int k = 0; k < kFinBatch; ++k) v[k] = own && k < KC ? src[int64_t(k) * dr] : 0.f;
    }
    int pos;
    const int64_t prow = pool_row(pos);
    if (pos < 0) return;
    if (own) {
      // Pair j of the rotation holds elements ia, ib; this column is one of them.
      const int j = pairing == MLA_ROPE_INTERLEAVED ? n / 2 : (n < dr / 2 ? n : n - dr / 2);
      int ia, ib;
      rope_pair(j, dr, pairing, ia, ib);
      first = n == ia;
      partner = first ? ib : ia;
      rope_angle(pos, j, dr, base, c, sn);
    }
    float s = 0.f;
    if (one_batch) {
#pragma unroll
      for (int k = 0; k < kFinBatch; ++k) s += v[k];
    } else if (own) {
      s = sum_chunks(src, dr, KC);
    }
    if (own) rowv[n] = s;
    __syncthreads();
    if (own) {
      const float xp = rowv[partner];
      const float r = first ? s * c - xp * sn : xp * sn + s * c;
      using XR = typename XS::raw;
      store_from_f32<XS>(static_cast<XR*>(rope_pool) + prow * dr, n, r);
    }
    return;
  }
  // Latent row: thread n owns columns n, n + blockDim.x, ...
  float* red = rowv;
  float amax = 0.f;
  constexpr int kCols = 2;  // columns per thread kept in registers (d_c <= 2 blockDim.x)
  float sv[kCols];
  int pos;
  int64_t prow = -1;
#pragma unroll
  for (int q = 0; q < kCols; ++q) {
    const int n = tid + q * int(blockDim.x);
    if (q == 0 && KC <= kFinBatch) {
      // One batch: issue the loads, then look up the row while they are in flight.
      float v[kFinBatch];
#pragma unroll
      for (int k = 0; k < kFinBatch; ++k)
        v[k] = n < dc && k < KC ? part_c[(int64_t(m) * KC + k) * dc + n] : 0.f;
      prow = pool_row(pos);
      float t = 0.f;
#pragma unroll
      for (int k = 0; k < kFinBatch; ++k) t += v[k];
      sv[q] = t;
    } else {
      sv[q] = n < dc ? sum_chunks(part_c + int64_t(m) * KC * dc + n, dc, KC) : 0.f;
    }
    if (n < dc) amax = fmaxf(amax, fabsf(sv[q]));
  }
  if (KC > kFinBatch) prow = pool_row(pos);
  if (pos < 0) return;
  if constexpr (sizeof(typename KVS::raw) == 1) {
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < nwaves; ++w) amax = fmaxf(amax, red[w]);
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    if (tid == 0) scale_pool[prow] = scale;
    uint8_t* cp = static_cast<uint8_t*>(c_pool) + prow * dc;
#pragma unroll
    for (int q = 0; q < kCols; ++q) {
      const int n = tid + q * int(blockDim.x);
      if (n < dc) {
        // Nearest-even e4m3fn (OCP) conversion of the gfx950 instruction; |y| <= 448 up to
        // the rounding of the division, clamped so that no code saturates to NaN.
        const float y = fminf(fmaxf(sv[q] / scale, -448.f), 448.f);
        cp[n] = uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFF);
      }
    }
  } else {
    using KR = typename KVS::raw;
    KR* cp = static_cast<KR*>(c_pool) + prow * dc;
#pragma unroll
    for (int q = 0; q < kCols; ++q) {
      const int n = tid + q * int(blockDim.x);
      if (n < dc) store_from_f32<KVS>(cp, n, sv[q]);
    }
  }
}

// q_rope[row, :] rotated in place; row = (b * s_q + i) * H + h, position seq_lens[b] - s_q + i.
template <typename S>
__global__ __launch_bounds__(64) void rope_query_kernel(typename S::raw* q, int sq, int H, int dr, float base,
                                                        int pairing, const int32_t* __restrict__ seq_lens) {
  const int row = blockIdx.x;
  const int bi = row / H, b = bi / sq, i = bi - b * sq;
  const int pos = seq_lens[b] - sq + i;
  typename S::raw* qr = q + int64_t(row) * dr;
  for (int j = threadIdx.x; j < dr / 2; j += 64) {
    int ia, ib;
    rope_pair(j, dr, pairing, ia, ib);
    float c, s;
    rope_angle(pos, j, dr, base, c, s);
    const float xa = load_as_f32<S>(qr, ia), xb = load_as_f32<S>(qr, ib);
    store_from_f32<S>(qr, ia, xa * c - xb * s);
    store_from_f32<S>(qr, ib, xa * s + xb * c);
  }
}

}  // namespace

int64_t cache_append_chunks(int32_t d_model) { return (int64_t(d_model) + kPK - 1) / kPK; }

int launch_cache_append(const CacheAppendArgs& a, hipStream_t s) {
  const int N = a.dc + a.dr;
  const int KC = int(cache_append_chunks(a.d_model));
  float* part_c = a.part;
  float* part_r = a.part + int64_t(a.M) * KC * a.dc;
  const bool mfma = a.x_dt == MLA_BF16 && proj_mfma_supported(a.M, a.d_model, a.dc, kPK) &&
                    (a.dr == 0 || proj_mfma_supported(a.M, a.d_model, a.dr, kPK));
  if (mfma) {
    if (int e = launch_proj_mfma(a.x, a.w_dkv, part_c, a.dc, a.w_kr, part_r, a.dr, a.M, a.d_model, kPK, s))
      return e;
  } else {
    const dim3 grid((N + kPN - 1) / kPN, KC, (a.M + kPM - 1) / kPM);
    if (a.x_dt == MLA_F32)
      hipLaunchKernelGGL(proj_partial_kernel<F32>, grid, dim3(256), 0, s, static_cast<const float*>(a.x),
                         static_cast<const float*>(a.w_dkv), static_cast<const float*>(a.w_kr), a.M, a.d_model,
                         a.dc, a.dr, part_c, part_r);
    else
      hipLaunchKernelGGL(proj_partial_kernel<BF16>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(a.x),
                         static_cast<const uint16_t*>(a.w_dkv), static_cast<const uint16_t*>(a.w_kr), a.M,
                         a.d_model, a.dc, a.dr, part_c, part_r);
    if (int e = int(hipGetLastError())) return e;
  }
  // One thread per latent column (up to 1024; d_c <= 2048 takes two per thread), and at
  // least d_r threads for the key's workgroup.
  const int fin_threads = std::min(1024, (std::max(a.dc, a.dr) + 63) / 64 * 64);
  const size_t lds = sizeof(float) * std::max(a.dr, 16);
#define MLA_FIN(XS, KVS)                                                                                    \
  hipLaunchKernelGGL((append_finalize_kernel<XS, KVS>), dim3(a.M, a.dr > 0 ? 2 : 1), dim3(fin_threads), lds, s, part_c, part_r, KC, a.M, a.sq, \
                     a.dc, a.dr, a.base, a.pairing, a.c_pool, a.scale_pool, a.rope_pool, a.bs, a.table,      \
                     a.max_blocks, a.seq_lens)
  if (a.x_dt == MLA_F32)
    MLA_FIN(F32, F32);
  else if (a.kv_dt == MLA_FP8_E4M3)
    MLA_FIN(BF16, FP8);
  else
    MLA_FIN(BF16, BF16);
#undef MLA_FIN
  return int(hipGetLastError());
}

int launch_rope_query(void* q, mla_dtype dt, int32_t B, int32_t sq, int32_t H, int32_t dr, float base,
                      int32_t pairing, const int32_t* seq_lens, hipStream_t s) {
  const dim3 grid(B * sq * H);
  if (dt == MLA_F32)
    hipLaunchKernelGGL(rope_query_kernel<F32>, grid, dim3(64), 0, s, static_cast<float*>(q), sq, H, dr, base,
                       pairing, seq_lens);
  else
    hipLaunchKernelGGL(rope_query_kernel<BF16>, grid, dim3(64), 0, s, static_cast<uint16_t*>(q), sq, H, dr, base,
                       pairing, seq_lens);
  return int(hipGetLastError());
}

}  // namespace mla
