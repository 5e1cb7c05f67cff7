// Cache write of the new tokens and the query's rotary embedding.
//
// The latent is the only KV state an MLA layer caches ("Operator Notes (1): MLA",
// section 2, c_kv = x . W_DKV); next to it sits the small decoupled key that carries the
// rotary position ("multi-head latent attention" glossary entry, paragraph on the
// decoupled RoPE key).  Per new token: c = x . W_DKV, kr = RoPE(x . W_KR, position), both
// stored at the token's row of the paged pool (fp8 caches store per-token scaled e4m3
// codes of c).
//
// Two kernels: a split-K projection (x rows against the [d_model, d_c + d_r] pair of
// weights; one lane per output column, 8 rows per wave, fp32 partial sums per K chunk,
// so that many workgroups stream the weights for the few rows of a decode step), then a
// finalize kernel per row that sums the partials, rotates the key, encodes and scatters.
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kPN = 64;   // output columns per projection workgroup (one per lane)
constexpr int kPM = 32;   // rows per projection workgroup (8 per wave)
constexpr int kPK = 256;  // K per projection workgroup (one split-K chunk)

// part[kc][m][n] = sum_{k in chunk kc} x[m][k] * W[k][n], W = [w_dkv | w_kr].
template <typename S>
__global__ __launch_bounds__(256) void proj_partial_kernel(const typename S::raw* __restrict__ x,
                                                           const typename S::raw* __restrict__ w_dkv,
                                                           const typename S::raw* __restrict__ w_kr,
                                                           int M, int K, int dc, int dr,
                                                           float* __restrict__ part) {
  const int N = dc + dr;
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
      if (m0 + r < M) part[(int64_t(kc) * M + m0 + r) * N + n] = acc[r];
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

// One wave per new token: sum the split-K partials, rotate the key, encode the latent and
// write both to the token's pool row.
template <typename XS, typename KVS>
__global__ __launch_bounds__(64) void append_finalize_kernel(const float* __restrict__ part, int KC, int M,
                                                             int sq, int dc, int dr, float base, int pairing,
                                                             void* c_pool, float* scale_pool, void* rope_pool,
                                                             int bs, const int32_t* __restrict__ table,
                                                             int max_blocks, const int32_t* __restrict__ seq_lens) {
  extern __shared__ float rowv[];  // [d_c + d_r]
  const int m = blockIdx.x, lane = threadIdx.x;
  const int b = m / sq, i = m - b * sq;
  const int pos = seq_lens[b] - sq + i;
  const int64_t prow = int64_t(table[int64_t(b) * max_blocks + pos / bs]) * bs + pos % bs;
  const int N = dc + dr;
  float amax = 0.f;
  for (int n = lane; n < N; n += 64) {
    float s = 0.f;
    for (int kc = 0; kc < KC; ++kc) s += part[(int64_t(kc) * M + m) * N + n];
    rowv[n] = s;
    if (n < dc) amax = fmaxf(amax, fabsf(s));
  }
  __syncthreads();
  for (int j = lane; j < dr / 2; j += 64) {
    int ia, ib;
    rope_pair(j, dr, pairing, ia, ib);
    float c, s;
    rope_angle(pos, j, dr, base, c, s);
    const float xa = rowv[dc + ia], xb = rowv[dc + ib];
    rowv[dc + ia] = xa * c - xb * s;
    rowv[dc + ib] = xa * s + xb * c;
  }
  __syncthreads();
  using XR = typename XS::raw;
  XR* rp = static_cast<XR*>(rope_pool) + prow * dr;
  for (int n = lane; n < dr; n += 64) store_from_f32<XS>(rp, n, rowv[dc + n]);
  if constexpr (sizeof(typename KVS::raw) == 1) {
    amax = wave_max(amax);
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    if (lane == 0) scale_pool[prow] = scale;
    uint8_t* cp = static_cast<uint8_t*>(c_pool) + prow * dc;
    for (int n = lane; n < dc; n += 64) {
      // Nearest-even e4m3fn (OCP) conversion of the gfx950 instruction; |y| <= 448 up to
      // the rounding of the division, clamped so that no code saturates to NaN.
      const float y = fminf(fmaxf(rowv[n] / scale, -448.f), 448.f);
      cp[n] = uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFF);
    }
  } else {
    using KR = typename KVS::raw;
    KR* cp = static_cast<KR*>(c_pool) + prow * dc;
    for (int n = lane; n < dc; n += 64) store_from_f32<KVS>(cp, n, rowv[n]);
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
  const dim3 grid((N + kPN - 1) / kPN, KC, (a.M + kPM - 1) / kPM);
  if (a.x_dt == MLA_F32)
    hipLaunchKernelGGL(proj_partial_kernel<F32>, grid, dim3(256), 0, s, static_cast<const float*>(a.x),
                       static_cast<const float*>(a.w_dkv), static_cast<const float*>(a.w_kr), a.M, a.d_model,
                       a.dc, a.dr, a.part);
  else
    hipLaunchKernelGGL(proj_partial_kernel<BF16>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(a.x),
                       static_cast<const uint16_t*>(a.w_dkv), static_cast<const uint16_t*>(a.w_kr), a.M,
                       a.d_model, a.dc, a.dr, a.part);
  if (int e = int(hipGetLastError())) return e;
  const size_t lds = sizeof(float) * N;
#define MLA_FIN(XS, KVS)                                                                                    \
  hipLaunchKernelGGL((append_finalize_kernel<XS, KVS>), dim3(a.M), dim3(64), lds, s, a.part, KC, a.M, a.sq, \
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
