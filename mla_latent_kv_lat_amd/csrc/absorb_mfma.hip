// Matrix-core per-head absorption products:  y[m, h, :] = x[m, h, :] . W[h]   (bf16 in,
// fp32 accumulation, bf16 out).  With W = W_UK this folds the key up-projection into the
// query, with W = W_UV it applies the value up-projection once to the attended latent
// ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE key).
//
// A workgroup owns one head, 64 output columns and a group of 32 rows; it stages that K x 64
// slice of W[h] and its rows of x in LDS and multiplies them.  The product is formed
// transposed, y^T[n, m] = W^T[n, :] . x^T[:, m], so that the staged weights are the A operand
// (read transposed from LDS) and the activation rows the B operand; bf16 results go back
// through LDS so that every output row's 128 bytes leave in one store instruction.  Every
// byte is fetched once per workgroup: the four waves share the activation rows through LDS
// (the load path of a compute unit, not HBM, bounds these small products).
#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kBN = 64;      // output columns per workgroup (one 16-column block per wave)
constexpr int kThreads = 256;

// Activation rows in LDS: row r's 8-column chunk c is stored at chunk c ^ (r & 15), so the
// 16 rows of one B-operand read hit distinct banks.
__device__ __forceinline__ int xswz(int r) { return r & 15; }

// Grid (H, N / 64, ceil(M / MG)): one workgroup per (head, 64-column tile, MG-row group).
// Every load of the workgroup (its MG activation rows and the K x 64 weight slice) is issued
// before the first wait, so a workgroup costs one memory latency.  Workgroup ids are dealt
// to the 8 XCDs round-robin, and the head is the fastest grid dimension: with H a multiple
// of 8, all column tiles (and row groups) of one head run on one XCD and share its
// activation rows (and weight slice) through that XCD's L2.
// F32OUT: y holds fp32 sums (the split-K partials of the cache-write projection) instead of
// bf16 results.  Column tiles from N / 64 on take a second weight matrix w2 [H, K, N2] and
// output y2 [M, H, N2] (N2 a multiple of 64; the grid then has N / 64 + N2 / 64 column tiles).
template <int K, int MG, bool F32OUT = false>
__global__ __launch_bounds__(kThreads) void absorb_mfma_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               void* __restrict__ y, int M,
                                                               int H, int N,
                                                               const uint16_t* __restrict__ w2 = nullptr,
                                                               void* __restrict__ y2 = nullptr, int N2 = 0) {
  constexpr int kBlocks = MG / 16;
  __shared__ __attribute__((aligned(16))) uint16_t wt[K * kBN];  // [k][64], chunks swizzled
  __shared__ __attribute__((aligned(16))) uint16_t xs[MG * K];   // [row][k], chunks swizzled
  int h = blockIdx.x, n0 = blockIdx.y * kBN, m0 = blockIdx.z * MG;
  if (n0 >= N) {  // a tile of the second matrix (workgroup-uniform)
    n0 -= N;
    w = w2;
    y = y2;
    N = N2;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, mm = lane & 15;

  // The MG rows of x (a row past M loads row M - 1 instead, always in range: row m of the
  // product depends on x row m only, and rows past M are never stored) and the weight slice.
  constexpr int kXPer = MG * K / 8 / kThreads;  // 16-byte activation chunks per thread
  constexpr int kPer = K * 8 / kThreads;        // 16-byte weight chunks per thread
  u32x4 xr[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int idx = tid + i * kThreads, r = idx / (K / 8), ch = idx % (K / 8);
    xr[i] = ld16(x + (int64_t(min(m0 + r, M - 1)) * H + h) * K + 8 * ch);
  }
  const uint16_t* wh = w + int64_t(h) * K * N + n0;
  u32x4 wr[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid + i * kThreads, k = idx >> 3, ch = idx & 7;
    wr[i] = ld16(wh + int64_t(k) * N + 8 * ch);
  }
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int idx = tid + i * kThreads, r = idx / (K / 8), ch = idx % (K / 8);
    *reinterpret_cast<u32x4*>(&xs[r * K + 8 * (ch ^ xswz(r))]) = xr[i];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid + i * kThreads, k = idx >> 3, ch = idx & 7;
    *reinterpret_cast<u32x4*>(&wt[k * kBN + 8 * (ch ^ swz128(k))]) = wr[i];
  }
  __syncthreads();
  // B operands: rows 16 i + mm, columns 32 s + 8 g + (0..7).
  bf16x8 bv[kBlocks][K / 32];
#pragma unroll
  for (int i = 0; i < kBlocks; ++i)
#pragma unroll
    for (int s2 = 0; s2 < K / 32; ++s2) {
      const int r = 16 * i + mm;
      bv[i][s2] = *reinterpret_cast<const bf16x8*>(&xs[r * K + 8 * ((4 * s2 + g) ^ xswz(r))]);
    }

  f32x4 acc[kBlocks];
#pragma unroll
  for (int i = 0; i < kBlocks; ++i) {
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K / 32; ++s)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_operand_tr(wt, 32 * s, 16 * wv, lane), bv[i][s],
                                                       acc[i], 0, 0, 0);
  }
  if constexpr (F32OUT) {
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int m = m0 + 16 * i + mm;
      if (m < M)
        *reinterpret_cast<f32x4*>(static_cast<float*>(y) + (int64_t(m) * H + h) * N + n0 + 16 * wv + 4 * g) = acc[i];
    }
  } else {
    // The MG x 64 bf16 result goes through LDS (in the activation buffer, once every wave is
    // done reading it) so that each row's 128 bytes are written by 8 lanes of one store:
    // row r's 16-byte chunk c sits at c ^ ((r >> 1) & 7).
    __syncthreads();
    uint16_t* ys = xs;
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int r = 16 * i + mm, col = 16 * wv + 4 * g;
      *reinterpret_cast<u32x2*>(&ys[r * kBN + 8 * ((col >> 3) ^ ((r >> 1) & 7)) + (col & 7)]) =
          u32x2{pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3])};
    }
    __syncthreads();
    constexpr int kRowsPerPass = kThreads / 8;
#pragma unroll
    for (int r = tid >> 3; r < MG; r += kRowsPerPass) {
      const int c = tid & 7, m = m0 + r;
      if (m < M)
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + (int64_t(m) * H + h) * N + n0 + 8 * c) =
            *reinterpret_cast<const u32x4*>(&ys[r * kBN + 8 * (c ^ ((r >> 1) & 7))]);
    }
  }
}

}  // namespace

bool proj_mfma_supported(int32_t M, int32_t K_total, int32_t N) {
  return K_total % 256 == 0 && N % kBN == 0 && M <= 32 * 65535;
}

// part[m, kc, n] = sum_{k < 256} x[m, 256 kc + k] * w[256 kc + k, n] (and part2 likewise
// with w2, N2 columns; N2 may be 0): the per-head kernel with the K chunks of x and w taken
// as the heads, fp32 out, both matrices in one launch.
int launch_proj_mfma(const void* x, const void* w, float* part, int32_t N, const void* w2, float* part2,
                     int32_t N2, int32_t M, int32_t K_total, hipStream_t s) {
  const int KC = K_total / 256;
  hipLaunchKernelGGL((absorb_mfma_kernel<256, 32, true>), dim3(KC, (N + N2) / kBN, (M + 31) / 32), dim3(kThreads),
                     0, s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), part, M, KC, N,
                     static_cast<const uint16_t*>(w2), part2, N2);
  return int(hipGetLastError());
}

bool absorb_mfma_supported(mla_dtype dt, int32_t M, int32_t K, int32_t N) {
  // The row groups are the grid's z dimension (at most 65535 groups of 32 rows).
  return dt == MLA_BF16 && (K == 128 || K == 512) && N % kBN == 0 && M <= 32 * 65535;
}

int launch_absorb_mfma(const void* x, const void* w, void* y, int32_t M, int32_t H, int32_t K,
                       int32_t N, hipStream_t s) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  auto* yp = static_cast<uint16_t*>(y);
  if (K == 128)
    hipLaunchKernelGGL((absorb_mfma_kernel<128, 32>), dim3(H, N / kBN, (M + 31) / 32), dim3(kThreads), 0, s,
                       xp, wp, yp, M, H, N);
  else
    hipLaunchKernelGGL((absorb_mfma_kernel<512, 32>), dim3(H, N / kBN, (M + 31) / 32), dim3(kThreads), 0, s,
                       xp, wp, yp, M, H, N);
  return int(hipGetLastError());
}

}  // namespace mla
