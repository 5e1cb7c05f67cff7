// Matrix-core per-head absorption products:  y[m, h, :] = x[m, h, :] . W[h]   (bf16 in,
// fp32 accumulation, bf16 out).  With W = W_UK this folds the key up-projection into the
// query, with W = W_UV it applies the value up-projection once to the attended latent
// ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE key).
//
// A workgroup owns one head and 64 output columns; it stages that K x 64 slice of W[h] in
// LDS once and then walks all M rows.  The product is formed transposed,
// y^T[n, m] = W^T[n, :] . x^T[:, m], so that the staged weights are the A operand (read
// transposed from LDS), the activation rows are the B operand straight from global
// memory, and each lane stores 4 consecutive output columns.
#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kBN = 64;      // output columns per workgroup (one 16-column block per wave)
constexpr int kThreads = 256;

template <int K>
__global__ __launch_bounds__(kThreads) void absorb_mfma_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ y, int M,
                                                               int H, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[K * kBN];  // [k][64], chunks swizzled
  const int n0 = blockIdx.x * kBN, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, mm = lane & 15;

  const uint16_t* wh = w + int64_t(h) * K * N + n0;
#pragma unroll
  for (int idx = tid; idx < K * 8; idx += kThreads) {
    const int k = idx >> 3, ch = idx & 7;
    *reinterpret_cast<u32x4*>(&wt[k * kBN + 8 * (ch ^ swz128(k))]) = ld16(wh + int64_t(k) * N + 8 * ch);
  }
  __syncthreads();

  bf16x8 a[K / 32];
#pragma unroll
  for (int s = 0; s < K / 32; ++s) a[s] = lds_operand_tr(wt, 32 * s, 16 * wv, lane);

  for (int m0 = 0; m0 < M; m0 += 16) {
    const int m = m0 + mm;
    const bool ok = m < M;
    const uint16_t* xr = x + (int64_t(m) * H + h) * K + 8 * g;
    bf16x8 bv[K / 32];
#pragma unroll
    for (int s = 0; s < K / 32; ++s)
      bv[s] = __builtin_bit_cast(bf16x8, ok ? ld16(xr + 32 * s) : u32x4{0, 0, 0, 0});
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K / 32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bv[s], acc, 0, 0, 0);
    if (ok) {
      const uint32_t w0 = uint32_t(f32_to_bf16_bits(acc[0])) | (uint32_t(f32_to_bf16_bits(acc[1])) << 16);
      const uint32_t w1 = uint32_t(f32_to_bf16_bits(acc[2])) | (uint32_t(f32_to_bf16_bits(acc[3])) << 16);
      *reinterpret_cast<u32x2*>(y + (int64_t(m) * H + h) * N + n0 + 16 * wv + 4 * g) = u32x2{w0, w1};
    }
  }
}

}  // namespace

bool absorb_mfma_supported(mla_dtype dt, int32_t K, int32_t N) {
  return dt == MLA_BF16 && (K == 128 || K == 512) && N % kBN == 0;
}

int launch_absorb_mfma(const void* x, const void* w, void* y, int32_t M, int32_t H, int32_t K,
                       int32_t N, hipStream_t s) {
  const dim3 grid(N / kBN, H);
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  auto* yp = static_cast<uint16_t*>(y);
  if (K == 128)
    hipLaunchKernelGGL(absorb_mfma_kernel<128>, grid, dim3(kThreads), 0, s, xp, wp, yp, M, H, N);
  else
    hipLaunchKernelGGL(absorb_mfma_kernel<512>, grid, dim3(kThreads), 0, s, xp, wp, yp, M, H, N);
  return int(hipGetLastError());
}

}  // namespace mla
