// General per-head absorption products (VALU):  y[m, h, :] = x[m, h, :] . W[h]
//
// With W = W_UK this is the query-side absorption, with W = W_UV the output-side one
// ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE key:
// the up-projections fold into the query and output projections).
//   x [M, H, K], W [H, K, N], y [M, H, N]; fp32 accumulation.
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kMB = 16;   // rows of x per workgroup
constexpr int kKC = 256;  // K chunk staged in LDS

template <typename S>
__global__ __launch_bounds__(256) void absorb_general_kernel(const typename S::raw* x,
                                                             const typename S::raw* w,
                                                             typename S::raw* y, int M, int H,
                                                             int K, int N) {
  __shared__ float xs[kMB][kKC];
  const int n = blockIdx.x * 256 + threadIdx.x, h = blockIdx.y, m0 = blockIdx.z * kMB;
  float acc[kMB] = {};
  for (int k0 = 0; k0 < K; k0 += kKC) {
    const int kc = min(kKC, K - k0);
    for (int idx = threadIdx.x; idx < kMB * kKC; idx += 256) {
      const int mm = idx / kKC, kk = idx % kKC, m = m0 + mm;
      xs[mm][kk] = (m < M && kk < kc) ? load_as_f32<S>(x, (int64_t(m) * H + h) * K + k0 + kk) : 0.f;
    }
    __syncthreads();
    if (n < N) {
      for (int kk = 0; kk < kc; ++kk) {
        const float wv = load_as_f32<S>(w, (int64_t(h) * K + k0 + kk) * N + n);
#pragma unroll
        for (int mm = 0; mm < kMB; ++mm) acc[mm] += xs[mm][kk] * wv;
      }
    }
    __syncthreads();
  }
  if (n < N) {
#pragma unroll
    for (int mm = 0; mm < kMB; ++mm) {
      const int m = m0 + mm;
      if (m < M) store_from_f32<S>(y, (int64_t(m) * H + h) * N + n, acc[mm]);
    }
  }
}

}  // namespace

int launch_absorb(const void* x, const void* w, void* y, mla_dtype dt, int32_t M, int32_t H,
                  int32_t K, int32_t N, hipStream_t s) {
  if (absorb_mfma_supported(dt, M, K, N)) return launch_absorb_mfma(x, w, y, M, H, K, N, s);
  const dim3 grid((N + 255) / 256, H, (M + kMB - 1) / kMB);
  if (dt == MLA_F32)
    hipLaunchKernelGGL(absorb_general_kernel<F32>, grid, dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(w),
                       static_cast<float*>(y), M, H, K, N);
  else
    hipLaunchKernelGGL(absorb_general_kernel<BF16>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                       static_cast<uint16_t*>(y), M, H, K, N);
  return int(hipGetLastError());
}

}  // namespace mla
