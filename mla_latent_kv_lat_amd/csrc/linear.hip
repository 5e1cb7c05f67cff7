// Skinny projections y = x . W (bf16 in, fp32 accumulation, bf16 out) for the query
// compression c_q = x W_DQ, the query up-projections and the output projection O W_O
// ("Operator Notes (1): MLA", sections 2 and 4), and for the folded weight products.
// These are weight-streaming products: few rows (the batch's new tokens), K and N in the
// thousands.  The matrix-core kernel of the cache write forms split-K partial sums (each
// 256-wide slice of K as a "head"), and linear_reduce_kernel adds the slices and rounds.
#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

// y[m, n .. n + 7] = bf16(sum over kc of part[m, kc, n .. n + 7]); one thread per 8 columns.
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* __restrict__ part,
                                                            uint16_t* __restrict__ y, int M, int KC, int N) {
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int n8 = N / 8;
  if (g >= int64_t(M) * n8) return;
  const int m = int(g / n8), n = int(g % n8) * 8;
  const float* p = part + int64_t(m) * KC * N + n;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < KC; ++kc) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p + int64_t(kc) * N);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + int64_t(kc) * N + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += a[e];
      acc[4 + e] += b[e];
    }
  }
  *reinterpret_cast<u32x4*>(y + int64_t(m) * N + n) =
      u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
            pack_bf16x2(acc[6], acc[7])};
}

}  // namespace

int launch_linear(const void* x, const void* w, void* y, int32_t M, int32_t K, int32_t N, float* part,
                  hipStream_t s) {
  int err = launch_proj_mfma(x, w, part, N, nullptr, nullptr, 0, M, K, 256, s);
  if (err) return err;
  const int64_t threads = int64_t(M) * (N / 8);
  hipLaunchKernelGGL(linear_reduce_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, part,
                     static_cast<uint16_t*>(y), M, K / 256, N);
  return int(hipGetLastError());
}

}  // namespace mla
