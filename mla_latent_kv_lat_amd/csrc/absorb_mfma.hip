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

constexpr int kTallRows = 128;  // rows per workgroup of the K = 128 product when M >= 128 (64 for K = 512)

struct Strides {
  int64_t m, h;
};
constexpr Strides kPacked{-1, 0};

// Activation rows in LDS: row r's 8-column chunk c is stored at chunk c ^ (r & 15), so the
// 16 rows of one B-operand read hit distinct banks.
__device__ __forceinline__ int xswz(int r) { return r & 15; }

// Grid (H, N / 64, ceil(M / MG)): one workgroup per (head, 64-column tile, MG-row group).
// Every load of the workgroup (its MG activation rows and the K x 64 weight slice) is issued
// before the first wait, so a workgroup costs one memory latency.  Workgroups are dealt to
// the n_xcd XCDs round-robin in launch order; when H is a multiple of n_xcd the launch index
// is remapped so that XCD x takes the heads h = x (mod n_xcd) and runs, head after head and
// column tile after column tile, all row groups of one (head, tile) back to back: the tile's
// weight slice and the head's activation rows are then read from HBM once and reused from
// that XCD's L2 (with the head as the fastest index instead, the row groups of one weight
// slice are spread over the whole launch and each refetches it).
// Element strides: x[m, h, :] starts at m x_st.m + h x_st.h and y[m, h, :] at m y_st.m +
// h y_st.h (a negative .m selects the packed layouts [M, H, K] / [M, H, N]).
// F32OUT: y holds fp32 sums (the split-K partials of the cache-write projection) instead of
// bf16 results.  Column tiles from N / 64 on take a second weight matrix w2 [H, K, N2] and
// output y2 [M, H, N2] (N2 a multiple of 64; the grid then has N / 64 + N2 / 64 column tiles).
template <int K, int MG, bool F32OUT = false>
__global__ __launch_bounds__(kThreads) void absorb_mfma_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               void* __restrict__ y, int M,
                                                               int H, int N,
                                                               int n_xcd, Strides x_st, Strides y_st,
                                                               const uint16_t* __restrict__ w2 = nullptr,
                                                               void* __restrict__ y2 = nullptr, int N2 = 0) {
  constexpr int kBlocks = MG / 16;
  __shared__ __attribute__((aligned(16))) uint16_t wt[K * kBN];  // [k][64], chunks swizzled
  __shared__ __attribute__((aligned(16))) uint16_t xs[MG * K];   // [row][k], chunks swizzled
  int h = blockIdx.x, n0 = blockIdx.y * kBN, m0 = blockIdx.z * MG;
  if (n_xcd > 1 && int(gridDim.x) % n_xcd == 0) {
    const int ncol = int(gridDim.y), nrg = int(gridDim.z);
    const int id = int(blockIdx.x) + int(gridDim.x) * (int(blockIdx.y) + ncol * int(blockIdx.z));
    const int j = id / n_xcd;  // position within this XCD's share
    h = (j / (ncol * nrg)) * n_xcd + id % n_xcd;
    n0 = ((j / nrg) % ncol) * kBN;
    m0 = (j % nrg) * MG;
  }
  if (n0 >= N) {  // a tile of the second matrix (workgroup-uniform)
    n0 -= N;
    w = w2;
    y = y2;
    N = N2;
  }
  const int64_t x_m = x_st.m >= 0 ? x_st.m : int64_t(H) * K, x_h = x_st.m >= 0 ? x_st.h : K;
  const int64_t y_m = y_st.m >= 0 ? y_st.m : int64_t(H) * N, y_h = y_st.m >= 0 ? y_st.h : N;
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
    xr[i] = ld16(x + int64_t(min(m0 + r, M - 1)) * x_m + h * x_h + 8 * ch);
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
  // Per k-step s: the weight operand (A, read transposed) once, then the B operands of every
  // row block (rows 16 i + mm, columns 32 s + 8 g + (0..7)).
  f32x4 acc[kBlocks];
#pragma unroll
  for (int i = 0; i < kBlocks; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < K / 32; ++s) {
    const bf16x8 av = lds_operand_tr(wt, 32 * s, 16 * wv, lane);
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int r = 16 * i + mm;
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&xs[r * K + 8 * ((4 * s + g) ^ xswz(r))]);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i], 0, 0, 0);
    }
  }
  if constexpr (F32OUT) {
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int m = m0 + 16 * i + mm;
      if (m < M)
        *reinterpret_cast<f32x4*>(static_cast<float*>(y) + int64_t(m) * y_m + h * y_h + n0 + 16 * wv + 4 * g) = acc[i];
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
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + int64_t(m) * y_m + h * y_h + n0 + 8 * c) =
            *reinterpret_cast<const u32x4*>(&ys[r * kBN + 8 * (c ^ ((r >> 1) & 7))]);
    }
  }
}

// The K = 512 product at large M, with K streamed: a workgroup (head, 64 columns, MG rows)
// walks K in chunks of 128, the weight and activation slices of chunk c + 1 loaded into
// registers while chunk c is multiplied from one of two LDS stages (2 x 32 KB for MG = 64,
// so two workgroups share a compute unit and their memory phases overlap).  The products of
// every output element run in the same k order as in absorb_mfma_kernel, so the results are
// the same bit for bit.
template <int MG>
__global__ __launch_bounds__(kThreads) void absorb_stream_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ w,
                                                                 uint16_t* __restrict__ y, int M, int H, int N,
                                                                 int n_xcd) {
  constexpr int K = 512, KC = 128, NC = K / KC, kBlocks = MG / 16;
  constexpr int kWPer = KC * 8 / kThreads;         // 16-byte weight chunks per thread and K chunk
  constexpr int kXPer = MG * (KC / 8) / kThreads;  // 16-byte activation chunks per thread and K chunk
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][KC * kBN];  // [k][64], chunks swizzled by swz128(k)
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MG * KC];   // [row][k], chunk c at c ^ xswz(row)
  int h = blockIdx.x, n0 = blockIdx.y * kBN, m0 = blockIdx.z * MG;
  if (n_xcd > 1 && int(gridDim.x) % n_xcd == 0) {
    const int ncol = int(gridDim.y), nrg = int(gridDim.z);
    const int id = int(blockIdx.x) + int(gridDim.x) * (int(blockIdx.y) + ncol * int(blockIdx.z));
    const int j = id / n_xcd;
    h = (j / (ncol * nrg)) * n_xcd + id % n_xcd;
    n0 = ((j / nrg) % ncol) * kBN;
    m0 = (j % nrg) * MG;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, mm = lane & 15;
  const uint16_t* wh = w + int64_t(h) * K * N + n0;
  u32x4 wr[kWPer], xr[kXPer];
  auto load = [&](int c) {
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int idx = tid + i * kThreads, k = idx >> 3, ch = idx & 7;
      wr[i] = ld16(wh + int64_t(c * KC + k) * N + 8 * ch);
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int idx = tid + i * kThreads, r = idx / (KC / 8), ch = idx % (KC / 8);
      xr[i] = ld16(x + (int64_t(min(m0 + r, M - 1)) * H + h) * K + c * KC + 8 * ch);
    }
  };
  auto stage = [&](int st) {
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int idx = tid + i * kThreads, k = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4*>(&wt[st][k * kBN + 8 * (ch ^ swz128(k))]) = wr[i];
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int idx = tid + i * kThreads, r = idx / (KC / 8), ch = idx % (KC / 8);
      *reinterpret_cast<u32x4*>(&xs[st][r * KC + 8 * (ch ^ xswz(r))]) = xr[i];
    }
  };
  f32x4 acc[kBlocks];
#pragma unroll
  for (int i = 0; i < kBlocks; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  stage(0);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int st = c & 1;
    if (c + 1 < NC) load(c + 1);
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      const bf16x8 av = lds_operand_tr(wt[st], 32 * s, 16 * wv, lane);
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) {
        const int r = 16 * i + mm;
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&xs[st][r * KC + 8 * ((4 * s + g) ^ xswz(r))]);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i], 0, 0, 0);
      }
    }
    if (c + 1 < NC) stage(st ^ 1);
    __syncthreads();  // stage st ^ 1 written; every wave done reading stage st
  }
  // bf16 results through LDS (stage 0's activation buffer), so that each output row's 128
  // bytes leave in one store: row r's 16-byte chunk c sits at c ^ ((r >> 1) & 7).
  uint16_t* ys = xs[0];
#pragma unroll
  for (int i = 0; i < kBlocks; ++i) {
    const int r = 16 * i + mm, col = 16 * wv + 4 * g;
    *reinterpret_cast<u32x2*>(&ys[r * kBN + 8 * ((col >> 3) ^ ((r >> 1) & 7)) + (col & 7)]) =
        u32x2{pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3])};
  }
  __syncthreads();
#pragma unroll
  for (int r = tid >> 3; r < MG; r += kThreads / 8) {
    const int c = tid & 7, m = m0 + r;
    if (m < M)
      *reinterpret_cast<u32x4*>(y + (int64_t(m) * H + h) * N + n0 + 8 * c) =
          *reinterpret_cast<const u32x4*>(&ys[r * kBN + 8 * (c ^ ((r >> 1) & 7))]);
  }
}

// The K = 128 product at large M, persistent over rows: a workgroup (head, 128 columns as
// two 64-column halves) keeps its 32 KB weight slice in LDS and walks the rows in groups of
// 64, group g + 1's activation rows loaded into registers while group g is multiplied from
// one of two LDS stages; group g's bf16 results are staged in the stage it was read from
// (once every wave is done with it) and leave as whole 128-byte row pieces.  The products of
// every output element run in the same k order as in absorb_mfma_kernel.
__global__ __launch_bounds__(kThreads) void absorb_rows_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ y, int M, int H, int N,
                                                               int n_xcd) {
  constexpr int K = 128, RG = 64, NH = 2, kBlocks = RG / 16;
  constexpr int kWPer = NH * K * 8 / kThreads;     // 16-byte weight chunks per thread
  constexpr int kXPer = RG * (K / 8) / kThreads;   // 16-byte activation chunks per thread and group
  __shared__ __attribute__((aligned(16))) uint16_t wt[NH][K * kBN];  // [k][64], chunks swizzled by swz128(k)
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][RG * K];    // [row][k], chunk c at c ^ xswz(row)
  int h = blockIdx.x, n0 = blockIdx.y * NH * kBN;
  if (n_xcd > 1 && int(gridDim.x) % n_xcd == 0) {
    const int ncol = int(gridDim.y);
    const int id = int(blockIdx.x) + int(gridDim.x) * int(blockIdx.y);
    const int j = id / n_xcd;
    h = (j / ncol) * n_xcd + id % n_xcd;
    n0 = (j % ncol) * NH * kBN;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, mm = lane & 15;
  const int ngroups = (M + RG - 1) / RG;
  u32x4 xr[kXPer];
  auto load = [&](int grp) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int idx = tid + i * kThreads, r = idx / (K / 8), ch = idx % (K / 8);
      xr[i] = ld16(x + (int64_t(min(grp * RG + r, M - 1)) * H + h) * K + 8 * ch);
    }
  };
  auto stage = [&](int st) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int idx = tid + i * kThreads, r = idx / (K / 8), ch = idx % (K / 8);
      *reinterpret_cast<u32x4*>(&xs[st][r * K + 8 * (ch ^ xswz(r))]) = xr[i];
    }
  };
  {
    u32x4 wr[kWPer];
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int idx = tid + i * kThreads, hh = idx / (K * 8), k = (idx >> 3) % K, ch = idx & 7;
      wr[i] = ld16(w + int64_t(h) * K * N + int64_t(k) * N + n0 + 64 * hh + 8 * ch);
    }
    load(0);
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int idx = tid + i * kThreads, hh = idx / (K * 8), k = (idx >> 3) % K, ch = idx & 7;
      *reinterpret_cast<u32x4*>(&wt[hh][k * kBN + 8 * (ch ^ swz128(k))]) = wr[i];
    }
    stage(0);
  }
  __syncthreads();
  for (int grp = 0; grp < ngroups; ++grp) {
    const int st = grp & 1;
    if (grp + 1 < ngroups) load(grp + 1);
    f32x4 acc[NH][kBlocks];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) acc[hh][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < K / 32; ++s2) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const bf16x8 av = lds_operand_tr(wt[hh], 32 * s2, 16 * wv, lane);
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) {
          const int r = 16 * i + mm;
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&xs[st][r * K + 8 * ((4 * s2 + g) ^ xswz(r))]);
          acc[hh][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[hh][i], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // every wave is done reading stage st
    // Results into stage st: 128-byte piece rp = 2 r + hh of row r, chunk c at c ^ ((rp >> 1) & 7).
    uint16_t* ys = xs[st];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) {
        const int rp = NH * (16 * i + mm) + hh, col = 16 * wv + 4 * g;
        *reinterpret_cast<u32x2*>(&ys[rp * kBN + 8 * ((col >> 3) ^ ((rp >> 1) & 7)) + (col & 7)]) =
            u32x2{pack_bf16x2(acc[hh][i][0], acc[hh][i][1]), pack_bf16x2(acc[hh][i][2], acc[hh][i][3])};
      }
    if (grp + 1 < ngroups) stage(st ^ 1);
    __syncthreads();  // results staged, next group's rows staged
#pragma unroll
    for (int rp = tid >> 3; rp < RG * NH; rp += kThreads / 8) {
      const int c = tid & 7, r = rp / NH, hh = rp % NH, m = grp * RG + r;
      if (m < M)
        *reinterpret_cast<u32x4*>(y + (int64_t(m) * H + h) * N + n0 + 64 * hh + 8 * c) =
            *reinterpret_cast<const u32x4*>(&ys[rp * kBN + 8 * (c ^ ((rp >> 1) & 7))]);
    }
  }
}

}  // namespace

bool proj_mfma_supported(int32_t M, int32_t K_total, int32_t N, int32_t kchunk) {
  return (kchunk == 128 || kchunk == 256) && K_total % kchunk == 0 && N % kBN == 0 && M <= 32 * 65535;
}

// part[m, kc, n] = sum_{k < kchunk} x[m, kchunk kc + k] * w[kchunk kc + k, n] (and part2
// likewise with w2, N2 columns; N2 may be 0): the per-head kernel with the K chunks of x and w
// taken as the heads, fp32 out, both matrices in one launch.
int launch_proj_mfma(const void* x, const void* w, float* part, int32_t N, const void* w2, float* part2,
                     int32_t N2, int32_t M, int32_t K_total, int32_t kchunk, hipStream_t s) {
  const int KC = K_total / kchunk;
  int cus = kDefaultCUs, n_xcd = kDefaultXcds;
  device_topology(&cus, &n_xcd);
  const dim3 grid(KC, (N + N2) / kBN, (M + 31) / 32);
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  const auto* w2p = static_cast<const uint16_t*>(w2);
  if (kchunk == 128)
    hipLaunchKernelGGL((absorb_mfma_kernel<128, 32, true>), grid, dim3(kThreads), 0, s, xp, wp, part, M, KC, N,
                       n_xcd, kPacked, kPacked, w2p, part2, N2);
  else
    hipLaunchKernelGGL((absorb_mfma_kernel<256, 32, true>), grid, dim3(kThreads), 0, s, xp, wp, part, M, KC, N,
                       n_xcd, kPacked, kPacked, w2p, part2, N2);
  return int(hipGetLastError());
}

bool absorb_mfma_supported(mla_dtype dt, int32_t M, int32_t K, int32_t N) {
  // The row groups are the grid's z dimension (at most 65535 groups of 32 rows).
  return dt == MLA_BF16 && (K == 128 || K == 512) && N % kBN == 0 && M <= 32 * 65535;
}

namespace {
int launch_absorb_t(const void* x, const void* w, void* y, int32_t M, int32_t H, int32_t K, int32_t N, Strides x_st,
                    Strides y_st, hipStream_t s) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  auto* yp = static_cast<uint16_t*>(y);
  int cus = kDefaultCUs, n_xcd = kDefaultXcds;
  device_topology(&cus, &n_xcd);
  if (K == 128 && M >= kTallRows && N % 128 == 0 && x_st.m < 0 && y_st.m < 0)
    hipLaunchKernelGGL(absorb_rows_kernel, dim3(H, N / 128), dim3(kThreads), 0, s, xp, wp, yp, M, H, N, n_xcd);
  else if (K == 128 && M >= kTallRows)
    hipLaunchKernelGGL((absorb_mfma_kernel<128, kTallRows>), dim3(H, N / kBN, (M + kTallRows - 1) / kTallRows),
                       dim3(kThreads), 0, s, xp, wp, yp, M, H, N, n_xcd, x_st, y_st);
  else if (K == 128)
    hipLaunchKernelGGL((absorb_mfma_kernel<128, 32>), dim3(H, N / kBN, (M + 31) / 32), dim3(kThreads), 0, s,
                       xp, wp, yp, M, H, N, n_xcd, x_st, y_st);
  else if (M >= 64 && x_st.m < 0 && y_st.m < 0)
    hipLaunchKernelGGL((absorb_stream_kernel<64>), dim3(H, N / kBN, (M + 63) / 64), dim3(kThreads), 0, s, xp, wp,
                       yp, M, H, N, n_xcd);
  else
    hipLaunchKernelGGL((absorb_mfma_kernel<512, 32>), dim3(H, N / kBN, (M + 31) / 32), dim3(kThreads), 0, s,
                       xp, wp, yp, M, H, N, n_xcd, x_st, y_st);
  return int(hipGetLastError());
}
}  // namespace

int launch_absorb_mfma(const void* x, const void* w, void* y, int32_t M, int32_t H, int32_t K,
                       int32_t N, hipStream_t s) {
  return launch_absorb_t(x, w, y, M, H, K, N, kPacked, kPacked, s);
}

// w_uvo[h, c, :] = w_uv[h, c, :] . w_o[h d_h .. h d_h + d_h, :]: the per-head product with the
// d_c rows c of w_uv[h] as its rows (x[c, h, :] at c d_h + h d_c d_h), w_o viewed as
// [n_h, d_h, d_model], and the result stored head-major (y[c, h, :] at c d_model + h d_c d_model).
int launch_fold_output(const void* w_uv, const void* w_o, void* w_uvo, int32_t n_h, int32_t d_c, int32_t d_h,
                       int32_t d_model, hipStream_t s) {
  return launch_absorb_t(w_uv, w_o, w_uvo, d_c, n_h, d_h, d_model, Strides{d_h, int64_t(d_c) * d_h},
                         Strides{d_model, int64_t(d_c) * d_model}, s);
}

}  // namespace mla
