// Utility kernels: the paged-cache lookup on its own, and the device's fp8 code table.
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

// dst[b, t, :] = pool[table[b, t / bs], t % bs, :] for t < seq_lens[b]; one workgroup per
// (token, sequence), 4-byte words.
__global__ __launch_bounds__(128) void gather_pages_kernel(const uint32_t* pool, int bs, int64_t words,
                                                           const int32_t* table, int max_blocks,
                                                           const int32_t* seq_lens, int max_seq_len,
                                                           uint32_t* dst) {
  const int t = blockIdx.x, b = blockIdx.y;
  if (t >= seq_lens[b]) return;
  const int64_t src_row = cache_row(true, b, t, 0, table, max_blocks, bs);
  const uint32_t* s = pool + src_row * words;
  uint32_t* d = dst + (int64_t(b) * max_seq_len + t) * words;
  for (int64_t i = threadIdx.x; i < words; i += 128) d[i] = s[i];
}

__global__ void fp8_table_kernel(float* out) { out[threadIdx.x] = e4m3_to_f32(threadIdx.x); }

}  // namespace

int launch_gather_pages(const void* pool, int32_t block_size, int64_t row_bytes, const int32_t* table,
                        int32_t B, int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                        void* dst, hipStream_t s) {
  hipLaunchKernelGGL(gather_pages_kernel, dim3(max_seq_len, B), dim3(128), 0, s,
                     static_cast<const uint32_t*>(pool), block_size, row_bytes / 4, table, max_blocks,
                     seq_lens, max_seq_len, static_cast<uint32_t*>(dst));
  return int(hipGetLastError());
}

int launch_fp8_table(float* out, hipStream_t s) {
  hipLaunchKernelGGL(fp8_table_kernel, dim3(1), dim3(256), 0, s, out);
  const int err = int(hipGetLastError());
  return err ? err : launch_fp8_bf16_table(out + 256, s);
}

}  // namespace mla
