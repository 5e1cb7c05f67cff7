// Device helpers shared by the HIP kernels: number formats and small reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

// Storage tags: the kernels read raw bits and convert in registers.
struct F32 { using raw = float; };
struct BF16 { using raw = uint16_t; };
struct FP8 { using raw = uint8_t; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// float -> bfloat16 bits, round to nearest even (the gfx950 conversion instruction).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// One OCP e4m3fn byte -> float, using the hardware fp8 conversion of gfx950.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(code & 0xFF), 0);
}

template <typename S>
__device__ __forceinline__ float load_as_f32(const typename S::raw* p, int64_t i);

template <>
__device__ __forceinline__ float load_as_f32<F32>(const float* p, int64_t i) { return p[i]; }

template <>
__device__ __forceinline__ float load_as_f32<BF16>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <>
__device__ __forceinline__ float load_as_f32<FP8>(const uint8_t* p, int64_t i) {
  return e4m3_to_f32(p[i]);
}

template <typename S>
__device__ __forceinline__ void store_from_f32(typename S::raw* p, int64_t i, float v);

template <>
__device__ __forceinline__ void store_from_f32<F32>(float* p, int64_t i, float v) { p[i] = v; }

template <>
__device__ __forceinline__ void store_from_f32<BF16>(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Row of the cache holding logical token t of sequence b (contiguous or paged).
__device__ __forceinline__ int64_t cache_row(bool paged, int b, int64_t t, int64_t T,
                                             const int32_t* table, int max_blocks, int bs) {
  if (!paged) return int64_t(b) * T + t;
  const int32_t blk = table[int64_t(b) * max_blocks + t / bs];
  return int64_t(blk) * bs + t % bs;
}

constexpr float kLn2 = 0.6931471805599453f;

}  // namespace mla
