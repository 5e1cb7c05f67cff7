// Vector types and LDS helpers shared by the matrix-core (MFMA) kernels.
//
// Operand layouts (lane l):
//   v_mfma_f32_16x16x32_bf16 (g = l / 16):
//     A[m][k]: lane holds A[l % 16][8g .. 8g + 7];  B[k][n]: B[8g .. 8g + 7][l % 16];
//     D[m][n]: lane holds D[4g .. 4g + 3][l % 16].
//   v_mfma_f32_32x32x16_bf16 (h = l / 32):
//     A[m][k]: lane holds A[l % 32][8h .. 8h + 7];  B[k][n]: B[8h .. 8h + 7][l % 32];
//     D[m][n]: element 4i + r of lane l is D[8i + 4h + r][l % 32]   (i, r in 0..3).
//   v_mfma_scale_f32_32x32x64_f8f6f4 (8-bit formats, h = l / 32): lane l holds row (A) or
//     column (B) l % 32, K values 16h .. 16h + 15 in bytes 0 .. 15 and 32 + 16h .. 32 + 16h + 15
//     in bytes 16 .. 31; its E8M0 scale operand applies to K block h (K 32h .. 32h + 31) of
//     that row or column.  D as for the bf16 form.  A product whose two operands follow any
//     one K order is unaffected by it; the block scales are not.
// On gfx950 the 32x32x16 form runs at twice the 16x16x32 form's throughput (the latter
// takes as long per instruction for half the work), so dense loops use 32x32x16.
// ds_read_b64_tr_b16: within each 16-lane group, lane 4r + q supplies the address of
// four consecutive 16-bit elements (row r, columns 4q .. 4q + 3 of a 4 x 16 block) and
// lane j receives column j (rows 0 .. 3).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));  // 32 fp8 codes: one f8f6f4 MFMA operand
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Chunk swizzle for LDS tiles whose rows are 128 bytes (8 chunks of 16 bytes, two rows
// per 64-bank cycle).  Applied as chunk ^ swz128(row): the 16 consecutive rows written by
// one 16-byte-per-lane store, and the 8 rows of each half of a transposed read (rows
// 8g + r and 8g + 4 + r), fall in distinct banks.
__device__ __forceinline__ int swz128(int row) {
  return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2) | ((row >> 2) & 1);
}

// Chunk swizzle for tiles whose rows are a multiple of 256 bytes, read with 32-column
// transposed reads (the decode kernel's staged rows): chunk ^ swz32(row).  On gfx950 a 16-byte LDS read serves 16 lanes
// (256 bytes) per cycle and a 16-byte write 8 lanes (128 bytes).  The swizzle is
// bijective on the low 4 row bits (16 rows read at one chunk each hit distinct banks); its
// low 3 bits are bijective on each aligned group of 8 rows (8 rows written at one chunk
// each hit distinct banks); and its high 2 bits are bijective on each aligned group of 4
// rows (the 4 rows of each transposed-read pass put their 64-byte column groups on
// distinct banks).
__device__ __forceinline__ int swz32(int row) {
  return ((row & 3) << 2) | ((row >> 2) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1);
}

// Transposed read of 4 bf16 (see the layout note above) from LDS.
__device__ __forceinline__ u32x2 lds_read_tr4(const uint16_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) s16x4*)(p)));
}

// A 16 x 32 (k x 16 columns) bf16 MFMA operand read transposed from a row-major LDS tile
// with 128-byte rows (64 columns, swizzled by swz128): rows k0 .. k0 + 31, columns
// c0 .. c0 + 15 (c0 a multiple of 16).  Lane l receives column c0 + l % 16, rows
// k0 + 8g .. k0 + 8g + 7.
__device__ __forceinline__ bf16x8 lds_operand_tr(const uint16_t* tile, int k0, int c0, int lane) {
  const int g = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int col = c0 + 4 * q;
  const int k_lo = k0 + 8 * g + r, k_hi = k_lo + 4;
  const u32x2 lo = lds_read_tr4(tile + k_lo * 64 + 8 * ((col >> 3) ^ swz128(k_lo)) + (col & 7));
  const u32x2 hi = lds_read_tr4(tile + k_hi * 64 + 8 * ((col >> 3) ^ swz128(k_hi)) + (col & 7));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// A 32 x 16 (m = 32 columns, k = 16 rows) bf16 A operand of v_mfma_f32_32x32x16_bf16, read
// transposed from a staged tile (1 KB rows, swz32): rows k0 .. k0 + 15, columns c0 .. c0 + 31
// (c0 a multiple of 32).  Lane l receives column c0 + l % 32 and rows k0 + 8h .. k0 + 8h + 7
// (h = l / 32): 16-lane group G reads columns c0 + 16 (G & 1) + (0..15) of rows
// k0 + 8 (G >> 1) + (0..7).
__device__ __forceinline__ bf16x8 lds_operand_tr512(const uint16_t* tile, int k0, int c0, int lane) {
  const int G = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int col = c0 + 16 * (G & 1) + 4 * q;
  const int k_lo = k0 + 8 * (G >> 1) + r, k_hi = k_lo + 4;
  const u32x2 lo = lds_read_tr4(tile + k_lo * 512 + 8 * ((col >> 3) ^ swz32(k_lo)) + (col & 7));
  const u32x2 hi = lds_read_tr4(tile + k_hi * 512 + 8 * ((col >> 3) ^ swz32(k_hi)) + (col & 7));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Two e4m3fn codes (low or high half-word of `w`) -> two bf16, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 8 codes (two dwords) -> 8 bf16 (four dwords).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = e4m3x2_to_bf16x2<false>(lo);
  r[1] = e4m3x2_to_bf16x2<true>(lo);
  r[2] = e4m3x2_to_bf16x2<false>(hi);
  r[3] = e4m3x2_to_bf16x2<true>(hi);
  return r;
}

// Two floats -> two bf16 (a in the low half), round to nearest even: one packed conversion
// (two scalar conversions plus a shift and an or when written element by element).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Cross-lane swap of gfx950, written as a single inline instruction (register operands
// only, no memory access).  v_permlane32_swap_b32 a, b exchanges the upper 32 lanes of a
// with the lower 32 lanes of b, so with a = b = x every lane ends up holding {x, x from
// lane ^ 32} in (a, b).  The builtin form is not used: the compiler folds max(first
// result, second result) down to the first result, dropping the partner lane.  The
// leading s_nop covers the two wait states the instruction needs after a VALU write of
// its operands.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

}  // namespace mla
