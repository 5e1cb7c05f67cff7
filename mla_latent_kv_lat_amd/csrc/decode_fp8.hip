// Matrix-core latent-attention decode with both products on fp8 operands, for an e4m3fn
// latent cache with one scale per token (d_c = 512, d_r = 64) on gfx950.
//
// The absorbed form ("multi-head latent attention" glossary entry, paragraph on the
// decoupled RoPE key; "Multi-Head Latent Attention and the compression of the KV cache",
// paragraph on the associativity argument) over a quantized cache (the quantized-cache
// direction of "Multi-Head Latent Attention (MLA) Explained", section "Which Models Use MLA
// and What Is Next").  Both contractions run on the 32 x 32 x 64 fp8 matrix instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4) straight on the stored codes:
//   S^T[tok, row] = ts[tok] * (codes[tok, :] . Q8[row, :]) + R[tok, :] . Q_rope[row, :]
//   O^T[col, row] += codes[tok, col]^T . P8^T[tok, row] * 2^e(row, tok / 32)
// Q8 is the query rounded to e4m3 per 128-column slice (scale max|slice| / 448, one
// accumulator per slice); the RoPE term stays a bf16 product.  P8 holds each probability
// times its token's scale, rounded to e4m3 after division by a power of two 2^e chosen per
// row and 32 tokens (the largest value lands in [128, 256)); the instruction applies 2^e
// itself through its per-lane block scale (E8M0): lane (n, h) of the B operand gives the
// scale of K block h (K 32 h .. 32 h + 31), and the operands are laid out in the
// instruction's K order so that block h is the step's half h.  The reference max of each row is an integer in
// base-2 units, so every rescale is an exact power of two and the rounding of a weight does
// not depend on where the reference stands (the product with a power of two commutes with
// rounding to 4 significant bits).
//
// The value product's K (64 tokens) sets the step: a workgroup owns 64 query rows of one
// sequence and walks its piece of the context in 64-token steps.  Eight waves, one score
// wave and one output wave on each SIMD:
//   * score waves 0 .. 3 (SIMD w): wave w owns rows 32 (w & 1) .. + 31 and half w >> 1 (tokens
//     32 (w >> 1) .. + 31) of every step: eight fp8 and four bf16 products, then the online
//     softmax of its rows over its half-stream (its own integer reference and sum), then the
//     rounded probabilities with their block scales and the stream's reference;
//   * output waves 4 .. 7 (SIMD w - 4): 128 columns each, eight fp8 products per step on V^T
//     operands read from the staged codes by 8-bit transposed LDS reads (ds_read_b64_tr_b8);
//     the two half-streams of a row meet here: the accumulator's reference is the larger of
//     the two, and each half's block scale is lowered by its distance to it (powers of two).
//     They also stage the cache: each wave copies 16 rows of every step straight from memory
//     into LDS (direct-to-LDS loads, two steps ahead, three buffers).
// One barrier per step: in step n the output waves issue the loads of step n + 2 (between the
// products, with fp8 value products), multiply step n - 1 and read the V^T operands of step n,
// and wait for step n + 1's loads; the score waves score step n.
#include <type_traits>

#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"
#include "decode_walk.h"

namespace mla {
namespace {

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kRows = 64;      // query rows per workgroup
constexpr int kStep = 64;      // tokens per step (K of the fp8 value product)
constexpr int kHalf = 32;      // tokens per score product (and per block scale)
constexpr int kThreads = 512;  // 4 score and 4 output waves
constexpr int kCols = 128;     // latent columns per output wave
constexpr int kStages = 3;     // staged steps in LDS (loads run two steps ahead)
constexpr int kLoadsPerStep = 11;  // direct-to-LDS loads per output wave and step
constexpr int kMaxPrefixBatch = 2 * kThreads;
// A half-stream's reference max only moves when a half's max exceeds it by more than this
// many base-2 units (it then moves to the ceiling of that max).
constexpr float kTau = 8.f;
static_assert(kMaxInKernelPrefixBatch <= kMaxPrefixBatch, "in-kernel tile prefix does not fit");

enum : int { kContig = 0, kPagedTile = 1, kPagedAny = 2 };

__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }

// Staged code rows are 512 bytes (32 chunks of 16 bytes, every row starting on bank 0); chunk c
// of row t sits at c ^ lat_swz(t), which permutes the low 4 chunk bits.  It is bijective on each
// aligned group of 16 rows (a score read takes one chunk of 16 rows per pass) and, on each
// aligned group of 8 rows, keeps bit 0 and permutes bits 1 .. 3 (a transposed read takes 8 rows
// at chunks c and c ^ 1 per pass: 16 distinct bank groups).
__device__ __forceinline__ int lat_swz(int t) { return ((t & 7) << 1) | ((t >> 3) & 1); }

// Probability rows hold 64 codes (4 chunks of 16 bytes); chunk c of row r sits at
// c ^ p_swz(r): the output waves' 16-byte operand reads (16 rows per pass) hit distinct banks.
__device__ __forceinline__ int p_swz(int row) { return (row >> 2) & 3; }

// Transposed read of 8 bytes: within each 16-lane group, lane 2 r + q supplies the address
// of bytes 8 q .. 8 q + 7 of row r of an 8 x 16 block, and lane j receives column j
// (rows 0 .. 7, row k in byte k).
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p)));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return uint32_t(reinterpret_cast<uintptr_t>(p)); }

// Direct-to-LDS loads (lane i writes LDS bytes [lds + size i, lds + size (i + 1)) from its
// own address, or from a wave-uniform base plus its 32-bit offset), written as inline assembly so that the compiler does not treat later LDS
// reads as dependent on them; completion is awaited explicitly (wait_vm) before the barrier
// that publishes the step.  The LDS address is made wave-uniform; the block carries the wait
// states the hardware needs between the read-first-lane, the M0 write and the load.
__device__ __forceinline__ void dma16(const void* addr, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(m0) : "memory");
}
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
  const uint64_t ps = (uint64_t(hi) << 32) | uint64_t(lo);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(ps), "s"(m0)
               : "memory");
}
// Loads of 4 bytes per lane issued by lanes 0 .. 15 only (called with every lane active): the
// exec mask is narrowed and restored inside the statement, so that no branch splits the
// caller's code and no lane repeats another's address.
__device__ __forceinline__ void dma4_s_16(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
  const uint64_t ps = (uint64_t(hi) << 32) | uint64_t(lo);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  uint64_t saved;
  asm volatile("s_mov_b32 m0, %3\n\ts_mov_b64 %0, exec\n\ts_mov_b64 exec, 0xffff\n\ts_nop 3\n\t"
               "global_load_lds_dword %1, %2\n\ts_mov_b64 exec, %0"
               : "=&s"(saved) : "v"(voff), "s"(ps), "s"(m0) : "memory");
}
__device__ __forceinline__ void dma4_16(const void* addr, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  uint64_t saved;
  asm volatile("s_mov_b32 m0, %2\n\ts_mov_b64 %0, exec\n\ts_mov_b64 exec, 0xffff\n\ts_nop 3\n\t"
               "global_load_lds_dword %1, off\n\ts_mov_b64 exec, %0"
               : "=&s"(saved) : "v"(addr), "s"(m0) : "memory");
}
// Scalar load of one int (a wave-uniform address) and its wait, in one block: a vector load
// would make the compiler wait for every outstanding vector-memory operation, the staged loads
// in flight included.  (The general paged layout does look its rows up with vector loads: its
// loads then wait for the previous step's, which have had a step to arrive.)
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  const uint64_t as = (uint64_t(hi) << 32) | uint64_t(lo);
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(as) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier after this wave's LDS accesses have completed (the direct-to-LDS loads in
// flight are left alone; a fence would wait for them).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct alignas(16) Smem8 {
  uint8_t lat8[kStages][kStep][kDC];   // staged codes, chunk c of row t at c ^ lat_swz(t); also
                                       // the output rows at the end (64 x 1 KB of bf16)
  uint16_t rope[kStages][kStep][kDR];  // staged RoPE rows, chunk c of row t at c ^ rope_swz(t)
  float ts[kStages][kStep];            // per-token scales
  // Probabilities of the step, double buffered: bf16 [row][tok] (8-token chunk c of row r at
  // c ^ p16_swz(r)) for a bf16 value product, or e4m3 codes [row][tok] (16-byte chunk c of row
  // r at c ^ p_swz(r)) in the first 4 KB of each buffer for the fp8 one.
  uint16_t p[2][kRows][kStep];
  int32_t psc[2][kRows][2];            // fp8 values: E8M0 byte of each (row, half) against its stream's reference
  float mref[2][kRows][2];             // reference each half-stream used in the step
  float fin_m[kRows][2], fin_l[kRows][2];
  int64_t prefix[kMaxPrefixBatch + 1];
  int64_t wave_tot[kThreads / 64];
};
static_assert(sizeof(Smem8::lat8) >= kRows * kDC * 2, "output staging does not fit");

__device__ __forceinline__ int p16_swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 v, float f) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = __bf16(float(v[e]) * f);
  return r;
}

// The latent score term is an fp8 product (query rounded per 128-column slice).  PV8: the
// value product in fp8 as well (P rounded with block scales), else in bf16 on the codes
// converted exactly (P times the token scale rounded to bf16).
template <int PK, bool PV8>
__device__ __forceinline__ void decode_piece8(Smem8& sm, const DecodeArgs& a, int b, int rb, int t_lo, int t_hi,
                                              int L, bool final_out, int64_t out_base) {
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(int(threadIdx.x)));
  const int lane = tid & 63, cn = lane & 31, ch = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rows = a.sq * a.H;
  const int r0 = rb * kRows;
  const int nsteps = t_hi > t_lo ? (t_hi - t_lo + kStep - 1) / kStep : 0;
  uint8_t(*p8)[kRows][kStep] = reinterpret_cast<uint8_t(*)[kRows][kStep]>(&sm.p[0][0][0]);
  auto p8buf = [&](int buf) { return reinterpret_cast<uint8_t(*)[kStep]>(reinterpret_cast<uint8_t*>(&sm.p[buf][0][0])); };
  (void)p8;

  if (w < 4) {
    // ================================ score waves ====================================
    const int hf = w >> 1;             // this wave's half of every step
    const int row = 32 * (w & 1) + cn;  // this lane's row of the workgroup
    // Query operands: q8[m] = the e4m3 codes of columns 64 m + 32 h .. + 31, rounded with the
    // scale qs[m / 2] of their 128-column slice (the partner lane holds the slice's other
    // half); qr[s] = RoPE dims 16 s + 8 h .. + 7 (bf16).
    bf16x8 qr[4];
    v8i q8[8];
    float qs[4];
    {
      const int64_t qrow = int64_t(b) * rows + r0 + row;
      const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + qrow * kDC;
      const uint16_t* qp = static_cast<const uint16_t*>(a.q_rope) + qrow * kDR + 8 * ch;
#pragma unroll
      for (int s = 0; s < 4; ++s) qr[s] = __builtin_bit_cast(bf16x8, ld16(qp + 16 * s));
      {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8 x[8];  // x[4 mm + i]: columns 128 j + 64 mm + 32 h + 8 i .. + 7
#pragma unroll
          for (int i = 0; i < 8; ++i)
            x[i] = __builtin_bit_cast(bf16x8, ld16(ql + 128 * j + 64 * (i >> 2) + 32 * ch + 8 * (i & 3)));
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(float(x[i][e])));
          amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
          qs[j] = amax > 0.f ? amax * (1.f / 448.f) : 1.f;
          const float inv = amax > 0.f ? 448.f / amax : 1.f;
#pragma unroll
          for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int d = 0; d < 8; ++d) {  // dword d: columns 64 m + 32 h + 4 d .. + 3
              const bf16x8 src = x[4 * mm + d / 2];
              const int o = 4 * (d % 2);
              auto qf = [&](int e) { return fminf(fmaxf(float(src[o + e]) * inv, -448.f), 448.f); };
              int wd = __builtin_amdgcn_cvt_pk_fp8_f32(qf(0), qf(1), 0, false);
              wd = __builtin_amdgcn_cvt_pk_fp8_f32(qf(2), qf(3), wd, true);
              q8[2 * j + mm][d] = wd;
            }
        }
      }
    }
    const int iq = (r0 + row) / a.H;
    const int lim = min(min(max(L - a.sq + iq + 1, 0), L), t_hi);
    const int iq_w = (r0 + 32 * (w & 1)) / a.H;
    const int lim_w = min(min(max(L - a.sq + iq_w + 1, 0), L), t_hi);
    float ref = -INFINITY, l_run = 0.f;  // this half-stream's reference and sum
    const float scale_log2 = a.scale_log2;

    // Operand offsets within the half (token n of the half is row 32 hf + n of the step; the
    // swizzles depend on the low 4 row bits only): code product m reads chunks 4 m + 2 h and
    // 4 m + 2 h + 1 of token n; RoPE k-step s reads chunk (2 s + h) ^ rope_swz(n).
    int boff[8];  // [2 (m % 4) + e]: chunk 4 (m % 4) + 2 h + e, plus 256 bytes per 4 products
#pragma unroll
    for (int t = 0; t < 8; ++t) boff[t] = cn * kDC + 16 * ((4 * (t >> 1) + 2 * ch + (t & 1)) ^ lat_swz(cn));
    int roff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) roff[t] = cn * kDR + 8 * ((2 * t + ch) ^ rope_swz(cn));

    auto score = [&](int n) {
      const int buf = n % kStages;
      const int pbuf = n & 1;
      // bf16 values: the two half-streams share a reference (the larger of their references
      // of the last step), so that they differ only in a step where one of them moves its own
      // and the output waves rarely rescale probabilities.  fp8 values absorb any difference
      // in the block scales, and each stream keeps its own.
      if (!PV8 && n > 0) {
        const float R = fmaxf(sm.mref[pbuf ^ 1][row][0], sm.mref[pbuf ^ 1][row][1]);
        if (R > ref) {
          l_run = ref == -INFINITY ? 0.f : l_run * __builtin_amdgcn_ldexpf(1.f, int(ref - R));
          ref = R;
        }
      }
      const uint8_t* l8 = &sm.lat8[buf][kHalf * hf][0];
      const uint16_t* rt = &sm.rope[buf][kHalf * hf][0];
      f32x16 accr, accq[4];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        accr[e] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) accq[j][e] = 0.f;
      }
      {
        auto codes = [&](int m) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(l8 + 256 * (m >> 2) + boff[2 * (m & 3)]);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(l8 + 256 * (m >> 2) + boff[2 * (m & 3) + 1]);
          return v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
        };
        // Eight fp8 products (one accumulator per 128-column slice), codes read two products
        // ahead, then the four bf16 RoPE products.
        v8i ring8[2] = {codes(0), codes(1)};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const v8i av = ring8[m & 1];
          if (m + 2 < 8) ring8[m & 1] = codes(m + 2);
          accq[m >> 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, q8[m], accq[m >> 1], 0, 0, 0, 127, 0, 127);
        }
        bf16x8 ar[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) ar[s] = *reinterpret_cast<const bf16x8*>(rt + roff[s]);
#pragma unroll
        for (int s = 0; s < 4; ++s) accr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[s], qr[s], accr, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
      // Lane (n, h) holds tokens 8 i + 4 h + r (e = 4 i + r) of row `row` in this half.
      f32x4 tsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) tsv[i] = *reinterpret_cast<const f32x4*>(&sm.ts[buf][kHalf * hf + 8 * i + 4 * ch]);
      float sv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float lat = qs[0] * accq[0][e] + qs[1] * accq[1][e] + qs[2] * accq[2][e] + qs[3] * accq[3][e];
        sv[e] = fmaf(lat, tsv[e >> 2][e & 3], accr[e]);
      }
      const int t0 = t_lo + n * kStep + kHalf * hf;
      if (t0 + kHalf > lim_w) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (t0 + 8 * (e >> 2) + 4 * ch + (e & 3) >= lim) sv[e] = -INFINITY;
      }
      float tmax = sv[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sv[e]);
      {
        float x0 = tmax, x1 = tmax;
        permlane32_swap(x0, x1);
        tmax = fmaxf(x0, x1);
      }
      tmax *= scale_log2;
      if (tmax > ref + kTau) {
        const float r_new = ceilf(tmax);
        l_run = ref == -INFINITY ? 0.f : l_run * __builtin_amdgcn_ldexpf(1.f, int(ref - r_new));
        ref = r_new;
      }
      const float neg_m = ref == -INFINITY ? 0.f : -ref;
      float pw[16], psum = 0.f, pmax = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, neg_m));
        psum += pe;
        pw[e] = pe * tsv[e >> 2][e & 3];
        if constexpr (PV8) pmax = fmaxf(pmax, pw[e]);
      }
      l_run += psum;
      if constexpr (PV8) {
        {
          float x0 = pmax, x1 = pmax;
          permlane32_swap(x0, x1);
          pmax = fmaxf(x0, x1);
        }
        // Block scale 2^e with e = floor(log2 pmax) - 7: E8M0 byte bexp - 7 (at least 0), and
        // the values are multiplied by 2^-e before rounding.
        const int sbyte = max(int((__float_as_uint(pmax) >> 23) & 0xFF) - 7, 0);
        const float mul = __uint_as_float(uint32_t(254 - sbyte) << 23);
        const int g = p_swz(row);
        uint8_t(*pp)[kStep] = p8buf(pbuf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int wd = __builtin_amdgcn_cvt_pk_fp8_f32(pw[4 * i] * mul, pw[4 * i + 1] * mul, 0, false);
          wd = __builtin_amdgcn_cvt_pk_fp8_f32(pw[4 * i + 2] * mul, pw[4 * i + 3] * mul, wd, true);
          const int chunk = 2 * hf + (i >> 1);
          *reinterpret_cast<int*>(&pp[row][16 * (chunk ^ g) + 8 * (i & 1) + 4 * ch]) = wd;
        }
        if (ch == 0) sm.psc[pbuf][row][hf] = sbyte;
      } else {
        const int g = p16_swz(row);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x2*>(&sm.p[pbuf][row][8 * ((4 * hf + i) ^ g) + 4 * ch]) =
              u32x2{pack_bf16x2(pw[4 * i], pw[4 * i + 1]), pack_bf16x2(pw[4 * i + 2], pw[4 * i + 3])};
      }
      if (ch == 0) sm.mref[pbuf][row][hf] = ref;
    };
    if (nsteps > 0) {
      barrier_lds();  // step 0 staged
      for (int n = 0; n < nsteps; ++n) {
        score(n);
        barrier_lds();
      }
    }
    // This stream's sum over both lane halves; the two streams of a row meet after the barrier.
    float x0 = l_run, x1 = l_run;
    permlane32_swap(x0, x1);
    if (ch == 0) {
      sm.fin_m[row][hf] = ref;
      sm.fin_l[row][hf] = x0 + x1;
    }
    __syncthreads();  // row sums published
    if (hf == 0 && ch == 0) {
      const float m0 = sm.fin_m[row][0], m1 = sm.fin_m[row][1];
      const float M = fmaxf(m0, m1);
      float lt = 0.f;
      if (M != -INFINITY) {
        if (m0 != -INFINITY) lt += sm.fin_l[row][0] * __builtin_amdgcn_ldexpf(1.f, int(m0 - M));
        if (m1 != -INFINITY) lt += sm.fin_l[row][1] * __builtin_amdgcn_ldexpf(1.f, int(m1 - M));
      }
      const float lse2 = lt > 0.f ? M + log2f(lt) : -INFINITY;
      if (final_out) {
        if (a.lse) a.lse[out_base + r0 + row] = lse2 * kLn2;
      } else {
        a.part_lse[out_base + r0 + row] = lse2;
      }
    }
  } else {
    // ================================ output waves ===================================
    const int q = w - 4;  // column quarter and share of the staged rows
    // ---------------------------------------------------------------- staging
    // Wave q stages rows 16 q .. 16 q + 15 of every step (tokens past the piece's last one
    // are clamped to it; the softmax masks them): latent rows two per load (lane i: row
    // 16 q + 2 k + i / 32, 16-byte chunk i % 32 fetched from chunk (i % 32) ^ lat_swz(row)), RoPE
    // rows eight per load (lane i: row 16 q + 8 k + i / 8, chunk (i % 8) ^ rope_swz(row)) and
    // the 16 scales (lanes 0 .. 15).
    const char* lat_g = static_cast<const char*>(a.c_kv);
    const char* rope_g = static_cast<const char*>(a.k_rope);
    const char* ts_g = reinterpret_cast<const char*>(a.kv_scale);
    const int32_t* tab = a.block_table + int64_t(b) * a.max_blocks;
    // A step's 11 loads per output wave: stage_prep once, then stage_part(k), k = 0 .. 10 (8
    // latent loads, 2 RoPE loads, the scales); stage issues all 11 at once.  With fp8 value
    // products they are spread between the products instead: a burst of 44 per compute unit
    // queues every output wave on the address unit (about one 64-byte line per clock).
    struct StageCtx {
      const char* lat_b;
      const char* rope_b;
      const char* ts_b;
      int tq, t_base, buf;
    };
    auto stage_prep = [&](int n) {
      StageCtx sc;
      sc.tq = t_lo + n * kStep + 16 * q;  // token of this wave's first row
      sc.buf = n % kStages;
      sc.lat_b = lat_g;
      sc.rope_b = rope_g;
      sc.ts_b = ts_g;
      sc.t_base = 0;
      if constexpr (PK != kPagedAny) {
        // One base per wave and step (the sequence, or the block holding the wave's 16 rows
        // and the clamp target: block_size a multiple of 32, halves 32-aligned), 32-bit
        // offsets from it (a sequence's rows span less than 2 GiB).
        int64_t base_row;
        if constexpr (PK == kContig) {
          base_row = int64_t(b) * a.T;
        } else {
          const int blk = min(sc.tq, t_hi - 1) / a.block_size;
          base_row = int64_t(sload_i32(tab + blk)) * a.block_size;
          sc.t_base = blk * a.block_size;
        }
        sc.lat_b = lat_g + base_row * kDC;
        sc.rope_b = rope_g + base_row * (kDR * 2);
        sc.ts_b = ts_g + base_row * 4;
      }
      return sc;
    };
    auto stage_part = [&](const StageCtx& sc, int k) {
      const int tl = t_hi - 1;
      // row 16 q + j of the step: its cache row (general paged layout, looked up lane by
      // lane) or its offset from the step's base
      auto crow = [&](int j) -> int64_t {
        const int t = min(sc.tq + j, tl);
        return int64_t(tab[t / a.block_size]) * a.block_size + t % a.block_size;
      };
      auto roff = [&](int j) { return uint32_t(min(sc.tq + j, tl) - sc.t_base); };
      if (k < 8) {
        const int j = 2 * k + ch;
        const uint32_t dst = lds_addr(&sm.lat8[sc.buf][16 * q + 2 * k][0]);
        const int chunk = cn ^ lat_swz(16 * q + j);
        if constexpr (PK == kPagedAny)
          dma16(lat_g + crow(j) * kDC + 16 * chunk, dst);
        else
          dma16_s(sc.lat_b, roff(j) * kDC + uint32_t(16 * chunk), dst);
      } else if (k < 10) {
        const int j = 8 * (k - 8) + (lane >> 3);
        const uint32_t dst = lds_addr(&sm.rope[sc.buf][16 * q + 8 * (k - 8)][0]);
        const int chunk = (lane & 7) ^ rope_swz(16 * q + j);
        if constexpr (PK == kPagedAny)
          dma16(rope_g + crow(j) * (kDR * 2) + 16 * chunk, dst);
        else
          dma16_s(sc.rope_b, roff(j) * (kDR * 2) + uint32_t(16 * chunk), dst);
      } else {
        const uint32_t dst = lds_addr(&sm.ts[sc.buf][16 * q]);
        if constexpr (PK == kPagedAny)
          dma4_16(ts_g + crow(lane & 15) * 4, dst);
        else
          dma4_s_16(sc.ts_b, roff(lane & 15) * 4, dst);
      }
    };
    auto stage = [&](int n) {
      const StageCtx sc = stage_prep(n);
#pragma unroll
      for (int k = 0; k < kLoadsPerStep; ++k) stage_part(sc, k);
    };

    // ---------------------------------------------------------------- value product
    f32x16 oacc[4][2];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[cb][rb2][e] = 0.f;
    // V^T operands of column block cb, read from the staged codes by 8-bit transposed reads
    // (the 16-lane group G covers columns 16 (G & 1) + (0..15) of 8 tokens, lane gi receiving
    // column gi).  fp8 values (A of the 32 x 32 x 64 product): lane l holds column
    // 128 q + 32 cb + l % 32 and, in the instruction's K order, tokens 16 h .. 16 h + 15 of the
    // step in bytes 0 .. 15 and 32 + 16 h .. 32 + 16 h + 15 in bytes 16 .. 31; read j covers
    // tokens 16 (G >> 1) + 8 (j & 1) + 32 (j >> 1) + (0..7).  bf16 values (A of 32 x 32 x 16,
    // converted before the product): k-step ks takes tokens 16 ks + 8 h + (0..7), read j = ks.
    // A token's swizzle depends on its low 4 bits only, so the reads differ by immediate
    // offsets plus, for fp8, one of two bases.  Column block cb's chunk is u + 2 cb with
    // u = 8 q + (G & 1) (bits 1 and 2 clear), so its swizzled byte offset is 16 ((u ^ swz) ^ 2 cb):
    // the base XORed with 32 cb.
    const int G = lane >> 4, gi = lane & 15;
    const int tok0 = (PV8 ? 16 : 8) * (G >> 1) + (gi >> 1);
    const int u = 8 * q + (G & 1);
    int vb[2];
#pragma unroll
    for (int jo = 0; jo < 2; ++jo) {
      const int tk = tok0 + (PV8 ? 8 * jo : 0);
      vb[jo] = tk * kDC + 8 * (gi & 1) + 16 * (u ^ lat_swz(tk));
    }
    v8i vop[4];
    auto read_v = [&](int n) {
      const uint8_t* vt = &sm.lat8[n % kStages][0][0];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int off = PV8 ? (vb[j & 1] ^ (32 * cb)) + 32 * (j >> 1) * kDC : (vb[0] ^ (32 * cb)) + 16 * j * kDC;
          const u32x2 v = lds_read_tr8(vt + off);
          vop[cb][2 * j] = int(v[0]);
          vop[cb][2 * j + 1] = int(v[1]);
        }
    };
    float m_acc[2] = {-INFINITY, -INFINITY};  // the accumulator's reference of rows 32 rb2 + n
    // issue_c: std::true_type to spread the loads of sc_next's step over the fp8 value products
    // (a compile-time choice, so that no branch splits the products from the loads)
    auto pv = [&](int n, auto issue_c, const StageCtx& sc_next) {
      constexpr bool issue = decltype(issue_c)::value;
      const int buf = n & 1;
      float al[2], f[2][2];
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2) {
        const int prow = 32 * rb2 + cn;
        const float m0 = sm.mref[buf][prow][0], m1 = sm.mref[buf][prow][1];
        const float mn = fmaxf(m0, m1);
        al[rb2] = mn == m_acc[rb2] ? 1.f
                  : m_acc[rb2] == -INFINITY ? 0.f
                                            : __builtin_amdgcn_ldexpf(1.f, int(m_acc[rb2] - mn));
        m_acc[rb2] = mn;
        f[rb2][0] = (m0 == mn || m0 == -INFINITY) ? 1.f : __builtin_amdgcn_ldexpf(1.f, int(m0 - mn));
        f[rb2][1] = (m1 == mn || m1 == -INFINITY) ? 1.f : __builtin_amdgcn_ldexpf(1.f, int(m1 - mn));
      }
      if (__any((al[0] != 1.f) | (al[1] != 1.f))) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2) oacc[cb][rb2] *= al[rb2];
      }
      if constexpr (PV8) {
        int sc[2];
        v8i pb[2];
#pragma unroll
        for (int rb2 = 0; rb2 < 2; ++rb2) {
          const int prow = 32 * rb2 + cn;
          // This lane's half: its block scale, lowered by the stream's distance to the
          // accumulator's reference (exact: integers in base 2).
          const float mh = ch ? sm.mref[buf][prow][1] : sm.mref[buf][prow][0];
          sc[rb2] = mh == -INFINITY ? 0 : max(sm.psc[buf][prow][ch] + int(mh - m_acc[rb2]), 0);
          // B operand (P^T): row prow, tokens 16 h .. + 15 (chunk h) and 32 + 16 h .. + 15
          // (chunk 2 + h), in the instruction's K order; the lane's scale is that of half h.
          const uint8_t* pr = &p8buf(buf)[prow][0];
          const u32x4 lo = *reinterpret_cast<const u32x4*>(pr + 16 * (ch ^ p_swz(prow)));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(pr + 16 * ((2 + ch) ^ p_swz(prow)));
          pb[rb2] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
        }
        // One load of the step two ahead after each product (the last three after the last).
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2) {
            const int i = 2 * cb + rb2;
            oacc[cb][rb2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[cb], pb[rb2], oacc[cb][rb2], 0, 0, 0,
                                                                            127, 0, sc[rb2]);
            if constexpr (issue) {
              stage_part(sc_next, i);
              if (i == 7)
                for (int k = 8; k < kLoadsPerStep; ++k) stage_part(sc_next, k);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      } else {
        // B operand (P^T) of k-step ks: row prow, tokens 16 ks + 8 h .. + 7 (chunk 2 ks + h);
        // k-steps 0, 1 belong to half 0, 2, 3 to half 1, scaled by that half's distance to
        // the accumulator's reference when one moved on its own in this step.
        const bool scale_p = __any((f[0][0] != 1.f) | (f[0][1] != 1.f) | (f[1][0] != 1.f) | (f[1][1] != 1.f));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 pb[2];
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2) {
            const int prow = 32 * rb2 + cn;
            pb[rb2] = *reinterpret_cast<const bf16x8*>(&sm.p[buf][prow][8 * ((2 * ks + ch) ^ p16_swz(prow))]);
            if (scale_p) pb[rb2] = scale_bf16x8(pb[rb2], f[rb2][ks >> 1]);
          }
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(uint32_t(vop[cb][2 * ks]),
                                                                           uint32_t(vop[cb][2 * ks + 1])));
#pragma unroll
            for (int rb2 = 0; rb2 < 2; ++rb2)
              oacc[cb][rb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[rb2], oacc[cb][rb2], 0, 0, 0);
          }
        }
      }
    };
    if (nsteps > 0) {
      // Loads run two steps ahead: step k goes to buffer k % 3 in step k - 2 (the prologue
      // issues steps 0 and 1), and each step ends by waiting for the next one's loads.
      stage(0);
      if (nsteps > 1) {
        stage(1);
        wait_vm<kLoadsPerStep>();
      } else {
        wait_vm<0>();
      }
      barrier_lds();  // step 0 staged
      // Step n: the products of step n - 1 (with the loads of step n + 2 while there is one),
      // then step n's values read, then wait for step n + 1's loads.
      auto step_end = [&](int n) {
        __builtin_amdgcn_sched_barrier(0);
        read_v(n);
        if (n + 2 < nsteps) wait_vm<kLoadsPerStep>();
        else wait_vm<0>();
        barrier_lds();  // step n scored, step n + 1 staged
      };
      const StageCtx none{};
      // The loads are spread over the fp8 value products (8 short products, each followed by
      // one or more loads).  The bf16 value product keeps the burst: spread over its 32
      // products it measured slower (946 against 885 us on the speculative fp8 workload).
      // The general paged layout looks its rows up lane by lane (vector loads the compiler
      // waits for), so it keeps the burst too.
      constexpr bool kSpread = PV8 && PK != kPagedAny;
      if (nsteps > 2) stage(2);
      step_end(0);
      int n = 1;
      if constexpr (kSpread) {
        for (; n + 2 < nsteps; ++n) {
          pv(n - 1, std::true_type{}, stage_prep(n + 2));
          __builtin_amdgcn_sched_barrier(0);
          read_v(n);
          wait_vm<kLoadsPerStep>();
          barrier_lds();
        }
      }
      // Otherwise a step's loads go out in one burst, and so do the last two steps'.
      for (; n < nsteps; ++n) {
        if (n + 2 < nsteps) stage(n + 2);
        pv(n - 1, std::false_type{}, none);
        step_end(n);
      }
      pv(nsteps - 1, std::false_type{}, none);
    }
    __syncthreads();  // row sums published
    float lt[2];
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2) {
      const int prow = 32 * rb2 + cn;
      const float m0 = sm.fin_m[prow][0], m1 = sm.fin_m[prow][1];
      lt[rb2] = 0.f;
      if (m_acc[rb2] != -INFINITY) {
        if (m0 != -INFINITY) lt[rb2] += sm.fin_l[prow][0] * __builtin_amdgcn_ldexpf(1.f, int(m0 - m_acc[rb2]));
        if (m1 != -INFINITY) lt[rb2] += sm.fin_l[prow][1] * __builtin_amdgcn_ldexpf(1.f, int(m1 - m_acc[rb2]));
      }
    }
    uint16_t* os = reinterpret_cast<uint16_t*>(&sm.lat8[0][0][0]);
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2) {
      const float inv = lt[rb2] > 0.f ? 1.f / lt[rb2] : 0.f;
      const int lrow = 32 * rb2 + cn;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int chunk = 16 * q + 4 * cb + i;
          const f32x4 v = f32x4{oacc[cb][rb2][4 * i], oacc[cb][rb2][4 * i + 1], oacc[cb][rb2][4 * i + 2],
                                oacc[cb][rb2][4 * i + 3]} * inv;
          *reinterpret_cast<u32x2*>(os + lrow * kDC + 8 * (chunk ^ (lrow & 15)) + 4 * ch) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    }
  }
  __syncthreads();
  {
    const uint16_t* os = reinterpret_cast<const uint16_t*>(&sm.lat8[0][0][0]);
    uint16_t* dst = static_cast<uint16_t*>(final_out ? a.o_lat : a.part_o);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int lrow = 8 * w + k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + lrow * kDC + 8 * (lane ^ (lrow & 15)));
      *reinterpret_cast<u32x4*>(dst + (out_base + r0 + lrow) * kDC + 8 * lane) = v;
    }
  }
  __syncthreads();  // the next piece stages into these buffers
}

// Launch bounds: 512 threads and at least 2 waves per SIMD, i.e. one 8-wave workgroup per
// compute unit (the kernel's LDS allows one); each wave may then hold up to 256 registers.
template <int PK, bool PV8>
__global__ __launch_bounds__(kThreads, 2) void decode_fp8_kernel(DecodeArgs a, int num_splits, int chunk,
                                                                 int rblocks, int n_units, int n_xcd) {
  __shared__ Smem8 sm;
  walk_pieces<32, kThreads>(a, num_splits, chunk, rblocks, n_units, n_xcd, sm.prefix, sm.wave_tot,
                            [&](int b, int rb, int t_lo, int t_hi, int L, bool fin, int64_t base)
                                __attribute__((always_inline)) {
                                  decode_piece8<PK, PV8>(sm, a, b, rb, t_lo, t_hi, L, fin, base);
                                });
}

template <int PK, bool PV8>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = p.rows / kRows;
  const int n_units = p.balanced ? p.num_splits * rblocks : a.B * p.num_splits * rblocks;
  const int n_xcd = p.n_xcd > 0 ? p.n_xcd : 1;
  const int grid = (n_units + n_xcd - 1) / n_xcd * n_xcd;
  hipLaunchKernelGGL((decode_fp8_kernel<PK, PV8>), dim3(grid), dim3(kThreads), 0, s, a, p.num_splits,
                     p.split_tokens, rblocks, n_units, n_xcd);
  return int(hipGetLastError());
}

}  // namespace

int launch_decode_fp8(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  if (a.kv_dt != MLA_FP8_E4M3 || p.rows % kRows) return int(hipErrorInvalidValue);
  const int pk = !a.paged ? kContig : a.block_size % kHalf == 0 ? kPagedTile : kPagedAny;
  auto by_layout = [&](auto pv8) {
    constexpr bool V = decltype(pv8)::value;
    if (pk == kContig) return launch_t<kContig, V>(a, p, s);
    return pk == kPagedTile ? launch_t<kPagedTile, V>(a, p, s) : launch_t<kPagedAny, V>(a, p, s);
  };
  if (a.fp8_scores == 2) return by_layout(std::true_type{});
  if (a.fp8_scores == 1) return by_layout(std::false_type{});
  return int(hipErrorInvalidValue);
}

}  // namespace mla
