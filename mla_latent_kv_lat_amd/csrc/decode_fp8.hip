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
// sequence and walks its piece of the context in 64-token steps.  Eight waves, three roles:
//   * loader waves 4, 5 (SIMDs 0, 1): wave 4 + l loads tokens 32 l .. 32 l + 31 of every
//     step (512-byte code rows, 128-byte RoPE rows, the scales; 16 bytes per lane, two steps
//     ahead in registers) and stages them in LDS as they are;
//   * score waves 0, 1 (SIMDs 0, 1): wave w owns rows 32 w .. 32 w + 31 and scores the
//     step's two 32-token halves one after the other (eight fp8 and four bf16 products
//     each), runs the online softmax on each in registers and publishes the rounded
//     probabilities with their block scales;
//   * output waves 2, 3, 6, 7 (SIMDs 2, 3): 128 columns each, eight fp8 products per step;
//     the V^T operands come from the staged codes by 8-bit transposed LDS reads
//     (ds_read_b64_tr_b8) one step ahead.
// One barrier per step, as in the bf16-value kernel: in step n the loaders stage step n + 1
// (and load step n + 3), the score waves score step n, the output waves multiply step n - 1
// and read the V^T operands of step n.
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
constexpr int kThreads = 512;  // 2 score, 2 loader and 4 output waves
constexpr int kCols = 128;     // latent columns per output wave
constexpr int kMaxPrefixBatch = 2 * kThreads;
// The reference max only moves when a half's max exceeds it by more than this many base-2
// units (it then moves to the ceiling of that max).
constexpr float kTau = 8.f;
static_assert(kMaxInKernelPrefixBatch <= kMaxPrefixBatch, "in-kernel tile prefix does not fit");

enum : int { kContig = 0, kPagedTile = 1, kPagedAny = 2 };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buf_ld4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }

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

struct Ctx {
  int b, lane, n, h, w;
  int t_hi;
  const int32_t* table;
  int max_blocks, bs;
  int64_t T;
};

__device__ __forceinline__ int64_t any_row(const Ctx& c, int t) {
  const int tc = min(t, c.t_hi - 1);
  return int64_t(c.table[int64_t(c.b) * c.max_blocks + tc / c.bs]) * c.bs + tc % c.bs;
}

// Staged steps are double buffered (loaders write buffer (n + 1) % 2 in step n).
struct alignas(16) Smem8 {
  uint8_t lat8[2][kStep][kDC];      // staged codes, chunk c of row t at c ^ swz32(t); also
                                    // the output rows at the end (64 x 1 KB of bf16)
  uint16_t rope[2][kStep][kDR];     // staged RoPE rows, chunk c of row t at c ^ rope_swz(t)
  uint8_t p8[2][kRows][kStep];      // rounded probabilities [row][tok], p_swz
  int32_t psc[2][kRows][2];         // E8M0 scale of each row's two 32-token halves
  float ts[2][kStep];               // per-token scales
  float alpha[2][kRows];            // rescale of the accumulators before the step
  float lsum[kRows];
  int64_t prefix[kMaxPrefixBatch + 1];
  int64_t wave_tot[kThreads / 64];
};
static_assert(sizeof(Smem8::lat8) >= kRows * kDC * 2, "output staging does not fit");

// A loader wave's registers for its 32 tokens of one step.
struct Load8 {
  u32x4 lat[16];  // load k: token 2 k + lane / 32, 16-byte chunk lane % 32
  u32x4 rope[4];  // load j: token 8 j + lane / 8, 16-byte chunk lane % 8
  float ts;       // scale of token lane % 32
};

template <int PK>
__device__ __forceinline__ void decode_piece8(Smem8& sm, const DecodeArgs& a, int b, int rb, int t_lo, int t_hi,
                                              int L, bool final_out, int64_t out_base) {
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(int(threadIdx.x)));
  Ctx c;
  c.b = b;
  c.lane = tid & 63;
  c.n = c.lane & 31;
  c.h = c.lane >> 5;
  c.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.table = a.block_table;
  c.max_blocks = a.max_blocks;
  c.bs = a.block_size;
  c.T = a.T;
  c.t_hi = t_hi;
  const int rows = a.sq * a.H;
  const int r0 = rb * kRows;
  const int nsteps = t_hi > t_lo ? (t_hi - t_lo + kStep - 1) / kStep : 0;

  if (c.w == 4 || c.w == 5) {
    // ================================ loader waves ===================================
    const int l = c.w - 4;
    auto lload = [&](Load8& r, int t0) {
      const int th = t0 + kHalf * l;
      if constexpr (PK == kPagedAny) {
        const char* lat = static_cast<const char*>(a.c_kv);
        const char* rope = static_cast<const char*>(a.k_rope);
#pragma unroll
        for (int k = 0; k < 16; ++k) r.lat[k] = ld16(lat + any_row(c, th + 2 * k + c.h) * kDC + 16 * c.n);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          r.rope[j] = ld16(rope + any_row(c, th + 8 * j + (c.lane >> 3)) * (kDR * 2) + 16 * (c.lane & 7));
        r.ts = a.kv_scale[any_row(c, th + c.n)];
        return;
      }
      const char* lat_base;
      const char* rope_base;
      const char* sc_base;
      uint32_t nrows, row0;
      if constexpr (PK == kContig) {
        const int64_t seq_row = int64_t(c.b) * c.T;
        lat_base = static_cast<const char*>(a.c_kv) + seq_row * kDC;
        rope_base = static_cast<const char*>(a.k_rope) + seq_row * (kDR * 2);
        sc_base = reinterpret_cast<const char*>(a.kv_scale + seq_row);
        nrows = uint32_t(c.t_hi);
        row0 = uint32_t(th);
      } else {
        // The half lies inside one block (block_size a multiple of 32, th a multiple of 32).
        const int blk = min(th, c.t_hi - 1) / c.bs;
        const int blk_t0 = blk * c.bs;
        const int64_t pool_row = int64_t(c.table[int64_t(c.b) * c.max_blocks + blk]) * c.bs;
        lat_base = static_cast<const char*>(a.c_kv) + pool_row * kDC;
        rope_base = static_cast<const char*>(a.k_rope) + pool_row * (kDR * 2);
        sc_base = reinterpret_cast<const char*>(a.kv_scale + pool_row);
        nrows = uint32_t(min(c.bs, c.t_hi - blk_t0));
        row0 = uint32_t(th - blk_t0);
      }
      // Ranges end at the last valid row: rows past it read zeros.
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(lat_base, nrows * kDC);
      const __amdgpu_buffer_rsrc_t rr = make_rsrc(rope_base, nrows * (kDR * 2));
#pragma unroll
      for (int k = 0; k < 16; ++k) r.lat[k] = buf_ld16(rl, (row0 + uint32_t(2 * k + c.h)) * kDC + 16 * c.n);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r.rope[j] = buf_ld16(rr, (row0 + uint32_t(8 * j + (c.lane >> 3))) * (kDR * 2) + 16 * (c.lane & 7));
      r.ts = buf_ld4f(make_rsrc(sc_base, nrows * 4), (row0 + uint32_t(c.n)) * 4);
    };
    auto lstage = [&](const Load8& r, int buf) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int row = kHalf * l + 2 * k + c.h;
        *reinterpret_cast<u32x4*>(&sm.lat8[buf][row][16 * (c.n ^ swz32(row))]) = r.lat[k];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = kHalf * l + 8 * j + (c.lane >> 3);
        *reinterpret_cast<u32x4*>(&sm.rope[buf][row][8 * ((c.lane & 7) ^ rope_swz(row))]) = r.rope[j];
      }
      if (c.h == 0) sm.ts[buf][kHalf * l + c.n] = r.ts;
    };
    if (nsteps > 0) {
      Load8 rx, ry;  // rx holds the even steps, ry the odd ones
      lload(rx, t_lo);
      lload(ry, t_lo + kStep);
      lstage(rx, 0);
      lload(rx, t_lo + 2 * kStep);
      __syncthreads();
      // Step n stages step n + 1 and loads step n + 3 in its place.
      auto lstep = [&](Load8& r, int n) {
        if (n + 1 < nsteps) lstage(r, (n + 1) % 2);
        lload(r, t_lo + (n + 3) * kStep);
        __syncthreads();
      };
      int n = 0;
      for (; n + 1 < nsteps; n += 2) {
        lstep(ry, n);
        lstep(rx, n + 1);
      }
      if (n < nsteps) lstep(ry, n);
    }
    __syncthreads();  // row sums published
  } else if (c.w < 2) {
    // ================================ score waves ====================================
    const int row = 32 * c.w + c.n;  // this lane's row of the workgroup
    // Query operands: q8[m] = the e4m3 codes of columns 64 m + 32 h .. + 31, rounded with the
    // scale qs[m / 2] of their 128-column slice (the partner lane holds the slice's other
    // half); qr[s] = RoPE dims 16 s + 8 h .. + 7 (bf16).
    bf16x8 qr[4];
    v8i q8[8];
    float qs[4];
    {
      const int64_t qrow = int64_t(b) * rows + r0 + row;
      const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + qrow * kDC;
      const uint16_t* qp = static_cast<const uint16_t*>(a.q_rope) + qrow * kDR + 8 * c.h;
#pragma unroll
      for (int s = 0; s < 4; ++s) qr[s] = __builtin_bit_cast(bf16x8, ld16(qp + 16 * s));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 x[8];  // x[4 mm + i]: columns 128 j + 64 mm + 32 h + 8 i .. + 7
#pragma unroll
        for (int i = 0; i < 8; ++i)
          x[i] = __builtin_bit_cast(bf16x8, ld16(ql + 128 * j + 64 * (i >> 2) + 32 * c.h + 8 * (i & 3)));
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
    const int iq = (r0 + row) / a.H;
    const int lim = min(min(max(L - a.sq + iq + 1, 0), L), t_hi);
    const int iq_w = (r0 + 32 * c.w) / a.H;
    const int lim_w = min(min(max(L - a.sq + iq_w + 1, 0), L), t_hi);
    float m_run = -INFINITY, l_run = 0.f;
    const float scale_log2 = a.scale_log2;

    // Operand offsets within a half (token n of the half is row 32 hf + n of the step; the
    // swizzles depend on the low 4 row bits only): code product m reads chunks
    // 4 m + 2 h, 4 m + 2 h + 1 of token n; RoPE k-step s chunk (2 s + h) ^ rope_swz(n).
    int boff[8];  // [2 (m % 4) + e]: chunk 4 (m % 4) + 2 h + e, plus 256 bytes per 4 products
#pragma unroll
    for (int t = 0; t < 8; ++t) boff[t] = c.n * kDC + 16 * ((4 * (t >> 1) + 2 * c.h + (t & 1)) ^ swz32(c.n));
    int roff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) roff[t] = c.n * kDR + 8 * ((2 * t + c.h) ^ rope_swz(c.n));
    const int prow_off = 4 * c.h;  // byte of this lane's 4 tokens within an 8-token group

    // Scores, softmax and rounded probabilities of half hf of step n.  Returns the half's
    // E8M0 block scale (before any later rescale) and sets alpha to the accumulator rescale.
    auto half = [&](int n, int hf, float& alpha) -> int {
      const int buf = n % 2;
      const uint8_t* l8 = &sm.lat8[buf][kHalf * hf][0];
      const uint16_t* rt = &sm.rope[buf][kHalf * hf][0];
      f32x16 accr, accq[4];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        accr[e] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) accq[j][e] = 0.f;
      }
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
      // Lane (n, h) holds tokens 8 i + 4 h + r (e = 4 i + r) of row `row` in this half.
      f32x4 tsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) tsv[i] = *reinterpret_cast<const f32x4*>(&sm.ts[buf][kHalf * hf + 8 * i + 4 * c.h]);
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
          if (t0 + 8 * (e >> 2) + 4 * c.h + (e & 3) >= lim) sv[e] = -INFINITY;
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
      alpha = 1.f;
      if (tmax > m_run + kTau) {
        const float m_new = ceilf(tmax);
        alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, int(m_run - m_new));
        m_run = m_new;
      }
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      float pw[16], psum = 0.f, pmax = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, neg_m));
        psum += p;
        pw[e] = p * tsv[e >> 2][e & 3];
        pmax = fmaxf(pmax, pw[e]);
      }
      l_run = l_run * alpha + psum;
      {
        float x0 = pmax, x1 = pmax;
        permlane32_swap(x0, x1);
        pmax = fmaxf(x0, x1);
      }
      // Block scale 2^e with e = floor(log2 pmax) - 7: E8M0 byte bexp - 7 (at least 0), and
      // the values are multiplied by 2^-e before rounding.
      const int sbyte = max(int((__float_as_uint(pmax) >> 23) & 0xFF) - 7, 0);
      const float mul = __uint_as_float(uint32_t(254 - sbyte) << 23);
      const int pbuf = n & 1;
      const int g = p_swz(row);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(pw[4 * i] * mul, pw[4 * i + 1] * mul, 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(pw[4 * i + 2] * mul, pw[4 * i + 3] * mul, wd, true);
        const int chunk = 2 * hf + (i >> 1);
        *reinterpret_cast<int*>(&sm.p8[pbuf][row][16 * (chunk ^ g) + 8 * (i & 1) + prow_off]) = wd;
      }
      return sbyte;
    };

    auto step = [&](int n) {
      float a0, a1;
      const int s0 = half(n, 0, a0);
      const float m_mid = m_run;
      const int s1 = half(n, 1, a1);
      // Half 0 was rounded against the reference after half 0; when half 1 moved it, the
      // exact power-of-two rescale goes into half 0's block scale (a scale below 2^-127
      // stays at 2^-127: such weights are negligible against the new reference).
      int s0f = s0;
      if (a1 != 1.f) s0f = m_mid == -INFINITY ? 0 : max(s0 + int(m_mid - m_run), 0);
      if (c.h == 0) {
        const int pbuf = n & 1;
        sm.psc[pbuf][row][0] = s0f;
        sm.psc[pbuf][row][1] = s1;
        sm.alpha[pbuf][row] = a0 * a1;
      }
    };
    if (nsteps > 0) {
      __syncthreads();  // step 0 staged
      for (int n = 0; n < nsteps; ++n) {
        step(n);
        __syncthreads();
      }
    }
    // Row sum over both lane halves, log-sum-exp.
    float x0 = l_run, x1 = l_run;
    permlane32_swap(x0, x1);
    const float l_tot = x0 + x1;
    if (c.h == 0) {
      sm.lsum[row] = l_tot;
      const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
      if (final_out) {
        if (a.lse) a.lse[out_base + r0 + row] = lse2 * kLn2;
      } else {
        a.part_lse[out_base + r0 + row] = lse2;
      }
    }
    __syncthreads();  // row sums published
  } else {
    // ================================ output waves ===================================
    const int q = (c.w & 1) + 2 * (c.w >> 2);
    f32x16 oacc[4][2];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[cb][rb2][e] = 0.f;
    // V^T operand of column block cb (A of the 32 x 32 x 64 product): lane l holds column
    // 128 q + 32 cb + l % 32 and, in the instruction's K order, tokens 16 h .. 16 h + 15 of
    // the step in bytes 0 .. 15 and tokens 32 + 16 h .. 32 + 16 h + 15 in bytes 16 .. 31.
    // Read j (bytes 8 j .. 8 j + 7): the 16-lane group G reads columns 16 (G & 1) + (0..15) of
    // tokens 16 (G >> 1) + 8 (j & 1) + 32 (j >> 1) + (0..7).
    const int G = c.lane >> 4, gi = c.lane & 15;
    const int tr_row = 16 * (G >> 1) + (gi >> 1);
    int voff[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = tr_row + 8 * (j & 1) + 32 * (j >> 1);
        const int col = kCols * q + 32 * cb + 16 * (G & 1) + 8 * (gi & 1);
        voff[cb][j] = tok * kDC + 16 * ((col >> 4) ^ swz32(tok)) + (col & 15);
      }
    v8i vop[4];
    auto read_v = [&](int n) {
      const uint8_t* vt = &sm.lat8[n % 2][0][0];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x2 v = lds_read_tr8(vt + voff[cb][j]);
          vop[cb][2 * j] = int(v[0]);
          vop[cb][2 * j + 1] = int(v[1]);
        }
    };
    auto pv = [&](int n) {
      const int buf = n & 1;
      float al[2];
      int sc[2];
      v8i pb[2];
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2) {
        const int prow = 32 * rb2 + c.n;
        al[rb2] = sm.alpha[buf][prow];
        sc[rb2] = sm.psc[buf][prow][c.h];
        const uint8_t* pr = &sm.p8[buf][prow][0];
        // B operand (P^T): row prow, tokens 16 h .. + 15 (chunk h) and 32 + 16 h .. + 15
        // (chunk 2 + h), in the instruction's K order; the lane's scale is that of half h.
        const u32x4 lo = *reinterpret_cast<const u32x4*>(pr + 16 * (c.h ^ p_swz(prow)));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(pr + 16 * ((2 + c.h) ^ p_swz(prow)));
        pb[rb2] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      }
      if (__any((al[0] != 1.f) | (al[1] != 1.f))) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2) oacc[cb][rb2] *= al[rb2];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rb2 = 0; rb2 < 2; ++rb2)
          oacc[cb][rb2] =
              __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[cb], pb[rb2], oacc[cb][rb2], 0, 0, 0, 127, 0, sc[rb2]);
    };
    if (nsteps > 0) {
      __syncthreads();  // step 0 staged
      read_v(0);
      __syncthreads();  // step 0 scored
      for (int n = 1; n < nsteps; ++n) {
        pv(n - 1);
        read_v(n);
        __syncthreads();
      }
      pv(nsteps - 1);
    }
    __syncthreads();  // row sums published
    uint16_t* os = reinterpret_cast<uint16_t*>(&sm.lat8[0][0][0]);
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2) {
      const float lt = sm.lsum[32 * rb2 + c.n];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int lrow = 32 * rb2 + c.n;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int chunk = 16 * q + 4 * cb + i;
          const f32x4 v = f32x4{oacc[cb][rb2][4 * i], oacc[cb][rb2][4 * i + 1], oacc[cb][rb2][4 * i + 2],
                                oacc[cb][rb2][4 * i + 3]} * inv;
          *reinterpret_cast<u32x2*>(os + lrow * kDC + 8 * (chunk ^ (lrow & 15)) + 4 * c.h) =
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
      const int lrow = 8 * c.w + k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + lrow * kDC + 8 * (c.lane ^ (lrow & 15)));
      *reinterpret_cast<u32x4*>(dst + (out_base + r0 + lrow) * kDC + 8 * c.lane) = v;
    }
  }
  __syncthreads();  // the next piece stages into these buffers
}

// Launch bounds: 512 threads and at least 2 waves per SIMD, i.e. one 8-wave workgroup per
// compute unit (the kernel's LDS allows one); each wave may then hold up to 256 registers.
template <int PK>
__global__ __launch_bounds__(kThreads, 2) void decode_fp8_kernel(DecodeArgs a, int num_splits, int chunk,
                                                                 int rblocks, int n_units, int n_xcd) {
  __shared__ Smem8 sm;
  walk_pieces<32, kThreads>(a, num_splits, chunk, rblocks, n_units, n_xcd, sm.prefix, sm.wave_tot,
                            [&](int b, int rb, int t_lo, int t_hi, int L, bool fin, int64_t base)
                                __attribute__((always_inline)) {
                                  decode_piece8<PK>(sm, a, b, rb, t_lo, t_hi, L, fin, base);
                                });
}

template <int PK>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = p.rows / kRows;
  const int n_units = p.balanced ? p.num_splits * rblocks : a.B * p.num_splits * rblocks;
  const int n_xcd = p.n_xcd > 0 ? p.n_xcd : 1;
  const int grid = (n_units + n_xcd - 1) / n_xcd * n_xcd;
  hipLaunchKernelGGL((decode_fp8_kernel<PK>), dim3(grid), dim3(kThreads), 0, s, a, p.num_splits,
                     p.split_tokens, rblocks, n_units, n_xcd);
  return int(hipGetLastError());
}

}  // namespace

int launch_decode_fp8(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  if (a.kv_dt != MLA_FP8_E4M3 || p.rows % kRows) return int(hipErrorInvalidValue);
  if (!a.paged) return launch_t<kContig>(a, p, s);
  return a.block_size % kHalf == 0 ? launch_t<kPagedTile>(a, p, s) : launch_t<kPagedAny>(a, p, s);
}

}  // namespace mla
