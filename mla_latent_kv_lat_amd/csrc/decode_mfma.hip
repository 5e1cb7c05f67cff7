// Matrix-core (MFMA) latent-attention decode kernel for d_c = 512, d_r = 64 on gfx950.
//
// The absorbed form lets all heads of a sequence attend over one shared latent
// ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE key;
// "Multi-Head Latent Attention and the compression of the KV cache", paragraph on the
// associativity argument).  With the query already multiplied by W_UK, the score of
// head h and token t is  q_lat[h] . c_kv[t] + q_rope[h] . k_rope[t],  and the latent is
// also the value.  Per sequence that is two dense products over a token tile:
//   S^T[tok, row] = C[tok, 0:512] . Q_lat^T + R[tok, 0:64] . Q_rope^T     (K = 576)
//   O^T[col, row] += C[tok, col]^T . P^T[tok, row]                          (K = tokens)
// where "row" runs over the (query token, head) pairs of the sequence.
//
// Work split.  A workgroup (8 waves, two per SIMD) owns 64 query rows of one sequence
// and one split of its context, and walks it in tiles of 32 tokens.  Wave w owns latent
// columns [64w, 64w + 64); waves 0-3 also own RoPE dims [16w, 16w + 16) (waves w and
// w + 4 share a SIMD, so every SIMD carries the same matrix-core work):
//   * a wave loads exactly its slice of every cache row from HBM into registers (no
//     other wave touches those bytes), two tiles ahead of the one it computes;
//   * phase 1: partial scores over its columns, MFMA with the cache slice as the A
//     operand straight from registers and the query slice as the B operand;
//   * the eight partial score tiles are summed through LDS; wave w runs the online
//     softmax of rows [8w, 8w + 8) and publishes bf16 probabilities;
//   * phase 2: its 64 output columns for all 64 rows, MFMA with its own cache slice
//     (written to wave-private LDS and read back transposed) as the A operand.
// The cache is read from HBM once per workgroup, and the only cross-wave traffic is the
// 64x32 score tile and the probabilities.
//
// Softmax runs in base-2 units (scores times softmax_scale * log2(e)); a whole wave
// skips the accumulator rescale when no row's running max moved.  fp8 (OCP e4m3fn)
// caches are converted exactly to bf16 in registers; the per-token scale multiplies the
// latent part of the score and the probability used in the PV product.
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kRows = 64;               // query rows per workgroup
constexpr int kTile = 32;               // tokens per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = kDC / kWaves;     // latent columns owned by one wave (64)
constexpr int kRopeWaves = 4;           // waves that also own RoPE dims
constexpr int kRopeW = kDR / kRopeWaves;  // RoPE dims per such wave (16)
constexpr int kSRows = kRows / kWaves;  // softmax rows per wave (8)
constexpr int kSPitch = kTile + 4;      // floats per row of a partial-score tile
constexpr int kPPitch = kTile + 8;      // bf16 per row of the probability tile

struct alignas(16) Smem {
  float spart[kWaves][kRows][kSPitch];  // partial S^T of each wave, stored [row][tok]
  uint16_t v[kWaves][kTile][kCols];     // wave-private cache slice, 16-byte chunks swizzled
  uint16_t p[kRows][kPPitch];           // probabilities (bf16), [row][tok]
  float alpha[kRows];                   // per-row rescale factor of the current tile
  float lsum[kRows];
};

// Chunk swizzle of a wave-private slice row (8 chunks of 16 bytes, two rows per 64-bank
// cycle): the 16 rows of one write and the 8 rows of each half of a transposed read land
// in distinct banks.
__device__ __forceinline__ int vswz(int tok) {
  return (((tok >> 1) & 1) << 1) | (((tok >> 3) & 1) << 2) | ((tok >> 2) & 1);
}

// Column layout of one lane's k-slices.  For k-step s (0..1) of the 64 latent columns of
// a wave, lane group g (= lane / 16) holds 8 consecutive columns starting here.  Any
// assignment works as long as the A (cache) and B (query) operands agree; this one gives
// each lane 16 contiguous columns.
__device__ __forceinline__ int kcol(int s, int g) { return 16 * g + 8 * s; }

template <bool FP8>
struct TileRegs;

template <>
struct TileRegs<false> {
  u32x4 lat[2][2];   // [token block][k-step]: 8 bf16 of one token
  u32x2 rope[2];     // [token block]: 4 bf16 of one token (RoPE waves only)
};

template <>
struct TileRegs<true> {
  u32x4 lat[2];      // [token block]: 16 fp8 codes of one token
  u32x2 rope[2];
  float ts1[2][4];   // scales of tokens 16blk + 4g + i (phase-1 output layout)
  float ts2[4];      // scales of the softmax lane's tokens
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

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

__device__ __forceinline__ u32x4 a_operand(const TileRegs<false>& t, int blk, int s) {
  return t.lat[blk][s];
}

__device__ __forceinline__ u32x4 a_operand(const TileRegs<true>& t, int blk, int s) {
  const u32x4 w = t.lat[blk];
  return s ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
}

struct Ctx {
  int b, lane, g, m, w;
  int t_hi;
  const int32_t* table;
  int max_blocks, bs;
  int64_t T;
};

template <bool PAGED>
__device__ __forceinline__ int64_t row_of(const Ctx& c, int t) {
  return cache_row(PAGED, c.b, t, c.T, c.table, c.max_blocks, c.bs);
}

// Issue the global loads of one tile (tokens t0 .. t0 + 31) for this lane.  Tokens at or
// past the split end are not read; their registers are zero.
template <bool FP8, bool PAGED>
__device__ __forceinline__ void load_tile(TileRegs<FP8>& r, const Ctx& c, const DecodeArgs& a, int t0) {
  const bool rope_wave = c.w < kRopeWaves;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int t = t0 + 16 * blk + c.m;
    const bool ok = t < c.t_hi;
    const int64_t row = ok ? row_of<PAGED>(c, t) : 0;
    if constexpr (FP8) {
      const uint8_t* base = static_cast<const uint8_t*>(a.c_kv) + row * kDC + kCols * c.w + 16 * c.g;
      r.lat[blk] = ok ? ld16(base) : u32x4{0, 0, 0, 0};
    } else {
      const uint16_t* base = static_cast<const uint16_t*>(a.c_kv) + row * kDC + kCols * c.w;
#pragma unroll
      for (int s = 0; s < 2; ++s) r.lat[blk][s] = ok ? ld16(base + kcol(s, c.g)) : u32x4{0, 0, 0, 0};
    }
    if (rope_wave) {
      const uint16_t* rp = static_cast<const uint16_t*>(a.k_rope) + row * kDR + kRopeW * c.w + 4 * c.g;
      r.rope[blk] = ok ? ld8(rp) : u32x2{0, 0};
    }
  }
  if constexpr (FP8) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * blk + 4 * c.g + i;
        r.ts1[blk][i] = t < c.t_hi ? a.kv_scale[row_of<PAGED>(c, t)] : 0.f;
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t0 + 4 * (c.lane >> 3) + e;
      r.ts2[e] = t < c.t_hi ? a.kv_scale[row_of<PAGED>(c, t)] : 0.f;
    }
  }
}

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeArgs a, int num_splits,
                                                                  int chunk, int rblocks, int n_units) {
  __shared__ Smem sm;

  // Workgroups are handed to the 8 XCDs round-robin by id; give each XCD a contiguous
  // range of work units so that the row blocks (and splits) of one sequence share an L2.
  const int per_xcd = gridDim.x / 8;
  const int unit = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (unit >= n_units) return;
  const int rb = unit % rblocks;
  const int split = (unit / rblocks) % num_splits;
  const int b = unit / (rblocks * num_splits);

  Ctx c;
  c.b = b;
  c.lane = threadIdx.x & 63;
  c.w = threadIdx.x >> 6;
  c.g = c.lane >> 4;
  c.m = c.lane & 15;
  c.table = a.block_table;
  c.max_blocks = a.max_blocks;
  c.bs = a.block_size;
  c.T = a.T;
  const bool rope_wave = c.w < kRopeWaves;

  const int rows = a.sq * a.H;
  const int r0 = rb * kRows;
  const int L = a.seq_lens ? a.seq_lens[b] : int(a.T);
  const int t_lo = split * chunk;
  c.t_hi = min(L, t_lo + chunk);
  if (num_splits > 1 && t_lo >= L) return;  // the combine reads only splits below L

  // Query operands (B of phase 1): rows r0 + 16j + m, this wave's latent / RoPE slice.
  bf16x8 qb[4][2];
  bf16x4 qrb[4];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat);
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = int64_t(b) * rows + r0 + 16 * j + c.m;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        qb[j][s] = __builtin_bit_cast(bf16x8, ld16(ql + row * kDC + kCols * c.w + kcol(s, c.g)));
      qrb[j] = rope_wave ? __builtin_bit_cast(bf16x4, ld8(qr + row * kDR + kRopeW * c.w + 4 * c.g))
                         : bf16x4{};
    }
  }

  // Softmax ownership: row r0 + 8w + (lane % 8), tokens 4 * (lane / 8) .. + 3 of each tile.
  const int srow = kSRows * c.w + (c.lane & 7);
  const int stok = 4 * (c.lane >> 3);
  const int iq = (r0 + srow) / a.H;
  const int vis = min(max(L - a.sq + iq + 1, 0), L);  // tokens this query row may see
  const int lim = min(vis, c.t_hi);
  float m_run = -INFINITY, l_run = 0.f;

  f32x4 oacc[4][4];  // O^T: cols 64w + 16cb + 4g + i, rows 16j + m
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j) oacc[cb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Transposed reads of the wave-private slice: lane (4r + q) of group g supplies token
  // 8g + r (+4) and columns 16cb + 4q .. +3; it receives column 16cb + (lane % 16).
  const int tr_r = c.m >> 2, tr_q = c.m & 3;

  // One tile: phase 1 consumes `tr`, which is then refilled with tile t0 + 2 * kTile
  // (when that tile exists), so two tiles are in flight while this one is computed.
  auto process = [&](TileRegs<FP8>& tr, int t0) {
    // ---- phase 1: partial scores of this wave's columns -------------------------------
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 sacc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int tok = 16 * blk + c.m;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 araw = a_operand(tr, blk, s);
        const bf16x8 av = __builtin_bit_cast(bf16x8, araw);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[j][s], sacc[j], 0, 0, 0);
        // Keep the (bf16) slice for phase 2: 16 bytes of token 16blk + m.
        const int ch = (kcol(s, c.g) >> 3) ^ vswz(tok);
        *reinterpret_cast<u32x4*>(&sm.v[c.w][tok][8 * ch]) = araw;
      }
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[j][i] *= tr.ts1[blk][i];
      }
      if (rope_wave) {
        const s16x4 ar = __builtin_bit_cast(s16x4, tr.rope[blk]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ar, __builtin_bit_cast(s16x4, qrb[j]),
                                                             sacc[j], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(&sm.spart[c.w][16 * j + c.m][16 * blk + 4 * c.g]) = sacc[j];
    }
    float ts2[4];
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ts2[e] = tr.ts2[e];
    }
    if (t0 + 2 * kTile < c.t_hi) load_tile<FP8, PAGED>(tr, c, a, t0 + 2 * kTile);
    __syncthreads();

    // ---- online softmax of row srow over tokens stok .. stok + 3 ------------------------
    {
      f32x4 sv = *reinterpret_cast<const f32x4*>(&sm.spart[0][srow][stok]);
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) sv += *reinterpret_cast<const f32x4*>(&sm.spart[ww][srow][stok]);
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] = t0 + stok + e < lim ? sv[e] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 8, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float p[4], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = exp2f(sv[e] - m_use);
        psum += p[e];
        if constexpr (FP8) p[e] *= ts2[e];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const uint32_t w0 = uint32_t(f32_to_bf16_bits(p[0])) | (uint32_t(f32_to_bf16_bits(p[1])) << 16);
      const uint32_t w1 = uint32_t(f32_to_bf16_bits(p[2])) | (uint32_t(f32_to_bf16_bits(p[3])) << 16);
      *reinterpret_cast<u32x2*>(&sm.p[srow][stok]) = u32x2{w0, w1};
      if (c.lane < 8) sm.alpha[srow] = alpha;
    }
    __syncthreads();

    // ---- phase 2: O^T[cols of this wave, 64 rows] += V^T P^T ---------------------------
    {
      float al[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) al[j] = sm.alpha[16 * j + c.m];
      const bool moved = (al[0] != 1.f) | (al[1] != 1.f) | (al[2] != 1.f) | (al[3] != 1.f);
      if (__any(moved)) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int j = 0; j < 4; ++j) oacc[cb][j] *= al[j];
      }
      bf16x8 pb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pb[j] = *reinterpret_cast<const bf16x8*>(&sm.p[16 * j + c.m][8 * c.g]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int col = 16 * cb + 4 * tr_q;
        const int tk0 = 8 * c.g + tr_r, tk1 = tk0 + 4;
        const uint16_t* p0 = &sm.v[c.w][tk0][8 * ((col >> 3) ^ vswz(tk0)) + (col & 7)];
        const uint16_t* p1 = &sm.v[c.w][tk1][8 * ((col >> 3) ^ vswz(tk1)) + (col & 7)];
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (__attribute__((address_space(3))) s16x4*)(p0)));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (__attribute__((address_space(3))) s16x4*)(p1)));
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int j = 0; j < 4; ++j)
          oacc[cb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[j], oacc[cb][j], 0, 0, 0);
      }
    }
  };

  // Tiles of the split; each process() call leaves the loads of the next two in flight.
  const int ntiles = (c.t_hi - t_lo + kTile - 1) / kTile;
  if (ntiles > 0) {
    TileRegs<FP8> ra, rb2;
    load_tile<FP8, PAGED>(ra, c, a, t_lo);
    if (ntiles > 1) load_tile<FP8, PAGED>(rb2, c, a, t_lo + kTile);
    for (int n = 0; n < ntiles; n += 2) {
      process(ra, t_lo + n * kTile);
      if (n + 1 < ntiles) process(rb2, t_lo + (n + 1) * kTile);
    }
  }

  // ---- finish: row sums, normalisation, outputs ---------------------------------------
  float l_tot = l_run + __shfl_xor(l_run, 8, 64);
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (c.lane < 8) sm.lsum[srow] = l_tot;
  __syncthreads();
  const bool single = num_splits == 1;
  if (c.lane < 8) {
    const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
    if (single) {
      if (a.lse) a.lse[int64_t(b) * rows + r0 + srow] = lse2 * kLn2;
    } else {
      a.part_lse[(int64_t(b) * num_splits + split) * rows + r0 + srow] = lse2;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lt = sm.lsum[16 * j + c.m];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int row = r0 + 16 * j + c.m;
    if (single) {
      uint16_t* o = static_cast<uint16_t*>(a.o_lat) + (int64_t(b) * rows + row) * kDC + kCols * c.w + 4 * c.g;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const f32x4 v = oacc[cb][j] * inv;
        const uint32_t w0 = uint32_t(f32_to_bf16_bits(v[0])) | (uint32_t(f32_to_bf16_bits(v[1])) << 16);
        const uint32_t w1 = uint32_t(f32_to_bf16_bits(v[2])) | (uint32_t(f32_to_bf16_bits(v[3])) << 16);
        *reinterpret_cast<u32x2*>(o + 16 * cb) = u32x2{w0, w1};
      }
    } else {
      float* o = a.part_o + ((int64_t(b) * num_splits + split) * rows + row) * kDC + kCols * c.w + 4 * c.g;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) *reinterpret_cast<f32x4*>(o + 16 * cb) = oacc[cb][j] * inv;
    }
  }
}

template <bool FP8, bool PAGED>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = p.rows / kRows;
  const int n_units = a.B * p.num_splits * rblocks;
  const int grid = (n_units + 7) / 8 * 8;
  hipLaunchKernelGGL((decode_mfma_kernel<FP8, PAGED>), dim3(grid), dim3(kThreads), 0, s, a,
                     p.num_splits, p.split_tokens, rblocks, n_units);
  return int(hipGetLastError());
}

}  // namespace

int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  if (a.kv_dt == MLA_FP8_E4M3)
    return a.paged ? launch_t<true, true>(a, p, s) : launch_t<true, false>(a, p, s);
  return a.paged ? launch_t<false, true>(a, p, s) : launch_t<false, false>(a, p, s);
}

// Decode of all 256 e4m3fn codes as this kernel family converts them (for tests).
__global__ void fp8_bf16_table_kernel(float* out) {
  const uint32_t code = threadIdx.x;
  const uint32_t bits = e4m3x2_to_bf16x2<false>(code);
  out[code] = bf16_bits_to_f32(bits & 0xFFFF);
}

int launch_fp8_bf16_table(float* out, hipStream_t s) {
  hipLaunchKernelGGL(fp8_bf16_table_kernel, dim3(1), dim3(256), 0, s, out);
  return int(hipGetLastError());
}

}  // namespace mla
