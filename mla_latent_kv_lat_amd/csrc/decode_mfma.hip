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
// Work split.  A workgroup owns 64 query rows of one sequence and one split of its
// context, walked in tiles of 32 tokens, with eight waves in two roles (one of each per
// SIMD, so the matrix cores stay busy while the other role does LDS / VALU work):
//   * score waves 0-3: wave p owns latent columns [128p, 128p + 128) and RoPE dims
//     [16p, 16p + 16).  It streams exactly that slice of every cache row from HBM into
//     registers, two tiles ahead; computes partial scores (MFMA, cache slice as the A
//     operand, query slice as the B operand); sums the four partial score tiles
//     through LDS; runs the online softmax of rows [16p, 16p + 16); and publishes the
//     tile's cache slice (in LDS, for the transposed reads) and the bf16 probabilities.
//   * output waves 4-7: wave 4 + q owns output columns [128q, 128q + 128) for all 64
//     rows and accumulates O^T += V^T P^T for the previous tile (MFMA, cache slice read
//     transposed from LDS as the A operand, probabilities as the B operand).
// Each step has two barriers.  Half A: score waves run phase 1 of tile n while output
// waves rescale and start PV of tile n - 1.  Half B: score waves run the softmax of
// tile n while output waves finish PV of tile n - 1.  Slices and probabilities are double
// buffered in LDS.  The cache is read from HBM once per workgroup.
//
// Softmax runs in base-2 units (scores times softmax_scale * log2(e)); output waves skip
// the accumulator rescale when no row's running max moved.  fp8 (OCP e4m3fn) caches are
// converted exactly to bf16 in registers; the per-token scale multiplies the latent part
// of the score and the probability used in the PV product.
#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kRows = 64;               // query rows per workgroup
constexpr int kTile = 32;               // tokens per tile
constexpr int kThreads = 512;           // 4 score waves + 4 output waves
constexpr int kCols = 128;              // latent columns per score wave / output wave
constexpr int kRopeW = 16;              // RoPE dims per score wave
constexpr int kSPitch = kTile + 4;      // floats per row of a partial-score tile
constexpr int kPPitch = kTile + 8;      // bf16 per row of the probability tile
constexpr int kSplitA = 3;              // output column blocks done in half A (of 8)

struct alignas(16) Smem {
  float spart[4][kRows][kSPitch];       // partial S^T of each score wave, [row][tok]
  uint16_t v[2][4][kTile][kCols];       // cache slices (double buffered), swz256 chunks
  uint16_t p[2][kRows][kPPitch];        // probabilities (double buffered), [row][tok]
  float alpha[2][kRows];                // per-row rescale factor of each buffered tile
  float lsum[kRows];
};

// Column layout of one score lane's k-slices: for k-step s (0..3) of its 128 latent
// columns, lane group g (= lane / 16) holds 8 consecutive columns starting here.  The A
// (cache) and B (query) operands use the same map; each lane gets 16 contiguous columns
// per pair of k-steps (one 16-byte load of fp8 codes).
__device__ __forceinline__ int kcol(int s, int g) { return 64 * (s >> 1) + 16 * g + 8 * (s & 1); }

template <bool FP8>
struct TileRegs;

template <>
struct TileRegs<false> {
  u32x4 lat[2][4];   // [token block][k-step]: 8 bf16 of one token
  u32x2 rope[2];     // [token block]: 4 bf16 of one token
};

template <>
struct TileRegs<true> {
  u32x4 lat[2][2];   // [token block][pair of k-steps]: 16 fp8 codes of one token
  u32x2 rope[2];
  float ts1[2][4];   // scales of tokens 16 blk + 4g + i (phase-1 output layout)
  float ts2[8];      // scales of tokens 8g + e (softmax layout)
};

__device__ __forceinline__ u32x4 a_operand(const TileRegs<false>& t, int blk, int s) {
  return t.lat[blk][s];
}

__device__ __forceinline__ u32x4 a_operand(const TileRegs<true>& t, int blk, int s) {
  const u32x4 w = t.lat[blk][s >> 1];
  return (s & 1) ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
}

struct Ctx {
  int b, lane, g, m, w;
  int t_hi;
  const int32_t* table;
  int max_blocks, bs;
  int64_t T;
};

// Cache layouts: contiguous [B, T, .]; paged with every 32-token tile inside one block
// (block_size a multiple of 32: one wave-uniform table entry per tile); paged general.
enum : int { kContig = 0, kPagedTile = 1, kPagedAny = 2 };

// Cache rows of the tokens of one tile.  Token indices are first clamped to the split's
// last valid token, so every lane always issues the same loads from valid rows: tokens
// past the split end get that row's (finite) data, and the softmax gives them weight 0.
// Issuing the same loads on every path keeps the compiler's wait counts exact, so the
// loads of the next tiles stay in flight while this one is computed.
template <int PK>
struct TileRows {
  int64_t base;
  int blk_t0;
  __device__ __forceinline__ TileRows(const Ctx& c, int t0) {
    if constexpr (PK == kContig) {
      base = int64_t(c.b) * c.T;
      blk_t0 = 0;
    } else if constexpr (PK == kPagedTile) {
      const int blk = min(t0, c.t_hi - 1) / c.bs;
      base = int64_t(c.table[int64_t(c.b) * c.max_blocks + blk]) * c.bs;
      blk_t0 = blk * c.bs;
    } else {
      base = 0;
      blk_t0 = 0;
    }
  }
  __device__ __forceinline__ int64_t row(const Ctx& c, int t) const {
    const int tc = min(t, c.t_hi - 1);
    if constexpr (PK == kContig) return base + tc;
    if constexpr (PK == kPagedTile) return base + (tc - blk_t0);
    return int64_t(c.table[int64_t(c.b) * c.max_blocks + tc / c.bs]) * c.bs + tc % c.bs;
  }
};

// Issue the global loads of one tile (tokens t0 .. t0 + 31) for this score lane.
template <bool FP8, int PK>
__device__ __forceinline__ void load_tile(TileRegs<FP8>& r, const Ctx& c, const DecodeArgs& a, int t0) {
  const TileRows<PK> rows(c, t0);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int64_t row = rows.row(c, t0 + 16 * blk + c.m);
    if constexpr (FP8) {
      const uint8_t* base = static_cast<const uint8_t*>(a.c_kv) + row * kDC + kCols * c.w + 16 * c.g;
#pragma unroll
      for (int h = 0; h < 2; ++h) r.lat[blk][h] = ld16(base + 64 * h);
    } else {
      const uint16_t* base = static_cast<const uint16_t*>(a.c_kv) + row * kDC + kCols * c.w;
#pragma unroll
      for (int s = 0; s < 4; ++s) r.lat[blk][s] = ld16(base + kcol(s, c.g));
    }
    r.rope[blk] = ld8(static_cast<const uint16_t*>(a.k_rope) + row * kDR + kRopeW * c.w + 4 * c.g);
  }
  if constexpr (FP8) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) r.ts1[blk][i] = a.kv_scale[rows.row(c, t0 + 16 * blk + 4 * c.g + i)];
#pragma unroll
    for (int e = 0; e < 8; ++e) r.ts2[e] = a.kv_scale[rows.row(c, t0 + 8 * c.g + e)];
  }
}

template <bool FP8, int PK>
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
  c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.g = c.lane >> 4;
  c.m = c.lane & 15;
  c.table = a.block_table;
  c.max_blocks = a.max_blocks;
  c.bs = a.block_size;
  c.T = a.T;

  const int rows = a.sq * a.H;
  const int r0 = rb * kRows;
  const int L = a.seq_lens ? a.seq_lens[b] : int(a.T);
  const int t_lo = split * chunk;
  c.t_hi = min(L, t_lo + chunk);
  if (num_splits > 1 && t_lo >= L) return;  // the combine reads only splits below L
  const int ntiles = (c.t_hi - t_lo + kTile - 1) / kTile;
  const int steps = ntiles > 0 ? ntiles + 1 : 0;
  const bool single = num_splits == 1;

  if (c.w < 4) {
    // ================================ score waves ===================================
    bf16x8 qb[4][4];
    bf16x4 qrb[4];
    {
      const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat);
      const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = int64_t(b) * rows + r0 + 16 * j + c.m;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          qb[j][s] = __builtin_bit_cast(bf16x8, ld16(ql + row * kDC + kCols * c.w + kcol(s, c.g)));
        qrb[j] = __builtin_bit_cast(bf16x4, ld8(qr + row * kDR + kRopeW * c.w + 4 * c.g));
      }
    }
    // Softmax ownership: row 16w + m, tokens 8g .. 8g + 7 of each tile.
    const int srow = 16 * c.w + c.m;
    const int iq = (r0 + srow) / a.H;
    const int vis = min(max(L - a.sq + iq + 1, 0), L);  // tokens this query row may see
    const int lim = min(vis, c.t_hi);
    float m_run = -INFINITY, l_run = 0.f;

    // Half A (phase 1 of tile n into buffer n % 2) and half B (its softmax).
    auto step = [&](TileRegs<FP8>& tr, int n) {
      const int t0 = t_lo + n * kTile;
      const int buf = n & 1;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x4 sacc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tok = 16 * blk + c.m;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 araw = a_operand(tr, blk, s);
          const bf16x8 av = __builtin_bit_cast(bf16x8, araw);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[j][s], sacc[j], 0, 0, 0);
          const int ch = (kcol(s, c.g) >> 3) ^ swz256(tok);
          *reinterpret_cast<u32x4*>(&sm.v[buf][c.w][tok][8 * ch]) = araw;
        }
        if constexpr (FP8) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[j][i] *= tr.ts1[blk][i];
        }
        const s16x4 ar = __builtin_bit_cast(s16x4, tr.rope[blk]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ar, __builtin_bit_cast(s16x4, qrb[j]),
                                                             sacc[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(&sm.spart[c.w][16 * j + c.m][16 * blk + 4 * c.g]) = sacc[j];
      }
      float ts2[8];
      if constexpr (FP8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ts2[e] = tr.ts2[e];
      }
      load_tile<FP8, PK>(tr, c, a, t0 + 2 * kTile);  // refill: two tiles ahead
      __syncthreads();

      // Online softmax of row srow over tokens 8g .. 8g + 7.
      f32x4 s0 = *reinterpret_cast<const f32x4*>(&sm.spart[0][srow][8 * c.g]);
      f32x4 s1 = *reinterpret_cast<const f32x4*>(&sm.spart[0][srow][8 * c.g + 4]);
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        s0 += *reinterpret_cast<const f32x4*>(&sm.spart[q][srow][8 * c.g]);
        s1 += *reinterpret_cast<const f32x4*>(&sm.spart[q][srow][8 * c.g + 4]);
      }
      float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[e] = t0 + 8 * c.g + e < lim ? sv[e] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      tmax = max_xor16_32(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float pr[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pr[e] = exp2f(sv[e] - m_use);
        psum += pr[e];
        if constexpr (FP8) pr[e] *= ts2[e];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      *reinterpret_cast<u32x4*>(&sm.p[buf][srow][8 * c.g]) =
          u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]), pack_bf16x2(pr[4], pr[5]),
                pack_bf16x2(pr[6], pr[7])};
      if (c.g == 0) sm.alpha[buf][srow] = alpha;
      __syncthreads();
    };

    if (steps > 0) {
      TileRegs<FP8> ra, rb2;
      load_tile<FP8, PK>(ra, c, a, t_lo);
      load_tile<FP8, PK>(rb2, c, a, t_lo + kTile);
      // Straight-line pairs: every path into the loop header has the same loads in flight.
      int n = 0;
      for (; n + 1 < ntiles; n += 2) {
        step(ra, n);
        step(rb2, n + 1);
      }
      if (n < ntiles) step(ra, n);
      // The output waves' last step (PV of the last tile).
      __syncthreads();
      __syncthreads();
    }

    const float l_tot = sum_xor16_32(l_run);
    if (c.g == 0) {
      sm.lsum[srow] = l_tot;
      const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
      if (single) {
        if (a.lse) a.lse[int64_t(b) * rows + r0 + srow] = lse2 * kLn2;
      } else {
        a.part_lse[(int64_t(b) * num_splits + split) * rows + r0 + srow] = lse2;
      }
    }
    __syncthreads();
  } else {
    // ================================ output waves ==================================
    const int q = c.w - 4;
    f32x4 oacc[8][4];  // O^T: cols 128q + 16cb + 4g + i, rows 16j + m
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) oacc[cb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 pb[4];

    for (int n = 0; n < steps; ++n) {
      const int buf = (n - 1) & 1;
      if (n > 0) {
        float al[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) al[j] = sm.alpha[buf][16 * j + c.m];
        const bool moved = (al[0] != 1.f) | (al[1] != 1.f) | (al[2] != 1.f) | (al[3] != 1.f);
        if (__any(moved)) {
#pragma unroll
          for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) oacc[cb][j] *= al[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pb[j] = *reinterpret_cast<const bf16x8*>(&sm.p[buf][16 * j + c.m][8 * c.g]);
        const uint16_t* vt = &sm.v[buf][q][0][0];
#pragma unroll
        for (int cb = 0; cb < kSplitA; ++cb) {
          const bf16x8 av = lds_operand_tr256(vt, 0, 16 * cb, c.lane);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            oacc[cb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[j], oacc[cb][j], 0, 0, 0);
        }
      }
      __syncthreads();
      if (n > 0) {
        const uint16_t* vt = &sm.v[buf][q][0][0];
#pragma unroll
        for (int cb = kSplitA; cb < 8; ++cb) {
          const bf16x8 av = lds_operand_tr256(vt, 0, 16 * cb, c.lane);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            oacc[cb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[j], oacc[cb][j], 0, 0, 0);
        }
      }
      __syncthreads();
    }
    __syncthreads();  // row sums published by the score waves

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lt = sm.lsum[16 * j + c.m];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int row = r0 + 16 * j + c.m;
      if (single) {
        uint16_t* o = static_cast<uint16_t*>(a.o_lat) + (int64_t(b) * rows + row) * kDC + kCols * q + 4 * c.g;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const f32x4 v = oacc[cb][j] * inv;
          *reinterpret_cast<u32x2*>(o + 16 * cb) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      } else {
        float* o = a.part_o + ((int64_t(b) * num_splits + split) * rows + row) * kDC + kCols * q + 4 * c.g;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) *reinterpret_cast<f32x4*>(o + 16 * cb) = oacc[cb][j] * inv;
      }
    }
  }
}

template <bool FP8, int PK>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = p.rows / kRows;
  const int n_units = a.B * p.num_splits * rblocks;
  const int grid = (n_units + 7) / 8 * 8;
  hipLaunchKernelGGL((decode_mfma_kernel<FP8, PK>), dim3(grid), dim3(kThreads), 0, s, a,
                     p.num_splits, p.split_tokens, rblocks, n_units);
  return int(hipGetLastError());
}

}  // namespace

int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int pk = !a.paged ? kContig : (a.block_size % kTile == 0 ? kPagedTile : kPagedAny);
  if (a.kv_dt == MLA_FP8_E4M3) {
    if (pk == kContig) return launch_t<true, kContig>(a, p, s);
    return pk == kPagedTile ? launch_t<true, kPagedTile>(a, p, s) : launch_t<true, kPagedAny>(a, p, s);
  }
  if (pk == kContig) return launch_t<false, kContig>(a, p, s);
  return pk == kPagedTile ? launch_t<false, kPagedTile>(a, p, s) : launch_t<false, kPagedAny>(a, p, s);
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
