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
// Two workgroup designs share the grid, the range walk and the output format:
//   * row-block score waves (decode_piece3, below): every layout, bf16 and fp8 caches;
//   * K-split score waves (decode_piece): the fp8 score product (fp8 query codes times the
//     stored codes), which needs the cache codes, not bf16, as its score operand.
//
// K-split design.  A workgroup owns 64 query rows of one sequence and one split of its
// context, walked in tiles of 32 tokens, with eight waves in two roles (one of each per
// SIMD, so the matrix cores stay busy while the other role does LDS / VALU work).  All
// products use the 32 x 32 x 16 bf16 matrix instruction (tokens or output columns on one
// side, 32 query rows on the other).
//   * score waves 0-3: wave p owns latent columns [128p, 128p + 128) and RoPE dims
//     [16p, 16p + 16).  It streams exactly that slice of every cache row from HBM into
//     registers, two tiles ahead; stages the tile's slice in LDS as bf16 (swizzled; the
//     output waves read it there as V); computes partial scores (MFMA, cache slice as the
//     A operand, query slice as the B operand, held in registers for the whole split)
//     into LDS.
//   * output waves 4-7: wave 4 + q owns output columns [128q, 128q + 128) for all 64
//     rows and accumulates O^T += V^T P^T (MFMA, cache slice read transposed from LDS as
//     the A operand, probabilities as the B operand).
//   * all eight waves share the online softmax: wave w sums the four partial scores of
//     rows [8w, 8w + 8) and publishes their bf16 probabilities.
// The three stages are pipelined over the tiles with one barrier per step: in step n the
// score waves stage and score tile n + 1, every wave runs the softmax of tile n, and the
// output waves multiply tile n - 1 (whose V^T operands they read from LDS in step n - 1)
// and read the operands of tile n.  A score wave runs its softmax while the matrix unit
// finishes its score products (issued first), and only then stores the partial scores and
// refills its registers.  Slices, partial scores and probabilities are double buffered in
// LDS.  The cache is read from HBM once per workgroup.  At the end the output waves park
// the normalised rows in LDS and all eight waves write them out as whole 1 KB rows (the
// accumulator layout would scatter 8-byte pieces over 32 rows per store instruction).
//
// Softmax runs in base-2 units (scores times softmax_scale * log2(e), exponentials by the
// hardware base-2 exponential; results that would be denormal flush to 0) against a per-row
// reference max that only moves when a tile exceeds it by more than kTau; output waves
// skip the accumulator rescale whenever no row's reference moved.  fp8 (OCP e4m3fn) caches are
// converted exactly to bf16 in registers; the per-token scale multiplies the latent part
// of the score and the probability used in the PV product (each score lane loads its
// token's scale once per tile and shares it through LDS).
#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"

#include <type_traits>

namespace mla {
namespace {

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kRows = 64;               // query rows per workgroup (two 32-row blocks)
constexpr int kTile = 32;               // tokens per tile
constexpr int kThreads = 512;           // 4 score waves + 4 output waves
constexpr int kCols = 128;              // latent columns per score wave / output wave
constexpr int kRopeW = 16;              // RoPE dims per score wave
constexpr int kPPitch = kTile;          // bf16 per row of the probability tile (swizzled, p_swz)
constexpr int kMaxPrefixBatch = 2 * kThreads;  // largest batch whose tile prefix each workgroup computes
// A row's reference max (the value its probabilities are taken relative to) only moves
// when a tile's max exceeds it by more than this many base-2 units, so probabilities stay
// below 2^kTau and the output waves almost never have to rescale their accumulators.
// The result is the same up to rounding: numerator and denominator share the reference.
constexpr float kTau = 8.f;

struct alignas(16) Smem {
  float spart[2][4][kRows][kTile];      // partial S of each score wave (double buffered), swizzled
  uint16_t v[2][4][kTile][kCols];       // staged cache slices (double buffered), swz32 chunks
  uint16_t p[2][kRows][kPPitch];        // probabilities (double buffered), [row][tok]
  float ts[2][4][kTile];                // fp8 per-token scales, one copy per score wave
  float alpha[2][kRows];                // per-row rescale factor of each buffered tile
  float lsum[kRows];
  int64_t prefix[kMaxPrefixBatch + 1];  // balanced ranges: the batch's tile prefix (small batches)
  int64_t wave_tot[kThreads / 64];
};
static_assert(kMaxInKernelPrefixBatch <= kMaxPrefixBatch, "in-kernel tile prefix does not fit");

// Partial-score rows hold 8 chunks of 4 tokens; chunk c of row r is stored at c ^ sp_swz(r),
// which keeps both the score waves' writes (8 lanes per LDS cycle: 8 rows, one chunk each)
// and the softmax reads (16 lanes per cycle: 2 rows, 8 chunks) on distinct LDS banks.
__device__ __forceinline__ int sp_swz(int row) { return row & 7; }

// Probability rows hold 4 chunks of 8 tokens (64 bytes); chunk c of row r is stored at
// c ^ p_swz(r), which keeps the softmax writes (16 lanes of 8 bytes: 2 rows) and the output
// waves' operand reads (16 lanes of 16 bytes: 16 rows, one chunk each) on distinct banks.
__device__ __forceinline__ int p_swz(int row) { return (row >> 2) & 3; }

// Softmax state of one lane: row `row` of the workgroup, tokens 4 tg .. 4 tg + 3 of each tile.
struct SoftmaxLane {
  int row, tg;
  int lim;    // tokens below this index are visible to the row (and inside the split)
  int lim_w;  // smallest lim over the wave's 8 rows: tiles below it need no masking
  float m_run, l_run;
};

// Online softmax of one tile for this lane's row and 4 tokens: sums the four partial
// scores, masks invisible tokens (only in tiles that reach past lim_w), moves the row's
// reference max when the tile exceeds it by more than kTau, and publishes the bf16
// probabilities and the row's rescale factor.  Rows are spread over all eight waves
// (8 rows per wave, 8 lanes per row), so the 8-lane reductions are DPP steps.
template <bool FP8>
__device__ __forceinline__ void softmax_tile(Smem& sm, SoftmaxLane& st, int buf, int t0, float scale_log2) {
  const int ch = 4 * (st.tg ^ sp_swz(st.row));
  f32x4 sv4 = *reinterpret_cast<const f32x4*>(&sm.spart[buf][0][st.row][ch]);
#pragma unroll
  for (int q = 1; q < 4; ++q) sv4 += *reinterpret_cast<const f32x4*>(&sm.spart[buf][q][st.row][ch]);
  float sv[4] = {sv4[0], sv4[1], sv4[2], sv4[3]};
  if (t0 + kTile > st.lim_w) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t0 + 4 * st.tg + e >= st.lim) sv[e] = -INFINITY;
  }
  float tmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  tmax = max8(tmax) * scale_log2;  // scale > 0: max commutes with it
  const bool grow = tmax > st.m_run + kTau;  // false while nothing is visible
  const float alpha = grow ? __builtin_amdgcn_exp2f(st.m_run - tmax) : 1.f;
  if (grow) st.m_run = tmax;
  const float neg_m = st.m_run == -INFINITY ? 0.f : -st.m_run;
  float pr[4], psum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pr[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, neg_m));
    psum += pr[e];
  }
  if constexpr (FP8) {
    const f32x4 t4 = *reinterpret_cast<const f32x4*>(&sm.ts[buf][0][4 * st.tg]);
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] *= t4[e];
  }
  st.l_run = st.l_run * alpha + psum;
  *reinterpret_cast<u32x2*>(&sm.p[buf][st.row][8 * ((st.tg >> 1) ^ p_swz(st.row)) + 4 * (st.tg & 1)]) =
      u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
  if (st.tg == 0) sm.alpha[buf][st.row] = alpha;
}

// Column layout of one score lane's k-slices: for k-step s (0..7) of its 128 latent
// columns, lane half h (= lane / 32) holds 8 consecutive columns starting here.  The A
// (cache) and B (query) operands use the same map; each lane gets 16 contiguous columns
// per pair of k-steps (one 16-byte load of fp8 codes).
__device__ __forceinline__ int kcol(int s, int h) { return 32 * (s >> 1) + 16 * h + 8 * (s & 1); }

template <bool FP8>
struct TileRegs;

// A score wave's tile registers.  A bf16 latent slice is loaded coalesced: load k covers
// whole 256-byte row slices of 4 consecutive tokens, 16 bytes per lane, so each load
// instruction touches few cache lines; the slice then goes through LDS, where the score
// product reads it back in operand layout.  An fp8 slice is half as many bytes and its
// tiles are compute-bound: it is loaded in operand layout (token n = lane % 32, the 16
// codes of k-steps 2k and 2k + 1 of lane half h), converted in registers and used as the
// score operand directly; LDS only gets the converted copy for the output waves.  The
// RoPE slice is loaded in operand layout (dims 8h .. 8h + 7 of the wave's 16).
template <>
struct TileRegs<false> {
  u32x4 lat[8];      // load k: token 4k + lane / 16, columns 8 (lane % 16) + (0..7)
  u32x4 rope;
};

template <>
struct TileRegs<true> {
  u32x4 lat[4];      // load k: token lane % 32, columns 32k + 16h + (0..15), fp8 codes
  u32x4 rope;
  float ts;          // scale of token lane % 32
};

// Token held by load k of this lane (bf16 caches).
__device__ __forceinline__ int lat_token(int k, int lane) { return 4 * k + (lane >> 4); }

struct Ctx {
  int b, lane, n, h, w;
  int t_hi;
  const int32_t* table;
  int max_blocks, bs;
  int64_t T;
};

// Cache layouts: contiguous [B, T, .]; paged with every 32-token tile inside one block
// (block_size a multiple of 32: one wave-uniform table entry per tile); paged general.
enum : int { kContig = 0, kPagedTile = 1, kPagedAny = 2 };

// Buffer resource (gfx9 raw buffer: stride 0, range-checked in bytes) over `bytes` bytes.
// A load whose offset is past the range returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buf_ld4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Cache row of a token (general paged layout).  Token indices are first clamped to the
// split's last valid token, so every lane always issues the same loads from valid rows.
__device__ __forceinline__ int64_t any_row(const Ctx& c, int t) {
  const int tc = min(t, c.t_hi - 1);
  return int64_t(c.table[int64_t(c.b) * c.max_blocks + tc / c.bs]) * c.bs + tc % c.bs;
}

// Issue the loads of one tile (tokens t0 .. t0 + 31; this lane's token is t0 + n).  Every
// lane issues the same loads on every path (tokens past the split end read zeros, or the
// split's last row in the general paged layout; the softmax gives them weight 0), which
// keeps the compiler's wait counts exact, so the loads of the next tiles stay in flight
// while this one is computed.  Contiguous and block-aligned paged caches use buffer
// resources whose range ends at the last valid row of the sequence (or of the tile's
// block), so rows past the end are never read.
template <bool FP8, int PK>
__device__ __forceinline__ void load_tile(TileRegs<FP8>& r, const Ctx& c, const DecodeArgs& a, int t0) {
  constexpr uint32_t kLatBytes = kDC * (FP8 ? 1 : 2);
  constexpr uint32_t kRopeBytes = kDR * 2;
  const char* lat_base;
  const char* rope_base;
  const char* sc_base = nullptr;
  uint32_t nrows, row0;  // rows addressable from the bases; row of token t0 (may be >= nrows)
  if constexpr (PK == kContig) {
    const int64_t seq_row = int64_t(c.b) * c.T;
    lat_base = static_cast<const char*>(a.c_kv) + seq_row * kLatBytes;
    rope_base = static_cast<const char*>(a.k_rope) + seq_row * kRopeBytes;
    if constexpr (FP8) sc_base = reinterpret_cast<const char*>(a.kv_scale + seq_row);
    nrows = uint32_t(c.t_hi);
    row0 = uint32_t(t0);
  } else if constexpr (PK == kPagedTile) {
    const int blk = min(t0, c.t_hi - 1) / c.bs;  // the tile lies inside this block
    const int blk_t0 = blk * c.bs;
    const int64_t pool_row = int64_t(c.table[int64_t(c.b) * c.max_blocks + blk]) * c.bs;
    lat_base = static_cast<const char*>(a.c_kv) + pool_row * kLatBytes;
    rope_base = static_cast<const char*>(a.k_rope) + pool_row * kRopeBytes;
    if constexpr (FP8) sc_base = reinterpret_cast<const char*>(a.kv_scale + pool_row);
    nrows = uint32_t(min(c.bs, c.t_hi - blk_t0));
    row0 = uint32_t(t0 - blk_t0);
  }
  if constexpr (PK == kContig || PK == kPagedTile) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(lat_base, nrows * kLatBytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rope_base, nrows * kRopeBytes);
    const uint32_t row = row0 + uint32_t(c.n);
    const uint32_t col0 = (kLatBytes / 4) * c.w;  // the wave's slice
#pragma unroll
    for (int k = 0; k < (FP8 ? 4 : 8); ++k) {
      if constexpr (FP8)
        r.lat[k] = buf_ld16(rl, row * kLatBytes + col0 + 32 * k + 16 * c.h);
      else
        r.lat[k] = buf_ld16(rl, (row0 + uint32_t(lat_token(k, c.lane))) * kLatBytes + col0 + 16 * (c.lane & 15));
    }
    if constexpr (FP8) r.ts = buf_ld4f(make_rsrc(sc_base, nrows * 4), row * 4);
    r.rope = buf_ld16(rr, row * kRopeBytes + 2 * (kRopeW * c.w + 8 * c.h));
  } else {
    const char* lat = static_cast<const char*>(a.c_kv);
    const int64_t col0 = (kLatBytes / 4) * c.w;
    const int64_t row = any_row(c, t0 + c.n);
#pragma unroll
    for (int k = 0; k < (FP8 ? 4 : 8); ++k) {
      if constexpr (FP8)
        r.lat[k] = ld16(lat + row * kLatBytes + col0 + 32 * k + 16 * c.h);
      else
        r.lat[k] = ld16(lat + any_row(c, t0 + lat_token(k, c.lane)) * kLatBytes + col0 + 16 * (c.lane & 15));
    }
    if constexpr (FP8) r.ts = a.kv_scale[row];
    r.rope = ld16(static_cast<const uint16_t*>(a.k_rope) + row * kDR + kRopeW * c.w + 8 * c.h);
  }
}

// One piece of work: query rows [64 rb, 64 rb + 64) of sequence b (length L) over its
// tokens [t_lo, t_hi).  A final piece covers the whole sequence and writes o_lat and lse;
// any other piece writes its normalised partial output and base-2 log-sum-exp.  Row r of
// the row block goes to row out_base + 64 rb + r of the target arrays.  Every wave of
// the workgroup calls it with the same arguments (it contains barriers).
template <bool FP8, int PK, bool QK8>
__device__ __forceinline__ void decode_piece(Smem& sm, const DecodeArgs& a, int b, int rb, int t_lo,
                                             int t_hi, int L, bool final_out, int64_t out_base) {
  // The thread index goes through an opaque copy so that nothing derived from it is
  // hoisted out of the caller's loop over pieces (that would keep it in registers across
  // the whole piece).
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

  const int rows = a.sq * a.H;
  const int r0 = rb * kRows;
  c.t_hi = t_hi;
  const int ntiles = t_hi > t_lo ? (t_hi - t_lo + kTile - 1) / kTile : 0;
  const int steps = ntiles > 0 ? ntiles + 1 : 0;
  const bool single = final_out;

  // Softmax ownership (all eight waves): row 8w + lane / 8, tokens 4 (lane % 8) + (0..3).
  auto init_lane = [&](SoftmaxLane& sl, int row8) {
    sl.row = row8 + (c.lane >> 3);
    sl.tg = c.lane & 7;
    const int iq = (r0 + sl.row) / a.H;  // query token of the row
    sl.lim = min(min(max(L - a.sq + iq + 1, 0), L), c.t_hi);
    // The group's first row has the smallest query index, hence the smallest limit.
    const int iq_w = (r0 + row8) / a.H;
    sl.lim_w = min(min(max(L - a.sq + iq_w + 1, 0), L), c.t_hi);
    sl.m_run = -INFINITY;
    sl.l_run = 0.f;
  };
  SoftmaxLane st, st2;
  init_lane(st, 8 * c.w);
  (void)st2;

  // Row sums and log-sum-exp of this lane's row, once its last tile is done.
  auto finish_rows = [&](const SoftmaxLane& sl) {
    const float l_tot = sum8(sl.l_run);
    if (sl.tg == 0) {
      sm.lsum[sl.row] = l_tot;
      const float lse2 = l_tot > 0.f ? sl.m_run + log2f(l_tot) : -INFINITY;
      if (single) {
        if (a.lse) a.lse[out_base + r0 + sl.row] = lse2 * kLn2;
      } else {
        a.part_lse[out_base + r0 + sl.row] = lse2;
      }
    }
  };

  if (c.w < 4) {
    // ================================ score waves ===================================
    // Query operands (B of phase 1): rows r0 + 32 rb2 + n, this wave's column slice.
    bf16x8 qb[2][8];
    bf16x8 qrb[2];
    {
      const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat);
      const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope);
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2) {
        const int64_t row = int64_t(b) * rows + r0 + 32 * rb2 + c.n;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          qb[rb2][s] = __builtin_bit_cast(bf16x8, ld16(ql + row * kDC + kCols * c.w + kcol(s, c.h)));
        qrb[rb2] = __builtin_bit_cast(bf16x8, ld16(qr + row * kDR + kRopeW * c.w + 8 * c.h));
      }
    }
    // fp8 score product: each row's 128-column slice (this wave's) is rounded to e4m3 with
    // scale max|x| / 448; q8[rb2][m] holds the codes of columns 64m + 32j + 16h + (0..15),
    // j = 0, 1, in the byte order of the cache operand (tr.lat[2m + j]).
    v8i q8[2][2];
    float qs[2];
    if constexpr (QK8) {
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2) {
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(float(qb[rb2][s][e])));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));  // the row's other 64 columns
        qs[rb2] = amax > 0.f ? amax * (1.f / 448.f) : 1.f;
        const float inv = amax > 0.f ? 448.f / amax : 1.f;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int d = 0; d < 8; ++d) {  // dword d: columns of k-step 4m + d / 2, half d % 2
            const bf16x8 src = qb[rb2][4 * m + d / 2];
            const int o = 4 * (d % 2);
            auto q = [&](int e) { return fminf(fmaxf(float(src[o + e]) * inv, -448.f), 448.f); };
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(q(0), q(1), 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(q(2), q(3), w, true);
            q8[rb2][m][d] = w;
          }
      }
    }
    // Tile n moves through the pipeline as: registers (loaded two tiles ahead) -> staged in
    // LDS and scored in step n - 1 -> softmax in step n -> product with V in step n + 1.
    // Each step ends with the workgroup's only barrier of that step.
    u32x4 av[8];  // latent score operands of the tile being scored
    bf16x8 ar;    // RoPE score operand
    // Stage tile n: write this wave's latent slice to v[n % 2] as bf16 (the output waves'
    // V) and set the score operands.  bf16: read the slice back in operand layout (LDS
    // operations of one wave complete in order, so no barrier is needed).  fp8: convert the
    // codes, which are already the operands.  Either way the registers are refilled with
    // tile n + 2 after the score product and the softmax (they are free meanwhile).
    auto stage = [&](TileRegs<FP8>& tr, int n) {
      const int buf = n & 1;
      uint16_t* vs = &sm.v[buf][c.w][0][0];
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 w = tr.lat[j];
          av[2 * j] = e4m3x8_to_bf16x8(w[0], w[1]);
          av[2 * j + 1] = e4m3x8_to_bf16x8(w[2], w[3]);
        }
        if (c.h == 0) sm.ts[buf][c.w][c.n] = tr.ts;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          *reinterpret_cast<u32x4*>(vs + c.n * kCols + 8 * ((kcol(s, c.h) >> 3) ^ swz32(c.n))) = av[s];
        ar = __builtin_bit_cast(bf16x8, tr.rope);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int tok = lat_token(k, c.lane);
          *reinterpret_cast<u32x4*>(vs + tok * kCols + 8 * ((c.lane & 15) ^ swz32(tok))) = tr.lat[k];
        }
        ar = __builtin_bit_cast(bf16x8, tr.rope);
#pragma unroll
        for (int s = 0; s < 8; ++s)
          av[s] = *reinterpret_cast<const u32x4*>(vs + c.n * kCols + 8 * ((kcol(s, c.h) >> 3) ^ swz32(c.n)));
      }
    };
    // Refill the registers of tile n with tile n + 2.
    auto refill_after_score = [&](TileRegs<FP8>& tr, int n) { load_tile<FP8, PK>(tr, c, a, t_lo + (n + 2) * kTile); };
    // Partial scores of the staged tile n into spart[n % 2]; `mid` runs once the latent
    // products are issued (the previous tile's softmax in the steady state).
    auto score = [&](const TileRegs<FP8>& tr, int n, auto mid) {
      const int buf = n & 1;
      f32x16 sacc[2];
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[rb2][e] = 0.f;
      if constexpr (!FP8) {
        // RoPE term first: the wave can leave the products' last instruction and run `mid`
        // (the previous tile's softmax) while the matrix unit finishes.
#pragma unroll
        for (int rb2 = 0; rb2 < 2; ++rb2)
          sacc[rb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar, qrb[rb2], sacc[rb2], 0, 0, 0);
      }
      if constexpr (QK8) {
        // Codes times codes, 64 columns per instruction (unit block scales).
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const v8i av8 = {int(tr.lat[2 * m][0]), int(tr.lat[2 * m][1]), int(tr.lat[2 * m][2]), int(tr.lat[2 * m][3]),
                           int(tr.lat[2 * m + 1][0]), int(tr.lat[2 * m + 1][1]), int(tr.lat[2 * m + 1][2]),
                           int(tr.lat[2 * m + 1][3])};
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2)
            sacc[rb2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av8, q8[rb2][m], sacc[rb2], 0, 0, 0, 127, 0, 127);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2)
            sacc[rb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[s]), qb[rb2][s],
                                                                sacc[rb2], 0, 0, 0);
      }
      mid();
      if constexpr (FP8) {
        // Scale the latent part of tokens 8i + 4h + r by their per-token scales (and, for
        // the fp8 product, row n's query scale).
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 tsv = *reinterpret_cast<const f32x4*>(&sm.ts[buf][c.w][8 * i + 4 * c.h]);
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[rb2][4 * i + r] *= QK8 ? tsv[r] * qs[rb2] : tsv[r];
        }
      }
      if constexpr (FP8) {
#pragma unroll
        for (int rb2 = 0; rb2 < 2; ++rb2)
          sacc[rb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar, qrb[rb2], sacc[rb2], 0, 0, 0);
      }
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2) {
        const int row = 32 * rb2 + c.n;
#pragma unroll
        for (int i = 0; i < 4; ++i)  // tokens 8i + 4h + (0..3) = chunk 2i + h
          *reinterpret_cast<f32x4*>(&sm.spart[buf][c.w][row][4 * ((2 * i + c.h) ^ sp_swz(row))]) =
              f32x4{sacc[rb2][4 * i], sacc[rb2][4 * i + 1], sacc[rb2][4 * i + 2], sacc[rb2][4 * i + 3]};
      }
    };
    // Step n (n + 1 < ntiles): stage and score tile n + 1, softmax of tile n.
    auto step = [&](TileRegs<FP8>& tr, int n) {
      stage(tr, n + 1);
      score(tr, n + 1, [&] { softmax_tile<FP8>(sm, st, n & 1, t_lo + n * kTile, a.scale_log2); });
      refill_after_score(tr, n + 1);
      __syncthreads();
    };

    if (steps > 0) {
      // Register set ra holds the even tiles, rb2 the odd ones.
      TileRegs<FP8> ra, rb2;
      load_tile<FP8, PK>(ra, c, a, t_lo);
      load_tile<FP8, PK>(rb2, c, a, t_lo + kTile);
      stage(ra, 0);
      score(ra, 0, [] {});
      refill_after_score(ra, 0);
      __syncthreads();
      // Straight-line pairs: every path into the loop header has the same loads in flight.
      int n = 0;
      for (; n + 2 < ntiles; n += 2) {
        step(rb2, n);
        step(ra, n + 1);
      }
      if (n + 1 < ntiles) {
        step(rb2, n);
        ++n;
      }
      softmax_tile<FP8>(sm, st, n & 1, t_lo + n * kTile, a.scale_log2);  // the last tile
      __syncthreads();
    }

    finish_rows(st);
    __syncthreads();
  } else {
    // ================================ output waves ==================================
    const int q = c.w - 4;
    f32x16 oacc[4][2];  // O^T: cols 128q + 32cb + 8i + 4h + r, rows 32 rb2 + n
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[cb][rb2][e] = 0.f;
    bf16x8 vop[4][2];  // V^T operands of one tile: [column block][token half]

    // V^T operands of tile n, read from LDS one step before its product.
    auto read_v = [&](int n) {
      const uint16_t* vt = &sm.v[n & 1][q][0][0];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vop[cb][ks] = lds_operand_tr32(vt, 16 * ks, 32 * cb, c.lane);
    };
    // O^T = O^T * alpha + V^T P^T for tile n.
    auto pv = [&](int n) {
      const int buf = n & 1;
      float al[2];
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2) al[rb2] = sm.alpha[buf][32 * rb2 + c.n];
      bf16x8 pb[2][2];  // [row block][token half]
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          pb[rb2][ks] = *reinterpret_cast<const bf16x8*>(
              &sm.p[buf][32 * rb2 + c.n][8 * ((2 * ks + c.h) ^ p_swz(32 * rb2 + c.n))]);
      if (__any((al[0] != 1.f) | (al[1] != 1.f))) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2) oacc[cb][rb2] *= al[rb2];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2)
            oacc[cb][rb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[cb][ks], pb[rb2][ks], oacc[cb][rb2], 0, 0, 0);
    };

    if (steps > 0) {
      __syncthreads();  // tile 0 staged and scored
      read_v(0);
      softmax_tile<FP8>(sm, st, 0, t_lo, a.scale_log2);
      __syncthreads();
      for (int n = 1; n < ntiles; ++n) {
        pv(n - 1);
        read_v(n);
        softmax_tile<FP8>(sm, st, n & 1, t_lo + n * kTile, a.scale_log2);
        __syncthreads();
      }
      pv(ntiles - 1);
    }
    finish_rows(st);
    __syncthreads();  // every row sum published

    // Normalised rows into LDS (the partial-score buffers are free now): row r's 16-byte
    // chunk c is stored at chunk c ^ (r & 15), so both the 8-byte writes (16 rows per LDS
    // cycle) and the row reads below are conflict-free.
    uint16_t* os = reinterpret_cast<uint16_t*>(&sm.spart[0][0][0][0]);
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
  // Every wave writes 8 whole rows (1 KB each, 16 bytes per lane).
  {
    const uint16_t* os = reinterpret_cast<const uint16_t*>(&sm.spart[0][0][0][0]);
    uint16_t* dst = static_cast<uint16_t*>(single ? a.o_lat : a.part_o);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int lrow = 8 * c.w + k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + lrow * kDC + 8 * (c.lane ^ (lrow & 15)));
      *reinterpret_cast<u32x4*>(dst + (out_base + r0 + lrow) * kDC + 8 * c.lane) = v;
    }
  }
  __syncthreads();  // the next piece stages into these buffers
}

// ---------------------------------------------------------------------------------------
// Row-block design.  A workgroup owns 64 query rows of one sequence and one split of its
// context in 32-token tiles, and the eight waves take three roles:
//   * loader waves 4, 5 (SIMDs 0, 1): wave 4 + l streams tokens 16 l .. 16 l + 15 of every
//     tile from HBM (whole 1 KB latent rows and 128-byte RoPE rows, 16 bytes per lane, two
//     tiles ahead in registers; fp8 codes converted to bf16 here) and stages them in LDS;
//   * score waves 0, 1 (SIMDs 0, 1): wave w owns rows 32 w .. 32 w + 31 over the whole
//     576-wide key (query operands in registers for the whole split), so a tile's scores
//     come out of one MFMA accumulator and the online softmax runs on it in registers
//     (16 tokens of one row per lane; the lane pair l, l ^ 32 shares a row);
//   * output waves 2, 3, 6, 7 (SIMDs 2, 3): O^T += V^T P^T over 128 columns each, V^T
//     operands read transposed from the staged tile one step ahead.
// Per tile that is 36 products on each score wave's SIMD and 32 on each output SIMD; the
// partial-score exchange of the K-split design is gone.  One barrier per step: in step n
// the loaders stage tile n + 1 (and load tile n + 3), the score waves score tile n and
// publish its probabilities, and the output waves multiply tile n - 1 and read the V^T
// operands of tile n.  The score waves read each product's cache operand from LDS four
// products ahead (scheduling-group barriers hold that order; left to itself the compiler
// issues each read right before its product and waits for it).
struct alignas(16) Smem3 {
  uint16_t lat[3][kTile][kDC];          // staged latent rows, chunk c of row t at c ^ swz32(t)
  uint16_t rope[3][kTile][kDR];         // staged RoPE rows, chunk c of row t at c ^ rope_swz(t)
  uint16_t p[2][kRows][kPPitch];        // probabilities (double buffered), [row][tok], p_swz
  float ts[3][kTile];                   // fp8 per-token scales
  float alpha[2][kRows];
  float lsum[kRows];
  int64_t prefix[kMaxPrefixBatch + 1];
  int64_t wave_tot[kThreads / 64];
};

__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }

// V^T operand (as lds_operand_tr32) from a staged tile with 1 KB rows.
__device__ __forceinline__ bf16x8 lds_operand_tr512(const uint16_t* tile, int k0, int c0, int lane) {
  const int G = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int col = c0 + 16 * (G & 1) + 4 * q;
  const int k_lo = k0 + 8 * (G >> 1) + r, k_hi = k_lo + 4;
  const u32x2 lo = lds_read_tr4(tile + k_lo * kDC + 8 * ((col >> 3) ^ swz32(k_lo)) + (col & 7));
  const u32x2 hi = lds_read_tr4(tile + k_hi * kDC + 8 * ((col >> 3) ^ swz32(k_hi)) + (col & 7));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// A loader wave's registers for its 16 tokens of one tile.
template <bool FP8>
struct LoadRegs {
  u32x4 lat[FP8 ? 8 : 16];  // bf16: load k = token k (1 KB row); fp8: tokens 2k + lane / 32
  u32x4 rope[2];            // load j: token 8 j + lane / 8, 16-byte chunk lane % 8
  float ts;                 // fp8: scale of token lane % 16
};

template <bool FP8, int PK, bool QK8>
__device__ __forceinline__ void decode_piece3(Smem3& sm, const DecodeArgs& a, int b, int rb, int t_lo,
                                              int t_hi, int L, bool final_out, int64_t out_base) {
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
  const int ntiles = t_hi > t_lo ? (t_hi - t_lo + kTile - 1) / kTile : 0;
  const bool single = final_out;

  if (c.w == 4 || c.w == 5) {
    // ================================ loader waves ===================================
    const int l = c.w - 4;
    auto lload = [&](LoadRegs<FP8>& r, int t0) {
      constexpr uint32_t kLatBytes = kDC * (FP8 ? 1 : 2);
      constexpr uint32_t kRopeBytes = kDR * 2;
      if constexpr (PK == kPagedAny) {
        // Rows looked up token by token (clamped to the split's last token: every lane
        // issues the same loads from valid rows; the softmax masks the surplus tokens).
        const char* lat = static_cast<const char*>(a.c_kv);
        const char* rope = static_cast<const char*>(a.k_rope);
        const int tb = t0 + 16 * l;
#pragma unroll
        for (int k = 0; k < (FP8 ? 8 : 16); ++k) {
          if constexpr (FP8)
            r.lat[k] = ld16(lat + any_row(c, tb + 2 * k + c.h) * kLatBytes + 16 * (c.lane & 31));
          else
            r.lat[k] = ld16(lat + any_row(c, tb + k) * kLatBytes + 16 * c.lane);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
          r.rope[j] = ld16(rope + any_row(c, tb + 8 * j + (c.lane >> 3)) * kRopeBytes + 16 * (c.lane & 7));
        if constexpr (FP8) r.ts = a.kv_scale[any_row(c, tb + (c.lane & 15))];
        return;
      }
      const char* lat_base;
      const char* rope_base;
      const char* sc_base = nullptr;
      uint32_t nrows, row0;
      if constexpr (PK == kContig) {
        const int64_t seq_row = int64_t(c.b) * c.T;
        lat_base = static_cast<const char*>(a.c_kv) + seq_row * kLatBytes;
        rope_base = static_cast<const char*>(a.k_rope) + seq_row * kRopeBytes;
        if constexpr (FP8) sc_base = reinterpret_cast<const char*>(a.kv_scale + seq_row);
        nrows = uint32_t(c.t_hi);
        row0 = uint32_t(t0);
      } else {
        const int blk = min(t0, c.t_hi - 1) / c.bs;  // the tile lies inside this block
        const int blk_t0 = blk * c.bs;
        const int64_t pool_row = int64_t(c.table[int64_t(c.b) * c.max_blocks + blk]) * c.bs;
        lat_base = static_cast<const char*>(a.c_kv) + pool_row * kLatBytes;
        rope_base = static_cast<const char*>(a.k_rope) + pool_row * kRopeBytes;
        if constexpr (FP8) sc_base = reinterpret_cast<const char*>(a.kv_scale + pool_row);
        nrows = uint32_t(min(c.bs, c.t_hi - blk_t0));
        row0 = uint32_t(t0 - blk_t0);
      }
      // Buffer descriptors whose range ends at the last valid row: rows past it read zeros.
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(lat_base, nrows * kLatBytes);
      const __amdgpu_buffer_rsrc_t rr = make_rsrc(rope_base, nrows * kRopeBytes);
      const uint32_t tb = row0 + uint32_t(16 * l);
#pragma unroll
      for (int k = 0; k < (FP8 ? 8 : 16); ++k) {
        if constexpr (FP8)
          r.lat[k] = buf_ld16(rl, (tb + uint32_t(2 * k + c.h)) * kLatBytes + 16 * (c.lane & 31));
        else
          r.lat[k] = buf_ld16(rl, (tb + uint32_t(k)) * kLatBytes + 16 * c.lane);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        r.rope[j] = buf_ld16(rr, (tb + uint32_t(8 * j + (c.lane >> 3))) * kRopeBytes + 16 * (c.lane & 7));
      if constexpr (FP8) r.ts = buf_ld4f(make_rsrc(sc_base, nrows * 4), (tb + uint32_t(c.lane & 15)) * 4);
    };
    auto lstage = [&](const LoadRegs<FP8>& r, int buf) {
#pragma unroll
      for (int k = 0; k < (FP8 ? 8 : 16); ++k) {
        if constexpr (FP8) {
          const int row = 16 * l + 2 * k + c.h;
          const u32x4 w = r.lat[k];
          const int ch = 2 * (c.lane & 31);
          *reinterpret_cast<u32x4*>(&sm.lat[buf][row][8 * (ch ^ swz32(row))]) = e4m3x8_to_bf16x8(w[0], w[1]);
          *reinterpret_cast<u32x4*>(&sm.lat[buf][row][8 * ((ch + 1) ^ swz32(row))]) = e4m3x8_to_bf16x8(w[2], w[3]);
        } else {
          const int row = 16 * l + k;
          *reinterpret_cast<u32x4*>(&sm.lat[buf][row][8 * (c.lane ^ swz32(row))]) = r.lat[k];
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 16 * l + 8 * j + (c.lane >> 3);
        *reinterpret_cast<u32x4*>(&sm.rope[buf][row][8 * ((c.lane & 7) ^ rope_swz(row))]) = r.rope[j];
      }
      if constexpr (FP8)
        if (c.lane < 16) sm.ts[buf][16 * l + c.lane] = r.ts;
    };
    if (ntiles > 0) {
      LoadRegs<FP8> rx, ry;  // rx holds the even tiles, ry the odd ones
      lload(rx, t_lo);
      lload(ry, t_lo + kTile);
      lstage(rx, 0);
      lload(rx, t_lo + 2 * kTile);
      __syncthreads();
      // Step n stages tile n + 1 and loads tile n + 3 in its place.
      auto lstep = [&](LoadRegs<FP8>& r, int n) {
        if (n + 1 < ntiles) lstage(r, (n + 1) % 3);
        lload(r, t_lo + (n + 3) * kTile);
        __syncthreads();
      };
      int n = 0;
      for (; n + 1 < ntiles; n += 2) {
        lstep(ry, n);
        lstep(rx, n + 1);
      }
      if (n < ntiles) lstep(ry, n);
    }
    __syncthreads();  // row sums published
  } else if (c.w < 2) {
    // ================================ score waves ====================================
    const int row = 32 * c.w + c.n;  // this lane's row of the workgroup
    bf16x8 qb[36];
    {
      const int64_t qrow = int64_t(b) * rows + r0 + row;
      const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + qrow * kDC + 8 * c.h;
      const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope) + qrow * kDR + 8 * c.h;
#pragma unroll
      for (int s = 0; s < 32; ++s) qb[s] = __builtin_bit_cast(bf16x8, ld16(ql + 16 * s));
#pragma unroll
      for (int s = 0; s < 4; ++s) qb[32 + s] = __builtin_bit_cast(bf16x8, ld16(qr + 16 * s));
    }
    const int iq = (r0 + row) / a.H;
    const int lim = min(min(max(L - a.sq + iq + 1, 0), L), t_hi);
    const int iq_w = (r0 + 32 * c.w) / a.H;
    const int lim_w = min(min(max(L - a.sq + iq_w + 1, 0), L), t_hi);
    float m_run = -INFINITY, l_run = 0.f;
    const float scale_log2 = a.scale_log2;

    // Operand offsets: k-step s = 8 j + t of the latent reads chunk 16 j + ((2 t + h) ^ swz32(n))
    // of row n (the swizzle only touches the low 4 chunk bits), RoPE k-step s chunk
    // (2 s + h) ^ rope_swz(n); the eight plus four lane offsets stay in registers and the rest
    // is immediate.
    int loff[8], roff[4];
#pragma unroll
    for (int t = 0; t < 8; ++t) loff[t] = c.n * kDC + 8 * ((2 * t + c.h) ^ swz32(c.n));
#pragma unroll
    for (int t = 0; t < 4; ++t) roff[t] = c.n * kDR + 8 * ((2 * t + c.h) ^ rope_swz(c.n));

    auto tile = [&](int n) {
      const int buf = n % 3;
      const uint16_t* lt = &sm.lat[buf][0][0];
      const uint16_t* rt = &sm.rope[buf][0][0];
      auto operand = [&](int s) {
        return s < 32 ? *reinterpret_cast<const bf16x8*>(lt + 128 * (s >> 3) + loff[s & 7])
                      : *reinterpret_cast<const bf16x8*>(rt + roff[s - 32]);
      };
      // Products s in order (one accumulator; RoPE products apart for fp8), each operand read
      // kPre products ahead.
      constexpr int kSteps = 36, kPre = 4;
      f32x16 acc, accr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[e] = 0.f;
        accr[e] = 0.f;
      }
      bf16x8 ring[kPre];
#pragma unroll
      for (int i = 0; i < kPre; ++i) ring[i] = operand(i);
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const bf16x8 av = ring[s % kPre];
        if (s + kPre < kSteps) ring[s % kPre] = operand(s + kPre);
        if (FP8 && s >= 32)
          accr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[s], accr, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[s], acc, 0, 0, 0);
      }
      // Issue order: the first kPre operand reads, then each product followed by the read
      // kPre products ahead.
#pragma unroll
      for (int i = 0; i < kPre; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s + kPre < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // Lane (n, h) holds tokens 8 i + 4 h + r (e = 4 i + r) of row `row`.
      float sv[16];
      f32x4 tsv[4];
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tsv[i] = *reinterpret_cast<const f32x4*>(&sm.ts[buf][8 * i + 4 * c.h]);
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[e] = fmaf(acc[e], tsv[e >> 2][e & 3], accr[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[e] = acc[e];
      }
      const int t0 = t_lo + n * kTile;
      if (t0 + kTile > lim_w) {
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
      const bool grow = tmax > m_run + kTau;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.f;
      if (grow) m_run = tmax;
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      float pr[16], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pr[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, neg_m));
        psum += pr[e];
      }
      if constexpr (FP8) {
#pragma unroll
        for (int e = 0; e < 16; ++e) pr[e] *= tsv[e >> 2][e & 3];
      }
      l_run = l_run * alpha + psum;
      const int pbuf = n & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x2*>(&sm.p[pbuf][row][8 * (i ^ p_swz(row)) + 4 * c.h]) =
            u32x2{pack_bf16x2(pr[4 * i], pr[4 * i + 1]), pack_bf16x2(pr[4 * i + 2], pr[4 * i + 3])};
      if (c.h == 0) sm.alpha[pbuf][row] = alpha;
    };
    if (ntiles > 0) {
      __syncthreads();  // tile 0 staged
      for (int n = 0; n < ntiles; ++n) {
        tile(n);
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
      if (single) {
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
    bf16x8 vop[4][2];
    auto read_v = [&](int n) {
      const uint16_t* vt = &sm.lat[n % 3][0][0];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vop[cb][ks] = lds_operand_tr512(vt, 16 * ks, kCols * q + 32 * cb, c.lane);
    };
    auto pv = [&](int n) {
      const int buf = n & 1;
      float al[2];
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2) al[rb2] = sm.alpha[buf][32 * rb2 + c.n];
      bf16x8 pb[2][2];
#pragma unroll
      for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          pb[rb2][ks] = *reinterpret_cast<const bf16x8*>(
              &sm.p[buf][32 * rb2 + c.n][8 * ((2 * ks + c.h) ^ p_swz(32 * rb2 + c.n))]);
      if (__any((al[0] != 1.f) | (al[1] != 1.f))) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2) oacc[cb][rb2] *= al[rb2];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int rb2 = 0; rb2 < 2; ++rb2)
            oacc[cb][rb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[cb][ks], pb[rb2][ks], oacc[cb][rb2], 0, 0, 0);
    };
    if (ntiles > 0) {
      __syncthreads();  // tile 0 staged
      read_v(0);
      __syncthreads();  // tile 0 scored
      for (int n = 1; n < ntiles; ++n) {
        pv(n - 1);
        read_v(n);
        __syncthreads();
      }
      pv(ntiles - 1);
    }
    __syncthreads();  // row sums published
    uint16_t* os = &sm.lat[0][0][0];
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
    const uint16_t* os = &sm.lat[0][0][0];
    uint16_t* dst = static_cast<uint16_t*>(single ? a.o_lat : a.part_o);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int lrow = 8 * c.w + k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + lrow * kDC + 8 * (c.lane ^ (lrow & 15)));
      *reinterpret_cast<u32x4*>(dst + (out_base + r0 + lrow) * kDC + 8 * c.lane) = v;
    }
  }
  __syncthreads();  // the next piece stages into these buffers
}

template <bool FP8, int PK, bool QK8, bool V3, typename SM>
__device__ __forceinline__ void piece(SM& sm, const DecodeArgs& a, int b, int rb, int t_lo, int t_hi, int L,
                                      bool fin, int64_t base) {
  if constexpr (V3) decode_piece3<FP8, PK, QK8>(sm, a, b, rb, t_lo, t_hi, L, fin, base);
  else decode_piece<FP8, PK, QK8>(sm, a, b, rb, t_lo, t_hi, L, fin, base);
}

// Grid: one workgroup per (row block, work unit), handed out XCD-aware.  Static splits:
// the unit is (sequence, split) and the piece is the split's token chunk.  Balanced ranges:
// the unit is a range of the batch's concatenated tiles, walked sequence by sequence; a
// sequence that lies wholly inside the range is a final piece, the range's cut first and
// last sequences write partials to the range's slots 0 and 1 (slot 0 when one sequence
// covers the whole range).
template <bool FP8, int PK, bool QK8, bool V3>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeArgs a, int num_splits,
                                                                  int chunk, int rblocks, int n_units) {
  __shared__ std::conditional_t<V3, Smem3, Smem> sm;

  // Workgroups are handed to the 8 XCDs round-robin by id; give each XCD a contiguous
  // range of work units so that the row blocks of one piece share an L2.
  const int per_xcd = gridDim.x / 8;
  const int unit = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (unit >= n_units) return;
  const int rb = unit % rblocks;
  const int rows = a.sq * a.H;
  auto seq_len = [&](int b) { return min(max(a.seq_lens ? a.seq_lens[b] : int(a.T), 0), int(a.T)); };

  if (a.prefix == nullptr) {
    const int split = (unit / rblocks) % num_splits;
    const int b = unit / (rblocks * num_splits);
    const int L = seq_len(b);
    const int t_lo = split * chunk;
    if (num_splits > 1 && t_lo >= L) return;  // the combine reads only splits below L
    const bool fin = num_splits == 1;
    piece<FP8, PK, QK8, V3>(sm, a, b, rb, t_lo, min(L, t_lo + chunk), L, fin,
                          fin ? int64_t(b) * rows : (int64_t(b) * num_splits + split) * rows);
    return;
  }

  // Tile prefix of the batch, computed here for small batches (unit 0 also stores it for the
  // combine), else read from the prefix kernel's output.  Up to 64 sequences every wave
  // scans the tile counts itself, one lane per sequence (32-bit sums: at most 64 * 2^20
  // tiles), and finds its first sequence with a ballot: no LDS, no barrier, one load
  // latency.  Larger batches are scanned by the workgroup in LDS.
  const bool wave_pfx = a.prefix_here && a.B >= 1 && a.B <= 64 && a.T <= (int64_t(1) << 25);
  int incl = 0;  // wave_pfx: inclusive tile prefix of sequence `lane`
  if (wave_pfx) {
    const int lane = threadIdx.x & 63;
    const int tl = lane < a.B ? (seq_len(lane) + kTile - 1) / kTile : 0;
    incl = tl;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (unit == 0 && threadIdx.x < 64) {
      int64_t* pg = const_cast<int64_t*>(a.prefix);
      if (lane < a.B) pg[lane] = incl - tl;
      if (lane == a.B - 1) pg[a.B] = incl;
    }
  } else if (a.prefix_here) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto tiles = [&](int i) { return i < a.B ? int64_t((seq_len(i) + kTile - 1) / kTile) : int64_t(0); };
    const int64_t t0 = tiles(2 * tid), t1 = tiles(2 * tid + 1);
    int64_t incl2 = t0 + t1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t v = __shfl_up(incl2, off, 64);
      if (lane >= off) incl2 += v;
    }
    if (lane == 63) sm.wave_tot[wave] = incl2;
    __syncthreads();
    for (int k = 0; k < wave; ++k) incl2 += sm.wave_tot[k];
    const int64_t excl = incl2 - t0 - t1;
    if (2 * tid < a.B) sm.prefix[2 * tid] = excl;
    if (2 * tid + 1 < a.B) sm.prefix[2 * tid + 1] = excl + t0;
    if (tid == kThreads - 1) sm.prefix[a.B] = incl2;  // 2 kThreads >= B: the total
    __syncthreads();
    if (unit == 0)
      for (int i = tid; i <= a.B; i += kThreads) const_cast<int64_t*>(a.prefix)[i] = sm.prefix[i];
  }
  // Prefix entries are the same for every lane: keep them in scalar registers.
  auto pre = [&](int i) -> int64_t {
    if (wave_pfx) return i == 0 ? int64_t(0) : int64_t(__builtin_amdgcn_readlane(incl, i - 1));
    const int64_t v = a.prefix_here ? sm.prefix[i] : a.prefix[i];
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
    return int64_t((uint64_t(hi) << 32) | lo);
  };

  const int w = unit / rblocks, n_ranges = n_units / rblocks;
  const int64_t total = pre(a.B);
  int64_t cur = total * w / n_ranges;
  const int64_t end = total * (w + 1) / n_ranges;
  if (cur >= end) return;
  // First sequence with tiles past the range start.
  int b = 0;
  if (wave_pfx) {
    // Lowest lane whose inclusive prefix passes cur (there is one: cur < total).
    const uint64_t past = __ballot(int((threadIdx.x & 63) < a.B) & int(int64_t(incl) > cur));
    b = __builtin_ctzll(past);
  } else {
    for (int hi = a.B - 1; b < hi;) {
      const int mid = (b + hi) / 2;
      if (pre(mid + 1) > cur) hi = mid;
      else b = mid + 1;
    }
  }
  for (bool first = true; cur < end; first = false) {
    const int64_t p0 = pre(b), p1 = pre(b + 1);
    const int64_t e = min(end, p1);
    const int L = seq_len(b);
    const bool fin = cur == p0 && e == p1;
    const int64_t base = fin ? int64_t(b) * rows : (int64_t(w) * 2 + (first ? 0 : 1)) * rows;
    piece<FP8, PK, QK8, V3>(sm, a, b, rb, int(cur - p0) * kTile, min(L, int(e - p0) * kTile), L, fin, base);
    cur = e;
    for (++b; b < a.B && pre(b + 1) <= cur;) ++b;  // skip sequences without tiles
  }
}

template <bool FP8, int PK, bool QK8 = false, bool V3 = !QK8>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = p.rows / kRows;
  const int n_units = p.balanced ? p.num_splits * rblocks : a.B * p.num_splits * rblocks;
  const int grid = (n_units + 7) / 8 * 8;
  hipLaunchKernelGGL((decode_mfma_kernel<FP8, PK, QK8, V3>), dim3(grid), dim3(kThreads), 0, s, a,
                     p.num_splits, p.split_tokens, rblocks, n_units);
  return int(hipGetLastError());
}

}  // namespace

int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int pk = !a.paged ? kContig : (a.block_size % kTile == 0 ? kPagedTile : kPagedAny);
  if (a.kv_dt == MLA_FP8_E4M3 && a.fp8_scores) {
    if (pk == kContig) return launch_t<true, kContig, true>(a, p, s);
    return pk == kPagedTile ? launch_t<true, kPagedTile, true>(a, p, s) : launch_t<true, kPagedAny, true>(a, p, s);
  }
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
