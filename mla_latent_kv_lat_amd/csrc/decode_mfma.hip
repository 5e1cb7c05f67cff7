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
// A workgroup owns 64 query rows of one sequence and one split of its context, walked in
// 32-token tiles, and its eight waves take three roles:
//   * loader waves 4, 5 (SIMDs 0, 1): wave 4 + l streams tokens 16 l .. 16 l + 15 of every
//     tile from HBM (whole 1 KB latent rows and 128-byte RoPE rows, 16 bytes per lane, two
//     tiles ahead in registers; fp8 codes are converted to bf16 here) and stages them in LDS;
//   * score waves 0, 1 (SIMDs 0, 1): wave w owns rows 32 w .. 32 w + 31 over the whole
//     576-wide key (query operands in registers for the whole split), so a tile's scores
//     come out of one MFMA accumulator and the online softmax runs on it in registers
//     (16 tokens of one row per lane; the lane pair l, l ^ 32 shares a row);
//   * output waves 2, 3, 6, 7 (SIMDs 2, 3): O^T += V^T P^T over 128 columns each, V^T
//     operands read transposed from the staged tile one step ahead.
// Per tile that is 36 products (bf16) on each score wave's SIMD and 32 on each output SIMD.
// One barrier per step: in step n the loaders stage tile n + 1 (and load tile n + 3), the
// score waves score tile n and publish its probabilities, and the output waves multiply
// tile n - 1 and read the V^T operands of tile n.  The score waves read each product's
// cache operand from LDS ahead of the product (scheduling-group barriers hold that order;
// left to itself the compiler issues each read right before its product and waits for it).
// At the end the output waves park the normalised rows in LDS and all eight waves write
// them out as whole 1 KB rows.
//
// Softmax runs in base-2 units (scores times softmax_scale * log2(e), exponentials by the
// hardware base-2 exponential; results that would be denormal flush to 0) against a per-row
// reference max that only moves when a tile exceeds it by more than kTau; output waves
// skip the accumulator rescale whenever no row's reference moved.  fp8 (OCP e4m3fn)
// caches are converted exactly to bf16; the per-token scale multiplies the latent part of
// the score and the probability used in the PV product.  (The fp8 score and value products
// run in their own kernel, decode_fp8.hip.)
#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"
#include "decode_walk.h"

namespace mla {
namespace {

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kRows = 64;               // query rows per workgroup (two 32-row blocks)
constexpr int kTile = 32;               // tokens per tile
constexpr int kThreads = 512;           // 2 score, 2 loader and 4 output waves
constexpr int kCols = 128;              // latent columns per output wave
constexpr int kPPitch = kTile;          // bf16 per row of the probability tile (swizzled, p_swz)
constexpr int kMaxPrefixBatch = 2 * kThreads;  // largest batch whose tile prefix each workgroup computes
// A row's reference max (the value its probabilities are taken relative to) only moves
// when a tile's max exceeds it by more than this many base-2 units, so probabilities stay
// below 2^kTau and the output waves almost never have to rescale their accumulators.
// The result is the same up to rounding: numerator and denominator share the reference.
constexpr float kTau = 8.f;
static_assert(kMaxInKernelPrefixBatch <= kMaxPrefixBatch, "in-kernel tile prefix does not fit");

// Probability rows hold 4 chunks of 8 tokens (64 bytes); chunk c of row r is stored at
// c ^ p_swz(r), which keeps the score waves' writes (16 lanes of 8 bytes: 16 rows, one chunk
// each) and the output waves' operand reads (16 lanes of 16 bytes: 16 rows) on distinct banks.
__device__ __forceinline__ int p_swz(int row) { return (row >> 2) & 3; }

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

// Staged tiles are double buffered: in step n the loaders write buffer (n + 1) % 2 while
// the score and output waves read buffer n % 2.
struct alignas(16) Smem {
  static constexpr int kNB = 2;
  uint16_t lat[kNB][kTile][kDC];        // staged latent rows (bf16), chunk c of row t at c ^ swz32(t)
  uint16_t rope[kNB][kTile][kDR];       // staged RoPE rows, chunk c of row t at c ^ rope_swz(t)
  uint16_t p[2][kRows][kPPitch];        // probabilities (double buffered), [row][tok], p_swz
  float ts[kNB][kTile];                 // fp8 per-token scales
  float alpha[2][kRows];
  float lsum[kRows];
  int64_t prefix[kMaxPrefixBatch + 1];
  int64_t wave_tot[kThreads / 64];
};

__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }

// A loader wave's registers for its 16 tokens of one tile.
template <bool FP8>
struct LoadRegs {
  u32x4 lat[FP8 ? 8 : 16];  // bf16: load k = token k (1 KB row); fp8: tokens 2k + lane / 32
  u32x4 rope[2];            // load j: token 8 j + lane / 8, 16-byte chunk lane % 8
  float ts;                 // fp8: scale of token lane % 16
};

// One piece of work: query rows [64 rb, 64 rb + 64) of sequence b (length L) over its
// tokens [t_lo, t_hi).  A final piece covers the whole sequence and writes o_lat and lse;
// any other piece writes its normalised partial output and base-2 log-sum-exp.  Row r of
// the row block goes to row out_base + 64 rb + r of the target arrays.  Every wave of
// the workgroup calls it with the same arguments (it contains barriers).
template <bool FP8, int PK>
__device__ __forceinline__ void decode_piece(Smem& sm, const DecodeArgs& a, int b, int rb, int t_lo,
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
  constexpr int kNB = Smem::kNB;

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
        if (n + 1 < ntiles) lstage(r, (n + 1) % kNB);
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
    // Query operands (B): qb[s] = columns 16 s + 8 h .. + 7 of the row for latent k-step s < 32,
    // RoPE dims 16 (s - 32) + 8 h .. + 7 for s = 32 .. 35.
    bf16x8 qb[36];
    {
      const int64_t qrow = int64_t(b) * rows + r0 + row;
      const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + qrow * kDC;
      const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope) + qrow * kDR + 8 * c.h;
#pragma unroll
      for (int s = 0; s < 32; ++s) qb[s] = __builtin_bit_cast(bf16x8, ld16(ql + 16 * s + 8 * c.h));
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
      const int buf = n % kNB;
      const uint16_t* lt = &sm.lat[buf][0][0];
      const uint16_t* rt = &sm.rope[buf][0][0];
      auto operand = [&](int s) {
        return s < 32 ? *reinterpret_cast<const bf16x8*>(lt + 128 * (s >> 3) + loff[s & 7])
                      : *reinterpret_cast<const bf16x8*>(rt + roff[s - 32]);
      };
      f32x16 acc, accr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[e] = 0.f;
        accr[e] = 0.f;
      }
      {
        // Products s in order (one accumulator; RoPE products apart for fp8), each operand
        // read kPre products ahead.
        constexpr int kSteps = 36, kPre = 4;
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
      const uint16_t* vt = &sm.lat[n % kNB][0][0];
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

// Launch bounds: 512 threads and at least 2 waves per SIMD (HIP's second argument counts
// waves per SIMD), i.e. one 8-wave workgroup per compute unit, which is what the kernel's
// 91 KB of LDS allows; each wave may then hold up to 256 registers.
template <bool FP8, int PK>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeArgs a, int num_splits,
                                                                  int chunk, int rblocks, int n_units, int n_xcd) {
  __shared__ Smem sm;
  walk_pieces<kTile, kThreads>(a, num_splits, chunk, rblocks, n_units, n_xcd, sm.prefix, sm.wave_tot,
                               [&](int b, int rb, int t_lo, int t_hi, int L, bool fin, int64_t base) __attribute__((always_inline)) {
                                 decode_piece<FP8, PK>(sm, a, b, rb, t_lo, t_hi, L, fin, base);
                               });
}

template <bool FP8, int PK>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = p.rows / kRows;
  const int n_units = p.balanced ? p.num_splits * rblocks : a.B * p.num_splits * rblocks;
  const int n_xcd = p.n_xcd > 0 ? p.n_xcd : 1;
  const int grid = (n_units + n_xcd - 1) / n_xcd * n_xcd;
  hipLaunchKernelGGL((decode_mfma_kernel<FP8, PK>), dim3(grid), dim3(kThreads), 0, s, a,
                     p.num_splits, p.split_tokens, rblocks, n_units, n_xcd);
  return int(hipGetLastError());
}

}  // namespace
int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int pk = !a.paged ? kContig : (a.block_size % kTile == 0 ? kPagedTile : kPagedAny);
  if (a.fp8_scores) return int(hipErrorInvalidValue);  // the fp8 products run in decode_fp8.hip
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
