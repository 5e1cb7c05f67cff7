// Latent-attention decode kernel for bf16 caches, d_c = 512, d_r = 64, on gfx950: 64 query
// rows per workgroup, two score waves per 32-row block taking alternate tiles.
//
// The absorbed form lets every head of a sequence attend over one shared latent
// ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE key;
// "Multi-Head Latent Attention and the compression of the KV cache", paragraph on the
// associativity argument).  With the query already multiplied by W_UK the score of query
// row r (a (query token, head) pair) and token t is  q_lat[r] . c_kv[t] + q_rope[r] . k_rope[t],
// and the latent is also the value.  Per tile of 32 tokens:
//   S^T[tok, row] = C[tok, 0:512] . Q_lat^T + R[tok, 0:64] . Q_rope^T   (36 products per 32 rows)
//   O^T[col, row] += C[tok, col]^T . P^T[tok, row]                      (16 products per 128 columns)
// on the 32 x 32 x 16 bf16 matrix instruction.
//
// Workgroup: 8 waves, wave i on SIMD i % 4.
//   * Score waves 0, 4 (SIMD 0) own rows 0..31 and waves 1, 5 (SIMD 1) rows 32..63, with
//     their query operands in registers.  Wave w takes the tiles of parity w / 4: it scores
//     tile t in step t and runs the softmax of tile t in step t + 1, while the other wave of
//     its SIMD scores tile t + 1.  So each SIMD's matrix unit has the products of one wave to
//     run while the other wave does its vector work, and every step carries 36 products per
//     score SIMD.
//   * Output waves 2, 3, 6, 7 (SIMDs 2, 3) own 128 latent columns each for all 64 rows.  In
//     step s they multiply tile s - 2 (probabilities published in step s - 1, V^T operands
//     read in step s - 1), read the V^T operands of tile s - 1, and issue the direct-to-LDS
//     loads of tile s + 2 (a quarter of each tile per wave).
//   * Tiles stream into a ring of 4 LDS slots (32 latent rows of 1 KB, chunk c of row t at
//     c ^ swz32(t), then 32 RoPE rows of 128 B): tile t is staged by the end of step t - 1,
//     read in steps t and t + 1, and its slot refilled with tile t + 4 in step t + 2.
// One barrier per step.
//
// Softmax in base 2 against a per-row reference fixed at the row's first visible tile and
// shared by the two score waves of the row through LDS: the output accumulators are never
// rescaled (probabilities of later tiles may exceed 1, up to 2^kGuard).  If any row's scores
// rise more than kGuard above its reference, the piece runs again with the reference set to
// the row's true max, found by a first pass over the scores.
#include <type_traits>

#include "decode_walk.h"
#include "device_common.h"
#include "lds_dma.h"
#include "mfma_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kTile = 32;          // tokens per tile
constexpr int kThreads = 512;      // 4 score and 4 output waves
constexpr int kRows = 64;          // query rows per workgroup
constexpr int kCols = 128;         // latent columns per output wave
constexpr int kSlots = 4;          // LDS ring of staged tiles
constexpr int kLoadsPerTile = 9;   // direct-to-LDS loads per output wave and tile
constexpr int kPrefixMax = 64;     // largest batch whose tile prefix the kernel computes itself
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
constexpr float kGuard = 64.f;     // largest rise (base 2) of a row's scores above its reference

enum : int { kContig = 0, kPagedTile = 1, kPagedAny = 2 };

struct alignas(16) SmemPair {
  uint16_t lat[kSlots][kTile][kDC];   // staged latent rows, chunk c of row t at c ^ swz32(t)
  uint16_t rope[kSlots][kTile][kDR];  // staged RoPE rows, chunk c of row t at c ^ rope_swz(t)
  uint16_t p[2][kRows][kTile];        // probabilities of the last two scored tiles, [row][tok], p_swz
  float mref[kRows];                  // each row's softmax reference (base 2)
  float lpart[2][kRows];              // per-parity row sums (epilogue) or row maxima (first pass)
  int flag[kThreads / 64];
  int64_t prefix[kPrefixMax + 1];
  int64_t wave_tot[kThreads / 64];
};

__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }
// Probability rows hold 4 chunks of 8 tokens; chunk c of row r is stored at c ^ p_swz(r).
__device__ __forceinline__ int p_swz(int row) { return (row >> 2) & 3; }

// One piece: query rows [64 rb, 64 rb + 64) of sequence b (length L) over its tokens
// [t_lo, t_hi).  A final piece covers the whole sequence and writes o_lat and lse; any other
// writes its normalised partial output and base-2 log-sum-exp to row out_base + 64 rb + r of
// the partial arrays.  Every wave calls it with the same arguments (it contains barriers).
template <int PK>
__device__ __forceinline__ void pair_piece(SmemPair& sm, const DecodeArgs& a, int b, int rb, int t_lo, int t_hi,
                                           int L, bool final_out, int64_t out_base) {
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(int(threadIdx.x)));
  const int lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int w = int(sgpr(uint32_t(threadIdx.x) >> 6));
  const bool is_score = (w & 2) == 0;  // waves 0, 1, 4, 5
  const int rows = a.sq * a.H;
  const int r0 = rb * kRows;
  const int ntiles = t_hi > t_lo ? (t_hi - t_lo + kTile - 1) / kTile : 0;

  // ------------------------------------------------------------ tile loads (output waves)
  // Output wave q stages rows 8 q .. 8 q + 7 of each tile: 8 latent rows (one 1 KB row per
  // load; lane i fetches chunk i ^ swz32(row), so chunk c lands at c ^ swz32(row)) and the
  // same 8 RoPE rows (one load; lane i fetches chunk (i % 8) ^ rope_swz(row) of row
  // 8 q + i / 8).  Tokens past the piece's last one are clamped to it (the softmax masks them).
  const int q = (w & 1) + 2 * (w >> 2);  // output waves 2, 3, 6, 7 -> 0, 1, 2, 3
  const int tlast = t_hi - 1;
  const char* lat_base = static_cast<const char*>(a.c_kv);
  const char* rope_base = static_cast<const char*>(a.k_rope);
  const int64_t seq_row0 = int64_t(b) * a.T;  // contiguous: first cache row of sequence b
  const uint32_t lat0 = lds_addr(&sm.lat[0][0][0]);
  const uint32_t rope0 = lds_addr(&sm.rope[0][0][0]);
  struct TileRows {
    int64_t row[8];  // cache row (contiguous: within the sequence; paged: within the pool) of rows 8 q + j
    int64_t rope;    // this lane's RoPE row (row 8 q + lane / 8)
  };
  auto tile_rows = [&](int k) {
    TileRows r;
    const int tt = t_lo + k * kTile + 8 * q;  // token of this wave's first row in the tile
    const int jj = lane >> 3;
    if constexpr (PK == kContig) {
#pragma unroll
      for (int j = 0; j < 8; ++j) r.row[j] = min(tt + j, tlast);
      r.rope = min(tt + jj, tlast);
    } else if constexpr (PK == kPagedTile) {
      // The whole tile lies in one block (block_size a multiple of 32).
      const int blk = (t_lo + k * kTile) / a.block_size;
      const int64_t prow0 =
          int64_t(sload_i32(a.block_table + int64_t(b) * a.max_blocks + blk)) * a.block_size - int64_t(blk) * a.block_size;
#pragma unroll
      for (int j = 0; j < 8; ++j) r.row[j] = prow0 + min(tt + j, tlast);
      r.rope = prow0 + min(tt + jj, tlast);
    } else {
      // Any block size: every row looked up on its own.
      const int32_t* tab = a.block_table + int64_t(b) * a.max_blocks;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = min(tt + j, tlast);
        r.row[j] = int64_t(sload_i32(tab + t / a.block_size)) * a.block_size + t % a.block_size;
      }
      r.rope = r.row[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) r.rope = jj == j ? r.row[j] : r.rope;
    }
    return r;
  };
  auto issue = [&](int k) {
    const TileRows r = tile_rows(k);
    const int slot = k % kSlots;
    // The swizzled chunk offsets are formed from an opaque copy of the lane index at every
    // issue: otherwise the compiler keeps all of them live across the products and spills.
    int ln;
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int trow = 8 * q + j;
      const uint32_t dst = lat0 + uint32_t((slot * kTile + trow) * (kDC * 2));
      const uint32_t chunk = uint32_t(16 * (ln ^ swz32(trow)));
      if constexpr (PK == kContig)  // one base per sequence; 32-bit offsets (a sequence spans < 2 GiB)
        dma16_s(lat_base + seq_row0 * (kDC * 2), uint32_t(r.row[j] * (kDC * 2)) + chunk, dst);
      else
        dma16_s(lat_base + r.row[j] * (kDC * 2), chunk, dst);
    }
    const uint32_t rchunk = uint32_t(16 * ((ln & 7) ^ rope_swz(8 * q + (ln >> 3))));
    const uint32_t rdst = rope0 + uint32_t((slot * kTile + 8 * q) * (kDR * 2));
    if constexpr (PK == kContig)
      dma16_s(rope_base + seq_row0 * (kDR * 2), uint32_t(r.rope * (kDR * 2)) + rchunk, rdst);
    else
      dma16_v(rope_base + r.rope * (kDR * 2) + rchunk, rdst);
  };
  // End of step s for an output wave: tile s + 1 staged by this wave (tile s + 2 may still be
  // in flight), then the barrier.
  auto out_sync = [&](int s) {
    if (s + 2 < ntiles) wait_vm<kLoadsPerTile>();
    else wait_vm<0>();
    barrier_lds();
  };
  auto out_start = [&]() {  // tiles 0 and 1 issued, tile 0 awaited
    if (ntiles > 0) issue(0);
    if (ntiles > 1) {
      issue(1);
      wait_vm<kLoadsPerTile>();
    } else {
      wait_vm<0>();
    }
  };

  // ------------------------------------------------------------ score waves' state
  const int rbk = w & 1, par = w >> 2;  // score wave: 32-row block, tile parity
  const int row = 32 * rbk + n;         // this lane's row of the workgroup
  const int iq = (r0 + row) / a.H;      // query token of this lane's row
  const int lim = min(min(max(L - a.sq + iq + 1, 0), L), t_hi);
  const int iq_w = (r0 + 32 * rbk) / a.H;
  const int lim_w = min(min(max(L - a.sq + iq_w + 1, 0), L), t_hi);  // lowest limit of the wave's rows
  const float scale_log2 = a.scale_log2;
  // Operand offsets (bf16 elements within a slot): latent k-step s = 8 j + u reads chunk
  // 16 j + ((2 u + h) ^ swz32(n)) of row n, RoPE k-step s chunk (2 s + h) ^ rope_swz(n).
  int loff[8], roff[4];
#pragma unroll
  for (int u = 0; u < 8; ++u) loff[u] = n * kDC + 8 * ((2 * u + h) ^ swz32(n));
#pragma unroll
  for (int u = 0; u < 4; ++u) roff[u] = n * kDR + 8 * ((2 * u + h) ^ rope_swz(n));
  bf16x8 qb[36];  // query operands (score waves; loaded below)

  // Score of tile t: the 36 products, operands read four products ahead.
  auto score = [&](int t) {
    const uint16_t* lt = &sm.lat[t % kSlots][0][0];
    const uint16_t* rt = &sm.rope[t % kSlots][0][0];
    auto operand = [&](int s) {
      return s < 32 ? *reinterpret_cast<const bf16x8*>(lt + 128 * (s >> 3) + loff[s & 7])
                    : *reinterpret_cast<const bf16x8*>(rt + roff[s - 32]);
    };
    // Two accumulators (even and odd k-steps), so that consecutive products do not wait for
    // each other's results.
    f32x16 acc[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[0][e] = acc[1][e] = 0.f;
    constexpr int kSteps = 36, kPre = 4;
    bf16x8 ring[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) ring[i] = operand(i);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 av = ring[s % kPre];
      if (s + kPre < kSteps) ring[s % kPre] = operand(s + kPre);
      acc[s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[s], acc[s & 1], 0, 0, 0);
    }
    // Issue order: the first kPre operand reads, then each product followed by the read kPre
    // products ahead (left alone the compiler reads each operand right before its product).
#pragma unroll
    for (int i = 0; i < kPre; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s + kPre < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    return acc[0] + acc[1];
  };
  // Masked scores of tile t (lane: 16 tokens 8 i + 4 h + r, e = 4 i + r, of row `row`; the
  // partner lane l ^ 32 holds the other 16) and the row's max over the tile in base-2 units.
  auto masked_max = [&](int t, const f32x16& acc, float (&sv)[16]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = acc[e];
    const int t0 = t_lo + t * kTile;
    if (t0 + kTile > lim_w) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (t0 + 8 * (e >> 2) + 4 * h + (e & 3) >= lim) sv[e] = -INFINITY;
    }
    float tmax = sv[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sv[e]);
    float x0 = tmax, x1 = tmax;
    permlane32_swap(x0, x1);
    return fmaxf(x0, x1) * scale_log2;
  };
  float l_run = 0.f;
  bool rise = false;  // a score of this lane's row rose more than kGuard above the reference
  // Softmax of tile t against the row's reference (set here at the row's first visible tile,
  // for the other score wave of the row as well): probabilities to sm.p[t & 1].
  auto softmax = [&](int t, const f32x16& acc) {
    float sv[16];
    const float tmax = masked_max(t, acc, sv);
    float m = sm.mref[row];
    if (m == -INFINITY && tmax != -INFINITY) {
      m = tmax;  // first visible tile of the row: nothing accumulated yet
      if (h == 0) sm.mref[row] = m;
    }
    rise |= tmax > m + kGuard;
    const float neg_m = m == -INFINITY ? 0.f : -m;
    float pr[16], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pr[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, neg_m));
      psum += pr[e];
    }
    l_run += psum;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x2*>(&sm.p[t & 1][row][8 * (i ^ p_swz(row)) + 4 * h]) =
          u32x2{pack_bf16x2(pr[4 * i], pr[4 * i + 1]), pack_bf16x2(pr[4 * i + 2], pr[4 * i + 3])};
  };

  // ------------------------------------------------------------ output waves' work
  auto read_v = [&](int t, bf16x8 (&vop)[4][2]) {  // V^T operands of tile t
    const uint16_t* vt = &sm.lat[t % kSlots][0][0];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vop[cb][ks] = lds_operand_tr512(vt, 16 * ks, kCols * q + 32 * cb, lane);
  };
  // Products of tile t (its V^T operands in vop); with tn >= 0 each operand is refilled with
  // tile tn's right after its two products, so the reads run under the remaining products.
  auto pv = [&](int t, bf16x8 (&vop)[4][2], f32x16 (&oacc)[4][2], int tn) {
    bf16x8 pb[2][2];
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pb[rb2][ks] = *reinterpret_cast<const bf16x8*>(
            &sm.p[t & 1][32 * rb2 + n][8 * ((2 * ks + h) ^ p_swz(32 * rb2 + n))]);
    const uint16_t* vn = &sm.lat[(tn < 0 ? 0 : tn) % kSlots][0][0];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int rb2 = 0; rb2 < 2; ++rb2)
          oacc[cb][rb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[cb][ks], pb[rb2][ks], oacc[cb][rb2], 0, 0, 0);
        if (tn >= 0) vop[cb][ks] = lds_operand_tr512(vn, 16 * ks, kCols * q + 32 * cb, lane);
      }
  };

  // ------------------------------------------------------------ passes
  // Pass 0 fixes each row's reference at its first visible tile; if any row rose more than
  // kGuard above it, pass 1 first finds every row's max over the piece (scores only) and runs
  // the tiles again against it.  The roles run their whole loops in separate branches (so the
  // query operands and the output accumulators never share a live range) through the same
  // sequence of barriers: pass 1's scan 1 + ntiles + 1, each main loop 1 + ntiles + 1, the
  // rerun decision 2, the row sums 1.
  uint16_t* os = &sm.lat[0][0][0];  // normalised rows parked for the output writes
  if (is_score) {
    // qb[s] = columns 16 s + 8 h .. + 7 of this lane's row for latent k-step s < 32, RoPE
    // dims 16 (s - 32) + 8 h .. + 7 for s = 32 .. 35 (B operand: row = lane % 32).
    {
      const int64_t qrow = int64_t(b) * rows + r0 + row;
      const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + qrow * kDC + 8 * h;
      const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope) + qrow * kDR + 8 * h;
#pragma unroll
      for (int s = 0; s < 32; ++s) qb[s] = __builtin_bit_cast(bf16x8, ld16(ql + 16 * s));
#pragma unroll
      for (int s = 0; s < 4; ++s) qb[32 + s] = __builtin_bit_cast(bf16x8, ld16(qr + 16 * s));
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    if (par == 0 && h == 0) sm.mref[row] = -INFINITY;
    for (int pass = 0; ntiles > 0; ++pass) {
      if (pass == 1) {
        float m_scan = -INFINITY;
        barrier_lds();
        for (int s = 0; s < ntiles; ++s) {
          if ((s & 1) == par) {
            float sv[16];
            m_scan = fmaxf(m_scan, masked_max(s, score(s), sv));
          }
          barrier_lds();
        }
        if (h == 0) sm.lpart[par][row] = m_scan;
        barrier_lds();
        if (par == 0 && h == 0) sm.mref[row] = fmaxf(sm.lpart[0][row], sm.lpart[1][row]);
        l_run = 0.f;
        rise = false;
      }
      // Step s: the wave of parity s & 1 scores tile s, the other runs the softmax of tile
      // s - 1 (whose scores it computed in step s - 1).
      f32x16 acc_keep;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_keep[e] = 0.f;
      barrier_lds();  // tile 0 staged, references set
      for (int s = 0; s <= ntiles; ++s) {
        if ((s & 1) == par) {
          if (s < ntiles) acc_keep = score(s);
        } else if (s >= 1) {
          softmax(s - 1, acc_keep);
        }
        barrier_lds();
      }
      if (pass == 1) break;
      const int rose = int(__any(rise));
      if (lane == 0) sm.flag[w] = rose;
      barrier_lds();
      const int again = sm.flag[0] | sm.flag[1] | sm.flag[4] | sm.flag[5];
      barrier_lds();
      if (!again) break;
    }
    float x0 = l_run, x1 = l_run;
    permlane32_swap(x0, x1);
    if (h == 0) sm.lpart[par][row] = x0 + x1;
    barrier_lds();
    if (par == 0 && h == 0) {
      const float l_tot = sm.lpart[0][row] + sm.lpart[1][row];
      const float m = sm.mref[row];
      const float lse2 = l_tot > 0.f ? m + log2f(l_tot) : -INFINITY;
      if (final_out) {
        if (a.lse) a.lse[out_base + r0 + row] = lse2 * kLn2;
      } else {
        a.part_lse[out_base + r0 + row] = lse2;
      }
    }
  } else {
    f32x16 oacc[4][2];
    bf16x8 vop[4][2];  // V^T operands of the next tile to multiply
    auto zero = [&]() {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[cb][rb2][e] = 0.f;
    };
    zero();  // also the output of a piece without tiles
    for (int pass = 0; ntiles > 0; ++pass) {
      if (pass == 1) {
        out_start();
        barrier_lds();
        for (int s = 0; s < ntiles; ++s) {
          if (s + 2 < ntiles) issue(s + 2);
          out_sync(s);
        }
        barrier_lds();
        zero();
      }
      out_start();
      barrier_lds();  // tile 0 staged, references set
      // Step s: products of tile s - 2 with the V^T reads of tile s - 1 between them, then the
      // loads of tile s + 2.
      for (int s = 0; s <= ntiles; ++s) {
        if (s >= 2) pv(s - 2, vop, oacc, s - 1 < ntiles ? s - 1 : -1);
        else if (s == 1) read_v(0, vop);
        if (s + 2 < ntiles) issue(s + 2);
        out_sync(s);
      }
      pv(ntiles - 1, vop, oacc, -1);
      if (pass == 1) break;
      if (lane == 0) sm.flag[w] = 0;
      barrier_lds();
      const int again = sm.flag[0] | sm.flag[1] | sm.flag[4] | sm.flag[5];
      barrier_lds();
      if (!again) break;
    }
    barrier_lds();  // row sums published
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2) {
      const int lrow = 32 * rb2 + n;
      const float lt = sm.lpart[0][lrow] + sm.lpart[1][lrow];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int chunk = 16 * q + 4 * cb + i;
          const f32x4 v = f32x4{oacc[cb][rb2][4 * i], oacc[cb][rb2][4 * i + 1], oacc[cb][rb2][4 * i + 2],
                                oacc[cb][rb2][4 * i + 3]} * inv;
          *reinterpret_cast<u32x2*>(os + lrow * kDC + 8 * (chunk ^ (lrow & 15)) + 4 * h) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    }
  }
  barrier_lds();
  {
    uint16_t* dst = static_cast<uint16_t*>(final_out ? a.o_lat : a.part_o);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int lrow = 8 * w + k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + lrow * kDC + 8 * (lane ^ (lrow & 15)));
      *reinterpret_cast<u32x4*>(dst + (out_base + r0 + lrow) * kDC + 8 * lane) = v;
    }
  }
  barrier_lds();  // the next piece stages into these buffers
}

// Launch bounds: 512 threads and 2 waves per SIMD (HIP's second argument counts waves per
// SIMD), i.e. one workgroup per compute unit, which is what the kernel's LDS allows; each
// wave may then hold up to 256 registers.
template <int PK>
__global__ __launch_bounds__(kThreads, 2) void pair_decode_kernel(DecodeArgs a, int num_splits, int chunk,
                                                                 int rblocks, int n_units, int n_xcd) {
  __shared__ SmemPair sm;
  walk_pieces<kTile, kThreads>(a, num_splits, chunk, rblocks, n_units, n_xcd, sm.prefix, sm.wave_tot,
                               [&](int b, int rb, int t_lo, int t_hi, int L, bool fin, int64_t base)
                                   __attribute__((always_inline)) { pair_piece<PK>(sm, a, b, rb, t_lo, t_hi, L, fin, base); });
}

template <int PK>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = p.rows / kRows;
  const int n_units = p.balanced ? p.num_splits * rblocks : a.B * p.num_splits * rblocks;
  const int n_xcd = p.n_xcd > 0 ? p.n_xcd : 1;
  const int grid = (n_units + n_xcd - 1) / n_xcd * n_xcd;
  hipLaunchKernelGGL((pair_decode_kernel<PK>), dim3(grid), dim3(kThreads), 0, s, a, p.num_splits, p.split_tokens,
                     rblocks, n_units, n_xcd);
  return int(hipGetLastError());
}

}  // namespace

int launch_decode_pair(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  if (a.kv_dt != MLA_BF16 || a.fp8_scores || a.dc != kDC || a.dr != kDR || p.rows % kRows != 0 ||
      (a.prefix_here && a.B > kPrefixMax))
    return int(hipErrorInvalidValue);
  if (!a.paged) return launch_t<kContig>(a, p, s);
  return a.block_size % kTile == 0 ? launch_t<kPagedTile>(a, p, s) : launch_t<kPagedAny>(a, p, s);
}

}  // namespace mla
