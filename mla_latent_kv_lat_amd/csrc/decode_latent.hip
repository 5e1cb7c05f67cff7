// Latent-attention decode kernel for d_c = 512, d_r = 64 on gfx950: one workgroup holds
// all query rows of a sequence piece, each wave carries its rows from the score to the
// output without handing anything to another wave.
//
// The absorbed form lets every head of a sequence attend over one shared latent
// ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE key;
// "Multi-Head Latent Attention and the compression of the KV cache", paragraph on the
// associativity argument).  With the query already multiplied by W_UK the score of query
// row r (a (query token, head) pair) and token t is  q_lat[r] . c_kv[t] + q_rope[r] . k_rope[t],
// and the latent is also the value.  Per tile of 32 tokens and per 32 query rows that is
//   S^T[tok, row] = C[tok, 0:512] . Q_lat^T + R[tok, 0:64] . Q_rope^T    (36 products, K = 576)
//   O^T[col, row] += C[tok, col]^T . P^T[tok, row]                       (32 products, K = 32)
// on the 32 x 32 x 16 bf16 matrix instruction.
//
// Workgroup: 4 waves, one per SIMD, 128 query rows (wave w owns rows 32 w .. 32 w + 31).
//   * Tiles stream into a ring of 4 LDS slots (36 KB each: 32 latent rows of 1 KB, then 32
//     RoPE rows of 128 B) by direct-to-LDS loads, two tiles ahead of the one being scored;
//     each wave issues a quarter of every tile (8 latent rows and 8 RoPE rows) and waits
//     for its own loads before the step's barrier.  A staged tile is read by every wave, so
//     each cache byte crosses the compute unit's load path once for all 128 rows.
//   * A wave keeps its rows' query operands (144 registers) for the whole piece, its output
//     accumulator O^T [512 x 32] in accumulation registers, and its probabilities in
//     registers: the score accumulator's lane layout (lane l: row l % 32, tokens
//     8 i + 4 (l / 32) + (0..3)) is used directly as the B operand of the value product by
//     numbering that product's 16 k positions in the same token order, and the V^T operands
//     are read transposed from the staged tile in that order.
//   * Step n: wait for tile n, barrier, then score, online softmax and value product of
//     tile n; the loads of tile n + 2 (into the slot of tile n - 2) are issued between the
//     value products.
// Softmax is in base 2 against a per-row reference fixed at the first visible tile's max:
// the accumulators are never rescaled inside the loop (probabilities of later tiles may
// exceed 1, up to 2^kGuard).  If any row's scores rise more than kGuard above its
// reference, the piece is run again with the reference set to the row's true max, found by
// a first pass over the scores (never the case unless logits rise by more than 44 natural
// units along a sequence).
#include <type_traits>

#include "device_common.h"
#include "lds_dma.h"
#include "mfma_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kTile = 32;                      // tokens per tile
constexpr int kThreads = 256;                  // 4 waves, one per SIMD
constexpr int kRowsWG = 128;                   // query rows per workgroup
constexpr int kSlots = 4;                      // LDS ring of staged tiles
constexpr int kAhead = 2;                      // tiles loaded ahead of the one being computed
constexpr int kVPre = 5;                       // value-product operands read ahead of their product
constexpr bool kLoadsInValue = true;           // tile loads issued between the value products
constexpr int kLatPitch = kDC * 2 + 64;        // bytes per staged latent row (1 KB + 64 B)
constexpr int kLatSlot = kTile * kLatPitch;    // 34 KB of latent rows per slot
constexpr int kRopeSlot = kTile * kDR * 2;     // 4 KB of RoPE rows per slot
constexpr int kSlotBytes = kLatSlot + kRopeSlot;
constexpr int kLoadsPerTile = 9;               // direct-to-LDS loads per wave and tile
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
constexpr float kGuard = 64.f;  // largest rise (base 2) of a row's scores above its reference
static_assert(kSlots * kSlotBytes >= kRowsWG * kDC * 2, "output staging must fit in the ring");

enum : int { kContig = 0, kPagedTile = 1, kPagedAny = 2 };

struct alignas(1024) SmemL {
  uint8_t ring[kSlots][kSlotBytes];
};

// Staged latent rows are 1088 bytes apart and 16-byte chunk c of row t sits at position
// c ^ lat_swz(t), which only permutes each aligned group of 4 chunks:
//   * score operand reads (16 lanes = 16 rows at one chunk) hit 16 distinct 16-byte bank
//     groups: the 64-byte pad puts rows t and t + 1 four groups apart, the swizzle separates
//     rows t and t + 4;
//   * transposed value-operand reads (32 lanes = an aligned group of 4 rows at 4 chunks, 8
//     bytes each) cover 32 distinct 8-byte bank pairs;
//   * the chunk's group of 4 (a 32-column block) is untouched, so every operand address is a
//     per-lane base plus a constant.
__device__ __forceinline__ int lat_swz(int row) { return (row >> 2) & 3; }
// Staged RoPE rows are 128 bytes; chunk c of row t at c ^ rope_swz(t) (16 rows at one chunk
// on distinct bank groups).
__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }

// Lane base address (bytes, within a slot) of the A operand of O^T += V^T P^T for k-step j,
// half hi of the operand, read transposed from the staged latent rows; the operand of the
// 32-column block cb is at this base + 64 cb.  Lane l receives column 32 cb + l % 32 at tokens
// 16 j + 4 g + (0..3) (hi = 0) and 16 j + 8 + 4 g + (0..3) (hi = 1), g = l / 32: the token
// order of the score accumulator's lanes.  Within each 16-lane group G, lane 4 r + q supplies
// row k0 + r, columns 16 (G & 1) + 4 q .. + 3 of the block.
__device__ __forceinline__ uint32_t v_base(int j, int hi, int lane) {
  const int G = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int k = 16 * j + 8 * hi + 4 * (G >> 1) + r;
  const int cc = 2 * (G & 1) + (q >> 1);  // chunk within the block's group of 4
  return uint32_t(k * kLatPitch + 16 * (cc ^ lat_swz(k)) + 8 * (q & 1));
}

// One piece: query rows [128 rb, 128 rb + 128) of sequence b (length L) over its tokens
// [t_lo, t_hi).  A final piece covers the whole sequence and writes o_lat and lse; any other
// writes its normalised partial output and base-2 log-sum-exp to row out_base + 128 rb + r of
// the partial arrays.  Every wave calls it with the same arguments (it contains barriers).
template <int PK>
__device__ __forceinline__ void decode_piece(SmemL& sm, const DecodeArgs& a, int b, int rb, int t_lo, int t_hi,
                                             int L, bool final_out, int64_t out_base) {
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(int(threadIdx.x)));
  const int lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int w = int(sgpr(uint32_t(threadIdx.x) >> 6));
  const int rows = a.sq * a.H;
  const int r0 = rb * kRowsWG;
  const int wrow0 = r0 + 32 * w;              // first query row of this wave
  const bool active = wrow0 < rows;           // rows % 32 == 0: a wave's rows are all valid or none
  const int ntiles = t_hi > t_lo ? (t_hi - t_lo + kTile - 1) / kTile : 0;
  const uint32_t ring = lds_addr(&sm.ring[0][0]);

  const int row = wrow0 + n;
  bf16x8 qb[36];  // query operands (loaded below, once the first tiles are in flight)

  // ------------------------------------------------------------ tile loads (ring)
  // Wave w stages rows 8 w .. 8 w + 7 of each tile: 8 latent rows (one 1 KB row per load;
  // lane i fetches the row's chunk i ^ lat_swz(row), so chunk c lands at c ^ lat_swz(row)) and
  // the same 8 RoPE rows (one load; lane i fetches chunk (i % 8) ^ rope_swz(row) of row
  // 8 w + i / 8).  Tokens past the piece's last one are clamped to it (the softmax masks them).
  const int tlast = t_hi - 1;
  const char* lat_base = static_cast<const char*>(a.c_kv);
  const char* rope_base = static_cast<const char*>(a.k_rope);
  const int64_t seq_row0 = int64_t(b) * a.T;  // contiguous: first cache row of sequence b
  // Rows of tile k staged by this wave, looked up once per tile (wave-uniform).
  struct TileRows {
    int64_t row[8];  // cache row (contiguous: within the sequence; paged: within the pool) of rows 8 w + j
    int64_t rope;    // this lane's RoPE row (row 8 w + lane / 8)
  };
  auto tile_rows = [&](int k) {
    TileRows r;
    const int tt = t_lo + k * kTile + 8 * w;  // token of this wave's first row in the tile
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
  // Load j of this wave's share of tile k (j < 8: latent row 8 w + j; j = 8: the 8 RoPE rows).
  auto issue_part = [&](int k, const TileRows& r, int j) {
    const uint32_t slot = ring + uint32_t(k % kSlots) * kSlotBytes;
    if (j < 8) {
      if constexpr (PK == kContig)  // one base per sequence; 32-bit offsets (a sequence spans < 2 GiB)
        dma16_s(lat_base + seq_row0 * (kDC * 2), uint32_t(r.row[j] * (kDC * 2)) + uint32_t(16 * (lane ^ lat_swz(8 * w + j))),
                slot + uint32_t((8 * w + j) * kLatPitch));
      else
        dma16_s(lat_base + r.row[j] * (kDC * 2), uint32_t(16 * (lane ^ lat_swz(8 * w + j))),
                slot + uint32_t((8 * w + j) * kLatPitch));
    } else {
      const uint32_t rope_chunk = uint32_t(16 * ((lane & 7) ^ rope_swz(8 * w + (lane >> 3))));
      const uint32_t dst = slot + uint32_t(kLatSlot + 8 * w * kDR * 2);
      if constexpr (PK == kContig)
        dma16_s(rope_base + seq_row0 * (kDR * 2), uint32_t(r.rope * (kDR * 2)) + rope_chunk, dst);
      else
        dma16_v(rope_base + r.rope * (kDR * 2) + rope_chunk, dst);
    }
  };
  auto issue = [&](int k) {
    const TileRows r = tile_rows(k);
#pragma unroll
    for (int j = 0; j < kLoadsPerTile; ++j) issue_part(k, r, j);
  };

  // ---------------------------------------------------------------- softmax state
  const int iq = row / a.H;  // query token of this lane's row
  const int lim = min(min(max(L - a.sq + iq + 1, 0), L), t_hi);
  const int iq_w = wrow0 / a.H;
  const int lim_w = min(min(max(L - a.sq + iq_w + 1, 0), L), t_hi);  // lowest limit of the wave's rows
  const float scale_log2 = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  bool rise = false;  // a score of this lane's row rose more than kGuard above the reference

  // Lane bases (bytes within a slot) of the score's A operands: latent k-step s reads chunk
  // 2 s + h of token n, at sbase[s & 1] + 64 (s >> 1); RoPE k-step 32 + u reads chunk
  // (2 u + h) ^ rope_swz(n) of RoPE row n.
  uint32_t sbase[2], rbase[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) sbase[u] = uint32_t(n * kLatPitch + 16 * ((2 * u + h) ^ lat_swz(n)));
#pragma unroll
  for (int u = 0; u < 4; ++u) rbase[u] = uint32_t(kLatSlot + n * (kDR * 2) + 16 * ((2 * u + h) ^ rope_swz(n)));
  uint32_t vbase[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) vbase[j][hi] = v_base(j, hi, lane);

  f32x16 oacc[16];  // zero also for a piece without tiles (its output is 0)
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[cb][e] = 0.f;

  // Score of tile k: the 36 products, operands read four products ahead.
  auto score = [&](int k) {
    const uint8_t* st = &sm.ring[k % kSlots][0];
    const uint8_t* sl[2] = {st + sbase[0], st + sbase[1]};
    const uint8_t* sr[4] = {st + rbase[0], st + rbase[1], st + rbase[2], st + rbase[3]};
    auto operand = [&](int s) {
      return s < 32 ? *reinterpret_cast<const bf16x8*>(sl[s & 1] + 64 * (s >> 1))
                    : *reinterpret_cast<const bf16x8*>(sr[s - 32]);
    };
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    constexpr int kSteps = 36, kPre = 4;
    bf16x8 ringop[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) ringop[i] = operand(i);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 av = ringop[s % kPre];
      if (s + kPre < kSteps) ringop[s % kPre] = operand(s + kPre);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[s], acc, 0, 0, 0);
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
    return acc;
  };

  // Masked scores of tile k (lane: 16 tokens of row `row`; the partner lane l ^ 32 holds the
  // other 16) and the row's max over the tile in base-2 units.
  auto masked_max = [&](int k, const f32x16& acc, float (&sv)[16]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = acc[e];
    const int t0 = t_lo + k * kTile;
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

  // Online softmax of tile k against the row's reference: probabilities packed as the value
  // product's B operands (element 4 i + r of k-step i / 2 is token 8 i + 4 h + r).
  auto softmax = [&](int k, const f32x16& acc, bf16x8 (&pb)[2]) {
    float sv[16];
    const float tmax = masked_max(k, acc, sv);
    if (m_run == -INFINITY) m_run = tmax;  // first visible tile: nothing accumulated yet
    rise |= tmax > m_run + kGuard;
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float pr[16], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pr[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, neg_m));
      psum += pr[e];
    }
    l_run += psum;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pb[j] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(pr[8 * j], pr[8 * j + 1]), pack_bf16x2(pr[8 * j + 2], pr[8 * j + 3]),
                                              pack_bf16x2(pr[8 * j + 4], pr[8 * j + 5]), pack_bf16x2(pr[8 * j + 6], pr[8 * j + 7])});
  };

  // Value product of tile k with probabilities pb.  With kd >= 0 the wave's 9 loads of tile
  // kd are issued between the products (one after every third), where their issue time
  // overlaps the matrix unit's work.
  auto value = [&](int k, const bf16x8 (&pb)[2], int kd) {
    const uint8_t* vt = &sm.ring[k % kSlots][0];
    const uint8_t* vb[2][2] = {{vt + vbase[0][0], vt + vbase[0][1]}, {vt + vbase[1][0], vt + vbase[1][1]}};
    auto vop_read = [&](int s) {  // operand of block s / 2, k-step s % 2
      const int cb = s >> 1, j = s & 1;
      const u32x2 lo = lds_read_tr4(reinterpret_cast<const uint16_t*>(vb[j][0] + 64 * cb));
      const u32x2 hi = lds_read_tr4(reinterpret_cast<const uint16_t*>(vb[j][1] + 64 * cb));
      return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    auto products = [&](auto with_loads) {
      constexpr bool kLoads = decltype(with_loads)::value;
      TileRows tr;
      if constexpr (kLoads) tr = tile_rows(kd);
      bf16x8 vop[kVPre];
#pragma unroll
      for (int i = 0; i < kVPre; ++i) vop[i] = vop_read(i);
#pragma unroll
      for (int s = 0; s < 32; ++s) {
        const int cb = s >> 1, j = s & 1;
        const bf16x8 av = vop[s % kVPre];
        if (s + kVPre < 32) vop[s % kVPre] = vop_read(s + kVPre);
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[j], oacc[cb], 0, 0, 0);
        if constexpr (kLoads)
          if (s % 3 == 0 && s / 3 < kLoadsPerTile) issue_part(kd, tr, s / 3);
      }
      // Issue order: the first kVPre operands' reads, then each product followed by the reads
      // of the operand kVPre products ahead (the loads, which the compiler cannot classify,
      // stay between the reads they sit between in the code).
#pragma unroll
      for (int i = 0; i < kVPre; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int s = 0; s < 32; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s + kVPre < 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    };
    if constexpr (kLoadsInValue) {
      if (kd >= 0) products(std::true_type{});
      else products(std::false_type{});
    } else {
      products(std::false_type{});
    }
  };

  // ---------------------------------------------------------------- main loop
  // Step k: tile k is resident, the next kAhead - 1 tiles are in flight, and tile k + kAhead
  // is issued into the slot of tile k - 1 (kAhead < kSlots).
  auto step_sync = [&](int k) {
    const int newer = min(kAhead - 1, ntiles - 1 - k);  // this wave's later tiles still in flight
    if (newer >= 2) wait_vm<2 * kLoadsPerTile>();
    else if (newer == 1) wait_vm<kLoadsPerTile>();
    else wait_vm<0>();
    barrier_lds();  // tile k staged by every wave; tile k - 1's slot is free
  };
  static_assert(kAhead >= 1 && kAhead < kSlots, "tile pipeline depth");
  auto start = [&]() {
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
      if (k < ntiles) issue(k);
  };

  // ---------------------------------------------------------------- query operands
  // qb[s] = columns 16 s + 8 h .. + 7 of this lane's row for latent k-step s < 32, RoPE dims
  // 16 (s - 32) + 8 h .. + 7 for s = 32 .. 35 (B operand: row = lane % 32).  Loaded while
  // the first tiles are in flight, then awaited together with them, so that no load of
  // the compiler's is outstanding inside the tile loop: a wait for one would also drain the
  // tile loads in flight, which the compiler does not count.
  if (ntiles > 0) start();
  if (active) {
    const int64_t qrow = int64_t(b) * rows + row;
    const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + qrow * kDC + 8 * h;
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope) + qrow * kDR + 8 * h;
#pragma unroll
    for (int s = 0; s < 32; ++s) qb[s] = __builtin_bit_cast(bf16x8, ld16(ql + 16 * s));
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[32 + s] = __builtin_bit_cast(bf16x8, ld16(qr + 16 * s));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // Pass 0 fixes each row's reference at its first visible tile; if any row of the
  // workgroup rose more than kGuard above it, pass 1 first finds every row's max over the
  // piece (scores only) and runs the tiles again against it.  Waves with and without rows
  // run separate loops (the branch is wave-uniform), so the accumulators stay in
  // accumulation registers across the loop.
  int* flag = reinterpret_cast<int*>(&sm.ring[0][0]) + kSlots * kSlotBytes / 4 - kThreads / 64;
  for (int pass = 0; ntiles > 0; ++pass) {
    float m_ref = -INFINITY;
    if (pass == 1) {
      start();
      if (active) {
        for (int k = 0; k < ntiles; ++k) {
          step_sync(k);
          if (k + kAhead < ntiles) issue(k + kAhead);
          float sv[16];
          m_ref = fmaxf(m_ref, masked_max(k, score(k), sv));
        }
      } else {
        for (int k = 0; k < ntiles; ++k) {
          step_sync(k);
          if (k + kAhead < ntiles) issue(k + kAhead);
        }
      }
    }
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[cb][e] = 0.f;
    m_run = m_ref;
    l_run = 0.f;
    rise = false;
    if (pass == 1) start();
    if (active) {
      // Score, softmax and value product of tile k in step k.  Steps that still issue loads,
      // then the last kAhead steps (separate loops, so that no branch inside the step merges
      // two versions of the accumulators).
      int k = 0;
      for (; k + kAhead < ntiles; ++k) {
        step_sync(k);
        if (!kLoadsInValue) issue(k + kAhead);
        bf16x8 pb[2];
        softmax(k, score(k), pb);
        value(k, pb, kLoadsInValue ? k + kAhead : -1);
      }
      for (; k < ntiles; ++k) {
        step_sync(k);
        bf16x8 pb[2];
        softmax(k, score(k), pb);
        value(k, pb, -1);
      }
    } else {
      for (int k = 0; k < ntiles; ++k) {
        step_sync(k);
        if (k + kAhead < ntiles) issue(k + kAhead);
      }
    }
    if (pass == 1) break;
    // Workgroup-wide decision, through four words at the end of the ring once every wave is
    // past its last read of the tiles.
    barrier_lds();
    const int rose = int(__any(rise));
    if (lane == 0) flag[w] = rose;
    barrier_lds();
    const int again = flag[0] | flag[1] | flag[2] | flag[3];
    barrier_lds();
    if (!again) break;
  }

  // ---------------------------------------------------------------- epilogue
  // Row sum over both lane halves; normalised rows parked in LDS (16-byte chunk c of row R
  // at c ^ (R & 15)) and written out as whole 1 KB rows by the wave that owns them.
  float x0 = l_run, x1 = l_run;
  permlane32_swap(x0, x1);
  const float l_tot = x0 + x1;
  barrier_lds();  // every wave is done with the ring
  uint8_t* stage = &sm.ring[0][0];
  if (active) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int R = 32 * w + n;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 4 * cb + i;
        const f32x4 v = f32x4{oacc[cb][4 * i], oacc[cb][4 * i + 1], oacc[cb][4 * i + 2], oacc[cb][4 * i + 3]} * inv;
        *reinterpret_cast<u32x2*>(stage + R * (kDC * 2) + 16 * (c ^ (R & 15)) + 8 * h) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    if (h == 0) {
      const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
      if (final_out) {
        if (a.lse) a.lse[out_base + row] = lse2 * kLn2;
      } else {
        a.part_lse[out_base + row] = lse2;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave reads back only its own rows
    uint16_t* dst = static_cast<uint16_t*>(final_out ? a.o_lat : a.part_o);
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const int R = 32 * w + k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + R * (kDC * 2) + 16 * (lane ^ (R & 15)));
      *reinterpret_cast<u32x4*>(dst + (out_base + r0 + R) * kDC + 8 * lane) = v;
    }
  }
  barrier_lds();  // the next piece stages into these bytes
}

// Grid: one workgroup per (row block, work unit), units handed out so that consecutive
// units share an XCD.  Static splits: the unit is (sequence, split).  Balanced ranges: the
// unit is a range of the batch's concatenated 32-token tiles, walked sequence by sequence;
// a sequence wholly inside the range is a final piece, the range's cut first and last
// sequences write partials to the range's slots 0 and 1 (slot 0 when one sequence covers
// the whole range).
template <int PK>
__global__ __launch_bounds__(kThreads, 1) void latent_decode_kernel(DecodeArgs a, int num_splits, int chunk,
                                                                   int rblocks, int n_units, int n_xcd) {
  __shared__ SmemL sm;

  const int per_xcd = int(gridDim.x) / n_xcd;
  const int unit = (int(blockIdx.x) % n_xcd) * per_xcd + int(blockIdx.x) / n_xcd;
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
    decode_piece<PK>(sm, a, b, rb, t_lo, min(L, t_lo + chunk), L, fin,
                     fin ? int64_t(b) * rows : (int64_t(b) * num_splits + split) * rows);
    return;
  }

  // Tile prefix of the batch: computed here by every wave for batches of up to 64 sequences
  // (one lane per sequence, 32-bit sums, a ballot finds the first sequence; unit 0 also
  // stores it for the combine), else read from the prefix kernel's output.
  const bool wave_pfx = a.prefix_here;
  int incl = 0;
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
  }
  auto pre = [&](int i) -> int64_t {
    if (wave_pfx) return i == 0 ? int64_t(0) : int64_t(__builtin_amdgcn_readlane(incl, i - 1));
    const int64_t v = a.prefix[i];
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
    return int64_t((uint64_t(hi) << 32) | lo);
  };

  const int w = unit / rblocks, n_ranges = n_units / rblocks;
  const int64_t total = pre(a.B);
  int64_t cur = total * w / n_ranges;
  const int64_t end = total * (w + 1) / n_ranges;
  if (cur >= end) return;
  int b = 0;
  if (wave_pfx) {
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
    decode_piece<PK>(sm, a, b, rb, int(cur - p0) * kTile, min(L, int(e - p0) * kTile), L, fin, base);
    cur = e;
    for (++b; b < a.B && pre(b + 1) <= cur;) ++b;  // skip sequences without tiles
  }
}

template <int PK>
int launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const int rblocks = (p.rows + kRowsWG - 1) / kRowsWG;
  const int n_units = p.balanced ? p.num_splits * rblocks : a.B * p.num_splits * rblocks;
  const int n_xcd = p.n_xcd > 0 ? p.n_xcd : 1;
  const int grid = (n_units + n_xcd - 1) / n_xcd * n_xcd;
  hipLaunchKernelGGL((latent_decode_kernel<PK>), dim3(grid), dim3(kThreads), 0, s, a, p.num_splits,
                     p.split_tokens, rblocks, n_units, n_xcd);
  return int(hipGetLastError());
}

}  // namespace

int launch_decode_latent(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  if (a.kv_dt != MLA_BF16 || a.fp8_scores) return int(hipErrorInvalidValue);
  if (!a.paged) return launch_t<kContig>(a, p, s);
  return a.block_size % kTile == 0 ? launch_t<kPagedTile>(a, p, s) : launch_t<kPagedAny>(a, p, s);
}

}  // namespace mla
