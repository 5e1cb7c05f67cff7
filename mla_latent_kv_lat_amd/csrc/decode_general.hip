// General latent-attention decode kernel (VALU) and the split-K combine kernel.
//
// The general kernel serves every shape the matrix-core kernel does not (fp32 caches,
// latent or RoPE widths other than 512 / 64, query-row counts that are not a multiple of
// 64).  One workgroup owns 4 query rows of one sequence and one split of its context.
// Scores follow the absorbed form: the head's query, already multiplied by W_UK, is
// dotted directly with the cached latent, plus the RoPE term ("multi-head latent
// attention" glossary entry, paragraph on the decoupled RoPE key).  Softmax is the
// streaming (online) form in base-2 units; the latent itself is the value.
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRB = 4;          // query rows per workgroup (one wave reduces each row)
constexpr int kTT = 256;        // tokens per step (one per thread in the score phase)
constexpr int kThreads = 256;
constexpr int kMaxCols = 8;     // output columns per thread: d_c <= 2048

template <typename QS, typename KVS, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_general_kernel(DecodeArgs a, int num_splits,
                                                                   int chunk) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, rblk = blockIdx.y, b = blockIdx.z;
  const int rows = a.sq * a.H;
  const int r0 = rblk * kRB;
  const int D = a.dc + a.dr;
  // Lengths are clamped to [0, T] like every other kernel of the call (the combine merges
  // only the splits below the clamped length).
  const int L = min(max(a.seq_lens ? a.seq_lens[b] : int(a.T), 0), int(a.T));
  const int t_lo = split * chunk;
  const int t_hi = min(L, t_lo + chunk);
  // The combine reads only splits that start below the sequence length.
  if (num_splits > 1 && t_lo >= L) return;

  float* q_s = smem;               // [kRB][D], multiplied by softmax_scale * log2(e)
  float* p_s = q_s + kRB * D;      // [kRB][kTT] scores, then probabilities
  float* red_s = p_s + kRB * kTT;  // [3][kRB]: rescale factor, running max, step sum

  using QR = typename QS::raw;
  using KR = typename KVS::raw;
  const QR* q_lat = static_cast<const QR*>(a.q_lat);
  const QR* q_rope = static_cast<const QR*>(a.q_rope);
  for (int idx = tid; idx < kRB * D; idx += kThreads) {
    const int r = idx / D, d = idx - r * D, row = r0 + r;
    float v = 0.f;
    if (row < rows) {
      const int64_t qrow = int64_t(b) * rows + row;
      v = d < a.dc ? load_as_f32<QS>(q_lat, qrow * a.dc + d)
                   : load_as_f32<QS>(q_rope, qrow * a.dr + (d - a.dc));
    }
    q_s[idx] = v * a.scale_log2;
  }
  int vis[kRB];  // query i of the sequence sees tokens t < L - s_q + i + 1
#pragma unroll
  for (int r = 0; r < kRB; ++r) {
    const int row = r0 + r;
    const int i = row / a.H;
    vis[r] = row < rows ? min(max(L - a.sq + i + 1, 0), L) : 0;
  }
  float m[kRB], l[kRB], acc[kRB][kMaxCols];
#pragma unroll
  for (int r = 0; r < kRB; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxCols; ++j) acc[r][j] = 0.f;
  }
  const KR* kv = static_cast<const KR*>(a.c_kv);
  const QR* kr = static_cast<const QR*>(a.k_rope);
  constexpr bool kFp8 = sizeof(KR) == 1;
  __syncthreads();

  for (int t0 = t_lo; t0 < t_hi; t0 += kTT) {
    // Scores: thread tid owns token t0 + tid.
    float sc[kRB];
#pragma unroll
    for (int r = 0; r < kRB; ++r) sc[r] = -INFINITY;
    const int t = t0 + tid;
    if (t < t_hi) {
      const int64_t crow = cache_row(PAGED, b, t, a.T, a.block_table, a.max_blocks, a.block_size);
      float dl[kRB] = {}, dp[kRB] = {};
      for (int d = 0; d < a.dc; ++d) {
        const float x = load_as_f32<KVS>(kv, crow * a.dc + d);
#pragma unroll
        for (int r = 0; r < kRB; ++r) dl[r] += q_s[r * D + d] * x;
      }
      for (int d = 0; d < a.dr; ++d) {
        const float x = load_as_f32<QS>(kr, crow * a.dr + d);
#pragma unroll
        for (int r = 0; r < kRB; ++r) dp[r] += q_s[r * D + a.dc + d] * x;
      }
      const float ts = kFp8 ? a.kv_scale[crow] : 1.f;
#pragma unroll
      for (int r = 0; r < kRB; ++r)
        if (t < vis[r]) sc[r] = dl[r] * ts + dp[r];
    }
#pragma unroll
    for (int r = 0; r < kRB; ++r) p_s[r * kTT + tid] = sc[r];
    __syncthreads();
    {
      // Wave w updates the statistics of row w over this step's tokens.
      const int r = wave;
      float v[kTT / 64];
      float cmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < kTT / 64; ++j) {
        v[j] = p_s[r * kTT + lane + 64 * j];
        cmax = fmaxf(cmax, v[j]);
      }
      cmax = wave_max(cmax);
      float m_old = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < kRB; ++rr)
        if (rr == r) m_old = m[rr];
      const float m_new = fmaxf(m_old, cmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float csum = 0.f;
#pragma unroll
      for (int j = 0; j < kTT / 64; ++j) {
        const float p = exp2f(v[j] - m_use);
        p_s[r * kTT + lane + 64 * j] = p;
        csum += p;
      }
      csum = wave_sum(csum);
      if (lane == 0) {
        red_s[r] = exp2f(m_old - m_use);
        red_s[kRB + r] = m_new;
        red_s[2 * kRB + r] = csum;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
      const float alpha = red_s[r];
      m[r] = red_s[kRB + r];
      l[r] = l[r] * alpha + red_s[2 * kRB + r];
#pragma unroll
      for (int j = 0; j < kMaxCols; ++j) acc[r][j] *= alpha;
    }
    // Weighted sum of latent rows: thread tid owns columns tid, tid + 256, ...
    const int nt = min(kTT, t_hi - t0);
    for (int tt = 0; tt < nt; ++tt) {
      const int64_t crow =
          cache_row(PAGED, b, t0 + tt, a.T, a.block_table, a.max_blocks, a.block_size);
      const float ts = kFp8 ? a.kv_scale[crow] : 1.f;
      float pr[kRB];
#pragma unroll
      for (int r = 0; r < kRB; ++r) pr[r] = p_s[r * kTT + tt] * ts;
#pragma unroll
      for (int j = 0; j < kMaxCols; ++j) {
        const int c = tid + j * kThreads;
        if (c < a.dc) {
          const float x = load_as_f32<KVS>(kv, crow * a.dc + c);
#pragma unroll
          for (int r = 0; r < kRB; ++r) acc[r][j] += pr[r] * x;
        }
      }
    }
    __syncthreads();
  }

  using OR = typename QS::raw;
#pragma unroll
  for (int r = 0; r < kRB; ++r) {
    const int row = r0 + r;
    if (row >= rows) continue;
    const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
    const float lse2 = l[r] > 0.f ? m[r] + log2f(l[r]) : -INFINITY;
    if (num_splits == 1) {
      OR* o = static_cast<OR*>(a.o_lat) + (int64_t(b) * rows + row) * a.dc;
#pragma unroll
      for (int j = 0; j < kMaxCols; ++j) {
        const int c = tid + j * kThreads;
        if (c < a.dc) store_from_f32<QS>(o, c, acc[r][j] * inv);
      }
      if (a.lse && tid == 0) a.lse[int64_t(b) * rows + row] = lse2 * kLn2;
    } else {
      const int64_t prow = (int64_t(b) * num_splits + split) * rows + row;
      float* o = static_cast<float*>(a.part_o) + prow * a.dc;
#pragma unroll
      for (int j = 0; j < kMaxCols; ++j) {
        const int c = tid + j * kThreads;
        if (c < a.dc) o[c] = acc[r][j] * inv;
      }
      if (tid == 0) a.part_lse[prow] = lse2;
    }
  }
}

// Merge the splits of one (sequence, query row): weights 2^(lse_s - max) over the splits
// that start below the sequence length; output = weighted mean of the normalised partial
// outputs; lse = max + log2(sum of weights), returned in natural-log units.  One wave per
// row, 8 consecutive columns per lane; the splits are read in batches whose loads are all
// in flight together, merged with a running maximum so no separate max pass is needed.
constexpr int kCombRows = 4;   // query rows (one per wave) per workgroup
constexpr int kCombBatch = 8;  // splits per batch (4 when a row has at most 4 pieces)
constexpr int kCombWaves = 4;  // waves sharing one row in the merge of balanced ranges

template <bool VEC>
__device__ __forceinline__ void load8_f32(float (&v)[8], const float* p, int c, int dc) {
  if (VEC) {  // dc % 8 == 0: the 8 columns are all in range or all out
    const bool ok = c < dc;
    const float4 x0 = ok ? *reinterpret_cast<const float4*>(p) : float4{0.f, 0.f, 0.f, 0.f};
    const float4 x1 = ok ? *reinterpret_cast<const float4*>(p + 4) : float4{0.f, 0.f, 0.f, 0.f};
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = c + k < dc ? p[k] : 0.f;
  }
}

// The same for bf16 partials (only written when dc % 8 == 0).
__device__ __forceinline__ void load8_f32(float (&v)[8], const uint16_t* p, int c, int dc) {
  const uint4 x = c < dc ? *reinterpret_cast<const uint4*>(p) : uint4{0u, 0u, 0u, 0u};
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf16_bits_to_f32(w[k] & 0xFFFFu);
    v[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
  }
}

// Weighted merge of np pieces of one row: piece j has base-2 log-sum-exp lse_of(j) (-inf:
// no weight) and its dc normalised values at part_of(j).  Writes the row of o and, if
// lse_out is set, its natural-log lse.
template <typename OS, typename PS, bool VEC, int NB = kCombBatch, typename LseF, typename PartF>
__device__ __forceinline__ void merge_row(const DecodeArgs& a, int np, LseF lse_of, PartF part_of,
                                          typename OS::raw* o, float* lse_out, int lane) {
  using PR = typename PS::raw;
  for (int c0 = 0; c0 < a.dc; c0 += 512) {
    const int c = c0 + 8 * lane;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float M = -INFINITY, tot = 0.f;
    for (int s0 = 0; s0 < np; s0 += NB) {
      float ls[NB], v[NB][8];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int sj = min(s0 + j, np - 1);  // in range; surplus entries get weight 0
        const float lj = lse_of(sj);
        ls[j] = s0 + j < np ? lj : -INFINITY;
        const PR* pj = part_of(sj) + c;
        if constexpr (sizeof(PR) == 2)
          load8_f32(v[j], pj, c, a.dc);
        else
          load8_f32<VEC>(v[j], pj, c, a.dc);
      }
      float bm = ls[0];
#pragma unroll
      for (int j = 1; j < NB; ++j) bm = fmaxf(bm, ls[j]);
      const float Mn = fmaxf(M, bm);
      if (Mn == -INFINITY) continue;  // nothing visible yet (uniform over the wave)
      const float r = exp2f(M - Mn);  // 0 while M is still -inf
      tot *= r;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= r;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float w = exp2f(ls[j] - Mn);
        tot += w;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = fmaf(w, v[j][k], acc[k]);
      }
      M = Mn;
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if constexpr (VEC && sizeof(typename OS::raw) == 2) {
      if (c < a.dc) {
        uint32_t pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pk[k] = uint32_t(f32_to_bf16_bits(acc[2 * k] * inv)) |
                  (uint32_t(f32_to_bf16_bits(acc[2 * k + 1] * inv)) << 16);
        *reinterpret_cast<uint4*>(o + c) = uint4{pk[0], pk[1], pk[2], pk[3]};
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (c + k < a.dc) store_from_f32<OS>(o, c + k, acc[k] * inv);
    }
    if (c0 == 0 && lane == 0 && lse_out) *lse_out = tot > 0.f ? (M + log2f(tot)) * kLn2 : -INFINITY;
  }
}

// Static splits: split s of sequence b covers tokens [s chunk, (s + 1) chunk); splits that
// start at or past the sequence length were not run.
template <typename OS, typename PS, bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, int S, int chunk) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = a.sq * a.H;
  const int row = blockIdx.x * kCombRows + wave, b = blockIdx.y;
  if (row >= rows) return;
  const int L = min(max(a.seq_lens ? a.seq_lens[b] : int(a.T), 0), int(a.T));
  const int nvalid = min(S, (L + chunk - 1) / chunk);
  const float* pl = a.part_lse + int64_t(b) * S * rows + row;
  const int64_t sstride = int64_t(rows) * a.dc;
  using PR = typename PS::raw;
  const PR* po = static_cast<const PR*>(a.part_o) + (int64_t(b) * S * rows + row) * a.dc;
  using OR = typename OS::raw;
  OR* o = static_cast<OR*>(a.o_lat) + (int64_t(b) * rows + row) * a.dc;
  merge_row<OS, PS, VEC>(
      a, nvalid, [&](int j) { return pl[int64_t(j) * rows]; }, [&](int j) { return po + j * sstride; }, o,
      a.lse ? a.lse + int64_t(b) * rows + row : nullptr, lane);
}

// Balanced ranges (bf16 output and partials): range w holds tiles
// [floor(total w / R), floor(total (w + 1) / R)) of the batch's concatenated tiles.  A
// sequence inside one range was written by the decode kernel; a sequence cut by range
// boundaries is merged from the partial of its first range (slot 1 when that range began
// in an earlier sequence, else slot 0) and slot 0 of each later range it reaches.  A
// sequence without tiles gets zeros and lse = -inf.
// Running merge, for the 8 columns c .. c + 7 of this lane, of the pieces first, first + step,
// ... below np of one row: base-2 max M of their log-sum-exps, the sum tot of their weights
// 2^(lse - M) and the weighted sum acc of their values.
template <int NB, typename LseF, typename PartF>
__device__ __forceinline__ void merge_state(int np, int first, int step, LseF lse_of, PartF part_of, int c, int dc,
                                            float& M, float& tot, float (&acc)[8]) {
  M = -INFINITY;
  tot = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int s0 = first; s0 < np; s0 += NB * step) {
    float ls[NB], v[NB][8];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int sj = min(s0 + j * step, np - 1);  // in range; surplus entries get weight 0
      const float lj = lse_of(sj);
      ls[j] = s0 + j * step < np ? lj : -INFINITY;
      load8_f32(v[j], part_of(sj) + c, c, dc);
    }
    float bm = ls[0];
#pragma unroll
    for (int j = 1; j < NB; ++j) bm = fmaxf(bm, ls[j]);
    const float Mn = fmaxf(M, bm);
    if (Mn == -INFINITY) continue;  // nothing visible yet (uniform over the wave)
    const float r = exp2f(M - Mn);  // 0 while M is still -inf
    tot *= r;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= r;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float w = exp2f(ls[j] - Mn);
      tot += w;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(w, v[j][k], acc[k]);
    }
    M = Mn;
  }
}

// Workgroups of 4 waves over (row group, sequence).  WPR waves share one row: wave g of a
// row merges pieces g, g + WPR, g + 2 WPR, ..., then (WPR > 1) the row's first wave merges
// their states from LDS.  WPR = 4 keeps four chains of loads in flight per row for
// sequences cut into many pieces; WPR = 1 (a whole row per wave) suits few pieces.
template <int WPR>
__global__ __launch_bounds__(256) void combine_ranges_kernel(DecodeArgs a, int R) {
  static_assert(WPR == 1 || WPR == kCombWaves, "one row per wave, or per workgroup");
  __shared__ float sh_acc[WPR > 1 ? WPR : 1][8][64];
  __shared__ float sh_m[WPR], sh_t[WPR];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = a.sq * a.H;
  const int g = wave % WPR;  // chain of this wave within its row
  const int row = blockIdx.x * (kCombWaves / WPR) + wave / WPR, b = blockIdx.y;
  if (row >= rows) return;  // WPR = 1 only (WPR = 4: one row per workgroup, all valid)
  const int64_t total = a.prefix[a.B], p0 = a.prefix[b], p1 = a.prefix[b + 1];
  uint16_t* o = static_cast<uint16_t*>(a.o_lat) + (int64_t(b) * rows + row) * a.dc;
  float* lse_out = a.lse ? a.lse + int64_t(b) * rows + row : nullptr;
  if (p1 == p0) {
    if (g == 0) {
      for (int c = 8 * lane; c < a.dc; c += 512) *reinterpret_cast<uint4*>(o + c) = uint4{0u, 0u, 0u, 0u};
      if (lane == 0 && lse_out) *lse_out = -INFINITY;
    }
    return;
  }
  // Range arithmetic in 32 bits whenever every intermediate fits: total R and
  // (x + 1) R + total - 1 <= total (R + 1) (64-bit division is long).
  const bool small = total * (R + 1) < (int64_t(1) << 32);
  auto range_lo = [&](int64_t w) {
    return small ? int64_t(uint32_t(total) * uint32_t(w) / uint32_t(R)) : total * w / R;
  };
  auto range_of = [&](int64_t x) {  // holds tile x
    return small ? int((uint32_t(x + 1) * uint32_t(R) + uint32_t(total) - 1u) / uint32_t(total)) - 1
                 : int(((x + 1) * R + total - 1) / total - 1);
  };
  const int w0 = range_of(p0), w1 = range_of(p1 - 1);
  if (w0 == w1) return;
  const int64_t slot0 = int64_t(w0) * 2 + (range_lo(w0) == p0 ? 0 : 1);
  // Piece j > 0 is slot 0 of range w0 + j; ranges without tiles (only when the batch has
  // fewer tiles than ranges) get weight 0 and read piece 0's values.
  const bool dense = total >= R;  // then every range holds a tile
  auto has_piece = [&](int j) { return j == 0 || dense || range_lo(w0 + j) < range_lo(w0 + j + 1); };
  auto slot_of = [&](int j) { return j == 0 || !has_piece(j) ? slot0 : int64_t(w0 + j) * 2; };
  const uint16_t* po = static_cast<const uint16_t*>(a.part_o) + int64_t(row) * a.dc;
  auto lse_of = [&](int j) { return has_piece(j) ? a.part_lse[slot_of(j) * rows + row] : -INFINITY; };
  auto part_of = [&](int j) { return po + slot_of(j) * rows * a.dc; };
  const int np = w1 - w0 + 1;
  for (int c0 = 0; c0 < a.dc; c0 += 512) {
    const int c = c0 + 8 * lane;
    float M, tot, acc[8];
    if (np <= 4 * WPR)
      merge_state<4>(np, g, WPR, lse_of, part_of, c, a.dc, M, tot, acc);
    else
      merge_state<kCombBatch>(np, g, WPR, lse_of, part_of, c, a.dc, M, tot, acc);
    if constexpr (WPR > 1) {
      if (g > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) sh_acc[g][k][lane] = acc[k];
        if (lane == 0) {
          sh_m[g] = M;
          sh_t[g] = tot;
        }
      }
      __syncthreads();
    }
    if (g == 0) {
      float Mn = M;
#pragma unroll
      for (int q = 1; q < WPR; ++q) Mn = fmaxf(Mn, sh_m[q]);
      float t = 0.f, x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (Mn != -INFINITY) {
#pragma unroll
        for (int q = 0; q < WPR; ++q) {
          const float mq = q == 0 ? M : sh_m[q];
          const float wq = mq == -INFINITY ? 0.f : exp2f(mq - Mn);
          t = fmaf(wq, q == 0 ? tot : sh_t[q], t);
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = fmaf(wq, q == 0 ? acc[k] : sh_acc[q][k][lane], x[k]);
        }
      }
      const float inv = t > 0.f ? 1.f / t : 0.f;
      if (c < a.dc) {
        uint32_t pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pk[k] = uint32_t(f32_to_bf16_bits(x[2 * k] * inv)) | (uint32_t(f32_to_bf16_bits(x[2 * k + 1] * inv)) << 16);
        *reinterpret_cast<uint4*>(o + c) = uint4{pk[0], pk[1], pk[2], pk[3]};
      }
      if (c0 == 0 && lane == 0 && lse_out) *lse_out = t > 0.f ? (Mn + log2f(t)) * kLn2 : -INFINITY;
    }
    if constexpr (WPR > 1) __syncthreads();  // the states are reused by the next 512 columns
  }
}

// Exclusive prefix sum over the batch of each sequence's 32-token tile count (lengths
// clamped to [0, T]); prefix[B] is the total.  One workgroup of 1024 threads, each summing
// a contiguous run of sequences, then a scan over the threads in LDS.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* seq_lens, int B, int64_t T,
                                                           int64_t* prefix) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  auto tiles = [&](int b) {
    const int64_t L = min(max(int64_t(seq_lens ? seq_lens[b] : T), int64_t(0)), T);
    return (L + 31) / 32;
  };
  const int per = (B + 1023) / 1024;
  const int lo = min(B, tid * per), hi = min(B, lo + per);
  int64_t sum = 0;
  for (int b = lo; b < hi; ++b) sum += tiles(b);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = tid > 0 ? part[tid - 1] : 0;
  for (int b = lo; b < hi; ++b) {
    prefix[b] = run;
    run += tiles(b);
  }
  if (tid == 1023) prefix[B] = part[1023];
}

template <typename QS, typename KVS, bool PAGED>
int launch_general_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const dim3 grid(p.num_splits, (p.rows + kRB - 1) / kRB, a.B);
  const size_t lds = sizeof(float) * (kRB * (a.dc + a.dr) + kRB * kTT + 3 * kRB);
  hipLaunchKernelGGL((decode_general_kernel<QS, KVS, PAGED>), grid, dim3(kThreads), lds, s, a,
                     p.num_splits, p.split_tokens);
  return int(hipGetLastError());
}

template <typename QS, typename KVS>
int launch_general_p(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  return a.paged ? launch_general_t<QS, KVS, true>(a, p, s) : launch_general_t<QS, KVS, false>(a, p, s);
}

}  // namespace

int launch_decode_general(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  if (a.q_dt == MLA_F32) return launch_general_p<F32, F32>(a, p, s);
  if (a.kv_dt == MLA_FP8_E4M3) return launch_general_p<BF16, FP8>(a, p, s);
  return launch_general_p<BF16, BF16>(a, p, s);
}

int launch_tile_prefix(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, a.seq_lens, a.B, a.T,
                     const_cast<int64_t*>(a.prefix));
  return int(hipGetLastError());
}

int launch_combine(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const dim3 grid((p.rows + kCombRows - 1) / kCombRows, a.B);
  const bool vec = a.dc % 8 == 0;
  if (p.balanced) {
    if (!a.part_bf16 || a.q_dt != MLA_BF16 || !vec) return int(hipErrorInvalidValue);
    // Four waves per row when the ranges cut the average sequence into 8 or more pieces.
    if (p.num_splits >= 8 * a.B)
      hipLaunchKernelGGL(combine_ranges_kernel<kCombWaves>, dim3(p.rows, a.B), dim3(64 * kCombWaves), 0, s, a,
                         p.num_splits);
    else
      hipLaunchKernelGGL(combine_ranges_kernel<1>, grid, dim3(64 * kCombWaves), 0, s, a, p.num_splits);
    return int(hipGetLastError());
  }
  if (a.part_bf16) {
    // Written only by the matrix-core kernel: bf16 output, dc a multiple of 8.
    if (a.q_dt != MLA_BF16 || !vec) return int(hipErrorInvalidValue);
    hipLaunchKernelGGL((combine_kernel<BF16, BF16, true>), grid, dim3(256), 0, s, a, p.num_splits, p.split_tokens);
  } else if (a.q_dt == MLA_F32) {
    if (vec) hipLaunchKernelGGL((combine_kernel<F32, F32, true>), grid, dim3(256), 0, s, a, p.num_splits, p.split_tokens);
    else hipLaunchKernelGGL((combine_kernel<F32, F32, false>), grid, dim3(256), 0, s, a, p.num_splits, p.split_tokens);
  } else {
    if (vec) hipLaunchKernelGGL((combine_kernel<BF16, F32, true>), grid, dim3(256), 0, s, a, p.num_splits, p.split_tokens);
    else hipLaunchKernelGGL((combine_kernel<BF16, F32, false>), grid, dim3(256), 0, s, a, p.num_splits, p.split_tokens);
  }
  return int(hipGetLastError());
}

}  // namespace mla
