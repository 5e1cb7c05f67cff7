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
#include "mfma_common.h"
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
// One batch of pieces (base-2 log-sum-exps ls, values v) into a running merge (M, tot, acc).
template <int NB>
__device__ __forceinline__ void merge_batch(const float (&ls)[NB], const float (&v)[NB][8], float& M, float& tot,
                                            float (&acc)[8]) {
  float bm = ls[0];
#pragma unroll
  for (int j = 1; j < NB; ++j) bm = fmaxf(bm, ls[j]);
  const float Mn = fmaxf(M, bm);
  if (Mn == -INFINITY) return;  // nothing visible yet (uniform over the wave)
  const float r = exp2f(M - Mn);  // 0 while M is still -inf
  // Rounded multiply and add spelled out: the compiler may otherwise contract tot r + w into
  // one fma in some call sites and not in others, and every caller must give the same bits.
  tot = __fmul_rn(tot, r);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = __fmul_rn(acc[k], r);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float w = exp2f(ls[j] - Mn);
    tot = __fadd_rn(tot, w);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(w, v[j][k], acc[k]);
  }
  M = Mn;
}

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
    merge_batch<NB>(ls, v, M, tot, acc);
  }
}

// Where the pieces of sequence b lie under balanced ranges (R ranges over the batch's
// concatenated tiles): range w holds tiles [floor(total w / R), floor(total (w + 1) / R)).
// A sequence with tiles inside one range (whole) was written by the decode kernel; a cut one
// has its first piece in slot 0 or 1 of range w0 (slot 1 when that range began in an
// earlier sequence) and slot 0 of each later range up to w1.
struct RangePieces {
  int64_t total, p0, p1, slot0;
  int R, w0, w1;
  bool small, dense;
  __device__ bool empty() const { return p1 == p0; }
  __device__ bool whole() const { return w0 == w1; }
  __device__ int np() const { return w1 - w0 + 1; }
  // Range arithmetic in 32 bits whenever every intermediate fits: total R and
  // (x + 1) R + total - 1 <= total (R + 1) (64-bit division is long).
  __device__ int64_t range_lo(int64_t w) const {
    return small ? int64_t(uint32_t(total) * uint32_t(w) / uint32_t(R)) : total * w / R;
  }
  __device__ int range_of(int64_t x) const {  // holds tile x
    return small ? int((uint32_t(x + 1) * uint32_t(R) + uint32_t(total) - 1u) / uint32_t(total)) - 1
                 : int(((x + 1) * R + total - 1) / total - 1);
  }
  // Piece j > 0 is slot 0 of range w0 + j; ranges without tiles (only when the batch has
  // fewer tiles than ranges) get weight 0 and read piece 0's values.
  __device__ bool has_piece(int j) const { return j == 0 || dense || range_lo(w0 + j) < range_lo(w0 + j + 1); }
  __device__ int64_t slot_of(int j) const { return j == 0 || !has_piece(j) ? slot0 : int64_t(w0 + j) * 2; }
};

__device__ __forceinline__ RangePieces range_pieces(int64_t total, int64_t p0, int64_t p1, int R) {
  RangePieces P;
  P.total = total;
  P.p0 = p0;
  P.p1 = p1;
  P.R = R;
  P.small = P.total * (R + 1) < (int64_t(1) << 32);
  P.dense = P.total >= R;
  P.w0 = P.w1 = 0;
  P.slot0 = 0;
  if (P.p1 > P.p0) {
    P.w0 = P.range_of(P.p0);
    P.w1 = P.range_of(P.p1 - 1);
    P.slot0 = int64_t(P.w0) * 2 + (P.range_lo(P.w0) == P.p0 ? 0 : 1);
  }
  return P;
}

// The same lookup in 32-bit arithmetic only (the caller guarantees total (R + 1) < 2^32):
// the fused merge below keeps its per-row bookkeeping in scalar registers and its code small.
struct Pieces32 {
  uint32_t total, p0, p1, R, slot0;
  int w0, w1;
  bool dense;
  __device__ uint32_t range_lo(uint32_t w) const { return total * w / R; }
  __device__ int range_of(uint32_t x) const { return int(((x + 1u) * R + total - 1u) / total) - 1; }
  __device__ bool empty() const { return p1 == p0; }
  __device__ bool whole() const { return w0 == w1; }
  __device__ int np() const { return w1 - w0 + 1; }
  __device__ bool has_piece(int j) const {
    return j == 0 || dense || range_lo(uint32_t(w0 + j)) < range_lo(uint32_t(w0 + j + 1));
  }
  __device__ uint32_t slot_of(int j) const { return j == 0 || !has_piece(j) ? slot0 : uint32_t(w0 + j) * 2u; }
};

__device__ __forceinline__ Pieces32 pieces32(uint32_t total, uint32_t p0, uint32_t p1, uint32_t R) {
  Pieces32 P;
  P.total = total;
  P.p0 = p0;
  P.p1 = p1;
  P.R = R;
  P.dense = total >= R;
  P.w0 = P.w1 = 0;
  P.slot0 = 0;
  if (p1 > p0) {
    P.w0 = P.range_of(p0);
    P.w1 = P.range_of(p1 - 1u);
    P.slot0 = uint32_t(P.w0) * 2u + (P.range_lo(uint32_t(P.w0)) == p0 ? 0u : 1u);
  }
  return P;
}

// A single merge state (M, tot, acc) as the row's 8 bf16 columns of this lane and its
// natural-log log-sum-exp.
__device__ __forceinline__ void finish_row(float M, float tot, const float (&acc)[8], uint32_t (&pk)[4],
                                           float& lse_nat) {
  const float Mn = M;
  float t = 0.f, x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (Mn != -INFINITY) {
    const float wq = exp2f(M - Mn);
    t = fmaf(wq, tot, t);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = fmaf(wq, acc[k], x[k]);
  }
  const float inv = t > 0.f ? 1.f / t : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    pk[k] = uint32_t(f32_to_bf16_bits(x[2 * k] * inv)) | (uint32_t(f32_to_bf16_bits(x[2 * k + 1] * inv)) << 16);
  lse_nat = t > 0.f ? (Mn + log2f(t)) * kLn2 : -INFINITY;
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
  const RangePieces P = range_pieces(a.prefix[a.B], a.prefix[b], a.prefix[b + 1], R);
  uint16_t* o = static_cast<uint16_t*>(a.o_lat) + (int64_t(b) * rows + row) * a.dc;
  float* lse_out = a.lse ? a.lse + int64_t(b) * rows + row : nullptr;
  if (P.empty()) {
    if (g == 0) {
      for (int c = 8 * lane; c < a.dc; c += 512) *reinterpret_cast<uint4*>(o + c) = uint4{0u, 0u, 0u, 0u};
      if (lane == 0 && lse_out) *lse_out = -INFINITY;
    }
    return;
  }
  if (P.whole()) return;
  const uint16_t* po = static_cast<const uint16_t*>(a.part_o) + int64_t(row) * a.dc;
  auto lse_of = [&](int j) { return P.has_piece(j) ? a.part_lse[P.slot_of(j) * rows + row] : -INFINITY; };
  auto part_of = [&](int j) { return po + P.slot_of(j) * rows * a.dc; };
  const int np = P.np();
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

// The merge of the balanced ranges' pieces (as combine_ranges_kernel<1> does it) feeding the
// output absorption out[m, h, :] = o_lat[m, h, :] . W_UV[h] (as absorb_mfma_kernel<512, MG>
// does it, d_c = 512), in one kernel: each merged row goes from registers into the
// product's LDS operand tile instead of through HBM.  Grid (H, d_h / 64, ceil(M / MG)),
// M = B s_q; workgroups of the first column tile also store the merged o_lat rows and lse.
// Each wave merges rows m0 + wave + 4 q.  Loads go out in three groups so that no wait is
// held up by a later need (the memory counter completes in order): the rows' places in the
// batch, then the first batch of pieces of all the wave's rows, then the weight slice,
// which stays in flight during the merge.
// The arithmetic of both halves is that of the two separate kernels, so o_lat, lse and out
// equal those of the decode call followed by the output absorption, bit for bit.
// Direct-to-LDS load of 16 bytes per lane from per-lane addresses: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16).  The LDS address goes through M0; the block carries the
// wait states the hardware needs after an SGPR written from a vector register (the
// read-first-lane) and after the M0 write.  Completion is awaited with s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* addr, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(m0) : "memory");
}

// Merge of one row cut into more than 4 pieces (the separate merge's arithmetic for such a
// row), kept out of line: rare, and its loop is long.
__device__ __forceinline__ void merge_many(const DecodeArgs& a, const Pieces32& P, int r, int lane, float& M, float& tot,
                                        float (&acc)[8]) {
  const int rows = a.sq * a.H;
  const uint16_t* po = static_cast<const uint16_t*>(a.part_o) + int64_t(r) * a.dc;
  auto lse_of = [&](int j) { return P.has_piece(j) ? a.part_lse[int64_t(P.slot_of(j)) * rows + r] : -INFINITY; };
  auto part_of = [&](int j) { return po + int64_t(P.slot_of(j)) * rows * a.dc; };
  merge_state<kCombBatch>(P.np(), 0, 1, lse_of, part_of, 8 * lane, a.dc, M, tot, acc);
}

template <int MG, int NH, int NW>
__global__ __launch_bounds__(64 * NW) void merge_absorb_kernel(DecodeArgs a, int R, const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ y, int N, int n_xcd) {
  // MG rows and NH halves of 64 output columns per workgroup (kBN = 64 NH), each half staged
  // as its own [K][64] weight tile; NW waves, each merging MG / NW rows and then computing
  // its 16-column blocks of the product.
  constexpr int K = 512, kBN = 64 * NH, kBlocks = MG / 16, RW = MG / NW;
  constexpr int kHalvesPerWave = NH * 4 / NW;  // NW = 4 NH: one half per wave; NW = 4: all halves
  static_assert(MG % NW == 0 && (NW == 4 || NW == 4 * NH), "workgroup shape");
  __shared__ __attribute__((aligned(16))) uint16_t wt[NH][K * 64];  // [k][64], chunks swizzled by swz128(k)
  __shared__ __attribute__((aligned(16))) uint16_t xs[MG * K];      // [row][k], chunk c at c ^ (row & 15)
  const int H = a.H, M = a.B * a.sq, rows = a.sq * a.H;
  int h = blockIdx.x, n0 = blockIdx.y * kBN, m0 = blockIdx.z * MG;
  if (n_xcd > 1 && int(gridDim.x) % n_xcd == 0) {  // per-XCD order, as in the absorption kernel
    const int ncol = int(gridDim.y), nrg = int(gridDim.z);
    const int id = int(blockIdx.x) + int(gridDim.x) * (int(blockIdx.y) + ncol * int(blockIdx.z));
    const int j = id / n_xcd;
    h = (j / (ncol * nrg)) * n_xcd + id % n_xcd;
    n0 = ((j / nrg) % ncol) * kBN;
    m0 = (j % nrg) * MG;
  }
  // The wave index as a wave-uniform (scalar) value, so that each row's bookkeeping (its
  // sequence, the range arithmetic, its kind) is scalar code and its loads scalar loads.
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool store_o = n0 == 0;  // one column tile per row stores the merged o_lat and lse

  // Merge: row kind 0 = past M, 1 = no tiles, 2 = whole (o_lat as written), 3 = cut into at
  // most 4 pieces (loaded here), 4 = more pieces (merged below, one row at a time).
  int kind[RW], np[RW], ob[RW], orow[RW];
  uint32_t pf0[RW], pf1[RW];
  const uint32_t total = uint32_t(a.prefix[a.B]);
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    const int m = m0 + wv + NW * q;
    const int b = m < M ? m / a.sq : 0;
    ob[q] = b;
    orow[q] = (m - b * a.sq) * H + h;
    pf0[q] = uint32_t(a.prefix[b]);
    pf1[q] = uint32_t(a.prefix[b + 1]);
  }
  Pieces32 P[RW];
  float ls[RW][4];
  u32x4 raw[RW][4];
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    const int m = m0 + wv + NW * q;
    const int b = ob[q], r = orow[q];
    P[q] = pieces32(total, pf0[q], pf1[q], uint32_t(R));
    kind[q] = m >= M ? 0 : P[q].empty() ? 1 : P[q].whole() ? 2 : P[q].np() <= 4 ? 3 : 4;
    np[q] = P[q].np();
    if (kind[q] == 2)
      raw[q][0] = ld16(static_cast<const uint16_t*>(a.o_lat) + (int64_t(b) * rows + r) * K + 8 * lane);
    if (kind[q] == 3) {
      const uint16_t* po = static_cast<const uint16_t*>(a.part_o) + int64_t(r) * K + 8 * lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sj = min(j, np[q] - 1);  // in range; surplus entries get weight 0
        const int64_t slot = P[q].slot_of(sj);
        const float lj = P[q].has_piece(sj) ? a.part_lse[slot * rows + r] : -INFINITY;
        ls[q][j] = j < np[q] ? lj : -INFINITY;
        raw[q][j] = ld16(po + slot * rows * K);
      }
    }
  }
  // Weight slice straight into LDS (64 loads of 1 KB = 8 rows of 64 columns; wave wv issues
  // 16): lane i of load d fills position i % 8 of row k = 8 d + i / 8, i.e. the row's chunk
  // (i % 8) ^ swz128(k).  Issued after the merge's loads, so that waiting for those does not
  // wait for these.
  // NH x 64 loads of 1 KB, dealt to the NW waves in turn.
#pragma unroll
  for (int i = 0; i < NH * (K / 8) / NW; ++i) {
    const int e = wv + NW * i, hh = e / (K / 8), d = e % (K / 8);
    const int k = 8 * d + (lane >> 3), ch = (lane & 7) ^ swz128(k);
    dma16(w + int64_t(h) * K * N + n0 + 64 * hh + int64_t(k) * N + 8 * ch,
          uint32_t(reinterpret_cast<uintptr_t>(&wt[hh][0])) + uint32_t(1024 * d));
  }
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    const int xr = wv + NW * q;  // row of the operand tile
    uint32_t pk[4] = {0u, 0u, 0u, 0u};
    float lse_nat = -INFINITY;
    if (kind[q] == 2) {
      pk[0] = raw[q][0][0];
      pk[1] = raw[q][0][1];
      pk[2] = raw[q][0][2];
      pk[3] = raw[q][0][3];
    } else if (kind[q] >= 3) {
      float M_ = -INFINITY, tot = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (kind[q] == 3) {
        float v[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[j][2 * k] = bf16_bits_to_f32(raw[q][j][k] & 0xFFFFu);
            v[j][2 * k + 1] = bf16_bits_to_f32(raw[q][j][k] >> 16);
          }
        merge_batch<4>(ls[q], v, M_, tot, acc);
      } else {
        merge_many(a, P[q], orow[q], lane, M_, tot, acc);
      }
      finish_row(M_, tot, acc, pk, lse_nat);
    }
    if (store_o && (kind[q] == 1 || kind[q] >= 3)) {
      uint16_t* o = static_cast<uint16_t*>(a.o_lat) + (int64_t(ob[q]) * rows + orow[q]) * K;
      *reinterpret_cast<uint4*>(o + 8 * lane) = uint4{pk[0], pk[1], pk[2], pk[3]};
      if (lane == 0 && a.lse) a.lse[int64_t(ob[q]) * rows + orow[q]] = lse_nat;
    }
    *reinterpret_cast<uint4*>(&xs[xr * K + 8 * (lane ^ (xr & 15))]) = uint4{pk[0], pk[1], pk[2], pk[3]};
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's weight loads have landed
  __syncthreads();

  // The product y^T[n, m] = W^T[n, :] . x^T[:, m] on v_mfma_f32_16x16x32_bf16, wave wv owning
  // columns 16 wv .. 16 wv + 15 of each half (the absorption kernel's layout and order).
  const int g = lane >> 4, mm = lane & 15;
  const int cb = wv & 3, h0 = kHalvesPerWave == NH ? 0 : wv >> 2;  // column block, first half
  f32x4 acc[kHalvesPerWave][kBlocks];
#pragma unroll
  for (int hh = 0; hh < kHalvesPerWave; ++hh)
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) acc[hh][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < K / 32; ++s2) {
#pragma unroll
    for (int hh = 0; hh < kHalvesPerWave; ++hh) {
      const bf16x8 av = lds_operand_tr(wt[h0 + hh], 32 * s2, 16 * cb, lane);
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) {
        const int r = 16 * i + mm;
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&xs[r * K + 8 * ((4 * s2 + g) ^ (r & 15))]);
        acc[hh][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[hh][i], 0, 0, 0);
      }
    }
  }
  // bf16 results through LDS (half hh of row r at ys[(NH r + hh) 64 ..], 16-byte chunk c of
  // that 128-byte piece at c ^ (r' >> 1) & 7 with r' = NH r + hh), so that each output row's
  // 64 NH columns leave in whole 128-byte pieces.
  __syncthreads();
  uint16_t* ys = xs;
#pragma unroll
  for (int hh = 0; hh < kHalvesPerWave; ++hh)
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int r = NH * (16 * i + mm) + h0 + hh, col = 16 * cb + 4 * g;
      *reinterpret_cast<u32x2*>(&ys[r * 64 + 8 * ((col >> 3) ^ ((r >> 1) & 7)) + (col & 7)]) =
          u32x2{pack_bf16x2(acc[hh][i][0], acc[hh][i][1]), pack_bf16x2(acc[hh][i][2], acc[hh][i][3])};
    }
  __syncthreads();
#pragma unroll
  for (int rp = tid >> 3; rp < MG * NH; rp += 8 * NW) {  // rp = NH r + hh: one 128-byte piece
    const int c = tid & 7, r = rp / NH, hh = rp % NH, m = m0 + r;
    if (m < M)
      *reinterpret_cast<u32x4*>(y + (int64_t(m) * H + h) * N + n0 + 64 * hh + 8 * c) =
          *reinterpret_cast<const u32x4*>(&ys[rp * 64 + 8 * (c ^ ((rp >> 1) & 7))]);
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

bool merge_absorb_fits(const DecodeArgs& a, const DecodePlan& p, int32_t d_h) {
  // Balanced ranges with the one-wave-per-row merge, bf16 rows of d_c = 512, d_h a multiple
  // of 64 (at most 65535 column tiles and row groups).
  // The batch's tiles times (ranges + 1) fit in 32 bits (the kernel's range arithmetic).
  const int64_t max_tiles = int64_t(a.B) * ((a.T + 31) / 32);
  return p.balanced && a.part_bf16 && a.q_dt == MLA_BF16 && a.dc == 512 && d_h % 64 == 0 && d_h / 64 <= 65535 &&
         p.num_splits < 8 * a.B && (int64_t(a.B) * a.sq + 15) / 16 <= 65535 &&
         max_tiles * (int64_t(p.num_splits) + 1) < (int64_t(1) << 32);
}

int launch_merge_absorb(const DecodeArgs& a, const DecodePlan& p, const void* w_uv, void* out, int32_t d_h,
                        hipStream_t s) {
  if (!merge_absorb_fits(a, p, d_h)) return int(hipErrorInvalidValue);
  const int M = a.B * a.sq;
  const int n_xcd = p.n_xcd > 0 ? p.n_xcd : 1;
  // 32 rows by 128 output columns per workgroup when d_h allows: each weight slice and each
  // row's pieces are then read once; else 16 rows by 64 columns.
  if (d_h % 128 == 0)
    hipLaunchKernelGGL((merge_absorb_kernel<32, 2, 8>), dim3(a.H, d_h / 128, (M + 31) / 32), dim3(512), 0, s, a,
                       p.num_splits, static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out), d_h, n_xcd);
  else
    hipLaunchKernelGGL((merge_absorb_kernel<16, 1, 4>), dim3(a.H, d_h / 64, (M + 15) / 16), dim3(256), 0, s, a,
                       p.num_splits, static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out), d_h, n_xcd);
  return int(hipGetLastError());
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
    // Four waves per row when the ranges cut the average sequence into 16 or more pieces (one
    // wave loads up to 8 pieces in one batch).
    if (p.num_splits >= 16 * a.B)
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
