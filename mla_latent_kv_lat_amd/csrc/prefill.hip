// Prefill in the explicit form: decompress the keys and values of every head from the
// latent, then run causal attention over them ("Operator Notes (1): MLA", section 2: K and
// V are restored from c_kv by the up-projections, then scaled dot-product attention with a
// softmax and a product with V; the RoPE key of the "multi-head latent attention" glossary
// entry, paragraph on the decoupled RoPE key, is appended to every head's key).  For long
// prompts this is cheaper than the absorbed form used by decode: per query, key and head it
// costs 2 (d_h + d_r) + 2 d_h flops instead of 2 (d_c + d_r) + 2 d_c, for a decompression
// of 2 d_c (2 d_h) flops per token and head.
//
// Three kernels:
//   * prefill_weights_kernel: wcat[h] = [W_UK[h] ; W_UV[h]^T] as 256 rows of d_c, so that
//     both halves of the decompression read their weights as rows;
//   * decompress_kernel: kv[m, h, 0:128] = c_kv[m] . W_UK[h]^T (the head's key),
//     kv[m, h, 128:256] = c_kv[m] . W_UV[h] (its value), a matrix product over all B * T
//     cache rows in tiles of 256 rows by one head;
//   * prefill_attn_kernel: 256 queries of one (sequence, head) per workgroup, 64-key tiles,
//     scores as S^T = K Q^T and outputs as O^T += V^T P^T on the 32 x 32 x 16 bf16 matrix
//     instruction, online softmax in base 2 per query lane.
#include "device_common.h"
#include "mfma_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kDH = 128;             // d_h
constexpr int kDC = 512;             // d_c
constexpr int kDR = 64;              // d_r
constexpr int kDQK = kDH + kDR;      // 192: key width of one head
constexpr int kNcat = 2 * kDH;       // 256: decompressed key then value of one head

// ---------------------------------------------------------------------------------------
// wcat[h][n][c] = W_UK[h][n][c] for n < 128, W_UV[h][c][n - 128] for n >= 128.
// Grid (H, 8): block y copies or transposes 32 rows of the head's 256.
__global__ __launch_bounds__(256) void prefill_weights_kernel(const uint16_t* __restrict__ w_uk,
                                                              const uint16_t* __restrict__ w_uv,
                                                              uint16_t* __restrict__ wcat) {
  __shared__ uint16_t t[kDC][34];  // [c][n], padded against bank conflicts
  const int h = blockIdx.x, n0 = blockIdx.y * 32, tid = threadIdx.x;
  uint16_t* dst = wcat + (int64_t(h) * kNcat + n0) * kDC;
  if (n0 < kDH) {
    const uint16_t* src = w_uk + (int64_t(h) * kDH + n0) * kDC;
    for (int i = tid; i < 32 * kDC / 8; i += 256)
      *reinterpret_cast<u32x4*>(dst + 8 * i) = *reinterpret_cast<const u32x4*>(src + 8 * i);
  } else {
    const uint16_t* src = w_uv + int64_t(h) * kDC * kDH + (n0 - kDH);
    for (int i = tid; i < kDC * 32; i += 256) t[i / 32][i % 32] = src[int64_t(i / 32) * kDH + i % 32];
    __syncthreads();
    for (int i = tid; i < 32 * kDC; i += 256) dst[i] = t[i % kDC][i / kDC];
  }
}

// ---------------------------------------------------------------------------------------
// kv[m, h, n] = sum_c x[m, c] * wcat[h][n][c] for a tile of 256 cache rows (m) and one
// head's 256 columns (n: key then value).  Eight waves, each a 64 (n) x 128 (m) block formed
// as D^T[n][m] (weights as the A operand, cache rows as the B operand: 6 operand reads per 8
// products), in K steps of 64 staged through LDS (double buffered, 64 KB per step).  LDS
// rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r sits at c ^ ((r >> 1) & 7),
// so the 16 rows of one operand read hit distinct banks.
constexpr int kGM = 256;   // cache rows per tile
constexpr int kGN = kNcat; // columns per tile: one head
constexpr int kGK = 64;    // K per stage
constexpr int kGThreads = 512;

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(kGThreads, 1) void decompress_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wcat,
                                                                  uint16_t* __restrict__ kv, int M, int H) {
  __shared__ __attribute__((aligned(16))) uint16_t sm[2][2][kGN * kGK];  // [buf][A = w, B = x]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m0 = blockIdx.x * kGM, h = blockIdx.y;
  const int wn = wv & 3, wm = wv >> 2;  // this wave's block: n 64 wn.., m 128 wm..
  const int n32 = lane & 31, hh = lane >> 5;

  // Global -> register loads of one stage: 256 rows x 8 chunks of each operand, 4 chunks per
  // thread per operand.
  const uint16_t* wrow = wcat + int64_t(h) * kNcat * kDC;
  u32x4 ra[4], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kGThreads * i, r = idx >> 3, ch = idx & 7;
      ra[i] = ld16(wrow + int64_t(r) * kDC + k0 + 8 * ch);
      rb[i] = ld16(x + int64_t(min(m0 + r, M - 1)) * kDC + k0 + 8 * ch);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kGThreads * i, r = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4*>(&sm[buf][0][r * kGK + 8 * (ch ^ gswz(r))]) = ra[i];
      *reinterpret_cast<u32x4*>(&sm[buf][1][r * kGK + 8 * (ch ^ gswz(r))]) = rb[i];
    }
  };

  f32x16 acc[2][4];  // [n block][m block]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  constexpr int kStages = kDC / kGK;
  for (int st = 0; st < kStages; ++st) {
    const int buf = st & 1;
    if (st + 1 < kStages) load((st + 1) * kGK);
    // Keep the next stage's loads here, ahead of this stage's products (the scheduler would
    // otherwise sink them next to the stores that consume them and expose their latency).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const int ch = 2 * ks + hh;
      bf16x8 av[2], bv[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rn = 64 * wn + 32 * j + n32;
        av[j] = *reinterpret_cast<const bf16x8*>(&sm[buf][0][rn * kGK + 8 * (ch ^ gswz(rn))]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rm = 128 * wm + 32 * j + n32;
        bv[j] = *reinterpret_cast<const bf16x8*>(&sm[buf][1][rm * kGK + 8 * (ch ^ gswz(rm))]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (st + 1 < kStages) {
      store(buf ^ 1);
      __syncthreads();
    }
  }
  __syncthreads();  // every wave done with the operand buffers
  // Stage the bf16 tile as [m][n] (reusing the operand buffers: 256 x 256 bf16 = 128 KB),
  // then store whole 512-byte rows.  Chunk c of row m sits at c ^ (m & 31).
  uint16_t* ot = &sm[0][0][0];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int m = 128 * wm + 32 * b + n32;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 64 * wn + 32 * a + 8 * i + 4 * hh;  // 4 consecutive n
        const uint32_t w0 = pack_bf16x2(acc[a][b][4 * i], acc[a][b][4 * i + 1]);
        const uint32_t w1 = pack_bf16x2(acc[a][b][4 * i + 2], acc[a][b][4 * i + 3]);
        *reinterpret_cast<u32x2*>(&ot[m * kGN + 8 * ((n >> 3) ^ (m & 31)) + (n & 7)]) = u32x2{w0, w1};
      }
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kGM * kGN / 8 / kGThreads; ++i) {
    const int idx = tid + kGThreads * i, m = idx >> 5, ch = idx & 31;
    if (m0 + m < M)
      *reinterpret_cast<u32x4*>(kv + (int64_t(m0 + m) * H + h) * kNcat + 8 * ch) =
          *reinterpret_cast<const u32x4*>(&ot[m * kGN + 8 * (ch ^ (m & 31))]);
  }
}

// ---------------------------------------------------------------------------------------
// Causal attention of the decompressed heads.  Query i of sequence b (length L) sits at
// position L - S + i and sees keys t <= L - S + i.
//
// A workgroup (8 waves, one per compute unit) owns 256 queries of one (sequence, head);
// wave w owns queries 32 w .. 32 w + 31.  Key tiles of 64 keys are staged in LDS (double
// buffered, one barrier per tile; the next tile's loads are in flight in registers while a
// tile is computed).  Per tile a wave forms S^T = K Q^T (keys as the A operand from LDS, its
// queries as the B operand held in registers), the online softmax in its lanes (lane n and
// n + 32 share query n), and O^T += V^T P^T (V read transposed from LDS).  The two key
// blocks of the score product alternate (independent accumulators) and every LDS operand is
// read a few products ahead of its use.  The query lane's reference max only moves when a
// tile exceeds it by more than kTau (base 2), so the accumulators are rarely rescaled;
// masking is applied only to tiles that reach past the wave's first query, and tiles
// entirely past its last query are skipped.  Workgroups are launched longest first (query
// blocks from the end of the prompt), which evens out the causal imbalance.
constexpr int kQB = 256;       // queries per workgroup
constexpr int kAttnThreads = 512;
constexpr int kKT = 64;        // keys per tile
// Staged rows are padded instead of swizzled, so every operand address is a per-lane base
// plus a constant.  Key rows: 192 bf16 + 8 (400 bytes: 16 consecutive rows read at one
// 16-byte chunk fall on distinct banks, as 400 / 16 = 25 is odd).  Value rows: 128 bf16 +
// 32 (320 bytes: the 4 rows of one transposed-read pass start 8 banks x 4 bytes apart... i.e.
// at distinct 32-byte bank groups).
constexpr int kKPitch = kDQK + 8;
constexpr int kVPitch = kDH + 32;
constexpr float kTau = 8.f;

struct alignas(16) AttnTile {
  uint16_t k[kKT * kKPitch];  // [key][200]: decompressed key, RoPE key, padding
  uint16_t v[kKT * kVPitch];  // [key][160]: value, padding (read transposed)
};

__device__ __forceinline__ void swap32_u32(uint32_t& a, uint32_t& b) {
  float fa = __builtin_bit_cast(float, a), fb = __builtin_bit_cast(float, b);
  permlane32_swap(fa, fb);
  a = __builtin_bit_cast(uint32_t, fa);
  b = __builtin_bit_cast(uint32_t, fb);
}

// Grid (H, query blocks, B): query block gridDim.y - 1 - blockIdx.y, so that the blocks with
// the most keys are dispatched first.
__global__ __launch_bounds__(kAttnThreads, 1) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ AttnTile sm[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int h = blockIdx.x, qblk = gridDim.y - 1 - blockIdx.y, b = blockIdx.z;
  const int S = a.S, H = a.H;
  const int L = min(max(a.seq_lens ? a.seq_lens[b] : a.T, 0), a.T);
  const int q0 = qblk * kQB;
  const int qi = q0 + 32 * wv + n;        // this lane's query
  const int pos = L - S + qi;             // its position; keys t <= pos are visible
  const int pos_first_w = L - S + q0 + 32 * wv;            // the wave's first query
  const int pos_last_w = L - S + min(q0 + 32 * wv + 32, S) - 1;
  // Keys the workgroup needs: up to the position of its last query.
  const int pos_last = L - S + min(q0 + kQB, S) - 1;
  const int nkeys = min(L, pos_last + 1);
  const int ntiles = nkeys > 0 ? (nkeys + kKT - 1) / kKT : 0;

  // Query operand (B of S^T = K Q^T): k-step s covers dims 16 s + 8 hh + (0..7) of
  // [q_nope | q_rope].
  bf16x8 qb[kDQK / 16];
  {
    const int64_t row = (int64_t(b) * S + min(qi, S - 1)) * H + h;
    const uint16_t* qn = static_cast<const uint16_t*>(a.q_nope) + row * kDH;
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope) + row * kDR;
#pragma unroll
    for (int s = 0; s < kDQK / 16; ++s)
      qb[s] = __builtin_bit_cast(bf16x8, s < kDH / 16 ? ld16(qn + 16 * s + 8 * hh) : ld16(qr + 16 * (s - kDH / 16) + 8 * hh));
  }

  // Tile loads: per key the 32 chunks of its kv row (16 of key, 16 of value) and the 8
  // chunks of its RoPE key; 4 + 1 chunks per thread.  Keys past the sequence load its last
  // row (always valid) and are masked.
  u32x4 pf[5];
  const uint16_t* kvh = static_cast<const uint16_t*>(a.kv) + int64_t(h) * kNcat;
  const uint16_t* kr = static_cast<const uint16_t*>(a.k_rope);
  auto load = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kAttnThreads * i, key = idx >> 5, ch = idx & 31;
      const int64_t t = int64_t(b) * a.T + min(t0 + key, L - 1);
      pf[i] = ld16(kvh + t * H * kNcat + 8 * ch);
    }
    const int key = tid >> 3, ch = tid & 7;
    const int64_t t = int64_t(b) * a.T + min(t0 + key, L - 1);
    pf[4] = ld16(kr + t * kDR + 8 * ch);
  };
  auto store = [&](AttnTile& tl) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kAttnThreads * i, key = idx >> 5, ch = idx & 31;
      uint16_t* dst = (ch < 16) ? &tl.k[key * kKPitch + 8 * ch] : &tl.v[key * kVPitch + 8 * (ch - 16)];
      *reinterpret_cast<u32x4*>(dst) = pf[i];
    }
    const int key = tid >> 3, ch = tid & 7;
    *reinterpret_cast<u32x4*>(&tl.k[key * kKPitch + 8 * (16 + ch)]) = pf[4];  // RoPE after the key
  };

  f32x16 oacc[kDH / 32];  // O^T: dims 32 db + 8 i + 4 hh + r, query n
#pragma unroll
  for (int d = 0; d < kDH / 32; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;

  auto compute = [&](const AttnTile& tl, int t0) {
    // S^T[key][query] for keys t0 + 32 kb + (8 i + 4 hh + r); product i is key block i % 2,
    // k-step i / 2, and its operand is read kPre products ahead.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
    constexpr int kSteps = 2 * (kDQK / 16), kPre = 4;
    const uint16_t* kbase = &tl.k[n * kKPitch + 8 * hh];
    auto operand = [&](int i) {
      return *reinterpret_cast<const bf16x8*>(kbase + (i & 1) * 32 * kKPitch + 16 * (i >> 1));
    };
    bf16x8 ring[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) ring[i] = operand(i);
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const bf16x8 av = ring[i % kPre];
      if (i + kPre < kSteps) ring[i % kPre] = operand(i + kPre);
      sacc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[i >> 1], sacc[i & 1], 0, 0, 0);
    }
    // The tile max of this query's 64 keys (half of them in the partner lane), masking only
    // where the tile reaches past the wave's first query; raw scores, scaled to base 2
    // afterwards (the scale is positive, so it commutes with the max) and inside the
    // exponent's fused multiply-add.
    float tmax = -INFINITY;
    if (t0 + kKT - 1 > pos_first_w) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = t0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (t > pos) sacc[kb][e] = -INFINITY;
          tmax = fmaxf(tmax, sacc[kb][e]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sacc[kb][e]);
    }
    {
      float x0 = tmax, x1 = tmax;
      permlane32_swap(x0, x1);
      tmax = fmaxf(x0, x1) * a.scale_log2;
    }
    // Move the reference only when the tile exceeds it by more than kTau.
    const bool grow = tmax > m_ref + kTau;  // false while nothing is visible
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - tmax) : 1.f;
    if (grow) m_ref = tmax;
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], a.scale_log2, neg_m));
        sacc[kb][e] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int d = 0; d < kDH / 32; ++d) oacc[d] *= alpha;
    }

    // P^T operands: k-step ks covers keys 16 ks + 8 hh + (0..7); this lane holds keys
    // 16 (ks % 2) + 4 hh + (0..3) (register group 2 (ks % 2)) and + 8 (group 2 (ks % 2) + 1)
    // of block ks / 2; one swap with the partner lane completes the operand.
    // V^T operands (transposed reads): lane l of 16-lane group G supplies row
    // 8 (G >> 1) + (l >> 2) % 4 (+ 4 for the second half) and columns 16 (G & 1) + 4 (l % 4)
    // of each 16-row x 32-column block; k-step ks adds 16 rows, column block d adds 32.
    const int G = lane >> 4;
    const uint16_t* vbase = &tl.v[(8 * (G >> 1) + ((lane >> 2) & 3)) * kVPitch + 16 * (G & 1) + 4 * (lane & 3)];
    auto voperand = [&](int ks, int d) {
      const u32x2 lo = lds_read_tr4(vbase + 16 * ks * kVPitch + 32 * d);
      const u32x2 hi = lds_read_tr4(vbase + (16 * ks + 4) * kVPitch + 32 * d);
      return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    bf16x8 vnext[kDH / 32];
#pragma unroll
    for (int d = 0; d < kDH / 32; ++d) vnext[d] = voperand(0, d);
#pragma unroll
    for (int ks = 0; ks < kKT / 16; ++ks) {
      const int kb = ks >> 1, g = 2 * (ks & 1);
      bf16x8 vcur[kDH / 32];
#pragma unroll
      for (int d = 0; d < kDH / 32; ++d) {
        vcur[d] = vnext[d];
        if (ks + 1 < kKT / 16) vnext[d] = voperand(ks + 1, d);
      }
      uint32_t u0 = pack_bf16x2(sacc[kb][4 * g], sacc[kb][4 * g + 1]);
      uint32_t u1 = pack_bf16x2(sacc[kb][4 * g + 2], sacc[kb][4 * g + 3]);
      uint32_t v0 = pack_bf16x2(sacc[kb][4 * g + 4], sacc[kb][4 * g + 5]);
      uint32_t v1 = pack_bf16x2(sacc[kb][4 * g + 6], sacc[kb][4 * g + 7]);
      swap32_u32(u0, v0);
      swap32_u32(u1, v1);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{u0, u1, v0, v1});
#pragma unroll
      for (int d = 0; d < kDH / 32; ++d)
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[d], pb, oacc[d], 0, 0, 0);
    }
  };

  if (ntiles > 0) {
    load(0);
    store(sm[0]);
    __syncthreads();
    if (ntiles > 1) load(kKT);
  }
  for (int j = 0; j < ntiles; ++j) {
    const int t0 = j * kKT;
    if (t0 <= pos_last_w) compute(sm[j & 1], t0);  // tiles past the wave's last query add nothing
    if (j + 1 < ntiles) {
      store(sm[(j + 1) & 1]);  // that buffer was last read in step j - 1, before its barrier
      __syncthreads();
      if (j + 2 < ntiles) load(t0 + 2 * kKT);
    }
  }

  float lt = l_run;
  {
    float x0 = lt, x1 = lt;
    permlane32_swap(x0, x1);
    lt = x0 + x1;
  }
  if (qi >= S) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int64_t row = (int64_t(b) * S + qi) * H + h;
  uint16_t* o = static_cast<uint16_t*>(a.out) + row * kDH;
#pragma unroll
  for (int d = 0; d < kDH / 32; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 32 * d + 8 * i + 4 * hh;
      *reinterpret_cast<u32x2*>(o + col) = u32x2{pack_bf16x2(oacc[d][4 * i] * inv, oacc[d][4 * i + 1] * inv),
                                                 pack_bf16x2(oacc[d][4 * i + 2] * inv, oacc[d][4 * i + 3] * inv)};
    }
  if (a.lse && hh == 0) a.lse[row] = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;
}

}  // namespace

namespace {
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

size_t prefill_workspace_bytes(int32_t B, int32_t T, int32_t H) {
  return round256(size_t(H) * kNcat * kDC * 2) + round256(size_t(B) * T * H * kNcat * 2);
}

int launch_prefill(PrefillArgs a, void* ws, hipStream_t s) {
  uint16_t* wcat = static_cast<uint16_t*>(ws);
  uint16_t* kv = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + round256(size_t(a.H) * kNcat * kDC * 2));
  hipLaunchKernelGGL(prefill_weights_kernel, dim3(a.H, kNcat / 32), dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.w_uk), static_cast<const uint16_t*>(a.w_uv), wcat);
  const int M = a.B * a.T;
  hipLaunchKernelGGL(decompress_kernel, dim3((M + kGM - 1) / kGM, a.H), dim3(kGThreads), 0, s,
                     static_cast<const uint16_t*>(a.c_kv), wcat, kv, M, a.H);
  a.kv = kv;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(a.H, (a.S + kQB - 1) / kQB, a.B), dim3(kAttnThreads), 0, s, a);
  return int(hipGetLastError());
}

}  // namespace mla
