// Work distribution of the 64-row matrix-core decode kernels: which pieces (sequence,
// row block, token range) one workgroup runs.
//
// Grid: one workgroup per (row block, work unit), handed out XCD-aware.  Static splits:
// the unit is (sequence, split) and the piece is the split's token chunk.  Balanced ranges:
// the unit is a range of the batch's concatenated 32-token tiles, walked sequence by
// sequence; a sequence that lies wholly inside the range is a final piece, the range's cut
// first and last sequences write partials to the range's slots 0 and 1 (slot 0 when one
// sequence covers the whole range).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "mla_internal.h"

namespace mla {

// piece(b, rb, t_lo, t_hi, L, final, out_base) runs query rows [64 rb, 64 rb + 64) of
// sequence b (length L) over tokens [t_lo, t_hi); final pieces write o_lat / lse at row
// out_base + 64 rb, the others their partials (it must be always_inline: a call would
// spill the kernel's registers).  lds_prefix holds kThreads * 2 + 1 entries,
// lds_wave_tot kThreads / 64.  Every wave of the workgroup runs the same pieces.
template <int kTile, int kThreads, class Piece>
__device__ __forceinline__ void walk_pieces(const DecodeArgs& a, int num_splits, int chunk, int rblocks,
                                            int n_units, int n_xcd, int64_t* lds_prefix,
                                            int64_t* lds_wave_tot, Piece&& piece) {
  // Workgroups are handed to the n_xcd XCDs round-robin by id; give each XCD a contiguous
  // range of work units so that the row blocks of one piece share an L2.
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
    piece(b, rb, t_lo, min(L, t_lo + chunk), L, fin,
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
    if (lane == 63) lds_wave_tot[wave] = incl2;
    __syncthreads();
    for (int k = 0; k < wave; ++k) incl2 += lds_wave_tot[k];
    const int64_t excl = incl2 - t0 - t1;
    if (2 * tid < a.B) lds_prefix[2 * tid] = excl;
    if (2 * tid + 1 < a.B) lds_prefix[2 * tid + 1] = excl + t0;
    if (tid == kThreads - 1) lds_prefix[a.B] = incl2;  // 2 kThreads >= B: the total
    __syncthreads();
    if (unit == 0)
      for (int i = tid; i <= a.B; i += kThreads) const_cast<int64_t*>(a.prefix)[i] = lds_prefix[i];
  }
  // Prefix entries are the same for every lane: keep them in scalar registers.
  auto pre = [&](int i) -> int64_t {
    if (wave_pfx) return i == 0 ? int64_t(0) : int64_t(__builtin_amdgcn_readlane(incl, i - 1));
    const int64_t v = a.prefix_here ? lds_prefix[i] : a.prefix[i];
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
    piece(b, rb, int(cur - p0) * kTile, min(L, int(e - p0) * kTile), L, fin, base);
    cur = e;
    for (++b; b < a.B && pre(b + 1) <= cur;) ++b;  // skip sequences without tiles
  }
}

}  // namespace mla
