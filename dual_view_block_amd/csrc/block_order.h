// Longest-first order of the anchor blocks of one packed training sequence.
//
// Each work-group of the training launches takes one (block, KV head); a
// block's work grows with its clean prefix, ceil(anchor / 64) tiles.  Blocks
// come in the caller's order (random anchors), so a long block can start
// last and set the launch's end.  Taking the blocks in decreasing tile count
// instead (ties by index) makes the launch a longest-first list schedule:
// work-group j processes the block of rank j.  The rank is selected on the
// device by one wave per work-group: the tile counts of up to 256 blocks sit
// four per lane; a binary search over the tile count finds the count T of the
// rank-j block (fewer than j+1 blocks have more tiles, at least j+1 have T or
// more), and the block is the (j - #{more than T})-th block with exactly T
// tiles in index order.  Ballots and scalar bit counts only: no memory beyond
// the anchors and no synchronisation, and every wave finds the same block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthrus {

// Blocks the device-side ranking handles; more are taken in the caller's order.
constexpr int kRankMaxBlocks = 256;

__device__ __forceinline__ int rank_count(const int (&t)[4], int thr) {  // #{blocks with t >= thr}
  int c = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) c += __builtin_popcountll(__ballot(t[u] >= thr));
  return c;
}

// The block of rank j (0 <= j < n <= kRankMaxBlocks) by tile count
// ceil(clamp(anchor, 0, max_len) / 64) descending, ties by index.  Called by
// a whole wave.
__device__ __forceinline__ int block_by_rank(const int32_t* __restrict__ anchors, int n, int max_len, int j) {
  const int lane = threadIdx.x & 63;
  int t[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int b = 64 * u + lane;
    int L = b < n ? anchors[b] : 0;
    L = L < 0 ? 0 : (L > max_len ? max_len : L);
    t[u] = b < n ? (L + 63) / 64 : -1;  // absent blocks rank below every real one
  }
  int lo = 0, hi = (max_len + 63) / 64;  // the rank-j tile count lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (rank_count(t, mid) > j) lo = mid;
    else hi = mid - 1;
  }
  int r = j - rank_count(t, lo + 1);  // position among the blocks with exactly lo tiles
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    unsigned long long m = __ballot(t[u] == lo);
    const int c = __builtin_popcountll(m);
    if (r < c) {
      for (int i = 0; i < r; ++i) m &= m - 1;  // drop the r lowest set bits
      return 64 * u + __builtin_ctzll(m);
    }
    r -= c;
  }
  return j;  // not reached for 0 <= j < n
}

}  // namespace orthrus
