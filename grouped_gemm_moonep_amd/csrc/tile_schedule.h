// The M-tile schedule of the grouped GEMMs, built with every plan (by extra
// workgroups of the planner's last kernel) and read by the GEMM kernels'
// tile decode.  Tile entry t of rank d holds (row, first slot, end slot,
// group start * 16 + group size).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moonep {

constexpr int kTileM = 256;        // rows of an M-tile
constexpr int kShortTileM = 128;   // a segment tail of at most this many rows runs as a short tile
constexpr int kGroupMax = 8;       // most M-tiles of one segment that share a weight slab in L2

__device__ __forceinline__ int tile_round_up(int n, int m) { return (n + m - 1) / m * m; }

// Built by one workgroup of 256 threads per rank (thread q takes active row
// q of the rank).  A segment of padded length len has floor(len/256) tiles of
// 256 rows; a remainder of more than 128 rows is one more tile of the same
// duration, and a remainder of at most 128 rows is a short tile (half the
// rows and half the duration).  Full-duration tiles come first, in segment
// order; a segment's n of them form ceil(n / 8) groups of nearly equal size
// (a segment of up to 8 tiles is one group, so its weight slabs are fetched
// once; with ntn N-tiles an M-tile's activations are then fetched about
// ntn n / 32 times, which grows slower than the weights saved).  The short
// tiles of every segment follow, in pairs.  Within each part all tiles run equally long, so the
// workgroups that share an XCD's L2 stay in step: a short tile among full
// ones frees its CU early, the tiles taken next start out of phase with
// their neighbours, and the operand slices they would have shared are
// fetched again.

// Exclusive block-wide scan of one value per thread (256 threads); *total
// gets the sum.
__device__ __forceinline__ int block_scan256(int v, int* total, int (&wsum)[4]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int x = v;                                     // inclusive scan within the wave
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += wsum[i];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();                               // wsum is reused by the next call
  return before + x - v;
}

// Per pass of 256 active rows: each row's first full tile, end of its full tiles, row,
// segment end, padded length and group size, so that all threads can write the tiles.
struct TileSchedLds {
  int t0[256], tend[256], row[256], end[256], len[256], grp[256];
};

// act, aend, an: [R][L2] active rows of each rank, their padded segment ends
// and real token counts (entries past the rank's last active row: row -1).
__device__ __forceinline__ void build_tile_schedule(const int32_t* act, const int32_t* aend,
                                                    const int32_t* an, int32_t* tiles,
                                                    int32_t* ntiles, int32_t* nfull, int d,
                                                    int L2, int tp, int max_tiles,
                                                    int (&wsum)[4], TileSchedLds& sl) {
  const int tid = threadIdx.x;
  int32_t* rank_tiles = tiles + (int64_t)d * max_tiles * 4;
  auto put = [&](int t, int row, int m0, int m1, int gs, int gm) {
    if (t >= max_tiles) return;
    int32_t* e = rank_tiles + (int64_t)t * 4;
    e[0] = row;
    e[1] = m0;
    e[2] = m1;
    e[3] = gs * 16 + gm;
  };
  // part 1: full-duration tiles
  int nfull_all = 0;
  for (int q0 = 0; q0 < L2; q0 += 256) {
    const int q = q0 + tid;
    const int row = q < L2 ? act[d * L2 + q] : -1;
    int end = 0, len = 0, nf = 0;
    if (row >= 0) {
      end = aend[d * L2 + q];
      len = tile_round_up(an[d * L2 + q], tp);
      const int rem = len % kTileM;
      nf = len / kTileM + (rem > kShortTileM ? 1 : 0);
    }
    int total;
    const int t0 = nfull_all + block_scan256(nf, &total, wsum);
    const int ng = (nf + kGroupMax - 1) / kGroupMax;
    const int g = ng > 0 ? (nf + ng - 1) / ng : 1;      // group size
    sl.t0[tid] = t0;
    sl.tend[tid] = t0 + nf;
    sl.row[tid] = row;
    sl.end[tid] = end;
    sl.len[tid] = len;
    sl.grp[tid] = g;
    __syncthreads();
    // every thread writes tiles t, t + 256, ...: the row of tile t is the first
    // one whose tiles end past t (one segment can hold hundreds of tiles)
    for (int t = nfull_all + tid; t < nfull_all + total; t += 256) {
      int lo = 0, hi = 255;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sl.tend[mid] > t) hi = mid;
        else lo = mid + 1;
      }
      const int j = t - sl.t0[lo], gq = sl.grp[lo], eq = sl.end[lo];
      const int m = eq - sl.len[lo] + j * kTileM;
      const int gs = sl.t0[lo] + j / gq * gq;
      put(t, sl.row[lo], m, m + kTileM < eq ? m + kTileM : eq, gs, min(gq, sl.tend[lo] - gs));
    }
    nfull_all += total;
    __syncthreads();                               // sl is rewritten by the next pass
  }
  // part 2: short tiles, in pairs
  int nshort_all = 0;
  for (int q0 = 0; q0 < L2; q0 += 256) {
    const int q = q0 + tid;
    const int row = q < L2 ? act[d * L2 + q] : -1;
    int end = 0, rem = 0;
    if (row >= 0) {
      end = aend[d * L2 + q];
      rem = tile_round_up(an[d * L2 + q], tp) % kTileM;
    }
    const int ns = rem > 0 && rem <= kShortTileM ? 1 : 0;
    int total;
    const int i = nshort_all + block_scan256(ns, &total, wsum);
    if (ns) put(nfull_all + i, row, end - rem, end, nfull_all + i / 2 * 2, 2);
    nshort_all += total;
  }
  // an odd last short tile is a group of its own (known only now)
  __syncthreads();
  if (tid == 0 && (nshort_all & 1) && nfull_all + nshort_all - 1 < max_tiles)
    rank_tiles[(int64_t)(nfull_all + nshort_all - 1) * 4 + 3] =
        (nfull_all + nshort_all - 1) * 16 + 1;
  if (tid == 0) {
    const int n = nfull_all + nshort_all;
    ntiles[d] = n < max_tiles ? n : max_tiles;
    nfull[d] = nfull_all < max_tiles ? nfull_all : max_tiles;
  }
}

}  // namespace moonep
