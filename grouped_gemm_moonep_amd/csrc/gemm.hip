// Forward grouped expert GEMMs of the MoonEP path on gfx950: the M-tile
// schedule built with every plan, the gate/up product with its SwiGLU
// epilogue and the down product (see gemm_core.h for the shared core).
#include "gemm_core.h"

namespace moonep {
namespace {

// ---------------------------------------------------------------------------
// The M-tile schedule, one workgroup of 256 threads per rank (thread q takes
// active row q).  A segment of padded length len has floor(len/256) tiles of
// 256 rows; a remainder of more than 128 rows is one more tile of the same
// duration, and a remainder of at most 128 rows is a short tile (MI = 2, half
// the duration).  Full-duration tiles come first, in segment order, in groups
// of up to kGroupM tiles of one segment; the short tiles of every segment
// follow, in pairs.  Within each part all tiles run equally long, so the
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

__global__ __launch_bounds__(256) void gemm_schedule(const int32_t* act, const int32_t* cu,
                                                     const int32_t* segn, int32_t* tiles,
                                                     int32_t* ntiles, int L2, int EB, int tp,
                                                     int max_tiles) {
  __shared__ int wsum[4];
  const int d = blockIdx.x, tid = threadIdx.x;
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
      end = cu[d * EB + row];
      len = round_up(segn[d * EB + row], tp);
      const int rem = len % BM;
      nf = len / BM + (rem > kHalfTileM ? 1 : 0);
    }
    int total;
    const int t0 = nfull_all + block_scan256(nf, &total, wsum);
    for (int j = 0; j < nf; ++j) {
      const int m = end - len + j * BM;
      const int gs = t0 + j / kGroupM * kGroupM;
      put(t0 + j, row, m, m + BM < end ? m + BM : end, gs, min(kGroupM, t0 + nf - gs));
    }
    nfull_all += total;
  }
  // part 2: short tiles, in pairs
  int nshort_all = 0;
  for (int q0 = 0; q0 < L2; q0 += 256) {
    const int q = q0 + tid;
    const int row = q < L2 ? act[d * L2 + q] : -1;
    int end = 0, rem = 0;
    if (row >= 0) {
      end = cu[d * EB + row];
      rem = round_up(segn[d * EB + row], tp) % BM;
    }
    const int ns = rem > 0 && rem <= kHalfTileM ? 1 : 0;
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
  }
}

// ---------------------------------------------------------------------------
// Tile bodies, templated on MI = 32-row MFMA blocks per wave: MI = 4 is the
// full 256-row tile (each wave 128 rows), MI = 2 the 128-row tile that ends a
// segment whose padded length is an odd multiple of 128 (each wave 64 rows),
// so a segment's last tile never computes 128 empty rows.

// gate/up: 32 MI x 2 rows per workgroup, 128 gate + 128 up columns, K = H.
template <int MI>
__device__ __forceinline__ void gateup_tile(const FfnArgs& a, const Ring& smem, int d,
                                            const Tile& tl, int nt) {
  const int n0 = nt * 128;
  const int rows_valid = tl.m1 - tl.m0;
  const int nvh = a.Hp - n0 < 128 ? a.Hp - n0 : 128;   // valid columns of each half
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 64, wn * 64 + 32, 128 + wn * 64, 128 + wn * 64 + 32};

  RowTileT<2 * MI> la;
  ColTile lb;
  la.init(a.x + ((int64_t)d * a.NvS + tl.m0) * a.H, a.H, rows_valid);
  lb.init(weight_row(a, 0, d, tl.row) + n0, weight_row(a, 1, d, tl.row) + n0, a.Hp, a.H, nvh,
          nvh);
  f32x16 acc[MI][4];
  zero_acc<MI>(acc);
  gemm_loop<MI>(la, lb, smem, a.H / BK, acc, wm * 32 * MI, nrow);

  // SwiGLU epilogue: blocks j = 0,1 are gate, j = 2,3 the matching up; the
  // wave's 32 MI x 64 block of Z is staged in LDS and stored as whole rows.
  // Rows past the segment fall outside the store range; columns past H' get
  // an out-of-range offset.
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  typedef Stage<32 * MI, 64> St;
  lds_t* reg = smem.base + wave * St::kBytes;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = acc[i][j][4 * q + e], u = acc[i][j + 2][4 * q + e];
          z[e] = g / (1.0f + __expf(-g)) * u;
        }
        St::put(reg, i * 32 + lr, j * 32 + acc_col(q, lh), pack_bf16x2(z[0], z[1]),
                pack_bf16x2(z[2], z[3]));
      }
  const Rsrc zs = make_rsrc(a.z + ((int64_t)d * a.NvS + tl.m0) * a.Hp + n0,
                            (int64_t)rows_valid * a.Hp * 2);
  St::flush(reg, zs, wm * 32 * MI, a.Hp, wn * 64, nvh);
}

// down: 32 MI x 2 rows per workgroup, 256 columns, K = H'.
template <int MI>
__device__ __forceinline__ void down_tile(const FfnArgs& a, const Ring& smem, int d,
                                          const Tile& tl, int nt) {
  const int n0 = nt * BN;
  const int rows_valid = tl.m1 - tl.m0;
  const int cols_valid = a.H - n0 < BN ? a.H - n0 : BN;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  RowTileT<2 * MI> la;
  RowTile lb;
  la.init(a.zin + ((int64_t)d * a.NvS + tl.m0) * a.Hp, a.Hp, rows_valid);
  lb.init(weight_row(a, 2, d, tl.row) + (int64_t)n0 * a.Hp, a.Hp, cols_valid);
  f32x16 acc[MI][4];
  zero_acc<MI>(acc);
  gemm_loop<MI>(la, lb, smem, a.Hp / BK, acc, wm * 32 * MI, nrow);

  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  typedef Stage<32 * MI, 128> St;
  lds_t* reg = smem.base + wave * St::kBytes;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        St::put(reg, i * 32 + lr, j * 32 + acc_col(q, lh),
                pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
  const Rsrc ys = make_rsrc(a.y + ((int64_t)d * a.NvS + tl.m0) * a.H + n0,
                            (int64_t)rows_valid * a.H * 2);
  St::flush(reg, ys, wm * 32 * MI, a.H, wn * 128, cols_valid);
}

MOONEP_TILE_KERNEL(ffn_gateup, gateup_tile)
MOONEP_TILE_KERNEL(ffn_down, down_tile)

}  // namespace

hipError_t launch_gemm_schedule(const Ctx& c, const moonep_plan_t& p, hipStream_t s) {
  const Dims& d = c.d;
  gemm_schedule<<<d.R, 256, 0, s>>>(p.aux + d.aux.act, p.cu_seqlens, p.seg_tokens,
                                   p.aux + d.aux.tiles, p.aux + d.aux.ntiles, 2 * d.L,
                                   d.E + d.B, d.tp, d.max_tiles);
  return hipGetLastError();
}

hipError_t launch_gateup(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* x_nvs,
                         const WeightRef& w, uint16_t* z, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, w);
  a.x = x_nvs;
  a.z = z;
  a.ntn = (c.d.Hp + 127) / 128;
  ffn_gateup<<<(unsigned)pad_grid((int64_t)a.nranks * a.max_tiles * a.ntn), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* z,
                       const WeightRef& w, uint16_t* y, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, w);
  a.zin = z;
  a.y = y;
  a.ntn = (c.d.H + BN - 1) / BN;
  ffn_down<<<(unsigned)pad_grid((int64_t)a.nranks * a.max_tiles * a.ntn), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moonep
