// Forward grouped expert GEMMs of the MoonEP path on gfx950: the gate/up
// product with its SwiGLU epilogue and the down product (see gemm_core.h for
// the shared core and tile_schedule.h for the M-tiles they walk).
#include "gemm_core.h"

namespace moonep {
namespace {

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
  gemm_loop<MI>(la, lb, smem, a.H / BK, acc, wm * 32 * MI, nrow);

  // SwiGLU epilogue: blocks j = 0,1 are gate, j = 2,3 the matching up; the
  // wave's 32 MI x 64 block of Z is staged in LDS and stored as whole rows.
  // Rows past the segment fall outside the store range; columns past H' get
  // an out-of-range offset.
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
          // silu(g) = g / (1 + e^-g) with the hardware reciprocal (~1 ulp of
          // fp32, far below Z's bf16 rounding) instead of an IEEE division
          // sequence: the epilogue runs with the matrix unit idle
          z[e] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        }
        St::put(reg, i, j, q, pack_bf16x2(z[0], z[1]),
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
  gemm_loop<MI>(la, lb, smem, a.Hp / BK, acc, wm * 32 * MI, nrow);

  typedef Stage<32 * MI, 128> St;
  lds_t* reg = smem.base + wave * St::kBytes;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        St::put(reg, i, j, q,
                pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
  const Rsrc ys = make_rsrc(a.y + ((int64_t)d * a.NvS + tl.m0) * a.H + n0,
                            (int64_t)rows_valid * a.H * 2);
  St::flush(reg, ys, wm * 32 * MI, a.H, wn * 128, cols_valid);
}

MOONEP_TILE_KERNEL(ffn_gateup, gateup_tile)
MOONEP_TILE_KERNEL(ffn_down, down_tile)

}  // namespace

hipError_t launch_gateup(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* x_nvs,
                         const WeightRef& w, uint16_t* z, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, w);
  a.x = x_nvs;
  a.z = z;
  a.ntn = (c.d.Hp + 127) / 128;
  ffn_gateup<<<(unsigned)tile_grid(a), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* z,
                       const WeightRef& w, uint16_t* y, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, w);
  a.zin = z;
  a.y = y;
  a.ntn = (c.d.H + BN - 1) / BN;
  ffn_down<<<(unsigned)tile_grid(a), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moonep
