// Backward grouped expert GEMMs of the MoonEP path on gfx950: the FFN
// backward data path (dZ, SwiGLU backward, dX) and the weight gradients
// into the fp32 [E+B,H,H'] gradient rows (see gemm_core.h for the shared
// core).
#include "gemm_core.h"

namespace moonep {
namespace {

// ---------------------------------------------------------------------------
// Backward of the grouped SwiGLU FFN (chain rule of the forward above):
//   dZ = dY Wd                                   (ffn_bwd_dz)
//   dU = dZ * silu(G), dG = dZ * U * silu'(G),   (ffn_bwd_gu: G, U recomputed
//   silu'(g) = sigma(g) (1 + g (1 - sigma(g)))    from X with the gate/up loop)
//   dX = dG Wg^T + dU Wu^T                       (ffn_bwd_dx: one K = 2H' loop)
// dZ, dG, dU and dX are stored as bf16 (round to nearest even).

// dZ tile: 32 MI x 2 rows, 256 columns of H' (two 128-column regions of Wd,
// which is [k = H][n = H'] for this product), K = H.
template <int MI>
__device__ __forceinline__ void bwd_dz_tile(const FfnArgs& a, const Ring& smem, int d,
                                            const Tile& tl, int nt) {
  const int n0 = nt * BN;
  const int rows_valid = tl.m1 - tl.m0;
  const int cols_valid = a.Hp - n0 < BN ? a.Hp - n0 : BN;
  const int nv0 = cols_valid < 128 ? cols_valid : 128, nv1 = cols_valid - nv0;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  RowTileT<2 * MI> la;
  ColTile lb;
  la.init(a.dy + ((int64_t)d * a.NvS + tl.m0) * a.H, a.H, rows_valid);
  const uint16_t* wd = weight_row(a, 2, d, tl.row) + n0;
  lb.init(wd, wd + 128, a.Hp, a.H, nv0, nv1);
  f32x16 acc[MI][4];
  gemm_loop<MI>(la, lb, smem, a.H / BK, acc, wm * 32 * MI, nrow);

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
  const Rsrc ds = make_rsrc(a.dz + ((int64_t)d * a.NvS + tl.m0) * a.Hp + n0,
                            (int64_t)rows_valid * a.Hp * 2);
  St::flush(reg, ds, wm * 32 * MI, a.Hp, wn * 128, cols_valid);
}

// dG, dU tile: the gate/up product of the forward (same tile, same loop),
// then per element the SwiGLU backward with dZ read from memory.
template <int MI>
__device__ __forceinline__ void bwd_gu_tile(const FfnArgs& a, const Ring& smem, int d,
                                            const Tile& tl, int nt) {
  const int n0 = nt * 128;
  const int rows_valid = tl.m1 - tl.m0;
  const int nvh = a.Hp - n0 < 128 ? a.Hp - n0 : 128;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 64, wn * 64 + 32, 128 + wn * 64, 128 + wn * 64 + 32};

  RowTileT<2 * MI> la;
  ColTile lb;
  la.init(a.x + ((int64_t)d * a.NvS + tl.m0) * a.H, a.H, rows_valid);
  lb.init(weight_row(a, 0, d, tl.row) + n0, weight_row(a, 1, d, tl.row) + n0, a.Hp, a.H, nvh,
          nvh);
  f32x16 acc[MI][4];
  gemm_loop<MI>(la, lb, smem, a.H / BK, acc, wm * 32 * MI, nrow);

  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  typedef Stage<32 * MI, 64> St;
  lds_t* reg_g = smem.base + wave * (2 * St::kBytes);
  lds_t* reg_u = reg_g + St::kBytes;
  const uint16_t* dzb = a.dz + ((int64_t)d * a.NvS + tl.m0) * a.Hp + n0;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  // every dZ read of the tile is issued before the first is used
  u32x2 dzv[MI][2][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm * 32 * MI + i * 32 + lr;
        const int n = wn * 64 + j * 32 + acc_col(q, lh);
        dzv[i][j][q] = u32x2{0u, 0u};
        if (m < rows_valid && n < nvh) dzv[i][j][q] = *(const u32x2*)(dzb + (int64_t)m * a.Hp + n);
      }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float dg[4], du[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned w = dzv[i][j][q][e >> 1];
          const unsigned bits = e & 1 ? (w & 0xFFFF0000u) : (w << 16);
          const float dz = __uint_as_float(bits);
          const float g = acc[i][j][4 * q + e], u = acc[i][j + 2][4 * q + e];
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));   // as in the forward
          du[e] = dz * (g * sg);
          dg[e] = dz * u * (sg * (1.0f + g * (1.0f - sg)));
        }
        St::put(reg_g, i, j, q, pack_bf16x2(dg[0], dg[1]),
                pack_bf16x2(dg[2], dg[3]));
        St::put(reg_u, i, j, q, pack_bf16x2(du[0], du[1]),
                pack_bf16x2(du[2], du[3]));
      }
  const int64_t base = ((int64_t)d * a.NvS + tl.m0) * a.Hp + n0;
  const int64_t range = (int64_t)rows_valid * a.Hp * 2;
  St::flush(reg_g, make_rsrc(a.dg + base, range), wm * 32 * MI, a.Hp, wn * 64, nvh);
  St::flush(reg_u, make_rsrc(a.du + base, range), wm * 32 * MI, a.Hp, wn * 64, nvh);
}

// dX tile: 32 MI x 2 rows, 256 columns of H, K = 2 H' over [dG | dU] and the
// matching rows of [Wg | Wu] (row h of each holds the H' values of that h).
template <int MI>
__device__ __forceinline__ void bwd_dx_tile(const FfnArgs& a, const Ring& smem, int d,
                                            const Tile& tl, int nt) {
  const int n0 = nt * BN;
  const int rows_valid = tl.m1 - tl.m0;
  const int cols_valid = a.H - n0 < BN ? a.H - n0 : BN;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  RowTile2<2 * MI> la;
  RowTile2<8> lb;
  const int64_t abase = ((int64_t)d * a.NvS + tl.m0) * a.Hp;
  la.init(a.dg + abase, a.du + abase, a.Hp, rows_valid, a.Hp);
  lb.init(weight_row(a, 0, d, tl.row) + (int64_t)n0 * a.Hp,
          weight_row(a, 1, d, tl.row) + (int64_t)n0 * a.Hp, a.Hp, cols_valid, a.Hp);
  f32x16 acc[MI][4];
  gemm_loop<MI>(la, lb, smem, 2 * a.Hp / BK, acc, wm * 32 * MI, nrow);

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
  const Rsrc xs = make_rsrc(a.dx + ((int64_t)d * a.NvS + tl.m0) * a.H + n0,
                            (int64_t)rows_valid * a.H * 2);
  St::flush(reg, xs, wm * 32 * MI, a.H, wn * 128, cols_valid);
}


MOONEP_TILE_KERNEL(ffn_bwd_dz, bwd_dz_tile)
MOONEP_TILE_KERNEL(ffn_bwd_gu, bwd_gu_tile)
MOONEP_TILE_KERNEL(ffn_bwd_dx, bwd_dx_tile)

// ---------------------------------------------------------------------------
struct WgradArgs {
  const uint16_t* a;        // [R*NvS][H]
  const uint16_t* b;        // [R*NvS][Hp]
  float* gh;                // [E][H][Hp]
  float* rb;                // [R*B][H][Hp]
  const int32_t* act;       // [R][2L]
  const int32_t* nact;      // [R] active rows (the first entries of act)
  const int32_t* cu;        // [R][E+B]
  const int32_t* segn;      // [R][E+B]
  int R, E, B, H, Hp, NvS, L2, EB, tp, rank0, nranks, ntm, ntn;
};

constexpr int kWgradChunk = 32;   // CUs per XCD

// dW[h][h'] += sum over the segment's tokens t of A[t][h] * B[t][h'].
// Tile: 256 h (MFMA rows) x 256 h' (MFMA columns), contraction over t.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void wgrad_kernel(WgradArgs a) {
  MOONEP_RING(smem);
  // Only real tiles are enumerated: the launched ranks' active rows, rank
  // after rank, each swept over its ntm x ntn output tiles (N fastest).  The
  // list is cut into chunks of 32 tiles, one wave of an XCD's CUs, and XCD x
  // takes chunks x, x + 8, x + 16, ...: each XCD gets a like share of every
  // segment, whose tiles last in proportion to its token count, so the XCDs
  // end together whether one rank or all are launched.  (Contiguous eighths
  // of the grid's padded bound gave whole XCDs only the empty tiles of unused
  // slots when one rank is launched alone; contiguous eighths of the real
  // tiles gave them unequal token counts.)  Uniform loads: the scalar cache
  // serves them.
  const int64_t per_row = (int64_t)a.ntm * a.ntn;
  int64_t nrows = 0;
  for (int i = 0; i < a.nranks; ++i) nrows += a.nact[a.rank0 + i];
  const int64_t total = nrows * per_row;
  const int64_t c = blockIdx.x / kXcds;
  const int64_t lt = ((c / kWgradChunk) * kXcds + blockIdx.x % kXcds) * kWgradChunk +
                     c % kWgradChunk;
  if (lt >= total) return;
  int64_t qi = lt / per_row;                           // active row across the launched ranks
  int d = a.rank0;
  for (; d < a.rank0 + a.nranks - 1 && qi >= a.nact[d]; ++d) qi -= a.nact[d];
  const int64_t rem = lt % per_row;
  const int tn = (int)(rem % a.ntn);
  const int tm = (int)(rem / a.ntn);
  const int row = a.act[d * a.L2 + (int)qi];
  if (row < 0) return;
  const int end = a.cu[d * a.EB + row];
  const int ntok = a.segn[d * a.EB + row];
  const int start = end - round_up(ntok, a.tp);
  const int m0 = tm * BM, n0 = tn * BN;
  const int mv = a.H - m0 < BM ? a.H - m0 : BM;
  const int nv = a.Hp - n0 < BN ? a.Hp - n0 : BN;
  const int mv0 = mv < 128 ? mv : 128, mv1 = mv - mv0;
  const int nv0 = nv < 128 ? nv : 128, nv1 = nv - nv0;
  const uint16_t* A = a.a + ((int64_t)d * a.NvS + start) * a.H + m0;
  const uint16_t* Bm = a.b + ((int64_t)d * a.NvS + start) * a.Hp + n0;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  ColTile la, lb;
  la.init(A, A + 128, a.H, ntok, mv0, mv1);
  lb.init(Bm, Bm + 128, a.Hp, ntok, nv0, nv1);
  f32x16 acc[4][4];
  gemm_loop<4>(la, lb, smem, (ntok + BK - 1) / BK, acc, wm * 128, nrow);

  // fp32 read-modify-write, 4 consecutive columns (16 bytes) per access,
  // masked to rows < H and columns < H'.  Plain global accesses: the 128-bit
  // buffer-load builtin of this toolchain is lowered to a 32-bit load.
  const int64_t rs = (int64_t)a.H * a.Hp;
  float* G = (row < a.E ? a.gh + (int64_t)row * rs : a.rb + ((int64_t)d * a.B + row - a.E) * rs) +
             (int64_t)m0 * a.Hp + n0;
  // The 16 reads of a row block are issued together before any write: a
  // read after a write the compiler cannot prove disjoint would otherwise
  // wait for each read in turn.
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = wm * 128 + i * 32 + lr;
    float* grow = G + (int64_t)m * a.Hp;
    f32x4 v[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nrow[j] + acc_col(q, lh);
        if (m < mv && n < nv) v[j][q] = *(const f32x4*)(grow + n);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nrow[j] + acc_col(q, lh);
        if (m < mv && n < nv) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[j][q][e] = __fadd_rn(v[j][q][e], acc[i][j][4 * q + e]);
          *(f32x4*)(grow + n) = v[j][q];
        }
      }
  }
}

}  // namespace

hipError_t launch_ffn_bwd(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* x,
                          const uint16_t* dy, const WeightRef& w, uint16_t* dz, uint16_t* dg,
                          uint16_t* du, uint16_t* dx, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, w);
  a.x = x; a.dy = dy; a.dz = dz; a.dg = dg; a.du = du; a.dx = dx;
  a.ntn = (c.d.Hp + BN - 1) / BN;
  ffn_bwd_dz<<<(unsigned)tile_grid(a), kThreads, 0, s>>>(a);
  a.ntn = (c.d.Hp + 127) / 128;
  ffn_bwd_gu<<<(unsigned)tile_grid(a), kThreads, 0, s>>>(a);
  a.ntn = (c.d.H + BN - 1) / BN;
  ffn_bwd_dx<<<(unsigned)tile_grid(a), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_wgrad(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* A,
                        const uint16_t* B, float* gh, float* rb, hipStream_t s) {
  const Dims& d = c.d;
  WgradArgs a;
  a.a = A; a.b = B; a.gh = gh; a.rb = rb;
  a.act = p.aux + d.aux.act; a.nact = p.aux + d.aux.nact;
  a.cu = p.cu_seqlens; a.segn = p.seg_tokens;
  a.R = d.R; a.E = d.E; a.B = d.B; a.H = d.H; a.Hp = d.Hp; a.NvS = (int)d.NvS;
  a.L2 = 2 * d.L; a.EB = d.E + d.B; a.tp = d.tp;
  a.rank0 = rank < 0 ? 0 : rank;
  a.nranks = rank < 0 ? d.R : 1;
  a.ntm = (d.H + BM - 1) / BM;
  a.ntn = (d.Hp + BN - 1) / BN;
  const int64_t total = (int64_t)a.nranks * a.L2 * a.ntm * a.ntn;
  const int64_t chunks = kXcds * kWgradChunk;   // the grid covers whole rounds of chunks
  wgrad_kernel<<<(unsigned)((total + chunks - 1) / chunks * chunks), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moonep
