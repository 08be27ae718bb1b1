// Grouped expert GEMMs of the MoonEP path on gfx950 (bf16 MFMA, fp32
// accumulation).
//
// MoonEP README (MoonshotAI/MoonEP mirror), "Usage > Integration" and
// "Weight buffer": the expert FFN of every rank is one grouped GEMM over a
// single [E+B,H,H'] tensor per projection (gate, up, down), addressed only by
// row index through cu_seqlens[E+B]; rows [0,E) are home experts, rows
// [E,E+B) the rank's prefetch slots.  "Gradient buffer": weight gradients go
// to an fp32 [E+B,H,H'] buffer whose prefetch rows live in a per-rank reduce
// buffer.  The FFN is SwiGLU: Z = silu(X Wg) * (X Wu), Y = Z Wd^T, every
// projection stored [H,H'].
//
// Kernels (all on the caller's stream):
//   gemm_schedule  one workgroup per rank: M-tiles (<= 256 rows, never
//                  crossing a segment) of every active row of the rank;
//   ffn_gateup     256x(128 gate + 128 up) tile, K = H, fused SwiGLU epilogue
//                  writing Z (bf16);
//   ffn_down       256x256 tile of Y = Z Wd^T, K = H';
//   wgrad          256x256 tile of dW += X_seg^T dY_seg over the segment's
//                  tokens, fp32 read-modify-write of the gradient row.
//
// CDNA4 mapping: 256 threads = 4 waves in a 2x2 grid, each wave a 128x128
// sub-tile as 4x4 v_mfma_f32_32x32x16_bf16 blocks (256 fp32 accumulators per
// lane).  K advances 64 per step through two 64 KiB LDS stages (A rows and
// B^T rows, 128 B each, 16-byte chunks XOR-swizzled by row so that MFMA
// fragment reads are bank-conflict free); the next step's global loads are
// in flight while the current step's MFMAs run.  Operands whose contraction
// index is not contiguous in memory (gate/up weights, both wgrad operands)
// are transposed 8x8 in registers (v_perm) on their way into LDS.
// Workgroup ids are remapped so that every XCD (own L2) works through a
// contiguous range of tiles: neighbouring tiles share weight or activation
// slabs in that XCD's L2.
#include "internal.h"

namespace moonep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kTileBytes = 256 * BK * 2;          // 32 KiB: 256 rows x 128 B
constexpr int kStageBytes = 2 * kTileBytes;       // A tile + B^T tile
constexpr int kXcds = 8;

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ int round_up(int n, int m) { return (n + m - 1) / m * m; }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Loader for an operand whose contraction index is contiguous: 256 tile rows
// x 64 k.  Thread t covers chunk t%8 (8 k) of rows t/8 + 32 i.
struct DirectTile {
  u32x4 v[8];
  __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int rows_valid,
                                       int64_t k0) {
    const int t = threadIdx.x, c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (t >> 3) + 32 * i;
      if (r < rows_valid)
        v[i] = *(const u32x4*)(base + (int64_t)r * ld + k0 + c * 8);
      else
        v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* tile) const {
    const int t = threadIdx.x, c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)(tile + lds_off((t >> 3) + 32 * i, c)) = v[i];
  }
};

// Loader for an operand stored [k][n] (n contiguous): 64 k x 256 tile rows
// (n).  Thread t covers n-chunk c = t%32 (8 n) and k-block kb = t/32 (8 k);
// the 8x8 block is transposed in registers so that each tile row holds 8
// consecutive k.  Rows [0,128) come from src0 and [128,256) from src1 (the
// gate and up weights side by side); pass src1 = src0 + 128 for one matrix.
// nv0 / nv1: valid columns of each half; k_valid: valid k rows.
struct TransTile {
  u32x4 v[8];
  __device__ __forceinline__ void load(const uint16_t* src0, const uint16_t* src1, int64_t ld,
                                       int64_t k0, int k_valid, int nv0, int nv1) {
    const int t = threadIdx.x, c = t & 31, kb = t >> 5;
    const int half = c >> 4;
    const int n = (c & 15) * 8;                 // within the half
    const uint16_t* src = half ? src1 : src0;
    const bool nok = n < (half ? nv1 : nv0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kb * 8 + i;
      if (nok && k < k_valid)
        v[i] = *(const u32x4*)(src + (k0 + k) * ld + n);
      else
        v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* tile) const {
    const int t = threadIdx.x, c = t & 31, kb = t >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sel = (j & 1) ? 0x07060302 : 0x05040100;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = __builtin_amdgcn_perm(v[2 * q + 1][j >> 1], v[2 * q][j >> 1], sel);
      *(u32x4*)(tile + lds_off(c * 8 + j, kb)) = o;
    }
  }
};

// One 64-deep step of MFMAs for a wave: A rows wm*128 + [0,128), B^T rows
// nrow[j] + [0,32) for the 4 column blocks.
__device__ __forceinline__ void mma_step(const char* A, const char* Bt, f32x16 acc[4][4], int arow0,
                                         const int nrow[4]) {
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *(const bf16x8*)(A + lds_off(arow0 + i * 32 + lr, 2 * kk + lh));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *(const bf16x8*)(Bt + lds_off(nrow[j] + lr, 2 * kk + lh));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
}

// Row (within the 32x32 block) of accumulator element v of this lane.
__device__ __forceinline__ int acc_row(int v, int lh) { return 8 * (v >> 2) + 4 * lh + (v & 3); }

// XCD-aware tile id: XCD x (= block id mod 8) walks the x-th contiguous
// eighth of the logical tile range.
__device__ __forceinline__ int64_t logical_tile() {
  const int64_t g = gridDim.x;                  // a multiple of kXcds
  const int64_t b = blockIdx.x;
  return (b % kXcds) * (g / kXcds) + b / kXcds;
}

struct Tile {
  int row, m0, m1;
};

struct FfnArgs {
  const uint16_t* x;        // [R*NvS][H]
  const uint16_t* home[3];  // [E][H][Hp]
  const uint16_t* pool[3];  // [R*B][H][Hp]
  uint16_t* z;              // [R*NvS][Hp]
  uint16_t* y;              // [R*NvS][H]
  const int32_t* tiles;     // [R][max_tiles][4]
  const int32_t* ntiles;    // [R]
  int R, E, B, H, Hp, NvS, max_tiles, rank0, nranks, ntn;
};

__device__ __forceinline__ const uint16_t* weight_row(const FfnArgs& a, int p, int d, int row) {
  const int64_t rs = (int64_t)a.H * a.Hp;
  return row < a.E ? a.home[p] + (int64_t)row * rs : a.pool[p] + ((int64_t)d * a.B + row - a.E) * rs;
}

__device__ __forceinline__ bool decode(const FfnArgs& a, int* d, Tile* tl, int* nt) {
  const int64_t lt = logical_tile();
  const int64_t total = (int64_t)a.nranks * a.max_tiles * a.ntn;
  if (lt >= total) return false;
  *nt = (int)(lt % a.ntn);
  const int t = (int)((lt / a.ntn) % a.max_tiles);
  *d = a.rank0 + (int)(lt / ((int64_t)a.ntn * a.max_tiles));
  if (t >= a.ntiles[*d]) return false;
  const int32_t* e = a.tiles + ((int64_t)*d * a.max_tiles + t) * 4;
  tl->row = e[0];
  tl->m0 = e[1];
  tl->m1 = e[2];
  return true;
}

// ---------------------------------------------------------------------------
__global__ void gemm_schedule(const int32_t* act, const int32_t* cu, const int32_t* segn,
                              int32_t* tiles, int32_t* ntiles, int L2, int EB, int tp,
                              int max_tiles) {
  if (threadIdx.x != 0) return;
  const int d = blockIdx.x;
  int t = 0;
  for (int q = 0; q < L2; ++q) {
    const int row = act[d * L2 + q];
    if (row < 0) break;
    const int end = cu[d * EB + row];
    const int len = round_up(segn[d * EB + row], tp);
    for (int m = end - len; m < end && t < max_tiles; m += BM, ++t) {
      int32_t* e = tiles + ((int64_t)d * max_tiles + t) * 4;
      e[0] = row;
      e[1] = m;
      e[2] = m + BM < end ? m + BM : end;
      e[3] = 0;
    }
  }
  ntiles[d] = t;
}

// ---------------------------------------------------------------------------
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void ffn_gateup(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  int d, nt;
  Tile tl;
  if (!decode(a, &d, &tl, &nt)) return;
  const int n0 = nt * 128;
  const int rows_valid = tl.m1 - tl.m0;
  const uint16_t* A = a.x + ((int64_t)d * a.NvS + tl.m0) * a.H;
  const uint16_t* Wg = weight_row(a, 0, d, tl.row) + n0;
  const uint16_t* Wu = weight_row(a, 1, d, tl.row) + n0;
  const int nvh = a.Hp - n0 < 128 ? a.Hp - n0 : 128;   // valid columns of each half
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 64, wn * 64 + 32, 128 + wn * 64, 128 + wn * 64 + 32};

  f32x16 acc[4][4];
  zero_acc(acc);
  DirectTile la;
  TransTile lb;
  const int nk = a.H / BK;
  la.load(A, a.H, rows_valid, 0);
  lb.load(Wg, Wu, a.Hp, 0, BK, nvh, nvh);
  la.store(smem);
  lb.store(smem + kTileBytes);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * kStageBytes;
    char* nxt = smem + ((kt + 1) & 1) * kStageBytes;
    if (kt + 1 < nk) {
      la.load(A, a.H, rows_valid, (int64_t)(kt + 1) * BK);
      lb.load(Wg, Wu, a.Hp, (int64_t)(kt + 1) * BK, BK, nvh, nvh);
    }
    mma_step(cur, cur + kTileBytes, acc, wm * 128, nrow);
    if (kt + 1 < nk) {
      la.store(nxt);
      lb.store(nxt + kTileBytes);
    }
    __syncthreads();
  }
  // SwiGLU epilogue: blocks j = 0,1 are gate, j = 2,3 the matching up.
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  uint16_t* Z = a.z + ((int64_t)d * a.NvS + tl.m0) * a.Hp + n0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * 64 + j * 32 + lr;
      if (n0 + n >= a.Hp) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + acc_row(v, lh);
        if (m < rows_valid) {
          const float g = acc[i][j][v], u = acc[i][j + 2][v];
          const float zz = g / (1.0f + __expf(-g)) * u;
          Z[(int64_t)m * a.Hp + n] = (uint16_t)bf16_rne(zz);
        }
      }
    }
}

// ---------------------------------------------------------------------------
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void ffn_down(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  int d, nt;
  Tile tl;
  if (!decode(a, &d, &tl, &nt)) return;
  const int n0 = nt * BN;
  const int rows_valid = tl.m1 - tl.m0;
  const uint16_t* A = a.z + ((int64_t)d * a.NvS + tl.m0) * a.Hp;
  const uint16_t* Wd = weight_row(a, 2, d, tl.row) + (int64_t)n0 * a.Hp;
  const int cols_valid = a.H - n0 < BN ? a.H - n0 : BN;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  f32x16 acc[4][4];
  zero_acc(acc);
  DirectTile la, lb;
  const int nk = a.Hp / BK;
  la.load(A, a.Hp, rows_valid, 0);
  lb.load(Wd, a.Hp, cols_valid, 0);
  la.store(smem);
  lb.store(smem + kTileBytes);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * kStageBytes;
    char* nxt = smem + ((kt + 1) & 1) * kStageBytes;
    if (kt + 1 < nk) {
      la.load(A, a.Hp, rows_valid, (int64_t)(kt + 1) * BK);
      lb.load(Wd, a.Hp, cols_valid, (int64_t)(kt + 1) * BK);
    }
    mma_step(cur, cur + kTileBytes, acc, wm * 128, nrow);
    if (kt + 1 < nk) {
      la.store(nxt);
      lb.store(nxt + kTileBytes);
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  uint16_t* Y = a.y + ((int64_t)d * a.NvS + tl.m0) * a.H + n0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nrow[j] + lr;
      if (n >= cols_valid) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + acc_row(v, lh);
        if (m < rows_valid) Y[(int64_t)m * a.H + n] = (uint16_t)bf16_rne(acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
struct WgradArgs {
  const uint16_t* a;        // [R*NvS][H]
  const uint16_t* b;        // [R*NvS][Hp]
  float* gh;                // [E][H][Hp]
  float* rb;                // [R*B][H][Hp]
  const int32_t* act;       // [R][2L]
  const int32_t* cu;        // [R][E+B]
  const int32_t* segn;      // [R][E+B]
  int R, E, B, H, Hp, NvS, L2, EB, tp, rank0, nranks, ntm, ntn;
};

// dW[h][h'] += sum over the segment's tokens t of A[t][h] * B[t][h'].
// Tile: 256 h (MFMA rows) x 256 h' (MFMA columns), contraction over t.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void wgrad_kernel(WgradArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  const int64_t lt = logical_tile();
  const int64_t total = (int64_t)a.nranks * a.L2 * a.ntm * a.ntn;
  if (lt >= total) return;
  const int tn = (int)(lt % a.ntn);
  const int tm = (int)((lt / a.ntn) % a.ntm);
  const int q = (int)((lt / ((int64_t)a.ntn * a.ntm)) % a.L2);
  const int d = a.rank0 + (int)(lt / ((int64_t)a.ntn * a.ntm * a.L2));
  const int row = a.act[d * a.L2 + q];
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

  f32x16 acc[4][4];
  zero_acc(acc);
  TransTile la, lb;
  const int nk = (ntok + BK - 1) / BK;
  if (nk > 0) {
    la.load(A, A + 128, a.H, 0, ntok, mv0, mv1);
    lb.load(Bm, Bm + 128, a.Hp, 0, ntok, nv0, nv1);
    la.store(smem);
    lb.store(smem + kTileBytes);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * kStageBytes;
    char* nxt = smem + ((kt + 1) & 1) * kStageBytes;
    if (kt + 1 < nk) {
      const int k0 = (kt + 1) * BK;
      la.load(A, A + 128, a.H, k0, ntok - k0, mv0, mv1);
      lb.load(Bm, Bm + 128, a.Hp, k0, ntok - k0, nv0, nv1);
    }
    mma_step(cur, cur + kTileBytes, acc, wm * 128, nrow);
    if (kt + 1 < nk) {
      la.store(nxt);
      lb.store(nxt + kTileBytes);
    }
    __syncthreads();
  }
  const int64_t rs = (int64_t)a.H * a.Hp;
  float* G = (row < a.E ? a.gh + (int64_t)row * rs : a.rb + ((int64_t)d * a.B + row - a.E) * rs) +
             (int64_t)m0 * a.Hp + n0;
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nrow[j] + lr;
      if (n >= nv) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + acc_row(v, lh);
        if (m < mv) {
          float* p = G + (int64_t)m * a.Hp + n;
          *p = __fadd_rn(*p, acc[i][j][v]);
        }
      }
    }
}

int64_t pad_grid(int64_t n) { return (n + kXcds - 1) / kXcds * kXcds; }

}  // namespace

hipError_t launch_ffn(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* x_nvs,
                      const uint16_t* const home[3], const uint16_t* const pool[3], uint16_t* z,
                      uint16_t* y, hipStream_t s) {
  const Dims& d = c.d;
  gemm_schedule<<<d.R, 64, 0, s>>>(p.aux + d.aux.act, p.cu_seqlens, p.seg_tokens, c.tiles,
                                   c.ntiles, 2 * d.L, d.E + d.B, d.tp, c.max_tiles);
  FfnArgs a;
  a.x = x_nvs;
  for (int i = 0; i < 3; ++i) {
    a.home[i] = home[i];
    a.pool[i] = pool[i];
  }
  a.z = z; a.y = y; a.tiles = c.tiles; a.ntiles = c.ntiles;
  a.R = d.R; a.E = d.E; a.B = d.B; a.H = d.H; a.Hp = d.Hp; a.NvS = (int)d.NvS;
  a.max_tiles = c.max_tiles;
  a.rank0 = rank < 0 ? 0 : rank;
  a.nranks = rank < 0 ? d.R : 1;
  a.ntn = (d.Hp + 127) / 128;
  ffn_gateup<<<(unsigned)pad_grid((int64_t)a.nranks * a.max_tiles * a.ntn), kThreads, 0, s>>>(a);
  a.ntn = (d.H + BN - 1) / BN;
  ffn_down<<<(unsigned)pad_grid((int64_t)a.nranks * a.max_tiles * a.ntn), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_wgrad(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* A,
                        const uint16_t* B, float* gh, float* rb, hipStream_t s) {
  const Dims& d = c.d;
  WgradArgs a;
  a.a = A; a.b = B; a.gh = gh; a.rb = rb;
  a.act = p.aux + d.aux.act; a.cu = p.cu_seqlens; a.segn = p.seg_tokens;
  a.R = d.R; a.E = d.E; a.B = d.B; a.H = d.H; a.Hp = d.Hp; a.NvS = (int)d.NvS;
  a.L2 = 2 * d.L; a.EB = d.E + d.B; a.tp = d.tp;
  a.rank0 = rank < 0 ? 0 : rank;
  a.nranks = rank < 0 ? d.R : 1;
  a.ntm = (d.H + BM - 1) / BM;
  a.ntn = (d.Hp + BN - 1) / BN;
  const int64_t total = (int64_t)a.nranks * a.L2 * a.ntm * a.ntn;
  wgrad_kernel<<<(unsigned)pad_grid(total), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moonep
