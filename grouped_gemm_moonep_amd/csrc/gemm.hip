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
// lane).  K advances 64 per step through two 72 KiB LDS stages (A rows and
// B^T rows of 64 k, padded to 144 B so that MFMA fragment reads are
// bank-conflict free).  Global loads are buffer loads
// (out-of-range offsets read zero: no branches at tile edges), issued one
// step ahead into registers; fragments are double-buffered in registers so
// LDS latency hides behind MFMAs; one barrier per step.  Operands whose
// contraction index is not contiguous in memory (gate/up weights, both wgrad
// operands) are transposed 8x8 in registers (v_perm) on their way into LDS.
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
// LDS tile rows hold 64 k (128 B) padded to 144 B: 16 consecutive rows then
// start in 16 different 16-byte bank groups, so the MFMA fragment reads (16
// rows per 16-lane group) are conflict-free, and every address is a
// per-thread base plus a compile-time offset.
constexpr int kRowBytes = 144;
constexpr int kTileBytes = 256 * kRowBytes;       // 36 KiB
constexpr int kStageBytes = 2 * kTileBytes;       // A tile + B^T tile
constexpr int kXcds = 8;

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kRowBytes + chunk * 16; }

__device__ __forceinline__ int round_up(int n, int m) { return (n + m - 1) / m * m; }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Global loads go through buffer resources: an offset past num_records
// returns zeros, so tile edges (segment end, matrix edge) need no branches.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;   // any offset >= num_records reads 0

// The descriptor must live in scalar registers; base and size are made
// provably wave-uniform (readfirstlane) so the compiler never wraps a load in
// a per-lane loop over descriptors.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)bytes;
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(n),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
// Stores past num_records are dropped: the epilogues need no branches.
__device__ __forceinline__ void bstore16(Rsrc r, uint32_t voff, unsigned v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, voff, 0, 0);
}

// Loader for an operand whose contraction index is contiguous: 256 tile rows
// x 64 k.  Thread t covers chunk t%8 (8 k) of rows t/8 + 32 i.
struct DirectTile {
  static constexpr int kCommitValu = 0;   // VALU per LDS write in commit()
  Rsrc rs;
  uint32_t voff[8];
  u32x4 v[8];
  // base: row 0, k 0 of the tile; ld: row stride (elements)
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int rows_valid) {
    const int t = threadIdx.x, c = t & 7;
    rs = make_rsrc(base, (int64_t)rows_valid * ld * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (t >> 3) + 32 * i;
      voff[i] = r < rows_valid ? (uint32_t)(r * ld * 2 + c * 16) : kOob;
    }
  }
  // the whole offset goes in the VGPR operand: the hardware range check
  // covers that operand, not the scalar offset
  __device__ __forceinline__ void issue(int64_t k0) {
    const uint32_t ko = (uint32_t)(k0 * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bload(rs, voff[i] + ko, 0);
  }
  __device__ __forceinline__ void commit(char* tile) const {
    const int t = threadIdx.x, c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)(tile + lds_off((t >> 3) + 32 * i, c)) = v[i];
  }
};

// Loader for an operand stored [k][n] (n contiguous): 64 k x 256 tile rows
// (n).  Threads 0-127 fill tile rows [0,128) from src0, threads 128-255 rows
// [128,256) from src1 (the gate and the up weights side by side, or two
// column halves of one matrix), so every wave reads one matrix.  Thread t
// covers k-block t%8 (8 k) and n-chunk (t/8)%16 (8 n); the 8x8 block is
// transposed in registers so that each tile row holds 8 consecutive k.  With
// k-blocks varying fastest, each 16-lane group of a transposed LDS write
// covers 16 different bank groups.
struct TransTile {
  static constexpr int kCommitValu = 2;   // v_perm per LDS write (4 per 8, 2 loaders)
  Rsrc rs;
  uint32_t voff[8];
  uint32_t ld2;
  u32x4 v[8];
  // src0/src1: k 0, n 0 of each half; ld: k stride (elements); k_total: valid
  // k rows from k 0; nv0/nv1: valid columns of each half
  __device__ __forceinline__ void init(const uint16_t* src0, const uint16_t* src1, int64_t ld,
                                       int64_t k_total, int nv0, int nv1) {
    const int t = threadIdx.x, half = t >> 7;
    const int kb = t & 7, n = ((t >> 3) & 15) * 8;
    const uint16_t* src = half ? src1 : src0;
    const int nv = half ? nv1 : nv0;
    rs = make_rsrc(src, k_total * ld * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kb * 8 + i;
      voff[i] = n < nv ? (uint32_t)(k * ld * 2 + n * 2) : kOob;
    }
    ld2 = (uint32_t)(ld * 2);
  }
  __device__ __forceinline__ void issue(int64_t k0) {
    const uint32_t ko = (uint32_t)(k0 * ld2);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bload(rs, voff[i] + ko, 0);
  }
  __device__ __forceinline__ void commit(char* tile) const {
    const int t = threadIdx.x, half = t >> 7;
    const int kb = t & 7, c = (t >> 3) & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sel = (j & 1) ? 0x07060302 : 0x05040100;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = __builtin_amdgcn_perm(v[2 * q + 1][j >> 1], v[2 * q][j >> 1], sel);
      *(u32x4*)(tile + lds_off(half * 128 + c * 8 + j, kb)) = o;
    }
  }
};

// MFMA fragments of one 16-deep sub-step for a wave: A rows arow0 + 32 i,
// B^T rows nrow[j] (+ lane%32), k-chunk 2 kk + lane/32.
struct Frags {
  bf16x8 a[4], b[4];
};

__device__ __forceinline__ void read_frags(Frags& f, const char* stage, int kk, int arow0,
                                           const int nrow[4]) {
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const char* A = stage;
  const char* Bt = stage + kTileBytes;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *(const bf16x8*)(A + lds_off(arow0 + i * 32 + lr, 2 * kk + lh));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = *(const bf16x8*)(Bt + lds_off(nrow[j] + lr, 2 * kk + lh));
}

__device__ __forceinline__ void mma16(f32x16 acc[4][4], const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Scheduling groups (LLVM AMDGPU sched_group_barrier masks).
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgDsRead = 0x100, kSgDsWrite = 0x200;
#define MOONEP_SG(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// One sub-step: 8 fragment reads for the next sub-step, then 16 MFMAs on the
// current fragments (the reads' latency hides behind the MFMAs).
#define MOONEP_SUBSTEP()      \
  do {                        \
    MOONEP_SG(kSgDsRead, 8);  \
    MOONEP_SG(kSgMfma, 16);   \
    __builtin_amdgcn_sched_barrier(0); \
  } while (0)

// The K loop shared by every GEMM here.  Two LDS stages; per 64-deep step:
// the next step's global loads are issued first; sub-steps 0-2 each read the
// following sub-step's fragments while 16 MFMAs run; during sub-step 2 the
// loaded tiles are transposed / written to the other stage, interleaved one
// LDS write per MFMA; one barrier; sub-step 3's MFMAs cover the read of the
// next step's first fragments.  Scheduling barriers pin this order (left
// alone, the compiler sinks the loads next to their consumers and exposes the
// memory latency).  The last step is peeled.
template <class TA, class TB>
__device__ __forceinline__ void gemm_loop(TA& la, TB& lb, char* smem, int nk, f32x16 acc[4][4],
                                          int arow0, const int nrow[4]) {
  if (nk <= 0) return;
  la.issue(0);
  lb.issue(0);
  la.commit(smem);
  lb.commit(smem + kTileBytes);
  __syncthreads();
  Frags f0, f1;
  read_frags(f0, smem, 0, arow0, nrow);
  int kt = 0;
  for (; kt + 1 < nk; ++kt) {
    char* cur = smem + (kt & 1) * kStageBytes;
    char* nxt = smem + ((kt + 1) & 1) * kStageBytes;
    __builtin_amdgcn_sched_barrier(0);
    la.issue((int64_t)(kt + 1) * BK);
    lb.issue((int64_t)(kt + 1) * BK);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(f1, cur, 1, arow0, nrow);
    mma16(acc, f0);
    MOONEP_SUBSTEP();
    read_frags(f0, cur, 2, arow0, nrow);
    mma16(acc, f1);
    MOONEP_SUBSTEP();
    read_frags(f1, cur, 3, arow0, nrow);
    mma16(acc, f0);
    la.commit(nxt);
    lb.commit(nxt + kTileBytes);
    MOONEP_SG(kSgDsRead, 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      MOONEP_SG(kSgValu, TA::kCommitValu + TB::kCommitValu);
      MOONEP_SG(kSgDsWrite, 1);
      MOONEP_SG(kSgMfma, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_frags(f0, nxt, 0, arow0, nrow);
    mma16(acc, f1);
    MOONEP_SUBSTEP();
  }
  char* cur = smem + (kt & 1) * kStageBytes;
  read_frags(f1, cur, 1, arow0, nrow);
  mma16(acc, f0);
  read_frags(f0, cur, 2, arow0, nrow);
  mma16(acc, f1);
  read_frags(f1, cur, 3, arow0, nrow);
  mma16(acc, f0);
  mma16(acc, f1);
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

// Within a rank, tiles are taken in groups of kGroupM M-tiles: the group's
// M-tiles for the first N-tile, then for the second, ...  Workgroups that run
// together on an XCD (32 CUs) then cover kGroupM M-tiles x 32/kGroupM
// N-tiles, so each weight slab in that XCD's L2 serves kGroupM workgroups and
// each activation slab 32/kGroupM.
constexpr int kGroupM = 4;

__device__ __forceinline__ bool decode(const FfnArgs& a, int* d, Tile* tl, int* nt) {
  const int64_t lt = logical_tile();
  const int64_t per_rank = (int64_t)a.max_tiles * a.ntn;
  const int64_t total = (int64_t)a.nranks * per_rank;
  if (lt >= total) return false;
  *d = a.rank0 + (int)(lt / per_rank);
  const int l = (int)(lt % per_rank);
  const int group = l / (kGroupM * a.ntn);
  const int gm = min(kGroupM, a.max_tiles - group * kGroupM);   // M-tiles in this group
  const int rem = l - group * kGroupM * a.ntn;
  *nt = rem / gm;
  const int t = group * kGroupM + rem % gm;
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
  const int nvh = a.Hp - n0 < 128 ? a.Hp - n0 : 128;   // valid columns of each half
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 64, wn * 64 + 32, 128 + wn * 64, 128 + wn * 64 + 32};

  DirectTile la;
  TransTile lb;
  la.init(a.x + ((int64_t)d * a.NvS + tl.m0) * a.H, a.H, rows_valid);
  lb.init(weight_row(a, 0, d, tl.row) + n0, weight_row(a, 1, d, tl.row) + n0, a.Hp, a.H, nvh,
          nvh);
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_loop(la, lb, smem, a.H / BK, acc, wm * 128, nrow);

  // SwiGLU epilogue: blocks j = 0,1 are gate, j = 2,3 the matching up.
  // Rows past the segment fall outside the store range; columns past H' get
  // an out-of-range offset.
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const Rsrc zs = make_rsrc(a.z + ((int64_t)d * a.NvS + tl.m0) * a.Hp + n0,
                            (int64_t)rows_valid * a.Hp * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * 64 + j * 32 + lr;
      const uint32_t col = n < nvh ? (uint32_t)(n * 2) : kOob;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + acc_row(v, lh);
        const float g = acc[i][j][v], u = acc[i][j + 2][v];
        const float zz = g / (1.0f + __expf(-g)) * u;
        bstore16(zs, col + (uint32_t)(m * a.Hp * 2), bf16_rne(zz));
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
  const int cols_valid = a.H - n0 < BN ? a.H - n0 : BN;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  DirectTile la, lb;
  la.init(a.z + ((int64_t)d * a.NvS + tl.m0) * a.Hp, a.Hp, rows_valid);
  lb.init(weight_row(a, 2, d, tl.row) + (int64_t)n0 * a.Hp, a.Hp, cols_valid);
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_loop(la, lb, smem, a.Hp / BK, acc, wm * 128, nrow);

  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const Rsrc ys = make_rsrc(a.y + ((int64_t)d * a.NvS + tl.m0) * a.H + n0,
                            (int64_t)rows_valid * a.H * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nrow[j] + lr;
      const uint32_t col = n < cols_valid ? (uint32_t)(n * 2) : kOob;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + acc_row(v, lh);
        bstore16(ys, col + (uint32_t)(m * a.H * 2), bf16_rne(acc[i][j][v]));
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

  TransTile la, lb;
  la.init(A, A + 128, a.H, ntok, mv0, mv1);
  lb.init(Bm, Bm + 128, a.Hp, ntok, nv0, nv1);
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_loop(la, lb, smem, (ntok + BK - 1) / BK, acc, wm * 128, nrow);

  // fp32 read-modify-write; rows past H and columns past H' are out of range
  const int64_t rs = (int64_t)a.H * a.Hp;
  float* G = (row < a.E ? a.gh + (int64_t)row * rs : a.rb + ((int64_t)d * a.B + row - a.E) * rs) +
             (int64_t)m0 * a.Hp + n0;
  const Rsrc gs = make_rsrc(G, (int64_t)mv * a.Hp * 4);
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nrow[j] + lr;
      const uint32_t col = n < nv ? (uint32_t)(n * 4) : kOob;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + acc_row(v, lh);
        const uint32_t off = col + (uint32_t)(m * a.Hp * 4);
        const float old = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gs, off, 0, 0));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, __fadd_rn(old, acc[i][j][v])),
                                              gs, off, 0, 0);
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
