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
// lane, in AGPRs).  K advances 32 per step through a ring of four 32 KiB LDS
// stages filled by LDS-DMA buffer loads issued three steps ahead (no staging
// registers, no LDS write instructions).  Operands contiguous along K are
// kept as 64-byte rows with an XOR chunk swizzle and read with ds_read_b128;
// operands stored [k][n] (gate/up weights, both weight-gradient operands) are
// kept as 256-byte k-rows and read with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16), which hands each lane one column's 4 consecutive k.
// Fragments are double-buffered in registers and every load and fragment
// read is slotted between MFMAs, so the matrix unit stays busy across the one
// barrier per step.  Buffer descriptors make tile edges branch-free
// (out-of-range loads read zero, out-of-range stores are dropped).
// Workgroup ids are remapped so that every XCD (own L2) works through a
// contiguous range of tiles: neighbouring tiles share weight or activation
// slabs in that XCD's L2.
#include "internal.h"

namespace moonep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 32;        // K advances 32 per step
constexpr int kStages = 4;                        // LDS ring depth
constexpr int kTileBytes = 256 * BK * 2;          // 16 KiB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;       // A tile + B tile
constexpr int kXcds = 8;
constexpr int kLoadsPerStep = 8;                  // LDS-DMA loads per wave per step

typedef __attribute__((address_space(3))) char lds_t;

__device__ __forceinline__ int round_up(int n, int m) { return (n + m - 1) / m * m; }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// Global loads go through buffer resources: an offset past num_records reads
// zero, so tile edges (segment end, matrix edge) need no branches.  The
// descriptor must live in scalar registers; base and size are made provably
// wave-uniform (readfirstlane) so the compiler never wraps a load in a
// per-lane loop over descriptors.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;   // any offset >= num_records reads 0

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)bytes;
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(n),
                                           0x00020000);
}
// 16 bytes per lane straight into LDS (LDS DMA): lane i lands at dst + 16 i.
// Issued through inline assembly so the compiler does not track it: its
// alias tracking cannot tell the four stage arrays apart and would insert a
// wait for every load in flight before LDS reads of other stages.  Every
// consumer is ordered explicitly instead (s_waitcnt vmcnt + barrier per
// step).  The instruction writes no register; its operands are read at
// issue; M0 carries the LDS base as an input operand.
typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));
struct DmaRsrc {
  u32x4s v;
};
__device__ __forceinline__ DmaRsrc make_dma_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)bytes;
  const uint64_t p = (uint64_t)(uintptr_t)base;
  DmaRsrc r;
  r.v[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r.v[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu);   // stride 0
  r.v[2] = __builtin_amdgcn_readfirstlane(n);
  r.v[3] = 0x00020000u;
  return r;
}
__device__ __forceinline__ void load_lds(const DmaRsrc& r, lds_t* dst, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r.v), "{m0}"(m0)
               : "memory");
}
// Stores past num_records are dropped: the epilogues need no branches.
__device__ __forceinline__ void bstore16(Rsrc r, uint32_t voff, unsigned v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, voff, 0, 0);
}

// ---------------------------------------------------------------------------
// Operand tiles in LDS (one per stage and operand, 16 KiB each).
//
// Row tile (operand contiguous along k): 256 rows x 32 k, rows of 64 B; the
// 16-byte chunk c of row r sits at chunk c ^ ((r >> 2) & 3), so the 16 rows
// read by a 16-lane group of an MFMA fragment load hit 16 distinct bank
// groups.  One LDS-DMA load (a wave, 1 KiB) fills 16 rows.
//
// Column tile (operand stored [k][n], n contiguous): two regions of 128
// columns (gate and up weights, or two column halves of one matrix), 32 k
// rows of 256 B each; chunk c of row k sits at chunk c ^ (4 (k & 3)).  One
// LDS-DMA load fills 4 rows of one region.  Fragments are read with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16): lane q of a 16-lane
// group points at row k0 + q/4, columns n0 + 4 (q%4) .. +3, and lane i then
// holds column n0 + i, rows k0 .. k0+3 -- the MFMA operand layout.
struct RowTile {
  static constexpr bool kRows = true;
  DmaRsrc rs;
  uint32_t voff[4];
  // base: row 0, k 0 of the tile; ld: row stride (elements)
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int rows_valid) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    rs = make_dma_rsrc(base, (int64_t)rows_valid * ld * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * (w * 4 + i) + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      voff[i] = r < rows_valid ? (uint32_t)(r * ld * 2 + c * 16) : kOob;
    }
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const { return (uint32_t)(k0 * 2); }
  // load i (0..3) of this wave for the k-block at byte offset ko
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t ko, bool valid) {
    load_lds(rs, tile + (wave_id() * 4 + i) * 1024, valid ? voff[i] + ko : kOob);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue1(tile, i, koff(k0), valid);
  }
  // 8 consecutive k (sub-step kk, lane half lh) of tile row `row`
  __device__ __forceinline__ static bf16x8 frag(const lds_t* tile, int row, int kk, int lh) {
    const int c = (2 * kk + lh) ^ ((row >> 2) & 3);
    return *(const __attribute__((address_space(3))) bf16x8*)(tile + row * 64 + c * 16);
  }
};

struct ColTile {
  static constexpr bool kRows = false;
  DmaRsrc rs0, rs1;
  uint32_t voff[4];
  uint32_t ld2;
  // src0/src1: k 0, n 0 of the two 128-column regions; ld: k stride
  // (elements); k_total: valid k rows from k 0; nv0/nv1: valid columns
  __device__ __forceinline__ void init(const uint16_t* src0, const uint16_t* src1, int64_t ld,
                                       int64_t k_total, int nv0, int nv1) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    rs0 = make_dma_rsrc(src0, k_total * ld * 2);
    rs1 = make_dma_rsrc(src1, k_total * ld * 2);
    ld2 = (uint32_t)(ld * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = w * 4 + i;                       // region b >> 3
      const int k = 4 * (b & 7) + (lane >> 4);
      const int col = 8 * ((lane & 15) ^ (4 * (k & 3)));
      const int nv = (b >> 3) ? nv1 : nv0;
      voff[i] = col < nv ? (uint32_t)(k * ld * 2 + col * 2) : kOob;
    }
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const { return (uint32_t)(k0 * ld2); }
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t ko, bool valid) {
    const int b = wave_id() * 4 + i;
    load_lds((b >> 3) ? rs1 : rs0, tile + b * 1024, valid ? voff[i] + ko : kOob);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue1(tile, i, koff(k0), valid);
  }
  // 8 consecutive k (sub-step kk, lane half lh) of tile column n (the lane's)
  __device__ __forceinline__ static bf16x8 frag(const lds_t* tile, int nb, int kk, int lh) {
    const int lane = threadIdx.x & 63, q = lane & 15, g = (lane >> 4) & 1;
    const lds_t* region = tile + (nb >> 7) * 8192;
    const int col = (nb & 127) + 16 * g + 4 * (q & 3);
    i16x4 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = 16 * kk + 8 * lh + 4 * hh + (q >> 2);
      const int off = k * 256 + (((col >> 3) ^ (4 * (k & 3))) << 4) + (col & 7) * 2;
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(region + off));
    }
    const i16x8 v = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
};

// MFMA fragments of one 16-deep sub-step for a wave: A rows arow0 + 32 i,
// B columns nrow[j] (+ lane%32).
struct Frags {
  bf16x8 a[4], b[4];
};

// Fragment q of a sub-step, in the order the MFMAs consume them: A0, B0..B3,
// A1..A3 (the MFMAs run i-major, so A0 and all of B are needed first).
template <class TA, class TB>
__device__ __forceinline__ void read_frag(Frags& f, int q, const lds_t* stage, int kk, int arow0,
                                          const int nrow[4]) {
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const lds_t* A = stage;
  const lds_t* Bt = stage + kTileBytes;
  if (q == 0 || q >= 5) {
    const int i = q == 0 ? 0 : q - 4;
    f.a[i] = TA::kRows ? RowTile::frag(A, arow0 + i * 32 + lr, kk, lh)
                       : ColTile::frag(A, arow0 + i * 32, kk, lh);
  } else {
    const int j = q - 1;
    f.b[j] = TB::kRows ? RowTile::frag(Bt, nrow[j] + lr, kk, lh)
                       : ColTile::frag(Bt, nrow[j], kk, lh);
  }
}

template <class TA, class TB>
__device__ __forceinline__ void read_frags(Frags& f, const lds_t* stage, int kk, int arow0,
                                           const int nrow[4]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) read_frag<TA, TB>(f, q, stage, kk, arow0, nrow);
}

__device__ __forceinline__ void mma1(f32x16 acc[4][4], const Frags& f, int idx) {
  const int i = idx >> 2, j = idx & 3;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Wait until at most N LDS-DMA loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else static_assert(N == 0, "unsupported count");
}

// Workgroup barrier without the LDS wait that __syncthreads() implies:
// fragment reads issued just before it stay in flight (their consumers wait
// for them).  The memory clobber keeps every LDS access on its side.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

#define MOONEP_PIN() __builtin_amdgcn_sched_barrier(0)

// The four LDS stages are four separate arrays and the K loop is unrolled by
// four, so every LDS access names its stage statically.
struct Stages {
  lds_t* p[kStages];
};

#define MOONEP_STAGE_ARRAYS(name)                                           \
  __shared__ __attribute__((aligned(16))) char name##0_[kStageBytes];      \
  __shared__ __attribute__((aligned(16))) char name##1_[kStageBytes];      \
  __shared__ __attribute__((aligned(16))) char name##2_[kStageBytes];      \
  __shared__ __attribute__((aligned(16))) char name##3_[kStageBytes];      \
  const Stages name = {{(lds_t*)name##0_, (lds_t*)name##1_, (lds_t*)name##2_, (lds_t*)name##3_}}

// One 32-deep step kt, held in stage S = kt % 4, as two runs of 16 MFMAs with
// every other instruction slotted between them (an MFMA occupies the matrix
// unit for 8 issue cycles of its wave, which covers a load's address
// arithmetic and issue):
//   run 1: MFMAs on f0 (sub-step 0); between the first eight, the eight
//          fragment reads of sub-step 1 (stage S) into f1;
//   wait for this wave's loads of step kt+1, barrier (every wave's loads of
//          step kt+1 have landed; every wave is done reading step kt-1);
//   run 2: MFMAs on f1; between the first eight, the eight LDS-DMA loads of
//          step kt+3 into stage (S+3)%4 and the fragment reads of step kt+1's
//          sub-step 0 (stage S+1) into f0.
// Loads past the last step use an out-of-range offset (they read nothing and
// keep the wait counts fixed).
template <int S, class TA, class TB>
__device__ __forceinline__ void kstep(TA& la, TB& lb, const Stages& st, int kt, int nk,
                                      Frags& f0, Frags& f1, f32x16 acc[4][4], int arow0,
                                      const int nrow[4]) {
  constexpr int N = (S + 1) % kStages, L = (S + kStages - 1) % kStages;
  MOONEP_PIN();
#pragma unroll
  for (int idx = 0; idx < 16; ++idx) {
    mma1(acc, f0, idx);
    if (idx < 8) read_frag<TA, TB>(f1, idx, st.p[S], 1, arow0, nrow);
    MOONEP_PIN();
  }
  wait_loads<kLoadsPerStep>();
  barrier_only();
  MOONEP_PIN();
  const int nx = kt + kStages - 1;
  const bool valid = nx < nk;
  const uint32_t koa = la.koff((int64_t)nx * BK), kob = lb.koff((int64_t)nx * BK);
#pragma unroll
  for (int idx = 0; idx < 16; ++idx) {
    mma1(acc, f1, idx);
    if (idx < 8) {
      if (idx < 4) la.issue1(st.p[L], idx, koa, valid);
      else lb.issue1(st.p[L] + kTileBytes, idx - 4, kob, valid);
      read_frag<TA, TB>(f0, idx, st.p[N], 0, arow0, nrow);
    }
    MOONEP_PIN();
  }
}

// The K loop shared by every GEMM here: a ring of 4 LDS stages filled by
// LDS-DMA loads issued 3 steps ahead (no staging registers, no LDS write
// instructions), one barrier per step.  The step count is rounded up to a
// multiple of 4 so the loop has no remainder: the extra steps load nothing
// (out-of-range offsets fill their stages with zeros) and add zero products.
template <class TA, class TB>
__device__ __forceinline__ void gemm_loop(TA& la, TB& lb, const Stages& st, int nk,
                                          f32x16 acc[4][4], int arow0, const int nrow[4]) {
  if (nk <= 0) return;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    la.issue(st.p[s], (int64_t)s * BK, s < nk);
    lb.issue(st.p[s] + kTileBytes, (int64_t)s * BK, s < nk);
  }
  wait_loads<2 * kLoadsPerStep>();
  barrier_only();
  Frags f0, f1;
  read_frags<TA, TB>(f0, st.p[0], 0, arow0, nrow);
  const int nk4 = (nk + kStages - 1) / kStages * kStages;
  for (int kt = 0; kt < nk4; kt += kStages) {
    kstep<0>(la, lb, st, kt + 0, nk, f0, f1, acc, arow0, nrow);
    kstep<1>(la, lb, st, kt + 1, nk, f0, f1, acc, arow0, nrow);
    kstep<2>(la, lb, st, kt + 2, nk, f0, f1, acc, arow0, nrow);
    kstep<3>(la, lb, st, kt + 3, nk, f0, f1, acc, arow0, nrow);
  }
  wait_loads<0>();
  // every wave is past its last fragment read before the stages are reused
  __syncthreads();
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
  const uint16_t* x;        // [R*NvS][H] (gate/up input)
  const uint16_t* home[3];  // [E][H][Hp]
  const uint16_t* pool[3];  // [R*B][H][Hp]
  uint16_t* z;              // [R*NvS][Hp] (gate/up output)
  const uint16_t* zin;      // [R*NvS][Hp] (down input)
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
// One workgroup of 256 threads per rank: thread q takes active row q, counts
// its M-tiles, a block-wide exclusive scan places them, and the thread writes
// its tiles.
__global__ __launch_bounds__(256) void gemm_schedule(const int32_t* act, const int32_t* cu,
                                                     const int32_t* segn, int32_t* tiles,
                                                     int32_t* ntiles, int L2, int EB, int tp,
                                                     int max_tiles) {
  __shared__ int wsum[4];
  __shared__ int s_total;
  const int d = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int base = 0;
  for (int q0 = 0; q0 < L2; q0 += 256) {
    const int q = q0 + tid;
    const int row = q < L2 ? act[d * L2 + q] : -1;
    int end = 0, len = 0, n = 0;
    if (row >= 0) {
      end = cu[d * EB + row];
      len = round_up(segn[d * EB + row], tp);
      n = (len + BM - 1) / BM;
    }
    int x = n;                                   // inclusive scan within the wave
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < wv; ++i) before += wsum[i];
    if (tid == 255) s_total = before + x;
    int t = base + before + x - n;
    for (int m = end - len; m < end; m += BM, ++t) {
      if (t >= max_tiles) break;
      int32_t* e = tiles + ((int64_t)d * max_tiles + t) * 4;
      e[0] = row;
      e[1] = m;
      e[2] = m + BM < end ? m + BM : end;
      e[3] = 0;
    }
    __syncthreads();
    base += s_total;
    __syncthreads();
  }
  if (tid == 0) ntiles[d] = base < max_tiles ? base : max_tiles;
}

// ---------------------------------------------------------------------------
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void ffn_gateup(FfnArgs a) {
  MOONEP_STAGE_ARRAYS(smem);
  int d, nt;
  Tile tl;
  if (!decode(a, &d, &tl, &nt)) return;
  const int n0 = nt * 128;
  const int rows_valid = tl.m1 - tl.m0;
  const int nvh = a.Hp - n0 < 128 ? a.Hp - n0 : 128;   // valid columns of each half
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 64, wn * 64 + 32, 128 + wn * 64, 128 + wn * 64 + 32};

  RowTile la;
  ColTile lb;
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
  MOONEP_STAGE_ARRAYS(smem);
  int d, nt;
  Tile tl;
  if (!decode(a, &d, &tl, &nt)) return;
  const int n0 = nt * BN;
  const int rows_valid = tl.m1 - tl.m0;
  const int cols_valid = a.H - n0 < BN ? a.H - n0 : BN;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int nrow[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  RowTile la, lb;
  la.init(a.zin + ((int64_t)d * a.NvS + tl.m0) * a.Hp, a.Hp, rows_valid);
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
  MOONEP_STAGE_ARRAYS(smem);
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

  ColTile la, lb;
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

static FfnArgs ffn_args(const Ctx& c, const moonep_plan_t& p, int rank,
                        const uint16_t* const home[3], const uint16_t* const pool[3]) {
  const Dims& d = c.d;
  FfnArgs a;
  for (int i = 0; i < 3; ++i) {
    a.home[i] = home[i];
    a.pool[i] = pool[i];
  }
  a.x = nullptr; a.z = nullptr; a.zin = nullptr; a.y = nullptr;
  a.tiles = p.aux + d.aux.tiles; a.ntiles = p.aux + d.aux.ntiles;
  a.R = d.R; a.E = d.E; a.B = d.B; a.H = d.H; a.Hp = d.Hp; a.NvS = (int)d.NvS;
  a.max_tiles = d.max_tiles;
  a.rank0 = rank < 0 ? 0 : rank;
  a.nranks = rank < 0 ? d.R : 1;
  a.ntn = 0;
  return a;
}

hipError_t launch_gemm_schedule(const Ctx& c, const moonep_plan_t& p, hipStream_t s) {
  const Dims& d = c.d;
  gemm_schedule<<<d.R, 256, 0, s>>>(p.aux + d.aux.act, p.cu_seqlens, p.seg_tokens,
                                   p.aux + d.aux.tiles, p.aux + d.aux.ntiles, 2 * d.L,
                                   d.E + d.B, d.tp, d.max_tiles);
  return hipGetLastError();
}

hipError_t launch_gateup(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* x_nvs,
                         const uint16_t* const home[3], const uint16_t* const pool[3],
                         uint16_t* z, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, home, pool);
  a.x = x_nvs;
  a.z = z;
  a.ntn = (c.d.Hp + 127) / 128;
  ffn_gateup<<<(unsigned)pad_grid((int64_t)a.nranks * a.max_tiles * a.ntn), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* z,
                       const uint16_t* const home[3], const uint16_t* const pool[3],
                       uint16_t* y, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, home, pool);
  a.zin = z;
  a.y = y;
  a.ntn = (c.d.H + BN - 1) / BN;
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
