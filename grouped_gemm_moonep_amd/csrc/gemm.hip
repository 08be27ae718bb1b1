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
// lane, in AGPRs).  K advances 64 per step.  Operand tiles (256 x 64 bf16,
// 32 KiB) rotate through a ring of five LDS slots (160 KiB) filled by LDS-DMA
// buffer loads (no staging registers, no LDS write instructions); weights are
// fetched two steps ahead, activations one.  Operands contiguous along K are
// kept as 128-byte rows (whole cache lines per load) with an XOR chunk
// swizzle and read with ds_read_b128; operands stored [k][n] (gate/up
// weights, both weight-gradient operands) are kept as 256-byte k-rows and read
// with the gfx950 transposing LDS read (ds_read_b64_tr_b16), which hands each
// lane one column's 4 consecutive k.  Fragments are double-buffered in
// registers and every load and fragment read is slotted between MFMAs, so the
// matrix unit stays busy across the one barrier per step.  Buffer descriptors
// make tile edges branch-free (out-of-range loads read zero, out-of-range
// stores are dropped).  Workgroup ids are remapped so that every XCD (own L2)
// works through a contiguous range of tiles: neighbouring tiles share weight
// or activation slabs in that XCD's L2.
#include "internal.h"

namespace moonep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 64;        // K advances 64 per step
constexpr int kHalfTileM = 128;                   // rows of a segment's short last tile
constexpr int kXcds = 8;
constexpr int kLoadsPerStep = 8;                  // LDS-DMA loads per wave per tile and step
constexpr int kTileOffB = 0;                      // B tile offset inside its slot

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
// Operand tiles in LDS: 256 rows (or columns) x 64 k of bf16 = 32 KiB, one
// per ring slot.
//
// Row tile (operand contiguous along k): rows of 128 B (64 k); the 16-byte
// chunk c of row r sits at position c ^ (r & 7), so the 8 rows read together
// by an MFMA fragment load hit 8 distinct bank groups.  One LDS-DMA load (a
// wave, 1 KiB) fills 8 rows, each a whole 128-byte cache line: the L1/L2 path
// costs per cache line touched, and half-line rows would halve its rate.
//
// Column tile (operand stored [k][n], n contiguous): two regions of 128
// columns (gate and up weights, or two column halves of one matrix), 64 k
// rows of 256 B each; chunk c of row k sits at position c ^ (4 (k & 3)).  One
// LDS-DMA load fills 4 rows of one region.  Fragments are read with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16): lane q of a 16-lane
// group points at row k0 + q/4, columns n0 + 4 (q%4) .. +3, and lane i then
// holds column n0 + i, rows k0 .. k0+3 -- the MFMA operand layout.
constexpr int kSlotBytes = 256 * BK * 2;          // 32 KiB
constexpr int kSlots = 5;                         // 160 KiB ring

template <int NL>          // loads per wave per step: the tile has 32 NL rows
struct RowTileT {
  static constexpr bool kRows = true;
  static constexpr int kLoads = NL;
  DmaRsrc rs;
  uint32_t voff;        // this lane's offset for load 0 of k-block 0
  uint32_t step;        // byte distance between consecutive loads of a wave (8 rows)
  // base: row 0, k 0 of the tile; ld: row stride (elements).  Rows at or
  // past rows_valid lie outside the descriptor's range and read zero.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int rows_valid) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    rs = make_dma_rsrc(base, (int64_t)rows_valid * ld * 2);
    const int r = 8 * NL * w + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    voff = (uint32_t)(r * ld * 2 + c * 16);
    step = (uint32_t)(16 * ld);
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const { return (uint32_t)(k0 * 2); }
  // load i (0..NL-1) of this wave for the k-block at byte offset ko
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t ko, bool valid) const {
    const uint32_t s = __builtin_amdgcn_readfirstlane(valid ? ko + (uint32_t)i * step : kOob);
    load_lds(rs, tile + (wave_id() * NL + i) * 1024, voff + s);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) issue1(tile, i, koff(k0), valid);
  }
  // 8 consecutive k (sub-step kk of 4, lane half lh) of tile row `row`
  __device__ __forceinline__ static bf16x8 frag(const lds_t* tile, int row, int kk, int lh) {
    const int c = (2 * kk + lh) ^ (row & 7);
    return *(const __attribute__((address_space(3))) bf16x8*)(tile + row * 128 + c * 16);
  }
};
typedef RowTileT<8> RowTile;      // 256 rows

// Row tile whose K range is the concatenation of two matrices: k < k1 from
// the first, k >= k1 from the second (both with the same rows).  koff passes
// the element index through; each load picks its source (a wave-uniform
// choice).
template <int NL>
struct RowTile2 {
  static constexpr bool kRows = true;
  static constexpr int kLoads = NL;
  RowTileT<NL> t0, t1;
  uint32_t k1;
  __device__ __forceinline__ void init(const uint16_t* base0, const uint16_t* base1, int64_t ld,
                                       int rows_valid, int k_first) {
    t0.init(base0, ld, rows_valid);
    t1.init(base1, ld, rows_valid);
    k1 = (uint32_t)k_first;
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const { return (uint32_t)k0; }
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t k, bool valid) const {
    if (k < k1) t0.issue1(tile, i, t0.koff(k), valid);
    else t1.issue1(tile, i, t1.koff(k - k1), valid);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) issue1(tile, i, koff(k0), valid);
  }
  __device__ __forceinline__ static bf16x8 frag(const lds_t* tile, int row, int kk, int lh) {
    return RowTileT<NL>::frag(tile, row, kk, lh);
  }
};

struct ColTile {
  static constexpr bool kRows = false;
  static constexpr int kLoads = 8;
  DmaRsrc rs;           // this wave's region (waves 0,1: region 0; waves 2,3: region 1)
  uint32_t voff;        // this lane's offset for load 0 of k-block 0 (out of range past nv)
  uint32_t ld2;
  // src0/src1: k 0, n 0 of the two 128-column regions; ld: k stride
  // (elements); k_total: valid k rows from k 0; nv0/nv1: valid columns
  __device__ __forceinline__ void init(const uint16_t* src0, const uint16_t* src1, int64_t ld,
                                       int64_t k_total, int nv0, int nv1) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int region = w >> 1;
    rs = make_dma_rsrc(region ? src1 : src0, k_total * ld * 2);
    ld2 = (uint32_t)(ld * 2);
    const int k = 32 * (w & 1) + (lane >> 4);        // load i adds 4 i rows
    const int col = 8 * ((lane & 15) ^ (4 * (k & 3)));
    voff = col < (region ? nv1 : nv0) ? (uint32_t)(k * ld * 2 + col * 2) : kOob;
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const { return (uint32_t)(k0 * ld2); }
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t ko, bool valid) const {
    const uint32_t s = __builtin_amdgcn_readfirstlane(valid ? ko + (uint32_t)(4 * i) * ld2 : kOob);
    load_lds(rs, tile + (wave_id() * 8 + i) * 1024, voff + s);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) issue1(tile, i, koff(k0), valid);
  }
  // 8 consecutive k (sub-step kk of 4, lane half lh) of tile column n (the lane's)
  __device__ __forceinline__ static bf16x8 frag(const lds_t* tile, int nb, int kk, int lh) {
    const int lane = threadIdx.x & 63, q = lane & 15, g = (lane >> 4) & 1;
    const lds_t* region = tile + (nb >> 7) * 16384;
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

// MFMA fragments of one 16-deep sub-step for a wave: A rows arow0 + 32 i
// (i < MI), B columns nrow[j] (+ lane%32).
template <int MI>
struct Frags {
  bf16x8 a[MI], b[4];
};

// Fragment q (< MI + 4) of a sub-step, in the order the MFMAs consume them:
// A0, B0..B3, A1..A(MI-1) (the MFMAs run i-major, so A0 and all of B are
// needed first).
template <int MI, class TA, class TB>
__device__ __forceinline__ void read_frag(Frags<MI>& f, int q, const lds_t* A, const lds_t* Bt,
                                          int kk, int arow0, const int nrow[4]) {
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  if (q == 0 || q >= 5) {
    const int i = q == 0 ? 0 : q - 4;
    f.a[i] = TA::kRows ? TA::frag(A, arow0 + i * 32 + lr, kk, lh)
                       : ColTile::frag(A, arow0 + i * 32, kk, lh);
  } else {
    const int j = q - 1;
    f.b[j] = TB::kRows ? TB::frag(Bt, nrow[j] + lr, kk, lh)
                       : ColTile::frag(Bt, nrow[j], kk, lh);
  }
}

// acc[i][j] accumulates the 32x32 block (A rows arow0+32i.., B columns
// nrow[j]..) transposed: the B fragment is the MFMA's first operand, so lane
// (lr, lh) holds, in element v, output row arow0 + 32 i + lr and output column
// nrow[j] + 8 (v/4) + 4 lh + v%4 -- four consecutive columns of one row per
// v/4, which the epilogues store as one 8- or 16-byte piece.
template <int MI>
__device__ __forceinline__ void mma1(f32x16 acc[MI][4], const Frags<MI>& f, int idx) {
  const int i = idx >> 2, j = idx & 3;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Wait until at most N LDS-DMA loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else static_assert(N == 0, "unsupported count");
}

// Workgroup barrier after this wave's LDS reads have completed (it writes no
// LDS itself: other waves may then overwrite what it read).  Fragment
// registers already loaded are not waited for again.
__device__ __forceinline__ void barrier_reads_done() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define MOONEP_PIN() __builtin_amdgcn_sched_barrier(0)

// The ring: kSlots slots of 32 KiB; step j's A tile sits in slot (2j+1) % 5,
// its B tile in slot 2j % 5.  Hence A(j) reuses the slot of B(j-2) and B(j)
// the slot of A(j-3): B tiles (weights) are loaded two steps ahead, A tiles
// one step ahead.  The K loop is unrolled over the ring period, so every slot
// address is a constant.
struct Ring {
  lds_t* base;
  template <int J>
  __device__ __forceinline__ lds_t* a() const { return base + ((2 * J + 1) % kSlots) * kSlotBytes; }
  template <int J>
  __device__ __forceinline__ lds_t* b() const { return base + ((2 * J) % kSlots) * kSlotBytes; }
};

#define MOONEP_RING(name)                                                          \
  __shared__ __attribute__((aligned(16))) char name##_[kSlots * kSlotBytes];       \
  const Ring name = {(lds_t*)name##_}

// One 64-deep step j (J = j mod 5) = 16 MI MFMAs per wave in four 16-deep
// sub-steps of 4 MI, with every other instruction slotted between MFMAs (an
// MFMA occupies the matrix unit for 8 issue cycles of its wave):
//   sub-steps 0..2 read the next sub-step's fragments while computing;
//   the loads of A(j+1) go out after MFMAs 1, 4, 7, ... and then the 8 loads
//   of B(j+2), spread over the rest of the step up to the barrier;
//   after MFMA P-9 (P = 16 MI): wait for A(j+1) and B(j+1) (the 8 most
//   recent loads are B(j+2)'s), wait for this wave's LDS reads, barrier;
//   the last 8 MFMAs read step j+1's first fragments.
// The barrier orders, for every wave, all reads of step j before any load
// issued after it, and the arrival of step j+1's tiles before any read of
// them.  A(j+2) then reuses B(j)'s slot and B(j+3) reuses A(j)'s.
template <int J, int MI, class TA, class TB>
__device__ __forceinline__ void kstep(const TA& la, const TB& lb, const Ring& ring, int j, int nk,
                                      Frags<MI>& f0, Frags<MI>& f1, f32x16 acc[MI][4], int arow0,
                                      const int nrow[4]) {
  constexpr int J1 = (J + 1) % kSlots, J2 = (J + 2) % kSlots;
  constexpr int P = 16 * MI, SUB = 4 * MI, NF = MI + 4;
  constexpr int NA = TA::kLoads, NB = TB::kLoads;
  constexpr int BAR = P - 9;                       // barrier after this MFMA
  constexpr int B0 = 3 * NA;                       // first B load position
  constexpr int BS = (BAR - B0) / NB > 0 ? (BAR - B0) / NB : 1;
  static_assert(B0 + BS * (NB - 1) <= BAR, "loads must precede the barrier");
  const lds_t* A = ring.a<J>();
  const lds_t* Bt = ring.b<J>();
  const lds_t* An = ring.a<J1>();
  const lds_t* Bn = ring.b<J1>();
  lds_t* la_dst = ring.a<J1>();
  lds_t* lb_dst = ring.b<J2>();
  const uint32_t koa = la.koff((int64_t)(j + 1) * BK), kob = lb.koff((int64_t)(j + 2) * BK);
  const bool va = j + 1 < nk, vb = j + 2 < nk;
  MOONEP_PIN();
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int sub = p / SUB, idx = p % SUB;
    mma1<MI>(acc, (sub & 1) ? f1 : f0, idx);
    if (sub < 3 && idx < NF)
      read_frag<MI, TA, TB>((sub & 1) ? f0 : f1, idx, A, Bt, sub + 1, arow0, nrow);
    if (p % 3 == 1 && p / 3 < NA) la.issue1(la_dst, p / 3, koa, va);
    if (p >= B0 && (p - B0) % BS == 0 && (p - B0) / BS < NB) lb.issue1(lb_dst, (p - B0) / BS, kob, vb);
    if (p == BAR) {
      MOONEP_PIN();
      wait_loads<kLoadsPerStep>();
      barrier_reads_done();
    }
    if (p > BAR && p - BAR - 1 < NF) read_frag<MI, TA, TB>(f0, p - BAR - 1, An, Bn, 0, arow0, nrow);
    MOONEP_PIN();
  }
}

// The K loop shared by every GEMM here.  The prologue loads B(0), A(0),
// B(1); each step then loads A(j+1) and B(j+2) (out-of-range offsets past
// the last step: they read nothing and keep the wait counts fixed).
template <int MI, class TA, class TB>
__device__ __forceinline__ void gemm_loop(const TA& la, const TB& lb, const Ring& ring, int nk,
                                          f32x16 acc[MI][4], int arow0, const int nrow[4]) {
  static_assert(TB::kLoads == kLoadsPerStep, "the barrier wait counts B loads");
  if (nk <= 0) return;
  lb.issue(ring.b<0>(), 0, true);
  la.issue(ring.a<0>(), 0, true);
  lb.issue(ring.b<1>(), BK, 1 < nk);
  wait_loads<kLoadsPerStep>();
  barrier_reads_done();
  Frags<MI> f0, f1;
#pragma unroll
  for (int q = 0; q < MI + 4; ++q)
    read_frag<MI, TA, TB>(f0, q, ring.a<0>(), ring.b<0>(), 0, arow0, nrow);
  for (int j = 0; j < nk; j += kSlots) {
    kstep<0, MI>(la, lb, ring, j, nk, f0, f1, acc, arow0, nrow);
    if (j + 1 < nk) kstep<1, MI>(la, lb, ring, j + 1, nk, f0, f1, acc, arow0, nrow);
    if (j + 2 < nk) kstep<2, MI>(la, lb, ring, j + 2, nk, f0, f1, acc, arow0, nrow);
    if (j + 3 < nk) kstep<3, MI>(la, lb, ring, j + 3, nk, f0, f1, acc, arow0, nrow);
    if (j + 4 < nk) kstep<4, MI>(la, lb, ring, j + 4, nk, f0, f1, acc, arow0, nrow);
  }
  wait_loads<0>();
  // every wave is past its last fragment read before the ring is reused
  __syncthreads();
}

template <int MI>
__device__ __forceinline__ void zero_acc(f32x16 acc[MI][4]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
}

// Column (within the 32x32 block) of accumulator elements 4q..4q+3 of this
// lane (the first of four consecutive columns).
__device__ __forceinline__ int acc_col(int q, int lh) { return 8 * q + 4 * lh; }

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Epilogue staging: a wave's bf16 output sub-tile (ROWS x NC columns) is
// written to LDS row-major (8-byte pieces straight from the accumulator
// layout), then read back 16 bytes per lane along whole rows and stored with
// 16-byte buffer stores, so every store instruction writes complete rows.
template <int ROWS, int NC>
struct Stage {
  static constexpr int kRowBytes = NC * 2 + 16;     // padded row (16-byte aligned)
  static constexpr int kBytes = ROWS * kRowBytes;
  __device__ __forceinline__ static void put(lds_t* reg, int row, int col, unsigned lo, unsigned hi) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    *(__attribute__((address_space(3))) u32x2*)(reg + row * kRowBytes + col * 2) = u32x2{lo, hi};
  }
  // store the staged sub-tile: rows [0,ROWS) to row m0 + r of `dst` (row
  // stride ld elements, rows past the descriptor range dropped), columns
  // [0,NC) to column c0 + c (columns at or past cols_valid dropped)
  __device__ __forceinline__ static void flush(const lds_t* reg, Rsrc dst, int m0, int64_t ld,
                                               int c0, int cols_valid) {
    constexpr int kLanesPerRow = NC / 8, kRowsPerInst = 64 / kLanesPerRow;
    const int lane = threadIdx.x & 63;
    const int r0 = lane / kLanesPerRow, ch = lane % kLanesPerRow;
    const int col = c0 + ch * 8;
#pragma unroll
    for (int t = 0; t < ROWS / kRowsPerInst; ++t) {
      const int r = t * kRowsPerInst + r0;
      const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(reg + r * kRowBytes + ch * 16);
      const uint32_t off = col < cols_valid ? (uint32_t)(((int64_t)(m0 + r) * ld + col) * 2) : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(v, dst, off, 0, 0);
    }
  }
};

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
  // backward: dY [R*NvS][H] in; dZ, dG, dU [R*NvS][Hp]; dX [R*NvS][H]
  const uint16_t* dy;
  uint16_t* dz;
  uint16_t* dg;
  uint16_t* du;
  uint16_t* dx;
  const int32_t* tiles;     // [R][max_tiles][4]
  const int32_t* ntiles;    // [R]
  int R, E, B, H, Hp, NvS, max_tiles, rank0, nranks, ntn;
};

__device__ __forceinline__ const uint16_t* weight_row(const FfnArgs& a, int p, int d, int row) {
  const int64_t rs = (int64_t)a.H * a.Hp;
  return row < a.E ? a.home[p] + (int64_t)row * rs : a.pool[p] + ((int64_t)d * a.B + row - a.E) * rs;
}

// Within a rank, tiles are taken in groups of up to kGroupM M-tiles of one
// segment (one expert): the group's M-tiles for the first N-tile, then for the
// second, ...  Workgroups that run together on an XCD (32 CUs) then cover
// kGroupM M-tiles x 32/kGroupM N-tiles of the same expert, so each weight
// slab in that XCD's L2 serves the group's workgroups, and a group never
// mixes two experts' weights.  Tile entry t holds (row, first slot, end slot,
// group start * 16 + group size); the workgroups of a group starting at tile
// g with size n are those with index l in [g ntn, (g + n) ntn), so l / ntn is
// a tile of the same group and names it.
constexpr int kGroupM = 4;

__device__ __forceinline__ bool decode(const FfnArgs& a, int* d, Tile* tl, int* nt) {
  const int64_t lt = logical_tile();
  const int64_t per_rank = (int64_t)a.max_tiles * a.ntn;
  const int64_t total = (int64_t)a.nranks * per_rank;
  if (lt >= total) return false;
  *d = a.rank0 + (int)(lt / per_rank);
  const int l = (int)(lt % per_rank);
  const int tp = l / a.ntn;
  if (tp >= a.ntiles[*d]) return false;
  const int32_t* base = a.tiles + (int64_t)*d * a.max_tiles * 4;
  const int grp = base[tp * 4 + 3];
  const int gs = grp >> 4, gm = grp & 15;
  const int rem = l - gs * a.ntn;
  *nt = rem / gm;
  const int32_t* e = base + (gs + rem % gm) * 4;
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
    const int t0 = base + before + x - n;      // first tile of this segment
    int t = t0;
    for (int m = end - len; m < end; m += BM, ++t) {
      if (t >= max_tiles) break;
      int32_t* e = tiles + ((int64_t)d * max_tiles + t) * 4;
      const int gs = t0 + (t - t0) / kGroupM * kGroupM;
      const int gm = min(kGroupM, t0 + n - gs);
      e[0] = row;
      e[1] = m;
      e[2] = m + BM < end ? m + BM : end;
      e[3] = gs * 16 + gm;
    }
    __syncthreads();
    base += s_total;
    __syncthreads();
  }
  if (tid == 0) ntiles[d] = base < max_tiles ? base : max_tiles;
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

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void ffn_gateup(FfnArgs a) {
  MOONEP_RING(smem);
  int d, nt;
  Tile tl;
  if (!decode(a, &d, &tl, &nt)) return;
  if (tl.m1 - tl.m0 <= kHalfTileM) gateup_tile<2>(a, smem, d, tl, nt);
  else gateup_tile<4>(a, smem, d, tl, nt);
}

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void ffn_down(FfnArgs a) {
  MOONEP_RING(smem);
  int d, nt;
  Tile tl;
  if (!decode(a, &d, &tl, &nt)) return;
  if (tl.m1 - tl.m0 <= kHalfTileM) down_tile<2>(a, smem, d, tl, nt);
  else down_tile<4>(a, smem, d, tl, nt);
}

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
  zero_acc<MI>(acc);
  gemm_loop<MI>(la, lb, smem, a.H / BK, acc, wm * 32 * MI, nrow);

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
  zero_acc<MI>(acc);
  gemm_loop<MI>(la, lb, smem, a.H / BK, acc, wm * 32 * MI, nrow);

  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  typedef Stage<32 * MI, 64> St;
  lds_t* reg_g = smem.base + wave * (2 * St::kBytes);
  lds_t* reg_u = reg_g + St::kBytes;
  const uint16_t* dzb = a.dz + ((int64_t)d * a.NvS + tl.m0) * a.Hp + n0;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm * 32 * MI + i * 32 + lr;
        const int n = wn * 64 + j * 32 + acc_col(q, lh);
        u32x2 dzv = {0u, 0u};
        if (m < rows_valid && n < nvh) dzv = *(const u32x2*)(dzb + (int64_t)m * a.Hp + n);
        float dg[4], du[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned bits = e & 1 ? (dzv[e >> 1] & 0xFFFF0000u) : (dzv[e >> 1] << 16);
          const float dz = __uint_as_float(bits);
          const float g = acc[i][j][4 * q + e], u = acc[i][j + 2][4 * q + e];
          const float sg = 1.0f / (1.0f + __expf(-g));
          du[e] = dz * (g * sg);
          dg[e] = dz * u * (sg * (1.0f + g * (1.0f - sg)));
        }
        St::put(reg_g, i * 32 + lr, j * 32 + acc_col(q, lh), pack_bf16x2(dg[0], dg[1]),
                pack_bf16x2(dg[2], dg[3]));
        St::put(reg_u, i * 32 + lr, j * 32 + acc_col(q, lh), pack_bf16x2(du[0], du[1]),
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
  zero_acc<MI>(acc);
  gemm_loop<MI>(la, lb, smem, 2 * a.Hp / BK, acc, wm * 32 * MI, nrow);

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
  const Rsrc xs = make_rsrc(a.dx + ((int64_t)d * a.NvS + tl.m0) * a.H + n0,
                            (int64_t)rows_valid * a.H * 2);
  St::flush(reg, xs, wm * 32 * MI, a.H, wn * 128, cols_valid);
}

#define MOONEP_TILE_KERNEL(name, body)                                              \
  __global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),       \
                            amdgpu_waves_per_eu(1, 1))) void name(FfnArgs a) {     \
    MOONEP_RING(smem);                                                             \
    int d, nt;                                                                     \
    Tile tl;                                                                       \
    if (!decode(a, &d, &tl, &nt)) return;                                          \
    if (tl.m1 - tl.m0 <= kHalfTileM) body<2>(a, smem, d, tl, nt);                  \
    else body<4>(a, smem, d, tl, nt);                                              \
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
  const int32_t* cu;        // [R][E+B]
  const int32_t* segn;      // [R][E+B]
  int R, E, B, H, Hp, NvS, L2, EB, tp, rank0, nranks, ntm, ntn;
};

// dW[h][h'] += sum over the segment's tokens t of A[t][h] * B[t][h'].
// Tile: 256 h (MFMA rows) x 256 h' (MFMA columns), contraction over t.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void wgrad_kernel(WgradArgs a) {
  MOONEP_RING(smem);
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
  zero_acc<4>(acc);
  gemm_loop<4>(la, lb, smem, (ntok + BK - 1) / BK, acc, wm * 128, nrow);

  // fp32 read-modify-write, 4 consecutive columns (16 bytes) per access,
  // masked to rows < H and columns < H'.  Plain global accesses: the 128-bit
  // buffer-load builtin of this toolchain is lowered to a 32-bit load.
  const int64_t rs = (int64_t)a.H * a.Hp;
  float* G = (row < a.E ? a.gh + (int64_t)row * rs : a.rb + ((int64_t)d * a.B + row - a.E) * rs) +
             (int64_t)m0 * a.Hp + n0;
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm * 128 + i * 32 + lr;
        const int n = nrow[j] + acc_col(q, lh);
        if (m < mv && n < nv) {
          f32x4* gp = (f32x4*)(G + (int64_t)m * a.Hp + n);
          f32x4 v = *gp;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __fadd_rn(v[e], acc[i][j][4 * q + e]);
          *gp = v;
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
  a.dy = nullptr; a.dz = nullptr; a.dg = nullptr; a.du = nullptr; a.dx = nullptr;
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

hipError_t launch_ffn_bwd(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* x,
                          const uint16_t* dy, const uint16_t* const home[3],
                          const uint16_t* const pool[3], uint16_t* dz, uint16_t* dg,
                          uint16_t* du, uint16_t* dx, hipStream_t s) {
  FfnArgs a = ffn_args(c, p, rank, home, pool);
  a.x = x; a.dy = dy; a.dz = dz; a.dg = dg; a.du = du; a.dx = dx;
  const int64_t slots = (int64_t)a.nranks * a.max_tiles;
  a.ntn = (c.d.Hp + BN - 1) / BN;
  ffn_bwd_dz<<<(unsigned)pad_grid(slots * a.ntn), kThreads, 0, s>>>(a);
  a.ntn = (c.d.Hp + 127) / 128;
  ffn_bwd_gu<<<(unsigned)pad_grid(slots * a.ntn), kThreads, 0, s>>>(a);
  a.ntn = (c.d.H + BN - 1) / BN;
  ffn_bwd_dx<<<(unsigned)pad_grid(slots * a.ntn), kThreads, 0, s>>>(a);
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
