// Shared core of the grouped expert GEMMs on gfx950 (forward, backward and
// weight gradients): operand tiles, the LDS ring, the MFMA K loop, epilogue
// staging and the tile schedule decode.  Included by gemm.hip and
// gemm_bwd.hip; everything here has internal linkage.
//
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
//   tile_schedule.h the M-tiles of each rank (<= 256 rows, never crossing a
//                  segment), built by the planner's last kernel;
//   gemm.hip       ffn_gateup (256 x (128
//                  gate + 128 up), K = H, fused SwiGLU writing Z), ffn_down
//                  (256 x 256 of Y = Z Wd^T, K = H');
//   gemm_bwd.hip   ffn_bwd_dz, ffn_bwd_gu, ffn_bwd_dx (the FFN backward) and
//                  wgrad_kernel (256 x 256 of dW += X_seg^T dY_seg, fp32
//                  read-modify-write of the gradient row).
//
// CDNA4 mapping: 256 threads = 4 waves in a 2x2 grid, each wave a 128x128
// sub-tile as 4x4 v_mfma_f32_32x32x16_bf16 blocks (256 fp32 accumulators per
// lane, in AGPRs).  K advances 64 per step.  Operand tiles (256 x 64 bf16,
// 32 KiB) rotate through a ring of five LDS slots (160 KiB) filled by LDS-DMA
// buffer loads (no staging registers, no LDS write instructions); weights are
// fetched two steps ahead, activations one.  Operands contiguous along K are
// kept as 128-byte rows (whole cache lines per load) with an XOR chunk
// swizzle that keeps 16 consecutive rows on distinct LDS banks, and read with
// ds_read_b128; operands stored [k][n] (gate/up weights, both weight-gradient
// operands) are kept as 256-byte k-rows and read with the gfx950 transposing
// LDS read (ds_read_b64_tr_b16), which hands each
// lane one column's 4 consecutive k.  Fragments are double-buffered in
// registers and every load and fragment read is slotted between MFMAs, so the
// matrix unit stays busy across the one barrier per step.  Buffer descriptors
// make tile edges branch-free (out-of-range loads read zero, out-of-range
// stores are dropped).  Workgroup ids are remapped so that every XCD (own L2)
// works through a contiguous range of tiles: neighbouring tiles share weight
// or activation slabs in that XCD's L2.
#pragma once

#include "internal.h"
#include "tile_schedule.h"

namespace moonep {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 64;        // K advances 64 per step
constexpr int kHalfTileM = kShortTileM;           // rows of a segment's short last tile
static_assert(BM == kTileM && kGemmTileM == kTileM, "one M-tile height everywhere");
constexpr int kXcds = 8;
constexpr int kLoadsPerStep = 8;                  // LDS-DMA loads per wave per tile and step

typedef __attribute__((address_space(3))) char lds_t;

__device__ __forceinline__ int round_up(int n, int m) { return (n + m - 1) / m * m; }

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
// ---------------------------------------------------------------------------
// Operand tiles in LDS: 256 rows (or columns) x 64 k of bf16 = 32 KiB, one
// per ring slot.
//
// Row tile (operand contiguous along k): rows of 128 B (64 k); the 16-byte
// chunk c of row r sits at position c ^ ((r >> 1) & 7).  The LDS serves 256
// bytes per clock, i.e. 16 lanes of a 16-byte fragment read, which here are
// 16 consecutive rows at the same chunk: two rows share each 256-byte window
// and the swizzle sends all 16 to distinct 16-byte bank groups (measured:
// no bank conflicts, where c ^ (r & 7) doubles the read time).  One LDS-DMA
// load (a wave, 1 KiB) fills 8 rows, each a whole 128-byte cache line: the
// L1/L2 path costs per cache line touched, and half-line rows would halve its
// rate.  Rows 8 apart differ in bit 2 of the swizzle, so even and odd loads
// of a wave use two lane offsets.
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
  uint32_t voff[2];     // this lane's offsets for even / odd loads of k-block 0
  uint32_t step;        // byte distance between consecutive loads of a wave (8 rows)
  uint32_t wlds;        // this wave's first 1 KiB block inside a slot
  __device__ __forceinline__ static int swz(int r) { return (r >> 1) & 7; }
  // base: row 0, k 0 of the tile; ld: row stride (elements).  Rows at or
  // past rows_valid lie outside the descriptor's range and read zero.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int rows_valid) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    rs = make_dma_rsrc(base, (int64_t)rows_valid * ld * 2);
    // lane -> LDS row r + 8 i (load i), position lane & 7, which holds the
    // global chunk (lane & 7) ^ swz(r + 8 i) = (lane & 7) ^ swz(r) ^ 4 (i & 1)
    const int r = 8 * NL * w + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    voff[0] = (uint32_t)(r * ld * 2 + c * 16);
    voff[1] = (uint32_t)(r * ld * 2 + (c ^ 4) * 16);
    step = (uint32_t)(16 * ld);
    wlds = (uint32_t)(w * NL * 1024);
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const { return (uint32_t)(k0 * 2); }
  // load i (0..NL-1) of this wave for the k-block at byte offset ko (kOob:
  // the step is past the end; kOob + i step stays out of range).  The step's
  // validity is folded into ko once and the wave's LDS block is kept from
  // init: each load then costs two scalar adds, which the compiler can slot
  // between MFMAs (a per-load select and wave-id computation made a burst of
  // ~50 scalar instructions at the top of every step, with the matrix unit
  // idle).
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t ko) const {
    const uint32_t s = ko + (uint32_t)i * step;
    load_lds(rs, tile + wlds + i * 1024, voff[i & 1] + s);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) const {
    const uint32_t ko = valid ? koff(k0) : kOob;
#pragma unroll
    for (int i = 0; i < NL; ++i) issue1(tile, i, ko);
  }
  // 8 consecutive k (sub-step kk of 4, lane half lh) of tile row `row`
  __device__ __forceinline__ static bf16x8 frag(const lds_t* tile, int row, int kk, int lh) {
    const int c = (2 * kk + lh) ^ swz(row);
    return *(const __attribute__((address_space(3))) bf16x8*)(tile + row * 128 + c * 16);
  }
};
typedef RowTileT<8> RowTile;      // 256 rows

// Row tile whose K range is the concatenation of two matrices: k < k1 from
// the first, k >= k1 from the second (same rows, same row stride, so the
// lane offsets are shared and only the descriptor differs).  koff encodes
// the step once: the byte offset within the matrix that holds k, with
// kSecond set for the second; kOob past the end.  Each load then selects a
// descriptor with scalar selects, with no branch in the MFMA stream (a
// per-load branch split every step into three copies of its loads).
template <int NL>
struct RowTile2 {
  static constexpr bool kRows = true;
  static constexpr int kLoads = NL;
  static constexpr uint32_t kSecond = 0x40000000u;
  RowTileT<NL> t;       // geometry and the first matrix's descriptor
  DmaRsrc rs1;          // the second matrix
  uint32_t k1;
  __device__ __forceinline__ void init(const uint16_t* base0, const uint16_t* base1, int64_t ld,
                                       int rows_valid, int k_first) {
    t.init(base0, ld, rows_valid);
    rs1 = make_dma_rsrc(base1, (int64_t)rows_valid * ld * 2);
    k1 = (uint32_t)k_first;
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const {
    return k0 < k1 ? (uint32_t)(k0 * 2) : ((uint32_t)((k0 - k1) * 2) | kSecond);
  }
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t ko) const {
    const bool second = (ko & kSecond) != 0;              // never set in kOob
    const uint32_t s = (ko & ~kSecond) + (uint32_t)i * t.step;
    DmaRsrc r;                                            // element-wise: scalar selects
#pragma unroll
    for (int e = 0; e < 4; ++e) r.v[e] = second ? rs1.v[e] : t.rs.v[e];
    load_lds(r, tile + t.wlds + i * 1024, t.voff[i & 1] + s);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) const {
    const uint32_t ko = valid ? koff(k0) : kOob;
#pragma unroll
    for (int i = 0; i < NL; ++i) issue1(tile, i, ko);
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
  uint32_t wlds;        // this wave's first 1 KiB block inside a slot
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
    wlds = (uint32_t)(w * 8 * 1024);
  }
  __device__ __forceinline__ uint32_t koff(int64_t k0) const { return (uint32_t)(k0 * ld2); }
  // ko: the step's byte offset, or kOob past the end
  __device__ __forceinline__ void issue1(lds_t* tile, int i, uint32_t ko) const {
    const uint32_t s = ko + (uint32_t)(4 * i) * ld2;
    load_lds(rs, tile + wlds + i * 1024, voff + s);
  }
  __device__ __forceinline__ void issue(lds_t* tile, int64_t k0, bool valid) const {
    const uint32_t ko = valid ? koff(k0) : kOob;
#pragma unroll
    for (int i = 0; i < 8; ++i) issue1(tile, i, ko);
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
  const uint32_t koa = j + 1 < nk ? la.koff((int64_t)(j + 1) * BK) : kOob;
  const uint32_t kob = j + 2 < nk ? lb.koff((int64_t)(j + 2) * BK) : kOob;
  MOONEP_PIN();
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int sub = p / SUB, idx = p % SUB;
    mma1<MI>(acc, (sub & 1) ? f1 : f0, idx);
    if (sub < 3 && idx < NF)
      read_frag<MI, TA, TB>((sub & 1) ? f0 : f1, idx, A, Bt, sub + 1, arow0, nrow);
    if (p % 3 == 1 && p / 3 < NA) la.issue1(la_dst, p / 3, koa);
    if (p >= B0 && (p - B0) % BS == 0 && (p - B0) / BS < NB) lb.issue1(lb_dst, (p - B0) / BS, kob);
    if (p == BAR) {
      MOONEP_PIN();
      wait_loads<kLoadsPerStep>();
      barrier_reads_done();
    }
    if (p > BAR && p - BAR - 1 < NF) read_frag<MI, TA, TB>(f0, p - BAR - 1, An, Bn, 0, arow0, nrow);
    MOONEP_PIN();
  }
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

// The K loop shared by every GEMM here; it sets acc to the product.  The
// prologue loads B(0), A(0), B(1); each step then loads A(j+1) and B(j+2)
// (out-of-range offsets past the last step: they read nothing and keep the
// wait counts fixed).
template <int MI, class TA, class TB>
__device__ __forceinline__ void gemm_loop(const TA& la, const TB& lb, const Ring& ring, int nk,
                                          f32x16 acc[MI][4], int arow0, const int nrow[4]) {
  static_assert(TB::kLoads == kLoadsPerStep, "the barrier wait counts B loads");
  if (nk <= 0) {
    zero_acc<MI>(acc);
    return;
  }
  lb.issue(ring.b<0>(), 0, true);
  la.issue(ring.a<0>(), 0, true);
  lb.issue(ring.b<1>(), BK, 1 < nk);
  // the accumulators are cleared while the first tiles are in flight (after
  // the wait they would hold the matrix unit back by ~1k cycles per tile)
  zero_acc<MI>(acc);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));   // cleared here, not later
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


// Column (within the 32x32 block) of accumulator elements 4q..4q+3 of this
// lane (the first of four consecutive columns).
__device__ __forceinline__ int acc_col(int q, int lh) { return 8 * q + 4 * lh; }

// Two fp32 -> two bf16 (lo in bits 0-15), round to nearest, ties to even, by
// the gfx950 packed conversion (one instruction; a shift-and-add rounding
// took about 9 vector instructions per pair, which the epilogues issue with
// the matrix unit idle).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Epilogue staging: a wave's bf16 output sub-tile (ROWS x NC columns) is
// written to LDS row-major (8-byte pieces straight from the accumulator
// layout), then read back 16 bytes per lane along whole rows and stored with
// 16-byte buffer stores, so every store instruction writes complete rows.
template <int ROWS, int NC>
// The padded row stride is 4 banks (mod 64) for NC = 128, so the 32 rows of a
// put instruction would meet two to a bank; rows 16..31 of every 32 keep the
// two 8-byte halves of each 16-byte chunk swapped, which puts them on the
// other two banks of each group of four (the flush swaps them back).
struct Stage {
  static constexpr int kRowBytes = NC * 2 + 16;     // padded row (16-byte aligned)
  static constexpr int kBytes = ROWS * kRowBytes;
  // this lane's accumulator piece (i, j, q) as bf16 pairs lo, hi: row 32 i + lane%32, columns
  // 32 j + 8 q + 4 (lane/32) .. +3 (the layout mma1 leaves)
  __device__ __forceinline__ static void put(lds_t* reg, int i, int j, int q, unsigned lo,
                                             unsigned hi) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
    const int lane_off = lr * kRowBytes + 8 * (lh ^ ((lr >> 4) & 1));
    const int off = lane_off + 32 * i * kRowBytes + 64 * j + 16 * q;
    *(__attribute__((address_space(3))) u32x2*)(reg + off) = u32x2{lo, hi};
  }
  // store the staged sub-tile: rows [0,ROWS) to row m0 + r of `dst` (row
  // stride ld elements, rows past the descriptor range dropped), columns
  // [0,NC) to column c0 + c (columns at or past cols_valid dropped)
  __device__ __forceinline__ static void flush(const lds_t* reg, Rsrc dst, int m0, int64_t ld,
                                               int c0, int cols_valid) {
    constexpr int kLanesPerRow = NC / 8, kRowsPerInst = 64 / kLanesPerRow;
    static_assert(16 % kRowsPerInst == 0, "an instruction's rows share the swap of their 16");
    const int lane = threadIdx.x & 63;
    const int r0 = lane / kLanesPerRow, ch = lane % kLanesPerRow;
    const int col = c0 + ch * 8;
#pragma unroll
    for (int t = 0; t < ROWS / kRowsPerInst; ++t) {
      const int r = t * kRowsPerInst + r0;
      u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(reg + r * kRowBytes + ch * 16);
      if ((((t * kRowsPerInst) >> 4) & 1) != 0) v = __builtin_shufflevector(v, v, 2, 3, 0, 1);
      const uint32_t off = col < cols_valid ? (uint32_t)(((int64_t)(m0 + r) * ld + col) * 2) : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(v, dst, off, 0, 0);
    }
  }
};

struct Tile {
  int row, m0, m1;
};

struct FfnArgs {
  const uint16_t* x;        // [R*NvS][H] (gate/up input)
  const uint16_t* home[3];  // rows [0,E) of rank d at home + d*hstride rows
  const uint16_t* pool[3];  // rows [E,E+B) of rank d at pool + d*pstride rows
  int64_t hstride, pstride;
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
  const int32_t* nfull;     // [R] full-duration tiles of each rank (the first ones)
  int R, E, B, H, Hp, NvS, max_tiles, rank0, nranks, ntn;
};

__device__ __forceinline__ const uint16_t* weight_row(const FfnArgs& a, int p, int d, int row) {
  const int64_t rs = (int64_t)a.H * a.Hp;
  return row < a.E ? a.home[p] + ((int64_t)d * a.hstride + row) * rs
                   : a.pool[p] + ((int64_t)d * a.pstride + row - a.E) * rs;
}

// Within a rank, tiles are taken in groups of up to kGroupMax M-tiles of one
// segment (one expert): the group's M-tiles for the first N-tile, then for the
// second, ...  Workgroups that run together on an XCD (32 CUs) then cover a
// group's n M-tiles x about 32/n N-tiles of the same expert, so each weight
// slab in that XCD's L2 serves the group's workgroups, and a group never
// mixes two experts' weights.  Tile entry t holds (row, first slot, end slot,
// group start * 16 + group size); the workgroups of a group starting at tile
// g with size n are those with index l in [g ntn, (g + n) ntn), so l / ntn is
// a tile of the same group and names it.
//
// The workgroups enumerate only real tiles, in two parts: every launched
// rank's full-duration tiles (rank after rank, each N-swept as above), then
// every rank's short tiles.  XCD x runs the x-th eighth of the first part,
// then the x-th eighth of the second, so every XCD holds the same mix of
// durations and finishes with the others, and the tiles an XCD runs together
// have one duration whatever the ranks' tile counts.  Splitting the grid's
// padded upper bound instead would give the empty tail of each rank's range
// to whole XCDs (one rank launched alone kept only five of the eight busy).
//
// The decode takes two rounds of loads, one value per lane in each: the
// launched ranks' tile counts (one rank per lane, prefix sums by lane
// shuffles, the rank by a ballot), then a window of 16 tile entries around
// the one the workgroup index names, which holds both that entry's group and
// the tile the workgroup takes (groups have at most 8 tiles), in place of a
// chain of dependent scalar loads.
static_assert(kGroupMax <= 8, "the decode window holds a group on either side of its entry");
__device__ __forceinline__ bool decode(const FfnArgs& a, int* d, Tile* tl, int* nt) {
  const int lane = threadIdx.x & 63;
  int f = 0, s = 0;                                    // rank rank0 + lane's full, short tiles
  if (lane < a.nranks) {
    f = a.nfull[a.rank0 + lane];
    s = a.ntiles[a.rank0 + lane] - f;
  }
  int cf = f, cs = s;                                  // inclusive prefix sums over lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yf = __shfl_up(cf, o, 64), ys = __shfl_up(cs, o, 64);
    if (lane >= o) {
      cf += yf;
      cs += ys;
    }
  }
  const int64_t nf = __builtin_amdgcn_readlane(cf, 63), ns = __builtin_amdgcn_readlane(cs, 63);
  const int64_t F = nf * a.ntn, Sx = ns * a.ntn;        // full and short workgroups
  const int64_t pf = (F + kXcds - 1) / kXcds, ps = (Sx + kXcds - 1) / kXcds;
  const int64_t x = blockIdx.x % kXcds, c = blockIdx.x / kXcds;
  const int64_t f0 = x * pf;
  const int64_t nfx = f0 < F ? (F - f0 < pf ? F - f0 : pf) : 0;   // this XCD's full ones
  const bool full = c < nfx;
  int64_t lt;
  if (full) {
    lt = f0 + c;
  } else {
    lt = x * ps + (c - nfx);
    if (c - nfx >= ps || lt >= Sx) return false;
  }
  // the rank: the first lane whose inclusive count of this part's tiles covers lt (lanes past
  // the launched ranks hold the total, which does)
  const int cpart = full ? cf : cs;
  const uint64_t hit = __ballot((int64_t)cpart * a.ntn > lt);
  const int r = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  const int64_t first = r > 0 ? __builtin_amdgcn_readlane(cpart, r - 1) : 0;
  *d = a.rank0 + r;
  if (!full) lt += (int64_t)__builtin_amdgcn_readlane(f, r) * a.ntn;   // short tiles follow full
  const int l = (int)(lt - first * a.ntn);
  const int tp = l / a.ntn;
  const int32_t* base = a.tiles + (int64_t)*d * a.max_tiles * 4;
  const int w0 = tp - 7 < 0 ? 0 : tp - 7;              // window: entries w0 .. w0 + 15
  const int ei = w0 * 4 + lane;
  const int v = ei < a.max_tiles * 4 ? base[ei] : 0;
  const int grp = __builtin_amdgcn_readlane(v, (tp - w0) * 4 + 3);
  const int gs = grp >> 4, gm = grp & 15;
  const int rem = l - gs * a.ntn;
  *nt = rem / gm;
  const int k = (gs + rem % gm - w0) * 4;
  tl->row = __builtin_amdgcn_readlane(v, k);
  tl->m0 = __builtin_amdgcn_readlane(v, k + 1);
  tl->m1 = __builtin_amdgcn_readlane(v, k + 2);
  return true;
}

// One kernel per tile body: a segment's short last tile (<= kHalfTileM rows)
// runs with MI = 2, every other tile with MI = 4.
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

int64_t pad_grid(int64_t n) { return (n + kXcds - 1) / kXcds * kXcds; }

}  // namespace

static inline FfnArgs ffn_args(const Ctx& c, const moonep_plan_t& p, int rank,
                               const WeightRef& w) {
  const Dims& d = c.d;
  FfnArgs a;
  for (int i = 0; i < 3; ++i) {
    a.home[i] = w.home[i];
    a.pool[i] = w.pool[i];
  }
  a.hstride = w.home_stride;
  a.pstride = w.pool_stride;
  a.x = nullptr; a.z = nullptr; a.zin = nullptr; a.y = nullptr;
  a.dy = nullptr; a.dz = nullptr; a.dg = nullptr; a.du = nullptr; a.dx = nullptr;
  a.tiles = p.aux + d.aux.tiles; a.ntiles = p.aux + d.aux.ntiles; a.nfull = p.aux + d.aux.nfull;
  a.R = d.R; a.E = d.E; a.B = d.B; a.H = d.H; a.Hp = d.Hp; a.NvS = (int)d.NvS;
  a.max_tiles = d.max_tiles;
  a.rank0 = rank < 0 ? 0 : rank;
  a.nranks = rank < 0 ? d.R : 1;
  a.ntn = 0;
  return a;
}

// Workgroups a tile launch needs: at most max_tiles tiles per launched rank,
// each swept over ntn N-tiles; rounding each part up per XCD adds at most two
// workgroups to each XCD.
static inline int64_t tile_grid(const FfnArgs& a) {
  return pad_grid((int64_t)a.nranks * a.max_tiles * a.ntn) + 2 * kXcds;
}

}  // namespace moonep
