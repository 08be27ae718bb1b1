// HBM-bound kernels of the MoonEP path on gfx950: dispatch (fused permute),
// combine (fused unpermute), prefetch_weight and reduce_grad.
//
// MoonEP README (MoonshotAI/MoonEP mirror), "API guide": dispatch writes
// each token straight into its expert-grouped slot of the destination rank
// (no separate permute pass), combine brings the K copies of a token back to
// token-major order, prefetch_weight fills the prefetch rows of the
// [E+B,H,H'] weight tensor, reduce_grad adds the prefetch-slot gradients of
// every rank into the owning home rows and zeroes the slots ("Gradient
// buffer").
//
// Design for CDNA4: one wave per token row, 16-byte vector loads and stores
// (64 lanes x 16 B = 1 KiB per instruction, fully coalesced), all loads of
// a row chunk in flight before the stores (combine: the K source rows of a
// column vector in flight before the sum), non-temporal loads for data read
// once.  Dispatch reads each token row once and
// writes it K times (scatter); combine gathers K rows and writes one.  The
// combine sum uses explicit round-to-nearest fp32 multiply and add
// (__fmul_rn / __fadd_rn) in ascending k, so it is bit-reproducible.
#include "internal.h"

namespace moonep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;          // 16-byte vectors per lane in flight
constexpr int kXcdsMove = 8;       // XCDs: workgroup b runs on XCD b mod 8
constexpr int kDispVecs = 16;       // 16-byte vectors per lane of one dispatch column chunk

__device__ __forceinline__ int round_up(int n, int m) { return (n + m - 1) / m * m; }

__device__ __forceinline__ float bf16_lo(unsigned v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(unsigned v) { return __uint_as_float(v & 0xFFFF0000u); }

// Two fp32 -> two bf16 (lo in bits 0-15), round to nearest, ties to even (the
// gfx950 packed conversion).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

struct DispatchArgs {
  const u32x4* x;        // [R*S][W/8]
  const float* rw;       // [R*S][K] or null
  u32x4* x_nvs;          // [R*NvS][W/8]
  float* rw_nvs;         // [R*NvS] or null
  const int32_t* dest;   // [R*S][K]
  const int32_t* cu;     // [R][E+B]
  const int32_t* segn;   // [R][E+B]
  const int32_t* act;    // [R][2L]
  int ntok, K, nv, EB, L2, tp, pad_parts, npad_used, NvS;
  int item_blocks;        // token workgroups (the padding workgroups follow them)
  int xcd_local;          // 1: one item per wave, a token's waves on one XCD; 0: a capped grid
};

// Padding item pb: zero the padding rows (and their route weights) of one
// part of one active row.
__device__ __forceinline__ void dispatch_pad(const DispatchArgs& a, int pb, int wv, int lane) {
  const int part = pb % a.pad_parts;
  const int dq = pb / a.pad_parts;        // d * 2L + q
  const int row = a.act[dq];
  if (row < 0) return;
  const int d = dq / a.L2;
  const int end = a.cu[d * a.EB + row];
  const int n = a.segn[d * a.EB + row];
  const int len = round_up(n, a.tp);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int i = end - len + n + part * kWaves + wv; i < end; i += a.pad_parts * kWaves) {
    const int64_t slot = (int64_t)d * a.NvS + i;
    u32x4* dst = a.x_nvs + slot * a.nv;
    for (int v = lane; v < a.nv; v += 64) __builtin_nontemporal_store(zero, dst + v);
    if (a.rw_nvs && lane == 0) a.rw_nvs[slot] = 0.0f;
  }
}

// Token item `it` = ((token, k) pair, column chunk of 64 kDispVecs vectors):
// the wave reads the chunk of the token's row and writes it to the pair's
// slot (and the pair's route weight).
__device__ __forceinline__ void dispatch_item(const DispatchArgs& a, int64_t it, int nch,
                                              int lane) {
  const int64_t p = it / nch;                           // (token, k) pair
  const int c0 = uniform((int)(it - p * nch)) * 64 * kDispVecs;
  const int tok = uniform((int)(p / a.K));
  const int slot = uniform(a.dest[p]);
  const u32x4* src = a.x + (int64_t)tok * a.nv;
  u32x4* dst = a.x_nvs + (int64_t)slot * a.nv;
  u32x4 buf[kDispVecs];
#pragma unroll
  for (int u = 0; u < kDispVecs; ++u) {
    const int v = c0 + u * 64 + lane;
    if (v < a.nv) buf[u] = src[v];
  }
#pragma unroll
  for (int u = 0; u < kDispVecs; ++u) {
    const int v = c0 + u * 64 + lane;
    if (v < a.nv) dst[v] = buf[u];            // non-temporal stores measured 15% slower
  }
  if (a.rw && c0 == 0 && lane == 0) a.rw_nvs[slot] = a.rw[p];
}

// Without a CU budget the grid has one piece of work per workgroup: the
// token items, one per wave, then the padding items (one part of one active
// row's padding per workgroup; launched first instead they measured the same
// within noise).  A token item is a (token, k) pair and a column chunk of 64
// kDispVecs vectors (the whole row up to 8192 columns).  The workgroups of a
// token run on one XCD, so its K waves take the row from that XCD's L2 (HBM
// reads 0.96 -> 0.48 GB at the headline, 1% faster).  One write per wave on a
// large grid measured 10-14% faster in the kernel than one wave writing all
// K slots of its tokens in a grid-stride loop; smaller chunks (7 or 4
// vectors) were 15-50% slower.  With a CU budget (num_cus) the grid is capped
// and every workgroup loops over the padding items, then over the token
// items.
__global__ __launch_bounds__(kThreads) void dispatch_kernel(DispatchArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nch = (a.nv + 64 * kDispVecs - 1) / (64 * kDispVecs);   // column chunks per row
  const int per_tok = a.K * nch;                          // items of a token
  if (a.xcd_local) {
    // token workgroups first, the padding workgroups after them (they fill
    // the tail of the token waves)
    const int b = (int)blockIdx.x;
    if (b >= a.item_blocks) {
      if (b - a.item_blocks < a.npad_used) dispatch_pad(a, b - a.item_blocks, wv, lane);
      return;
    }
    // the wpt workgroups of token t are t's group of 8 tokens x wpt, at the
    // position of t in its group: all on XCD t mod 8, so the K reads of its
    // row share that XCD's L2
    const int wpt = (per_tok + kWaves - 1) / kWaves;
    const int c = b / kXcdsMove;
    const int tok = (c / wpt) * kXcdsMove + b % kXcdsMove;
    const int item = (c % wpt) * kWaves + wv;
    if (tok >= a.ntok || item >= per_tok) return;
    dispatch_item(a, (int64_t)tok * per_tok + item, nch, lane);
    return;
  }
  for (int pb = blockIdx.x; pb < a.npad_used; pb += gridDim.x) dispatch_pad(a, pb, wv, lane);
  const int64_t items = (int64_t)a.ntok * per_tok;
  for (int64_t it = (int64_t)blockIdx.x * kWaves + wv; it < items; it += (int64_t)gridDim.x * kWaves)
    dispatch_item(a, it, nch, lane);
}

struct CombineArgs {
  const u32x4* y;        // [R*NvS][W/8]
  const float* rw_nvs;   // [R*NvS] or null
  u32x4* out;            // [R*S][W/8]
  float* rw_sk;          // [R*S][K] or null
  const int32_t* dest;   // [R*S][K]
  int ntok, K, nv;
};


// One wave per (token, column chunk of 64 kCombVecs 16-byte vectors = 3 KiB),
// on a grid of one chunk per wave: the wave reads the chunk of the token's K
// source rows, kCombRows rows at a time, and adds them in ascending k.
// Contiguous pieces of each source row measured faster than one 16-byte
// vector of all K rows at a time (5.79 against 5.28 TB/s on the same
// gather), and one piece of work per wave on a large grid faster than a loop
// (chunks of 7, 4 and 2 vectors and 3 or 4 rows in flight were within 2% of
// this or slower).
constexpr int kCombVecs = 3;
constexpr int kCombRows = 2;      // source rows in flight

template <bool kWeighted>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nchunks = (a.nv + 64 * kCombVecs - 1) / (64 * kCombVecs);
  const int64_t items = (int64_t)a.ntok * nchunks;
  for (int64_t it = (int64_t)blockIdx.x * kWaves + wv; it < items; it += (int64_t)gridDim.x * kWaves) {
    const int tok = uniform((int)(it / nchunks));
    const int c0 = uniform((int)(it % nchunks)) * 64 * kCombVecs;
    const int32_t* dk = a.dest + (int64_t)tok * a.K;
    u32x4* dst = a.out + (int64_t)tok * a.nv;
    float acc[kCombVecs][8];
    for (int k0 = 0; k0 < a.K; k0 += kCombRows) {
      const int kn = a.K - k0 < kCombRows ? a.K - k0 : kCombRows;
      u32x4 yv[kCombRows][kCombVecs];
      int slot[kCombRows];
#pragma unroll
      for (int r = 0; r < kCombRows; ++r) {
        slot[r] = r < kn ? uniform(dk[k0 + r]) : 0;
#pragma unroll
        for (int u = 0; u < kCombVecs; ++u) {
          const int v = c0 + u * 64 + lane;
          if (r < kn && v < a.nv) yv[r][u] = __builtin_nontemporal_load(a.y + (int64_t)slot[r] * a.nv + v);
        }
      }
#pragma unroll
      for (int r = 0; r < kCombRows; ++r)
        if (r < kn) {
          const int k = k0 + r;
          const float wk = kWeighted ? a.rw_nvs[slot[r]] : 1.0f;
#pragma unroll
          for (int u = 0; u < kCombVecs; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float pj0 = (j & 1) ? bf16_hi(yv[r][u][j >> 1]) : bf16_lo(yv[r][u][j >> 1]);
              const float pj = kWeighted ? __fmul_rn(wk, pj0) : pj0;
              acc[u][j] = (k == 0) ? pj : __fadd_rn(acc[u][j], pj);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kCombVecs; ++u) {
      const int v = c0 + u * 64 + lane;
      if (v < a.nv) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[u][2 * j], acc[u][2 * j + 1]);
        __builtin_nontemporal_store(o, dst + v);
      }
    }
    if (kWeighted && a.rw_sk && c0 == 0 && lane < a.K)
      a.rw_sk[(int64_t)tok * a.K + lane] = a.rw_nvs[dk[lane]];
  }
}

// prefetch: workgroup = (projection, 16 KiB column chunk of a weight row); it
// copies that chunk of every used slot in turn, so at any moment the
// workgroups sweep the rows of one slot together (a moving window, which
// measured 3-8% faster than each workgroup streaming its own 256 KiB piece).
struct PrefetchArgs {
  const u32x4* home[3];  // home row e of rank d at home + (d*hstride + e) rows
  u32x4* pool[3];        // slot j of rank d at pool + (d*pstride + j) rows
  const int32_t* pf;     // [R*B] prefetch_src
  const int32_t* aux_pf; // used slot list
  const int32_t* aux_pf_n;
  int64_t row_vecs;
  int64_t hstride, pstride;
  int B;
  int nchunks;           // 16 KiB chunks per row
};

constexpr int kPrefetchVecs = 4;   // 16-byte vectors per thread of one chunk

__global__ __launch_bounds__(kThreads) void prefetch_kernel(PrefetchArgs a) {
  const int n = *a.aux_pf_n;
  const int proj = blockIdx.x % 3;
  for (int ch = blockIdx.x / 3; ch < a.nchunks; ch += gridDim.x / 3) {
    const int64_t v0 = (int64_t)ch * (kThreads * kPrefetchVecs) + threadIdx.x;
    for (int q = 0; q < n; ++q) {
      const int slot = a.aux_pf[q];
      const int e = a.pf[slot];
      const int d = slot / a.B;
      const u32x4* src = a.home[proj] + ((int64_t)d * a.hstride + e) * a.row_vecs;
      u32x4* dst = a.pool[proj] + ((int64_t)d * a.pstride + slot - d * a.B) * a.row_vecs;
      u32x4 b[kPrefetchVecs];
#pragma unroll
      for (int u = 0; u < kPrefetchVecs; ++u) {
        const int64_t v = v0 + u * kThreads;
        if (v < a.row_vecs) b[u] = __builtin_nontemporal_load(src + v);
      }
#pragma unroll
      for (int u = 0; u < kPrefetchVecs; ++u) {
        const int64_t v = v0 + u * kThreads;
        if (v < a.row_vecs) __builtin_nontemporal_store(b[u], dst + v);
      }
    }
  }
}

// reduce_grad: work item = (expert with copies, projection, chunk).
struct ReduceArgs {
  f32x4* gh[3];          // [E][row_vecs]
  f32x4* rb[3];          // [R*B][row_vecs]
  const int32_t* dup_n;
  const int32_t* dup_e;
  const int32_t* dup_first;
  const int32_t* dup_cnt;
  const int32_t* hold;
  int64_t row_vecs;
  int chunk_vecs, nchunks;
};

__global__ __launch_bounds__(kThreads) void reduce_grad_kernel(ReduceArgs a) {
  const int n = *a.dup_n;
  const int64_t items = (int64_t)n * 3 * a.nchunks;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int chunk = (int)(it % a.nchunks);
    const int proj = (int)((it / a.nchunks) % 3);
    const int q = (int)(it / ((int64_t)a.nchunks * 3));
    const int e = a.dup_e[q];
    const int first = a.dup_first[q];
    const int cnt = a.dup_cnt[q];
    f32x4* g = a.gh[proj] + (int64_t)e * a.row_vecs;
    const int64_t v0 = (int64_t)chunk * a.chunk_vecs;
    int64_t v1 = v0 + a.chunk_vecs;
    if (v1 > a.row_vecs) v1 = a.row_vecs;
    for (int64_t v = v0 + threadIdx.x; v < v1; v += kThreads) {
      f32x4 acc = g[v];
      for (int h = 0; h < cnt; ++h) {
        f32x4* rbs = a.rb[proj] + (int64_t)a.hold[first + h] * a.row_vecs;
        const f32x4 r = __builtin_nontemporal_load(rbs + v);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __fadd_rn(acc[j], r[j]);
        __builtin_nontemporal_store(zero, rbs + v);
      }
      g[v] = acc;
    }
  }
}

// copy_rows: the used slots of every rank (rows [0, cu_seqlens[d][E+B-1]),
// padding rows included) from one [R,NvS,W] buffer to another; 16-byte
// vectors, grid-stride over (rank, row).
struct CopyArgs {
  const u32x4* src;
  u32x4* dst;
  const int32_t* cu;     // [R][E+B]
  int R, EB, nv, NvS;
};

__global__ __launch_bounds__(kThreads) void copy_rows_kernel(CopyArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t rows = (int64_t)a.R * a.NvS;
  for (int64_t g = (int64_t)blockIdx.x * kWaves + wv; g < rows; g += (int64_t)gridDim.x * kWaves) {
    const int d = (int)(g / a.NvS);
    const int i = (int)(g - (int64_t)d * a.NvS);
    if (i >= a.cu[d * a.EB + a.EB - 1]) continue;
    const u32x4* s = a.src + g * a.nv;
    u32x4* t = a.dst + g * a.nv;
    for (int v0 = 0; v0 < a.nv; v0 += 64 * kUnroll) {
      u32x4 buf[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + u * 64 + lane;
        if (v < a.nv) buf[u] = __builtin_nontemporal_load(s + v);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + u * 64 + lane;
        if (v < a.nv) __builtin_nontemporal_store(buf[u], t + v);   // 2-3% faster than plain
      }
    }
  }
}

int prefetch_chunks(const Dims& d) {
  const int64_t row_vecs = (int64_t)d.H * d.Hp / 8;
  return (int)((row_vecs + kThreads * kPrefetchVecs - 1) / (kThreads * kPrefetchVecs));
}

constexpr int kReduceChunkVecs = kThreads * 16;   // 64 KiB of fp32 per reduce_grad work item

int reduce_chunks(const Dims& d) {
  const int64_t row_vecs = (int64_t)d.H * d.Hp / 4;
  return (int)((row_vecs + kReduceChunkVecs - 1) / kReduceChunkVecs);
}

int capped_grid(const Ctx& c, int64_t want) {
  int64_t cap = want;
  if (c.d.num_cus > 0) cap = (int64_t)c.d.num_cus * 8;
  if (want < cap) cap = want;
  return (int)(cap < 1 ? 1 : cap);
}

}  // namespace

// Grid sizes of the data-movement launches (workgroups), shared by the
// launchers below and by moonep_launch_grid.  With a CU budget (num_cus > 0)
// every grid is at most num_cus * 8.
DispatchGrid dispatch_grid(const Ctx& c, int W) {
  const Dims& d = c.d;
  DispatchGrid g;
  const int nv = W / 8;
  g.pad_parts = (d.tp + 4 * kWaves - 1) / (4 * kWaves);
  g.npad_used = d.R * 2 * d.L * g.pad_parts;
  const int nch = (nv + 64 * kDispVecs - 1) / (64 * kDispVecs);
  const int64_t wpt = ((int64_t)d.K * nch + kWaves - 1) / kWaves;
  const int64_t want = ((int64_t)d.R * d.S + kXcdsMove - 1) / kXcdsMove * kXcdsMove * wpt;
  if (d.num_cus > 0) {
    // a CU budget: the whole grid (padding and token items) within it
    g.xcd_local = 0;
    g.item_blocks = 0;
    g.blocks = capped_grid(c, g.npad_used + want);
  } else {
    g.xcd_local = 1;
    g.item_blocks = (int)want;
    g.blocks = want + g.npad_used;
  }
  return g;
}

int64_t combine_grid(const Ctx& c, int W) {
  const int nchunks = (W / 8 + 64 * kCombVecs - 1) / (64 * kCombVecs);
  return capped_grid(c, ((int64_t)c.d.R * c.d.S * nchunks + kWaves - 1) / kWaves);
}

int64_t copy_grid(const Ctx& c) {
  return capped_grid(c, ((int64_t)c.d.R * c.d.NvS + kWaves - 1) / kWaves);
}

// three workgroups (projections) per 16 KiB column chunk; a CU budget makes them loop over chunks
int64_t prefetch_grid(const Ctx& c) {
  return capped_grid(c, 3LL * prefetch_chunks(c.d)) / 3 * 3;
}

// at most eight workgroups per CU of the device, fewer when there are fewer work items
int64_t reduce_grad_grid(const Ctx& c) {
  const Dims& d = c.d;
  const int64_t max_items = (int64_t)d.R * d.B * 3 * reduce_chunks(d);
  const int64_t dev = (int64_t)c.num_cu_device * 8;
  return capped_grid(c, max_items < dev ? max_items : dev);
}

hipError_t launch_dispatch(const Ctx& c, const moonep_plan_t& p, const uint16_t* x,
                           int W, const float* rw, uint16_t* x_nvs, float* rw_nvs,
                           hipStream_t s) {
  const Dims& d = c.d;
  DispatchArgs a;
  a.x = (const u32x4*)x; a.rw = rw; a.x_nvs = (u32x4*)x_nvs; a.rw_nvs = rw_nvs;
  a.dest = p.dest; a.cu = p.cu_seqlens; a.segn = p.seg_tokens; a.act = p.aux + d.aux.act;
  a.ntok = d.R * d.S; a.K = d.K; a.nv = W / 8; a.EB = d.E + d.B; a.L2 = 2 * d.L;
  a.tp = d.tp; a.NvS = (int)d.NvS;
  const DispatchGrid g = dispatch_grid(c, W);
  a.pad_parts = g.pad_parts;
  a.npad_used = g.npad_used;
  a.xcd_local = g.xcd_local;
  a.item_blocks = g.item_blocks;
  dispatch_kernel<<<(unsigned)g.blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const Ctx& c, const moonep_plan_t& p, const uint16_t* y, int W,
                          const float* rw_nvs, uint16_t* out, float* rw_sk, hipStream_t s) {
  const Dims& d = c.d;
  CombineArgs a;
  a.y = (const u32x4*)y; a.rw_nvs = rw_nvs; a.out = (u32x4*)out; a.rw_sk = rw_sk;
  a.dest = p.dest; a.ntok = d.R * d.S; a.K = d.K; a.nv = W / 8;
  const unsigned blocks = (unsigned)combine_grid(c, W);
  if (rw_nvs)
    combine_kernel<true><<<blocks, kThreads, 0, s>>>(a);
  else
    combine_kernel<false><<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const Ctx& c, const moonep_plan_t& p, const uint16_t* src, int W,
                            uint16_t* dst, hipStream_t s) {
  const Dims& d = c.d;
  CopyArgs a;
  a.src = (const u32x4*)src; a.dst = (u32x4*)dst; a.cu = p.cu_seqlens;
  a.R = d.R; a.EB = d.E + d.B; a.nv = W / 8; a.NvS = (int)d.NvS;
  const unsigned blocks = (unsigned)copy_grid(c);
  copy_rows_kernel<<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefetch(const Ctx& c, const moonep_plan_t& p, const WeightRef& w,
                           hipStream_t s) {
  const Dims& d = c.d;
  PrefetchArgs a;
  for (int i = 0; i < 3; ++i) {
    a.home[i] = (const u32x4*)w.home[i];
    a.pool[i] = (u32x4*)w.pool[i];
  }
  a.hstride = w.home_stride;
  a.pstride = w.pool_stride;
  a.B = d.B;
  a.pf = p.prefetch_src;
  a.aux_pf = p.aux + d.aux.pf;
  a.aux_pf_n = p.aux + d.aux.pf_n;
  a.row_vecs = (int64_t)d.H * d.Hp / 8;
  a.nchunks = prefetch_chunks(d);
  const unsigned blocks = (unsigned)prefetch_grid(c);
  prefetch_kernel<<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_reduce_grad(const Ctx& c, const moonep_plan_t& p, float* const gh[3],
                              float* const rb[3], hipStream_t s) {
  const Dims& d = c.d;
  ReduceArgs a;
  for (int i = 0; i < 3; ++i) {
    a.gh[i] = (f32x4*)gh[i];
    a.rb[i] = (f32x4*)rb[i];
  }
  a.dup_n = p.aux + d.aux.dup_n;
  a.dup_e = p.aux + d.aux.dup_e;
  a.dup_first = p.aux + d.aux.dup_first;
  a.dup_cnt = p.aux + d.aux.dup_cnt;
  a.hold = p.aux + d.aux.hold;
  a.row_vecs = (int64_t)d.H * d.Hp / 4;
  a.chunk_vecs = kReduceChunkVecs;
  a.nchunks = reduce_chunks(d);
  const unsigned blocks = (unsigned)reduce_grad_grid(c);
  reduce_grad_kernel<<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moonep
