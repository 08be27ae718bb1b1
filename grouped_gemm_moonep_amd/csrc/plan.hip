// Balanced redundant-expert planner on gfx950.
//
// What the planner must guarantee comes from the MoonEP README (MoonshotAI/
// MoonEP mirror): every EP rank receives exactly S*K token slots (item 1),
// planning runs on the GPU straight from the router output (item 2), a rank
// duplicates experts of at most one remote home group so B = E/R slots are
// enough for training ("How to set B"), dispatched tokens are grouped by the
// row of the [E+B,H,H'] weight tensor and cu_seqlens holds each row's padded
// end offset ("API guide > dispatch fwd").  The pages do not print the
// algorithm; the kernels implement this spec:
//   group loads W_g, keep_g = min(W_g, S*K); donors by larger excess, then
//   lower id; receivers by larger deficit, then lower id; a donor gives each
//   receiver its whole need, and when its remaining excess is short it gives
//   anyway, shrinks its own keep and queues itself for the shortfall;
//   the experts of a group are laid on a line by (load, id); the line is cut
//   into the home piece [0, keep) and the donations in order; tokens of an
//   expert are ordered by (rank, token); home experts use their own row,
//   remote experts rows E, E+1, ... in ascending id while slots last, and
//   their home row beyond B; rows are padded to token_padding.
//
// Three kernels, all on the caller's stream:
//   plan_hist   (R x chunks workgroups): per-chunk expert counts from 64-bit
//                LDS lane masks (order-independent), routing validation;
//   plan_solve  (one workgroup of 1024 threads): counts, loads, lines, the
//                serial chain-greedy (at most 2R steps), each rank's active
//                rows with their padded ends, prefetch slots;
//   plan_assign (R x chunks workgroups): stable rank of each token among the
//                earlier tokens of the same expert (popcount of the lane
//                masks below it), its line position (the chunk's base summed
//                from the earlier chunks' counts), piece, row and slot;
//                padding slots get src = -1.  At the same time one more
//                workgroup per rank writes that rank's cu_seqlens and
//                seg_tokens and builds its grouped-GEMM tile schedule
//                (tile_schedule.h), and one more the reduce_grad tables:
//                work that only reads the solve's results, kept off its
//                single workgroup.
#include "internal.h"
#include "tile_schedule.h"

namespace moonep {
namespace {

constexpr int kSolveThreads = 1024;

struct PlanArgs {
  int R, S, K, E, B, L, tp, nch, max_tiles;
  int NvS;
  const int32_t* topk;
  const int32_t* tpe;
  int32_t* cc;
  int32_t* chunk_err;
  int32_t* shift;
  int32_t* pieces;
  int32_t* npieces;
  int32_t* line;
  int32_t* efix;
  int32_t* aend;      // [R][2L] padded end slot of each rank's active row q
  int32_t* an;        // [R][2L] real tokens of each rank's active row q
  int32_t* rend;      // [R] end of each rank's last segment (its used slots)
  int32_t* counts;
  int32_t* dest;
  int32_t* src;
  int32_t* cu;
  int32_t* segn;
  int32_t* pf;
  int32_t* stats;
  int32_t* aux;
  AuxLayout ax;
};

__device__ __forceinline__ int round_up(int n, int m) { return (n + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// plan_hist: one workgroup per (chunk of 256 tokens, rank).  Lane l of wave w
// sets bit l of mask[w][e] for each of its experts; the old value of the OR
// tells whether the token already named e (a repeated id).
__global__ __launch_bounds__(kPlanChunk) void plan_hist(PlanArgs a) {
  __shared__ unsigned long long mask[4][kMaxE];
  __shared__ int s_err;
  const int ch = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < 4 * a.E; i += kPlanChunk) mask[i / a.E][i % a.E] = 0ull;
  if (tid == 0) s_err = 0;
  __syncthreads();
  const int s = ch * kPlanChunk + tid;
  const int w = tid >> 6;
  const unsigned long long bit = 1ull << (tid & 63);
  int err = 0;
  if (s < a.S) {
    const int32_t* t = a.topk + ((int64_t)r * a.S + s) * a.K;
    for (int k = 0; k < a.K; ++k) {
      const int e = t[k];
      if ((unsigned)e >= (unsigned)a.E) {
        err |= MOONEP_ROUTE_ID_RANGE;
      } else {
        const unsigned long long old = atomicOr(&mask[w][e], bit);
        if (old & bit) err |= MOONEP_ROUTE_REPEAT;
      }
    }
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  int32_t* out = a.cc + ((int64_t)r * a.nch + ch) * a.E;
  for (int e = tid; e < a.E; e += kPlanChunk)
    out[e] = __popcll(mask[0][e]) + __popcll(mask[1][e]) + __popcll(mask[2][e]) +
             __popcll(mask[3][e]);
  if (tid == 0) a.chunk_err[r * a.nch + ch] = s_err;
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of two values at once over all kSolveThreads
// threads (16 waves): a shuffle scan within each wave, then wave 0 scans the
// 16 wave totals with shuffles.  Two barriers.  scratch holds 64 ints; its
// halves are written and read on either side of the first barrier of the
// next call, so back-to-back calls need no barrier in between.
constexpr int kSolveWaves = kSolveThreads / 64;
__device__ __forceinline__ void block_scan2(int x, int y, int* ex, int* ey, int* tx, int* ty,
                                            int* scratch /*[64]*/) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int ix = x, iy = y;
  for (int o = 1; o < 64; o <<= 1) {
    const int ax = __shfl_up(ix, o, 64), ay = __shfl_up(iy, o, 64);
    if (lane >= o) {
      ix += ax;
      iy += ay;
    }
  }
  if (lane == 63) {
    scratch[wv] = ix;
    scratch[kSolveWaves + wv] = iy;
  }
  __syncthreads();
  if (wv == 0) {
    int sx = lane < kSolveWaves ? scratch[lane] : 0;
    int sy = lane < kSolveWaves ? scratch[kSolveWaves + lane] : 0;
    for (int o = 1; o < kSolveWaves; o <<= 1) {
      const int ax = __shfl_up(sx, o, 64), ay = __shfl_up(sy, o, 64);
      if (lane >= o) {
        sx += ax;
        sy += ay;
      }
    }
    if (lane < kSolveWaves) {
      scratch[2 * kSolveWaves + lane] = sx;        // inclusive prefixes of the wave totals
      scratch[3 * kSolveWaves + lane] = sy;
    }
  }
  __syncthreads();
  *ex = (wv ? scratch[2 * kSolveWaves + wv - 1] : 0) + ix - x;
  *ey = (wv ? scratch[3 * kSolveWaves + wv - 1] : 0) + iy - y;
  *tx = scratch[3 * kSolveWaves - 1];
  *ty = scratch[4 * kSolveWaves - 1];
}

// Sums of two (rank, expert) columns of the chunk counts (chunk c at col[c E]),
// KB chunks of each in flight at a time: unconditional loads, the indices
// clamped into the column and the surplus masked afterwards (a load under a
// condition becomes a branch with a wait after it).
template <int KB>
__device__ __forceinline__ void column_sums(const int32_t* col0, const int32_t* col1, bool has1,
                                            int nch, int E, int& run0, int& run1) {
  for (int ch0 = 0; ch0 < nch; ch0 += KB) {
    int v0[KB], v1[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int c = min(ch0 + u, nch - 1);
      v0[u] = col0[(int64_t)c * E];
      v1[u] = col1[(int64_t)c * E];
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const bool ok = ch0 + u < nch;
      run0 += ok ? v0[u] : 0;
      run1 += ok && has1 ? v1[u] : 0;
    }
  }
}

// Wave-wide sum (all 64 lanes get it).
__device__ __forceinline__ int wave_sum(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// plan_solve: the single-workgroup part.
__global__ __launch_bounds__(kSolveThreads) void plan_solve(PlanArgs a) {
  __shared__ int T[kMaxE];
  __shared__ int aline[kMaxE];
  __shared__ int W[kMaxR], keep[kMaxR], X[kMaxR], need[kMaxR];
  __shared__ int donors[kMaxR], queue[2 * kMaxR + 2];
  __shared__ int recv_g[kMaxR], recv_lo[kMaxR], recv_hi[kMaxR];
  __shared__ int ent_n[2 * kMaxE], ent_lo[2 * kMaxE], ent_row[2 * kMaxE];
  __shared__ int act_row[2 * kMaxE];
  __shared__ int nact[kMaxR], nrem[kMaxR], npf[kMaxR], pfpre[kMaxR];
  __shared__ int ord_len[3 * kMaxE], ord_ent[3 * kMaxE], ord_cnt[3 * kMaxE];  // phase F
  __shared__ int scan_scratch[4 * kSolveWaves];
  __shared__ int s_err, s_maxload, s_ndon, s_dups, s_pad, s_nd, s_nq;

  const int tid = threadIdx.x;
  const int R = a.R, E = a.E, L = a.L, B = a.B, nch = a.nch;
  const int C = a.S * a.K;
  const int RE = R * E;
  if (tid == 0) {
    s_err = 0; s_maxload = 0; s_ndon = 0; s_dups = 0; s_pad = 0; s_nd = 0; s_nq = 0;
  }
  for (int e = tid; e < E; e += kSolveThreads) T[e] = 0;
  // phase F's visit-order slots and per-rank counts (cleared here, where a
  // barrier follows anyway)
  const int S3 = 3 * L;
  const int nslot = R * S3;
  for (int i = tid; i < nslot; i += kSolveThreads) {
    ord_len[i] = 0;
    ord_ent[i] = -1;
  }
  for (int d = tid; d < R; d += kSolveThreads) {
    nrem[d] = 0;
    npf[d] = 0;
  }
  __syncthreads();

  // Phase A: counts per (r, e) summed over the chunks and the expert loads
  // T_e (an order-independent integer sum in LDS).  Two (r, e) columns per
  // pass with all their chunk loads in flight together, and the per-chunk
  // error bits loaded beside them.  (Each plan_assign workgroup sums the
  // chunks before its own, so nothing is written back here.)
  {
    // the first 1024 chunks' error bits load beside the counts (a loop of its
    // own would wait for them first)
    int cerr = a.chunk_err[min(tid, R * nch - 1)];
    for (int i = tid + kSolveThreads; i < R * nch; i += kSolveThreads) cerr |= a.chunk_err[i];
    for (int i0 = tid; i0 < RE; i0 += 2 * kSolveThreads) {
      const int i1 = i0 + kSolveThreads;
      const bool has1 = i1 < RE;
      const int32_t* col0 = a.cc + (int64_t)(i0 / E) * nch * E + (i0 % E);
      const int32_t* col1 = has1 ? a.cc + (int64_t)(i1 / E) * nch * E + (i1 % E) : col0;
      int run0 = 0, run1 = 0;
      column_sums<16>(col0, col1, has1, nch, E, run0, run1);
      a.counts[i0] = run0;
      atomicAdd(&T[i0 % E], run0);
      if (a.tpe && a.tpe[i0] != run0) cerr |= MOONEP_ROUTE_COUNTS;
      if (has1) {
        a.counts[i1] = run1;
        atomicAdd(&T[i1 % E], run1);
        if (a.tpe && a.tpe[i1] != run1) cerr |= MOONEP_ROUTE_COUNTS;
      }
    }
    if (cerr) atomicOr(&s_err, cerr);
  }
  __syncthreads();
  const int err = s_err;

  if (err) {
    // Safe no-op plan: no segment, no prefetch, every token keeps a slot in
    // its own rank's region (written by plan_assign).
    for (int i = tid; i < R * (E + B); i += kSolveThreads) { a.cu[i] = 0; a.segn[i] = 0; }
    for (int i = tid; i < R * B; i += kSolveThreads) a.pf[i] = -1;
    for (int i = tid; i < 2 * E; i += kSolveThreads) a.aux[a.ax.act + i] = -1;
    for (int d = tid; d < R; d += kSolveThreads) {
      a.aux[a.ax.nact + d] = 0;
      a.rend[d] = 0;
    }
    if (tid == 0) {
      a.aux[a.ax.pf_n] = 0;
      a.aux[a.ax.dup_n] = 0;
      a.stats[MOONEP_STAT_ERROR] = err;
      for (int i = 1; i < MOONEP_STAT_FIXED; ++i) a.stats[i] = 0;
      for (int r = 0; r < R; ++r) {
        a.stats[MOONEP_STAT_REMOTE_GROUP + r] = -1;
        a.stats[MOONEP_STAT_REMOTE_GROUP + R + r] = 0;
      }
    }
    return;
  }

  // Phase C: line start of every expert (experts of a group by (T, id)), the
  // group loads W_g and the largest load.
  // Four lanes per expert (adjacent lanes of one wave), each scanning a
  // quarter of the group, then summed with shuffles; the group loads from
  // the same quarters (lanes of the group's first expert).
  {
    int mx = 0;
    for (int e0 = 0; e0 < E; e0 += kSolveThreads / 4) {
      const int e = e0 + (tid >> 2), part = tid & 3;
      int acc = 0, tot = 0, te = 0;
      if (e < E) {
        const int g = e / L;
        te = T[e];
        const int f0 = g * L + (part * L) / 4, f1 = g * L + ((part + 1) * L) / 4;
        // eight loads in flight, then their sums (read one by one, each LDS
        // read's latency was exposed)
        for (int b = f0; b < f1; b += 8) {
          int tf[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) tf[u] = T[min(b + u, E - 1)];   // masked below
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int f = b + u;
            const int v = f < f1 ? tf[u] : 0;
            acc += (v < te || (v == te && f < e)) ? v : 0;
            tot += v;
          }
        }
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      tot += __shfl_xor(tot, 1, 64);
      tot += __shfl_xor(tot, 2, 64);
      if (e < E && part == 0) {
        aline[e] = acc;
        a.line[e] = acc;
        if (e % L == 0) W[e / L] = tot;
      }
      mx = max(mx, te);
    }
    // the largest load: a wave maximum, then one LDS atomic per wave
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
    if ((tid & 63) == 0 && mx > 0) atomicMax(&s_maxload, mx);
  }
  __syncthreads();

  // Phase D: keep/excess/deficit per group; each group finds its position
  // among the donors (by (-X, g)) and the receivers (by (-D, r)) from the
  // group loads directly; then the chain-greedy itself (one thread, at most
  // 2R steps); then the line pieces of every group (one thread per group).
  for (int g = tid; g < R; g += kSolveThreads) {
    const int wg = W[g];
    const int xg = wg > C ? wg - C : 0, dg = wg < C ? C - wg : 0;
    keep[g] = wg < C ? wg : C;
    X[g] = xg;
    need[g] = dg;
    recv_g[g] = -1;
    recv_lo[g] = 0;
    recv_hi[g] = 0;
    int pd = 0, pr = 0;
    for (int h0 = 0; h0 < R; h0 += 8) {             // eight loads in flight
      int wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) wv[u] = W[min(h0 + u, R - 1)];     // masked below
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int h = h0 + u, wh = h < R ? wv[u] : C;   // past R: neither donor nor receiver
        const int xh = wh > C ? wh - C : 0, dh = wh < C ? C - wh : 0;
        pd += xh > 0 && (xh > xg || (xh == xg && h < g));
        pr += dh > 0 && (dh > dg || (dh == dg && h < g));
      }
    }
    if (xg > 0) {
      donors[pd] = g;
      atomicAdd(&s_nd, 1);
    }
    if (dg > 0) {
      queue[pr] = g;
      atomicAdd(&s_nq, 1);
    }
  }
  __syncthreads();
  // The chain-greedy itself, on wave 0 with its state in registers: lane j
  // holds queue entry j, donor j (by position) and its excess, group j's
  // need, keep and donation count, and donation j once made; every step reads
  // and writes single lanes (readlane, a lane select) instead of LDS, whose
  // latency made up the loop's time.  The queue never exceeds R entries (the
  // initial receivers plus each donor at most once) and there are at most R
  // donations, so one lane each suffices (R <= 64).  A donor's donations are
  // consecutive, so each starts at the donor's final keep plus what the donor
  // gave before it.
  if (tid < 64) {
    const int lane = tid;
    // lane `at` of v becomes val (at is wave-uniform)
    auto writelane = [lane](int val, int at, int v) { return lane == at ? val : v; };
    const int nd = s_nd, nq = s_nq;
    int qv = lane < nq ? queue[lane] : 0;
    const int dv = lane < nd ? donors[lane] : 0;
    const int dx = lane < nd ? X[dv] : 0;
    int needv = lane < R ? need[lane] : 0;
    int keepv = lane < R ? keep[lane] : 0;
    int cntv = 0;
    int dong = 0, donr = 0, dona = 0, donc = 0, donk = 0;
    int qt = nq, qh = 0, ndon = 0, i = 0, given = 0, k = 0, bad = 0;
    int x = nd ? __builtin_amdgcn_readlane(dx, 0) : 0;
    while (qh < qt) {
      const int r = __builtin_amdgcn_readlane(qv, qh);
      ++qh;
      const int dn = __builtin_amdgcn_readlane(needv, r);
      if (i >= nd || ndon >= R) { bad = 1; break; }
      const int g = __builtin_amdgcn_readlane(dv, i);
      dong = writelane(g, ndon, dong);
      donr = writelane(r, ndon, donr);
      dona = writelane(dn, ndon, dona);
      donc = writelane(given, ndon, donc);
      donk = writelane(k, ndon, donk);
      cntv = writelane(k + 1, g, cntv);
      ++ndon;
      given += dn;
      ++k;
      if (dn <= x) {
        x -= dn;
        if (x == 0 && i + 1 < nd) {
          ++i;
          x = __builtin_amdgcn_readlane(dx, i);
          given = 0;
          k = 0;
        }
      } else {
        const int sh = dn - x;
        keepv = writelane(__builtin_amdgcn_readlane(keepv, g) - sh, g, keepv);
        needv = writelane(sh, g, needv);
        if (qt >= 64) { bad = 1; break; }
        qv = writelane(g, qt, qv);
        ++qt;
        ++i;
        x = i < nd ? __builtin_amdgcn_readlane(dx, i) : 0;
        given = 0;
        k = 0;
      }
    }
    // pieces of every group's line: [0, keep) to the home rank, then the
    // group's donations in emission order
    const int kg = __shfl(keepv, dong, 64);              // final keep of donation lane's donor
    if (lane < ndon) {
      const int lo = kg + donc, hi = lo + dona;
      int32_t* pg = a.pieces + (int64_t)dong * (R + 1) * 2;
      const int pi = (kg > 0 ? 1 : 0) + donk;
      pg[2 * pi] = hi;
      pg[2 * pi + 1] = donr;
      recv_g[donr] = dong;        // each rank receives from at most one group
      recv_lo[donr] = lo;
      recv_hi[donr] = hi;
    }
    if (lane < R) {
      int32_t* pg = a.pieces + (int64_t)lane * (R + 1) * 2;
      if (keepv > 0) {
        pg[0] = keepv;
        pg[1] = lane;
      }
      a.npieces[lane] = (keepv > 0 ? 1 : 0) + cntv;
      keep[lane] = keepv;
    }
    if (lane == 0) {
      s_ndon = ndon;
      if (bad) s_err = 8;   // internal: inconsistent counts (cannot happen)
    }
  }
  __syncthreads();

  // Phase E: tokens of each candidate expert on each rank: entry (d, i),
  // i < L home expert d*L+i against [0, keep_d); i >= L the i-L-th expert of
  // the group rank d receives from, against the received piece.
  const int L2 = 2 * L;
  for (int idx = tid; idx < R * L2; idx += kSolveThreads) {
    const int d = idx / L2, i = idx - (idx / L2) * L2;
    int e, lo, hi;
    if (i < L) {
      e = d * L + i; lo = 0; hi = keep[d];
    } else if (recv_g[d] >= 0) {
      e = recv_g[d] * L + (i - L); lo = recv_lo[d]; hi = recv_hi[d];
    } else {
      e = -1; lo = 0; hi = 0;
    }
    int n = 0, rlo = 0;
    if (e >= 0) {
      const int a0 = aline[e], a1 = aline[e] + T[e];
      rlo = a0 > lo ? a0 : lo;
      const int rhi = a1 < hi ? a1 : hi;
      n = rhi > rlo ? rhi - rlo : 0;
    }
    ent_n[idx] = n;
    ent_lo[idx] = rlo;
  }
  __syncthreads();
  // Rows: home experts use their own row; the j-th remote expert with tokens
  // (ascending id) prefetch row E+j while j < B, its home row after that.
  // Phase F starts in the same loop: each rank's active rows are laid out in
  // ascending row order, the lower group's rows first (the rank's home
  // experts or the remote experts that keep home rows), prefetch rows last;
  // every active entry takes a visit-order slot (3L per rank), and one
  // block-wide scan over all slots (below) gives each row's start and its
  // index among the rank's active rows.  Per rank: its remote experts and
  // used prefetch rows.
  for (int idx = tid; idx < R * L2; idx += kSolveThreads) {
    const int d = idx / L2, i = idx - (idx / L2) * L2;
    const int n = ent_n[idx];
    int row = -1;
    if (n > 0) {
      if (i < L) {
        row = d * L + i;
      } else {
        int j = 0;
        for (int q0 = L; q0 < i; q0 += 8) {          // eight loads in flight
          int nv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) nv[u] = ent_n[d * L2 + min(q0 + u, L2 - 1)];   // masked below
#pragma unroll
          for (int u = 0; u < 8; ++u) j += q0 + u < i && nv[u] > 0;
        }
        row = j < B ? E + j : recv_g[d] * L + (i - L);
      }
      const int g = recv_g[d];
      const bool home_first = g < 0 || d < g;
      const bool pf = row >= E;
      int o;
      if (i < L) o = (home_first ? 0 : L) + i;
      else if (pf) o = 2 * L + (i - L);
      else o = (home_first ? L : 0) + (i - L);
      ord_len[d * S3 + o] = round_up(n, a.tp);
      ord_ent[d * S3 + o] = idx;
      if (i >= L) atomicAdd(&nrem[d], 1);    // the rank's remote experts
      if (pf) atomicAdd(&npf[d], 1);         // of which in prefetch rows
    }
    ent_row[idx] = row;
  }
  __syncthreads();

  int tot_cnt, tot_len;
  {
    const int per = (nslot + kSolveThreads - 1) / kSolveThreads;
    const int b0 = min(nslot, tid * per), b1 = min(nslot, b0 + per);
    int sl = 0, sc = 0;
    for (int i = b0; i < b1; ++i) { sl += ord_len[i]; sc += ord_ent[i] >= 0; }
    int pl, pc;
    block_scan2(sl, sc, &pl, &pc, &tot_len, &tot_cnt, scan_scratch);
    for (int i = b0; i < b1; ++i) {          // exclusive prefixes, in place
      const int l = ord_len[i];
      ord_len[i] = pl;
      ord_cnt[i] = pc;
      pl += l;
      pc += ord_ent[i] >= 0;
    }
  }
  __syncthreads();
  {
    int pad = 0;
    for (int i = tid; i < nslot; i += kSolveThreads) {
      const int idx = ord_ent[i];
      if (idx < 0) continue;
      const int d = i / S3;
      const int q = ord_cnt[i] - ord_cnt[d * S3];
      const int start = ord_len[i] - ord_len[d * S3];
      const int n = ent_n[idx];
      const int len = round_up(n, a.tp);
      const int row = ent_row[idx];
      const int ie = idx - d * L2;
      const bool home = ie < L;
      const int e = home ? d * L + ie : recv_g[d] * L + (ie - L);
      a.shift[d * E + e] = start - ent_lo[idx];
      // an expert all of whose tokens land here: the assignment needs no piece search
      a.efix[2 * e] = n == T[e] ? d : -1;
      if (n == T[e]) a.efix[2 * e + 1] = start - ent_lo[idx];
      act_row[d * L2 + q] = row;
      a.aend[d * L2 + q] = start + len;
      a.an[d * L2 + q] = n;
      if (row >= E) a.pf[d * B + (row - E)] = e;
      pad += len - n;
    }
    pad = wave_sum(pad);
    if ((tid & 63) == 0 && pad) atomicAdd(&s_pad, pad);
  }
  // per rank, in the same pass (it reads only the scan's prefixes and the
  // counts of the rows loop)
  for (int d = tid; d < R; d += kSolveThreads) {
    // the used prefetch rows of the ranks before d (eight loads in flight)
    int pre = 0;
    for (int h0 = 0; h0 < d; h0 += 8) {
      int nv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) nv[u] = npf[min(h0 + u, R - 1)];   // masked below
#pragma unroll
      for (int u = 0; u < 8; ++u) pre += h0 + u < d ? nv[u] : 0;
    }
    pfpre[d] = pre;
    const int next = d + 1 < R ? ord_cnt[(d + 1) * S3] : tot_cnt;
    nact[d] = next - ord_cnt[d * S3];
    a.aux[a.ax.nact + d] = nact[d];
    // the rank's segments lie back to back from slot 0
    a.rend[d] = (d + 1 < R ? ord_len[(d + 1) * S3] : tot_len) - ord_len[d * S3];
    const int rem = nrem[d];
    a.stats[MOONEP_STAT_REMOTE_GROUP + d] = rem ? recv_g[d] : -1;
    a.stats[MOONEP_STAT_REMOTE_GROUP + R + d] = rem;
    atomicAdd(&s_dups, rem);
  }
  __syncthreads();
  for (int i = tid; i < R * B; i += kSolveThreads) {
    const int d = i / B, j = i - (i / B) * B;
    if (j >= npf[d]) a.pf[i] = -1;
    else a.aux[a.ax.pf + pfpre[d] + j] = i;      // used prefetch slots in (d, j) order
  }
  for (int i = tid; i < R * L2; i += kSolveThreads) {
    const int d = i / L2, q = i - (i / L2) * L2;
    a.aux[a.ax.act + i] = q < nact[d] ? act_row[i] : -1;
    if (q >= nact[d]) a.an[i] = 0;              // entries past the active rows hold no tokens
  }
  if (tid == 0) a.aux[a.ax.pf_n] = R > 0 ? pfpre[R - 1] + npf[R - 1] : 0;

  if (tid == 0) {
    a.stats[MOONEP_STAT_ERROR] = s_err;
    a.stats[MOONEP_STAT_DUPS] = s_dups;
    a.stats[MOONEP_STAT_MAX_LOAD] = s_maxload;
    a.stats[MOONEP_STAT_DONATIONS] = s_ndon;
    a.stats[MOONEP_STAT_PAD_ROWS] = s_pad;
    const float tbar = (float)((double)R * a.S * a.K / E);
    const float mv = (float)((double)s_maxload / tbar - 1.0);
    a.stats[MOONEP_STAT_MAXVIO] = __float_as_int(mv);
    a.stats[6] = 0;
    a.stats[7] = 0;
  }
}

// ---------------------------------------------------------------------------
// plan_assign: one workgroup per (chunk, rank).
constexpr int kShiftLds = 4096;     // shift table staged in LDS up to R*E ints
constexpr int kPiecesLds = 1024;    // piece table staged in LDS up to this many ints

__global__ __launch_bounds__(kPlanChunk) void plan_assign(PlanArgs a) {
  const int tid = threadIdx.x;
  const int L2 = 2 * a.L, EB = a.E + a.B;
  if ((int)blockIdx.x == a.nch) {
    // the grid's first extra column: rank d's cu_seqlens and seg_tokens, then its
    // grouped-GEMM tile schedule, both from plan_solve's active rows, alongside the
    // token assignment
    __shared__ int s_act[2 * kMaxE], s_aend[2 * kMaxE], s_an[2 * kMaxE];
    __shared__ int wsum[4];
    __shared__ TileSchedLds sl;
    const int d = blockIdx.y;
    if (a.stats[MOONEP_STAT_ERROR] == 0) {     // (a failed plan has its zeros already)
      const int na = a.aux[a.ax.nact + d];
      for (int q = tid; q < na; q += kPlanChunk) {
        s_act[q] = a.aux[a.ax.act + d * L2 + q];
        s_aend[q] = a.aend[d * L2 + q];
        s_an[q] = a.an[d * L2 + q];
      }
      __syncthreads();
      // each row's entry: the end of the last active row at or below it (the rows are
      // ascending), its token count if it is active itself
      for (int row = tid; row < EB; row += kPlanChunk) {
        int lo = 0, hi = na;                   // first q with s_act[q] > row lies in [lo, hi]
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_act[mid] <= row) lo = mid + 1;
          else hi = mid;
        }
        a.cu[d * EB + row] = lo > 0 ? s_aend[lo - 1] : 0;
        a.segn[d * EB + row] = lo > 0 && s_act[lo - 1] == row ? s_an[lo - 1] : 0;
      }
    }
    build_tile_schedule(a.aux + a.ax.act, a.aend, a.an, a.aux + a.ax.tiles,
                        a.aux + a.ax.ntiles, a.aux + a.ax.nfull, d, L2, a.tp, a.max_tiles,
                        wsum, sl);
    return;
  }
  if ((int)blockIdx.x == a.nch + 1) {
    // the second extra column (one workgroup): the reduce_grad tables.  The home
    // experts that have prefetch copies (ascending), the first holder of each and
    // their count, and the holder slots d B + j of each expert in ascending rank.
    // Rank d holds expert e in slot j iff prefetch_src[d B + j] = e, at most once.
    if (blockIdx.y != 0 || a.stats[MOONEP_STAT_ERROR] != 0) return;
    __shared__ int hcnt[kMaxE], hfirst[kMaxE];
    __shared__ unsigned long long hmask[kMaxE];
    __shared__ int wsum[4];
    const int E = a.E, RB = a.R * a.B;
    for (int e = tid; e < E; e += kPlanChunk) {
      hcnt[e] = 0;
      hmask[e] = 0ull;
    }
    constexpr int kPer = kMaxE / kPlanChunk;   // R B <= E <= kMaxE slots, kPer per thread
    int pe[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kPlanChunk;
      pe[u] = i < RB ? a.pf[i] : -1;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (pe[u] >= 0) {
        const int d = (tid + u * kPlanChunk) / a.B;
        atomicAdd(&hcnt[pe[u]], 1);
        atomicOr(&hmask[pe[u]], 1ull << d);
      }
    __syncthreads();
    // one exclusive scan over the experts (kPer consecutive ones per thread) of
    // (has copies) in the low 16 bits and (copies) in the high 16 (each total <= E)
    int v[kPer], sum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid * kPer + u;
      const int c = e < E ? hcnt[e] : 0;
      v[u] = (c > 0 ? 1 : 0) | (c << 16);
      sum += v[u];
    }
    int total;
    int run = block_scan256(sum, &total, wsum);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid * kPer + u;
      if (e < E && v[u] != 0) {
        const int q = run & 0xFFFF, first = run >> 16;
        a.aux[a.ax.dup_e + q] = e;
        a.aux[a.ax.dup_first + q] = first;
        a.aux[a.ax.dup_cnt + q] = v[u] >> 16;
        hfirst[e] = first;
      }
      run += v[u];
    }
    if (tid == 0) a.aux[a.ax.dup_n] = total & 0xFFFF;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (pe[u] >= 0) {
        const int i = tid + u * kPlanChunk, d = i / a.B;
        const int k = __popcll(hmask[pe[u]] & ((1ull << d) - 1ull));
        a.aux[a.ax.hold + hfirst[pe[u]] + k] = i;
      }
    return;
  }
  __shared__ unsigned long long mask[4][kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ int s_shift[kShiftLds];
  __shared__ int s_pieces[kPiecesLds];
  __shared__ int s_np[kMaxR];
  __shared__ int s_plo[kPlanChunk], s_phi[kPlanChunk];
  __shared__ int s_efix[2 * kMaxE];
  const int ch = blockIdx.x, r = blockIdx.y;
  const int s = ch * kPlanChunk + tid;
  const int w = tid >> 6, lane = tid & 63;
  const unsigned long long bit = 1ull << lane;
  const int64_t tok = (int64_t)r * a.S + s;
  // the lookup tables of this chunk, staged in LDS when they fit
  const int npc = a.R * (a.R + 1) * 2;
  const bool tab = a.R * a.E <= kShiftLds && npc <= kPiecesLds;
  // Every global load of the staging is issued before the first value is
  // used, so the workgroup waits for one round of memory latency (the
  // tables were written by the previous kernel, possibly on another XCD):
  // this token's expert ids; the padding of this thread's active row (rows
  // ch, ch + nch, ... of the rank: thread t takes row ch + t nch, its padded
  // end and token count; entries past the rank's active rows have no tokens)
  // and the end of the rank's last segment; for this thread's first expert
  // the line start, up to 16 earlier chunks and 8 lower ranks (the chunk's
  // line position of the expert is their sum); the first entries of the
  // per-expert shortcut, shift and piece tables.  Larger shapes load the
  // rest in further rounds.  The loads do not wait for the plan's error flag
  // (they stay in bounds whatever the tables hold).
  int ids[kMaxK];
  if ((a.K & 3) == 0 && ((uintptr_t)a.topk & 15) == 0) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int k = 0; k < kMaxK; k += 4) {
      i32x4 v = {0, 0, 0, 0};
      if (s < a.S && k < a.K) v = *(const i32x4*)(a.topk + tok * a.K + k);
      ids[k] = v[0]; ids[k + 1] = v[1]; ids[k + 2] = v[2]; ids[k + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) ids[k] = (s < a.S && k < a.K) ? a.topk[tok * a.K + k] : 0;
  }
  const int q_pad = ch + tid * a.nch;
  const int pad_end = q_pad < L2 ? a.aend[r * L2 + q_pad] : 0;
  const int pad_n = q_pad < L2 ? a.an[r * L2 + q_pad] : 0;
  const int last = a.rend[r];
  const int RE = a.R * a.E;
  constexpr int kShiftU = 12;                      // shift entries per thread in the first round
  constexpr int kEfixU = 4;                        // shortcut entries per thread in the first round
  // experts tid and tid + 256 (the second only when E > 256); indices are
  // clamped into range and the surplus masked when summing, so no load sits
  // under a lane condition
  const int32_t* colr = a.cc + (int64_t)r * a.nch * a.E;   // chunk c of expert e at colr[c E + e]
  const int cmax = ch > 0 ? ch - 1 : 0, rmax = r > 0 ? r - 1 : 0;
  const bool two = a.E > kPlanChunk;
  const int ex0 = min(tid, a.E - 1), ex1 = min(tid + kPlanChunk, a.E - 1);
  int t[25], t1[25];
  t[24] = a.line[ex0];
#pragma unroll
  for (int u = 0; u < 16; ++u) t[u] = colr[(int64_t)min(u, cmax) * a.E + ex0];
#pragma unroll
  for (int u = 0; u < 8; ++u) t[16 + u] = a.counts[min(u, rmax) * a.E + ex0];
#pragma unroll
  for (int u = 0; u < 25; ++u) t1[u] = 0;
  if (two) {
    t1[24] = a.line[ex1];
#pragma unroll
    for (int u = 0; u < 16; ++u) t1[u] = colr[(int64_t)min(u, cmax) * a.E + ex1];
#pragma unroll
    for (int u = 0; u < 8; ++u) t1[16 + u] = a.counts[min(u, rmax) * a.E + ex1];
  }
  int sh[kShiftU];
#pragma unroll
  for (int u = 0; u < kShiftU; ++u) {
    const int i = tid + u * kPlanChunk;
    sh[u] = tab && i < RE ? a.shift[i] : 0;
  }
  int ef[kEfixU];
#pragma unroll
  for (int u = 0; u < kEfixU; ++u) {
    const int i = tid + u * kPlanChunk;
    ef[u] = i < 2 * a.E ? a.efix[i] : 0;
  }
  const int pc0 = tab && tid < npc ? a.pieces[tid] : 0;
  const int np0 = tid < a.R ? a.npieces[tid] : 0;
  const int err = a.stats[MOONEP_STAT_ERROR];
  if (!err) {
    for (int i = tid; i < 4 * a.E; i += kPlanChunk) mask[i / a.E][i % a.E] = 0ull;
    {
      // the line start, the first 16 earlier chunks and 8 lower ranks of both experts
      int v0 = t[24], v1 = t1[24];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        v0 += u < ch ? t[u] : 0;
        v1 += u < ch ? t1[u] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v0 += u < r ? t[16 + u] : 0;
        v1 += u < r ? t1[16 + u] : 0;
      }
      // further rounds (both experts' loads together) past 16 chunks or 8 ranks
      for (int c0 = 16; c0 < ch; c0 += 16) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int c = min(c0 + u, cmax);
          t[u] = colr[(int64_t)c * a.E + ex0];
          t1[u] = two ? colr[(int64_t)c * a.E + ex1] : 0;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          v0 += c0 + u < ch ? t[u] : 0;
          v1 += c0 + u < ch ? t1[u] : 0;
        }
      }
      for (int q0 = 8; q0 < r; q0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int q = min(q0 + u, rmax);
          t[u] = a.counts[q * a.E + ex0];
          t1[u] = two ? a.counts[q * a.E + ex1] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          v0 += q0 + u < r ? t[u] : 0;
          v1 += q0 + u < r ? t1[u] : 0;
        }
      }
      if (tid < a.E) s_base[tid] = v0;
      if (two && tid + kPlanChunk < a.E) s_base[tid + kPlanChunk] = v1;
    }
#pragma unroll
    for (int u = 0; u < kShiftU; ++u) {
      const int i = tid + u * kPlanChunk;
      if (tab && i < RE) s_shift[i] = sh[u];
    }
#pragma unroll
    for (int u = 0; u < kEfixU; ++u) {
      const int i = tid + u * kPlanChunk;
      if (i < 2 * a.E) s_efix[i] = ef[u];
    }
    if (tab && tid < npc) s_pieces[tid] = pc0;
    if (tid < a.R) s_np[tid] = np0;
    // further rounds for larger shapes (each a batch of independent loads)
    for (int i = tid + 2 * kPlanChunk; i < a.E; i += kPlanChunk) {
      const int32_t* ci = a.cc + (int64_t)r * a.nch * a.E + i;
      int v = a.line[i];
      for (int c0 = 0; c0 < ch; c0 += 16) {
#pragma unroll
        for (int u = 0; u < 16; ++u) t[u] = c0 + u < ch ? ci[(int64_t)(c0 + u) * a.E] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) v += t[u];
      }
      for (int q0 = 0; q0 < r; q0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = q0 + u < r ? a.counts[(q0 + u) * a.E + i] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) v += t[u];
      }
      s_base[i] = v;
    }
    if (tab) {
      for (int i = tid + kShiftU * kPlanChunk; i < RE; i += kPlanChunk) s_shift[i] = a.shift[i];
      for (int i = tid + kPlanChunk; i < npc; i += kPlanChunk) s_pieces[i] = a.pieces[i];
    }
    for (int i = tid + kEfixU * kPlanChunk; i < 2 * a.E; i += kPlanChunk) s_efix[i] = a.efix[i];
    for (int i = tid + kPlanChunk; i < a.R; i += kPlanChunk) s_np[i] = a.npieces[i];
    __syncthreads();
    if (s < a.S)
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (k < a.K) atomicOr(&mask[w][ids[k]], bit);
    // the padding range of this thread's row (in flight during the assignment)
    if (pad_n > 0) {
      s_plo[tid] = pad_end - round_up(pad_n, a.tp) + pad_n;
      s_phi[tid] = pad_end;
    } else {
      s_plo[tid] = 0;
      s_phi[tid] = 0;
    }
    __syncthreads();
    if (s < a.S) {
      // unrolled over k with the ids in registers, so the LDS lookups of a
      // token's K slots overlap instead of running one chain after another;
      // the token's K destinations leave as 16-byte stores when K % 4 == 0
      // (and dest is 16-byte aligned)
      int dk[kMaxK];
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        if (k >= a.K) break;
        const int e = ids[k];
        // the token's rank among the chunk's tokens of expert e: earlier lanes of
        // its wave and all lanes of the waves before (the four masks read together)
        const unsigned long long m0 = mask[0][e], m1 = mask[1][e], m2 = mask[2][e],
                                 m3 = mask[3][e];
        const unsigned long long mw = w == 0 ? m0 : w == 1 ? m1 : w == 2 ? m2 : m3;
        const int below = __popcll(mw & (bit - 1)) + (w > 0 ? __popcll(m0) : 0) +
                          (w > 1 ? __popcll(m1) : 0) + (w > 2 ? __popcll(m2) : 0);
        const int pos = s_base[e] + below;
        int d = s_efix[2 * e];
        int slot;
        if (d >= 0) {
          slot = s_efix[2 * e + 1] + pos;          // the expert's tokens all go to rank d
        } else {
          // the expert is split over ranks: the piece of its group's line holding pos
          const int g = e / a.L;
          const int32_t* pg = (tab ? (const int32_t*)s_pieces : a.pieces) + (int64_t)g * (a.R + 1) * 2;
          const int np = s_np[g];
          // the first piece whose end lies past pos: count the pieces ending at or
          // before it (ends ascend), eight independent reads at a time (indices
          // clamped to the group's pieces, the surplus masked)
          int cnt = 0;
          const int plast = np > 0 ? np - 1 : 0;
          for (int p0 = 0; p0 < np; p0 += 8) {
            int hv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) hv[u] = pg[2 * min(p0 + u, plast)];
#pragma unroll
            for (int u = 0; u < 8; ++u) cnt += p0 + u < np && pos >= hv[u] ? 1 : 0;
          }
          d = cnt < np ? pg[2 * cnt + 1] : pg[1];
          slot = (unsigned)d < (unsigned)a.R
                     ? (tab ? s_shift[d * a.E + e] : a.shift[d * a.E + e]) + pos : -1;
        }
        const int32_t id = (int32_t)(tok * a.K + k);
        if ((unsigned)slot < (unsigned)a.NvS) {
          dk[k] = d * a.NvS + slot;
          a.src[(int64_t)d * a.NvS + slot] = id;
        } else {
          dk[k] = r * a.NvS + s * a.K + k;          // cannot happen for a valid plan
        }
      }
      int32_t* drow = a.dest + tok * a.K;
      if ((a.K & 3) == 0 && ((uintptr_t)a.dest & 15) == 0) {
        typedef int i32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int k = 0; k < kMaxK; k += 4)
          if (k < a.K) *(i32x4*)(drow + k) = i32x4{dk[k], dk[k + 1], dk[k + 2], dk[k + 3]};
      } else {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
          if (k < a.K) drow[k] = dk[k];
      }
    }
    // padding slots of this rank's active rows handled by this chunk (rows ch, ch + nch,
    // ...; thread t found the range of row ch + t nch): the whole workgroup clears one
    // row's range after the other
    const int npad = L2 > ch ? min((L2 - ch + a.nch - 1) / a.nch, kPlanChunk) : 0;
    for (int t = 0; t < npad; ++t) {
      const int lo = s_plo[t], hi = s_phi[t];
      for (int i = lo + tid; i < hi; i += kPlanChunk) a.src[(int64_t)r * a.NvS + i] = -1;
    }
    // rows past the first 256 of the chunk (more than 256 nch active rows), a thread each
    for (int q0 = kPlanChunk; ch + q0 * a.nch < L2; q0 += kPlanChunk) {
      const int q = ch + (q0 + tid) * a.nch;
      const int n = q < L2 ? a.an[r * L2 + q] : 0;
      if (n > 0) {
        const int end = a.aend[r * L2 + q];
        for (int i = end - round_up(n, a.tp) + n; i < end; ++i) a.src[(int64_t)r * a.NvS + i] = -1;
      }
    }
    // this chunk's share of the tail past the last segment
    const int span = (a.NvS - last + a.nch - 1) / a.nch;
    const int t0 = last + ch * span;
    const int t1 = min(a.NvS, t0 + span);
    for (int i = t0 + tid; i < t1; i += kPlanChunk) a.src[(int64_t)r * a.NvS + i] = -1;
  } else {
    if (s < a.S)
      for (int k = 0; k < a.K; ++k) {
        const int32_t id = (int32_t)(tok * a.K + k);
        a.dest[id] = r * a.NvS + s * a.K + k;
      }
    const int span = (a.NvS + a.nch - 1) / a.nch;
    const int t0 = ch * span;
    const int t1 = min(a.NvS, t0 + span);
    for (int i = t0 + tid; i < t1; i += kPlanChunk) a.src[(int64_t)r * a.NvS + i] = -1;
  }
}

}  // namespace

hipError_t launch_plan(const Ctx& c, const int32_t* topk, const int32_t* tpe,
                       const moonep_plan_t& p, hipStream_t s) {
  const Dims& d = c.d;
  PlanArgs a;
  a.R = d.R; a.S = d.S; a.K = d.K; a.E = d.E; a.B = d.B; a.L = d.L; a.tp = d.tp;
  a.nch = d.nch; a.NvS = (int)d.NvS; a.max_tiles = d.max_tiles;
  a.topk = topk; a.tpe = tpe;
  a.cc = c.cc; a.chunk_err = c.chunk_err; a.shift = c.shift;
  a.pieces = c.pieces; a.npieces = c.npieces; a.line = c.line; a.efix = c.efix;
  a.aend = c.aend; a.an = c.an; a.rend = c.rend;
  a.counts = p.counts; a.dest = p.dest; a.src = p.src; a.cu = p.cu_seqlens;
  a.segn = p.seg_tokens; a.pf = p.prefetch_src; a.stats = p.stats; a.aux = p.aux;
  a.ax = d.aux;
  const dim3 grid(d.nch, d.R);
  plan_hist<<<grid, kPlanChunk, 0, s>>>(a);
  plan_solve<<<1, kSolveThreads, 0, s>>>(a);
  plan_assign<<<dim3(d.nch + 2, d.R), kPlanChunk, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moonep
