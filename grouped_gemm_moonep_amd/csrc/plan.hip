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
//                serial chain-greedy (at most 2R steps), rows, cu_seqlens,
//                prefetch and reduce tables, per-chunk line bases;
//   plan_assign (R x chunks workgroups): stable rank of each token among the
//                earlier tokens of the same expert (popcount of the lane
//                masks below it), its line position, piece, row and slot;
//                padding slots get src = -1.  One more workgroup per rank
//                builds that rank's grouped-GEMM tile schedule
//                (tile_schedule.h) at the same time.
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
  int32_t* rankpre;
  int32_t* shift;
  int32_t* pieces;
  int32_t* npieces;
  int32_t* line;
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
// Block-wide exclusive scan of v over all kSolveThreads threads.
__device__ int block_exclusive_scan(int v, int* total, int* scratch /*[32]*/) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wv] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < kSolveThreads / 64; ++i) {
      const int t = scratch[i];
      scratch[i] = run;
      run += t;
    }
    scratch[16] = run;
  }
  __syncthreads();
  const int res = x - v + scratch[wv];
  *total = scratch[16];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------------------
// plan_solve: the single-workgroup part.
__global__ __launch_bounds__(kSolveThreads) void plan_solve(PlanArgs a) {
  __shared__ int T[kMaxE];
  __shared__ int aline[kMaxE];
  __shared__ int W[kMaxR], keep[kMaxR], X[kMaxR], D[kMaxR], need[kMaxR];
  __shared__ int donors[kMaxR], queue[2 * kMaxR + 2];
  __shared__ int don_g[kMaxR + 1], don_r[kMaxR + 1], don_amt[kMaxR + 1], don_lo[kMaxR + 1];
  __shared__ int recv_g[kMaxR], recv_lo[kMaxR], recv_hi[kMaxR];
  __shared__ int ent_n[2 * kMaxE], ent_lo[2 * kMaxE], ent_row[2 * kMaxE];
  __shared__ int act_row[2 * kMaxE], act_end[2 * kMaxE], act_n[2 * kMaxE];
  __shared__ int nact[kMaxR], nrem[kMaxR], npf[kMaxR];
  __shared__ int hcount[kMaxE];
  __shared__ int ord_len[3 * kMaxE], ord_ent[3 * kMaxE], ord_cnt[3 * kMaxE];  // phase F
  __shared__ int scan_scratch[32];
  __shared__ int s_err, s_maxload, s_ndon, s_dups, s_pad;

  const int tid = threadIdx.x;
  const int R = a.R, E = a.E, L = a.L, B = a.B, nch = a.nch;
  const int C = a.S * a.K;
  const int RE = R * E;
  if (tid == 0) {
    s_err = 0; s_maxload = 0; s_ndon = 0; s_dups = 0; s_pad = 0;
  }
  __syncthreads();

  // Phase A: counts per (r, e) and exclusive per-chunk prefix (in place).
  // Loads are batched 16 at a time so each thread keeps 16 in flight.
  for (int idx = tid; idx < RE; idx += kSolveThreads) {
    const int r = idx / E, e = idx - (idx / E) * E;
    int32_t* col = a.cc + (int64_t)r * nch * E + e;
    int run = 0;
    for (int ch0 = 0; ch0 < nch; ch0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = ch0 + u < nch ? col[(int64_t)(ch0 + u) * E] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (ch0 + u < nch) {
          col[(int64_t)(ch0 + u) * E] = run;
          run += v[u];
        }
    }
    a.counts[idx] = run;
    if (a.tpe && a.tpe[idx] != run) atomicOr(&s_err, MOONEP_ROUTE_COUNTS);
  }
  for (int i = tid; i < R * nch; i += kSolveThreads) {
    const int v = a.chunk_err[i];
    if (v) atomicOr(&s_err, v);
  }
  __syncthreads();

  // Phase B: expert loads T_e and the exclusive prefix over ranks.
  for (int e = tid; e < E; e += kSolveThreads) {
    int run = 0;
    for (int r0 = 0; r0 < R; r0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = r0 + u < R ? a.counts[(r0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (r0 + u < R) {
          a.rankpre[(r0 + u) * E + e] = run;
          run += v[u];
        }
    }
    T[e] = run;
    atomicMax(&s_maxload, run);
  }
  __syncthreads();
  const int err = s_err;

  if (err) {
    // Safe no-op plan: no segment, no prefetch, every token keeps a slot in
    // its own rank's region (written by plan_assign).
    for (int i = tid; i < R * (E + B); i += kSolveThreads) { a.cu[i] = 0; a.segn[i] = 0; }
    for (int i = tid; i < R * B; i += kSolveThreads) a.pf[i] = -1;
    for (int i = tid; i < 2 * E; i += kSolveThreads) a.aux[a.ax.act + i] = -1;
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

  // Phase C: line start of every expert (experts of a group by (T, id)),
  // group loads.
  for (int e = tid; e < E; e += kSolveThreads) {
    const int g = e / L;
    const int te = T[e];
    int acc = 0;
    for (int f = g * L; f < (g + 1) * L; ++f) {
      const int tf = T[f];
      if (tf < te || (tf == te && f < e)) acc += tf;
    }
    aline[e] = acc;
    a.line[e] = acc;
  }
  for (int g = tid; g < R; g += kSolveThreads) {
    int w = 0;
    for (int f = g * L; f < (g + 1) * L; ++f) w += T[f];
    W[g] = w;
  }
  __syncthreads();

  // Phase D: keep/excess/deficit per group, donors ordered by (-X, g) and
  // receivers by (-D, r) (each group finds its own position), then the
  // chain-greedy itself (one thread, at most 2R steps), then the line pieces
  // of every group (one thread per group).
  for (int g = tid; g < R; g += kSolveThreads) {
    keep[g] = W[g] < C ? W[g] : C;
    X[g] = W[g] - keep[g];
    D[g] = C - keep[g];
    need[g] = D[g];
    recv_g[g] = -1;
    recv_lo[g] = 0;
    recv_hi[g] = 0;
  }
  __syncthreads();
  for (int g = tid; g < R; g += kSolveThreads) {
    int pos = 0;
    if (X[g] > 0) {
      for (int h = 0; h < R; ++h)
        if (X[h] > 0 && (X[h] > X[g] || (X[h] == X[g] && h < g))) ++pos;
      donors[pos] = g;
    }
    if (D[g] > 0) {
      pos = 0;
      for (int h = 0; h < R; ++h)
        if (D[h] > 0 && (D[h] > D[g] || (D[h] == D[g] && h < g))) ++pos;
      queue[pos] = g;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int nd = 0, qt = 0;
    for (int g = 0; g < R; ++g) {
      nd += X[g] > 0;
      qt += D[g] > 0;
    }
    int qh = 0;
    int ndon = 0;
    int i = 0;
    int x = nd ? X[donors[0]] : 0;
    int bad = 0;
    while (qh < qt && !bad) {
      const int r = queue[qh++];
      const int dn = need[r];
      if (i >= nd || ndon >= R) { bad = 1; break; }
      const int g = donors[i];
      don_g[ndon] = g; don_r[ndon] = r; don_amt[ndon] = dn; ++ndon;
      if (dn <= x) {
        x -= dn;
        if (x == 0 && i + 1 < nd) { ++i; x = X[donors[i]]; }
      } else {
        const int sh = dn - x;
        keep[g] -= sh;
        need[g] = sh;
        if (qt >= 2 * kMaxR + 2) { bad = 1; break; }
        queue[qt++] = g;
        ++i;
        x = i < nd ? X[donors[i]] : 0;
      }
    }
    s_ndon = ndon;
    if (bad) s_err = 8;   // internal: inconsistent counts (cannot happen)
  }
  __syncthreads();
  // pieces of every group's line: [0, keep) to the home rank, then the
  // group's donations in emission order
  const int ndon_all = s_ndon;
  for (int g = tid; g < R; g += kSolveThreads) {
    int np = 0, lo = 0;
    int32_t* pg = a.pieces + (int64_t)g * (R + 1) * 2;
    if (keep[g] > 0) {
      lo = keep[g];
      pg[0] = lo; pg[1] = g; np = 1;
    }
    for (int q = 0; q < ndon_all; ++q) {
      if (don_g[q] != g) continue;
      const int dlo = lo;
      lo += don_amt[q];
      pg[2 * np] = lo; pg[2 * np + 1] = don_r[q]; ++np;
      recv_g[don_r[q]] = g;        // each rank receives from at most one group
      recv_lo[don_r[q]] = dlo;
      recv_hi[don_r[q]] = lo;
    }
    a.npieces[g] = np;
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
  for (int idx = tid; idx < R * L2; idx += kSolveThreads) {
    const int d = idx / L2, i = idx - (idx / L2) * L2;
    int row = -1;
    if (ent_n[idx] > 0) {
      if (i < L) {
        row = d * L + i;
      } else {
        int j = 0;
        for (int q = L; q < i; ++q) j += ent_n[d * L2 + q] > 0;
        row = j < B ? E + j : recv_g[d] * L + (i - L);
      }
    }
    ent_row[idx] = row;
  }
  __syncthreads();

  // Phase F: lay each rank's active rows out in ascending row order: the
  // lower group's rows first (the rank's home experts or the remote experts
  // that keep home rows), prefetch rows last.  Every active entry gets a
  // visit-order slot (3L per rank); one block-wide scan over all slots gives
  // each row's start and its index among the rank's active rows.
  const int S3 = 3 * L;
  const int nslot = R * S3;
  for (int i = tid; i < nslot; i += kSolveThreads) {
    ord_len[i] = 0;
    ord_ent[i] = -1;
  }
  for (int d = tid; d < R; d += kSolveThreads) { nrem[d] = 0; npf[d] = 0; }
  __syncthreads();
  for (int idx = tid; idx < R * L2; idx += kSolveThreads) {
    const int n = ent_n[idx];
    if (n == 0) continue;
    const int d = idx / L2, i = idx - (idx / L2) * L2;
    const int g = recv_g[d];
    const bool home_first = g < 0 || d < g;
    int o;
    if (i < L) o = (home_first ? 0 : L) + i;
    else if (ent_row[idx] >= E) o = 2 * L + (i - L);
    else o = (home_first ? L : 0) + (i - L);
    ord_len[d * S3 + o] = round_up(n, a.tp);
    ord_ent[d * S3 + o] = idx;
  }
  __syncthreads();
  int tot_cnt;
  {
    const int per = (nslot + kSolveThreads - 1) / kSolveThreads;
    const int b0 = min(nslot, tid * per), b1 = min(nslot, b0 + per);
    int sl = 0, sc = 0;
    for (int i = b0; i < b1; ++i) { sl += ord_len[i]; sc += ord_ent[i] >= 0; }
    int tot_len;
    int pl = block_exclusive_scan(sl, &tot_len, scan_scratch);
    int pc = block_exclusive_scan(sc, &tot_cnt, scan_scratch);
    for (int i = b0; i < b1; ++i) {          // exclusive prefixes, in place
      const int l = ord_len[i];
      ord_len[i] = pl;
      ord_cnt[i] = pc;
      pl += l;
      pc += ord_ent[i] >= 0;
    }
  }
  __syncthreads();
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
    act_row[d * L2 + q] = row;
    act_end[d * L2 + q] = start + len;
    act_n[d * L2 + q] = n;
    if (!home) atomicAdd(&nrem[d], 1);
    if (row >= E) {
      a.pf[d * B + (row - E)] = e;
      atomicAdd(&npf[d], 1);
    }
    if (len > n) atomicAdd(&s_pad, len - n);
  }
  __syncthreads();
  for (int d = tid; d < R; d += kSolveThreads) {
    const int next = d + 1 < R ? ord_cnt[(d + 1) * S3] : tot_cnt;
    nact[d] = next - ord_cnt[d * S3];
    a.aux[a.ax.nact + d] = nact[d];
    const int rem = nrem[d];
    a.stats[MOONEP_STAT_REMOTE_GROUP + d] = rem ? recv_g[d] : -1;
    a.stats[MOONEP_STAT_REMOTE_GROUP + R + d] = rem;
    atomicAdd(&s_dups, rem);
  }
  __syncthreads();
  for (int i = tid; i < R * B; i += kSolveThreads) {
    const int d = i / B, j = i - (i / B) * B;
    if (j >= npf[d]) a.pf[i] = -1;
  }
  for (int i = tid; i < R * L2; i += kSolveThreads) {
    const int d = i / L2, q = i - (i / L2) * L2;
    a.aux[a.ax.act + i] = q < nact[d] ? act_row[i] : -1;
  }

  // Phase G: cu_seqlens and seg_tokens for every (rank, row).
  const int EB = E + B;
  // The rank's active rows are in ascending row order: binary search for
  // the last one at or below `row`.
  for (int idx = tid; idx < R * EB; idx += kSolveThreads) {
    const int d = idx / EB, row = idx - (idx / EB) * EB;
    const int* ar = act_row + d * L2;
    int lo = 0, hi = nact[d];          // first q with ar[q] > row lies in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ar[mid] <= row) lo = mid + 1;
      else hi = mid;
    }
    int end = 0, n = 0;
    if (lo > 0) {
      end = act_end[d * L2 + lo - 1];
      if (ar[lo - 1] == row) n = act_n[d * L2 + lo - 1];
    }
    a.cu[idx] = end;
    a.segn[idx] = n;
  }

  // Phase G2: used prefetch slots in (d, j) order.
  if (tid == 0) {
    int k = 0;
    for (int d = 0; d < R; ++d)
      for (int j = 0; j < npf[d]; ++j) a.aux[a.ax.pf + k++] = d * B + j;
    a.aux[a.ax.pf_n] = k;
  }

  // Phase G3: holders of every home expert that has prefetch copies, in
  // ascending rank (the reduce_grad order).
  for (int e = tid; e < E; e += kSolveThreads) {
    const int g = e / L, i = e - g * L;
    int cnt = 0;
    for (int d = 0; d < R; ++d)
      if (recv_g[d] == g && ent_row[d * L2 + L + i] >= E) ++cnt;
    hcount[e] = cnt;
  }
  __syncthreads();
  {
    const int e = tid;
    const int has = (e < E && hcount[e] > 0) ? 1 : 0;
    const int cnt = e < E ? hcount[e] : 0;
    int nexp, nhold;
    const int q = block_exclusive_scan(has, &nexp, scan_scratch);
    const int first = block_exclusive_scan(cnt, &nhold, scan_scratch);
    if (has) {
      const int g = e / L, i = e - g * L;
      a.aux[a.ax.dup_e + q] = e;
      a.aux[a.ax.dup_first + q] = first;
      a.aux[a.ax.dup_cnt + q] = cnt;
      int k = 0;
      for (int d = 0; d < R; ++d) {
        const int row = ent_row[d * L2 + L + i];
        if (recv_g[d] == g && row >= E) a.aux[a.ax.hold + first + k++] = d * B + (row - E);
      }
    }
    if (tid == 0) a.aux[a.ax.dup_n] = nexp;
  }

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
  if (blockIdx.x == a.nch) {
    // the grid's extra column: rank blockIdx.y's grouped-GEMM tile schedule,
    // built from plan_solve's segments alongside the token assignment
    __shared__ int wsum[4];
    build_tile_schedule(a.aux + a.ax.act, a.cu, a.segn, a.aux + a.ax.tiles,
                        a.aux + a.ax.ntiles, a.aux + a.ax.nfull, blockIdx.y, 2 * a.L,
                        a.E + a.B, a.tp, a.max_tiles,
                        wsum);
    return;
  }
  __shared__ unsigned long long mask[4][kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ int s_shift[kShiftLds];
  __shared__ int s_pieces[kPiecesLds];
  __shared__ int s_np[kMaxR];
  const int ch = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int err = a.stats[MOONEP_STAT_ERROR];
  const int s = ch * kPlanChunk + tid;
  const int w = tid >> 6, lane = tid & 63;
  const unsigned long long bit = 1ull << lane;
  const int64_t tok = (int64_t)r * a.S + s;
  // the lookup tables of this chunk, staged in LDS when they fit
  const int npc = a.R * (a.R + 1) * 2;
  const bool tab = a.R * a.E <= kShiftLds && npc <= kPiecesLds;
  if (!err) {
    for (int i = tid; i < 4 * a.E; i += kPlanChunk) mask[i / a.E][i % a.E] = 0ull;
    // line position of this chunk's first token of expert e: the expert's
    // line start + tokens of lower ranks + tokens of earlier chunks of rank r
    const int32_t* gbase = a.cc + ((int64_t)r * a.nch + ch) * a.E;
    for (int i = tid; i < a.E; i += kPlanChunk)
      s_base[i] = gbase[i] + a.line[i] + a.rankpre[r * a.E + i];
    for (int i = tid; i < a.R; i += kPlanChunk) s_np[i] = a.npieces[i];
    if (tab) {
      for (int i = tid; i < a.R * a.E; i += kPlanChunk) s_shift[i] = a.shift[i];
      for (int i = tid; i < npc; i += kPlanChunk) s_pieces[i] = a.pieces[i];
    }
    __syncthreads();
    if (s < a.S)
      for (int k = 0; k < a.K; ++k) atomicOr(&mask[w][a.topk[tok * a.K + k]], bit);
    __syncthreads();
    if (s < a.S) {
      for (int k = 0; k < a.K; ++k) {
        const int e = a.topk[tok * a.K + k];
        int below = __popcll(mask[w][e] & (bit - 1));
        for (int v = 0; v < w; ++v) below += __popcll(mask[v][e]);
        const int pos = s_base[e] + below;
        const int g = e / a.L;
        const int32_t* pg = (tab ? (const int32_t*)s_pieces : a.pieces) + (int64_t)g * (a.R + 1) * 2;
        const int np = s_np[g];
        int d = pg[1];
        for (int p = 0; p < np; ++p) {
          if (pos < pg[2 * p]) { d = pg[2 * p + 1]; break; }
        }
        const int32_t id = (int32_t)(tok * a.K + k);
        if ((unsigned)d >= (unsigned)a.R) {       // cannot happen for a valid plan
          a.dest[id] = r * a.NvS + s * a.K + k;
          continue;
        }
        const int slot = (tab ? s_shift[d * a.E + e] : a.shift[d * a.E + e]) + pos;
        if ((unsigned)slot >= (unsigned)a.NvS) {  // cannot happen for a valid plan
          a.dest[id] = r * a.NvS + s * a.K + k;
          continue;
        }
        a.dest[id] = d * a.NvS + slot;
        a.src[(int64_t)d * a.NvS + slot] = id;
      }
    }
    // padding slots of this rank's active rows handled by this chunk
    const int L2 = 2 * a.L, EB = a.E + a.B;
    for (int q = ch; q < L2; q += a.nch) {
      const int row = a.aux[a.ax.act + r * L2 + q];
      if (row < 0) break;
      const int end = a.cu[r * EB + row];
      const int n = a.segn[r * EB + row];
      const int len = round_up(n, a.tp);
      for (int i = end - len + n + tid; i < end; i += kPlanChunk)
        a.src[(int64_t)r * a.NvS + i] = -1;
    }
    // this chunk's share of the tail past the last segment
    const int last = a.cu[r * EB + EB - 1];
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
  a.cc = c.cc; a.chunk_err = c.chunk_err; a.rankpre = c.rankpre; a.shift = c.shift;
  a.pieces = c.pieces; a.npieces = c.npieces; a.line = c.line;
  a.counts = p.counts; a.dest = p.dest; a.src = p.src; a.cu = p.cu_seqlens;
  a.segn = p.seg_tokens; a.pf = p.prefetch_src; a.stats = p.stats; a.aux = p.aux;
  a.ax = d.aux;
  const dim3 grid(d.nch, d.R);
  plan_hist<<<grid, kPlanChunk, 0, s>>>(a);
  plan_solve<<<1, kSolveThreads, 0, s>>>(a);
  plan_assign<<<dim3(d.nch + 1, d.R), kPlanChunk, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moonep
