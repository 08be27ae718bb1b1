// Host side of the C ABI: configuration checks, handle scratch, argument
// validation, and the launches.  Nothing here runs on the CPU instead of the
// GPU: every step of the path is a kernel.
#include <stdlib.h>
#include <string.h>

#include "internal.h"

namespace moonep {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dims_from_config(const moonep_config_t* cfg, Dims* out) {
  if (!cfg) return false;
  const moonep_config_t& c = *cfg;
  if (c.R < 1 || c.R > kMaxR) return false;
  if (c.E < c.R || c.E % c.R || c.E > 1024) return false;
  if ((int64_t)c.R * c.E > kMaxRE) return false;
  if (c.K < 1 || c.K > c.E || c.K > kMaxK) return false;
  if (c.S < 1) return false;
  if ((int64_t)c.R * c.S * c.K >= (int64_t(1) << 31)) return false;
  const int L = c.E / c.R;
  if (c.B < 0 || c.B > L) return false;
  if ((int64_t)c.R * (c.E + c.B) > kMaxRE) return false;
  if (c.token_padding < 1) return false;
  if (c.H < 64 || c.H % 64 || c.Hp < 64 || c.Hp % 64) return false;
  if (c.H > 65536 || c.Hp > 65536) return false;   // a tile's lane offsets stay below 2^26
  if (c.num_cus < 0) return false;
  const int64_t nvs = (int64_t)c.S * c.K + 2LL * L * c.token_padding;
  if ((int64_t)c.R * nvs >= (int64_t(1) << 31)) return false;
  const int64_t wmax = c.H > c.Hp ? c.H : c.Hp;
  if ((int64_t)c.R * nvs * wmax >= (int64_t(1) << 40)) return false;
  // The GEMM kernels address a weight row (H x H' bf16) and a segment's
  // operand rows (at most S*K rows of H or H' bf16) through one buffer
  // descriptor each, whose offsets are 31 bits.
  if ((int64_t)c.H * c.Hp * 2 >= (int64_t(1) << 31)) return false;
  if ((int64_t)c.S * c.K * wmax * 2 >= (int64_t(1) << 31)) return false;
  Dims d;
  d.R = c.R; d.S = c.S; d.K = c.K; d.E = c.E; d.B = c.B; d.H = c.H;
  d.Hp = c.Hp; d.tp = c.token_padding; d.num_cus = c.num_cus;
  d.L = L;
  d.NvS = nvs;
  d.nch = (int)ceil_div(c.S, kPlanChunk);
  const int64_t RB = (int64_t)c.R * c.B;
  AuxLayout& a = d.aux;
  a.act = 0;
  a.pf_n = a.act + 2LL * c.E;
  a.pf = a.pf_n + 1;
  a.dup_n = a.pf + RB;
  a.dup_e = a.dup_n + 1;
  a.dup_first = a.dup_e + RB;
  a.dup_cnt = a.dup_first + RB;
  a.hold = a.dup_cnt + RB;
  d.max_tiles = (int)(ceil_div(d.NvS, kGemmTileM) + 2 * d.L);
  a.tiles = a.hold + RB;
  a.ntiles = a.tiles + 4LL * c.R * d.max_tiles;
  a.nfull = a.ntiles + c.R;
  a.nact = a.nfull + c.R;
  a.total = a.nact + c.R;
  *out = d;
  return true;
}

}  // namespace moonep

using namespace moonep;

static bool aligned(const void* p, size_t a) {
  return ((uintptr_t)p % a) == 0;
}

static moonep_status_t hip_status(hipError_t e) {
  return e == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

// Separate tensors: home [E] shared by every rank, pool [R*B].
static WeightRef split_ref(const Dims& d, const uint16_t* const home[3],
                           const uint16_t* const pool[3]) {
  WeightRef w;
  for (int p = 0; p < 3; ++p) {
    w.home[p] = home[p];
    w.pool[p] = const_cast<uint16_t*>(pool[p]);
  }
  w.home_stride = 0;
  w.pool_stride = d.B;
  return w;
}

// Per-rank [E+B] views, back to back: rank d's row i at views + (d*(E+B)+i) rows.
static WeightRef views_ref(const Dims& d, const uint16_t* const views[3]) {
  WeightRef w;
  const int64_t rs = (int64_t)d.H * d.Hp;
  for (int p = 0; p < 3; ++p) {
    w.home[p] = views[p];
    w.pool[p] = (views[p] && d.B > 0) ? const_cast<uint16_t*>(views[p]) + d.E * rs : nullptr;
  }
  w.home_stride = d.E + d.B;
  w.pool_stride = d.E + d.B;
  return w;
}

static bool plan_ok(const moonep_plan_t* p) {
  if (!p) return false;
  const int32_t* a[] = {p->counts, p->dest, p->src, p->cu_seqlens,
                        p->seg_tokens, p->prefetch_src, p->stats, p->aux};
  for (const int32_t* q : a)
    if (!q || !aligned(q, 4)) return false;
  return true;
}

static hipError_t run_ffn(const Ctx& c, const moonep_plan_t& p, int rank, const uint16_t* x,
                          const WeightRef& w, uint16_t* z, uint16_t* y, hipStream_t s) {
  hipError_t e = launch_gateup(c, p, rank, x, w, z, s);
  if (e == hipSuccess) e = launch_down(c, p, rank, z, w, y, s);
  return e;
}

// Buffers of the FFN backward: all present and 16-byte aligned; dZ, dG and dU
// distinct from each other and from every other buffer; dX may reuse the
// storage of dY or X (both are consumed before dX is written).
static bool bwd_buffers_ok(const Ctx& c, int rank, const void* x, const void* dy,
                           const void* dz, const void* dg, const void* du, const void* dx) {
  if (rank < -1 || rank >= c.d.R) return false;
  const void* all[] = {x, dy, dz, dg, du, dx};
  for (const void* q : all)
    if (!q || !aligned(q, 16)) return false;
  const void* ws[] = {dz, dg, du};
  const void* other[] = {x, dy, dx, dz, dg, du};
  for (int i = 0; i < 3; ++i)
    for (int k = 0; k < 6; ++k)
      if (ws[i] == other[k] && k != 3 + i) return false;
  return true;
}

extern "C" {

int32_t moonep_abi_version(void) { return MOONEP_ABI_VERSION; }

const char* moonep_status_string(moonep_status_t s) {
  switch (s) {
    case MOONEP_OK: return "ok";
    case MOONEP_ERR_ARG: return "invalid argument (null/misaligned pointer, width or rank)";
    case MOONEP_ERR_CONFIG: return "configuration outside the supported range";
    case MOONEP_ERR_MODE: return "training call needs B == E/R";
    case MOONEP_ERR_HIP: return "HIP runtime error";
    case MOONEP_ERR_NOMEM: return "device allocation failed";
    case MOONEP_ERR_SCRATCH:
      return "configuration needs more planning scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int64_t moonep_nvs(const moonep_config_t* cfg) {
  Dims d;
  return dims_from_config(cfg, &d) ? d.NvS : -1;
}

int64_t moonep_plan_len(const moonep_config_t* cfg, int32_t which) {
  Dims d;
  if (!dims_from_config(cfg, &d)) return -1;
  switch (which) {
    case MOONEP_PLAN_COUNTS: return (int64_t)d.R * d.E;
    case MOONEP_PLAN_DEST: return (int64_t)d.R * d.S * d.K;
    case MOONEP_PLAN_SRC: return (int64_t)d.R * d.NvS;
    case MOONEP_PLAN_CU_SEQLENS: return (int64_t)d.R * (d.E + d.B);
    case MOONEP_PLAN_SEG_TOKENS: return (int64_t)d.R * (d.E + d.B);
    case MOONEP_PLAN_PREFETCH_SRC: return (int64_t)d.R * d.B;
    case MOONEP_PLAN_STATS: return MOONEP_STAT_FIXED + 2LL * d.R;
    case MOONEP_PLAN_AUX: return d.aux.total;
    default: return -1;
  }
}

int64_t moonep_launch_grid(const moonep_config_t* cfg, int32_t which, int32_t W,
                           int32_t device_cus) {
  Ctx c;
  if (!dims_from_config(cfg, &c.d) || device_cus < 1) return -1;
  c.num_cu_device = device_cus;
  const bool rows = which == MOONEP_GRID_DISPATCH || which == MOONEP_GRID_COMBINE ||
                    which == MOONEP_GRID_COPY;
  if (rows && (W <= 0 || W % 8)) return -1;
  switch (which) {
    case MOONEP_GRID_DISPATCH: return dispatch_grid(c, W).blocks;
    case MOONEP_GRID_COMBINE: return combine_grid(c, W);
    case MOONEP_GRID_COPY: return copy_grid(c);
    case MOONEP_GRID_PREFETCH: return prefetch_grid(c);
    case MOONEP_GRID_REDUCE_GRAD: return reduce_grad_grid(c);
    default: return -1;
  }
}

moonep_status_t moonep_create(const moonep_config_t* cfg, moonep_handle_t* out) {
  if (!out) return MOONEP_ERR_ARG;
  Dims d;
  if (!dims_from_config(cfg, &d)) return MOONEP_ERR_CONFIG;
  moonep_ctx* h = (moonep_ctx*)calloc(1, sizeof(moonep_ctx));
  if (!h) return MOONEP_ERR_NOMEM;
  Ctx& c = h->c;
  c.d = d;
  if (hipGetDevice(&c.device) != hipSuccess ||
      hipDeviceGetAttribute(&c.num_cu_device, hipDeviceAttributeMultiprocessorCount,
                            c.device) != hipSuccess) {
    free(h);
    return MOONEP_ERR_HIP;
  }
  struct { int32_t** p; int64_t n; } allocs[] = {
      {&c.cc, (int64_t)d.R * d.nch * d.E},
      {&c.shift, (int64_t)d.R * d.E},
      {&c.pieces, (int64_t)d.R * (d.R + 1) * 2},
      {&c.npieces, d.R},
      {&c.line, d.E},
      {&c.chunk_err, (int64_t)d.R * d.nch},
      {&c.efix, 2LL * d.E},
      {&c.aend, 2LL * d.E},
      {&c.an, 2LL * d.E},
      {&c.rend, d.R},
  };
  for (auto& a : allocs) {
    if (hipMalloc((void**)a.p, (size_t)a.n * sizeof(int32_t)) != hipSuccess) {
      moonep_destroy(h);
      return MOONEP_ERR_NOMEM;
    }
  }
  *out = h;
  return MOONEP_OK;
}

moonep_status_t moonep_destroy(moonep_handle_t h) {
  if (!h) return MOONEP_OK;
  Ctx& c = h->c;
  int32_t* ptrs[] = {c.cc, c.shift, c.pieces, c.npieces, c.line,
                     c.chunk_err, c.efix, c.aend, c.an, c.rend};
  hipError_t err = hipSuccess;
  for (int32_t* p : ptrs)
    if (p) {
      hipError_t e = hipFree(p);
      if (e != hipSuccess) err = e;
    }
  free(h);
  return hip_status(err);
}

moonep_status_t moonep_plan(moonep_handle_t h, const int32_t* topk,
                            const int32_t* tokens_per_expert,
                            const moonep_plan_t* plan, hipStream_t stream) {
  if (!h || !topk || !aligned(topk, 4) || !plan_ok(plan)) return MOONEP_ERR_ARG;
  if (tokens_per_expert && !aligned(tokens_per_expert, 4)) return MOONEP_ERR_ARG;
  return hip_status(launch_plan(h->c, topk, tokens_per_expert, *plan, stream));
}

moonep_status_t moonep_dispatch(moonep_handle_t h, const moonep_plan_t* plan,
                                const uint16_t* x, int32_t W, const float* rw,
                                uint16_t* x_nvs, float* rw_nvs,
                                hipStream_t stream) {
  if (!h || !plan_ok(plan) || !x || !x_nvs) return MOONEP_ERR_ARG;
  if (W <= 0 || W % 8 || !aligned(x, 16) || !aligned(x_nvs, 16)) return MOONEP_ERR_ARG;
  if ((rw == nullptr) != (rw_nvs == nullptr)) return MOONEP_ERR_ARG;
  if (rw && (!aligned(rw, 4) || !aligned(rw_nvs, 4))) return MOONEP_ERR_ARG;
  return hip_status(launch_dispatch(h->c, *plan, x, W, rw, x_nvs, rw_nvs, stream));
}

moonep_status_t moonep_combine(moonep_handle_t h, const moonep_plan_t* plan,
                               const uint16_t* y_nvs, int32_t W,
                               const float* rw_nvs, uint16_t* out,
                               float* rw_sk, hipStream_t stream) {
  if (!h || !plan_ok(plan) || !y_nvs || !out) return MOONEP_ERR_ARG;
  if (W <= 0 || W % 8 || !aligned(y_nvs, 16) || !aligned(out, 16)) return MOONEP_ERR_ARG;
  if (rw_sk && !rw_nvs) return MOONEP_ERR_ARG;
  if ((rw_nvs && !aligned(rw_nvs, 4)) || (rw_sk && !aligned(rw_sk, 4))) return MOONEP_ERR_ARG;
  return hip_status(launch_combine(h->c, *plan, y_nvs, W, rw_nvs, out, rw_sk, stream));
}

moonep_status_t moonep_copy_rows(moonep_handle_t h, const moonep_plan_t* plan,
                                 const uint16_t* src_nvs, int32_t W, uint16_t* dst_nvs,
                                 hipStream_t stream) {
  if (!h || !plan_ok(plan) || !src_nvs || !dst_nvs) return MOONEP_ERR_ARG;
  if (W <= 0 || W % 8 || !aligned(src_nvs, 16) || !aligned(dst_nvs, 16)) return MOONEP_ERR_ARG;
  if ((const void*)src_nvs == (const void*)dst_nvs) return MOONEP_ERR_ARG;
  return hip_status(launch_copy_rows(h->c, *plan, src_nvs, W, dst_nvs, stream));
}

moonep_status_t moonep_prefetch_weight(moonep_handle_t h, const moonep_plan_t* plan,
                                       const uint16_t* const home[3],
                                       uint16_t* const pool[3], hipStream_t stream) {
  if (!h || !plan_ok(plan) || !home || !pool) return MOONEP_ERR_ARG;
  for (int p = 0; p < 3; ++p) {
    if (!home[p] || !aligned(home[p], 16)) return MOONEP_ERR_ARG;
    if (h->c.d.B > 0 && (!pool[p] || !aligned(pool[p], 16))) return MOONEP_ERR_ARG;
  }
  if (h->c.d.B == 0) return MOONEP_OK;
  return hip_status(launch_prefetch(h->c, *plan, split_ref(h->c.d, home, pool), stream));
}

static bool weights_ok(const Ctx& c, const uint16_t* const home[3],
                       const uint16_t* const pool[3], int p0, int p1) {
  if (!home || !pool) return false;
  for (int p = p0; p < p1; ++p) {
    if (!home[p] || !aligned(home[p], 16)) return false;
    if (c.d.B > 0 && (!pool[p] || !aligned(pool[p], 16))) return false;
  }
  return true;
}

static bool views_ok(const uint16_t* const views[3], int p0, int p1) {
  if (!views) return false;
  for (int p = p0; p < p1; ++p)
    if (!views[p] || !aligned(views[p], 16)) return false;
  return true;
}

moonep_status_t moonep_expert_gateup(moonep_handle_t h, const moonep_plan_t* plan,
                                     int32_t rank, const uint16_t* x_nvs,
                                     const uint16_t* const home[3],
                                     const uint16_t* const pool[3], uint16_t* z_nvs,
                                     hipStream_t stream) {
  if (!h || !plan_ok(plan) || !x_nvs || !z_nvs) return MOONEP_ERR_ARG;
  if (rank < -1 || rank >= h->c.d.R) return MOONEP_ERR_ARG;
  if (!aligned(x_nvs, 16) || !aligned(z_nvs, 16) || (void*)z_nvs == (void*)x_nvs)
    return MOONEP_ERR_ARG;
  if (!weights_ok(h->c, home, pool, 0, 2)) return MOONEP_ERR_ARG;
  return hip_status(launch_gateup(h->c, *plan, rank, x_nvs, split_ref(h->c.d, home, pool), z_nvs,
                                  stream));
}

moonep_status_t moonep_expert_down(moonep_handle_t h, const moonep_plan_t* plan,
                                   int32_t rank, const uint16_t* z_nvs,
                                   const uint16_t* const home[3],
                                   const uint16_t* const pool[3], uint16_t* y_nvs,
                                   hipStream_t stream) {
  if (!h || !plan_ok(plan) || !z_nvs || !y_nvs) return MOONEP_ERR_ARG;
  if (rank < -1 || rank >= h->c.d.R) return MOONEP_ERR_ARG;
  if (!aligned(z_nvs, 16) || !aligned(y_nvs, 16) || (void*)z_nvs == (void*)y_nvs)
    return MOONEP_ERR_ARG;
  if (!weights_ok(h->c, home, pool, 2, 3)) return MOONEP_ERR_ARG;
  return hip_status(launch_down(h->c, *plan, rank, z_nvs, split_ref(h->c.d, home, pool), y_nvs,
                                stream));
}

moonep_status_t moonep_expert_ffn(moonep_handle_t h, const moonep_plan_t* plan,
                                  int32_t rank, const uint16_t* x_nvs,
                                  const uint16_t* const home[3],
                                  const uint16_t* const pool[3], uint16_t* z_ws,
                                  uint16_t* y_nvs, hipStream_t stream) {
  if (!h || !plan_ok(plan) || !x_nvs || !z_ws || !y_nvs) return MOONEP_ERR_ARG;
  if (rank < -1 || rank >= h->c.d.R) return MOONEP_ERR_ARG;
  if (!aligned(x_nvs, 16) || !aligned(z_ws, 16) || !aligned(y_nvs, 16)) return MOONEP_ERR_ARG;
  if ((void*)z_ws == (void*)x_nvs || (void*)z_ws == (void*)y_nvs) return MOONEP_ERR_ARG;
  if (!weights_ok(h->c, home, pool, 0, 3)) return MOONEP_ERR_ARG;
  return hip_status(run_ffn(h->c, *plan, rank, x_nvs, split_ref(h->c.d, home, pool), z_ws, y_nvs,
                            stream));
}

moonep_status_t moonep_expert_ffn_views(moonep_handle_t h, const moonep_plan_t* plan,
                                        int32_t rank, const uint16_t* x_nvs,
                                        const uint16_t* const views[3], uint16_t* z_ws,
                                        uint16_t* y_nvs, hipStream_t stream) {
  if (!h || !plan_ok(plan) || !x_nvs || !z_ws || !y_nvs) return MOONEP_ERR_ARG;
  if (rank < -1 || rank >= h->c.d.R) return MOONEP_ERR_ARG;
  if (!aligned(x_nvs, 16) || !aligned(z_ws, 16) || !aligned(y_nvs, 16)) return MOONEP_ERR_ARG;
  if ((void*)z_ws == (void*)x_nvs || (void*)z_ws == (void*)y_nvs) return MOONEP_ERR_ARG;
  if (!views_ok(views, 0, 3)) return MOONEP_ERR_ARG;
  return hip_status(run_ffn(h->c, *plan, rank, x_nvs, views_ref(h->c.d, views), z_ws, y_nvs,
                            stream));
}

moonep_status_t moonep_prefetch_weight_views(moonep_handle_t h, const moonep_plan_t* plan,
                                             uint16_t* const views[3], hipStream_t stream) {
  if (!h || !plan_ok(plan) || !views) return MOONEP_ERR_ARG;
  const uint16_t* cv[3] = {views[0], views[1], views[2]};
  if (!views_ok(cv, 0, 3)) return MOONEP_ERR_ARG;
  if (h->c.d.B == 0) return MOONEP_OK;
  return hip_status(launch_prefetch(h->c, *plan, views_ref(h->c.d, cv), stream));
}

moonep_status_t moonep_expert_ffn_bwd(moonep_handle_t h, const moonep_plan_t* plan,
                                      int32_t rank, const uint16_t* x_nvs,
                                      const uint16_t* dy_nvs, const uint16_t* const home[3],
                                      const uint16_t* const pool[3], uint16_t* dz_ws,
                                      uint16_t* dg_nvs, uint16_t* du_nvs, uint16_t* dx_nvs,
                                      hipStream_t stream) {
  if (!h || !plan_ok(plan)) return MOONEP_ERR_ARG;
  if (!bwd_buffers_ok(h->c, rank, x_nvs, dy_nvs, dz_ws, dg_nvs, du_nvs, dx_nvs))
    return MOONEP_ERR_ARG;
  if (!weights_ok(h->c, home, pool, 0, 3)) return MOONEP_ERR_ARG;
  return hip_status(launch_ffn_bwd(h->c, *plan, rank, x_nvs, dy_nvs, split_ref(h->c.d, home, pool),
                                   dz_ws, dg_nvs, du_nvs, dx_nvs, stream));
}

moonep_status_t moonep_expert_ffn_bwd_views(moonep_handle_t h, const moonep_plan_t* plan,
                                            int32_t rank, const uint16_t* x_nvs,
                                            const uint16_t* dy_nvs,
                                            const uint16_t* const views[3], uint16_t* dz_ws,
                                            uint16_t* dg_nvs, uint16_t* du_nvs,
                                            uint16_t* dx_nvs, hipStream_t stream) {
  if (!h || !plan_ok(plan)) return MOONEP_ERR_ARG;
  if (!bwd_buffers_ok(h->c, rank, x_nvs, dy_nvs, dz_ws, dg_nvs, du_nvs, dx_nvs))
    return MOONEP_ERR_ARG;
  if (!views_ok(views, 0, 3)) return MOONEP_ERR_ARG;
  return hip_status(launch_ffn_bwd(h->c, *plan, rank, x_nvs, dy_nvs, views_ref(h->c.d, views),
                                   dz_ws, dg_nvs, du_nvs, dx_nvs, stream));
}

moonep_status_t moonep_expert_wgrad(moonep_handle_t h, const moonep_plan_t* plan,
                                    int32_t rank, const uint16_t* a_nvs,
                                    const uint16_t* b_nvs, float* grad_home,
                                    float* reduce_buf, hipStream_t stream) {
  if (!h || !plan_ok(plan) || !a_nvs || !b_nvs || !grad_home) return MOONEP_ERR_ARG;
  if (rank < -1 || rank >= h->c.d.R) return MOONEP_ERR_ARG;
  if (h->c.d.B != h->c.d.L) return MOONEP_ERR_MODE;
  if (!reduce_buf) return MOONEP_ERR_ARG;
  if (!aligned(a_nvs, 16) || !aligned(b_nvs, 16) || !aligned(grad_home, 16) ||
      !aligned(reduce_buf, 16))
    return MOONEP_ERR_ARG;
  return hip_status(launch_wgrad(h->c, *plan, rank, a_nvs, b_nvs, grad_home, reduce_buf, stream));
}

moonep_status_t moonep_reduce_grad(moonep_handle_t h, const moonep_plan_t* plan,
                                   float* const grad_home[3], float* const reduce_buf[3],
                                   hipStream_t stream) {
  if (!h || !plan_ok(plan) || !grad_home || !reduce_buf) return MOONEP_ERR_ARG;
  if (h->c.d.B != h->c.d.L) return MOONEP_ERR_MODE;
  for (int p = 0; p < 3; ++p)
    if (!grad_home[p] || !reduce_buf[p] || !aligned(grad_home[p], 16) ||
        !aligned(reduce_buf[p], 16))
      return MOONEP_ERR_ARG;
  return hip_status(launch_reduce_grad(h->c, *plan, grad_home, reduce_buf, stream));
}

moonep_status_t moonep_read_stats(moonep_handle_t h, const moonep_plan_t* plan,
                                  int32_t* host_stats, hipStream_t stream) {
  if (!h || !plan_ok(plan) || !host_stats) return MOONEP_ERR_ARG;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return MOONEP_ERR_HIP;
  e = hipMemcpy(host_stats, plan->stats,
                sizeof(int32_t) * (MOONEP_STAT_FIXED + 2 * h->c.d.R), hipMemcpyDeviceToHost);
  return hip_status(e);
}

}  // extern "C"
