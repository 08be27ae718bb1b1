// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moonep.h"

namespace moonep {

// Tokens handled by one workgroup of the planning kernels (4 waves of 64).
constexpr int kPlanChunk = 256;
constexpr int kMaxR = 64;
constexpr int kMaxRE = 16384;
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;

// Offsets (int32 elements) of the derived tables inside plan.aux.
struct AuxLayout {
  int64_t act;      // [R][2L] active rows of each rank, ascending, -1 padded
  int64_t pf_n;     // [1] used prefetch slots
  int64_t pf;       // [R*B] used slots d*B+j in ascending (d, j)
  int64_t dup_n;    // [1] home experts that have prefetch copies
  int64_t dup_e;    // [R*B] such experts, ascending
  int64_t dup_first;// [R*B] first holder of each
  int64_t dup_cnt;  // [R*B] holder count of each
  int64_t hold;     // [R*B] holder slots d*B+j grouped by expert, ascending d
  int64_t tiles;    // [R][max_tiles][4] grouped-GEMM M-tiles (row, first slot, end slot, 0)
  int64_t ntiles;   // [R] M-tiles of each rank
  int64_t nfull;    // [R] of which full-duration (they come first)
  int64_t nact;     // [R] active rows of each rank (the first entries of act)
  int64_t total;
};

struct Dims {
  int R, S, K, E, B, H, Hp, tp, num_cus;
  int L;          // E / R
  int64_t NvS;    // slots per rank
  int nch;        // planning chunks per rank
  int max_tiles;  // grouped-GEMM M-tiles per rank, upper bound
  AuxLayout aux;
};

struct Ctx {
  Dims d;
  int device;
  int num_cu_device;
  // planning scratch (device)
  int32_t* cc;        // [R][nch][E] expert counts of each planning chunk
  int32_t* shift;     // [R][E] slot - line position for (d, e)
  int32_t* pieces;    // [R groups][R+1][2] (hi, rank) of each line piece
  int32_t* npieces;   // [R]
  int32_t* line;      // [E] line start a_e
  int32_t* chunk_err; // [R][nch] routing error bits found per chunk
  int32_t* efix;      // [E][2] (rank, slot - line position) of an expert whose tokens all
                      // go to one rank, rank -1 for an expert split over ranks
  int32_t* aend;      // [R][2E/R] padded end slot of each rank's active row q
  int32_t* an;        // [R][2E/R] real tokens of each rank's active row q
  int32_t* rend;      // [R] end of each rank's last segment (its used slots)
};

bool dims_from_config(const moonep_config_t* cfg, Dims* out);

// Where the weight row `row` of rank d lives (projection p, H*Hp elements per
// row): rows [0,E) at home[p] + (d*home_stride + row) rows, rows [E,E+B) at
// pool[p] + (d*pool_stride + row-E) rows.  Separate tensors home [E] and
// pool [R*B] have strides 0 and B; per-rank [E+B] views laid out back to back
// ([R][E+B]) have home = the views, pool = the views + E rows, both strides
// E+B.
struct WeightRef {
  const uint16_t* home[3];
  uint16_t* pool[3];
  int64_t home_stride, pool_stride;
};

// Kernel launchers (each returns hipGetLastError() after its launches).
hipError_t launch_plan(const Ctx& c, const int32_t* topk, const int32_t* tpe,
                       const moonep_plan_t& p, hipStream_t s);
// Workgroups of each data-movement launch (move.hip); dispatch also needs the
// split of its grid into token and padding workgroups.
struct DispatchGrid {
  int xcd_local;      // 1: one item per wave, a token's waves on one XCD; 0: a capped grid
  int item_blocks;    // token workgroups (the padding workgroups follow them)
  int npad_used;      // padding items: (rank, active row, part)
  int pad_parts;      // parts each active row's padding is split into
  int64_t blocks;     // the whole grid
};
DispatchGrid dispatch_grid(const Ctx& c, int W);
int64_t combine_grid(const Ctx& c, int W);
int64_t copy_grid(const Ctx& c);
int64_t prefetch_grid(const Ctx& c);
int64_t reduce_grad_grid(const Ctx& c);

hipError_t launch_dispatch(const Ctx& c, const moonep_plan_t& p,
                           const uint16_t* x, int W, const float* rw,
                           uint16_t* x_nvs, float* rw_nvs, hipStream_t s);
hipError_t launch_combine(const Ctx& c, const moonep_plan_t& p,
                          const uint16_t* y, int W, const float* rw_nvs,
                          uint16_t* out, float* rw_sk, hipStream_t s);
hipError_t launch_copy_rows(const Ctx& c, const moonep_plan_t& p,
                            const uint16_t* src, int W, uint16_t* dst,
                            hipStream_t s);
hipError_t launch_prefetch(const Ctx& c, const moonep_plan_t& p, const WeightRef& w,
                           hipStream_t s);
hipError_t launch_reduce_grad(const Ctx& c, const moonep_plan_t& p,
                              float* const gh[3], float* const rb[3],
                              hipStream_t s);
hipError_t launch_gateup(const Ctx& c, const moonep_plan_t& p, int rank,
                         const uint16_t* x_nvs, const WeightRef& w, uint16_t* z,
                         hipStream_t s);
hipError_t launch_down(const Ctx& c, const moonep_plan_t& p, int rank,
                       const uint16_t* z, const WeightRef& w, uint16_t* y, hipStream_t s);
hipError_t launch_ffn_bwd(const Ctx& c, const moonep_plan_t& p, int rank,
                          const uint16_t* x, const uint16_t* dy, const WeightRef& w,
                          uint16_t* dz, uint16_t* dg, uint16_t* du, uint16_t* dx,
                          hipStream_t s);
hipError_t launch_wgrad(const Ctx& c, const moonep_plan_t& p, int rank,
                        const uint16_t* a, const uint16_t* b, float* gh,
                        float* rb, hipStream_t s);

// M-tile of the grouped GEMMs (rows of one segment handled by a workgroup).
constexpr int kGemmTileM = 256;

}  // namespace moonep

// The object behind a moonep_handle_t.
struct moonep_ctx {
  moonep::Ctx c;
};
