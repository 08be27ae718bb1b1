/*
 * moonep.h -- C ABI of the MoonEP hot path on AMD MI355X (gfx950).
 *
 * The operations are those of the MoonEP README (MoonshotAI/MoonEP mirror),
 * section "API guide": a planner that makes every EP rank receive exactly
 * S*K token slots, dispatch (fused permute), prefetch_weight, the grouped
 * expert FFN over one [E+B,H,H'] weight tensor per projection addressed by
 * cu_seqlens ("Usage > Integration > Weight buffer"), combine (fused
 * unpermute) and reduce_grad ("Gradient buffer").
 *
 * One call serves all R EP ranks at once.  The ranks are R disjoint regions
 * of the memory of one GPU: rank d's dispatched rows are rows
 * [d*NvS, (d+1)*NvS) of every [R,NvS,...] array, and a "remote" store is a
 * plain store into another rank's region.
 *
 * Conventions for every entry point:
 *  - every pointer is a DEVICE pointer, allocated and owned by the caller,
 *    unless the comment says host;
 *  - bf16 values are passed as their 16-bit patterns (uint16_t);
 *  - every array is dense row-major with the shape given in brackets;
 *  - all work is enqueued on `stream`; no call synchronises the host except
 *    moonep_read_stats;
 *  - host-side argument checks run before anything is enqueued; on any error
 *    nothing is enqueued and a nonzero moonep_status_t comes back;
 *  - a routing the pages do not allow (expert id outside [0,E) or one expert
 *    twice in a token) is found on the device: it sets a sticky flag in
 *    stats[MOONEP_STAT_ERROR] and the plan becomes a safe no-op plan (every
 *    token keeps a slot in its own rank's region, no segment, no prefetch),
 *    so that later calls stay in bounds; read it with moonep_read_stats;
 *  - one handle serves one stream at a time (it owns plan scratch).
 */
#ifndef MOONEP_H
#define MOONEP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOONEP_ABI_VERSION 1

typedef int32_t moonep_status_t;
enum {
  MOONEP_OK = 0,
  MOONEP_ERR_ARG = 1,     /* null / misaligned pointer, bad width or rank  */
  MOONEP_ERR_CONFIG = 2,  /* configuration outside the supported range     */
  MOONEP_ERR_MODE = 3,    /* training call with B != E/R                   */
  MOONEP_ERR_HIP = 4,     /* a HIP runtime call or kernel launch failed    */
  MOONEP_ERR_NOMEM = 5,   /* scratch allocation in moonep_create failed    */
  MOONEP_ERR_SCRATCH = 6  /* moonep_plan_noalloc: the configuration needs
                             more planning scratch than the library holds  */
};

/* Problem sizes, in the README's notation ("Usage > Integration"):
 * R EP ranks, S tokens per rank, top-K experts per token, E routed experts
 * (E/R homed on each rank), B prefetch slots per rank, hidden size H, expert
 * FFN size Hp (H'), token_padding the row-length granularity of cu_seqlens.
 * num_cus: 0 = use the whole GPU for the data-movement kernels, else an
 * upper bound on their workgroups in flight (the README's num_sms knob).
 * Supported: 1 <= R <= 64, E % R == 0, E <= 1024, R*E <= 16384, 1 <= K <= min(E, 32),
 * 1 <= S, R*S*K < 2^31, 0 <= B <= E/R, R*(E+B) <= 16384,
 * token_padding >= 1, H % 64 == 0, Hp % 64 == 0, H, Hp <= 65536, R*NvS*max(H,Hp) < 2^40,
 * H*Hp < 2^30 and S*K*max(H,Hp) < 2^30 (the GEMMs address one weight row and
 * one segment's operand rows with 31-bit buffer offsets). */
typedef struct {
  int32_t R, S, K, E, B, H, Hp, token_padding, num_cus;
} moonep_config_t;

typedef struct moonep_ctx* moonep_handle_t;

/* Layout of the stats array of a plan (int32). */
enum {
  MOONEP_STAT_ERROR = 0,       /* sticky error bits, see MOONEP_ROUTE_*      */
  MOONEP_STAT_DUPS = 1,        /* redundant experts: (rank, remote expert)   */
  MOONEP_STAT_MAX_LOAD = 2,    /* max_e T_e                                  */
  MOONEP_STAT_DONATIONS = 3,   /* donations made by the planner              */
  MOONEP_STAT_PAD_ROWS = 4,    /* padding slots inside segments, all ranks   */
  MOONEP_STAT_MAXVIO = 5,      /* maxvio as float32 bits                     */
  MOONEP_STAT_REMOTE_GROUP = 8,/* [R] home group a rank duplicates from, -1  */
  /* followed by [R] number of remote experts per rank                      */
  MOONEP_STAT_FIXED = 8        /* stats length = MOONEP_STAT_FIXED + 2*R     */
};
enum {
  MOONEP_ROUTE_ID_RANGE = 1,   /* an expert id outside [0, E)                */
  MOONEP_ROUTE_REPEAT = 2,     /* one expert twice in one token              */
  MOONEP_ROUTE_COUNTS = 4      /* tokens_per_expert disagrees with topk      */
};

/* The plan: caller-owned int32 device arrays, all written by moonep_plan and
 * read by the other calls (the README's MoonEPCommPlan plus cu_seqlens).
 * Sizes come from moonep_plan_len(). */
typedef struct {
  int32_t* counts;       /* [R,E]   tokens of rank r routed to expert e      */
  int32_t* dest;         /* [R,S,K] global slot d*NvS+i of token (r,s,k)     */
  int32_t* src;          /* [R,NvS] (r*S+s)*K+k held by a slot, -1 = none    */
  int32_t* cu_seqlens;   /* [R,E+B] inclusive padded end offset of each row  */
  int32_t* seg_tokens;   /* [R,E+B] real tokens in each row                  */
  int32_t* prefetch_src; /* [R,B]   home expert copied into prefetch slot j  */
  int32_t* stats;        /* [MOONEP_STAT_FIXED + 2R]                         */
  int32_t* aux;          /* derived tables used by the other calls           */
} moonep_plan_t;

enum {
  MOONEP_PLAN_COUNTS = 0, MOONEP_PLAN_DEST, MOONEP_PLAN_SRC,
  MOONEP_PLAN_CU_SEQLENS, MOONEP_PLAN_SEG_TOKENS, MOONEP_PLAN_PREFETCH_SRC,
  MOONEP_PLAN_STATS, MOONEP_PLAN_AUX, MOONEP_PLAN_NARRAYS
};

int32_t moonep_abi_version(void);
const char* moonep_status_string(moonep_status_t status);

/* Token slots per rank: S*K real slots plus the padding of at most 2*E/R
 * active rows (E/R home rows and the rows of at most one remote home group,
 * README "How to set B"), each padded by less than token_padding:
 * NvS = S*K + 2*(E/R)*token_padding.  Returns -1 for an invalid config. */
int64_t moonep_nvs(const moonep_config_t* cfg);

/* Number of int32 elements of plan array `which` (MOONEP_PLAN_*), -1 on an
 * invalid config or index. */
int64_t moonep_plan_len(const moonep_config_t* cfg, int32_t which);

/* Workgroups that a data-movement call launches for this configuration
 * (README "API guide", Buffer(..., num_sms, ...): the CU budget caps the
 * grids of the data-movement kernels; planning and GEMM grids are not
 * capped).  which: MOONEP_GRID_*.  W: row width in elements for dispatch,
 * combine and copy (a positive multiple of 8; ignored otherwise).
 * device_cus: the device's compute units (reduce_grad launches at most 8
 * workgroups per CU).  Host only: no GPU call is made.  With cfg->num_cus > 0
 * every result is at most num_cus * 8.  Returns -1 for an invalid config,
 * which, W or device_cus. */
enum {
  MOONEP_GRID_DISPATCH = 0, MOONEP_GRID_COMBINE, MOONEP_GRID_COPY,
  MOONEP_GRID_PREFETCH, MOONEP_GRID_REDUCE_GRAD
};
int64_t moonep_launch_grid(const moonep_config_t* cfg, int32_t which, int32_t W,
                           int32_t device_cus);

/* Validate cfg (host) and allocate the handle's scratch on the current
 * device (the README's Buffer(...)).  *out is untouched on error. */
moonep_status_t moonep_create(const moonep_config_t* cfg, moonep_handle_t* out);
/* Free the scratch (the README's buffer.destroy()).  NULL is a no-op. */
moonep_status_t moonep_destroy(moonep_handle_t h);

/* Plan (README "API guide > dispatch fwd", planning part).
 * topk [R,S,K] int32 expert ids, k in the router's order.
 * tokens_per_expert [R,E] int32 local counts, or NULL; when given it is
 * checked against topk (MOONEP_ROUTE_COUNTS on mismatch).
 * Writes every array of *plan.  Planning follows the spec P1-P9: group loads,
 * chain-greedy donations that give every rank exactly S*K slots with at most
 * one remote home group, expert lines sorted by (load, id), tokens of an
 * expert in (rank, token) order, rows E..E+B-1 for the first B remote
 * experts in ascending id and home rows for the rest, rows padded to
 * token_padding. */
moonep_status_t moonep_plan(moonep_handle_t h, const int32_t* topk,
                            const int32_t* tokens_per_expert,
                            const moonep_plan_t* plan, hipStream_t stream);

/* Planning without a handle and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels and
 * results as moonep_plan (every plan array bit-identical), with the
 * configuration passed directly; the planning scratch is a fixed array of
 * MOONEP_NOALLOC_SCRATCH_BYTES in the library's device memory, one per GPU,
 * which the GPU holds until the process ends.  The scratch needed, in int32
 * elements each rounded up to 64, is R*ceil(S/256)*E + R*E + 2*R*(R+1)
 * + R + E + R*ceil(S/256) + 3*(2*E) + R; MOONEP_ERR_SCRATCH (nothing enqueued) when it
 * exceeds the array (e.g. R=8, E=256 fits up to S of about 64000).  Calls
 * that overlap on one GPU (different streams or host threads) share the
 * array and race; calls on one stream are ordered.  The first call with a
 * device current looks the array's device address up (hipGetSymbolAddress);
 * no call allocates or frees memory. */
#define MOONEP_NOALLOC_SCRATCH_BYTES (2 * 1024 * 1024)
moonep_status_t moonep_plan_noalloc(const moonep_config_t* cfg, const int32_t* topk,
                                    const int32_t* tokens_per_expert,
                                    const moonep_plan_t* plan, hipStream_t stream);

/* Dispatch (README "API guide > dispatch fwd"; also "combine bwd", which is a
 * re-dispatch of the output gradient with the saved plan).
 * x [R,S,W] bf16 rows, W % 8 == 0 (W = H forward, W = H' or H for gradients).
 * rw [R,S,K] fp32 route weights or NULL.
 * Writes x_nvs [R,NvS,W]: slot dest[r,s,k] gets a bit copy of row x[r,s];
 * padding slots inside a segment get zeros; slots past a rank's last segment
 * are not written.  rw_nvs [R,NvS] (or NULL iff rw is NULL) gets rw[r,s,k]
 * at the same slots and 0 at padding slots. */
moonep_status_t moonep_dispatch(moonep_handle_t h, const moonep_plan_t* plan,
                                const uint16_t* x, int32_t W, const float* rw,
                                uint16_t* x_nvs, float* rw_nvs,
                                hipStream_t stream);

/* Combine (README "API guide > combine fwd"; also "dispatch bwd" when
 * rw_nvs is NULL).  y_nvs [R,NvS,W] bf16, W % 8 == 0.
 * out[r,s,:] = bf16_rne(acc) with acc = p_0 then acc = acc + p_k for
 * k = 1..K-1 in fp32 round-to-nearest, p_k = rw_nvs[slot_k] * y_nvs[slot_k]
 * (fp32 product, no fused multiply-add) or y_nvs[slot_k] if rw_nvs is NULL.
 * rw_sk [R,S,K] (or NULL) gets rw_nvs[slot_k] (requires rw_nvs). */
moonep_status_t moonep_combine(moonep_handle_t h, const moonep_plan_t* plan,
                               const uint16_t* y_nvs, int32_t W,
                               const float* rw_nvs, uint16_t* out,
                               float* rw_sk, hipStream_t stream);

/* Copy of the used slots (README "API guide > zero_copy"): with zero_copy
 * off, dispatch hands back a new tensor copied out of the communication
 * buffer, and combine first copies its input into that buffer.  This call is
 * that copy: for every rank d, rows [0, cu_seqlens[d][E+B-1]) of src_nvs
 * [R,NvS,W] bf16 (padding rows included) are copied to dst_nvs; the rows past
 * the last segment are not touched.  W % 8 == 0; src and dst must differ. */
moonep_status_t moonep_copy_rows(moonep_handle_t h, const moonep_plan_t* plan,
                                 const uint16_t* src_nvs, int32_t W,
                                 uint16_t* dst_nvs, hipStream_t stream);

/* Prefetch (README "API guide > dispatch fwd", prefetch_weight; "Weight
 * buffer").  home[p] [E,H,Hp] bf16 for p = gate, up, down; pool[p]
 * [R,B,H,Hp]: pool[p][d][j] becomes a bit copy of home[p][prefetch_src[d][j]]
 * for every used slot; unused slots are not written.  Row i of rank d's
 * [E+B,H,Hp] view is home[p]+i*H*Hp for i < E, else pool[p]+(d*B+i-E)*H*Hp.
 * Pointer arrays home/pool are HOST arrays of 3 device pointers. */
moonep_status_t moonep_prefetch_weight(moonep_handle_t h,
                                       const moonep_plan_t* plan,
                                       const uint16_t* const home[3],
                                       uint16_t* const pool[3],
                                       hipStream_t stream);

/* Grouped SwiGLU expert FFN (README "Usage > Integration"): for rank d
 * (rank = -1: all ranks) and every row i with cu_seqlens length > 0, over the
 * row's padded segment X of x_nvs [R,NvS,H]:
 *   G = X Wg_i, U = X Wu_i (bf16 MFMA, fp32 accumulation),
 *   Z = bf16_rne(silu(G) * U) -> z_ws [R,NvS,Hp],
 *   Y = bf16_rne(Z Wd_i^T)    -> y_nvs [R,NvS,H],
 * with every projection stored [H,Hp] and rows resolved as in
 * moonep_prefetch_weight.  y_nvs may equal x_nvs (in-place, the README's
 * zero_copy); no other aliasing.  Slots outside segments are not written.
 * The same as moonep_expert_gateup followed by moonep_expert_down. */
moonep_status_t moonep_expert_ffn(moonep_handle_t h, const moonep_plan_t* plan,
                                  int32_t rank, const uint16_t* x_nvs,
                                  const uint16_t* const home[3],
                                  const uint16_t* const pool[3],
                                  uint16_t* z_ws, uint16_t* y_nvs,
                                  hipStream_t stream);

/* First half of the grouped SwiGLU FFN (README "Usage > Integration"): the
 * gate and up projections and the SwiGLU product,
 * z_nvs = bf16_rne(silu(X Wg_i) * (X Wu_i)) per segment, as in
 * moonep_expert_ffn.  Reads home[0..1] and pool[0..1] only (home[2],
 * pool[2] may be NULL); z_nvs [R,NvS,Hp] must not alias x_nvs. */
moonep_status_t moonep_expert_gateup(moonep_handle_t h, const moonep_plan_t* plan,
                                     int32_t rank, const uint16_t* x_nvs,
                                     const uint16_t* const home[3],
                                     const uint16_t* const pool[3],
                                     uint16_t* z_nvs, hipStream_t stream);

/* Second half (README "Usage > Integration"): y_nvs = bf16_rne(Z Wd_i^T) per
 * segment, Z = z_nvs [R,NvS,Hp], y_nvs [R,NvS,H] (must not alias z_nvs).
 * Reads home[2] and pool[2] only (the other entries may be NULL). */
moonep_status_t moonep_expert_down(moonep_handle_t h, const moonep_plan_t* plan,
                                   int32_t rank, const uint16_t* z_nvs,
                                   const uint16_t* const home[3],
                                   const uint16_t* const pool[3],
                                   uint16_t* y_nvs, hipStream_t stream);

/* Backward of the grouped SwiGLU FFN (the framework-side step between the
 * README's "combine bwd" and "dispatch bwd"; derived from the forward of
 * "Usage > Integration" by the chain rule).  For rank d (-1: all ranks) and
 * every row i with cu_seqlens length > 0, over the row's padded segment:
 *   dZ = bf16_rne(dY Wd_i)                        -> dz_ws  [R,NvS,Hp]
 *   G = X Wg_i, U = X Wu_i recomputed (fp32), s = sigma(G),
 *   dU = bf16_rne(dZ * G s)                       -> du_nvs [R,NvS,Hp]
 *   dG = bf16_rne(dZ * U * s (1 + G (1 - s)))     -> dg_nvs [R,NvS,Hp]
 *   dX = bf16_rne(dG Wg_i^T + dU Wu_i^T)          -> dx_nvs [R,NvS,H]
 * x_nvs [R,NvS,H] is the forward input and dy_nvs [R,NvS,H] the gradient of
 * the loss w.r.t. the FFN output rows y_nvs (a route-weighted loss scales it
 * by rw_nvs first).  Weights resolve as in moonep_prefetch_weight.  dG and
 * dU feed moonep_expert_wgrad (dWg = X^T dG, dWu = X^T dU); dWd = dY^T Z uses
 * the forward's Z.  dx_nvs may equal x_nvs or dy_nvs; dz_ws, dg_nvs and
 * du_nvs alias nothing.  Slots outside segments are not written. */
moonep_status_t moonep_expert_ffn_bwd(moonep_handle_t h, const moonep_plan_t* plan,
                                      int32_t rank, const uint16_t* x_nvs,
                                      const uint16_t* dy_nvs,
                                      const uint16_t* const home[3],
                                      const uint16_t* const pool[3],
                                      uint16_t* dz_ws, uint16_t* dg_nvs,
                                      uint16_t* du_nvs, uint16_t* dx_nvs,
                                      hipStream_t stream);

/* Weight gradient of one projection (README "Gradient buffer"): for rank d
 * (-1: all) and every row i with length > 0, dW_i += A_seg^T B_seg in fp32,
 * A = a_nvs [R,NvS,H] bf16, B = b_nvs [R,NvS,Hp] bf16 (gate/up: A = x,
 * B = dG or dU; down: A = dY, B = Z).  Row i < E is grad_home [E,H,Hp] fp32
 * row i; row i >= E is reduce_buf [R,B,H,Hp] fp32 slot (d, i-E).  Training
 * only: MOONEP_ERR_MODE unless B == E/R. */
moonep_status_t moonep_expert_wgrad(moonep_handle_t h,
                                    const moonep_plan_t* plan, int32_t rank,
                                    const uint16_t* a_nvs,
                                    const uint16_t* b_nvs, float* grad_home,
                                    float* reduce_buf, hipStream_t stream);

/* reduce_grad (README "Gradient buffer", "API guide > dispatch bwd"): for
 * every home expert e and every used slot (d,j) with prefetch_src[d][j] == e,
 * in ascending d: grad_home[p][e] += reduce_buf[p][d][j] (fp32
 * round-to-nearest, no fused operations), then reduce_buf[p][d][j] = 0, for
 * p = gate, up, down.  HOST arrays of 3 device pointers.  Training only:
 * MOONEP_ERR_MODE unless B == E/R. */
moonep_status_t moonep_reduce_grad(moonep_handle_t h,
                                   const moonep_plan_t* plan,
                                   float* const grad_home[3],
                                   float* const reduce_buf[3],
                                   hipStream_t stream);

/* ---- Symmetric [E+B,H,Hp] buffers on virtual memory ----
 *
 * The README's contract ("Usage > Integration > Weight buffer", "Gradient
 * buffer") is one contiguous virtual range [E+B,H,Hp] per projection and
 * rank.  Its rows [0,E) are every rank's home experts, each chunk physically
 * the home rank's memory mapped everywhere; its rows [E,E+B) are the rank's
 * prefetch slots (for fp32 gradients: its reduce buffer), from a separate
 * allocation.  A symbuf builds exactly that for the R ranks of one GPU with
 * hipMemCreate / hipMemAddressReserve / hipMemMap on the current device:
 *   physical: per rank d, one chunk of E/R rows (home) and one of B rows
 *             (slots), so E + R*B rows in all;
 *   views [R,E+B,H,Hp]: rank d's [E+B] view starts at row d*(E+B); its rows
 *             [0,E) map the R home chunks in rank order, its rows [E,E+B) its
 *             own slot chunk;
 *   home  [E,H,Hp]: the home chunks in rank order;
 *   slots [R,B,H,Hp]: the slot chunks in rank order (for gradients: the
 *             README's [R,B,H,Hp] view of every rank's reduce buffer).
 * The ranges alias: a write through one is seen through every other range
 * that maps the same chunk (in stream order).  `home` and `slots` are what
 * the entry points above take as home[p]/pool[p] and grad_home/reduce_buf;
 * `views` is what the *_views entry points below take.  Rows start
 * uninitialised. */
typedef struct moonep_symbuf* moonep_symbuf_t;

typedef struct {
  void* views;             /* device address, [R,E+B,H,Hp]                   */
  void* home;              /* device address, [E,H,Hp]                       */
  void* slots;             /* device address, [R,B,H,Hp]; NULL when B == 0   */
  int64_t row_bytes;       /* H*Hp*elem_bytes                                */
  int64_t physical_bytes;  /* HBM it allocated: (E + R*B) * row_bytes, or
                              E * row_bytes when it maps another's slots     */
  int64_t granularity;     /* the device's minimum VMM granularity, bytes    */
} moonep_symbuf_info_t;

/* Minimum VMM allocation granularity of the current device, bytes (host
 * out). */
moonep_status_t moonep_vmm_granularity(int64_t* out);

/* Create the symbuf of one projection for the handle's configuration, on
 * the current device.  elem_bytes: 2 for bf16 weights, 4 for fp32
 * gradients.  slots_from: NULL, or a symbuf of the same R, B, row size and
 * device whose slot chunks this one maps instead of allocating its own (the
 * README's prefetch pool, one process-wide allocation that every layer's
 * [E+B] range shares; MOONEP_ERR_ARG if it does not match).  Shared chunks
 * stay allocated until every symbuf that maps them is destroyed.
 * (E/R)*H*Hp*elem_bytes and B*H*Hp*elem_bytes must be multiples of the
 * granularity (MOONEP_ERR_CONFIG otherwise).  MOONEP_ERR_NOMEM when the
 * physical memory is not there, MOONEP_ERR_HIP when another VMM call fails;
 * on any error nothing stays allocated.  The symbuf does not depend on the
 * handle after this call. */
moonep_status_t moonep_symbuf_create(moonep_handle_t h, int32_t elem_bytes,
                                     moonep_symbuf_t slots_from, moonep_symbuf_t* out);

/* Addresses and sizes of a symbuf (host out). */
moonep_status_t moonep_symbuf_info(moonep_symbuf_t b, moonep_symbuf_info_t* out);

/* Synchronise the symbuf's device, then unmap and free everything it holds.
 * NULL is a no-op. */
moonep_status_t moonep_symbuf_destroy(moonep_symbuf_t b);

/* prefetch_weight over per-rank views, the README's own signature (rows
 * [0,E) of each full_*_weight are the sources, rows [E,E+B) the slots):
 * views[p] [R,E+B,H,Hp] bf16 (a symbuf's `views`, or any tensor of that
 * layout), and for every used slot (d,j): row E+j of rank d's view becomes
 * a bit copy of row prefetch_src[d][j] of the same view.  HOST array of 3
 * device pointers. */
moonep_status_t moonep_prefetch_weight_views(moonep_handle_t h,
                                             const moonep_plan_t* plan,
                                             uint16_t* const views[3],
                                             hipStream_t stream);

/* moonep_expert_ffn with every expert located purely by row index in rank
 * d's [E+B] view (README "Usage > Integration": the grouped GEMM consumes one
 * [E+B,H,H'] tensor per projection selected by cu_seqlens): row i of rank d
 * is views[p] + (d*(E+B) + i)*H*Hp.  Otherwise identical to
 * moonep_expert_ffn, including aliasing rules and results. */
moonep_status_t moonep_expert_ffn_views(moonep_handle_t h, const moonep_plan_t* plan,
                                        int32_t rank, const uint16_t* x_nvs,
                                        const uint16_t* const views[3],
                                        uint16_t* z_ws, uint16_t* y_nvs,
                                        hipStream_t stream);

/* moonep_expert_ffn_bwd with weights located as in moonep_expert_ffn_views. */
moonep_status_t moonep_expert_ffn_bwd_views(moonep_handle_t h,
                                            const moonep_plan_t* plan, int32_t rank,
                                            const uint16_t* x_nvs,
                                            const uint16_t* dy_nvs,
                                            const uint16_t* const views[3],
                                            uint16_t* dz_ws, uint16_t* dg_nvs,
                                            uint16_t* du_nvs, uint16_t* dx_nvs,
                                            hipStream_t stream);

/* Synchronise `stream` and copy the plan's stats array to host_stats
 * (MOONEP_STAT_FIXED + 2R int32, HOST memory).  For tests and reports. */
moonep_status_t moonep_read_stats(moonep_handle_t h, const moonep_plan_t* plan,
                                  int32_t* host_stats, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOONEP_H */
