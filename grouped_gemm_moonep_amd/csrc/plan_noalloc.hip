// moonep_plan without a handle and without allocating: the planning scratch
// (per-chunk expert counts, slot shifts, line pieces, line starts, per-chunk
// error bits, per-expert destinations, the padded end and token count of each
// rank's active rows, each rank's used slots) lives in one file-scope device array instead
// of the handle's device allocations, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  The kernels are the planner's own (launch_plan); only
// where their scratch comes from differs.
//
// The array is one per GPU (each device that loads the library holds its own
// copy until the process ends).  Host code never passes the array's name to
// a kernel: its device address on the current device is looked up once with
// hipGetSymbolAddress, on the first call made with that device current, and
// kept per device.  Every call on a GPU shares that GPU's array, so calls
// that overlap on one GPU (two streams, or two host threads) race; calls in
// one stream are ordered.  Nothing in the scratch has to start at zero: every
// element a kernel reads was written earlier in the same call.
#include <mutex>

#include "internal.h"

namespace moonep {
namespace {

constexpr int64_t kScratchInts = MOONEP_NOALLOC_SCRATCH_BYTES / 4;
static __device__ __align__(256) int32_t scratch[kScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int32_t* g_scratch[kMaxDevices];     // device address of `scratch`, per device

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }   // 256-byte pieces

// int32 elements of every planning scratch array of `d`, in the order they
// are carved out of the array.
struct Carve {
  int64_t n[10];
  int64_t total() const {
    int64_t t = 0;
    for (int64_t v : n) t += pad64(v);
    return t;
  }
};

Carve carve(const Dims& d) {
  return Carve{{(int64_t)d.R * d.nch * d.E, (int64_t)d.R * d.E, (int64_t)d.R * (d.R + 1) * 2,
                (int64_t)d.R, (int64_t)d.E, (int64_t)d.R * d.nch, 2LL * d.E, 2LL * d.E,
                2LL * d.E, (int64_t)d.R}};
}

bool plan_arrays_ok(const moonep_plan_t* p) {
  if (!p) return false;
  const int32_t* a[] = {p->counts, p->dest, p->src, p->cu_seqlens,
                        p->seg_tokens, p->prefetch_src, p->stats, p->aux};
  for (const int32_t* q : a)
    if (!q || (uintptr_t)q % 4) return false;
  return true;
}

// The device address of this device's scratch array (looked up on the first
// call with the device current).
hipError_t device_scratch(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = (int32_t*)ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace moonep

using namespace moonep;

extern "C" moonep_status_t moonep_plan_noalloc(const moonep_config_t* cfg, const int32_t* topk,
                                               const int32_t* tokens_per_expert,
                                               const moonep_plan_t* plan, hipStream_t stream) {
  Dims d;
  if (!dims_from_config(cfg, &d)) return MOONEP_ERR_CONFIG;
  if (!topk || (uintptr_t)topk % 4 || !plan_arrays_ok(plan)) return MOONEP_ERR_ARG;
  if (tokens_per_expert && (uintptr_t)tokens_per_expert % 4) return MOONEP_ERR_ARG;
  const Carve cv = carve(d);
  if (cv.total() > kScratchInts) return MOONEP_ERR_SCRATCH;
  int32_t* base = nullptr;
  if (device_scratch(&base) != hipSuccess) return MOONEP_ERR_HIP;
  Ctx c;
  c.d = d;
  c.device = 0;
  c.num_cu_device = 0;
  int32_t** dst[10] = {&c.cc, &c.shift, &c.pieces, &c.npieces, &c.line, &c.chunk_err,
                        &c.efix, &c.aend, &c.an, &c.rend};
  int64_t off = 0;
  for (int i = 0; i < 10; ++i) {
    *dst[i] = base + off;
    off += pad64(cv.n[i]);
  }
  return launch_plan(c, topk, tokens_per_expert, *plan, stream) == hipSuccess ? MOONEP_OK
                                                                              : MOONEP_ERR_HIP;
}
