// Symmetric [E+B,H,Hp] buffers of one projection, built with the HIP virtual
// memory API.  This is the weight and gradient buffer layout of the MoonEP
// README ("Usage > Integration > Weight buffer" and "Gradient buffer") for
// the R ranks that share one GPU.
//
// Physical memory: per rank d, one chunk of E/R rows (its home experts, or
// their gradients) and one chunk of B rows (its prefetch slots, or its reduce
// buffer).  Three virtual ranges map those chunks:
//   views [R][E+B]: rank d's contiguous [E+B] range starts at row d*(E+B);
//                   its rows [0,E) map the R home chunks in rank order, and
//                   its rows [E,E+B) map its own slot chunk;
//   home  [E]:      the home chunks in rank order;
//   slots [R][B]:   the slot chunks in rank order.
// Every home chunk is therefore mapped R+1 times and every slot chunk twice,
// so the buffer costs E + R*B rows of HBM whatever the number of views.  A
// symbuf may instead map the slot chunks of another one (the prefetch pool
// is one process-wide allocation shared by every layer): it then adds only
// E rows, and the shared chunks live until the last symbuf mapping them is
// destroyed.
#include <stdlib.h>

#include <memory>
#include <new>
#include <vector>

#include "internal.h"

using namespace moonep;

namespace {

struct Mapping {
  char* va;
  size_t size;
};

// Physical chunks, released when the last symbuf holding them lets go.
struct Chunks {
  std::vector<hipMemGenericAllocationHandle_t> h;
  ~Chunks() {
    for (auto x : h) (void)hipMemRelease(x);   // best effort at teardown
  }
};

}  // namespace

struct moonep_symbuf {
  int device = 0;
  int R = 0, E = 0, B = 0, L = 0;
  size_t row_bytes = 0, gran = 0;
  bool own_slots = true;
  std::shared_ptr<Chunks> home_chunks, slot_chunks;
  std::vector<Mapping> maps;
  std::vector<Mapping> ranges;   // reservations
  char* views = nullptr;
  char* home = nullptr;
  char* slots = nullptr;
};

static hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

// Releases everything `b` holds, in reverse order of creation; returns the
// first error met (and keeps going).
static hipError_t release(moonep_symbuf* b) {
  hipError_t err = hipSuccess;
  auto keep = [&](hipError_t e) {
    if (e != hipSuccess && err == hipSuccess) err = e;
  };
  for (const Mapping& m : b->maps) keep(hipMemUnmap(m.va, m.size));
  for (const Mapping& r : b->ranges) keep(hipMemAddressFree(r.va, r.size));
  b->maps.clear();
  b->ranges.clear();
  b->home_chunks.reset();
  b->slot_chunks.reset();
  return err;
}

static hipError_t reserve(moonep_symbuf* b, size_t size, char** out) {
  void* va = nullptr;
  hipError_t e = hipMemAddressReserve(&va, size, b->gran, nullptr, 0);
  if (e != hipSuccess) return e;
  b->ranges.push_back({(char*)va, size});
  *out = (char*)va;
  return hipSuccess;
}

static hipError_t map(moonep_symbuf* b, char* va, size_t size,
                      hipMemGenericAllocationHandle_t h) {
  hipError_t e = hipMemMap(va, size, 0, h, 0);
  if (e != hipSuccess) return e;
  b->maps.push_back({va, size});
  return hipSuccess;
}

extern "C" {

moonep_status_t moonep_vmm_granularity(int64_t* out) {
  if (!out) return MOONEP_ERR_ARG;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return MOONEP_ERR_HIP;
  hipMemAllocationProp prop = device_prop(device);
  size_t g = 0;
  if (hipMemGetAllocationGranularity(&g, &prop, hipMemAllocationGranularityMinimum) !=
      hipSuccess)
    return MOONEP_ERR_HIP;
  *out = (int64_t)g;
  return MOONEP_OK;
}

moonep_status_t moonep_symbuf_create(moonep_handle_t h, int32_t elem_bytes,
                                     moonep_symbuf_t slots_from, moonep_symbuf_t* out) {
  if (!h || !out || (elem_bytes != 2 && elem_bytes != 4)) return MOONEP_ERR_ARG;
  *out = nullptr;
  const Dims& d = h->c.d;
  if (slots_from && (slots_from->R != d.R || slots_from->B != d.B ||
                     slots_from->row_bytes != (size_t)d.H * d.Hp * elem_bytes))
    return MOONEP_ERR_ARG;
  moonep_symbuf* b = new (std::nothrow) moonep_symbuf;
  if (!b) return MOONEP_ERR_NOMEM;
  b->R = d.R; b->E = d.E; b->B = d.B; b->L = d.L;
  b->row_bytes = (size_t)d.H * d.Hp * elem_bytes;
  if (hipGetDevice(&b->device) != hipSuccess) {
    delete b;
    return MOONEP_ERR_HIP;
  }
  hipMemAllocationProp prop = device_prop(b->device);
  if (hipMemGetAllocationGranularity(&b->gran, &prop, hipMemAllocationGranularityMinimum) !=
          hipSuccess ||
      b->gran == 0) {
    delete b;
    return MOONEP_ERR_HIP;
  }
  const size_t home_chunk = (size_t)d.L * b->row_bytes;
  const size_t slot_chunk = (size_t)d.B * b->row_bytes;
  if (home_chunk % b->gran || slot_chunk % b->gran) {
    delete b;
    return MOONEP_ERR_CONFIG;
  }
  if (slots_from && slots_from->device != b->device) {
    delete b;
    return MOONEP_ERR_ARG;
  }
  moonep_status_t st = MOONEP_OK;
  hipError_t e = hipSuccess;
  // physical chunks (the slot chunks possibly another symbuf's)
  b->home_chunks = std::make_shared<Chunks>();
  b->slot_chunks = slots_from ? slots_from->slot_chunks : std::make_shared<Chunks>();
  b->own_slots = !slots_from;
  for (int r = 0; r < d.R && e == hipSuccess; ++r) {
    hipMemGenericAllocationHandle_t ph;
    e = hipMemCreate(&ph, home_chunk, &prop, 0);
    if (e == hipSuccess) b->home_chunks->h.push_back(ph);
    if (e == hipSuccess && slot_chunk && !slots_from) {
      e = hipMemCreate(&ph, slot_chunk, &prop, 0);
      if (e == hipSuccess) b->slot_chunks->h.push_back(ph);
    }
  }
  if (e == hipErrorOutOfMemory) st = MOONEP_ERR_NOMEM;
  // virtual ranges and their mappings
  const size_t view_rows = (size_t)d.E + d.B;
  if (e == hipSuccess) e = reserve(b, (size_t)d.R * view_rows * b->row_bytes, &b->views);
  if (e == hipSuccess) e = reserve(b, (size_t)d.E * b->row_bytes, &b->home);
  if (e == hipSuccess && slot_chunk) e = reserve(b, (size_t)d.R * slot_chunk, &b->slots);
  for (int r = 0; r < d.R && e == hipSuccess; ++r) {
    char* view = b->views + (size_t)r * view_rows * b->row_bytes;
    for (int g = 0; g < d.R && e == hipSuccess; ++g)
      e = map(b, view + (size_t)g * home_chunk, home_chunk, b->home_chunks->h[g]);
    if (e == hipSuccess && slot_chunk)
      e = map(b, view + (size_t)d.E * b->row_bytes, slot_chunk, b->slot_chunks->h[r]);
    if (e == hipSuccess)
      e = map(b, b->home + (size_t)r * home_chunk, home_chunk, b->home_chunks->h[r]);
    if (e == hipSuccess && slot_chunk)
      e = map(b, b->slots + (size_t)r * slot_chunk, slot_chunk, b->slot_chunks->h[r]);
  }
  // read/write access from the device, over every fully mapped range
  hipMemAccessDesc acc = {};
  acc.location = prop.location;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  for (size_t i = 0; i < b->ranges.size() && e == hipSuccess; ++i)
    e = hipMemSetAccess(b->ranges[i].va, b->ranges[i].size, &acc, 1);
  if (e != hipSuccess) {
    (void)release(b);   // the first error is the one reported
    delete b;
    return st != MOONEP_OK ? st : MOONEP_ERR_HIP;
  }
  *out = b;
  return MOONEP_OK;
}

moonep_status_t moonep_symbuf_info(moonep_symbuf_t b, moonep_symbuf_info_t* out) {
  if (!b || !out) return MOONEP_ERR_ARG;
  out->views = b->views;
  out->home = b->home;
  out->slots = b->slots;
  out->row_bytes = (int64_t)b->row_bytes;
  out->physical_bytes =
      ((int64_t)b->E + (b->own_slots ? (int64_t)b->R * b->B : 0)) * (int64_t)b->row_bytes;
  out->granularity = (int64_t)b->gran;
  return MOONEP_OK;
}

moonep_status_t moonep_symbuf_destroy(moonep_symbuf_t b) {
  if (!b) return MOONEP_OK;
  // no kernel may still use the ranges when they are unmapped
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess && cur != b->device) e = hipSetDevice(b->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (cur != b->device) (void)hipSetDevice(cur);   // restore the caller's device
  hipError_t r = release(b);
  delete b;
  return (e == hipSuccess && r == hipSuccess) ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // extern "C"
