// Record table and C entry points of the launch timing (prof.hpp).
#include "../../include/mtl.h"

#include <hip/hip_runtime.h>

#include "prof.hpp"

namespace mtl {
namespace prof {
namespace {

struct Rec {
  Slot ev;
  int kind;
  double flop, bytes;
  const char* name;
};
Rec recs[MTL_PROF_MAX];
int count = 0;
bool on = false;
int events_device = -1;  // the device the events were created on (-1: none yet)

}  // namespace

bool enabled() { return on; }

Slot* begin(int kind, const char* name, double flop, double bytes) {
  if (count >= MTL_PROF_MAX) return nullptr;
  Rec& r = recs[count++];
  r.kind = kind;
  r.flop = flop;
  r.bytes = bytes;
  r.name = name;
  return &r.ev;
}

}  // namespace prof
}  // namespace mtl

using namespace mtl::prof;

extern "C" {

mtl_status mtl_prof_start(void) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MTL_E_HIP;
  if (events_device != dev) {
    if (events_device >= 0) {
      int cur = dev;
      if (hipSetDevice(events_device) != hipSuccess) return MTL_E_HIP;
      for (Rec& r : recs) {
        (void)hipEventDestroy(r.ev.start);
        (void)hipEventDestroy(r.ev.stop);
      }
      if (hipSetDevice(cur) != hipSuccess) return MTL_E_HIP;
      events_device = -1;
    }
    for (Rec& r : recs)
      if (hipEventCreate(&r.ev.start) != hipSuccess || hipEventCreate(&r.ev.stop) != hipSuccess) return MTL_E_HIP;
    events_device = dev;
  }
  count = 0;
  on = true;
  return MTL_OK;
}

mtl_status mtl_prof_stop(int32_t* n_records) {
  if (!n_records) return MTL_E_NULL;
  on = false;
  *n_records = count;
  return MTL_OK;
}

mtl_status mtl_prof_record(int32_t i, int32_t* kind, double* flop, double* bytes, float* ms, const char** name) {
  if (!kind || !flop || !bytes || !ms || !name) return MTL_E_NULL;
  if (on) return MTL_E_UNSUPPORTED;
  if (i < 0 || i >= count) return MTL_E_SHAPE;
  const Rec& r = recs[i];
  if (hipEventSynchronize(r.ev.stop) != hipSuccess) return MTL_E_HIP;
  if (hipEventElapsedTime(ms, r.ev.start, r.ev.stop) != hipSuccess) return MTL_E_HIP;
  *kind = r.kind;
  *flop = r.flop;
  *bytes = r.bytes;
  *name = r.name;
  return MTL_OK;
}

}  // extern "C"
