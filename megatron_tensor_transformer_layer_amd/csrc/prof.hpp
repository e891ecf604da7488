// Opt-in timing of the library's launches, for measurement.  While it is on
// (mtl_prof_start), each group of launches an entry point makes -- one GEMM or
// GEMM pair, the attention kernels, one reduce, one column-sum pair, one
// quantisation pair -- is bracketed by two HIP events recorded on the stream
// it runs on, and kept with its kind and its algorithmic FLOP and HBM bytes.
// Off (the default), timed() only calls the launch.
#pragma once

#include <hip/hip_runtime.h>

namespace mtl {
namespace prof {

enum Kind { GEMM = 0, ATTN = 1, REDUCE = 2, COLSUM = 3, QUANT = 4, GATHER = 5 };

struct Slot {
  hipEvent_t start, stop;
};

bool enabled();
// The next record's events, or nullptr once the table is full.
Slot* begin(int kind, const char* name, double flop, double bytes);

template <class F>
hipError_t timed(int kind, const char* name, double flop, double bytes, hipStream_t s, F&& launch) {
  Slot* sl = enabled() ? begin(kind, name, flop, bytes) : nullptr;
  if (!sl) return launch();
  hipError_t e = hipEventRecord(sl->start, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  return hipEventRecord(sl->stop, s);
}

}  // namespace prof
}  // namespace mtl
