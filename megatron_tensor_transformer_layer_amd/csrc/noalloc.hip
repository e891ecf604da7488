// The MLP backward for callers that cannot allocate device memory: its scratch
// is a file-scope device array instead of a caller's buffer.
#include "../../include/mtl.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace {

// mtl_mlp_bwd_noalloc's scratch.  Every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in for
// the symbol): it uses the device address looked up once per device below.
static __device__ __align__(256) unsigned char scratch[MTL_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
void* scratch_addr[MAX_DEVICES];
std::mutex scratch_mu;

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current).
mtl_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MTL_E_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MTL_E_HIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return MTL_OK;
}

}  // namespace

extern "C" mtl_status mtl_mlp_bwd_noalloc(const mtl_layer_cfg* c, const void* dy, const void* h, const void* gz,
                                          const void* a, const void* w1, const void* w2, void* dh_partial, float* dw1,
                                          float* db1, float* dw2, float* db2, mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  // the kept codes live in the caller's scratch of the forward calls, which
  // this entry point does not see
  if (c->flags & MTL_F_KEEP_CODES) return MTL_E_UNSUPPORTED;
  // refused before any HIP call when the configuration needs more scratch
  if (mtl::mlp_bwd_scratch_bytes(c) > (size_t)MTL_NOALLOC_SCRATCH_BYTES) return MTL_E_WORKSPACE;
  void* ws = nullptr;
  if ((st = device_scratch(&ws)) != MTL_OK) return st;
  // the kernels of mtl_mlp_bwd write every scratch byte they later read, so
  // nothing needs clearing between calls
  return mtl_mlp_bwd(c, dy, h, gz, a, w1, w2, dh_partial, dw1, db1, dw2, db2, ws, MTL_NOALLOC_SCRATCH_BYTES,
                     stream);
}
