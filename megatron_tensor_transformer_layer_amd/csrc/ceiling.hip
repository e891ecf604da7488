// The matrix cores' own rate on this chip, for judging the GEMMs against: a
// kernel that issues the 128x128-per-wave MFMA stream of the 256x256 GEMM tiles
// (4 waves per workgroup, one workgroup per CU) with every operand already in
// registers -- no global loads in the loop, no LDS, no barrier, no epilogue.
// Its time is what the MFMAs alone take at the clock the chip holds under that
// load, on operands of the caller's distribution.
#include "../../include/mtl.h"

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace mtl {
namespace {

// Operand fragments per wave: 2 k-steps x (4 row fragments of A + 4 column
// fragments of B), 16 bytes per lane each.
constexpr int FRAGS = 16;
constexpr int SLOTS = 64;  // waves w and w + 64 read the same fragments

template <int KIND>
__global__ __launch_bounds__(256, 1) void mfma_ceiling_kernel(const u32x4* __restrict__ data, int64_t iters,
                                                              float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const u32x4* src = data + (size_t)(wave % SLOTS) * FRAGS * 64 + lane;
  u32x4 fa[2][4], fb[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[kk][i] = src[(kk * 8 + i) * 64];
      fb[kk][i] = src[(kk * 8 + 4 + i) * 64];
    }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
    if (KIND == 0) {  // bf16: two 32x32x16 k-steps per tile
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[kk][i], fb[kk][j], acc[i][j]);
    } else if (KIND == 1) {  // fp8 E4M3: one 32x32x64 k-step per tile, 32 bytes per lane per operand
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32_f8<0, 0>(fa[0][i], fa[1][i], fb[0][j], fb[1][j], acc[i][j]);
    } else {  // MXFP4: one 32x32x64 k-step per tile, 16 bytes per lane per operand, unit scales
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma32_mxfp4(fa[0][i], fb[0][j], acc[i][j], 0x7f7f7f7fu, 0x7f7f7f7fu, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace mtl

extern "C" mtl_status mtl_mfma_ceiling(const void* data, size_t data_bytes, int32_t kind, int64_t workgroups,
                                       int64_t iters, float* out, mtl_stream_t stream) {
  if (!data || !out) return MTL_E_NULL;
  if (((uintptr_t)data | (uintptr_t)out) & 15) return MTL_E_ALIGN;
  if (kind < 0 || kind > 2) return MTL_E_UNSUPPORTED;
  if (data_bytes < (size_t)MTL_CEILING_DATA_BYTES || workgroups <= 0 || workgroups > (1 << 20) || iters <= 0)
    return MTL_E_SHAPE;
  const dim3 grid((unsigned)workgroups), block(256);
  const hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(mtl::mfma_ceiling_kernel<0>, grid, block, 0, s, (const mtl::u32x4*)data, iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(mtl::mfma_ceiling_kernel<1>, grid, block, 0, s, (const mtl::u32x4*)data, iters, out);
  else
    hipLaunchKernelGGL(mtl::mfma_ceiling_kernel<2>, grid, block, 0, s, (const mtl::u32x4*)data, iters, out);
  return hipGetLastError() == hipSuccess ? MTL_OK : MTL_E_HIP;
}
