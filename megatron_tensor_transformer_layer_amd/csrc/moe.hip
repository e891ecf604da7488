// MoE routing and data movement for one expert-parallel rank, gfx950.
//
// Readings (the site summary's MoE deploy step gives 256 experts, a top-8
// router and EP 16 but no formula): the k largest fp32 logits per token, ties to
// the lower expert id, in slot order of decreasing logit; gates are the softmax
// over the k selected logits; rank r of ep owns experts [r*E/ep, (r+1)*E/ep);
// its assignments are grouped by expert with tokens ascending (a stable order),
// dropless.  The expert GEMMs run on the grouped modes of gemm_bf16.
//
// Every kernel here is deterministic: selection is exact comparison of the
// given fp32 values, the permutation is a scan, and every sum runs in a fixed
// order (slot order for the combine and the scatter of dX).
#include "common.hpp"
#include "kernels.hpp"

namespace mtl {

// ---------------------------------------------------------------- route
// Selection order: larger logit first, ties to the lower expert id; -0 and +0
// are equal, and NaN ranks below every number (-inf included), so a row with
// NaN logits still yields k distinct valid ids.  The order is taken on an
// integer key: NaN -> INT_MIN, otherwise the float's bits mapped monotonically
// onto signed integers (zero of either sign -> 0).
__device__ __forceinline__ int route_key(float f) {
  if (f != f) return INT_MIN;
  const int b = f == 0.f ? 0 : __float_as_int(f);
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float route_value(int key) {
  if (key == INT_MIN) return __int_as_float(0x7fc00000);
  return __int_as_float(key >= 0 ? key : key ^ 0x7fffffff);
}

// One wave per token; lane l holds logits l, l+64, ... (E <= 1024).  Round r
// of k picks the largest untaken key (lowest id among equals) by a wave
// butterfly; lane r keeps it, so slot r's id and gate are written by lane r.
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                        int32_t* __restrict__ idx, float* __restrict__ gates) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* row = logits + t * E;
  constexpr int PER = 16;
  int v[PER];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? route_key(row[e]) : INT_MIN;
    if (e >= E) taken |= 1u << j;
  }
  float mine_v = -INFINITY;
  int mine_i = 0;
  for (int r = 0; r < k; ++r) {
    // (INT_MIN, past every id) loses to every untaken candidate, a NaN included;
    // k <= E leaves at least one candidate per round
    int bv = INT_MIN;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      if (!(taken & (1u << j)) && (v[j] > bv || (v[j] == bv && e < bi))) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const int ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) {
      mine_v = route_value(bv);
      mine_i = bi;
    }
  }
  // softmax over the k selected logits; slot 0 holds the largest (a NaN among
  // them, or an all -inf selection, makes the gates NaN)
  const float top = __shfl(mine_v, 0);
  const float ex = lane < k ? expf(mine_v - top) : 0.f;
  float z = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
  if (lane < k) {
    idx[t * k + lane] = mine_i;
    gates[t * k + lane] = ex / z;
  }
}

hipError_t moe_route(const float* logits, int T, int E, int k, int32_t* idx, float* gates, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, T, E, k, idx, gates);
  return hipGetLastError();
}

// ---------------------------------------------------------------- router backward
// Load-balancing loss (the site's --moe-aux-loss-coeff; the pages give no
// formula, the Switch Transformer form is taken): L = alpha * E * sum_e f_e P_e
// with f_e = c_e / (T k) the share of the T*k assignments routed to e and P_e
// the token mean of the full softmax over all E logits; c_e is a constant of
// the backward.  With coef = alpha E / (T^2 k):
//   L = coef * sum_t q_t,  q_t = sum_e p_te c_e,
//   dL/dl_te = coef * p_te (c_e - q_t).
// The gates are the softmax over the k selected logits, whose backward is
//   dl_j += g_j (dg_j - sum_s g_s dg_s)  for the selected j.

// c_e over all T*k assignments: one workgroup, an LDS histogram (integer, so
// the result does not depend on the order of the atomic adds).
__global__ __launch_bounds__(1024) void moe_router_counts_kernel(const int32_t* __restrict__ idx, int64_t n, int E,
                                                                 int32_t* __restrict__ counts) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < 1024; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = hist[e];
}

// One wave per token; lane l holds experts l, l+64, ... (PER of them, E <= 64 PER).
template <int PER>
__global__ __launch_bounds__(256) void moe_router_bwd_kernel(const float* __restrict__ logits,
                                                             const int32_t* __restrict__ idx,
                                                             const float* __restrict__ gates,
                                                             const float* __restrict__ dgates,
                                                             const int32_t* __restrict__ counts, int T, int E, int k,
                                                             float coef, float* __restrict__ dlogits,
                                                             uint16_t* __restrict__ dlogits_bf16,
                                                             float* __restrict__ q_out) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* row = logits + t * E;
  float l[PER], c[PER];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    l[j] = e < E ? row[e] : -INFINITY;
    c[j] = e < E ? (float)counts[e] : 0.f;
    m = fmaxf(m, l[j]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    l[j] = lane + 64 * j < E ? expf(l[j] - m) : 0.f;  // l now holds the unnormalised p
    z += l[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
  const float inv = 1.f / z;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    l[j] *= inv;
    q += l[j] * c[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) q += __shfl_xor(q, off);
  // the gate softmax backward: lanes s < k hold slot s
  const float gs = lane < k ? gates[t * k + lane] : 0.f;
  const float dgs = lane < k ? dgates[t * k + lane] : 0.f;
  const int is = lane < k ? idx[t * k + lane] : -1;
  float inner = gs * dgs;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) inner += __shfl_xor(inner, off);
  float dl[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) dl[j] = coef * l[j] * (c[j] - q);
  for (int s = 0; s < k; ++s) {
    const int js = __shfl(is, s);
    const float add = __shfl(gs, s) * (__shfl(dgs, s) - inner);
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (lane + 64 * j == js) dl[j] += add;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      dlogits[t * E + e] = dl[j];
      dlogits_bf16[t * E + e] = (uint16_t)f32_to_bf16_bits(dl[j]);
    }
  }
  if (lane == 0) q_out[t] = q;
}

// L = coef * sum_t q_t, one workgroup in a fixed order (deterministic).
__global__ __launch_bounds__(1024) void moe_router_aux_kernel(const float* __restrict__ q, int T, float coef,
                                                              float* __restrict__ out) {
  __shared__ float part[1024];
  float s = 0.f;
  for (int t = threadIdx.x; t < T; t += blockDim.x) s += q[t];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = coef * part[0];
}

hipError_t moe_router_bwd(const float* logits, const int32_t* idx, const float* gates, const float* dgates, int T,
                          int E, int k, float alpha, int32_t* counts, float* q, float* aux_loss, float* dlogits,
                          uint16_t* dlogits_bf16, hipStream_t s) {
  if (T <= 0 || E <= 0 || E > 1024 || k <= 0 || k > 64) return hipErrorInvalidValue;
  const float coef = (float)((double)alpha * E / ((double)T * T * k));
  hipLaunchKernelGGL(moe_router_counts_kernel, dim3(1), dim3(1024), 0, s, idx, (int64_t)T * k, E, counts);
  const dim3 grid((unsigned)((T + 3) / 4));
  if (E <= 256)
    hipLaunchKernelGGL(moe_router_bwd_kernel<4>, grid, dim3(256), 0, s, logits, idx, gates, dgates, counts, T, E, k,
                       coef, dlogits, dlogits_bf16, q);
  else
    hipLaunchKernelGGL(moe_router_bwd_kernel<16>, grid, dim3(256), 0, s, logits, idx, gates, dgates, counts, T, E,
                       k, coef, dlogits, dlogits_bf16, q);
  if (aux_loss) hipLaunchKernelGGL(moe_router_aux_kernel, dim3(1), dim3(1024), 0, s, q, T, coef, aux_loss);
  return hipGetLastError();
}

// ---------------------------------------------------------------- permute
// One workgroup of 1024 threads per local expert, in two launches.  Thread t
// owns a contiguous chunk of the (token, slot) entries.  The first launch
// counts each expert's matches and clears the inverse map; the second takes
// the expert's base offset from the counts of the experts before it, counts
// its chunk's matches again, exclusive-scans them over the threads and writes
// the matches in entry order.  Entry order is (token, slot), so tokens ascend
// within an expert.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < 16; ++w) {
      const int c = sh[w];
      sh[w] = acc;
      acc += c;
    }
    sh[16] = acc;
  }
  __syncthreads();
  const int excl = sh[wave] + x - v;
  total = sh[16];
  __syncthreads();
  return excl;
}

__device__ __forceinline__ int chunk_matches(const int32_t* __restrict__ idx, int64_t b0, int64_t b1, int ex) {
  int c = 0;
  for (int64_t j = b0; j < b1; ++j) c += (idx[j] == ex);
  return c;
}

__global__ __launch_bounds__(1024) void moe_permute_count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                                 int e_lo, int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ slot_row) {
  __shared__ int sh[17];
  const int e = blockIdx.x;
  const int64_t n = (int64_t)T * k;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)e * blockDim.x + threadIdx.x; j < n; j += stride) slot_row[j] = -1;
  const int64_t chunk = (n + 1023) / 1024;
  const int64_t b0 = min(n, threadIdx.x * chunk), b1 = min(n, b0 + chunk);
  int total;
  block_exclusive_scan(chunk_matches(idx, b0, b1, e_lo + e), sh, total);
  if (threadIdx.x == 0) counts[e] = total;
}

__global__ __launch_bounds__(1024) void moe_permute_scatter_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                                   int e_lo, int E_l,
                                                                   const int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ ptok,
                                                                   int32_t* __restrict__ pslot,
                                                                   int32_t* __restrict__ slot_row) {
  __shared__ int sh[17];
  __shared__ int base_sh;
  const int e = blockIdx.x, ex = e_lo + e;
  if (threadIdx.x == 0) {
    int base = 0;
    for (int i = 0; i < e; ++i) base += counts[i];
    base_sh = base;
    offsets[e] = base;
    if (e == E_l - 1) offsets[E_l] = base + counts[e];
  }
  const int64_t n = (int64_t)T * k;
  const int64_t chunk = (n + 1023) / 1024;
  const int64_t b0 = min(n, threadIdx.x * chunk), b1 = min(n, b0 + chunk);
  int total;
  const int excl = block_exclusive_scan(chunk_matches(idx, b0, b1, ex), sh, total);  // its barriers publish base_sh
  int pos = base_sh + excl;
  for (int64_t j = b0; j < b1; ++j) {
    if (idx[j] == ex) {
      ptok[pos] = (int32_t)(j / k);
      pslot[pos] = (int32_t)(j % k);
      slot_row[j] = pos;
      ++pos;
    }
  }
}

hipError_t moe_permute(const int32_t* idx, int T, int k, int e_lo, int E_l, int32_t* counts, int32_t* offsets,
                       int32_t* ptok, int32_t* pslot, int32_t* slot_row, hipStream_t s) {
  if (E_l <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_permute_count_kernel, dim3((unsigned)E_l), dim3(1024), 0, s, idx, T, k, e_lo, counts,
                     slot_row);
  hipLaunchKernelGGL(moe_permute_scatter_kernel, dim3((unsigned)E_l), dim3(1024), 0, s, idx, T, k, e_lo, E_l, counts,
                     offsets, ptok, pslot, slot_row);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gather
// xp[i] = x[ptok[i]] for i < offsets[E_l]; 16 bytes per thread.
__global__ __launch_bounds__(256) void moe_gather_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ ptok,
                                                          const int32_t* __restrict__ offsets, int E_l, int64_t max_rows,
                                                          int64_t h, uint16_t* __restrict__ xp) {
  const int64_t nv = h / 8;
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = v / nv, c = v % nv;
  if (i >= max_rows || i >= offsets[E_l]) return;
  const int64_t t = ptok[i];
  *reinterpret_cast<u32x4*>(xp + i * h + c * 8) = *reinterpret_cast<const u32x4*>(x + t * h + c * 8);
}

hipError_t moe_gather(const uint16_t* x, const int32_t* ptok, const int32_t* offsets, int E_l, int64_t max_rows,
                      int64_t h, uint16_t* xp, hipStream_t s) {
  const int64_t nthreads = max_rows * (h / 8);
  if (nthreads <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_gather_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, s, x, ptok, offsets,
                     E_l, max_rows, h, xp);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine and dX scatter
// out[t] = sum over slots s (ascending) with slot_row[t,s] >= 0 of
//          (gates ? gates[t,s] : 1) * rows[slot_row[t,s]]; fp32 sum, bf16 out.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ rows,
                                                           const int32_t* __restrict__ slot_row,
                                                           const float* __restrict__ gates, int T, int k, int64_t h,
                                                           uint16_t* __restrict__ out) {
  const int64_t nv = h / 8;
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = v / nv, c = v % nv;
  if (t >= T) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = 0; s < k; ++s) {
    const int32_t r = slot_row[t * k + s];
    if (r < 0) continue;
    const float g = gates ? gates[t * k + s] : 1.f;
    const u32x4 x = *reinterpret_cast<const u32x4*>(rows + (int64_t)r * h + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += g * bf16_lo(x[j]);
      acc[2 * j + 1] += g * bf16_hi(x[j]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  *reinterpret_cast<u32x4*>(out + t * h + c * 8) = o;
}

hipError_t moe_combine(const uint16_t* rows, const int32_t* slot_row, const float* gates, int T, int k, int64_t h,
                       uint16_t* out, hipStream_t s) {
  const int64_t nthreads = (int64_t)T * (h / 8);
  if (nthreads <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, s, rows, slot_row,
                     gates, T, k, h, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine backward
// For every local assignment row i (token t, slot s): dye[i] = g[t,s] * dy[t]
// and dgates[t,s] = <ye[i], dy[t]> (fp32, one wave per row, fixed lane order);
// dgates of slots whose expert is not local are zero.
__global__ __launch_bounds__(256) void moe_gate_grad_zero_kernel(const int32_t* __restrict__ slot_row, int64_t n,
                                                                  float* __restrict__ dgates) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n && slot_row[j] < 0) dgates[j] = 0.f;
}

__global__ __launch_bounds__(256) void moe_combine_bwd_kernel(const uint16_t* __restrict__ dy,
                                                               const uint16_t* __restrict__ ye,
                                                               const int32_t* __restrict__ ptok,
                                                               const int32_t* __restrict__ pslot,
                                                               const int32_t* __restrict__ offsets, int E_l,
                                                               int64_t max_rows, const float* __restrict__ gates, int k,
                                                               int64_t h, uint16_t* __restrict__ dye,
                                                               float* __restrict__ dgates) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= max_rows || i >= offsets[E_l]) return;
  const int64_t t = ptok[i];
  const int s = pslot[i];
  const float g = gates[t * k + s];
  float dot = 0.f;
  for (int64_t c = lane; c < h / 8; c += 64) {
    const u32x4 d = *reinterpret_cast<const u32x4*>(dy + t * h + c * 8);
    const u32x4 y = *reinterpret_cast<const u32x4*>(ye + i * h + c * 8);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d0 = bf16_lo(d[j]), d1 = bf16_hi(d[j]);
      dot += bf16_lo(y[j]) * d0 + bf16_hi(y[j]) * d1;
      o[j] = pack_bf16x2(g * d0, g * d1);
    }
    *reinterpret_cast<u32x4*>(dye + i * h + c * 8) = o;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
  if (lane == 0) dgates[t * k + s] = dot;
}

hipError_t moe_combine_bwd(const uint16_t* dy, const uint16_t* ye, const int32_t* ptok, const int32_t* pslot,
                           const int32_t* slot_row, const int32_t* offsets, int E_l, int64_t max_rows,
                           const float* gates, int T, int k, int64_t h, uint16_t* dye, float* dgates, hipStream_t s) {
  const int64_t n = (int64_t)T * k;
  if (n > 0) {
    hipLaunchKernelGGL(moe_gate_grad_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, slot_row, n,
                       dgates);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (max_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_combine_bwd_kernel, dim3((unsigned)((max_rows + 3) / 4)), dim3(256), 0, s, dy, ye, ptok,
                     pslot, offsets, E_l, max_rows, gates, k, h, dye, dgates);
  return hipGetLastError();
}

}  // namespace mtl
