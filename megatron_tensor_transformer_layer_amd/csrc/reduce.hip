// HBM-streaming reductions for gfx950.
//
// reduce_partials: the on-device stand-in for the tensor-parallel all-reduce
// that follows a row-parallel linear: out = sum_i partial_i (+ bias) (+ residual),
// summed in fp32 in rank order, written bf16.  Every lane moves 16 bytes per
// load; the grid is a multiple of the 256 CUs and strides over the row range.
//
// allgather_rows: the on-device stand-in for the sequence-parallel all-gather
// that precedes a column-parallel linear: rank i's share of a [rows, cols]
// tensor is rows [i*rows/t, (i+1)*rows/t) of its own full-size buffer; the
// t-1 peer shares are copied into the calling rank's buffer in place.  One
// launch moves all of them, 16 bytes per lane.
//
// colsum_bf16: the bias gradients of the four linears are column sums of a
// [rows, cols] bf16 gradient.  Deterministic two-stage sum: stage 1 gives each
// 256-thread block 512 columns x 64 rows (16-byte loads, all 16 of a lane in
// flight at once, fp32 accumulate, the four waves combined in a fixed order)
// and writes one partial row to the workspace; stage 2 adds the partial rows,
// four waves each taking every fourth one, combined in wave order.
#include "common.hpp"
#include "kernels.hpp"

namespace mtl {

constexpr int MAX_PARTIALS = 16;

struct ReduceArgs {
  const uint16_t* p[MAX_PARTIALS];
  const uint16_t* bias;
  const uint16_t* residual;
  uint16_t* out;
  int t;
  int64_t cols;  // multiple of 8
  int64_t begin, count;  // element range (row_begin*cols, rows*cols)
};

// T > 0: exactly T partials, whose loads are all issued before the first add;
// T == 0: a.t partials, one at a time.  The sum is in rank order either way.
// The partials are read once: nontemporal loads keep them out of the caches.
template <int T>
__global__ __launch_bounds__(256) void reduce_partials_kernel(ReduceArgs a) {
  const int64_t nvec = a.count / 8;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = a.begin + v * 8;
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (T > 0) {
      u32x4 x[T];
#pragma unroll
      for (int i = 0; i < T; ++i) x[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.p[i] + e));
#pragma unroll
      for (int i = 0; i < T; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[2 * j] += bf16_lo(x[i][j]);
          s[2 * j + 1] += bf16_hi(x[i][j]);
        }
    } else {
      for (int i = 0; i < a.t; ++i) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.p[i] + e));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[2 * j] += bf16_lo(x[j]);
          s[2 * j + 1] += bf16_hi(x[j]);
        }
      }
    }
    if (a.bias) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(a.bias + (e % a.cols));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += bf16_lo(x[j]);
        s[2 * j + 1] += bf16_hi(x[j]);
      }
    }
    if (a.residual) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(a.residual + e);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += bf16_lo(x[j]);
        s[2 * j + 1] += bf16_hi(x[j]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(s[2 * j], s[2 * j + 1]);
    *reinterpret_cast<u32x4*>(a.out + e) = o;
  }
}

hipError_t reduce_partials(int t, const uint16_t* const* partials, const uint16_t* bias, const uint16_t* residual,
                           uint16_t* out, int64_t cols, int64_t row_begin, int64_t row_end, hipStream_t s) {
  if (t < 1 || t > MAX_PARTIALS) return hipErrorInvalidValue;
  ReduceArgs a{};
  for (int i = 0; i < t; ++i) a.p[i] = partials[i];
  a.bias = bias;
  a.residual = residual;
  a.out = out;
  a.t = t;
  a.cols = cols;
  a.begin = row_begin * cols;
  a.count = (row_end - row_begin) * cols;
  if (a.count <= 0) return hipSuccess;
  const int64_t nvec = a.count / 8;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  switch (t) {
    case 1: hipLaunchKernelGGL(reduce_partials_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(reduce_partials_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(reduce_partials_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(reduce_partials_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(reduce_partials_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

struct GatherArgs {
  const uint16_t* src[MAX_PARTIALS];  // the t-1 peer buffers, in rank order
  int64_t first[MAX_PARTIALS];        // element offset of each peer's share
  uint16_t* out;
  int64_t share;                      // elements per share (multiple of 8)
  int peers;
};

__global__ __launch_bounds__(256) void allgather_rows_kernel(GatherArgs a) {
  const int64_t vper = a.share / 8;
  const int64_t nvec = vper * a.peers;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(v / vper);
    const int64_t e = a.first[i] + (v - (int64_t)i * vper) * 8;
    *reinterpret_cast<u32x4*>(a.out + e) = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.src[i] + e));
  }
}

hipError_t allgather_rows(int t, int rank, const uint16_t* const* bufs, uint16_t* out, int64_t rows, int64_t cols,
                          hipStream_t s) {
  if (t < 1 || t > MAX_PARTIALS || rank < 0 || rank >= t || rows % t) return hipErrorInvalidValue;
  GatherArgs a{};
  a.out = out;
  a.share = rows / t * cols;
  for (int i = 0; i < t; ++i) {
    if (i == rank) continue;
    a.src[a.peers] = bufs[i];
    a.first[a.peers] = (int64_t)i * a.share;
    ++a.peers;
  }
  if (a.peers == 0 || a.share == 0) return hipSuccess;
  int64_t blocks = (a.share / 8 * a.peers + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(allgather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

constexpr int CS_ROWS = 64;   // rows per stage-1 block (16 per wave)
constexpr int CS_COLS = 512;  // columns per stage-1 block (8 per lane)

size_t colsum_ws_floats(int64_t rows, int64_t cols) {
  return (size_t)((rows + CS_ROWS - 1) / CS_ROWS) * (size_t)cols;
}

// Up to two column sums in one pair of launches (the bias gradients that are
// ready at the same point of a backward pass).
struct ColsumArgs {
  const uint16_t* x[2];
  float* out[2];
  float* ws[2];
  int64_t cols[2];
  int64_t rows, chunks;
  int split1, split2;  // stage-1 / stage-2 blocks of job 0
  int accumulate;
};

// Stage 1: block (column slab, row chunk); wave w sums rows r0+w, r0+w+4, ...
// of its 512 columns; the four wave sums are added in wave order through LDS.
__global__ __launch_bounds__(256) void colsum_stage1(ColsumArgs a) {
  __shared__ f32x4 part[3][64][2];
  const int job = (int)blockIdx.x < a.split1 ? 0 : 1;
  const int slab = (int)blockIdx.x - (job ? a.split1 : 0);
  const uint16_t* x = a.x[job];
  const int64_t cols = a.cols[job];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)slab * CS_COLS + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * CS_ROWS;
  const int64_t r1 = min(a.rows, r0 + CS_ROWS);
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c < cols) {
    constexpr int PER = CS_ROWS / 4;  // rows of this wave: r0 + wave + 4i
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t r = r0 + wave + 4 * i;
      v[i] = r < r1 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + r * cols + c)) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += bf16_lo(v[i][j]);
        s[2 * j + 1] += bf16_hi(v[i][j]);
      }
  }
  if (wave > 0) {
    part[wave - 1][lane][0] = f32x4{s[0], s[1], s[2], s[3]};
    part[wave - 1][lane][1] = f32x4{s[4], s[5], s[6], s[7]};
  }
  __syncthreads();
  if (wave == 0 && c < cols) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const f32x4 p0 = part[w][lane][0], p1 = part[w][lane][1];
      s[0] += p0[0]; s[1] += p0[1]; s[2] += p0[2]; s[3] += p0[3];
      s[4] += p1[0]; s[5] += p1[1]; s[6] += p1[2]; s[7] += p1[3];
    }
    float* w = a.ws[job] + (int64_t)blockIdx.y * cols + c;
    *reinterpret_cast<f32x4*>(w) = f32x4{s[0], s[1], s[2], s[3]};
    *reinterpret_cast<f32x4*>(w + 4) = f32x4{s[4], s[5], s[6], s[7]};
  }
}

// Stage 2: 256 columns per block, 4 per lane; wave w adds chunk partials
// w, w+4, w+8, ... in order, and the four wave sums are added in wave order.
__global__ __launch_bounds__(256) void colsum_stage2(ColsumArgs a) {
  __shared__ f32x4 part[3][64];
  const int job = (int)blockIdx.x < a.split2 ? 0 : 1;
  const int blk = (int)blockIdx.x - (job ? a.split2 : 0);
  const float* ws = a.ws[job];
  const int64_t cols = a.cols[job], chunks = a.chunks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)blk * 256 + lane * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (c < cols) {
    int64_t k = wave;
    for (; k + 28 < chunks; k += 32) {  // eight loads in flight
      f32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const f32x4*>(ws + (k + 4 * i) * cols + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; k < chunks; k += 4) s += *reinterpret_cast<const f32x4*>(ws + k * cols + c);
  }
  if (wave > 0) part[wave - 1][lane] = s;
  __syncthreads();
  if (wave == 0 && c < cols) {
#pragma unroll
    for (int w = 0; w < 3; ++w) s += part[w][lane];
    f32x4* o = reinterpret_cast<f32x4*>(a.out[job] + c);
    *o = a.accumulate ? *o + s : s;
  }
}

hipError_t colsum_bf16(const ColsumJob* jobs, int njobs, int64_t rows, bool accumulate, float* ws, hipStream_t s) {
  if (njobs < 1 || njobs > 2) return hipErrorInvalidValue;
  ColsumArgs a{};
  a.rows = rows;
  a.chunks = (rows + CS_ROWS - 1) / CS_ROWS;
  a.accumulate = accumulate ? 1 : 0;
  int64_t b1 = 0, b2 = 0, off = 0;
  for (int j = 0; j < njobs; ++j) {
    a.x[j] = jobs[j].x;
    a.out[j] = jobs[j].out;
    a.cols[j] = jobs[j].cols;
    a.ws[j] = ws + off;
    off += a.chunks * jobs[j].cols;
    b1 += (jobs[j].cols + CS_COLS - 1) / CS_COLS;
    b2 += (jobs[j].cols + 255) / 256;
    if (j == 0) {
      a.split1 = (int)b1;
      a.split2 = (int)b2;
    }
  }
  if (b1 == 0) return hipSuccess;
  if (a.chunks > 0) {
    hipLaunchKernelGGL(colsum_stage1, dim3((unsigned)b1, (unsigned)a.chunks), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colsum_stage2, dim3((unsigned)b2), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mtl
