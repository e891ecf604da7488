// MXFP4 and MXFP6 (OCP Microscaling: FP4 E2M1 or FP6 E2M3 elements in blocks
// of 32 along K sharing an E8M0 scale) quantisation and GEMMs for gfx950.
//
// Format: the scale of a block is 2^e with e = floor(log2(max |v|)) - 2
// (clamped at -127), stored as e + 127; each element is v / 2^e rounded to the
// nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even code, saturating at
// 6) with the sign of v; two codes per byte, the even element in the low
// nibble.  Finite inputs only.
//
// The GEMMs multiply on v_mfma_scale_f32_32x32x64_f8f6f4 with the block
// scales fed per lane: in a 32 x 64 operand fragment lane l holds row l % 32
// and the 32 elements k = (l / 32) * 32 .. +31 (16 bytes in FP4, 24 in FP6),
// i.e. exactly one scale block, whose E8M0 byte it passes as its scale.
#include "common.hpp"
#include "kernels.hpp"

namespace mtl {

// ---------------------------------------------------------------- quantise
// Four lanes per block of 32 elements: 16 bytes in and 4 bytes of codes out per
// lane, the block's amax exchanged among its four lanes, one scale byte.
__device__ __forceinline__ uint32_t e2m1_code(float y, uint32_t sign) {
  const float a = fabsf(y);
  uint32_t c;
  if (a <= 0.25f) c = 0;        // ties: 0.25 -> 0
  else if (a < 0.75f) c = 1;    // 0.5
  else if (a <= 1.25f) c = 2;   // 1 (0.75 and 1.25 -> 1)
  else if (a < 1.75f) c = 3;    // 1.5
  else if (a <= 2.5f) c = 4;    // 2 (1.75 and 2.5 -> 2)
  else if (a < 3.5f) c = 5;     // 3
  else if (a <= 5.0f) c = 6;    // 4 (3.5 and 5 -> 4)
  else c = 7;                   // 6, and everything above
  return c | (sign << 3);
}

// Eight codes (one 32-bit word, element 2j in the low nibble of byte j) of four
// packed bf16 pairs under the block's E8M0 byte sc: gfx950's
// v_cvt_scalef32_pk_fp4_f32 divides each value by the fp32 scale 2^(sc-127),
// rounds to the nearest E2M1 value with ties to the even code, saturates at
// +-6 and keeps the sign (also of zero) -- the rule above (checked bit for bit
// against the oracle on every finite bf16 value).  The scale must be a normal
// fp32 number, so sc = 0 (a block whose largest magnitude is below 2^-125)
// takes the comparisons of e2m1_code instead.
__device__ __forceinline__ uint32_t e2m1_pack8(const u32x4& v, uint32_t sc) {
  if (sc == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t bits = (h & 1) ? (v[h >> 1] >> 16) : (v[h >> 1] & 0xffffu);
      const float y = __uint_as_float(bits << 16) * 0x1p127f;
      w |= e2m1_code(y, bits >> 15) << (4 * h);
    }
    return w;
  }
  const float scale = __uint_as_float(sc << 23);
  // fp32 operands (exact widenings of the bf16 pair); the packed-bf16 form of
  // the instruction was folded into one conversion for all four pairs by this
  // compiler, so it is not used
  auto lo = [&](int j) { return __uint_as_float(v[j] << 16); };
  auto hi = [&](int j) { return __uint_as_float(v[j] & 0xffff0000u); };
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo(0), hi(0), scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo(1), hi(1), scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo(2), hi(2), scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo(3), hi(3), scale, 3);
  return w;
}

template <bool GO>  // scales in GEMM order (else plain)
__global__ __launch_bounds__(256) void mxfp4_quant_kernel(const uint16_t* __restrict__ x, int64_t nchunks,
                                                          int64_t nblocks, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  // chunk i = elements 8i .. 8i+7: consecutive lanes read consecutive 16 bytes,
  // and the four lanes 4b .. 4b+3 of a group hold block b's 32 elements
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = i < nchunks;  // nchunks % 4 == 0, so a group is all in or all out
  const u32x4 v = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + i * 8)) : u32x4{0, 0, 0, 0};
  uint32_t mx = 0;  // largest magnitude bits: integer order is value order for finite bf16
#pragma unroll
  for (int j = 0; j < 4; ++j) mx = max(mx, max(v[j] & 0x7fffu, (v[j] >> 16) & 0x7fffu));
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2));
  // amax = 2^(E-127) * 1.m for exponent field E >= 1; e = max(E - 129, -127),
  // so the E8M0 byte is max(E - 2, 0) (also for zero or subnormal amax)
  const int E = (int)(mx >> 7);
  const uint32_t sc = (uint32_t)max(E - 2, 0);
  const uint32_t w = e2m1_pack8(v, sc);
  if (!ok) return;
  *reinterpret_cast<uint32_t*>(codes + i * 4) = w;
  if ((i & 3) == 0) {
    const int64_t blk = i >> 2;  // row blk / nblocks, block blk % nblocks
    scales[GO ? mx_scale_index<true>(blk / nblocks, blk % nblocks, nblocks) : blk] = (uint8_t)sc;
  }
}

// The E8M0 byte and codes of one block of 32 bf16 values (bits), as
// mxfp4_quant_kernel forms them.
__device__ __forceinline__ void e2m1_block(const uint32_t (&bits)[32], u32x4& w, uint32_t& sc) {
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) mx = max(mx, bits[i] & 0x7fffu);
  const int E = (int)(mx >> 7);
  sc = (uint32_t)max(E - 2, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = {bits[8 * q] | (bits[8 * q + 1] << 16), bits[8 * q + 2] | (bits[8 * q + 3] << 16),
                     bits[8 * q + 4] | (bits[8 * q + 5] << 16), bits[8 * q + 6] | (bits[8 * q + 7] << 16)};
    w[q] = e2m1_pack8(v, sc);
  }
}

// Along rows, for shapes the tiled kernel below does not cover: lane l of a
// 64-lane group takes column c0 + l and one block of 32 rows, so the 64 lanes
// read 128 consecutive bytes per row; the lane then holds its block's 32
// elements and writes their 16 code bytes and the scale byte at row c of the
// transposed codes.
template <bool GO>
__global__ __launch_bounds__(256) void mxfp4_quant_t_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int64_t c = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t rb = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);  // block of 32 rows
  if (c >= cols || rb * 32 >= rows) return;
  uint32_t bits[32];
  const uint16_t* p = x + rb * 32 * cols + c;
#pragma unroll
  for (int i = 0; i < 32; ++i) bits[i] = p[(int64_t)i * cols];
  u32x4 w;
  uint32_t sc;
  e2m1_block(bits, w, sc);
  *reinterpret_cast<u32x4*>(codes + c * (rows / 2) + rb * 16) = w;
  scales[mx_scale_index<GO>(c, rb, rows / 32)] = (uint8_t)sc;
}

// Tiled quantisation of x [rows, cols] (rows % 64 == 0, cols % 128 == 0): a
// workgroup stages a 64 x 128 tile in LDS with coalesced 16-byte loads, then
// (ROWWISE) each thread quantises one 32-element block along a row -- codes
// [rows, cols/2], scales [rows, cols/32] -- and/or (COLWISE) one 32-element
// block down a column -- the codes of x^T, [cols, rows/2], and scales
// [cols, rows/32].  Both directions from one read of x.
template <bool ROWWISE, bool COLWISE, bool GO>
__global__ __launch_bounds__(256) void mxfp4_quant_tile_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                               int64_t cols, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               uint8_t* __restrict__ codes_t,
                                                               uint8_t* __restrict__ scales_t) {
  constexpr int TR = 64, TC = 128, LROW = TC * 2 + 16;  // LDS row stride (bytes), padded
  __shared__ __attribute__((aligned(16))) char tile[TR * LROW];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * TR, c0 = (int64_t)blockIdx.x * TC;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {  // 16 rows of 16 lanes x 16 bytes per pass
    const int r = pass * 16 + (t >> 4), ch = t & 15;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (r0 + r) * cols + c0 + ch * 8));
    *reinterpret_cast<u32x4*>(tile + r * LROW + ch * 16) = v;
  }
  __syncthreads();
  if constexpr (ROWWISE) {  // thread: row t / 4, block t % 4 (4 threads write 64 contiguous code bytes)
    const int r = t >> 2, b = t & 3;
    uint32_t bits[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * LROW + b * 64 + q * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bits[q * 8 + 2 * j] = v[j] & 0xffffu;
        bits[q * 8 + 2 * j + 1] = v[j] >> 16;
      }
    }
    u32x4 w;
    uint32_t sc;
    e2m1_block(bits, w, sc);
    *reinterpret_cast<u32x4*>(codes + (r0 + r) * (cols / 2) + c0 / 2 + b * 16) = w;
    scales[mx_scale_index<GO>(r0 + r, c0 / 32 + b, cols / 32)] = (uint8_t)sc;
  }
  if constexpr (COLWISE) {  // thread: column t / 2, row block t % 2
    const int c = t >> 1, rb = t & 1;
    uint32_t bits[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) bits[i] = *reinterpret_cast<const uint16_t*>(tile + (rb * 32 + i) * LROW + c * 2);
    u32x4 w;
    uint32_t sc;
    e2m1_block(bits, w, sc);
    *reinterpret_cast<u32x4*>(codes_t + (c0 + c) * (rows / 2) + r0 / 2 + rb * 16) = w;
    scales_t[mx_scale_index<GO>(c0 + c, r0 / 32 + rb, rows / 32)] = (uint8_t)sc;
  }
}

// FP6 E2M3 code of y (|y| < 8 by the block scale): below 1 the spacing is 1/8
// (subnormals, code = rint(8|y|)); in [2^E, 2^(E+1)) it is 2^(E-3); ties to
// even through rint, a rounding up to 2^(E+1) moves to the next exponent, and
// past 7.5 saturates.
__device__ __forceinline__ uint32_t e2m3_code(float y, uint32_t sign) {
  const float a = fabsf(y);
  uint32_t c;
  if (a < 1.0f) {
    c = (uint32_t)__builtin_rintf(a * 8.0f);  // 8 is the code of 1.0
  } else {
    int E = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;           // 0, 1 or 2
    uint32_t q = (uint32_t)__builtin_rintf(a * __uint_as_float((uint32_t)(130 - E) << 23));  // 8 .. 16
    if (q == 16) {
      ++E;
      q = 8;
    }
    c = E > 2 ? 31u : (((uint32_t)(E + 1) << 3) | (q - 8));
  }
  return c | (sign << 5);
}

// MXFP6: four lanes per block as for MXFP4; each lane's 8 codes are 48
// consecutive bits of the block's 24 bytes, written as three 16-bit words.
template <bool GO>  // codes and scales in GEMM order (else plain)
__global__ __launch_bounds__(256) void mxfp6_quant_kernel(const uint16_t* __restrict__ x, int64_t nchunks,
                                                          int64_t nblocks, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = i < nchunks;
  const u32x4 v = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + i * 8)) : u32x4{0, 0, 0, 0};
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) mx = max(mx, max(v[j] & 0x7fffu, (v[j] >> 16) & 0x7fffu));
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2));
  const int E = (int)(mx >> 7);
  const uint32_t sc = (uint32_t)max(E - 2, 0);  // E2M3's largest exponent is 2 as well
  const float mul = __uint_as_float((254u - sc) << 23);
  uint64_t w = 0;
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const uint32_t bits = (h & 1) ? (v[h >> 1] >> 16) : (v[h >> 1] & 0xffffu);
    const float y = __uint_as_float(bits << 16) * mul;
    w |= (uint64_t)e2m3_code(y, bits >> 15) << (6 * h);
  }
  if (!ok) return;
  if constexpr (GO) {
    // the lane's bytes 6j .. 6j+5 of block q of row r, word by word (no word
    // straddles a head/tail or half boundary)
    const int64_t blk = i >> 2, r = blk / nblocks, q = blk % nblocks;
    uint8_t* row = codes + r * nblocks * 24;
    const int o = 6 * (int)(i & 3);
#pragma unroll
    for (int t = 0; t < 3; ++t)
      *reinterpret_cast<uint16_t*>(row + mx6_code_offset(r, q, o + 2 * t)) = (uint16_t)(w >> (16 * t));
    if ((i & 3) == 0) scales[mx_scale_index<true>(r, q, nblocks)] = (uint8_t)sc;
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(codes + i * 6);
    dst[0] = (uint16_t)w;
    dst[1] = (uint16_t)(w >> 16);
    dst[2] = (uint16_t)(w >> 32);
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)sc;
  }
}

hipError_t mxfp6_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                          hipStream_t s, bool gemm_order) {
  const int64_t nchunks = rows * (cols / 32) * 4;
  if (nchunks <= 0) return hipSuccess;
  const int64_t grid = (nchunks + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (gemm_order && (rows % 32 || cols % 256)) return hipErrorInvalidValue;
  if (gemm_order)
    hipLaunchKernelGGL(mxfp6_quant_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, x, nchunks, cols / 32, codes,
                       scales);
  else
    hipLaunchKernelGGL(mxfp6_quant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, x, nchunks, cols / 32, codes,
                       scales);
  return hipGetLastError();
}

hipError_t mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                          hipStream_t s, bool gemm_order) {
  const int64_t nchunks = rows * (cols / 32) * 4;
  if (nchunks <= 0) return hipSuccess;
  const int64_t grid = (nchunks + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (gemm_order && (rows % 32 || cols % 256)) return hipErrorInvalidValue;
  if (gemm_order)
    hipLaunchKernelGGL(mxfp4_quant_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, x, nchunks, cols / 32, codes,
                       scales);
  else
    hipLaunchKernelGGL(mxfp4_quant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, x, nchunks, cols / 32, codes,
                       scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM
// The MXFP4 products, and the MXFP6 ones on GEMM-order operands, run on the
// bf16 GEMM's pipeline (gemm.hip).  Here: the MXFP6 GEMM on plain-order
// operands, C [M, N] (bf16, row stride ldc) = A B^T, A [M, K] and B [N, K]
// (codes K*3/4 bytes per row, scales K/32 bytes per row).  128 x 128 tiles, 4
// waves of 64 x 64 (2 x 2 MFMA blocks of 32 x 32); K slabs of 128 elements (96
// code bytes and 4 scale bytes per row, 58 KB of LDS for both buffers, two
// workgroups per CU) through two LDS buffers, the next slab loaded into
// registers while the current one is multiplied; a lane's fragment is 24 bytes
// (32 elements of 6 bits), read as three 8-byte words.  LDS rows are padded to
// 112 bytes: the 16 rows a half-wave reads then start 28 banks apart (mod 64),
// on 16 distinct pairs of banks.  M, N % 128 == 0, K % 128 == 0.
namespace {
constexpr int MT = 128;
constexpr int KS6 = 128, ROWB6 = KS6 * 6 / 8;  // 96 code bytes per row and slab
constexpr int LROW6 = ROWB6 + 16;               // LDS row stride
constexpr int TILEB6 = MT * LROW6;              // 14 KB per operand and slab
constexpr int SCB6 = MT * (KS6 / 32);           // 512 B of scales per operand and slab
constexpr int BUF6 = 2 * TILEB6 + 2 * SCB6;
}  // namespace

__global__ __launch_bounds__(256, 2) void mxfp6_gemm_kernel(Mxfp4GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char lds_[2 * BUF6];
  const int ntn = g.N / MT;
  const int ntiles = (g.M / MT) * ntn;
  const int u = xcd_index(blockIdx.x, ntiles);
  const int tm = u / ntn, tn = u % ntn;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t kb = (int64_t)g.K * 6 / 8, ks = g.K / 32;
  const uint8_t* a0 = g.a + (int64_t)tm * MT * kb;
  const uint8_t* b0 = g.b + (int64_t)tn * MT * kb;
  const uint8_t* sa0 = g.sa + (int64_t)tm * MT * ks;
  const uint8_t* sb0 = g.sb + (int64_t)tn * MT * ks;
  const int nslab = g.K / KS6;

  // 128 rows x 6 chunks of 16 bytes per operand: 3 per thread; 4 scale bytes of
  // one row of A (threads 0..127) or B (128..255)
  u32x4 ra[3], rb[3];
  uint32_t rsc;
  auto load = [&](int s) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int idx = t + 256 * i, r = idx / 6, c = idx % 6;
      ra[i] = *reinterpret_cast<const u32x4*>(a0 + r * kb + s * ROWB6 + c * 16);
      rb[i] = *reinterpret_cast<const u32x4*>(b0 + r * kb + s * ROWB6 + c * 16);
    }
    rsc = *reinterpret_cast<const uint32_t*>((t < 128 ? sa0 : sb0) + (t & 127) * ks + s * 4);
  };
  auto store = [&](char* buf) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int idx = t + 256 * i, off = (idx / 6) * LROW6 + (idx % 6) * 16;
      *reinterpret_cast<u32x4*>(buf + off) = ra[i];
      *reinterpret_cast<u32x4*>(buf + TILEB6 + off) = rb[i];
    }
    *reinterpret_cast<uint32_t*>(buf + 2 * TILEB6 + (t < 128 ? 0 : SCB6) + (t & 127) * 4) = rsc;
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  typedef int i32x8 __attribute__((ext_vector_type(8)));
  load(0);
  store(lds_);
  __syncthreads();
  for (int s = 0; s < nslab; ++s) {
    const bool more = s + 1 < nslab;
    if (more) load(s + 1);
    const char* buf = lds_ + (s & 1) * BUF6;
#pragma unroll
    for (int kk = 0; kk < KS6 / 64; ++kk) {
      const int blk = kk * 2 + (lane >> 5);  // this lane's 32-element block of the slab
      i32x8 fa[2], fb[2];
      int sca[2], scb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        const u32x2* p = reinterpret_cast<const u32x2*>(buf + r * LROW6 + blk * 24);
        const u32x2 x0 = p[0], x1 = p[1], x2 = p[2];
        fa[i] = i32x8{(int)x0[0], (int)x0[1], (int)x1[0], (int)x1[1], (int)x2[0], (int)x2[1], 0, 0};
        sca[i] = (int)(uint8_t)buf[2 * TILEB6 + r * 4 + blk];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + (lane & 31);
        const u32x2* p = reinterpret_cast<const u32x2*>(buf + TILEB6 + r * LROW6 + blk * 24);
        const u32x2 x0 = p[0], x1 = p[1], x2 = p[2];
        fb[j] = i32x8{(int)x0[0], (int)x0[1], (int)x1[0], (int)x1[1], (int)x2[0], (int)x2[1], 0, 0};
        scb[j] = (int)(uint8_t)buf[2 * TILEB6 + SCB6 + r * 4 + blk];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)  // format 2: FP6 E2M3
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 2, 2, 0, scb[j], 0,
                                                                      sca[i]);
    }
    if (more) store(lds_ + ((s + 1) & 1) * BUF6);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = (int64_t)tm * MT + wm * 64 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = tn * MT + wn * 64 + j * 32 + 8 * q + 4 * (lane >> 5);
        *reinterpret_cast<u32x2*>(g.c + m * g.ldc + n) =
            u32x2{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                  pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
      }
  }
}

hipError_t mxfp6_gemm(const Mxfp4GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  if (g.M % MT || g.N % MT || g.K % KS6) return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)(g.M / MT) * (g.N / MT);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mxfp6_gemm_kernel, dim3((unsigned)tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <bool GO>
static void launch_quant_tiles(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                               uint8_t* codes_t, uint8_t* scales_t, hipStream_t s) {
  const dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 64));
  if (codes && codes_t)
    hipLaunchKernelGGL((mxfp4_quant_tile_kernel<true, true, GO>), grid, dim3(256), 0, s, x, rows, cols, codes, scales,
                       codes_t, scales_t);
  else if (codes_t)
    hipLaunchKernelGGL((mxfp4_quant_tile_kernel<false, true, GO>), grid, dim3(256), 0, s, x, rows, cols, codes,
                       scales, codes_t, scales_t);
  else
    hipLaunchKernelGGL((mxfp4_quant_tile_kernel<true, false, GO>), grid, dim3(256), 0, s, x, rows, cols, codes,
                       scales, codes_t, scales_t);
}

hipError_t mxfp4_quantize_both(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                               uint8_t* codes_t, uint8_t* scales_t, hipStream_t s, bool gemm_order) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (rows % 64 || cols % 128 || rows / 64 > 65535 || cols / 128 > INT32_MAX) return hipErrorInvalidValue;
  // GEMM order: K % 256 for each written direction (cols for the row-wise
  // scales, rows for the column-wise ones)
  if (gemm_order && ((codes && cols % 256) || (codes_t && rows % 256))) return hipErrorInvalidValue;
  if (gemm_order) launch_quant_tiles<true>(x, rows, cols, codes, scales, codes_t, scales_t, s);
  else launch_quant_tiles<false>(x, rows, cols, codes, scales, codes_t, scales_t, s);
  return hipGetLastError();
}

hipError_t mxfp4_quantize_t(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                            hipStream_t s, bool gemm_order) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (rows % 32) return hipErrorInvalidValue;
  if (gemm_order && (rows % 256 || cols % 32)) return hipErrorInvalidValue;
  if (rows % 64 == 0 && cols % 128 == 0 && rows / 64 <= 65535)  // whole 64 x 128 tiles
    return mxfp4_quantize_both(x, rows, cols, nullptr, nullptr, codes, scales, s, gemm_order);
  const int64_t gx = (cols + 63) / 64, gy = (rows / 32 + 3) / 4;
  if (gx > INT32_MAX || gy > 65535) return hipErrorInvalidValue;
  if (gemm_order)
    hipLaunchKernelGGL(mxfp4_quant_t_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, rows, cols,
                       codes, scales);
  else
    hipLaunchKernelGGL(mxfp4_quant_t_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, rows, cols,
                       codes, scales);
  return hipGetLastError();
}

}  // namespace mtl
