// Device-side building blocks shared by the gfx950 kernels: vector types,
// bf16 packing, the MFMA wrappers, the attention tiles' LDS swizzle, the normal
// CDF/density behind GeLU, transpose reads from LDS and the LDS DMA load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 converts two
// values per instruction (NaN stays NaN).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32].
// Operand a: lane l supplies row (l % 32) with 8 k-values; operand b: lane l
// supplies column (l % 32) with 8 k-values.  The k-slot -> k mapping only has to
// agree between a and b.  Result: lane l, register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l % 32].
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// v_mfma_f32_32x32x64_f8f6f4 with OCP fp8 operands: D[32x32] += A[32x64] * B[64x32].
// Each operand is 32 bytes per lane (lane l: row or column l % 32, 32 k-values);
// FA / FB select the format of a / b (0 = E4M3, 1 = E5M2).  Same result layout
// as mfma32.  Scale operands 0 select the unscaled instruction.
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma32_f8(const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1,
                                            const f32x16& c) {
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const i32x8_t a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8_t b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// MXFP4 x MXFP4 32x32x64 MFMA: a and b hold 32 E2M1 codes per lane (one
// 16-byte chunk; the instruction reads four registers for this format), sa and
// sb four E8M0 scale bytes of which byte kk applies.
__device__ __forceinline__ f32x16 mfma32_mxfp4(const u32x4& a, const u32x4& b, const f32x16& c, uint32_t sa,
                                               uint32_t sb, int kk) {
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const i32x4_t a4 = __builtin_bit_cast(i32x4_t, a), b4 = __builtin_bit_cast(i32x4_t, b);
  const i32x8_t va = __builtin_shufflevector(a4, a4, 0, 1, 2, 3, -1, -1, -1, -1);
  const i32x8_t vb = __builtin_shufflevector(b4, b4, 0, 1, 2, 3, -1, -1, -1, -1);
  switch (kk & 3) {  // op_sel must be a constant: kk is one after unrolling
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, c, 4, 4, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, c, 4, 4, 1, (int)sa, 1, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, c, 4, 4, 2, (int)sa, 2, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, c, 4, 4, 3, (int)sa, 3, (int)sb);
  }
}

// MXFP6 (E2M3) operand of one lane: 24 bytes (32 codes of 6 bits) from a
// 16-byte head and an 8-byte tail; the instruction reads six registers for
// this format, the last two stay undefined.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x8 mx6_operand(const u32x4& head, const u32x2& tail) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  const i32x4_t h = __builtin_bit_cast(i32x4_t, head);
  const i32x2_t t2 = __builtin_bit_cast(i32x2_t, tail);
  const i32x4_t t = __builtin_shufflevector(t2, t2, 0, 1, -1, -1);
  return __builtin_shufflevector(h, t, 0, 1, 2, 3, 4, 5, -1, -1);
}
// MXFP6 x MXFP6 32x32x64 MFMA; scales as mfma32_mxfp4.
__device__ __forceinline__ f32x16 mfma32_mxfp6(const i32x8& a, const i32x8& b, const f32x16& c, uint32_t sa,
                                               uint32_t sb, int kk) {
  switch (kk & 3) {  // op_sel must be a constant: kk is one after unrolling
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 1, (int)sa, 1, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 2, (int)sa, 2, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 3, (int)sa, 3, (int)sb);
  }
}

// ---------------------------------------------------------------- LDS tiles
// A k-contiguous tile of R rows x 64 bf16 (128 B per row) is stored as eight
// 16-byte chunks per row, chunk c of row r at physical chunk c ^ (r & 7): eight
// consecutive rows reading the same logical chunk hit eight distinct bank groups.
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ (row & 7u)) << 4);
}

// ---------------------------------------------------------------- GeLU
// Exact-form GeLU z * Phi(z) and its derivative Phi(z) + z * phi(z).  The normal
// CDF uses the rational approximation of erfc in Abramowitz & Stegun (1964),
// formula 7.1.26 (|error of erf| <= 1.5e-7): erfc(x) = poly(t) * exp(-x^2),
// t = 1 / (1 + p x), x >= 0.  With x = |z| / sqrt(2), exp(-x^2) = exp(-z^2 / 2)
// is also the unnormalised normal density, so one exp serves both Phi and phi.
__device__ __forceinline__ void normal_cdf_pdf(float z, float& cdf, float& pdf) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * x);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = __expf(-x * x);
  const float half_erfc = 0.5f * poly * e;
  cdf = z >= 0.f ? 1.0f - half_erfc : half_erfc;
  pdf = 0.39894228040143268f * e;
}

// ---------------------------------------------------------------- LDS DMA
#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lanes 4R..4R+3 each name 8
// bytes (4 bf16) of row R of a 4 x 16 block; lane i receives column i, i.e. the
// four row-R elements of its column.
__device__ __forceinline__ u32x2 read_tr(const LDS_AS char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p));
}

// A raw buffer resource over [base, base + bytes): loads past the end return 0
// (the range check covers the VGPR offset only, not soffset).
// The words are made wave-uniform explicitly: the DMA takes the resource in SGPRs.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b), __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16*lane
// (buffer_load_dwordx4 ... lds; the LDS base travels in M0).  Issued as inline
// assembly so that the compiler does not fence every later LDS read on it: the
// caller waits (vmcnt) before the barrier that publishes the data.  M0 is saved
// and restored; s_nop covers the M0 -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait for this wave's compiler-visible vector loads with the s_waitcnt builtin
// (vmcnt 0, expcnt and lgkmcnt untouched), which the compiler's own wait
// tracking sees: loads completed here are not waited for again later, e.g. at
// the top of a loop whose body also issues LDS DMA, where a compiler-inserted
// vmcnt(0) would wait for that DMA too.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8); map w to a logical work index so that each XCD takes a
// contiguous run of the n work units, which then share that XCD's L2.
__device__ __forceinline__ int xcd_index(int w, int n) {
  if ((n & 7) == 0) return (w & 7) * (n >> 3) + (w >> 3);
  return w;
}
__device__ __forceinline__ uint32_t lds_addr(const LDS_AS void* p) { return (uint32_t)(uintptr_t)p; }

}  // namespace mtl
