// Host-side launch interface of the gfx950 kernels (internal to libmtl.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtl {

// ---------------------------------------------------------------- GEMM
enum GemmEpi : int {
  EPI_BF16 = 0,       // C = acc                      (bf16)
  EPI_BF16_BIAS = 1,  // C = acc + bias[n]            (bf16)
  EPI_BIAS_GELU = 2,  // C = acc + bias[n]; C2 = GeLU(C) (both bf16)
  EPI_DGELU = 3,      // C = acc * GeLU'(aux[m][n])   (bf16, aux bf16)
  EPI_F32 = 4,        // C = acc                      (fp32)
  EPI_F32_ACC = 5,    // C += acc                     (fp32)
};

enum GemmLayout : int {
  GEMM_FWD = 0,    // A[m][k] (lda), B[k][n] (ldb)
  GEMM_DGRAD = 1,  // A[m][k] (lda), B[n][k] (ldb)
  GEMM_WGRAD = 2,  // A[k][m] (lda), B[k][n] (ldb)
};

struct GemmArgs {
  const uint16_t* a;
  const uint16_t* b;
  int64_t lda, ldb;
  int M, N, K;
  void* c;
  int64_t ldc;
  const uint16_t* bias;  // [N] bf16 (EPI_BF16_BIAS, EPI_BIAS_GELU)
  void* c2;              // second output (EPI_BIAS_GELU)
  int64_t ldc2;
  const uint16_t* aux;   // GeLU input Z (EPI_DGELU)
  int64_t ld_aux;
};

// Requirements (checked by the caller): K % 8 == 0 when an operand is
// k-contiguous, M % 8 == 0 when A is mn-contiguous, N % 8 == 0 always,
// 16-byte aligned base pointers and leading dimensions multiple of 8.
hipError_t gemm_bf16(const GemmArgs& p, GemmLayout layout, int epi, hipStream_t s);

// ---------------------------------------------------------------- attention
// Causal attention over `heads` heads of a head-interleaved QKV tensor
// [tokens, 3*heads*d] (row stride ld_qkv), rows ordered [batch][seq].
struct AttnArgs {
  const uint16_t* qkv;
  int64_t ld_qkv;
  uint16_t* o;  // [tokens, heads*d], row stride ld_o
  int64_t ld_o;
  float* lse;   // [heads, tokens]
  int seq, batch, heads, d;
  float scale;
  // backward
  const uint16_t* dout;  // dO [tokens, heads*d], stride ld_o
  const uint16_t* out;   // O (forward output), stride ld_o
  const float* lse_in;
  float* delta;          // D = rowsum(dO * O), [heads, tokens]
  uint16_t* dqkv;        // [tokens, 3*heads*d], stride ld_qkv
};
hipError_t attention_fwd(const AttnArgs& a, hipStream_t s);
hipError_t attention_bwd(const AttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------- reductions
// out[r, :] = sum_i partials[i][r, :] (+ bias) (+ residual) for r in [row_begin, row_end).
hipError_t reduce_partials(int t, const uint16_t* const* partials, const uint16_t* bias, const uint16_t* residual,
                           uint16_t* out, int64_t cols, int64_t row_begin, int64_t row_end, hipStream_t s);
// out[c] (=|+=) sum_r x[r][c], fp32; deterministic two-stage; ws holds
// colsum_ws_floats(rows, cols) floats.
size_t colsum_ws_floats(int64_t rows, int64_t cols);
hipError_t colsum_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* out, bool accumulate,
                       float* ws, hipStream_t s);

}  // namespace mtl
