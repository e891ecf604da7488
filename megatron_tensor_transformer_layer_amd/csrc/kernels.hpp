// Host-side launch interface of the gfx950 kernels (internal to libmtl.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct mtl_layer_cfg;  // include/mtl.h

namespace mtl {

// ---------------------------------------------------------------- GEMM
enum GemmEpi : int {
  EPI_BF16 = 0,       // C = acc                      (bf16)
  EPI_BF16_BIAS = 1,  // C = acc + bias[n]            (bf16)
  EPI_BIAS_GELU = 2,  // z = acc + bias[n]; C = GeLU'(z), C2 = GeLU(z) (both bf16); bias may be null
  EPI_DGELU = 3,      // C = acc * aux[m][n], aux = GeLU'(z) as EPI_BIAS_GELU wrote it (bf16)
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
  const uint16_t* aux;   // GeLU'(z) (EPI_DGELU)
  int64_t ld_aux;
  // Grouped (MoE experts): group e owns rows [offsets[e], offsets[e+1]).
  //  GROUP_M: those rows of A, C (and C2, aux) form expert e's M; B advances by
  //           stride_b elements per group; N and K are fixed.
  //  GROUP_K: those rows of A and B form expert e's K (A and B mn-contiguous);
  //           C advances by stride_c elements per group; M and N are fixed.
  const int32_t* offsets;  // nullptr = one plain GEMM
  int groups;
  int group_mode;
  int64_t stride_b, stride_c;
  // fp8 operands (gemm_fp8): each operand's dequantisation factor 1/s (device scalars)
  const float* scale_a;
  const float* scale_b;
  // Optional, plain (ungrouped) GEMMs with a bf16 output: every wave writes the
  // largest bf16 magnitude bit pattern (sign cleared) it stored of output
  // amax_out (0: c, 1: c2) to amax_part[tile * waves + wave] -- the stage-1
  // partials of that tensor's per-tensor amax.  The launcher sets *amax_nparts
  // (a host int) to the number of entries written and refuses more than
  // amax_cap.
  uint32_t* amax_part;
  int amax_out;
  int amax_cap;
  int* amax_nparts;
  // MXFP4 operands (gemm_mxfp4_tiled): E8M0 scales of A [M, K/16] and B [N, K/16]
  // bytes, K counting code bytes
  const uint8_t* mx_sa;
  const uint8_t* mx_sb;
  // Split contraction (plain bf16 GEMMs with an fp32 epilogue, gemm_bf16_pair_ksplit):
  // ksplit > 1 runs every tile as ksplit workgroups, part j taking k in
  // [j*k_chunk, min(K, (j+1)*k_chunk)) and writing its own fp32 C at
  // c + j*split_stride_c elements.  0 or 1: no split.
  int ksplit;
  int k_chunk;
  int64_t split_stride_c;
  // 1: plain stores, the output stays in the caches for the kernel that reads
  // it next; 0: nontemporal stores (the output streams to memory)
  int keep_cached;
};

enum GemmGroupMode : int { GROUP_M = 0, GROUP_K = 1 };

// Workgroups needed by a GROUP_M launch with at most max_rows grouped rows.
int64_t gemm_group_m_grid(int64_t max_rows, int groups, int N);

// Requirements (checked by the caller): K % 8 == 0 when an operand is
// k-contiguous, M % 8 == 0 when A is mn-contiguous, N % 8 == 0 always,
// 16-byte aligned base pointers and leading dimensions multiple of 8.
hipError_t gemm_bf16(const GemmArgs& p, GemmLayout layout, int epi, hipStream_t s);

// Two independent GEMMs, launched as one kernel where a fused configuration
// exists (the backward's dgrad/wgrad pairs), else as two launches.  Same
// requirements as gemm_bf16 for each.
hipError_t gemm_bf16_pair(const GemmArgs& p1, GemmLayout l1, int e1, const GemmArgs& p2, GemmLayout l2, int e2,
                          hipStream_t s);
// p1 wgrad (EPI_F32 / EPI_F32_ACC) beside p2, a dgrad in p2.ksplit fp32 parts (see GemmArgs::ksplit).
hipError_t gemm_bf16_pair_ksplit(const GemmArgs& p1, int e1, const GemmArgs& p2, hipStream_t s);

// fp8 GEMM: C = (A . B^T) * (*scale_a) * (*scale_b), fp32 accumulate, with the
// epilogues above.  A [M][K] and B [N][K] are fp8 codes (both k-contiguous; a, b
// point at bytes, lda/ldb in bytes), fmt_a/fmt_b 0 = E4M3, 1 = E5M2.  Supported:
// (E4M3, E4M3) with BF16 / BF16_BIAS / BIAS_GELU, (E5M2, E4M3) with BF16 / DGELU,
// (E4M3, E5M2) with F32 / F32_ACC.  K % 16 == 0, lda and ldb % 16 == 0, not grouped.
hipError_t gemm_fp8(const GemmArgs& p, int fmt_a, int fmt_b, int epi, hipStream_t s);
// A backward pair in one launch where a fused configuration exists: pw an
// E4M3 x E5M2 wgrad (EPI_F32 / EPI_F32_ACC), pd an E5M2 x E4M3 dgrad (EPI_BF16 /
// EPI_DGELU); else two launches.  Same requirements as gemm_fp8 for each.
hipError_t gemm_fp8_pair(const GemmArgs& pw, int epi_w, const GemmArgs& pd, int epi_d, hipStream_t s);

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
  // attention_fwd_full: keys and values of a separate chunk [kv_seq, ...], stride ld_qkv
  const uint16_t* kv;
  int kv_seq;
  // attention_bwd_full: dK, dV into the key columns of dkv (kv's layout), dQ into dq (stride ld_o)
  uint16_t* dkv;
  uint16_t* dq;
  // Optional (attention_fwd: O; attention_bwd: dQKV): every wave writes the
  // largest bf16 magnitude bit pattern it stored to amax_part[workgroup *
  // waves + wave], the stage-1 partials of that tensor's per-tensor amax; the
  // launcher sets *amax_nparts (a host int) to the count and refuses more than
  // amax_cap.
  uint32_t* amax_part;
  int amax_cap;
  int* amax_nparts;
  // attention_bwd: when dout_parts is set, dO arrives as two fp32 parts (dO's
  // layout, the second dout_part_stride floats after the first); the D pass
  // sums them (part 0 + part 1), rounds the sum to bf16 into dout_w and forms D
  // from that, and the backward reads dout (= dout_w).
  const float* dout_parts;
  int64_t dout_part_stride;
  uint16_t* dout_w;
};
hipError_t attention_fwd(const AttnArgs& a, hipStream_t s);
// Queries of a.qkv against all a.kv_seq keys of a.kv (no mask; kv_seq % 64 == 0).
hipError_t attention_fwd_full(const AttnArgs& a, hipStream_t s);
// Log-sum-exp merge of nparts partial attention results (O_j [tokens, heads*d]
// bf16 at o_parts + j*o_stride, L_j [heads, tokens] fp32 at lse_parts +
// j*lse_stride) into o and lse, summed in ascending j.
struct CpMergeArgs {
  const uint16_t* o_parts;
  const float* lse_parts;
  int64_t o_stride, lse_stride;
  int nparts;
  int64_t tokens;
  int heads, d;
  uint16_t* o;
  float* lse;
};
hipError_t cp_merge(const CpMergeArgs& a, hipStream_t s);
// dqkv[tok, n*3d + i] += sum_j parts[j][tok, n*d + i] (the query columns of a
// head-interleaved [tokens, 3*heads*d] tensor), fp32 in ascending j, bf16 out.
struct CpDqSumArgs {
  uint16_t* dqkv;
  const uint16_t* parts;
  int64_t part_stride;
  int nparts;
  int64_t tokens;
  int heads, d;
};
hipError_t cp_dq_sum(const CpDqSumArgs& a, hipStream_t s);

// ---------------------------------------------------------------- MXFP4
// Scale matrices come in two orders.  Plain: [rows, K/32], block q of row r at
// r * K/32 + q.  GEMM order (rows % 32 == 0, K % 256 == 0): the 8 scale bytes
// of the rows of one 32-row block rb in one 256-k slab s fill the 256-byte
// group rb * K/256 + s, block q (0..7 within the slab) of row r at byte
// 4 * (r % 32 + 32 * (q % 2)) + q / 2 of it -- lane l of a 32x32x64 MFMA
// fragment (row l % 32, k half l / 32) reads its four k steps' scales as the
// one word at 4 * l.
template <bool GEMM_ORDER>
__host__ __device__ __forceinline__ int64_t mx_scale_index(int64_t r, int64_t q, int64_t nblocks) {
  if constexpr (!GEMM_ORDER) return r * nblocks + q;
  return ((r >> 5) * (nblocks >> 3) + (q >> 3)) * 256 + ((r & 31) + 32 * (q & 1)) * 4 + ((q & 7) >> 1);
}
// x [rows, cols] bf16 (cols % 32 == 0) -> codes [rows, cols/2] (two E2M1 per
// byte, even element low) and E8M0 scales, plain or (gemm_order: rows % 32 ==
// 0, cols % 256 == 0) in GEMM order.
hipError_t mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                          hipStream_t s, bool gemm_order = false);
// c [M, N] bf16 (row stride ldc) = A B^T over K, A [M, K] and B [N, K] in
// MXFP4 or MXFP6 (codes and scales as the quantisers write them).
struct Mxfp4GemmArgs {
  const uint8_t* a;
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  uint16_t* c;
  int64_t ldc;
  int M, N, K;
  // MXFP4 epilogues (MXFP6 is EPI_BF16 only), as the bf16 GEMM's:
  int epi;               // EPI_* (0: bf16 C)
  const uint16_t* bias;  // [N] (EPI_BF16_BIAS, EPI_BIAS_GELU)
  uint16_t* c2;          // GeLU(z) [M, N], row stride ldc (EPI_BIAS_GELU)
  const uint16_t* aux;   // GeLU'(z) [M, N], row stride ldc (EPI_DGELU)
  float* c32;            // fp32 C [M, N], row stride ldc (EPI_F32, EPI_F32_ACC)
  int scale_order;       // gemm_mxfp4_tiled: 0 plain (EPI_BF16 only), 1 GEMM order (M, N % 32 == 0)
  int keep_cached;       // as GemmArgs::keep_cached
};
// MXFP4 on the bf16 GEMM's pipeline (256 x 256, 256 x 192 or 128 x 128 tiles,
// two slabs in flight), for K % 256 == 0.
hipError_t gemm_mxfp4_tiled(const Mxfp4GemmArgs& g, hipStream_t s);
// A weight gradient gw (EPI_F32 / EPI_F32_ACC) and a data gradient gd (EPI_BF16 /
// EPI_DGELU) on MXFP4 operands in GEMM order: one launch on 256 x 256 tiles
// when both fill the chip, else gd then gw.
hipError_t gemm_mxfp4_pair(const Mxfp4GemmArgs& gw, const Mxfp4GemmArgs& gd, hipStream_t s);
// MXFP4 quantisation of x [rows, cols] down its columns (blocks of 32 rows of
// one column): codes of x^T, [cols, rows/2] bytes, and the scales of x^T,
// plain [cols, rows/32] or in GEMM order (rows % 256 == 0, cols % 32 == 0)
// (rows % 32 == 0, cols % 8 == 0).
hipError_t mxfp4_quantize_t(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                            hipStream_t s, bool gemm_order = false);
// Both directions at once from one read of x (rows % 64 == 0, cols % 128 ==
// 0): codes/scales as mxfp4_quantize, codes_t/scales_t as mxfp4_quantize_t;
// either pair may be null (not both).  gemm_order: both scale matrices in GEMM
// order (rows and cols % 256 == 0).
hipError_t mxfp4_quantize_both(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                               uint8_t* codes_t, uint8_t* scales_t, hipStream_t s, bool gemm_order = false);
// The same for MXFP6 (FP6 E2M3 elements): codes [rows, cols*3/4], 32 elements
// of 6 bits per 24 bytes, element j at bits 6j.. of the little-endian block;
// the GEMM takes K % 128 == 0.
hipError_t mxfp6_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                          hipStream_t s, bool gemm_order = false);
// Byte offset, within its row's codes, of byte o (0..23) of block q of row r
// in MXFP6 GEMM code order.
__host__ __device__ __forceinline__ int64_t mx6_code_offset(int64_t r, int64_t q, int o) {
  const int64_t slab = (q >> 2) * 96;
  const int b = (int)(q & 3);
  if (o < 16) return slab + b * 16 + o;
  return slab + 64 + (b >> 1) * 16 + (((b & 1) ^ ((r >> 4) & 1)) * 8) + (o - 16);
}
hipError_t mxfp6_gemm(const Mxfp4GemmArgs& g, hipStream_t s);
// MXFP6 codes in GEMM order (mxfp6_quantize with gemm_order): per row, each
// slab of 128 k (4 blocks, 96 bytes) holds the blocks' first 16 bytes in
// chunks 0..3 and their last 8 bytes in chunk 4 (blocks 0, 1) and chunk 5
// (blocks 2, 3), the two halves of each of those chunks swapped in rows with
// (row / 16) odd.  Scales in GEMM order.
hipError_t gemm_mxfp6_tiled(const Mxfp4GemmArgs& g, hipStream_t s);
hipError_t attention_bwd(const AttnArgs& a, hipStream_t s);
// The backward of attention_fwd_full for queries whose D = rowsum(dO * O) is
// already in a.delta (kv_seq == seq, seq % 64 == 0): no D launch.
hipError_t attention_bwd_full(const AttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------- reductions
// out[r, :] = sum_i partials[i][r, :] (+ bias) (+ residual) for r in [row_begin, row_end).
hipError_t reduce_partials(int t, const uint16_t* const* partials, const uint16_t* bias, const uint16_t* residual,
                           uint16_t* out, int64_t cols, int64_t row_begin, int64_t row_end, hipStream_t s);
// Sequence-parallel all-gather stand-in: copies rows [i*rows/t, (i+1)*rows/t)
// of bufs[i] into out for every i != rank (rows % t == 0, cols % 8 == 0).
hipError_t allgather_rows(int t, int rank, const uint16_t* const* bufs, uint16_t* out, int64_t rows, int64_t cols,
                          hipStream_t s);
// For one or two jobs j: out_j[c] (=|+=) sum_r x_j[r][c] over [rows, cols_j]
// row-major bf16, fp32, deterministic, two launches for all jobs together;
// ws holds colsum_ws_floats(rows, cols_0 + cols_1) floats.
struct ColsumJob {
  const uint16_t* x;
  int64_t cols;
  float* out;
};
size_t colsum_ws_floats(int64_t rows, int64_t cols);
hipError_t colsum_bf16(const ColsumJob* jobs, int njobs, int64_t rows, bool accumulate, float* ws, hipStream_t s);

// ---------------------------------------------------------------- fp8 scaling
// rec[0..2] = {amax, s, 1/s} of n bf16 values for format fmt (0 = E4M3, 1 = E5M2);
// ws holds fp8_amax_ws_bytes().
size_t fp8_amax_ws_bytes();
hipError_t fp8_amax(const uint16_t* x, int64_t n, int fmt, float* rec, void* ws, hipStream_t s);
// codes of x [rows, cols] (bf16) scaled by rec[1]: out [rows, cols] and/or
// out_t [cols, rows] (either may be null).  cols % 8 == 0; rows % 16 == 0 when
// out_t is given; 16-byte aligned pointers.
hipError_t fp8_cast(const uint16_t* x, int64_t rows, int64_t cols, int fmt, const float* rec, uint8_t* out,
                    uint8_t* out_t, hipStream_t s);
// fp8_amax then fp8_cast (rec written too) of 1..3 tensors in two launches:
// stage 1 of every amax, then every cast, each cast block finishing its
// tensor's amax from the stage-1 partials.  Each tensor's record and codes are
// those of fp8_amax + fp8_cast on it alone.  ws holds fp8_amax_ws_bytes().
// Same shape rules as fp8_cast.
struct QuantJob {
  const uint16_t* x;
  int64_t rows, cols;
  int fmt;
  float* rec;
  uint8_t* out;
  uint8_t* out_t;
  // the amax stage-1 partials of x written by the kernel that produced it
  // (nullptr: the quantisation computes them)
  const uint32_t* part;
  int nparts;
};
hipError_t fp8_quantize_n(const QuantJob* jobs, int n, void* ws, hipStream_t s);

// ---------------------------------------------------------------- MoE data movement
// Top-k expert ids per token (descending logit, ties to the lower id) and the
// softmax of the selected logits.  E <= 1024, k <= min(E, 64).
hipError_t moe_route(const float* logits, int T, int E, int k, int32_t* idx, float* gates, hipStream_t s);
// Router backward: counts [E] (assignments per expert), q [T] scratch,
// aux_loss (1 float, NULL: not computed), dlogits [T, E] fp32 and its bf16
// rounding dlogits_bf16 (the operand of the router's dgrad and wgrad GEMMs).
hipError_t moe_router_bwd(const float* logits, const int32_t* idx, const float* gates, const float* dgates, int T,
                          int E, int k, float alpha, int32_t* counts, float* q, float* aux_loss, float* dlogits,
                          uint16_t* dlogits_bf16, hipStream_t s);
// Stable grouping of the (token, slot) entries whose expert lies in
// [e_lo, e_lo + E_l): counts[E_l], offsets[E_l + 1], ptok/pslot[N] and the
// inverse slot_row[T*k] (row of the entry, or -1 when its expert is not local).
hipError_t moe_permute(const int32_t* idx, int T, int k, int e_lo, int E_l, int32_t* counts, int32_t* offsets,
                       int32_t* ptok, int32_t* pslot, int32_t* slot_row, hipStream_t s);
// xp[i] = x[ptok[i]] for i < offsets[E_l] (max_rows bounds the grid).
hipError_t moe_gather(const uint16_t* x, const int32_t* ptok, const int32_t* offsets, int E_l, int64_t max_rows,
                      int64_t h, uint16_t* xp, hipStream_t s);
// out[t] = sum_{s ascending, slot_row[t,s] >= 0} (gates ? gates[t,s] : 1) * rows[slot_row[t,s]].
hipError_t moe_combine(const uint16_t* rows, const int32_t* slot_row, const float* gates, int T, int k, int64_t h,
                       uint16_t* out, hipStream_t s);
// dye[i] = gates[t,s] * dy[t]; dgates[t,s] = <ye[i], dy[t]> (0 for non-local slots).
hipError_t moe_combine_bwd(const uint16_t* dy, const uint16_t* ye, const int32_t* ptok, const int32_t* pslot,
                           const int32_t* slot_row, const int32_t* offsets, int E_l, int64_t max_rows,
                           const float* gates, int T, int k, int64_t h, uint16_t* dye, float* dgates, hipStream_t s);

// Scratch bytes mtl_mlp_bwd needs for a valid configuration (defined with the
// entry points; used by the entry point that allocates nothing).
size_t mlp_bwd_scratch_bytes(const ::mtl_layer_cfg* c);

}  // namespace mtl
