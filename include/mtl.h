/*
 * mtl.h -- C ABI of libmtl.so: one tensor-parallel rank's share of a
 * transformer layer's training step (forward, dgrad, wgrad) on an AMD MI355X
 * (gfx950), plus the expert-parallel MoE expert block.
 *
 * What is computed.  The layer is the one the Megatron tutorial
 * (cf-1.com/news/5344657, section 2.2, "tensor parallelism") splits across t
 * cards: the fused QKV projection is split by output columns -- whole attention
 * heads, heads/t per rank (section 4.2: 12 heads on TP 2 gives 6 per card) --
 * self-attention runs over the rank's heads, the output projection is split by
 * rows, the first MLP linear by columns and the second by rows, so each
 * row-parallel linear yields a partial sum that an all-reduce adds across the t
 * ranks.  On one device the t partials are added by mtl_reduce.  Attention is
 * causal scaled dot-product attention (scale 1/sqrt(d), d = hidden/heads); the
 * MLP activation is the exact (erf) GeLU; every linear has a bias; the
 * row-parallel biases are added once, after the sum.  Sizes must divide as the
 * tutorial's section 2.2 and the guide's integer-check section
 * (ai.lansai.wang/82226) require: hidden and heads by the TP degree.
 *
 * Conventions (all calls).
 *  - Every pointer argument is a device pointer unless stated; buffers are
 *    owned and allocated by the caller; the library never allocates, frees or
 *    synchronises.  Calls are asynchronous and ordered on `stream`
 *    (a hipStream_t; NULL = the null stream).
 *  - Tensors are dense row-major; bf16 tensors are 16-bit bfloat16 bit
 *    patterns; gradients of weights and biases are fp32.  S = seq*micro_batch
 *    token rows ordered [micro-batch][sequence]; h = hidden, f = ffn,
 *    d = h/heads, t = tp.
 *  - Weights are the rank-local shard stored [in, out]:
 *      w_qkv [h, 3h/t]  head-interleaved: column n*3d + j*d + i is local head n,
 *                       component j in (q, k, v), index i
 *      b_qkv [3h/t]     w_o [h/t, h]     w1 [h, f/t]   b1 [f/t]   w2 [f/t, h]
 *    b_o [h] and b2 [h] are whole (added by mtl_reduce, once).
 *  - Pointers must be 16-byte aligned.  Validation happens before any launch;
 *    on error nothing is launched and no output is touched.  A kernel fault
 *    surfaces at the caller's next synchronisation of `stream`.
 *  - Calls are stateless and reentrant; two calls may run concurrently on
 *    different streams only if they share no output or scratch buffer.
 */
#ifndef MTL_H
#define MTL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* mtl_stream_t; /* same type as hipStream_t */

typedef enum mtl_status {
  MTL_OK = 0,
  MTL_E_NULL = 1,         /* a required pointer is NULL */
  MTL_E_DIVISIBILITY = 2, /* hidden % heads, heads % tp or ffn % tp != 0 (MoE: experts % ep) */
  MTL_E_RANK = 3,         /* rank outside [0, tp) (MoE: [0, ep)) */
  MTL_E_SHAPE = 4,        /* a size <= 0, or outside what the kernels tile (see mtl_validate) */
  MTL_E_ALIGN = 5,        /* a pointer is not 16-byte aligned */
  MTL_E_WORKSPACE = 6,    /* scratch buffer smaller than mtl_workspace_bytes reports */
  MTL_E_UNSUPPORTED = 7,  /* unsupported precision / flag combination */
  MTL_E_HIP = 8           /* a HIP launch failed (no device, bad stream, ...) */
} mtl_status;

enum { MTL_PREC_BF16 = 0, MTL_PREC_FP8_HYBRID = 1, MTL_PREC_MXFP4 = 2 };
enum { MTL_FP8_E4M3 = 0, MTL_FP8_E5M2 = 1 };
#define MTL_FP8_AMAX_SCRATCH 4096 /* bytes of scratch mtl_fp8_amax needs */

enum {
  MTL_F_RESIDUAL = 1,   /* mtl_reduce callers add residuals; recorded for validation only */
  MTL_F_WGRAD_ACCUM = 2, /* weight/bias gradients are accumulated (+=) instead of written */
  /* fp8 or MXFP4: the forward calls also write the codes the backward calls
   * need of their operands into a region at the start of the scratch
   * (mtl_workspace_bytes counts it; each call's own scratch follows it), and
   * the backward calls read them there instead of quantising those tensors
   * again (bit-identical results: the same tensor and recipe give the same
   * codes).  fp8: the transposed E4M3 codes and scale records of x, o
   * (mtl_attn_fwd) and h, a (mtl_mlp_fwd), and the E4M3 codes of their weights
   * in both orientations (w_qkv, w_o; w1, w2).  MXFP4: the codes of x, o, h and
   * a blocked down their token columns and the weights' codes blocked both ways,
   * each tensor quantised both ways from one read.  The caller passes the same
   * scratch buffer to the rank's four calls of a step, leaves that region alone
   * between a forward call and its backward, and passes the backward the same
   * x, h and weights (and saved o, a) as the forward -- as a training step
   * does. */
  MTL_F_KEEP_CODES = 4,
  /* With MTL_F_KEEP_CODES: the forward calls do not quantise the weights; every
   * call takes the four weights' codes (and, in fp8, scale records) from the
   * kept region, where an earlier forward call with the same scratch (and
   * without this flag) wrote them.  For the micro-batches after the first of a
   * step with gradient accumulation, whose weights have not changed since: the
   * caller guarantees that (the bf16 weights passed are then not read by the
   * forward calls, nor by the backward calls, which read the kept codes). */
  MTL_F_REUSE_WEIGHTS = 8,
  /* the names of these two flags when only fp8 had them */
  MTL_F_FP8_KEEP_CODES = MTL_F_KEEP_CODES,
  MTL_F_FP8_REUSE_WEIGHTS = MTL_F_REUSE_WEIGHTS
};

/* Layer configuration: the pretraining flags --hidden-size, --num-attention-heads,
 * --ffn-hidden-size, --seq-length, --micro-batch-size,
 * --tensor-model-parallel-size and this process's TP rank (tutorial section 4.1;
 * site navi2ai.com/sites/1106, deploy steps 5 and 6). */
typedef struct mtl_layer_cfg {
  int32_t hidden, heads, ffn, seq, micro_batch, tp, rank;
  int32_t precision; /* MTL_PREC_* */
  int32_t flags;     /* MTL_F_* */
} mtl_layer_cfg;

/* Short text for a status code (static storage). */
const char* mtl_status_str(mtl_status s);

/* Host-only check of a layer configuration; makes no HIP call.  Rules: every
 * size > 0; hidden % heads == 0; heads % tp == 0 and ffn % tp == 0 (the
 * tutorial's section 2.2: 3 heads on TP 8 is an error; section 4.2: 768/12 on
 * TP 2 is legal); 0 <= rank < tp; d = hidden/heads in {64, 128} and
 * (ffn/tp) % 8 == 0 (MTL_E_SHAPE otherwise: the attention kernels are built for
 * those head sizes and the GEMMs move 16-byte vectors); tp <= 16; every GEMM
 * operand under 4 GiB: (max(S, w) + 256) * w * 2 < 2^32 bytes with
 * w = max(h, 3h/t, f/t).  precision MTL_PREC_BF16, MTL_PREC_FP8_HYBRID or
 * MTL_PREC_MXFP4; fp8 also needs S % 16 == 0 and (ffn/tp) % 16 == 0 (fp8 GEMMs
 * contract over 16-byte chunks of codes); MXFP4 needs S, h, h/t, 3h/t and f/t
 * all multiples of 256 (every GEMM dimension a multiple of the MX GEMM's
 * 128-row tiles, every contraction a multiple of its 256-deep K slabs). */
mtl_status mtl_validate(const mtl_layer_cfg* cfg);

/* Bytes of device scratch (*scratch_bytes) that suffice for every call of this
 * configuration.  In bf16 the forward calls need none (their scratch may be
 * NULL); in fp8 every call needs it for the operands' codes. */
mtl_status mtl_workspace_bytes(const mtl_layer_cfg* cfg, size_t* scratch_bytes);

/* Attention half of the rank's forward (column-parallel QKV, causal attention
 * over the rank's heads/t heads, row-parallel output projection):
 *   qkv     = x . w_qkv + b_qkv          [S, 3h/t] bf16 (saved for backward)
 *   o       = attention(qkv)             [S, h/t]  bf16 (saved)
 *   lse     = row log-sum-exp of scaled scores, [heads/t, S] fp32 (saved)
 *   partial = o . w_o                    [S, h]    bf16, this rank's partial sum
 * x [S, h] bf16.  scratch: see mtl_workspace_bytes (NULL allowed in bf16).
 *
 * fp8 (MTL_PREC_FP8_HYBRID, the site summary's --fp8-format hybrid): each GEMM
 * operand is quantised per tensor (mtl_fp8_amax + mtl_fp8_cast) -- E4M3 for
 * activations and weights, E5M2 for gradients -- the product accumulates in
 * fp32 and is multiplied by both operands' 1/s in the epilogue; outputs, bias,
 * GeLU, attention and the reductions stay bf16/fp32 as in the bf16 path.
 *
 * MXFP4 (MTL_PREC_MXFP4, the site summary's 4-bit training read as OCP MXFP4,
 * see mtl_mxfp4_quantize): every GEMM of the four linears, forward, dgrad and
 * wgrad, takes both operands quantised to MXFP4 with the 32-element blocks
 * along that GEMM's contraction (mtl_mxfp4_quantize for an operand whose K runs
 * along its rows, mtl_mxfp4_quantize_t for one whose K runs down its columns:
 * a weight in the forward, the activations and gradients in a weight
 * gradient) and multiplies them on the block-scaled MFMA with fp32
 * accumulation and the same epilogues (bias, GeLU, GeLU', fp32 wgrad) as the
 * bf16 path; attention, the bias gradients and the reductions stay bf16/fp32. */
mtl_status mtl_attn_fwd(const mtl_layer_cfg* cfg, const void* x, const void* w_qkv, const void* b_qkv,
                        const void* w_o, void* qkv, void* o, float* lse, void* partial, void* scratch,
                        size_t scratch_bytes, mtl_stream_t stream);

/* The all-reduce stand-in (tutorial section 2.2: the row-parallel outputs are
 * summed across the t ranks):
 *   out[r, :] = sum_{i<t} partials[i][r, :] (+ bias) (+ residual[r, :])
 * for rows r in [row_begin, row_end); other rows of `out` are not touched (a
 * rank's reduce-scatter share).  `partials` is a HOST array of t device
 * pointers to [rows, cols] bf16; bias [cols] bf16 or NULL; residual [rows, cols]
 * bf16 or NULL; out [rows, cols] bf16 (may alias residual, not a partial).
 * Sum in fp32 in rank order.  cols % 8 == 0, 1 <= t <= 16. */
mtl_status mtl_reduce(int32_t t, const void* const* partials, const void* bias, const void* residual, void* out,
                      int64_t rows, int64_t cols, int64_t row_begin, int64_t row_end, mtl_stream_t stream);

/* The sequence-parallel all-gather stand-in.  With sequence parallelism
 * (ai.lansai.wang/82226, the table of parallelism strategies: its EP row asks
 * for it whenever TP and EP are combined; the pages give no algorithm) the
 * all-reduce after a row-parallel linear becomes a reduce-scatter -- each rank
 * keeps the rows [rank*rows/t, (rank+1)*rows/t) of the sum, which is
 * mtl_reduce with that row range -- and the full tensor is gathered again
 * before the next column-parallel linear.  Each rank holds a full-size
 * [rows, cols] bf16 buffer with its own share in place; this call copies the
 * t-1 peer shares, rows [i*rows/t, (i+1)*rows/t) of bufs[i] for every i !=
 * rank, into the same rows of `out` (normally bufs[rank]: an in-place gather).
 * `bufs` is a HOST array of t device pointers; bufs[rank] is not read and may
 * be NULL.  rows % t == 0, cols % 8 == 0, 1 <= t <= 16; the rows of `out` in
 * the caller's own share are not touched.  Errors: MTL_E_RANK for rank outside
 * [0, t), MTL_E_UNSUPPORTED when a peer buffer is `out`. */
mtl_status mtl_allgather_rows(int32_t t, int32_t rank, const void* const* bufs, void* out, int64_t rows, int64_t cols,
                              mtl_stream_t stream);

/* Context-parallel causal attention, forward: one CP rank's share.  Context
 * parallelism (ai.lansai.wang/82226, the table of parallelism strategies and the
 * tolerance section; navi2ai.com/sites/1106, --context-parallel-size) cuts the
 * sequence across ranks while attention still needs every earlier rank's keys
 * and values; the pages give no algorithm.  Here the sequence is cp contiguous
 * chunks of `chunk` tokens and rank `rank` holds the queries of chunk `rank`.
 * Its result is those rows of causal attention over the whole sequence: the
 * rank's own chunk is attended causally, chunks rank-1, ..., 0 (the ring order
 * in which a peer would pass them on) with every key visible, and the partial
 * results are merged by their row log-sum-exp; later chunks are fully masked
 * and not read.
 * qkv_chunks: HOST array of cp device pointers, chunk j's head-interleaved QKV
 * [chunk, 3*heads*head_dim] bf16 (head n: q, k, v at columns n*3d + [0, d),
 * [d, 2d), [2d, 3d)); only entries 0..rank are read.  o: [chunk, heads*head_dim]
 * bf16; lse: [heads, chunk] fp32 natural-log row log-sum-exp of the scaled
 * scores (scale 1/sqrt(head_dim)).  scratch: device memory of at least
 * mtl_cp_attn_scratch_bytes() bytes (none for rank 0), caller-owned, contents
 * undefined afterwards.  Micro-batch 1.  chunk % 64 == 0, head_dim 64 or 128,
 * 1 <= cp <= MTL_CP_MAX.  Errors: MTL_E_RANK, MTL_E_SHAPE, MTL_E_NULL,
 * MTL_E_ALIGN (pointers 16-byte aligned), MTL_E_WORKSPACE. */
#define MTL_CP_MAX 64
mtl_status mtl_cp_attn_scratch_bytes(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                                     size_t* scratch_bytes);
mtl_status mtl_cp_attn_fwd(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                           const void* const* qkv_chunks, void* o, float* lse, void* scratch, size_t scratch_bytes,
                           mtl_stream_t stream);

/* Context-parallel causal attention, backward: the gradients that CP rank
 * `rank`'s output gradient sends into the QKV of the sequence (same chunks and
 * reading as mtl_cp_attn_fwd).  o and lse: the rank's merged forward results;
 * dout: dO of its rows, [chunk, heads*head_dim] bf16.  Writes
 *   dqkv [chunk, 3*heads*head_dim] bf16, head-interleaved like the QKV: the
 *     query columns get the complete dQ of the rank's queries (over all chunks
 *     0..rank); the key and value columns get the dK, dV of the rank's own chunk
 *     from its own queries only (the later ranks' queries add their shares);
 *   dkv_chunks[j] for j < rank (HOST array of device pointers, entries 0..rank-1
 *     read): the key and value columns of a [chunk, 3*heads*head_dim] bf16
 *     tensor of chunk j's layout get the dK, dV share of chunk j's keys from the
 *     rank's queries -- what it hands back to chunk j's owner; query columns
 *     are not touched.
 * scratch: at least mtl_cp_attn_bwd_scratch_bytes() bytes (D = rowsum(dO*O)
 * and one dQ partial per earlier chunk), caller-owned.  dQ sums the rank's own
 * chunk first, then chunks rank-1, ..., 0, in fp32 over bf16 partials.
 * Errors as mtl_cp_attn_fwd; MTL_E_UNSUPPORTED when a dkv_chunks entry is dqkv. */
mtl_status mtl_cp_attn_bwd_scratch_bytes(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                                         size_t* scratch_bytes);
mtl_status mtl_cp_attn_bwd(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                           const void* const* qkv_chunks, const void* o, const float* lse, const void* dout,
                           void* dqkv, void* const* dkv_chunks, void* scratch, size_t scratch_bytes,
                           mtl_stream_t stream);

/* MXFP4 quantisation.  The site summary (navi2ai.com/sites/1106, its precision
 * list and deploy step 7) names 4-bit floating-point training (NVFP4 on
 * Blackwell) without a format; the CDNA4 counterpart taken here is OCP MXFP4:
 * FP4 E2M1 elements in blocks of 32 consecutive elements along a row sharing
 * an E8M0 scale 2^e, e = floor(log2(max |v|)) - 2 clamped at -127 (byte e+127);
 * elements v / 2^e rounded to the nearest E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4,
 * 6), ties to the even code, saturating at 6, with the sign of v.
 * x: [rows, cols] bf16 row-major (the GEMM's K along the row), finite values;
 * codes: [rows, cols/2] bytes, element 2i in the low nibble of byte i; scales:
 * [rows, cols/32] bytes.  cols % 32 == 0; pointers 16-byte aligned.  Errors:
 * MTL_E_NULL, MTL_E_ALIGN, MTL_E_SHAPE. */
mtl_status mtl_mxfp4_quantize(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                              mtl_stream_t stream);

/* GEMM on MXFP4 operands with CDNA4's block-scaled MFMA: c [M, N] bf16 (row
 * stride ldc elements) = A . B^T over K, with A [M, K] and B [N, K] given as
 * the codes and scales mtl_mxfp4_quantize writes (a weight W [K, N] enters as
 * its transpose [N, K]).  Products of the scaled elements are exact in fp32 and
 * summed in fp32.  M % 128 == 0, N % 128 == 0, K % 256 == 0, ldc >= N, ldc % 8
 * == 0.  Errors: MTL_E_NULL, MTL_E_ALIGN, MTL_E_SHAPE. */
mtl_status mtl_mxfp4_gemm(int64_t M, int64_t N, int64_t K, const void* a_codes, const void* a_scales,
                          const void* b_codes, const void* b_scales, void* c, int64_t ldc, mtl_stream_t stream);

/* MXFP4 quantisation along the rows of x [rows, cols] (blocks of 32 rows of
 * one column, the scale rule and rounding of mtl_mxfp4_quantize): the codes and
 * scales of x^T, codes [cols, rows/2] bytes and scales [cols, rows/32] bytes,
 * as mtl_mxfp4_gemm takes an operand whose K runs down the columns of a
 * row-major tensor (a weight W [K, N] in a forward product, an activation or
 * gradient [tokens, features] in a weight-gradient product).  rows % 32 == 0,
 * cols % 8 == 0, rows <= 2^23; pointers 16-byte aligned.  Errors: MTL_E_NULL,
 * MTL_E_ALIGN, MTL_E_SHAPE. */
mtl_status mtl_mxfp4_quantize_t(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                                mtl_stream_t stream);

/* MXFP6: the same as mtl_mxfp4_quantize / mtl_mxfp4_gemm with FP6 E2M3 elements
 * (sign, 2 exponent bits of bias 1, 3 mantissa bits; magnitudes k/8 below 1,
 * then steps of 1/8, 1/4, 1/2 up to 7.5; the largest exponent is again 2, so
 * the block scale rule is the same).  codes: [rows, cols*3/4] bytes, each
 * block of 32 elements in 24 bytes with element j at bits 6j .. 6j+5 of the
 * block read as a little-endian number.  The GEMM takes M % 128 == 0,
 * N % 128 == 0, K % 128 == 0. */
mtl_status mtl_mxfp6_quantize(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                              mtl_stream_t stream);
mtl_status mtl_mxfp6_gemm(int64_t M, int64_t N, int64_t K, const void* a_codes, const void* a_scales,
                          const void* b_codes, const void* b_scales, void* c, int64_t ldc, mtl_stream_t stream);

/* The MX quantisers and GEMMs with a choice of byte order (the same values
 * either way).  elem: MTL_MX_E2M1 (MXFP4) or MTL_MX_E2M3 (MXFP6).
 * MTL_MX_ORDER_PLAIN: codes and scales as mtl_mxfp4_quantize /
 * mtl_mxfp6_quantize write them (the calls above).
 * MTL_MX_ORDER_GEMM (rows % 32 == 0, cols % 256 == 0), the order the GEMM
 * reads fastest, one load per lane:
 *   scales: the rows' scale bytes in groups of 256 bytes, one group per 32-row
 *     block rb and 256-element span s of the row, group rb * cols/256 + s;
 *     block q (0..7 within the span) of row r at byte 4 * (r % 32 + 32 * (q %
 *     2)) + q / 2 of the group.
 *   MXFP4 codes: plain.
 *   MXFP6 codes: per row, each 128-element span (4 blocks, 96 bytes) holds
 *     the four blocks' first 16 bytes at 16 b, then their last 8 bytes: blocks
 *     0 and 1 in bytes 64..79, blocks 2 and 3 in bytes 80..95, block 2j at the
 *     first 8 of those bytes and 2j + 1 at the last 8 -- swapped in rows r with
 *     (r / 16) odd.
 * The GEMM: as mtl_mxfp4_gemm on operands of that order; MTL_MX_ORDER_GEMM
 * takes M % 32 == 0, N % 32 == 0, K % 256 == 0.  Errors: MTL_E_NULL,
 * MTL_E_ALIGN, MTL_E_SHAPE, MTL_E_UNSUPPORTED (elem or order). */
#define MTL_MX_E2M1 0
#define MTL_MX_E2M3 1
#define MTL_MX_ORDER_PLAIN 0
#define MTL_MX_ORDER_GEMM 1
mtl_status mtl_mx_quantize_ordered(int32_t elem, const void* x, int64_t rows, int64_t cols, void* codes,
                                   void* scales, int32_t order, mtl_stream_t stream);
mtl_status mtl_mx_gemm_ordered(int32_t elem, int64_t M, int64_t N, int64_t K, const void* a_codes,
                               const void* a_scales, const void* b_codes, const void* b_scales, void* c, int64_t ldc,
                               int32_t order, mtl_stream_t stream);

/* MLP half of the rank's forward (column-parallel fc1 with fused GeLU,
 * row-parallel fc2), with z = h . w1 + b1 in fp32:
 *   gz      = GeLU'(z)        [S, f/t] bf16 (saved: the backward needs z only
 *                             through the GeLU derivative)
 *   a       = GeLU(z)         [S, f/t] bf16 (saved)
 *   partial = a . w2          [S, h]   bf16, this rank's partial sum
 * h [S, h] bf16 is the reduced attention output.  scratch as for mtl_attn_fwd;
 * in fp8, a is quantised from its bf16 values. */
mtl_status mtl_mlp_fwd(const mtl_layer_cfg* cfg, const void* h, const void* w1, const void* b1, const void* w2,
                       void* gz, void* a, void* partial, void* scratch, size_t scratch_bytes, mtl_stream_t stream);

/* MLP backward given dy = dL/dY [S, h] bf16 (every rank holds all of it):
 *   dz         = (dy . w2^T) * gz            (scratch, bf16; gz = GeLU'(z) from mtl_mlp_fwd)
 *   dw2        = a^T . dy                    [f/t, h] fp32
 *   dw1        = h^T . dz                    [h, f/t] fp32
 *   db1        = colsum(dz)                  [f/t] fp32
 *   db2        = colsum(dy)                  [h] fp32, skipped when NULL
 *   dh_partial = dz . w1^T                   [S, h] bf16, this rank's partial
 * With MTL_F_WGRAD_ACCUM the fp32 gradients are added to what the buffers hold. */
mtl_status mtl_mlp_bwd(const mtl_layer_cfg* cfg, const void* dy, const void* h, const void* gz, const void* a,
                       const void* w1, const void* w2, void* dh_partial, float* dw1, float* db1, float* dw2,
                       float* db2, void* scratch, size_t scratch_bytes, mtl_stream_t stream);

/* mtl_mlp_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and outputs, with the scratch taken from a
 * device array inside the library of MTL_NOALLOC_SCRATCH_BYTES bytes instead of
 * a caller's buffer.  It allocates nothing and calls no allocating routine.
 * Every GPU the library runs on holds one such array until the process ends;
 * the first call on a device (with that device current) looks up its address.
 * Status: mtl_validate's; MTL_E_UNSUPPORTED with MTL_F_KEEP_CODES (the kept
 * codes are in the scratch the forward calls were given); MTL_E_WORKSPACE, before any HIP call, when the
 * configuration needs more scratch than the array holds (in bf16 the MLP
 * backward needs 2*S*(f/t) bytes for dz plus 4*ceil(S/64)*(f/t + h) for the
 * column sums: S = 4096 with f/t = 4096 and h = 8192 takes 35 MiB; the fp8
 * path's operand codes need far more at such sizes); otherwise as mtl_mlp_bwd.
 * All calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams, or from several threads) race and give wrong results. */
#define MTL_NOALLOC_SCRATCH_BYTES (48u << 20)
mtl_status mtl_mlp_bwd_noalloc(const mtl_layer_cfg* cfg, const void* dy, const void* h, const void* gz,
                               const void* a, const void* w1, const void* w2, void* dh_partial, float* dw1,
                               float* db1, float* dw2, float* db2, mtl_stream_t stream);

/* Attention backward given dh = dL/dH [S, h] bf16 (reduced) and the saved
 * qkv, o, lse of mtl_attn_fwd:
 *   do         = dh . w_o^T                  (scratch, bf16)
 *   dw_o       = o^T . dh                    [h/t, h] fp32
 *   db_o       = colsum(dh)                  [h] fp32, skipped when NULL
 *   dqkv       = attention backward          (scratch, bf16)
 *   dw_qkv     = x^T . dqkv                  [h, 3h/t] fp32
 *   db_qkv     = colsum(dqkv)                [3h/t] fp32
 *   dx_partial = dqkv . w_qkv^T              [S, h] bf16, this rank's partial
 * The attention backward is deterministic (no atomics).  In fp8 the six GEMMs
 * of mtl_mlp_bwd / mtl_attn_bwd take E5M2 gradients and E4M3 activations and
 * weights (dgrad: gradient x weight; wgrad: activation^T x gradient); the
 * bias gradients are column sums of the bf16 gradients. */
mtl_status mtl_attn_bwd(const mtl_layer_cfg* cfg, const void* dh, const void* x, const void* qkv, const void* o,
                        const float* lse, const void* w_qkv, const void* w_o, void* dx_partial, float* dw_qkv,
                        float* db_qkv, float* dw_o, float* db_o, void* scratch, size_t scratch_bytes,
                        mtl_stream_t stream);

/* Where mtl_attn_bwd leaves its two intermediate gradients in its scratch: dO
 * [S, h/t] at byte offset *do_offset and dQKV [S, 3h/t] at *dqkv_offset, bf16
 * row-major (dQKV in the head-interleaved layout of qkv).  They stay there until
 * the scratch is reused; a caller may read them once the call's stream has
 * drained (to check the attention backward on its own, or to reuse dQKV).
 * Host-only; status as mtl_validate. */
mtl_status mtl_attn_bwd_scratch_layout(const mtl_layer_cfg* cfg, size_t* do_offset, size_t* dqkv_offset);

/* fp8 per-tensor scaling (the site summary's --fp8-format hybrid; the pages give
 * no encoding or scaling rule, read as OCP E4M3 (bias 7, max 448, no infinity)
 * and E5M2 (bias 15, max 57344) with current scaling).
 * rec[0..2] = {amax, s, 1/s} for n bf16 values x: amax = max |x| (exact),
 * s = fmt_max / amax in fp32 with correct rounding (1 when amax is 0, inf or
 * NaN), 1/s likewise.  rec: 16-byte aligned device floats; scratch >=
 * MTL_FP8_AMAX_SCRATCH bytes.  Deterministic. */
mtl_status mtl_fp8_amax(const void* x, int64_t n, int32_t format, float* rec, void* scratch, size_t scratch_bytes,
                        mtl_stream_t stream);

/* Codes of x [rows, cols] bf16: code = round-to-nearest-even of the fp32
 * product x*rec[1] onto the format's grid, saturated to +-fmt_max, NaN -> 0x7F.
 * out [rows, cols] and/or out_t [cols, rows] (the transposed copy a weight
 * gradient needs) -- either may be NULL, not both.  cols % 8 == 0; rows % 16 == 0
 * when out_t is given. */
mtl_status mtl_fp8_cast(const void* x, int64_t rows, int64_t cols, int32_t format, const float* rec, void* out,
                        void* out_t, mtl_stream_t stream);

/* mtl_fp8_amax over the rows*cols values of x, then mtl_fp8_cast with the
 * record it wrote, in one launch fewer (the cast finishes the amax): rec and
 * the codes are bit-identical to the two calls.  Arguments and rules as there
 * (scratch >= MTL_FP8_AMAX_SCRATCH bytes).  This is how the layer entry points
 * quantise their GEMM operands. */
mtl_status mtl_fp8_quantize(const void* x, int64_t rows, int64_t cols, int32_t format, float* rec, void* out,
                            void* out_t, void* scratch, size_t scratch_bytes, mtl_stream_t stream);

/* One fp8 GEMM on codes the caller already holds (from mtl_fp8_quantize or
 * mtl_fp8_cast): C[M, N] = (A . B^T) * a_rec[2] * b_rec[2] (+ bias[n]),
 * accumulated in fp32, where A [M, K] and B [N, K] are k-contiguous codes
 * (row stride K) in formats fmt_a, fmt_b and a_rec, b_rec their scale records
 * {amax, s, 1/s} (device memory).  The format pairs of the hybrid recipe:
 *   E4M3 x E4M3 (forward): C bf16, bias (bf16 [N]) optional;
 *   E5M2 x E4M3 (dgrad: gradient x weight): C bf16, no bias;
 *   E4M3 x E5M2 (wgrad: activation x gradient): C fp32, no bias.
 * ldc >= N, ldc % 8 == 0.  K % 16 == 0 and every operand under 4 GiB
 * ((M + 256) * K < 2^32, likewise N).  It runs the kernel and tile shape a
 * layer call runs for a product of this shape and formats when that product
 * is launched alone (every fp8 GEMM of the layer calls except the output
 * projection's backward pair); for callers that keep quantised weights. */
mtl_status mtl_fp8_gemm(int64_t M, int64_t N, int64_t K, const void* a, int32_t fmt_a, const float* a_rec,
                        const void* b, int32_t fmt_b, const float* b_rec, const void* bias, void* c, int64_t ldc,
                        mtl_stream_t stream);

/* ------------------------------------------------------------------------
 * MoE expert block of one expert-parallel rank.
 *
 * The site summary's MoE deploy step (navi2ai.com/sites/1106, step 6) runs 256
 * experts with a top-8 router on expert-parallel size 16, and the guide's table
 * of parallel strategies (ai.lansai.wang/82226) names the grouped GEMM as the
 * MoE compute path.  The pages print no router formula; this library reads it
 * as: the k largest fp32 logits of a token (ties to the lower expert id, slots
 * in decreasing-logit order), gates = softmax over those k logits, no capacity
 * limit (dropless), rank r of ep owning experts [r*E/ep, (r+1)*E/ep).  The
 * rank's assignments are grouped by expert with tokens ascending; each expert
 * is GeLU(x W1_e) W2_e without biases; a token's output is the gate-weighted
 * sum of its local experts' rows in slot order -- the rank's partial of the
 * combine (the all-to-all that brings the other ranks' experts is not part of
 * this library).
 *
 * Sizes: T = tokens, h = hidden, f = ffn, E = experts, k = topk,
 * E_l = E/ep local experts, N = number of local assignments (offsets[E_l]),
 * N_max = T * min(k, E_l) -- the most N can be, which sizes every per-row
 * buffer (rows past N are never touched).  Expert weights are stored
 * w1 [E_l, h, f] and w2 [E_l, f, h] bf16; their gradients fp32 of the same shape.
 * Integer outputs (ids, counts, offsets, permutation) are exact and
 * deterministic; so is every floating-point output from run to run.
 * ---------------------------------------------------------------------- */

/* --num-experts, --moe-router-topk, --expert-model-parallel-size and this
 * process's EP rank; tokens = micro-batch x sequence length. */
typedef struct mtl_moe_cfg {
  int32_t tokens, hidden, ffn, experts, topk, ep, rank;
  int32_t precision; /* MTL_PREC_BF16 only */
  int32_t flags;     /* MTL_F_WGRAD_ACCUM or 0 */
} mtl_moe_cfg;

/* Host-only check; makes no HIP call.  Every size > 0; experts % ep == 0
 * (MTL_E_DIVISIBILITY); 0 <= rank < ep (MTL_E_RANK); hidden % 8 == 0,
 * ffn % 8 == 0, experts <= 1024, topk <= min(experts, 64), tokens * topk < 2^31,
 * (max(N_max, w) + 256) * w * 2 < 2^32 bytes with w = max(h, f) (MTL_E_SHAPE). */
mtl_status mtl_moe_validate(const mtl_moe_cfg* cfg);

/* N_max = tokens * min(topk, experts/ep): rows of xp, gz, a, ye and of the
 * backward scratch; and the backward's scratch bytes.  Either output may be NULL. */
mtl_status mtl_moe_sizes(const mtl_moe_cfg* cfg, int64_t* max_rows, size_t* scratch_bytes);

/* Router selection: logits [T, E] fp32 -> topk_idx [T, k] int32, gates [T, k]
 * fp32 (softmax of the selected logits, computed in fp32).  Logits must not be NaN. */
mtl_status mtl_moe_route(const mtl_moe_cfg* cfg, const float* logits, int32_t* topk_idx, float* gates,
                         mtl_stream_t stream);

/* The MoE router's linear (replicated on every expert-parallel rank; the site
 * summary's MoE deploy step routes each token to --moe-router-topk experts of
 * --num-experts):
 *   logits = x . w_r    [T, E] fp32 (bf16 operands, fp32 accumulate)
 * x [T, h] bf16, w_r [h, E] bf16.  E % 8 == 0.  The routing itself is
 * mtl_moe_route.  The router calls read tokens, hidden, experts, topk and
 * flags of cfg; ffn only has to pass mtl_moe_validate (the experts' sizes do
 * not enter). */
mtl_status mtl_moe_router_fwd(const mtl_moe_cfg* cfg, const void* x, const void* w_r, float* logits,
                              mtl_stream_t stream);

/* Scratch bytes of mtl_moe_router_bwd. */
mtl_status mtl_moe_router_sizes(const mtl_moe_cfg* cfg, size_t* scratch_bytes);

/* Router backward with the load-balancing loss.  The deploy step sets
 * --moe-aux-loss-coeff (alpha) without a formula; the Switch Transformer form
 * is taken:
 *   L_aux = alpha * E * sum_e f_e P_e,   f_e = c_e / (T k),
 *   P_e = mean over tokens of softmax(logits_t)_e (over all E experts),
 * c_e = assignments routed to expert e in topk_idx (a constant of the
 * backward).  Computed:
 *   aux_loss  [1] fp32 (device; NULL to skip the value, the gradient is kept)
 *   dlogits   [T, E] fp32 = backward of the gate softmax over the k selected
 *             logits given dgates, plus dL_aux/dlogits
 *   dw_r      [h, E] fp32 = x^T . dlogits   (+= with MTL_F_WGRAD_ACCUM)
 *   dx        [T, h] bf16 = dlogits . w_r^T (the router's share of dL/dx)
 * The two products take dlogits rounded to bf16.  logits, topk_idx [T, k]
 * int32 (ids in [0, E)) and gates [T, k] fp32 are those of mtl_moe_router_fwd
 * and mtl_moe_route; dgates [T, k] fp32 is dL/dgates summed over the ranks
 * that hold the experts (on one rank, what mtl_moe_bwd returns).  0 <=
 * aux_coeff < inf.  scratch: mtl_moe_router_sizes bytes. */
mtl_status mtl_moe_router_bwd(const mtl_moe_cfg* cfg, const void* x, const void* w_r, const float* logits,
                              const int32_t* topk_idx, const float* gates, const float* dgates, float aux_coeff,
                              float* aux_loss, float* dlogits, float* dw_r, void* dx, void* scratch,
                              size_t scratch_bytes, mtl_stream_t stream);

/* Stable grouping of this rank's assignments by local expert:
 *   counts   [E_l]     assignments per local expert
 *   offsets  [E_l + 1] exclusive prefix sum; offsets[E_l] = N
 *   perm_token, perm_slot [N_max]: row i < N is assignment (token, slot)
 *   slot_row [T, k]    inverse map: the row of (t, s), or -1 when the slot's
 *                      expert is not on this rank
 * topk_idx [T, k] int32 with every id in [0, E). */
mtl_status mtl_moe_permute(const mtl_moe_cfg* cfg, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                           int32_t* perm_token, int32_t* perm_slot, int32_t* slot_row, mtl_stream_t stream);

/* Expert forward (grouped GEMMs over the E_l local experts):
 *   xp = x[perm_token]                     [N_max, h] bf16 (saved)
 *   with z = xp_e . w1_e per expert in fp32:
 *   gz = GeLU'(z)                          [N_max, f] bf16 (saved)
 *   a  = GeLU(z)                           [N_max, f] bf16 (saved)
 *   ye = a_e . w2_e per expert             [N_max, h] bf16 (saved, not gate-scaled)
 *   y_partial[t] = sum over local slots s of t, ascending, of gates[t,s] * ye[row]
 *                                          [T, h] bf16 (zero rows for tokens with no local expert)
 * x [T, h] bf16; the routing arrays are those of mtl_moe_route/permute. */
mtl_status mtl_moe_fwd(const mtl_moe_cfg* cfg, const void* x, const int32_t* offsets, const int32_t* perm_token,
                       const int32_t* slot_row, const float* gates, const void* w1, const void* w2, void* xp, void* gz,
                       void* a, void* ye, void* y_partial, mtl_stream_t stream);

/* Expert backward given dy = dL/dY [T, h] bf16:
 *   dye       = gates[t,s] * dy[t] per row       (scratch)
 *   dgates    = <ye[row], dy[t]>                 [T, k] fp32, 0 on non-local slots
 *   dz        = (dye_e . w2_e^T) * gz            (scratch; gz = GeLU'(z) from mtl_moe_fwd)
 *   dw2[e]    = a_e^T . dye_e                    [E_l, f, h] fp32
 *   dw1[e]    = xp_e^T . dz_e                    [E_l, h, f] fp32 (zero for an expert with no rows)
 *   dx_partial[t] = sum over local slots of t, ascending, of (dz_e . w1_e^T)[row]
 *                                                [T, h] bf16
 * The gradient through the gate softmax into the logits is not computed here.
 * With MTL_F_WGRAD_ACCUM, dw1/dw2 are added to. */
mtl_status mtl_moe_bwd(const mtl_moe_cfg* cfg, const void* dy, const int32_t* offsets, const int32_t* perm_token,
                       const int32_t* perm_slot, const int32_t* slot_row, const float* gates, const void* xp,
                       const void* gz, const void* a, const void* ye, const void* w1, const void* w2, void* dx_partial,
                       float* dw1, float* dw2, float* dgates, void* scratch, size_t scratch_bytes,
                       mtl_stream_t stream);

/* ---------------------------------------------------------------- launch timing
 * Measurement aid, not part of the layer's arithmetic.  The guide's section on
 * performance reports asks for per-step timings that separate the parts of a
 * step; these calls give them per launch group.  Between mtl_prof_start and
 * mtl_prof_stop every group of launches the dense-layer entry points make
 * (mtl_attn_fwd, mtl_mlp_fwd, mtl_mlp_bwd, mtl_attn_bwd, mtl_reduce,
 * mtl_allgather_rows) and the MoE expert calls (mtl_moe_fwd, mtl_moe_bwd) is
 * bracketed by two HIP events recorded on its stream, and kept, in launch
 * order, with its kind (MTL_PROF_*), a static name and its algorithmic FLOP
 * (2MNK per GEMM, the causal triangle for attention) and HBM bytes (every
 * element read and written once; the fp8 quantisation reads its input twice,
 * once for the amax and once for the cast).  The MoE groups carry 0 FLOP and
 * 0 bytes: their row counts live on the device.  A group is one GEMM or GEMM
 * pair, the attention kernels of one call, one reduce, one gather, one
 * column-sum pair or one fp8 quantisation pair.  At most MTL_PROF_MAX groups are
 * kept; later ones run untimed.
 *
 * mtl_prof_start: on the current device; the first call (and a call on another
 * device) creates the 2 * MTL_PROF_MAX events, later calls reuse them.  Clears
 * the table.  MTL_E_HIP if there is no device.
 * mtl_prof_stop: stops recording; *n_records = number of groups kept.
 * mtl_prof_record: group i (0 <= i < n_records) after mtl_prof_stop; waits for
 * its stop event and returns the elapsed milliseconds between its two events.
 * MTL_E_SHAPE for i out of range, MTL_E_UNSUPPORTED while recording.
 * Process-wide state: not for concurrent use from several threads, and not
 * while a stream is being captured into a graph. */
#define MTL_PROF_MAX 2048
enum { MTL_PROF_GEMM = 0, MTL_PROF_ATTN = 1, MTL_PROF_REDUCE = 2, MTL_PROF_COLSUM = 3, MTL_PROF_QUANT = 4,
       MTL_PROF_GATHER = 5 };
mtl_status mtl_prof_start(void);
mtl_status mtl_prof_stop(int32_t* n_records);
mtl_status mtl_prof_record(int32_t i, int32_t* kind, double* flop, double* bytes, float* ms, const char** name);

/* ---------------------------------------------------------------- MFMA ceiling
 * Measurement aid, not part of the layer's arithmetic: the rate the matrix
 * cores reach on their own, the yardstick for the GEMMs' share of the MFMA peak
 * (the site's precision section puts the layer's linears on the matrix cores in
 * bf16, fp8 and fp4).  Each of `workgroups` workgroups of 4 waves issues, per
 * wave, `iters` times the MFMA stream of one 128x128 output tile over one
 * k-slab -- 32 v_mfma_f32_32x32x16_bf16 (kind 0), or 16
 * v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands (kind 1) or on E2M1
 * operands with unit E8M0 scales (kind 2), into 16 independent 32x32 fp32
 * accumulators -- with every operand fragment loaded from `data` once before
 * the loop: no other memory traffic, no LDS, no barrier.  FLOP per launch =
 * workgroups * 4 * iters * 1048576 (kind 0) or 2097152 (kinds 1 and 2); 256
 * workgroups and 128 (bf16) or 64 (fp8, fp4) iterations issue exactly the
 * MFMAs of a 4096x4096x4096 GEMM in 256x256 tiles.
 * data: device, >= MTL_CEILING_DATA_BYTES bytes of operand values (bf16, E4M3
 * codes or packed E2M1 codes; the distribution is the caller's); wave w reads the 16 KiB at
 * (w % 64) * 16 KiB.  out: device fp32 [workgroups * 256], each lane's sum of
 * its accumulators (keeps the MFMAs live).  16-byte aligned pointers
 * (MTL_E_ALIGN).  MTL_E_UNSUPPORTED for another kind; MTL_E_SHAPE for a short
 * data buffer, workgroups outside [1, 2^20] or iters <= 0. */
#define MTL_CEILING_DATA_BYTES (1u << 20)
mtl_status mtl_mfma_ceiling(const void* data, size_t data_bytes, int32_t kind, int64_t workgroups, int64_t iters,
                            float* out, mtl_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MTL_H */
