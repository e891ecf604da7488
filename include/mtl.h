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

enum { MTL_PREC_BF16 = 0, MTL_PREC_FP8_HYBRID = 1 };

enum {
  MTL_F_RESIDUAL = 1,   /* mtl_reduce callers add residuals; recorded for validation only */
  MTL_F_WGRAD_ACCUM = 2 /* weight/bias gradients are accumulated (+=) instead of written */
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
 * those head sizes and the GEMMs move 16-byte vectors); tp <= 16. */
mtl_status mtl_validate(const mtl_layer_cfg* cfg);

/* Bytes of device scratch the backward calls need (*scratch_bytes) for this
 * configuration.  The forward calls need none. */
mtl_status mtl_workspace_bytes(const mtl_layer_cfg* cfg, size_t* scratch_bytes);

/* Attention half of the rank's forward (column-parallel QKV, causal attention
 * over the rank's heads/t heads, row-parallel output projection):
 *   qkv     = x . w_qkv + b_qkv          [S, 3h/t] bf16 (saved for backward)
 *   o       = attention(qkv)             [S, h/t]  bf16 (saved)
 *   lse     = row log-sum-exp of scaled scores, [heads/t, S] fp32 (saved)
 *   partial = o . w_o                    [S, h]    bf16, this rank's partial sum
 * x [S, h] bf16. */
mtl_status mtl_attn_fwd(const mtl_layer_cfg* cfg, const void* x, const void* w_qkv, const void* b_qkv,
                        const void* w_o, void* qkv, void* o, float* lse, void* partial, mtl_stream_t stream);

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

/* MLP half of the rank's forward (column-parallel fc1 with fused GeLU,
 * row-parallel fc2):
 *   z       = h . w1 + b1     [S, f/t] bf16 (saved)
 *   a       = GeLU(z)         [S, f/t] bf16 (saved; GeLU of the fp32 z)
 *   partial = a . w2          [S, h]   bf16, this rank's partial sum
 * h [S, h] bf16 is the reduced attention output. */
mtl_status mtl_mlp_fwd(const mtl_layer_cfg* cfg, const void* h, const void* w1, const void* b1, const void* w2,
                       void* z, void* a, void* partial, mtl_stream_t stream);

/* MLP backward given dy = dL/dY [S, h] bf16 (every rank holds all of it):
 *   dz         = (dy . w2^T) * GeLU'(z)      (scratch, bf16)
 *   dw2        = a^T . dy                    [f/t, h] fp32
 *   dw1        = h^T . dz                    [h, f/t] fp32
 *   db1        = colsum(dz)                  [f/t] fp32
 *   db2        = colsum(dy)                  [h] fp32, skipped when NULL
 *   dh_partial = dz . w1^T                   [S, h] bf16, this rank's partial
 * With MTL_F_WGRAD_ACCUM the fp32 gradients are added to what the buffers hold. */
mtl_status mtl_mlp_bwd(const mtl_layer_cfg* cfg, const void* dy, const void* h, const void* z, const void* a,
                       const void* w1, const void* w2, void* dh_partial, float* dw1, float* db1, float* dw2,
                       float* db2, void* scratch, size_t scratch_bytes, mtl_stream_t stream);

/* Attention backward given dh = dL/dH [S, h] bf16 (reduced) and the saved
 * qkv, o, lse of mtl_attn_fwd:
 *   do         = dh . w_o^T                  (scratch, bf16)
 *   dw_o       = o^T . dh                    [h/t, h] fp32
 *   db_o       = colsum(dh)                  [h] fp32, skipped when NULL
 *   dqkv       = attention backward          (scratch, bf16)
 *   dw_qkv     = x^T . dqkv                  [h, 3h/t] fp32
 *   db_qkv     = colsum(dqkv)                [3h/t] fp32
 *   dx_partial = dqkv . w_qkv^T              [S, h] bf16, this rank's partial
 * The attention backward is deterministic (no atomics). */
mtl_status mtl_attn_bwd(const mtl_layer_cfg* cfg, const void* dh, const void* x, const void* qkv, const void* o,
                        const float* lse, const void* w_qkv, const void* w_o, void* dx_partial, float* dw_qkv,
                        float* db_qkv, float* dw_o, float* db_o, void* scratch, size_t scratch_bytes,
                        mtl_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MTL_H */
