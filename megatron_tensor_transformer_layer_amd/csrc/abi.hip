// extern "C" entry points of libmtl.so (declared and documented in include/mtl.h):
// configuration checks, scratch carving and the launch sequence of each block.
#include "../../include/mtl.h"

#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.hpp"

using namespace mtl;

namespace {

constexpr size_t ALIGN = 256;
inline size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Dims {
  int64_t S, h, heads_l, d, f_l, qkv_l, o_l;
};

Dims dims_of(const mtl_layer_cfg* c) {
  Dims d;
  d.S = (int64_t)c->seq * c->micro_batch;
  d.h = c->hidden;
  d.heads_l = c->heads / c->tp;
  d.d = c->hidden / c->heads;
  d.f_l = c->ffn / c->tp;
  d.qkv_l = 3 * d.heads_l * d.d;
  d.o_l = d.heads_l * d.d;
  return d;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename... P>
mtl_status check_ptrs(P... ps) {
  const void* arr[] = {static_cast<const void*>(ps)...};
  for (const void* p : arr)
    if (!p) return MTL_E_NULL;
  for (const void* p : arr)
    if (!aligned16(p)) return MTL_E_ALIGN;
  return MTL_OK;
}

inline mtl_status hip_status(hipError_t e) { return e == hipSuccess ? MTL_OK : MTL_E_HIP; }

#define MTL_TRY(expr)                          \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return MTL_E_HIP;    \
  } while (0)

GemmArgs gemm(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t M, int64_t N, int64_t K, void* c,
              int64_t ldc) {
  GemmArgs g{};
  g.a = static_cast<const uint16_t*>(a);
  g.b = static_cast<const uint16_t*>(b);
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.c = c;
  g.ldc = ldc;
  return g;
}

struct MlpScratch {
  uint16_t* dz;
  float* ws;
};
struct AttnScratch {
  uint16_t* dout;
  uint16_t* dqkv;
  float* delta;
  float* ws;
};

size_t mlp_scratch(const Dims& d, MlpScratch* s, char* base) {
  size_t off = 0;
  if (s) s->dz = reinterpret_cast<uint16_t*>(base + off);
  off += up(d.S * d.f_l * 2);
  if (s) s->ws = reinterpret_cast<float*>(base + off);
  off += up(colsum_ws_floats(d.S, d.f_l > d.h ? d.f_l : d.h) * 4);
  return off;
}

size_t attn_scratch(const Dims& d, AttnScratch* s, char* base) {
  size_t off = 0;
  if (s) s->dout = reinterpret_cast<uint16_t*>(base + off);
  off += up(d.S * d.o_l * 2);
  if (s) s->dqkv = reinterpret_cast<uint16_t*>(base + off);
  off += up(d.S * d.qkv_l * 2);
  if (s) s->delta = reinterpret_cast<float*>(base + off);
  off += up(d.heads_l * d.S * 4);
  if (s) s->ws = reinterpret_cast<float*>(base + off);
  off += up(colsum_ws_floats(d.S, d.qkv_l > d.h ? d.qkv_l : d.h) * 4);
  return off;
}

}  // namespace

extern "C" {

const char* mtl_status_str(mtl_status s) {
  switch (s) {
    case MTL_OK: return "ok";
    case MTL_E_NULL: return "a required pointer is NULL";
    case MTL_E_DIVISIBILITY: return "sizes do not divide (hidden % heads, heads % tp, ffn % tp, experts % ep)";
    case MTL_E_RANK: return "rank outside [0, tp) or [0, ep)";
    case MTL_E_SHAPE: return "a size is <= 0 or outside what the kernels tile";
    case MTL_E_ALIGN: return "a pointer is not 16-byte aligned";
    case MTL_E_WORKSPACE: return "scratch buffer too small";
    case MTL_E_UNSUPPORTED: return "unsupported precision or flag combination";
    case MTL_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

mtl_status mtl_validate(const mtl_layer_cfg* c) {
  if (!c) return MTL_E_NULL;
  if (c->hidden <= 0 || c->heads <= 0 || c->ffn <= 0 || c->seq <= 0 || c->micro_batch <= 0 || c->tp <= 0)
    return MTL_E_SHAPE;
  if (c->hidden % c->heads != 0 || c->heads % c->tp != 0 || c->ffn % c->tp != 0) return MTL_E_DIVISIBILITY;
  if (c->rank < 0 || c->rank >= c->tp) return MTL_E_RANK;
  const int d = c->hidden / c->heads;
  if (d != 64 && d != 128) return MTL_E_SHAPE;
  if ((c->ffn / c->tp) % 8 != 0) return MTL_E_SHAPE;
  if (c->tp > 16) return MTL_E_SHAPE;
  if ((int64_t)c->seq * c->micro_batch > (int64_t)1 << 30) return MTL_E_SHAPE;
  {
    // every GEMM operand is addressed with 32-bit byte offsets
    const Dims d = dims_of(c);
    const int64_t w = std::max({d.h, d.qkv_l, d.f_l});
    if ((std::max(d.S, w) + 256) * w * 2 >= ((int64_t)1 << 32)) return MTL_E_SHAPE;
  }
  if (c->precision != MTL_PREC_BF16) return MTL_E_UNSUPPORTED;
  if (c->flags & ~(MTL_F_RESIDUAL | MTL_F_WGRAD_ACCUM)) return MTL_E_UNSUPPORTED;
  return MTL_OK;
}

mtl_status mtl_workspace_bytes(const mtl_layer_cfg* c, size_t* scratch_bytes) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if (!scratch_bytes) return MTL_E_NULL;
  const Dims d = dims_of(c);
  const size_t a = mlp_scratch(d, nullptr, nullptr), b = attn_scratch(d, nullptr, nullptr);
  *scratch_bytes = a > b ? a : b;
  return MTL_OK;
}

mtl_status mtl_attn_fwd(const mtl_layer_cfg* c, const void* x, const void* w_qkv, const void* b_qkv, const void* w_o,
                        void* qkv, void* o, float* lse, void* partial, mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(x, w_qkv, b_qkv, w_o, qkv, o, lse, partial)) != MTL_OK) return st;
  const Dims d = dims_of(c);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  GemmArgs g = gemm(x, d.h, w_qkv, d.qkv_l, d.S, d.qkv_l, d.h, qkv, d.qkv_l);
  g.bias = static_cast<const uint16_t*>(b_qkv);
  MTL_TRY(gemm_bf16(g, GEMM_FWD, EPI_BF16_BIAS, s));

  AttnArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.ld_qkv = d.qkv_l;
  a.o = static_cast<uint16_t*>(o);
  a.ld_o = d.o_l;
  a.lse = lse;
  a.seq = c->seq;
  a.batch = c->micro_batch;
  a.heads = (int)d.heads_l;
  a.d = (int)d.d;
  a.scale = 1.0f / sqrtf((float)d.d);
  MTL_TRY(attention_fwd(a, s));

  g = gemm(o, d.o_l, w_o, d.h, d.S, d.h, d.o_l, partial, d.h);
  MTL_TRY(gemm_bf16(g, GEMM_FWD, EPI_BF16, s));
  return MTL_OK;
}

mtl_status mtl_reduce(int32_t t, const void* const* partials, const void* bias, const void* residual, void* out,
                      int64_t rows, int64_t cols, int64_t row_begin, int64_t row_end, mtl_stream_t stream) {
  if (!partials || !out) return MTL_E_NULL;
  if (t < 1 || t > 16 || rows <= 0 || cols <= 0 || cols % 8 != 0) return MTL_E_SHAPE;
  if (row_begin < 0 || row_end > rows || row_begin > row_end) return MTL_E_SHAPE;
  for (int i = 0; i < t; ++i) {
    if (!partials[i]) return MTL_E_NULL;
    if (!aligned16(partials[i])) return MTL_E_ALIGN;
    if (partials[i] == out) return MTL_E_UNSUPPORTED;
  }
  if (!aligned16(out) || (bias && !aligned16(bias)) || (residual && !aligned16(residual))) return MTL_E_ALIGN;
  const uint16_t* p[16];
  for (int i = 0; i < t; ++i) p[i] = static_cast<const uint16_t*>(partials[i]);
  return hip_status(reduce_partials(t, p, static_cast<const uint16_t*>(bias), static_cast<const uint16_t*>(residual),
                                    static_cast<uint16_t*>(out), cols, row_begin, row_end,
                                    reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_mlp_fwd(const mtl_layer_cfg* c, const void* h, const void* w1, const void* b1, const void* w2, void* z,
                       void* a, void* partial, mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(h, w1, b1, w2, z, a, partial)) != MTL_OK) return st;
  const Dims d = dims_of(c);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  GemmArgs g = gemm(h, d.h, w1, d.f_l, d.S, d.f_l, d.h, z, d.f_l);
  g.bias = static_cast<const uint16_t*>(b1);
  g.c2 = a;
  g.ldc2 = d.f_l;
  MTL_TRY(gemm_bf16(g, GEMM_FWD, EPI_BIAS_GELU, s));

  g = gemm(a, d.f_l, w2, d.h, d.S, d.h, d.f_l, partial, d.h);
  MTL_TRY(gemm_bf16(g, GEMM_FWD, EPI_BF16, s));
  return MTL_OK;
}

mtl_status mtl_mlp_bwd(const mtl_layer_cfg* c, const void* dy, const void* h, const void* z, const void* a,
                       const void* w1, const void* w2, void* dh_partial, float* dw1, float* db1, float* dw2,
                       float* db2, void* scratch, size_t scratch_bytes, mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(dy, h, z, a, w1, w2, dh_partial, dw1, db1, dw2, scratch)) != MTL_OK) return st;
  if (db2 && !aligned16(db2)) return MTL_E_ALIGN;
  const Dims d = dims_of(c);
  MlpScratch ws;
  if (scratch_bytes < mlp_scratch(d, &ws, static_cast<char*>(scratch))) return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool accum = (c->flags & MTL_F_WGRAD_ACCUM) != 0;
  const int wepi = accum ? EPI_F32_ACC : EPI_F32;

  // dz = (dy . w2^T) * GeLU'(z)
  GemmArgs g = gemm(dy, d.h, w2, d.h, d.S, d.f_l, d.h, ws.dz, d.f_l);
  g.aux = static_cast<const uint16_t*>(z);
  g.ld_aux = d.f_l;
  MTL_TRY(gemm_bf16(g, GEMM_DGRAD, EPI_DGELU, s));
  // dw2 = a^T . dy
  g = gemm(a, d.f_l, dy, d.h, d.f_l, d.h, d.S, dw2, d.h);
  MTL_TRY(gemm_bf16(g, GEMM_WGRAD, wepi, s));
  // dw1 = h^T . dz
  g = gemm(h, d.h, ws.dz, d.f_l, d.h, d.f_l, d.S, dw1, d.f_l);
  MTL_TRY(gemm_bf16(g, GEMM_WGRAD, wepi, s));
  MTL_TRY(colsum_bf16(ws.dz, d.S, d.f_l, d.f_l, db1, accum, ws.ws, s));
  if (db2) MTL_TRY(colsum_bf16(static_cast<const uint16_t*>(dy), d.S, d.h, d.h, db2, accum, ws.ws, s));
  // dh_partial = dz . w1^T
  g = gemm(ws.dz, d.f_l, w1, d.f_l, d.S, d.h, d.f_l, dh_partial, d.h);
  MTL_TRY(gemm_bf16(g, GEMM_DGRAD, EPI_BF16, s));
  return MTL_OK;
}

mtl_status mtl_attn_bwd(const mtl_layer_cfg* c, const void* dh, const void* x, const void* qkv, const void* o,
                        const float* lse, const void* w_qkv, const void* w_o, void* dx_partial, float* dw_qkv,
                        float* db_qkv, float* dw_o, float* db_o, void* scratch, size_t scratch_bytes,
                        mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(dh, x, qkv, o, lse, w_qkv, w_o, dx_partial, dw_qkv, db_qkv, dw_o, scratch)) != MTL_OK)
    return st;
  if (db_o && !aligned16(db_o)) return MTL_E_ALIGN;
  const Dims d = dims_of(c);
  AttnScratch ws;
  if (scratch_bytes < attn_scratch(d, &ws, static_cast<char*>(scratch))) return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool accum = (c->flags & MTL_F_WGRAD_ACCUM) != 0;
  const int wepi = accum ? EPI_F32_ACC : EPI_F32;

  // do = dh . w_o^T
  GemmArgs g = gemm(dh, d.h, w_o, d.h, d.S, d.o_l, d.h, ws.dout, d.o_l);
  MTL_TRY(gemm_bf16(g, GEMM_DGRAD, EPI_BF16, s));
  // dw_o = o^T . dh
  g = gemm(o, d.o_l, dh, d.h, d.o_l, d.h, d.S, dw_o, d.h);
  MTL_TRY(gemm_bf16(g, GEMM_WGRAD, wepi, s));
  if (db_o) MTL_TRY(colsum_bf16(static_cast<const uint16_t*>(dh), d.S, d.h, d.h, db_o, accum, ws.ws, s));

  AttnArgs at{};
  at.qkv = static_cast<const uint16_t*>(qkv);
  at.ld_qkv = d.qkv_l;
  at.ld_o = d.o_l;
  at.seq = c->seq;
  at.batch = c->micro_batch;
  at.heads = (int)d.heads_l;
  at.d = (int)d.d;
  at.scale = 1.0f / sqrtf((float)d.d);
  at.dout = ws.dout;
  at.out = static_cast<const uint16_t*>(o);
  at.lse_in = lse;
  at.delta = ws.delta;
  at.dqkv = ws.dqkv;
  MTL_TRY(attention_bwd(at, s));

  // dw_qkv = x^T . dqkv ; db_qkv = colsum(dqkv) ; dx_partial = dqkv . w_qkv^T
  g = gemm(x, d.h, ws.dqkv, d.qkv_l, d.h, d.qkv_l, d.S, dw_qkv, d.qkv_l);
  MTL_TRY(gemm_bf16(g, GEMM_WGRAD, wepi, s));
  MTL_TRY(colsum_bf16(ws.dqkv, d.S, d.qkv_l, d.qkv_l, db_qkv, accum, ws.ws, s));
  g = gemm(ws.dqkv, d.qkv_l, w_qkv, d.qkv_l, d.S, d.h, d.qkv_l, dx_partial, d.h);
  MTL_TRY(gemm_bf16(g, GEMM_DGRAD, EPI_BF16, s));
  return MTL_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- MoE

namespace {

struct MoeDims {
  int64_t T, h, f, E, k, El, e_lo, nmax;
};

MoeDims moe_dims(const mtl_moe_cfg* c) {
  MoeDims d;
  d.T = c->tokens;
  d.h = c->hidden;
  d.f = c->ffn;
  d.E = c->experts;
  d.k = c->topk;
  d.El = c->experts / c->ep;
  d.e_lo = (int64_t)c->rank * d.El;
  d.nmax = d.T * (d.k < d.El ? d.k : d.El);
  return d;
}

struct MoeScratch {
  uint16_t* dye;  // [N_max, h]; reused for dxp once the wgrads have read dye
  uint16_t* dz;   // [N_max, f]
};

size_t moe_scratch(const MoeDims& d, MoeScratch* s, char* base) {
  size_t off = 0;
  if (s) s->dye = reinterpret_cast<uint16_t*>(base + off);
  off += up(d.nmax * d.h * 2);
  if (s) s->dz = reinterpret_cast<uint16_t*>(base + off);
  off += up(d.nmax * d.f * 2);
  return off;
}

GemmArgs grouped(const MoeDims& d, GemmGroupMode mode, const int32_t* offsets, int64_t stride_b, int64_t stride_c) {
  GemmArgs g{};
  g.offsets = offsets;
  g.groups = (int)d.El;
  g.group_mode = mode;
  g.stride_b = stride_b;
  g.stride_c = stride_c;
  return g;
}

}  // namespace

extern "C" {

mtl_status mtl_moe_validate(const mtl_moe_cfg* c) {
  if (!c) return MTL_E_NULL;
  if (c->tokens <= 0 || c->hidden <= 0 || c->ffn <= 0 || c->experts <= 0 || c->topk <= 0 || c->ep <= 0)
    return MTL_E_SHAPE;
  if (c->experts % c->ep != 0) return MTL_E_DIVISIBILITY;
  if (c->rank < 0 || c->rank >= c->ep) return MTL_E_RANK;
  if (c->hidden % 8 != 0 || c->ffn % 8 != 0) return MTL_E_SHAPE;
  if (c->experts > 1024 || c->topk > c->experts || c->topk > 64) return MTL_E_SHAPE;
  if ((int64_t)c->tokens * c->topk >= ((int64_t)1 << 31)) return MTL_E_SHAPE;
  {
    // every grouped-GEMM operand is addressed with 32-bit byte offsets
    const MoeDims d = moe_dims(c);
    const int64_t w = std::max(d.h, d.f);
    if ((std::max(d.nmax, w) + 256) * w * 2 >= ((int64_t)1 << 32)) return MTL_E_SHAPE;
  }
  if (c->precision != MTL_PREC_BF16) return MTL_E_UNSUPPORTED;
  if (c->flags & ~MTL_F_WGRAD_ACCUM) return MTL_E_UNSUPPORTED;
  return MTL_OK;
}

mtl_status mtl_moe_sizes(const mtl_moe_cfg* c, int64_t* max_rows, size_t* scratch_bytes) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  const MoeDims d = moe_dims(c);
  if (max_rows) *max_rows = d.nmax;
  if (scratch_bytes) *scratch_bytes = moe_scratch(d, nullptr, nullptr);
  return MTL_OK;
}

mtl_status mtl_moe_route(const mtl_moe_cfg* c, const float* logits, int32_t* topk_idx, float* gates,
                         mtl_stream_t stream) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(logits, topk_idx, gates)) != MTL_OK) return st;
  return hip_status(moe_route(logits, c->tokens, c->experts, c->topk, topk_idx, gates,
                              reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_moe_permute(const mtl_moe_cfg* c, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                           int32_t* perm_token, int32_t* perm_slot, int32_t* slot_row, mtl_stream_t stream) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(topk_idx, counts, offsets, perm_token, perm_slot, slot_row)) != MTL_OK) return st;
  const MoeDims d = moe_dims(c);
  return hip_status(moe_permute(topk_idx, (int)d.T, (int)d.k, (int)d.e_lo, (int)d.El, counts, offsets, perm_token,
                                perm_slot, slot_row, reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_moe_fwd(const mtl_moe_cfg* c, const void* x, const int32_t* offsets, const int32_t* perm_token,
                       const int32_t* slot_row, const float* gates, const void* w1, const void* w2, void* xp, void* z,
                       void* a, void* ye, void* y_partial, mtl_stream_t stream) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(x, offsets, perm_token, slot_row, gates, w1, w2, xp, z, a, ye, y_partial)) != MTL_OK) return st;
  const MoeDims d = moe_dims(c);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  MTL_TRY(moe_gather(static_cast<const uint16_t*>(x), perm_token, offsets, (int)d.El, d.nmax, d.h,
                     static_cast<uint16_t*>(xp), s));
  // z = xp_e . w1_e, a = GeLU(z)   (the grid covers N_max rows; M carries N_max)
  GemmArgs g = grouped(d, GROUP_M, offsets, d.h * d.f, 0);
  g.a = static_cast<const uint16_t*>(xp);
  g.lda = d.h;
  g.b = static_cast<const uint16_t*>(w1);
  g.ldb = d.f;
  g.M = (int)d.nmax;
  g.N = (int)d.f;
  g.K = (int)d.h;
  g.c = z;
  g.ldc = d.f;
  g.c2 = a;
  g.ldc2 = d.f;
  MTL_TRY(gemm_bf16(g, GEMM_FWD, EPI_BIAS_GELU, s));
  // ye = a_e . w2_e
  g = grouped(d, GROUP_M, offsets, d.f * d.h, 0);
  g.a = static_cast<const uint16_t*>(a);
  g.lda = d.f;
  g.b = static_cast<const uint16_t*>(w2);
  g.ldb = d.h;
  g.M = (int)d.nmax;
  g.N = (int)d.h;
  g.K = (int)d.f;
  g.c = ye;
  g.ldc = d.h;
  MTL_TRY(gemm_bf16(g, GEMM_FWD, EPI_BF16, s));
  MTL_TRY(moe_combine(static_cast<const uint16_t*>(ye), slot_row, gates, (int)d.T, (int)d.k, d.h,
                      static_cast<uint16_t*>(y_partial), s));
  return MTL_OK;
}

mtl_status mtl_moe_bwd(const mtl_moe_cfg* c, const void* dy, const int32_t* offsets, const int32_t* perm_token,
                       const int32_t* perm_slot, const int32_t* slot_row, const float* gates, const void* xp,
                       const void* z, const void* a, const void* ye, const void* w1, const void* w2, void* dx_partial,
                       float* dw1, float* dw2, float* dgates, void* scratch, size_t scratch_bytes,
                       mtl_stream_t stream) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(dy, offsets, perm_token, perm_slot, slot_row, gates, xp, z, a, ye, w1, w2, dx_partial, dw1,
                       dw2, dgates, scratch)) != MTL_OK)
    return st;
  const MoeDims d = moe_dims(c);
  MoeScratch ws;
  if (scratch_bytes < moe_scratch(d, &ws, static_cast<char*>(scratch))) return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int wepi = (c->flags & MTL_F_WGRAD_ACCUM) ? EPI_F32_ACC : EPI_F32;

  MTL_TRY(moe_combine_bwd(static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ye), perm_token, perm_slot,
                          slot_row, offsets, (int)d.El, d.nmax, gates, (int)d.T, (int)d.k, d.h, ws.dye, dgates, s));
  // dz = (dye_e . w2_e^T) * GeLU'(z)
  GemmArgs g = grouped(d, GROUP_M, offsets, d.f * d.h, 0);
  g.a = ws.dye;
  g.lda = d.h;
  g.b = static_cast<const uint16_t*>(w2);
  g.ldb = d.h;
  g.M = (int)d.nmax;
  g.N = (int)d.f;
  g.K = (int)d.h;
  g.c = ws.dz;
  g.ldc = d.f;
  g.aux = static_cast<const uint16_t*>(z);
  g.ld_aux = d.f;
  MTL_TRY(gemm_bf16(g, GEMM_DGRAD, EPI_DGELU, s));
  // dw2[e] = a_e^T . dye_e   (K = the expert's rows; K carries N_max for the range check)
  g = grouped(d, GROUP_K, offsets, 0, d.f * d.h);
  g.a = static_cast<const uint16_t*>(a);
  g.lda = d.f;
  g.b = ws.dye;
  g.ldb = d.h;
  g.M = (int)d.f;
  g.N = (int)d.h;
  g.K = (int)d.nmax;
  g.c = dw2;
  g.ldc = d.h;
  MTL_TRY(gemm_bf16(g, GEMM_WGRAD, wepi, s));
  // dw1[e] = xp_e^T . dz_e
  g = grouped(d, GROUP_K, offsets, 0, d.h * d.f);
  g.a = static_cast<const uint16_t*>(xp);
  g.lda = d.h;
  g.b = ws.dz;
  g.ldb = d.f;
  g.M = (int)d.h;
  g.N = (int)d.f;
  g.K = (int)d.nmax;
  g.c = dw1;
  g.ldc = d.f;
  MTL_TRY(gemm_bf16(g, GEMM_WGRAD, wepi, s));
  // dxp = dz_e . w1_e^T into the dye buffer (dye is dead after dw2), then the
  // slot-ordered scatter-add into dx_partial
  uint16_t* dxp = ws.dye;
  g = grouped(d, GROUP_M, offsets, d.h * d.f, 0);
  g.a = ws.dz;
  g.lda = d.f;
  g.b = static_cast<const uint16_t*>(w1);
  g.ldb = d.f;
  g.M = (int)d.nmax;
  g.N = (int)d.h;
  g.K = (int)d.f;
  g.c = dxp;
  g.ldc = d.h;
  MTL_TRY(gemm_bf16(g, GEMM_DGRAD, EPI_BF16, s));
  MTL_TRY(moe_combine(dxp, slot_row, nullptr, (int)d.T, (int)d.k, d.h, static_cast<uint16_t*>(dx_partial), s));
  return MTL_OK;
}

}  // extern "C"
