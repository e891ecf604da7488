// extern "C" entry points of libmtl.so (declared and documented in include/mtl.h):
// configuration checks, scratch carving and the launch sequence of each block.
#include "../../include/mtl.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>

#include "kernels.hpp"
#include "prof.hpp"

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

// Algorithmic FLOP and bytes of the launch groups, for the launch timing
// (prof.hpp): 2*M*N*K per GEMM, every operand element read once and every
// output element written once.
inline double gemm_flop(int64_t M, int64_t N, int64_t K) { return 2.0 * M * N * K; }
inline double gemm_bytes(int64_t M, int64_t N, int64_t K, int in_b, int out_b) {
  return (double)in_b * ((double)M * K + (double)K * N) + (double)out_b * M * N;
}
// causal attention forward: QK^T and PV over the seq*(seq+1)/2 visible pairs
// of every local head and micro-batch element; the backward counts twice that
inline double attn_flop(const mtl_layer_cfg* c, int64_t heads_l, int64_t d) {
  return 4.0 * c->micro_batch * ((double)c->seq * (c->seq + 1) / 2) * d * heads_l;
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

// Bump allocation over a caller's scratch buffer (base == nullptr: sizing only).
struct Bump {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += up(bytes);
    return p;
  }
};

// An fp8 copy of one bf16 tensor [rows, cols]: its scale record {amax, s, 1/s}
// and the row-major codes q and/or the transposed codes qt ([cols, rows]).
struct Q8 {
  float* rec;
  uint8_t* q;
  uint8_t* qt;
  int64_t rows, cols;
  int fmt;
};
Q8 q8(Bump& b, int64_t rows, int64_t cols, int fmt, bool normal, bool trans) {
  Q8 q{};
  q.rec = b.take<float>(16);
  q.q = normal ? b.take<uint8_t>(rows * cols) : nullptr;
  q.qt = trans ? b.take<uint8_t>(rows * cols) : nullptr;
  q.rows = rows;
  q.cols = cols;
  q.fmt = fmt;
  return q;
}
constexpr int E4M3 = 0, E5M2 = 1;
// Capacity (entries) of a buffer of amax stage-1 partials written by a GEMM
// epilogue or the attention kernels, and whether an M x N output fits it: a
// GEMM writes one entry per wave of each tile, at most 4 per 128 x 128 tile.
constexpr int AMAX_PART_CAP = 65536;
inline bool amax_fits(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128) * 4 <= AMAX_PART_CAP; }

// Quantise 1..3 bf16 tensors (x, its Q8) in one amax launch and one cast launch.
// part / nparts: the tensor's amax stage-1 partials, written by the kernel that
// produced it (nullptr: computed here).
struct QIn {
  const void* x;
  const Q8* q;
  const uint32_t* part = nullptr;
  int nparts = 0;
};
hipError_t quantize(std::initializer_list<QIn> in, void* amax_ws, hipStream_t s) {
  QuantJob jobs[3];
  int n = 0;
  double bytes = 0;  // the amax pass and the cast each read the tensor; one byte per code written
  for (const QIn& e : in) {
    if (n == 3) return hipErrorInvalidValue;
    jobs[n++] = QuantJob{static_cast<const uint16_t*>(e.x), e.q->rows, e.q->cols, e.q->fmt, e.q->rec, e.q->q,
                         e.q->qt, e.part, e.nparts};
    bytes += (double)e.q->rows * e.q->cols * ((e.part ? 2 : 4) + (e.q->q ? 1 : 0) + (e.q->qt ? 1 : 0));
  }
  return prof::timed(prof::QUANT, "fp8_quantize", 0, bytes, s, [&] { return fp8_quantize_n(jobs, n, amax_ws, s); });
}

// fp8 GEMM C[M, N] = A . B^T over K, both operands k-contiguous codes.
GemmArgs gemm8_args(const Q8& a, const uint8_t* a_codes, const Q8& b, const uint8_t* b_codes, int64_t M, int64_t N,
                    int64_t K, void* c, int64_t ldc, const void* bias = nullptr, void* c2 = nullptr,
                    const void* aux = nullptr) {
  GemmArgs g{};
  g.a = reinterpret_cast<const uint16_t*>(a_codes);
  g.b = reinterpret_cast<const uint16_t*>(b_codes);
  g.lda = K;
  g.ldb = K;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.c = c;
  g.ldc = ldc;
  g.bias = static_cast<const uint16_t*>(bias);
  g.c2 = c2;
  g.ldc2 = ldc;
  g.aux = static_cast<const uint16_t*>(aux);
  g.ld_aux = ldc;
  g.scale_a = a.rec + 2;
  g.scale_b = b.rec + 2;
  return g;
}
// Where a GEMM's epilogue leaves the amax partials of its bf16 output `out`
// (0: c, 1: c2), and the count it wrote.
struct AmaxOut {
  uint32_t* part = nullptr;
  int out = 0;
  int* nparts = nullptr;
};
inline void set_amax(GemmArgs& g, const AmaxOut& m) {
  g.amax_part = m.part;
  g.amax_out = m.out;
  g.amax_cap = AMAX_PART_CAP;
  g.amax_nparts = m.nparts;
}
hipError_t gemm8(const char* name, const Q8& a, const uint8_t* a_codes, const Q8& b, const uint8_t* b_codes,
                 int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, int epi, hipStream_t s,
                 const void* bias = nullptr, void* c2 = nullptr, const void* aux = nullptr,
                 const AmaxOut& amx = AmaxOut{}, bool keep_cached = false) {
  const int out_b = (epi == EPI_F32 || epi == EPI_F32_ACC) ? 4 : (epi == EPI_BIAS_GELU ? 4 : 2);
  return prof::timed(prof::GEMM, name, gemm_flop(M, N, K), gemm_bytes(M, N, K, 1, out_b), s, [&] {
    GemmArgs g = gemm8_args(a, a_codes, b, b_codes, M, N, K, c, ldc, bias, c2, aux);
    set_amax(g, amx);
    g.keep_cached = keep_cached;
    return gemm_fp8(g, a.fmt, b.fmt, epi, s);
  });
}
// A timed bf16 GEMM (2-byte operands; out_b bytes per output element).
hipError_t gemm16(const char* name, const GemmArgs& g, GemmLayout l, int epi, int out_b, hipStream_t s) {
  return prof::timed(prof::GEMM, name, gemm_flop(g.M, g.N, g.K), gemm_bytes(g.M, g.N, g.K, 2, out_b), s,
                     [&] { return gemm_bf16(g, l, epi, s); });
}
// A timed pair of independent bf16 GEMMs (one launch where a fused kernel exists).
hipError_t gemm16_pair(const char* name, const GemmArgs& g1, GemmLayout l1, int e1, int ob1, const GemmArgs& g2,
                       GemmLayout l2, int e2, int ob2, hipStream_t s) {
  return prof::timed(prof::GEMM, name, gemm_flop(g1.M, g1.N, g1.K) + gemm_flop(g2.M, g2.N, g2.K),
                     gemm_bytes(g1.M, g1.N, g1.K, 2, ob1) + gemm_bytes(g2.M, g2.N, g2.K, 2, ob2), s,
                     [&] { return gemm_bf16_pair(g1, l1, e1, g2, l2, e2, s); });
}
// A timed wgrad beside a dgrad split along its contraction into fp32 parts.
hipError_t gemm16_pair_ksplit(const char* name, const GemmArgs& gw, int ew, const GemmArgs& gd, hipStream_t s) {
  return prof::timed(prof::GEMM, name, gemm_flop(gw.M, gw.N, gw.K) + gemm_flop(gd.M, gd.N, gd.K),
                     gemm_bytes(gw.M, gw.N, gw.K, 2, 4) + gemm_bytes(gd.M, gd.N, gd.K, 2, 4 * gd.ksplit), s,
                     [&] { return gemm_bf16_pair_ksplit(gw, ew, gd, s); });
}
// A timed fp8 wgrad/dgrad pair.
hipError_t gemm8_pair(const char* name, const GemmArgs& gw, int ew, const GemmArgs& gd, int ed, hipStream_t s) {
  return prof::timed(prof::GEMM, name, gemm_flop(gw.M, gw.N, gw.K) + gemm_flop(gd.M, gd.N, gd.K),
                     gemm_bytes(gw.M, gw.N, gw.K, 1, 4) + gemm_bytes(gd.M, gd.N, gd.K, 1, 2), s,
                     [&] { return gemm_fp8_pair(gw, ew, gd, ed, s); });
}

// An MXFP4 copy of one GEMM operand, K-contiguous: codes [rows, k/2] bytes and
// scales (rows * k/32 bytes) in the GEMM's order (k = the GEMM's contraction;
// rows and k are multiples of 256 in the layer).
struct MX4 {
  uint8_t* q;
  uint8_t* s;
  int64_t rows, k;
};
MX4 mx4(Bump& b, int64_t rows, int64_t k) {
  MX4 m{};
  m.q = b.take<uint8_t>(rows * k / 2);
  m.s = b.take<uint8_t>(rows * k / 32);
  m.rows = rows;
  m.k = k;
  return m;
}
inline double mx4_bytes(const MX4& m) { return (double)m.rows * m.k * (2.0 + 0.5 + 1.0 / 32); }
// x [rows, k] quantised along its rows into m ([rows, k])
hipError_t mxq(const void* x, const MX4& m, hipStream_t s) {
  return prof::timed(prof::QUANT, "mx_quantize_rows", 0, mx4_bytes(m), s,
                     [&] { return mxfp4_quantize(static_cast<const uint16_t*>(x), m.rows, m.k, m.q, m.s, s, true); });
}
// x [k, rows] quantised down its columns into m ([rows, k] = x^T)
hipError_t mxqt(const void* x, const MX4& m, hipStream_t s) {
  return prof::timed(prof::QUANT, "mx_quantize_cols", 0, mx4_bytes(m), s,
                     [&] { return mxfp4_quantize_t(static_cast<const uint16_t*>(x), m.k, m.rows, m.q, m.s, s, true); });
}
// x [r, k] quantised both ways from one read: along its rows into m ([r, k])
// and down its columns into mt ([k, r])
hipError_t mxq2(const void* x, const MX4& m, const MX4& mt, hipStream_t s) {
  return prof::timed(prof::QUANT, "mx_quantize_both", 0, mx4_bytes(m) + mx4_bytes(mt) - 2.0 * m.rows * m.k, s, [&] {
    return mxfp4_quantize_both(static_cast<const uint16_t*>(x), m.rows, m.k, m.q, m.s, mt.q, mt.s, s, true);
  });
}
// C [a.rows, b.rows] = A . B^T on MXFP4 codes, epilogue epi (fp32 C for the wgrad epilogues)
Mxfp4GemmArgs mx_args(const MX4& a, const MX4& b, int epi, void* c, const void* bias = nullptr, void* c2 = nullptr,
                      const void* aux = nullptr, bool keep_cached = false) {
  Mxfp4GemmArgs g{};
  g.keep_cached = keep_cached;
  g.a = a.q;
  g.sa = a.s;
  g.b = b.q;
  g.sb = b.s;
  g.M = (int)a.rows;
  g.N = (int)b.rows;
  g.K = (int)a.k;
  g.ldc = b.rows;
  g.epi = epi;
  g.scale_order = 1;
  const bool f32 = epi == EPI_F32 || epi == EPI_F32_ACC;
  if (f32) g.c32 = static_cast<float*>(c);
  else g.c = static_cast<uint16_t*>(c);
  g.bias = static_cast<const uint16_t*>(bias);
  g.c2 = static_cast<uint16_t*>(c2);
  g.aux = static_cast<const uint16_t*>(aux);
  return g;
}
inline double mx_gemm_bytes(const Mxfp4GemmArgs& g) {
  const int out_b = (g.epi == EPI_F32 || g.epi == EPI_F32_ACC) ? 4 : (g.epi == EPI_BIAS_GELU ? 4 : 2);
  return ((double)g.M + g.N) * (g.K / 2.0 + g.K / 32.0) + (double)out_b * g.M * g.N;
}
hipError_t mxgemm(const char* name, const MX4& a, const MX4& b, int epi, void* c, hipStream_t s,
                  const void* bias = nullptr, void* c2 = nullptr, const void* aux = nullptr,
                  bool keep_cached = false) {
  const Mxfp4GemmArgs g = mx_args(a, b, epi, c, bias, c2, aux, keep_cached);
  return prof::timed(prof::GEMM, name, gemm_flop(a.rows, b.rows, a.k), mx_gemm_bytes(g), s,
                     [&] { return gemm_mxfp4_tiled(g, s); });
}
// A timed MXFP4 weight-gradient / data-gradient pair (one launch where both fill the chip).
hipError_t mxgemm_pair(const char* name, const Mxfp4GemmArgs& gw, const Mxfp4GemmArgs& gd, hipStream_t s) {
  return prof::timed(prof::GEMM, name, gemm_flop(gw.M, gw.N, gw.K) + gemm_flop(gd.M, gd.N, gd.K),
                     mx_gemm_bytes(gw) + mx_gemm_bytes(gd), s, [&] { return gemm_mxfp4_pair(gw, gd, s); });
}

struct MlpScratch {
  uint16_t* dz;
  float* ws;
  // fp8 copies
  Q8 dy, w2, a_t, dz8, h_t, w1;
  void* amax_ws;
  uint32_t* dz_part;  // dz's amax partials from the fc2 dgrad epilogue
  // MXFP4 copies
  MX4 m_dy, m_dy_t, m_w2, m_a_t, m_dz, m_dz_t, m_h_t, m_w1;
};
struct AttnScratch {
  uint16_t* dout;
  float* dout_parts;  // the two fp32 halves of dO (proj_bwd_ksplit)
  uint16_t* dqkv;
  float* delta;
  float* ws;
  Q8 dh, wo, o_t, dqkv8, x_t, wqkv;
  void* amax_ws;
  uint32_t* dqkv_part;  // dqkv's amax partials from the attention backward
  MX4 m_dh, m_dh_t, m_wo, m_o_t, m_dqkv, m_dqkv_t, m_x_t, m_wqkv;
};
struct AttnFwdScratch {
  Q8 x, wqkv_t, o, wo_t;
  void* amax_ws;
  uint32_t* o_part;  // o's amax partials from the attention forward
  MX4 m_x, m_wqkv_t, m_o, m_wo_t;
};
struct MlpFwdScratch {
  Q8 h, w1_t, a, w2_t;
  void* amax_ws;
  uint32_t* a_part;  // a's amax partials from the fc1 forward epilogue
  MX4 m_h, m_w1_t, m_a, m_w2_t;
};

inline bool is_fp8(const mtl_layer_cfg* c) { return c->precision == MTL_PREC_FP8_HYBRID; }
inline bool is_mx4(const mtl_layer_cfg* c) { return c->precision == MTL_PREC_MXFP4; }
// The bf16 output projection's backward runs dO = dH . W_o^T in two fp32 halves
// of its contraction (hidden) beside dW_o = O^T . dH, all on 256 x 256 tiles,
// when the data gradient has few output tiles and twice the wgrad's contraction
// or more (hidden >= 1.5 tokens) and the halves with the wgrad fill the chip
// about once; the attention backward's D pass sums the halves.  Otherwise both
// run on 128 x 128 tiles.
inline bool proj_bwd_ksplit(const mtl_layer_cfg* c, const Dims& d) {
  if (is_fp8(c) || is_mx4(c)) return false;
  const int64_t td = ((d.S + 255) / 256) * ((d.o_l + 255) / 256), tw = ((d.o_l + 255) / 256) * ((d.h + 255) / 256);
  return 2 * d.h >= 3 * d.S && td < 240 && tw + 2 * td >= 192 && tw + 2 * td <= 320;
}
inline int proj_bwd_kchunk(const Dims& d) { return (int)(((d.h + 1) / 2 + 63) / 64 * 64); }
inline bool keeps_codes(const mtl_layer_cfg* c) { return is_fp8(c) && (c->flags & MTL_F_KEEP_CODES); }
inline bool keeps_mx(const mtl_layer_cfg* c) { return is_mx4(c) && (c->flags & MTL_F_KEEP_CODES); }
inline bool reuses_weights(const mtl_layer_cfg* c) {
  return (keeps_codes(c) || keeps_mx(c)) && (c->flags & MTL_F_REUSE_WEIGHTS);
}

// With MTL_F_KEEP_CODES, written by the forward calls at the start of the
// scratch and read there by the backward calls, which then do not quantise
// these tensors again (the same tensor and recipe give the same codes):
//  fp8: the transposed E4M3 codes (and scale records) of x, o, h and a, and the
//  four weights' E4M3 codes in both orientations;
//  MXFP4: the column-blocked codes of x, o, h and a (the wgrad operands) and
//  the four weights' codes blocked both ways (the forward's and the dgrad's
//  operands), all from one read of each tensor.
struct Kept {
  Q8 x_t, o_t, h_t, a_t;
  Q8 wqkv, wo, w1, w2;
  MX4 m_x_t, m_o_t, m_h_t, m_a_t;
  MX4 m_wqkv, m_wqkv_t, m_wo, m_wo_t, m_w1, m_w1_t, m_w2, m_w2_t;
};
size_t kept_scratch(const mtl_layer_cfg* c, const Dims& d, Kept* k, char* base) {
  Bump b{base};
  Kept t{};
  if (keeps_codes(c)) {
    t.x_t = q8(b, d.S, d.h, E4M3, false, true);
    t.o_t = q8(b, d.S, d.o_l, E4M3, false, true);
    t.h_t = q8(b, d.S, d.h, E4M3, false, true);
    t.a_t = q8(b, d.S, d.f_l, E4M3, false, true);
    t.wqkv = q8(b, d.h, d.qkv_l, E4M3, true, true);
    t.wo = q8(b, d.o_l, d.h, E4M3, true, true);
    t.w1 = q8(b, d.h, d.f_l, E4M3, true, true);
    t.w2 = q8(b, d.f_l, d.h, E4M3, true, true);
  } else if (keeps_mx(c)) {
    t.m_x_t = mx4(b, d.h, d.S);
    t.m_o_t = mx4(b, d.o_l, d.S);
    t.m_h_t = mx4(b, d.h, d.S);
    t.m_a_t = mx4(b, d.f_l, d.S);
    t.m_wqkv = mx4(b, d.h, d.qkv_l);
    t.m_wqkv_t = mx4(b, d.qkv_l, d.h);
    t.m_wo = mx4(b, d.o_l, d.h);
    t.m_wo_t = mx4(b, d.h, d.o_l);
    t.m_w1 = mx4(b, d.h, d.f_l);
    t.m_w1_t = mx4(b, d.f_l, d.h);
    t.m_w2 = mx4(b, d.f_l, d.h);
    t.m_w2_t = mx4(b, d.h, d.f_l);
  } else {
    return 0;
  }
  if (k) *k = t;
  return b.off;
}
// A forward operand quantised row-major into the call's scratch whose
// transposed copy and record go to the kept region.
inline Q8 with_kept(Q8 q, const Q8& kept) {
  q.rec = kept.rec;
  q.qt = kept.qt;
  return q;
}

size_t mlp_scratch(const mtl_layer_cfg* c, const Dims& d, MlpScratch* s, char* base) {
  Bump b{base};
  MlpScratch t{};
  t.dz = b.take<uint16_t>(d.S * d.f_l * 2);
  t.ws = b.take<float>(colsum_ws_floats(d.S, d.f_l + d.h) * 4);
  if (is_fp8(c)) {
    t.dy = q8(b, d.S, d.h, E5M2, true, true);
    t.w2 = q8(b, d.f_l, d.h, E4M3, true, false);
    t.a_t = q8(b, d.S, d.f_l, E4M3, false, true);
    t.dz8 = q8(b, d.S, d.f_l, E5M2, true, true);
    t.h_t = q8(b, d.S, d.h, E4M3, false, true);
    t.w1 = q8(b, d.h, d.f_l, E4M3, true, false);
    t.amax_ws = b.take<char>(fp8_amax_ws_bytes());
    t.dz_part = b.take<uint32_t>(AMAX_PART_CAP * 4);
  }
  if (is_mx4(c)) {
    t.m_dy = mx4(b, d.S, d.h);
    t.m_dy_t = mx4(b, d.h, d.S);
    t.m_w2 = mx4(b, d.f_l, d.h);
    t.m_a_t = mx4(b, d.f_l, d.S);
    t.m_dz = mx4(b, d.S, d.f_l);
    t.m_dz_t = mx4(b, d.f_l, d.S);
    t.m_h_t = mx4(b, d.h, d.S);
    t.m_w1 = mx4(b, d.h, d.f_l);
  }
  if (s) *s = t;
  return b.off;
}

size_t attn_scratch(const mtl_layer_cfg* c, const Dims& d, AttnScratch* s, char* base) {
  Bump b{base};
  AttnScratch t{};
  t.dout = b.take<uint16_t>(d.S * d.o_l * 2);
  t.dout_parts = proj_bwd_ksplit(c, d) ? b.take<float>(2 * d.S * d.o_l * 4) : nullptr;
  t.dqkv = b.take<uint16_t>(d.S * d.qkv_l * 2);
  t.delta = b.take<float>(d.heads_l * d.S * 4);
  t.ws = b.take<float>(colsum_ws_floats(d.S, d.qkv_l + d.h) * 4);
  if (is_fp8(c)) {
    t.dh = q8(b, d.S, d.h, E5M2, true, true);
    t.wo = q8(b, d.o_l, d.h, E4M3, true, false);
    t.o_t = q8(b, d.S, d.o_l, E4M3, false, true);
    t.dqkv8 = q8(b, d.S, d.qkv_l, E5M2, true, true);
    t.x_t = q8(b, d.S, d.h, E4M3, false, true);
    t.wqkv = q8(b, d.h, d.qkv_l, E4M3, true, false);
    t.amax_ws = b.take<char>(fp8_amax_ws_bytes());
    t.dqkv_part = b.take<uint32_t>(AMAX_PART_CAP * 4);
  }
  if (is_mx4(c)) {
    t.m_dh = mx4(b, d.S, d.h);
    t.m_dh_t = mx4(b, d.h, d.S);
    t.m_wo = mx4(b, d.o_l, d.h);
    t.m_o_t = mx4(b, d.o_l, d.S);
    t.m_dqkv = mx4(b, d.S, d.qkv_l);
    t.m_dqkv_t = mx4(b, d.qkv_l, d.S);
    t.m_x_t = mx4(b, d.h, d.S);
    t.m_wqkv = mx4(b, d.h, d.qkv_l);
  }
  if (s) *s = t;
  return b.off;
}

size_t attn_fwd_scratch(const mtl_layer_cfg* c, const Dims& d, AttnFwdScratch* s, char* base) {
  if (!is_fp8(c) && !is_mx4(c)) return 0;
  Bump b{base};
  AttnFwdScratch t{};
  if (is_fp8(c)) {
    t.x = q8(b, d.S, d.h, E4M3, true, false);
    t.wqkv_t = q8(b, d.h, d.qkv_l, E4M3, false, true);
    t.o = q8(b, d.S, d.o_l, E4M3, true, false);
    t.wo_t = q8(b, d.o_l, d.h, E4M3, false, true);
    t.amax_ws = b.take<char>(fp8_amax_ws_bytes());
    t.o_part = b.take<uint32_t>(AMAX_PART_CAP * 4);
  } else {
    t.m_x = mx4(b, d.S, d.h);
    t.m_wqkv_t = mx4(b, d.qkv_l, d.h);
    t.m_o = mx4(b, d.S, d.o_l);
    t.m_wo_t = mx4(b, d.h, d.o_l);
  }
  if (s) *s = t;
  return b.off;
}

size_t mlp_fwd_scratch(const mtl_layer_cfg* c, const Dims& d, MlpFwdScratch* s, char* base) {
  if (!is_fp8(c) && !is_mx4(c)) return 0;
  Bump b{base};
  MlpFwdScratch t{};
  if (is_fp8(c)) {
    t.h = q8(b, d.S, d.h, E4M3, true, false);
    t.w1_t = q8(b, d.h, d.f_l, E4M3, false, true);
    t.a = q8(b, d.S, d.f_l, E4M3, true, false);
    t.w2_t = q8(b, d.f_l, d.h, E4M3, false, true);
    t.amax_ws = b.take<char>(fp8_amax_ws_bytes());
    t.a_part = b.take<uint32_t>(AMAX_PART_CAP * 4);
  } else {
    t.m_h = mx4(b, d.S, d.h);
    t.m_w1_t = mx4(b, d.f_l, d.h);
    t.m_a = mx4(b, d.S, d.f_l);
    t.m_w2_t = mx4(b, d.h, d.f_l);
  }
  if (s) *s = t;
  return b.off;
}

}  // namespace

namespace mtl {
size_t mlp_bwd_scratch_bytes(const mtl_layer_cfg* c) {
  const Dims d = dims_of(c);
  return mlp_scratch(c, d, nullptr, nullptr);
}
}  // namespace mtl

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
  if (c->precision != MTL_PREC_BF16 && c->precision != MTL_PREC_FP8_HYBRID && c->precision != MTL_PREC_MXFP4)
    return MTL_E_UNSUPPORTED;
  if (c->precision == MTL_PREC_MXFP4) {
    // every M, N of the MX GEMMs a multiple of 128 and every K of 256
    const Dims d = dims_of(c);
    for (int64_t v : {d.S, d.h, d.o_l, d.qkv_l, d.f_l})
      if (v % 256 != 0) return MTL_E_SHAPE;
    // the column-direction quantiser's grid takes at most 2^23 rows (S, h, h/t or f/t)
    if (std::max({d.S, d.h, d.o_l, d.f_l}) > ((int64_t)1 << 23)) return MTL_E_SHAPE;
  }
  // fp8 GEMMs contract over 16-byte code chunks: every K (h, 3h/t, h/t, f/t, S)
  // must be a multiple of 16
  if (c->precision == MTL_PREC_FP8_HYBRID &&
      (((int64_t)c->seq * c->micro_batch) % 16 != 0 || (c->ffn / c->tp) % 16 != 0))
    return MTL_E_SHAPE;
  if (c->flags & ~(MTL_F_RESIDUAL | MTL_F_WGRAD_ACCUM | MTL_F_KEEP_CODES | MTL_F_REUSE_WEIGHTS))
    return MTL_E_UNSUPPORTED;
  if ((c->flags & MTL_F_KEEP_CODES) && c->precision != MTL_PREC_FP8_HYBRID && c->precision != MTL_PREC_MXFP4)
    return MTL_E_UNSUPPORTED;
  if ((c->flags & MTL_F_REUSE_WEIGHTS) && !(c->flags & MTL_F_KEEP_CODES)) return MTL_E_UNSUPPORTED;
  return MTL_OK;
}

mtl_status mtl_workspace_bytes(const mtl_layer_cfg* c, size_t* scratch_bytes) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if (!scratch_bytes) return MTL_E_NULL;
  const Dims d = dims_of(c);
  *scratch_bytes = kept_scratch(c, d, nullptr, nullptr) +
                   std::max({mlp_scratch(c, d, nullptr, nullptr), attn_scratch(c, d, nullptr, nullptr),
                             attn_fwd_scratch(c, d, nullptr, nullptr), mlp_fwd_scratch(c, d, nullptr, nullptr)});
  return MTL_OK;
}

mtl_status mtl_attn_fwd(const mtl_layer_cfg* c, const void* x, const void* w_qkv, const void* b_qkv, const void* w_o,
                        void* qkv, void* o, float* lse, void* partial, void* scratch, size_t scratch_bytes,
                        mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(x, w_qkv, b_qkv, w_o, qkv, o, lse, partial)) != MTL_OK) return st;
  const Dims d = dims_of(c);
  AttnFwdScratch ws{};
  Kept kp{};
  if (is_fp8(c) || is_mx4(c)) {
    if ((st = check_ptrs(scratch)) != MTL_OK) return st;
    const size_t kb = kept_scratch(c, d, &kp, static_cast<char*>(scratch));
    if (scratch_bytes < kb || scratch_bytes - kb < attn_fwd_scratch(c, d, &ws, static_cast<char*>(scratch) + kb))
      return MTL_E_WORKSPACE;
    if (keeps_codes(c)) {
      ws.x = with_kept(ws.x, kp.x_t);
      ws.o = with_kept(ws.o, kp.o_t);
      ws.wqkv_t = kp.wqkv;  // the forward's cast writes both orientations
      ws.wo_t = kp.wo;
    }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  // qkv = x . w_qkv + b_qkv
  if (keeps_mx(c)) {  // x and w_qkv both ways; the backward takes the other blocking
    MTL_TRY(mxq2(x, ws.m_x, kp.m_x_t, s));
    if (!reuses_weights(c)) MTL_TRY(mxq2(w_qkv, kp.m_wqkv, kp.m_wqkv_t, s));
    MTL_TRY(mxgemm("qkv_fwd", ws.m_x, kp.m_wqkv_t, EPI_BF16_BIAS, qkv, s, b_qkv, nullptr, nullptr, true));
  } else if (is_mx4(c)) {
    MTL_TRY(mxq(x, ws.m_x, s));
    MTL_TRY(mxqt(w_qkv, ws.m_wqkv_t, s));
    MTL_TRY(mxgemm("qkv_fwd", ws.m_x, ws.m_wqkv_t, EPI_BF16_BIAS, qkv, s, b_qkv, nullptr, nullptr, true));
  } else if (is_fp8(c)) {
    if (reuses_weights(c)) MTL_TRY(quantize({{x, &ws.x}}, ws.amax_ws, s));
    else MTL_TRY(quantize({{x, &ws.x}, {w_qkv, &ws.wqkv_t}, {w_o, &ws.wo_t}}, ws.amax_ws, s));
    MTL_TRY(gemm8("qkv_fwd", ws.x, ws.x.q, ws.wqkv_t, ws.wqkv_t.qt, d.S, d.qkv_l, d.h, qkv, d.qkv_l, EPI_BF16_BIAS,
                  s, b_qkv, nullptr, nullptr, AmaxOut{}, true));  // the attention reads qkv next
  } else {
    GemmArgs g = gemm(x, d.h, w_qkv, d.qkv_l, d.S, d.qkv_l, d.h, qkv, d.qkv_l);
    g.bias = static_cast<const uint16_t*>(b_qkv);
    g.keep_cached = 1;  // the attention reads qkv next
    MTL_TRY(gemm16("qkv_fwd", g, GEMM_FWD, EPI_BF16_BIAS, 2, s));
  }

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
  int no = 0;  // fp8: the attention kernel leaves o's amax partials
  if (is_fp8(c)) {
    a.amax_part = ws.o_part;
    a.amax_cap = AMAX_PART_CAP;
    a.amax_nparts = &no;
  }
  MTL_TRY(prof::timed(prof::ATTN, "attn_fwd", attn_flop(c, d.heads_l, d.d),
                      2.0 * d.S * (d.qkv_l + d.o_l) + 4.0 * d.S * d.heads_l, s, [&] { return attention_fwd(a, s); }));

  // partial = o . w_o
  if (keeps_mx(c)) {
    MTL_TRY(mxq2(o, ws.m_o, kp.m_o_t, s));
    if (!reuses_weights(c)) MTL_TRY(mxq2(w_o, kp.m_wo, kp.m_wo_t, s));
    MTL_TRY(mxgemm("proj_fwd", ws.m_o, kp.m_wo_t, EPI_BF16, partial, s));
  } else if (is_mx4(c)) {
    MTL_TRY(mxq(o, ws.m_o, s));
    MTL_TRY(mxqt(w_o, ws.m_wo_t, s));
    MTL_TRY(mxgemm("proj_fwd", ws.m_o, ws.m_wo_t, EPI_BF16, partial, s));
  } else if (is_fp8(c)) {
    MTL_TRY(quantize({{o, &ws.o, ws.o_part, no}}, ws.amax_ws, s));
    MTL_TRY(gemm8("proj_fwd", ws.o, ws.o.q, ws.wo_t, ws.wo_t.qt, d.S, d.h, d.o_l, partial, d.h, EPI_BF16, s));
  } else {
    GemmArgs g = gemm(o, d.o_l, w_o, d.h, d.S, d.h, d.o_l, partial, d.h);
    MTL_TRY(gemm16("proj_fwd", g, GEMM_FWD, EPI_BF16, 2, s));
  }
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
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const double n = (double)(row_end - row_begin) * cols;
  const double bytes = 2.0 * n * (t + 1 + (residual ? 1 : 0)) + (bias ? 2.0 * cols : 0.0);
  return hip_status(prof::timed(prof::REDUCE, "reduce", 0, bytes, s, [&] {
    return reduce_partials(t, p, static_cast<const uint16_t*>(bias), static_cast<const uint16_t*>(residual),
                           static_cast<uint16_t*>(out), cols, row_begin, row_end, s);
  }));
}

mtl_status mtl_allgather_rows(int32_t t, int32_t rank, const void* const* bufs, void* out, int64_t rows, int64_t cols,
                              mtl_stream_t stream) {
  if (!bufs || !out) return MTL_E_NULL;
  if (t < 1 || t > 16 || rows <= 0 || cols <= 0 || cols % 8 != 0 || rows % t != 0) return MTL_E_SHAPE;
  if (rank < 0 || rank >= t) return MTL_E_RANK;
  if (!aligned16(out)) return MTL_E_ALIGN;
  const uint16_t* p[16] = {};
  for (int i = 0; i < t; ++i) {
    if (i == rank) continue;  // the caller's own share is already in place and is not read
    if (!bufs[i]) return MTL_E_NULL;
    if (!aligned16(bufs[i])) return MTL_E_ALIGN;
    if (bufs[i] == out) return MTL_E_UNSUPPORTED;
    p[i] = static_cast<const uint16_t*>(bufs[i]);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const double bytes = 2.0 * 2.0 * (double)(rows - rows / t) * cols;  // t-1 shares read and written
  return hip_status(prof::timed(prof::GATHER, "allgather", 0, bytes, s, [&] {
    return allgather_rows(t, rank, p, static_cast<uint16_t*>(out), rows, cols, s);
  }));
}

static mtl_status cp_check(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim) {
  if (cp < 1 || cp > MTL_CP_MAX) return MTL_E_SHAPE;
  if (rank < 0 || rank >= cp) return MTL_E_RANK;
  if (chunk <= 0 || chunk > INT32_MAX || chunk % 64 != 0 || heads <= 0 || (head_dim != 64 && head_dim != 128))
    return MTL_E_SHAPE;
  // the kernels address a chunk's QKV through 32-bit buffer offsets; the row
  // width is bounded first so that the byte-range product cannot wrap
  const int64_t row_bytes = (int64_t)3 * heads * head_dim * 2;
  if (row_bytes > (int64_t)INT32_MAX) return MTL_E_SHAPE;
  if (chunk + 64 > (int64_t)UINT32_MAX / row_bytes) return MTL_E_SHAPE;
  return MTL_OK;
}

// One partial (O_j, L_j) per key chunk the rank's queries see; none for rank 0.
static size_t cp_slot_o(int64_t chunk, int32_t heads, int32_t head_dim) { return up(chunk * heads * head_dim * 2); }
static size_t cp_slot_l(int64_t chunk, int32_t heads) { return up(chunk * heads * 4); }

mtl_status mtl_cp_attn_scratch_bytes(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                                     size_t* scratch_bytes) {
  mtl_status st = cp_check(cp, rank, chunk, heads, head_dim);
  if (st != MTL_OK) return st;
  if (!scratch_bytes) return MTL_E_NULL;
  *scratch_bytes = rank == 0 ? 0 : (size_t)(rank + 1) * (cp_slot_o(chunk, heads, head_dim) + cp_slot_l(chunk, heads));
  return MTL_OK;
}

mtl_status mtl_cp_attn_fwd(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                           const void* const* qkv_chunks, void* o, float* lse, void* scratch, size_t scratch_bytes,
                           mtl_stream_t stream) {
  mtl_status st = cp_check(cp, rank, chunk, heads, head_dim);
  if (st != MTL_OK) return st;
  if (!qkv_chunks) return MTL_E_NULL;
  for (int j = 0; j <= rank; ++j)
    if ((st = check_ptrs(qkv_chunks[j])) != MTL_OK) return st;
  if ((st = check_ptrs(o, lse)) != MTL_OK) return st;
  size_t need = 0;
  mtl_cp_attn_scratch_bytes(cp, rank, chunk, heads, head_dim, &need);
  if (need) {
    if ((st = check_ptrs(scratch)) != MTL_OK) return st;
    if (scratch_bytes < need) return MTL_E_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  AttnArgs a{};
  a.ld_qkv = 3 * (int64_t)heads * head_dim;
  a.ld_o = (int64_t)heads * head_dim;
  a.seq = (int)chunk;
  a.batch = 1;
  a.heads = heads;
  a.d = head_dim;
  a.scale = 1.0f / sqrtf((float)head_dim);
  a.qkv = static_cast<const uint16_t*>(qkv_chunks[rank]);
  if (rank == 0) {  // the first chunk sees only itself
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    return hip_status(attention_fwd(a, s));
  }
  // ring order: the rank's own chunk (causal), then chunks rank-1, ..., 0 as
  // they would arrive from the previous rank (every key visible); chunks
  // after the rank are masked out entirely and take no work
  const size_t so = cp_slot_o(chunk, heads, head_dim), sl = cp_slot_l(chunk, heads);
  char* base = static_cast<char*>(scratch);
  uint16_t* o_parts = reinterpret_cast<uint16_t*>(base);
  float* l_parts = reinterpret_cast<float*>(base + (size_t)(rank + 1) * so);
  for (int k = 0; k <= rank; ++k) {
    a.o = reinterpret_cast<uint16_t*>(base + (size_t)k * so);
    a.lse = reinterpret_cast<float*>(base + (size_t)(rank + 1) * so + (size_t)k * sl);
    if (k == 0) {
      MTL_TRY(attention_fwd(a, s));
    } else {
      a.kv = static_cast<const uint16_t*>(qkv_chunks[rank - k]);
      a.kv_seq = (int)chunk;
      MTL_TRY(attention_fwd_full(a, s));
    }
  }
  CpMergeArgs m{};
  m.o_parts = o_parts;
  m.lse_parts = l_parts;
  m.o_stride = (int64_t)(so / 2);
  m.lse_stride = (int64_t)(sl / 4);
  m.nparts = rank + 1;
  m.tokens = chunk;
  m.heads = heads;
  m.d = head_dim;
  m.o = static_cast<uint16_t*>(o);
  m.lse = lse;
  return hip_status(cp_merge(m, s));
}

// D = rowsum(dO * O) of the rank's queries, then one dQ partial per earlier chunk.
mtl_status mtl_cp_attn_bwd_scratch_bytes(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                                         size_t* scratch_bytes) {
  mtl_status st = cp_check(cp, rank, chunk, heads, head_dim);
  if (st != MTL_OK) return st;
  if (!scratch_bytes) return MTL_E_NULL;
  *scratch_bytes = cp_slot_l(chunk, heads) + (size_t)rank * cp_slot_o(chunk, heads, head_dim);
  return MTL_OK;
}

mtl_status mtl_cp_attn_bwd(int32_t cp, int32_t rank, int64_t chunk, int32_t heads, int32_t head_dim,
                           const void* const* qkv_chunks, const void* o, const float* lse, const void* dout,
                           void* dqkv, void* const* dkv_chunks, void* scratch, size_t scratch_bytes,
                           mtl_stream_t stream) {
  mtl_status st = cp_check(cp, rank, chunk, heads, head_dim);
  if (st != MTL_OK) return st;
  if (!qkv_chunks || (rank > 0 && !dkv_chunks)) return MTL_E_NULL;
  for (int j = 0; j <= rank; ++j)
    if ((st = check_ptrs(qkv_chunks[j])) != MTL_OK) return st;
  for (int j = 0; j < rank; ++j) {
    if ((st = check_ptrs(dkv_chunks[j])) != MTL_OK) return st;
    if (dkv_chunks[j] == dqkv) return MTL_E_UNSUPPORTED;
  }
  if ((st = check_ptrs(o, lse, dout, dqkv, scratch)) != MTL_OK) return st;
  size_t need = 0;
  mtl_cp_attn_bwd_scratch_bytes(cp, rank, chunk, heads, head_dim, &need);
  if (scratch_bytes < need) return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(scratch);
  const size_t so = cp_slot_o(chunk, heads, head_dim);
  uint16_t* dq_parts = reinterpret_cast<uint16_t*>(base + cp_slot_l(chunk, heads));
  AttnArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv_chunks[rank]);
  a.ld_qkv = 3 * (int64_t)heads * head_dim;
  a.ld_o = (int64_t)heads * head_dim;
  a.seq = (int)chunk;
  a.batch = 1;
  a.heads = heads;
  a.d = head_dim;
  a.scale = 1.0f / sqrtf((float)head_dim);
  a.dout = static_cast<const uint16_t*>(dout);
  a.out = static_cast<const uint16_t*>(o);
  a.lse_in = lse;
  a.delta = reinterpret_cast<float*>(base);
  a.dqkv = static_cast<uint16_t*>(dqkv);
  // the rank's own chunk (causal; also computes D), then chunks rank-1, ..., 0
  // in ring order: dK, dV of chunk j to dkv_chunks[j], dQ to a partial
  MTL_TRY(attention_bwd(a, s));
  for (int k = 1; k <= rank; ++k) {
    a.kv = static_cast<const uint16_t*>(qkv_chunks[rank - k]);
    a.kv_seq = (int)chunk;
    a.dkv = static_cast<uint16_t*>(dkv_chunks[rank - k]);
    a.dq = reinterpret_cast<uint16_t*>(base + cp_slot_l(chunk, heads) + (size_t)(k - 1) * so);
    MTL_TRY(attention_bwd_full(a, s));
  }
  if (rank == 0) return MTL_OK;
  CpDqSumArgs q{};
  q.dqkv = static_cast<uint16_t*>(dqkv);
  q.parts = dq_parts;
  q.part_stride = (int64_t)(so / 2);
  q.nparts = rank;
  q.tokens = chunk;
  q.heads = heads;
  q.d = head_dim;
  return hip_status(cp_dq_sum(q, s));
}

mtl_status mtl_mxfp4_quantize(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                              mtl_stream_t stream) {
  mtl_status st = check_ptrs(x, codes, scales);
  if (st != MTL_OK) return st;
  if (rows <= 0 || cols <= 0 || cols % 32 != 0 || rows > INT32_MAX || cols > INT32_MAX) return MTL_E_SHAPE;
  return hip_status(mxfp4_quantize(static_cast<const uint16_t*>(x), rows, cols, static_cast<uint8_t*>(codes),
                                   static_cast<uint8_t*>(scales), reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_mxfp4_gemm(int64_t M, int64_t N, int64_t K, const void* a_codes, const void* a_scales,
                          const void* b_codes, const void* b_scales, void* c, int64_t ldc, mtl_stream_t stream) {
  mtl_status st = check_ptrs(a_codes, a_scales, b_codes, b_scales, c);
  if (st != MTL_OK) return st;
  if (M <= 0 || N <= 0 || K <= 0 || M % 128 || N % 128 || K % 256 || ldc < N || ldc % 8) return MTL_E_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MTL_E_SHAPE;
  Mxfp4GemmArgs g{};
  g.a = static_cast<const uint8_t*>(a_codes);
  g.sa = static_cast<const uint8_t*>(a_scales);
  g.b = static_cast<const uint8_t*>(b_codes);
  g.sb = static_cast<const uint8_t*>(b_scales);
  g.c = static_cast<uint16_t*>(c);
  g.ldc = ldc;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  return hip_status(gemm_mxfp4_tiled(g, reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_mxfp4_quantize_t(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                                mtl_stream_t stream) {
  mtl_status st = check_ptrs(x, codes, scales);
  if (st != MTL_OK) return st;
  if (rows <= 0 || cols <= 0 || rows % 32 != 0 || cols % 8 != 0 || rows > ((int64_t)1 << 23) || cols > INT32_MAX)
    return MTL_E_SHAPE;
  return hip_status(mxfp4_quantize_t(static_cast<const uint16_t*>(x), rows, cols, static_cast<uint8_t*>(codes),
                                     static_cast<uint8_t*>(scales), reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_mxfp6_quantize(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                              mtl_stream_t stream) {
  mtl_status st = check_ptrs(x, codes, scales);
  if (st != MTL_OK) return st;
  if (rows <= 0 || cols <= 0 || cols % 32 != 0 || rows > INT32_MAX || cols > INT32_MAX) return MTL_E_SHAPE;
  return hip_status(mxfp6_quantize(static_cast<const uint16_t*>(x), rows, cols, static_cast<uint8_t*>(codes),
                                   static_cast<uint8_t*>(scales), reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_mxfp6_gemm(int64_t M, int64_t N, int64_t K, const void* a_codes, const void* a_scales,
                          const void* b_codes, const void* b_scales, void* c, int64_t ldc, mtl_stream_t stream) {
  mtl_status st = check_ptrs(a_codes, a_scales, b_codes, b_scales, c);
  if (st != MTL_OK) return st;
  if (M <= 0 || N <= 0 || K <= 0 || M % 128 || N % 128 || K % 128 || ldc < N || ldc % 8) return MTL_E_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MTL_E_SHAPE;
  Mxfp4GemmArgs g{};
  g.a = static_cast<const uint8_t*>(a_codes);
  g.sa = static_cast<const uint8_t*>(a_scales);
  g.b = static_cast<const uint8_t*>(b_codes);
  g.sb = static_cast<const uint8_t*>(b_scales);
  g.c = static_cast<uint16_t*>(c);
  g.ldc = ldc;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  return hip_status(mxfp6_gemm(g, reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_mx_quantize_ordered(int32_t elem, const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                                   int32_t order, mtl_stream_t stream) {
  mtl_status st = check_ptrs(x, codes, scales);
  if (st != MTL_OK) return st;
  if (elem != MTL_MX_E2M1 && elem != MTL_MX_E2M3) return MTL_E_UNSUPPORTED;
  if (order != MTL_MX_ORDER_PLAIN && order != MTL_MX_ORDER_GEMM) return MTL_E_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || cols % 32 != 0 || rows > INT32_MAX || cols > INT32_MAX) return MTL_E_SHAPE;
  const bool go = order == MTL_MX_ORDER_GEMM;
  if (go && (rows % 32 || cols % 256)) return MTL_E_SHAPE;
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* q = static_cast<uint8_t*>(codes);
  auto* sc = static_cast<uint8_t*>(scales);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return hip_status(elem == MTL_MX_E2M1 ? mxfp4_quantize(xs, rows, cols, q, sc, s, go)
                                        : mxfp6_quantize(xs, rows, cols, q, sc, s, go));
}

mtl_status mtl_mx_gemm_ordered(int32_t elem, int64_t M, int64_t N, int64_t K, const void* a_codes,
                               const void* a_scales, const void* b_codes, const void* b_scales, void* c, int64_t ldc,
                               int32_t order, mtl_stream_t stream) {
  mtl_status st = check_ptrs(a_codes, a_scales, b_codes, b_scales, c);
  if (st != MTL_OK) return st;
  if (elem != MTL_MX_E2M1 && elem != MTL_MX_E2M3) return MTL_E_UNSUPPORTED;
  if (order != MTL_MX_ORDER_PLAIN && order != MTL_MX_ORDER_GEMM) return MTL_E_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || ldc < N || ldc % 8) return MTL_E_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MTL_E_SHAPE;
  if (order == MTL_MX_ORDER_GEMM ? (M % 32 || N % 32 || K % 256)
                                 : (M % 128 || N % 128 || K % (elem == MTL_MX_E2M1 ? 256 : 128)))
    return MTL_E_SHAPE;
  Mxfp4GemmArgs g{};
  g.a = static_cast<const uint8_t*>(a_codes);
  g.sa = static_cast<const uint8_t*>(a_scales);
  g.b = static_cast<const uint8_t*>(b_codes);
  g.sb = static_cast<const uint8_t*>(b_scales);
  g.c = static_cast<uint16_t*>(c);
  g.ldc = ldc;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.scale_order = order;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (elem == MTL_MX_E2M1) return hip_status(gemm_mxfp4_tiled(g, s));
  return hip_status(order == MTL_MX_ORDER_GEMM ? gemm_mxfp6_tiled(g, s) : mxfp6_gemm(g, s));
}

mtl_status mtl_mlp_fwd(const mtl_layer_cfg* c, const void* h, const void* w1, const void* b1, const void* w2, void* gz,
                       void* a, void* partial, void* scratch, size_t scratch_bytes, mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(h, w1, b1, w2, gz, a, partial)) != MTL_OK) return st;
  const Dims d = dims_of(c);
  MlpFwdScratch ws{};
  Kept kp{};
  if (is_fp8(c) || is_mx4(c)) {
    if ((st = check_ptrs(scratch)) != MTL_OK) return st;
    const size_t kb = kept_scratch(c, d, &kp, static_cast<char*>(scratch));
    if (scratch_bytes < kb || scratch_bytes - kb < mlp_fwd_scratch(c, d, &ws, static_cast<char*>(scratch) + kb))
      return MTL_E_WORKSPACE;
    if (keeps_codes(c)) {
      ws.h = with_kept(ws.h, kp.h_t);
      ws.a = with_kept(ws.a, kp.a_t);
      ws.w1_t = kp.w1;  // the forward's cast writes both orientations
      ws.w2_t = kp.w2;
    }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  if (keeps_mx(c)) {  // as below, keeping the other blocking of h, a and the weights for the backward
    MTL_TRY(mxq2(h, ws.m_h, kp.m_h_t, s));
    if (!reuses_weights(c)) MTL_TRY(mxq2(w1, kp.m_w1, kp.m_w1_t, s));
    MTL_TRY(mxgemm("fc1_fwd", ws.m_h, kp.m_w1_t, EPI_BIAS_GELU, gz, s, b1, a));
    MTL_TRY(mxq2(a, ws.m_a, kp.m_a_t, s));
    if (!reuses_weights(c)) MTL_TRY(mxq2(w2, kp.m_w2, kp.m_w2_t, s));
    MTL_TRY(mxgemm("fc2_fwd", ws.m_a, kp.m_w2_t, EPI_BF16, partial, s));
    return MTL_OK;
  }
  if (is_mx4(c)) {
    // z = h . w1 + b1: gz = GeLU'(z), a = GeLU(z); partial = a . w2
    MTL_TRY(mxq(h, ws.m_h, s));
    MTL_TRY(mxqt(w1, ws.m_w1_t, s));
    MTL_TRY(mxgemm("fc1_fwd", ws.m_h, ws.m_w1_t, EPI_BIAS_GELU, gz, s, b1, a));
    MTL_TRY(mxq(a, ws.m_a, s));
    MTL_TRY(mxqt(w2, ws.m_w2_t, s));
    MTL_TRY(mxgemm("fc2_fwd", ws.m_a, ws.m_w2_t, EPI_BF16, partial, s));
    return MTL_OK;
  }

  if (is_fp8(c)) {
    // z = h . w1 + b1: gz = GeLU'(z), a = GeLU(z); partial = a . w2 (a re-quantised from bf16)
    if (reuses_weights(c)) MTL_TRY(quantize({{h, &ws.h}}, ws.amax_ws, s));
    else MTL_TRY(quantize({{h, &ws.h}, {w1, &ws.w1_t}, {w2, &ws.w2_t}}, ws.amax_ws, s));
    // the fc1 epilogue leaves a's amax partials, so a's quantisation reads it once
    int na = 0;
    const AmaxOut am = amax_fits(d.S, d.f_l) ? AmaxOut{ws.a_part, 1, &na} : AmaxOut{};
    MTL_TRY(gemm8("fc1_fwd", ws.h, ws.h.q, ws.w1_t, ws.w1_t.qt, d.S, d.f_l, d.h, gz, d.f_l, EPI_BIAS_GELU, s, b1,
                  a, nullptr, am));
    MTL_TRY(quantize({{a, &ws.a, am.part, na}}, ws.amax_ws, s));
    MTL_TRY(gemm8("fc2_fwd", ws.a, ws.a.q, ws.w2_t, ws.w2_t.qt, d.S, d.h, d.f_l, partial, d.h, EPI_BF16, s));
    return MTL_OK;
  }
  GemmArgs g = gemm(h, d.h, w1, d.f_l, d.S, d.f_l, d.h, gz, d.f_l);
  g.bias = static_cast<const uint16_t*>(b1);
  g.c2 = a;
  g.ldc2 = d.f_l;
  MTL_TRY(gemm16("fc1_fwd", g, GEMM_FWD, EPI_BIAS_GELU, 4, s));  // two bf16 outputs: GeLU'(z) and GeLU(z)

  g = gemm(a, d.f_l, w2, d.h, d.S, d.h, d.f_l, partial, d.h);
  MTL_TRY(gemm16("fc2_fwd", g, GEMM_FWD, EPI_BF16, 2, s));
  return MTL_OK;
}

// db1 = colsum(dz) and, when wanted, db2 = colsum(dy): one pair of launches.
static hipError_t mlp_bias_grads(const Dims& d, const MlpScratch& ws, const void* dy, float* db1, float* db2,
                                 bool accum, hipStream_t s) {
  const ColsumJob jobs[2] = {{ws.dz, d.f_l, db1}, {static_cast<const uint16_t*>(dy), d.h, db2}};
  const double bytes = 2.0 * d.S * (d.f_l + (db2 ? d.h : 0)) + 4.0 * (d.f_l + (db2 ? d.h : 0));
  return prof::timed(prof::COLSUM, "colsum_mlp", 0, bytes, s,
                     [&] { return colsum_bf16(jobs, db2 ? 2 : 1, d.S, accum, ws.ws, s); });
}

// db_qkv = colsum(dqkv) and, when wanted, db_o = colsum(dh): one pair of launches.
static hipError_t attn_bias_grads(const Dims& d, const AttnScratch& ws, const void* dh, float* db_qkv,
                                  float* db_o, bool accum, hipStream_t s) {
  const ColsumJob jobs[2] = {{ws.dqkv, d.qkv_l, db_qkv}, {static_cast<const uint16_t*>(dh), d.h, db_o}};
  const double bytes = 2.0 * d.S * (d.qkv_l + (db_o ? d.h : 0)) + 4.0 * (d.qkv_l + (db_o ? d.h : 0));
  return prof::timed(prof::COLSUM, "colsum_attn", 0, bytes, s,
                     [&] { return colsum_bf16(jobs, db_o ? 2 : 1, d.S, accum, ws.ws, s); });
}

mtl_status mtl_mlp_bwd(const mtl_layer_cfg* c, const void* dy, const void* h, const void* gz, const void* a,
                       const void* w1, const void* w2, void* dh_partial, float* dw1, float* db1, float* dw2,
                       float* db2, void* scratch, size_t scratch_bytes, mtl_stream_t stream) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(dy, h, gz, a, w1, w2, dh_partial, dw1, db1, dw2, scratch)) != MTL_OK) return st;
  if (db2 && !aligned16(db2)) return MTL_E_ALIGN;
  const Dims d = dims_of(c);
  MlpScratch ws;
  Kept kp{};
  const size_t kb = kept_scratch(c, d, &kp, static_cast<char*>(scratch));
  if (scratch_bytes < kb || scratch_bytes - kb < mlp_scratch(c, d, &ws, static_cast<char*>(scratch) + kb))
    return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool accum = (c->flags & MTL_F_WGRAD_ACCUM) != 0;
  const int wepi = accum ? EPI_F32_ACC : EPI_F32;

  if (is_mx4(c)) {
    // every operand quantised along its product's contraction (with
    // MTL_F_KEEP_CODES the weights' and a's, h's codes come from mtl_mlp_fwd)
    const bool kept = keeps_mx(c);
    MTL_TRY(mxq2(dy, ws.m_dy, ws.m_dy_t, s));
    if (kept) ws.m_w2 = kp.m_w2;
    else MTL_TRY(mxq(w2, ws.m_w2, s));
    // each wgrad with its dgrad in one launch
    if (kept) ws.m_a_t = kp.m_a_t;
    else MTL_TRY(mxqt(a, ws.m_a_t, s));
    MTL_TRY(mxgemm_pair("fc2_bwd", mx_args(ws.m_a_t, ws.m_dy_t, wepi, dw2),
                        mx_args(ws.m_dy, ws.m_w2, EPI_DGELU, ws.dz, nullptr, nullptr, gz), s));
    MTL_TRY(mxq2(ws.dz, ws.m_dz, ws.m_dz_t, s));
    if (kept) ws.m_w1 = kp.m_w1;
    else MTL_TRY(mxq(w1, ws.m_w1, s));
    if (kept) ws.m_h_t = kp.m_h_t;
    else MTL_TRY(mxqt(h, ws.m_h_t, s));
    MTL_TRY(mxgemm_pair("fc1_bwd", mx_args(ws.m_h_t, ws.m_dz_t, wepi, dw1),
                        mx_args(ws.m_dz, ws.m_w1, EPI_BF16, dh_partial), s));
    MTL_TRY(mlp_bias_grads(d, ws, dy, db1, db2, accum, s));
    return MTL_OK;
  }
  if (is_fp8(c)) {
    // E5M2 gradients, E4M3 activations and weights; wgrad operands transposed
    if (keeps_codes(c)) {  // a's transposed codes and w2's codes come from mtl_mlp_fwd
      ws.a_t = kp.a_t;
      ws.w2 = kp.w2;
      MTL_TRY(quantize({{dy, &ws.dy}}, ws.amax_ws, s));
    } else {
      MTL_TRY(quantize({{dy, &ws.dy}, {w2, &ws.w2}, {a, &ws.a_t}}, ws.amax_ws, s));
    }
    // dw2 = a^T . dy with dz = (dy . w2^T) * gz in one launch, then dw1 = h^T . dz with dh_partial = dz . w1^T;
    // the dgrad epilogue leaves dz's amax partials
    int nz = 0;
    const AmaxOut az = amax_fits(d.S, d.f_l) ? AmaxOut{ws.dz_part, 0, &nz} : AmaxOut{};
    GemmArgs gdz = gemm8_args(ws.dy, ws.dy.q, ws.w2, ws.w2.q, d.S, d.f_l, d.h, ws.dz, d.f_l, nullptr, nullptr, gz);
    set_amax(gdz, az);
    MTL_TRY(gemm8_pair("fc2_bwd", gemm8_args(ws.a_t, ws.a_t.qt, ws.dy, ws.dy.qt, d.f_l, d.h, d.S, dw2, d.h), wepi,
                       gdz, EPI_DGELU, s));
    if (keeps_codes(c)) {  // and h's and w1's
      ws.h_t = kp.h_t;
      ws.w1 = kp.w1;
      MTL_TRY(quantize({{ws.dz, &ws.dz8, az.part, nz}}, ws.amax_ws, s));
    } else {
      MTL_TRY(quantize({{ws.dz, &ws.dz8, az.part, nz}, {h, &ws.h_t}, {w1, &ws.w1}}, ws.amax_ws, s));
    }
    MTL_TRY(gemm8_pair("fc1_bwd", gemm8_args(ws.h_t, ws.h_t.qt, ws.dz8, ws.dz8.qt, d.h, d.f_l, d.S, dw1, d.f_l), wepi,
                       gemm8_args(ws.dz8, ws.dz8.q, ws.w1, ws.w1.q, d.S, d.h, d.f_l, dh_partial, d.h), EPI_BF16, s));
    MTL_TRY(mlp_bias_grads(d, ws, dy, db1, db2, accum, s));
    return MTL_OK;
  }
  // dz = (dy . w2^T) * gz, gz = GeLU'(z), with the independent dw2 = a^T . dy in the same
  // launch; the wgrad tiles go first, so their fp32 output drains under the
  // dgrad tiles' main loops
  GemmArgs g = gemm(dy, d.h, w2, d.h, d.S, d.f_l, d.h, ws.dz, d.f_l);
  g.aux = static_cast<const uint16_t*>(gz);
  g.ld_aux = d.f_l;
  GemmArgs g2 = gemm(a, d.f_l, dy, d.h, d.f_l, d.h, d.S, dw2, d.h);
  MTL_TRY(gemm16_pair("fc2_bwd", g2, GEMM_WGRAD, wepi, 4, g, GEMM_DGRAD, EPI_DGELU, 2, s));
  MTL_TRY(mlp_bias_grads(d, ws, dy, db1, db2, accum, s));
  // dw1 = h^T . dz and dh_partial = dz . w1^T
  g = gemm(h, d.h, ws.dz, d.f_l, d.h, d.f_l, d.S, dw1, d.f_l);
  g2 = gemm(ws.dz, d.f_l, w1, d.f_l, d.S, d.h, d.f_l, dh_partial, d.h);
  MTL_TRY(gemm16_pair("fc1_bwd", g, GEMM_WGRAD, wepi, 4, g2, GEMM_DGRAD, EPI_BF16, 2, s));
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
  Kept kp{};
  const size_t kb = kept_scratch(c, d, &kp, static_cast<char*>(scratch));
  if (scratch_bytes < kb || scratch_bytes - kb < attn_scratch(c, d, &ws, static_cast<char*>(scratch) + kb))
    return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool accum = (c->flags & MTL_F_WGRAD_ACCUM) != 0;
  const int wepi = accum ? EPI_F32_ACC : EPI_F32;
  const bool f8 = is_fp8(c);

  if (is_mx4(c)) {
    MTL_TRY(mxq2(dh, ws.m_dh, ws.m_dh_t, s));
    if (keeps_mx(c)) ws.m_wo = kp.m_wo;  // with o's column-blocked codes, from mtl_attn_fwd
    else MTL_TRY(mxq(w_o, ws.m_wo, s));
    if (keeps_mx(c)) ws.m_o_t = kp.m_o_t;
    else MTL_TRY(mxqt(o, ws.m_o_t, s));
    MTL_TRY(mxgemm_pair("proj_bwd", mx_args(ws.m_o_t, ws.m_dh_t, wepi, dw_o),
                        mx_args(ws.m_dh, ws.m_wo, EPI_BF16, ws.dout), s));
  } else if (f8) {
    // do = dh . w_o^T ; dw_o = o^T . dh
    if (keeps_codes(c)) {  // o's transposed codes and w_o's codes come from mtl_attn_fwd
      ws.o_t = kp.o_t;
      ws.wo = kp.wo;
      MTL_TRY(quantize({{dh, &ws.dh}}, ws.amax_ws, s));
    } else {
      MTL_TRY(quantize({{dh, &ws.dh}, {w_o, &ws.wo}, {o, &ws.o_t}}, ws.amax_ws, s));
    }
    MTL_TRY(gemm8_pair("proj_bwd", gemm8_args(ws.o_t, ws.o_t.qt, ws.dh, ws.dh.qt, d.o_l, d.h, d.S, dw_o, d.h), wepi,
                       gemm8_args(ws.dh, ws.dh.q, ws.wo, ws.wo.q, d.S, d.o_l, d.h, ws.dout, d.o_l), EPI_BF16, s));
  } else if (proj_bwd_ksplit(c, d)) {
    // dw_o = o^T . dh beside the two halves (over hidden) of do = dh . w_o^T in fp32
    GemmArgs g = gemm(dh, d.h, w_o, d.h, d.S, d.o_l, d.h, ws.dout_parts, d.o_l);
    g.ksplit = 2;
    g.k_chunk = proj_bwd_kchunk(d);
    g.split_stride_c = d.S * d.o_l;
    GemmArgs g2 = gemm(o, d.o_l, dh, d.h, d.o_l, d.h, d.S, dw_o, d.h);
    MTL_TRY(gemm16_pair_ksplit("proj_bwd", g2, wepi, g, s));
  } else {
    // dw_o = o^T . dh and do = dh . w_o^T, one launch (wgrad tiles first)
    GemmArgs g = gemm(dh, d.h, w_o, d.h, d.S, d.o_l, d.h, ws.dout, d.o_l);
    GemmArgs g2 = gemm(o, d.o_l, dh, d.h, d.o_l, d.h, d.S, dw_o, d.h);
    MTL_TRY(gemm16_pair("proj_bwd", g2, GEMM_WGRAD, wepi, 4, g, GEMM_DGRAD, EPI_BF16, 2, s));
  }

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
  if (!is_fp8(c) && !is_mx4(c) && proj_bwd_ksplit(c, d)) {  // D's pass forms dO from the halves
    at.dout_parts = ws.dout_parts;
    at.dout_part_stride = d.S * d.o_l;
    at.dout_w = ws.dout;
  }
  at.out = static_cast<const uint16_t*>(o);
  at.lse_in = lse;
  at.delta = ws.delta;
  at.dqkv = ws.dqkv;
  int nq = 0;  // fp8: the attention backward leaves dqkv's amax partials
  if (f8) {
    at.amax_part = ws.dqkv_part;
    at.amax_cap = AMAX_PART_CAP;
    at.amax_nparts = &nq;
  }
  // reads qkv, o, dO and lse; writes dqkv (D = rowsum(dO * O) on the way)
  MTL_TRY(prof::timed(prof::ATTN, "attn_bwd", 2.0 * attn_flop(c, d.heads_l, d.d),
                      2.0 * d.S * (2 * d.qkv_l + 2 * d.o_l) + 4.0 * d.S * d.heads_l, s,
                      [&] { return attention_bwd(at, s); }));

  if (is_mx4(c)) {
    MTL_TRY(mxq2(ws.dqkv, ws.m_dqkv, ws.m_dqkv_t, s));
    if (keeps_mx(c)) ws.m_wqkv = kp.m_wqkv;  // with x's column-blocked codes, from mtl_attn_fwd
    else MTL_TRY(mxq(w_qkv, ws.m_wqkv, s));
    if (keeps_mx(c)) ws.m_x_t = kp.m_x_t;
    else MTL_TRY(mxqt(x, ws.m_x_t, s));
    MTL_TRY(mxgemm_pair("qkv_bwd", mx_args(ws.m_x_t, ws.m_dqkv_t, wepi, dw_qkv),
                        mx_args(ws.m_dqkv, ws.m_wqkv, EPI_BF16, dx_partial), s));
    MTL_TRY(attn_bias_grads(d, ws, dh, db_qkv, db_o, accum, s));
    return MTL_OK;
  }
  if (f8) {
    // dw_qkv = x^T . dqkv ; dx_partial = dqkv . w_qkv^T
    if (keeps_codes(c)) {  // and x's and w_qkv's
      ws.x_t = kp.x_t;
      ws.wqkv = kp.wqkv;
      MTL_TRY(quantize({{ws.dqkv, &ws.dqkv8, ws.dqkv_part, nq}}, ws.amax_ws, s));
    } else {
      MTL_TRY(quantize({{ws.dqkv, &ws.dqkv8, ws.dqkv_part, nq}, {x, &ws.x_t}, {w_qkv, &ws.wqkv}}, ws.amax_ws, s));
    }
    MTL_TRY(gemm8_pair("qkv_bwd",
                       gemm8_args(ws.x_t, ws.x_t.qt, ws.dqkv8, ws.dqkv8.qt, d.h, d.qkv_l, d.S, dw_qkv, d.qkv_l), wepi,
                       gemm8_args(ws.dqkv8, ws.dqkv8.q, ws.wqkv, ws.wqkv.q, d.S, d.h, d.qkv_l, dx_partial, d.h),
                       EPI_BF16, s));
    MTL_TRY(attn_bias_grads(d, ws, dh, db_qkv, db_o, accum, s));
    return MTL_OK;
  }
  // dw_qkv = x^T . dqkv and dx_partial = dqkv . w_qkv^T, one launch; then
  // db_qkv = colsum(dqkv) and db_o = colsum(dh)
  GemmArgs g = gemm(x, d.h, ws.dqkv, d.qkv_l, d.h, d.qkv_l, d.S, dw_qkv, d.qkv_l);
  GemmArgs g2 = gemm(ws.dqkv, d.qkv_l, w_qkv, d.qkv_l, d.S, d.h, d.qkv_l, dx_partial, d.h);
  MTL_TRY(gemm16_pair("qkv_bwd", g, GEMM_WGRAD, wepi, 4, g2, GEMM_DGRAD, EPI_BF16, 2, s));
  MTL_TRY(attn_bias_grads(d, ws, dh, db_qkv, db_o, accum, s));
  return MTL_OK;
}

mtl_status mtl_attn_bwd_scratch_layout(const mtl_layer_cfg* c, size_t* do_offset, size_t* dqkv_offset) {
  mtl_status st = mtl_validate(c);
  if (st != MTL_OK) return st;
  if (!do_offset || !dqkv_offset) return MTL_E_NULL;
  // the same carving as mtl_attn_bwd, over a base address of 0
  AttnScratch ws;
  const size_t kb = kept_scratch(c, dims_of(c), nullptr, nullptr);
  attn_scratch(c, dims_of(c), &ws, reinterpret_cast<char*>(ALIGN));
  *do_offset = kb + (size_t)(reinterpret_cast<char*>(ws.dout) - reinterpret_cast<char*>(ALIGN));
  *dqkv_offset = kb + (size_t)(reinterpret_cast<char*>(ws.dqkv) - reinterpret_cast<char*>(ALIGN));
  return MTL_OK;
}

// ---------------------------------------------------------------- fp8 scaling

mtl_status mtl_fp8_amax(const void* x, int64_t n, int32_t format, float* rec, void* scratch, size_t scratch_bytes,
                        mtl_stream_t stream) {
  mtl_status st = check_ptrs(x, rec, scratch);
  if (st != MTL_OK) return st;
  if (n <= 0) return MTL_E_SHAPE;
  if (format != MTL_FP8_E4M3 && format != MTL_FP8_E5M2) return MTL_E_UNSUPPORTED;
  if (scratch_bytes < fp8_amax_ws_bytes()) return MTL_E_WORKSPACE;
  return hip_status(fp8_amax(static_cast<const uint16_t*>(x), n, format, rec, scratch,
                             reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_fp8_cast(const void* x, int64_t rows, int64_t cols, int32_t format, const float* rec, void* out,
                        void* out_t, mtl_stream_t stream) {
  mtl_status st = check_ptrs(x, rec);
  if (st != MTL_OK) return st;
  if (!out && !out_t) return MTL_E_NULL;
  if ((out && !aligned16(out)) || (out_t && !aligned16(out_t))) return MTL_E_ALIGN;
  if (rows <= 0 || cols <= 0 || cols % 8 != 0 || (out_t && rows % 16 != 0)) return MTL_E_SHAPE;
  if (format != MTL_FP8_E4M3 && format != MTL_FP8_E5M2) return MTL_E_UNSUPPORTED;
  return hip_status(fp8_cast(static_cast<const uint16_t*>(x), rows, cols, format, rec, static_cast<uint8_t*>(out),
                             static_cast<uint8_t*>(out_t), reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_fp8_quantize(const void* x, int64_t rows, int64_t cols, int32_t format, float* rec, void* out,
                            void* out_t, void* scratch, size_t scratch_bytes, mtl_stream_t stream) {
  mtl_status st = check_ptrs(x, rec, scratch);
  if (st != MTL_OK) return st;
  if (!out && !out_t) return MTL_E_NULL;
  if ((out && !aligned16(out)) || (out_t && !aligned16(out_t))) return MTL_E_ALIGN;
  if (rows <= 0 || cols <= 0 || cols % 8 != 0 || (out_t && rows % 16 != 0)) return MTL_E_SHAPE;
  if (format != MTL_FP8_E4M3 && format != MTL_FP8_E5M2) return MTL_E_UNSUPPORTED;
  if (scratch_bytes < fp8_amax_ws_bytes()) return MTL_E_WORKSPACE;
  const QuantJob job{static_cast<const uint16_t*>(x), rows, cols, format, rec, static_cast<uint8_t*>(out),
                     static_cast<uint8_t*>(out_t)};
  return hip_status(fp8_quantize_n(&job, 1, scratch, reinterpret_cast<hipStream_t>(stream)));
}

mtl_status mtl_fp8_gemm(int64_t M, int64_t N, int64_t K, const void* a, int32_t fmt_a, const float* a_rec,
                        const void* b, int32_t fmt_b, const float* b_rec, const void* bias, void* c, int64_t ldc,
                        mtl_stream_t stream) {
  mtl_status st = check_ptrs(a, a_rec, b, b_rec, c);
  if (st != MTL_OK) return st;
  if (bias && !aligned16(bias)) return MTL_E_ALIGN;
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 || ldc < N || ldc % 8) return MTL_E_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MTL_E_SHAPE;
  if ((M + 256) * K >= ((int64_t)1 << 32) || (N + 256) * K >= ((int64_t)1 << 32)) return MTL_E_SHAPE;
  int epi;
  if (fmt_a == MTL_FP8_E4M3 && fmt_b == MTL_FP8_E4M3) epi = bias ? EPI_BF16_BIAS : EPI_BF16;
  else if (fmt_a == MTL_FP8_E5M2 && fmt_b == MTL_FP8_E4M3 && !bias) epi = EPI_BF16;
  else if (fmt_a == MTL_FP8_E4M3 && fmt_b == MTL_FP8_E5M2 && !bias) epi = EPI_F32;
  else return MTL_E_UNSUPPORTED;
  GemmArgs g{};
  g.a = static_cast<const uint16_t*>(a);
  g.b = static_cast<const uint16_t*>(b);
  g.lda = K;
  g.ldb = K;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.c = c;
  g.ldc = ldc;
  g.bias = static_cast<const uint16_t*>(bias);
  g.scale_a = a_rec + 2;
  g.scale_b = b_rec + 2;
  return hip_status(gemm_fp8(g, fmt_a, fmt_b, epi, reinterpret_cast<hipStream_t>(stream)));
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

// The router GEMMs address x [T, h] and w_r [h, E] with 32-bit byte offsets.
static mtl_status router_check(const mtl_moe_cfg* c) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  if (c->experts % 8 != 0) return MTL_E_SHAPE;
  const int64_t T = c->tokens, h = c->hidden, E = c->experts;
  if ((T + 256) * h * 2 >= ((int64_t)1 << 32) || (h + 256) * E * 2 >= ((int64_t)1 << 32) ||
      (T + 256) * E * 2 >= ((int64_t)1 << 32))
    return MTL_E_SHAPE;
  return MTL_OK;
}

mtl_status mtl_moe_router_fwd(const mtl_moe_cfg* c, const void* x, const void* w_r, float* logits,
                              mtl_stream_t stream) {
  mtl_status st = router_check(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(x, w_r, logits)) != MTL_OK) return st;
  const int64_t T = c->tokens, h = c->hidden, E = c->experts;
  return hip_status(gemm_bf16(gemm(x, h, w_r, E, T, E, h, logits, E), GEMM_FWD, EPI_F32,
                              reinterpret_cast<hipStream_t>(stream)));
}

// Router backward scratch: dlogits in bf16 [T, E], counts [E] int32, q [T] fp32.
static size_t router_scratch(const mtl_moe_cfg* c, uint16_t** dl16, int32_t** counts, float** q, char* base) {
  Bump b{base};
  uint16_t* a = b.take<uint16_t>((int64_t)c->tokens * c->experts * 2);
  int32_t* n = b.take<int32_t>((int64_t)c->experts * 4);
  float* r = b.take<float>((int64_t)c->tokens * 4);
  if (dl16) *dl16 = a;
  if (counts) *counts = n;
  if (q) *q = r;
  return b.off;
}

mtl_status mtl_moe_router_sizes(const mtl_moe_cfg* c, size_t* scratch_bytes) {
  mtl_status st = router_check(c);
  if (st != MTL_OK) return st;
  if (scratch_bytes) *scratch_bytes = router_scratch(c, nullptr, nullptr, nullptr, nullptr);
  return MTL_OK;
}

mtl_status mtl_moe_router_bwd(const mtl_moe_cfg* c, const void* x, const void* w_r, const float* logits,
                              const int32_t* topk_idx, const float* gates, const float* dgates, float aux_coeff,
                              float* aux_loss, float* dlogits, float* dw_r, void* dx, void* scratch,
                              size_t scratch_bytes, mtl_stream_t stream) {
  mtl_status st = router_check(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(x, w_r, logits, topk_idx, gates, dgates, dlogits, dw_r, dx, scratch)) != MTL_OK) return st;
  if (!(aux_coeff >= 0.f) || aux_coeff == INFINITY) return MTL_E_SHAPE;
  uint16_t* dl16;
  int32_t* counts;
  float* q;
  if (scratch_bytes < router_scratch(c, &dl16, &counts, &q, static_cast<char*>(scratch))) return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t T = c->tokens, h = c->hidden, E = c->experts;
  MTL_TRY(moe_router_bwd(logits, topk_idx, gates, dgates, (int)T, (int)E, c->topk, aux_coeff, counts, q, aux_loss,
                         dlogits, dl16, s));
  // dw_r = x^T . dlogits and dx = dlogits . w_r^T, on the bf16 rounding of dlogits
  const int wepi = (c->flags & MTL_F_WGRAD_ACCUM) ? EPI_F32_ACC : EPI_F32;
  MTL_TRY(gemm_bf16_pair(gemm(x, h, dl16, E, h, E, T, dw_r, E), GEMM_WGRAD, wepi,
                         gemm(dl16, E, w_r, E, T, h, E, dx, h), GEMM_DGRAD, EPI_BF16, s));
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
                       const int32_t* slot_row, const float* gates, const void* w1, const void* w2, void* xp, void* gz,
                       void* a, void* ye, void* y_partial, mtl_stream_t stream) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(x, offsets, perm_token, slot_row, gates, w1, w2, xp, gz, a, ye, y_partial)) != MTL_OK) return st;
  const MoeDims d = moe_dims(c);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  // (MoE launch groups are timed without FLOP or bytes: the row counts that
  // fix them live on the device)
  MTL_TRY(prof::timed(prof::GATHER, "moe_gather", 0, 0, s, [&] {
    return moe_gather(static_cast<const uint16_t*>(x), perm_token, offsets, (int)d.El, d.nmax, d.h,
                      static_cast<uint16_t*>(xp), s);
  }));
  // z = xp_e . w1_e: gz = GeLU'(z), a = GeLU(z)   (the grid covers N_max rows; M carries N_max)
  GemmArgs g = grouped(d, GROUP_M, offsets, d.h * d.f, 0);
  g.a = static_cast<const uint16_t*>(xp);
  g.lda = d.h;
  g.b = static_cast<const uint16_t*>(w1);
  g.ldb = d.f;
  g.M = (int)d.nmax;
  g.N = (int)d.f;
  g.K = (int)d.h;
  g.c = gz;
  g.ldc = d.f;
  g.c2 = a;
  g.ldc2 = d.f;
  MTL_TRY(prof::timed(prof::GEMM, "moe_fc1_fwd", 0, 0, s, [&] { return gemm_bf16(g, GEMM_FWD, EPI_BIAS_GELU, s); }));
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
  MTL_TRY(prof::timed(prof::GEMM, "moe_fc2_fwd", 0, 0, s, [&] { return gemm_bf16(g, GEMM_FWD, EPI_BF16, s); }));
  MTL_TRY(prof::timed(prof::GATHER, "moe_combine", 0, 0, s, [&] {
    return moe_combine(static_cast<const uint16_t*>(ye), slot_row, gates, (int)d.T, (int)d.k, d.h,
                       static_cast<uint16_t*>(y_partial), s);
  }));
  return MTL_OK;
}

mtl_status mtl_moe_bwd(const mtl_moe_cfg* c, const void* dy, const int32_t* offsets, const int32_t* perm_token,
                       const int32_t* perm_slot, const int32_t* slot_row, const float* gates, const void* xp,
                       const void* gz, const void* a, const void* ye, const void* w1, const void* w2, void* dx_partial,
                       float* dw1, float* dw2, float* dgates, void* scratch, size_t scratch_bytes,
                       mtl_stream_t stream) {
  mtl_status st = mtl_moe_validate(c);
  if (st != MTL_OK) return st;
  if ((st = check_ptrs(dy, offsets, perm_token, perm_slot, slot_row, gates, xp, gz, a, ye, w1, w2, dx_partial, dw1,
                       dw2, dgates, scratch)) != MTL_OK)
    return st;
  const MoeDims d = moe_dims(c);
  MoeScratch ws;
  if (scratch_bytes < moe_scratch(d, &ws, static_cast<char*>(scratch))) return MTL_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int wepi = (c->flags & MTL_F_WGRAD_ACCUM) ? EPI_F32_ACC : EPI_F32;

  MTL_TRY(prof::timed(prof::GATHER, "moe_combine_bwd", 0, 0, s, [&] {
    return moe_combine_bwd(static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ye), perm_token, perm_slot,
                           slot_row, offsets, (int)d.El, d.nmax, gates, (int)d.T, (int)d.k, d.h, ws.dye, dgates, s);
  }));
  // dz = (dye_e . w2_e^T) * gz, gz = GeLU'(z)
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
  g.aux = static_cast<const uint16_t*>(gz);
  g.ld_aux = d.f;
  MTL_TRY(prof::timed(prof::GEMM, "moe_fc2_dgrad", 0, 0, s, [&] { return gemm_bf16(g, GEMM_DGRAD, EPI_DGELU, s); }));
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
  MTL_TRY(prof::timed(prof::GEMM, "moe_fc2_wgrad", 0, 0, s, [&] { return gemm_bf16(g, GEMM_WGRAD, wepi, s); }));
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
  MTL_TRY(prof::timed(prof::GEMM, "moe_fc1_wgrad", 0, 0, s, [&] { return gemm_bf16(g, GEMM_WGRAD, wepi, s); }));
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
  MTL_TRY(prof::timed(prof::GEMM, "moe_fc1_dgrad", 0, 0, s, [&] { return gemm_bf16(g, GEMM_DGRAD, EPI_BF16, s); }));
  MTL_TRY(prof::timed(prof::GATHER, "moe_scatter", 0, 0, s, [&] {
    return moe_combine(dxp, slot_row, nullptr, (int)d.T, (int)d.k, d.h, static_cast<uint16_t*>(dx_partial), s);
  }));
  return MTL_OK;
}

}  // extern "C"
