// Causal multi-head attention, backward, for gfx950 (the forward is in
// attn_fwd.hip).
//
// Operation (per head n, per micro-batch element): S = Q K^T * scale with key
// j > query i masked, P = row-softmax(S), O = P V; the row log-sum-exp L is
// saved.  Backward: D_i = sum(dO_i * O_i); P is recomputed from L; dV = P^T dO,
// dP = dO V^T, dS = P * (dP - D), dQ = dS K * scale, dK = dS^T Q * scale.
//
// Layout: Q, K, V of head n are columns [n*3d, n*3d+d), [+d, +2d), [+2d, +3d) of
// the head-interleaved QKV tensor; O is [tokens, heads*d].
//
// CDNA4 design.  All products use v_mfma_f32_32x32x16_bf16.  Where the softmax
// is a row operation the scores are formed transposed (S^T = K Q^T): a lane then
// owns one query and 16 of the 32 keys of a block, so row max / row sum are
// in-register reductions plus one exchange with lane l^32, and the bf16 P values
// in the accumulator registers are directly the "b" operand of the next MFMA
// (the k-slot order of that MFMA is chosen to match the accumulator layout).
// The "a" operand that pairs with them (V^T, K^T, Q^T or dO^T) is read straight
// from the natural-layout tile with ds_read_b64_tr_b16.  Tiles arrive by LDS
// DMA (buffer_load ... lds) in their global layout, with swizzles that keep
// every access pattern free of bank conflicts on the 64-bank LDS.  Causal work
// is balanced by pairing mirrored blocks inside a workgroup; the backward is one
// fused deterministic pass (no floating-point atomics, bit-identical run to run).
#include "common.hpp"
#include "kernels.hpp"

namespace mtl {

constexpr float LOG2E = 1.4426950408889634f;

// b-operand from registers r = 8*half .. 8*half+7 of an fp32 32x32 accumulator.
__device__ __forceinline__ u32x4 pack_half(const f32x16& p, int half) {
  const int o = half * 8;
  return u32x4{pack_bf16x2(p[o + 0], p[o + 1]), pack_bf16x2(p[o + 2], p[o + 3]), pack_bf16x2(p[o + 4], p[o + 5]),
               pack_bf16x2(p[o + 6], p[o + 7])};
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32); }

// ============================================================== backward: D
// delta[n][tok] = sum_i dO[tok][n*d+i] * O[tok][n*d+i]; eight lanes per
// (token, head) row, each taking d/8 elements in 16-byte loads.  With dO in two
// fp32 parts, the pass first forms dO = bf16(part 0 + part 1) and stores it.
template <int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(AttnArgs a) {
  constexpr int V = D / 64;  // 16-byte vectors per lane and tensor (1 or 2)
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int sub = threadIdx.x & 7;
  const int64_t tokens = (int64_t)a.seq * a.batch;
  const bool ok = row < tokens * a.heads;
  const int64_t tok = ok ? row / a.heads : 0;
  const int n = ok ? (int)(row % a.heads) : 0;
  float acc = 0.f;
  if (ok) {
    const int64_t e0 = tok * a.ld_o + (int64_t)n * D + sub * V * 8;  // this lane's first element
    const u32x4* po = reinterpret_cast<const u32x4*>(a.out + e0);
    u32x4 vo[V], vd[V];
    if (a.dout_parts) {
      const f32x4* p0 = reinterpret_cast<const f32x4*>(a.dout_parts + e0);
      const f32x4* p1 = reinterpret_cast<const f32x4*>(a.dout_parts + a.dout_part_stride + e0);
      f32x4 x[2 * V], y[2 * V];
#pragma unroll
      for (int i = 0; i < 2 * V; ++i) {  // read once
        x[i] = __builtin_nontemporal_load(p0 + i);
        y[i] = __builtin_nontemporal_load(p1 + i);
      }
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const f32x4 s0 = x[2 * i] + y[2 * i], s1 = x[2 * i + 1] + y[2 * i + 1];
        vd[i] = u32x4{pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]), pack_bf16x2(s1[0], s1[1]),
                      pack_bf16x2(s1[2], s1[3])};
        reinterpret_cast<u32x4*>(a.dout_w + e0)[i] = vd[i];
      }
    } else {
      const u32x4* pd = reinterpret_cast<const u32x4*>(a.dout + e0);
#pragma unroll
      for (int i = 0; i < V; ++i) vd[i] = pd[i];
    }
#pragma unroll
    for (int i = 0; i < V; ++i) vo[i] = __builtin_nontemporal_load(po + i);
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc += bf16_lo(vo[i][j]) * bf16_lo(vd[i][j]) + bf16_hi(vo[i][j]) * bf16_hi(vd[i][j]);
  }
#pragma unroll
  for (int off = 4; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (ok && sub == 0) a.delta[(int64_t)n * tokens + tok] = acc;
}

// ============================================================== backward
// One fused, balanced, deterministic pass.  Workgroup w (4 waves) computes
//   part 1: dK and dV of key block w (64 keys), over query blocks w .. n-1;
//   part 2: dQ of query block w (64 queries), over key blocks 0 .. w;
// (n - w) + (w + 1) = n + 1 block steps for every workgroup.  Each 64 x 64 block
// step is split in 32 x 32 quarters over the waves; the two partial sums of each
// output quarter are added through LDS at the end of a part (fixed order, no
// atomics).  One LDS stage of <= 65 KB and <= 256 VGPRs let two workgroups share
// a CU.  Tiles arrive by LDS DMA in their global layout; Q, dO and K tiles are
// read both row-wise (ds_read_b128) and transposed (ds_read_b64_tr_b16).
template <int D>
struct BwdTiles {
  static constexpr int RB = 2 * D;
  static constexpr int TILE = 64 * RB;
  static constexpr int PER_TILE = TILE / 1024;
  // one swizzle that keeps both access patterns bank-conflict free on 64 banks
  static __device__ __forceinline__ int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // DMA of ntiles 64-row tiles: tile i = rows [row0, row0+64) of column block
  // cols[i] of src[i] (row stride ld[i]) into dst + i*TILE.
  static __device__ __forceinline__ void load(int ntiles, const i32x4* rs, const int64_t* ld, const int64_t* col,
                                              int64_t row0, LDS_AS char* dst) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per_wave = ntiles * PER_TILE / 4;
    for (int q = 0; q < per_wave; ++q) {
      const int I = wave * per_wave + q;
      const int t = I / PER_TILE;
      const int o = (I % PER_TILE) * 1024 + lane * 16;
      const int row = o / RB;
      const int c = ((o % RB) >> 4) ^ swz(row);
      const uint32_t voff = (uint32_t)(((row0 + row) * ld[t] + col[t] + c * 8) * 2);
      dma16(rs[t], voff, 0u, lds_addr(dst + I * 1024));
    }
  }
  // The same DMA of two tiles in a loop over block steps: PW instructions per
  // wave; lane_off is the lane's part of the byte offset of instruction q (row
  // and column chunk within tile t = I / PER_TILE, plus the tile's column
  // block), the same at every step; the step adds the uniform row0 * ld[t] * 2.
  static constexpr int PW = 2 * PER_TILE / 4;
  static __device__ __forceinline__ uint32_t lane_off(const int64_t* ld, const int64_t* col, int q) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int I = wave * PW + q;
    const int t = I / PER_TILE;
    const int o = (I % PER_TILE) * 1024 + lane * 16;
    const int row = o / RB;
    const int c = ((o % RB) >> 4) ^ swz(row);
    return (uint32_t)((row * ld[t] + col[t] + c * 8) * 2);
  }
  static __device__ __forceinline__ void load2(const i32x4* rs, const uint32_t (&lo)[PW], const uint32_t* step,
                                               LDS_AS char* dst) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int q = 0; q < PW; ++q) {
      const int I = wave * PW + q;
      const int t = I / PER_TILE;
      dma16(rs[t], lo[q] + step[t], 0u, lds_addr(dst + I * 1024));
    }
  }
  // row fragment: rows row0 + l%32, 8 columns of k step ks
  static __device__ __forceinline__ u32x4 rfrag(const LDS_AS char* t, int row0, int ks, int lane) {
    const int row = row0 + (lane & 31);
    const int c = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const LDS_AS u32x4*>(t + row * RB + ((c ^ swz(row)) << 4));
  }
  // transposed fragment: rows = columns i*32 + l%32 of the tile; k slots = tile
  // rows r0 + ks*16 + 8*(j/4) + 4*(l/32) + j%4 (a 32x32 accumulator's row order)
  static __device__ __forceinline__ u32x4 tfrag(const LDS_AS char* t, int r0, int i, int ks, int lane) {
    const int G = lane >> 4, R = (lane >> 2) & 3, c4 = lane & 3;
    const int row = r0 + ks * 16 + 4 * (G >> 1) + R;
    const int col = i * 32 + (G & 1) * 16 + 4 * c4;
    const int off = ((col & 7) >> 2) * 8;
    const u32x2 lo = read_tr(t + row * RB + (((col >> 3) ^ swz(row)) << 4) + off);
    const u32x2 hi = read_tr(t + (row + 8) * RB + (((col >> 3) ^ swz(row + 8)) << 4) + off);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

// FULL: the queries of a.qkv (with their dO, LSE and D) against every key of a
// separate chunk a.kv of the same length, no mask; dK and dV go to the key
// columns of a.dkv (the chunk's layout), dQ to a.dq ([tokens, heads*d], stride
// ld_o).  Otherwise causal self-attention of a.qkv into a.dqkv.
template <int D, bool FULL>
__global__ __launch_bounds__(256, 2) void attn_bwd_kernel(AttnArgs a) {
  using T = BwdTiles<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  // part 1: [K | V | Q | dO] tiles + LSE, D; part 2: [K | V] tiles
  __shared__ __attribute__((aligned(1024))) char sm_[4 * T::TILE + 2 * 64 * 4];
  LDS_AS char* sm = (LDS_AS char*)sm_;
  LDS_AS char* tK = sm;
  LDS_AS char* tV = sm + T::TILE;
  LDS_AS char* tQ = sm + 2 * T::TILE;
  LDS_AS char* tO = sm + 3 * T::TILE;
  float* sl = reinterpret_cast<float*>(sm_ + 4 * T::TILE);  // [0,64) lse*log2e, [64,128) delta

  // one work unit = (block w, head, batch element), a head's units on one XCD
  const int nblk = (a.seq + 63) / 64;
  const int u = xcd_index(blockIdx.x, nblk * a.heads * a.batch);
  const int w = u % nblk, n = (u / nblk) % a.heads, b = u / (nblk * a.heads);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int tid = threadIdx.x;
  const int64_t tokens = (int64_t)a.seq * a.batch;
  const int64_t tok0 = (int64_t)b * a.seq;
  const int64_t colq = (int64_t)n * 3 * D, colo = (int64_t)n * D;
  const float c = a.scale * LOG2E;
  uint32_t amx = 0;  // largest bf16 magnitude of dQKV this wave stores
  const i32x4 rq = make_rsrc(a.qkv, (uint32_t)(tokens * a.ld_qkv * 2));
  const i32x4 ro = make_rsrc(a.dout, (uint32_t)(tokens * a.ld_o * 2));
  // K and V tiles: the resource rk from token ktok0 (FULL: kv_seq == seq)
  const i32x4 rk = FULL ? make_rsrc(a.kv, (uint32_t)(tokens * a.ld_qkv * 2)) : rq;
  const int64_t ktok0 = tok0;
  const float* lse = a.lse_in + (int64_t)n * tokens + tok0;
  const float* dlt = a.delta + (int64_t)n * tokens + tok0;

  // ---------------------------------------------------------------- part 1
  {
    const int kh = wave & 1, qh = wave >> 1;
    const int k0 = w * 64;
    const int kw = k0 + kh * 32;
    const int key = kw + (lane & 31);
    {
      const i32x4 rs[2] = {rk, rk};
      const int64_t ld[2] = {a.ld_qkv, a.ld_qkv};
      const int64_t col[2] = {colq + D, colq + 2 * D};
      T::load(2, rs, ld, col, ktok0 + k0, tK);
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      dk[i] = f32x16{};
      dv[i] = f32x16{};
    }
    const i32x4 rs_qo[2] = {rq, ro};
    const int64_t ld_qo[2] = {a.ld_qkv, a.ld_o};
    uint32_t lo_qo[T::PW];
    {
      const int64_t col[2] = {colq, colo};
#pragma unroll
      for (int q = 0; q < T::PW; ++q) lo_qo[q] = T::lane_off(ld_qo, col, q);
    }
    for (int qb = FULL ? 0 : w; qb < nblk; ++qb) {
      const int q0 = qb * 64;
      {
        const uint32_t step[2] = {(uint32_t)((tok0 + q0) * ld_qo[0] * 2), (uint32_t)((tok0 + q0) * ld_qo[1] * 2)};
        T::load2(rs_qo, lo_qo, step, tQ);
      }
      if (tid < 128) {
        const int qq = q0 + (tid & 63);
        sl[tid] = qq < a.seq ? (tid < 64 ? lse[qq] * LOG2E : dlt[qq]) : 0.f;
      }
      wait_dma();
      __syncthreads();
      const int qw = q0 + qh * 32;
      if (FULL || qw + 31 >= kw) {
        // S[q][key], dP[q][key]: rows = this wave's 32 queries, column = key
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sc = mfma32(T::rfrag(tQ, qh * 32, ks, lane), T::rfrag(tK, kh * 32, ks, lane), sc);
          dp = mfma32(T::rfrag(tO, qh * 32, ks, lane), T::rfrag(tV, kh * 32, ks, lane), dp);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int ql = qh * 32 + 8 * r4 + 4 * g;  // local query of registers 4*r4 ..
          const f32x4 L = *reinterpret_cast<const f32x4*>(sl + ql);
          const f32x4 Dl = *reinterpret_cast<const f32x4*>(sl + 64 + ql);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            const int qg = q0 + ql + e;
            float pv = __builtin_amdgcn_exp2f(sc[r] * c - L[e]);
            if ((!FULL && key > qg) || qg >= a.seq) pv = 0.f;
            sc[r] = pv;
            dp[r] = pv * (dp[r] - Dl[e]);
          }
        }
        // dV^T[dim][key] += dO^T P ; dK^T[dim][key] += Q^T dS  (k = this wave's 32 queries)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4 pb = pack_half(sc, hf);
          const u32x4 sb = pack_half(dp, hf);
#pragma unroll
          for (int i = 0; i < DB; ++i) {
            dv[i] = mfma32(T::tfrag(tO, qh * 32, i, hf, lane), pb, dv[i]);
            dk[i] = mfma32(T::tfrag(tQ, qh * 32, i, hf, lane), sb, dk[i]);
          }
        }
      }
      __syncthreads();
    }
    // add the qh = 1 partials to qh = 0 through LDS (the tiles are free now)
    float* mg = reinterpret_cast<float*>(sm_) + kh * (2 * DB * 16 * 64);
    if (qh == 1) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          mg[(i * 16 + r) * 64 + lane] = dk[i][r];
          mg[((DB + i) * 16 + r) * 64 + lane] = dv[i][r];
        }
    }
    __syncthreads();
    if (qh == 0 && key < a.seq) {
      uint16_t* kout = (FULL ? a.dkv : a.dqkv) + (ktok0 + key) * a.ld_qkv + colq + D;
      uint16_t* vout = kout + D;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int dim = i * 32 + 8 * gg + 4 * g;
          float kv[4], vv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * gg + e;
            kv[e] = (dk[i][r] + mg[(i * 16 + r) * 64 + lane]) * a.scale;
            vv[e] = dv[i][r] + mg[((DB + i) * 16 + r) * 64 + lane];
          }
          const u32x2 wk = {pack_bf16x2(kv[0], kv[1]), pack_bf16x2(kv[2], kv[3])};
          const u32x2 wv = {pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
          *reinterpret_cast<u32x2*>(kout + dim) = wk;
          *reinterpret_cast<u32x2*>(vout + dim) = wv;
#pragma unroll
          for (int k = 0; k < 2; ++k)
            amx = max(amx, max(max(wk[k] & 0x7fffu, (wk[k] >> 16) & 0x7fffu),
                               max(wv[k] & 0x7fffu, (wv[k] >> 16) & 0x7fffu)));
        }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- part 2
  {
    const int qh = wave & 1, kh = wave >> 1;
    const int q0 = w * 64;
    const int qw = q0 + qh * 32;
    const int q = qw + (lane & 31);
    const bool qok = q < a.seq;
    const uint16_t* qrow = a.qkv + (tok0 + q) * a.ld_qkv + colq;
    const uint16_t* orow = a.dout + (tok0 + q) * a.ld_o + colo;
    u32x4 qf[KS], df[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = qok ? *reinterpret_cast<const u32x4*>(qrow + ks * 16 + g * 8) : u32x4{0, 0, 0, 0};
      df[ks] = qok ? *reinterpret_cast<const u32x4*>(orow + ks * 16 + g * 8) : u32x4{0, 0, 0, 0};
    }
    const float L2 = qok ? lse[q] * LOG2E : 0.f;
    const float Dq = qok ? dlt[q] : 0.f;
    f32x16 dq[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dq[i] = f32x16{};
    const i32x4 rs_kv[2] = {rk, rk};
    uint32_t lo_kv[T::PW];
    {
      const int64_t ld[2] = {a.ld_qkv, a.ld_qkv};
      const int64_t col[2] = {colq + D, colq + 2 * D};
#pragma unroll
      for (int q = 0; q < T::PW; ++q) lo_kv[q] = T::lane_off(ld, col, q);
    }
    for (int kb = 0; kb < (FULL ? nblk : w + 1); ++kb) {
      const int k0 = kb * 64;
      {
        const uint32_t st = (uint32_t)((ktok0 + k0) * a.ld_qkv * 2);
        const uint32_t step[2] = {st, st};
        T::load2(rs_kv, lo_kv, step, tK);
      }
      wait_dma();
      __syncthreads();
      const int kw = k0 + kh * 32;
      if (FULL || kw <= qw + 31) {
        // S^T[key][q], dP^T[key][q]: rows = this wave's 32 keys, column = query
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sc = mfma32(T::rfrag(tK, kh * 32, ks, lane), qf[ks], sc);
          dp = mfma32(T::rfrag(tV, kh * 32, ks, lane), df[ks], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kw + 8 * (r >> 2) + 4 * g + (r & 3);
          float pv = __builtin_amdgcn_exp2f(sc[r] * c - L2);
          if ((!FULL && kk > q) || !qok) pv = 0.f;
          dp[r] = pv * (dp[r] - Dq);
        }
        // dQ^T[dim][q] += K^T dS^T (k = this wave's 32 keys)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4 sb = pack_half(dp, hf);
#pragma unroll
          for (int i = 0; i < DB; ++i) dq[i] = mfma32(T::tfrag(tK, kh * 32, i, hf, lane), sb, dq[i]);
        }
      }
      __syncthreads();
    }
    float* mg = reinterpret_cast<float*>(sm_) + qh * (DB * 16 * 64);
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mg[(i * 16 + r) * 64 + lane] = dq[i][r];
    }
    __syncthreads();
    if (kh == 0 && qok) {
      uint16_t* qout = FULL ? a.dq + (tok0 + q) * a.ld_o + colo : a.dqkv + (tok0 + q) * a.ld_qkv + colq;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int dim = i * 32 + 8 * gg + 4 * g;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (dq[i][4 * gg + e] + mg[(i * 16 + 4 * gg + e) * 64 + lane]) * a.scale;
          const u32x2 wq = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(qout + dim) = wq;
#pragma unroll
          for (int k = 0; k < 2; ++k) amx = max(amx, max(wq[k] & 0x7fffu, (wq[k] >> 16) & 0x7fffu));
        }
    }
  }
  if (a.amax_part) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amx = max(amx, (uint32_t)__shfl_xor((int)amx, off));
    if (lane == 0) a.amax_part[blockIdx.x * 4 + wave] = amx;
  }
}

// ============================================================== launchers
// with_delta: compute D = rowsum(dO * O) first (the FULL calls of one set of
// queries reuse the D of their first call)
template <int D, bool FULL>
static hipError_t bwd_d(const AttnArgs& a, bool with_delta, hipStream_t s) {
  if (with_delta) {
    const int64_t rows = (int64_t)a.seq * a.batch * a.heads;
    hipLaunchKernelGGL(attn_delta_kernel<D>, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t units = (int64_t)((a.seq + 63) / 64) * a.heads * a.batch;
  if (units > INT32_MAX) return hipErrorInvalidValue;
  if (a.amax_part) {
    if (units * 4 > a.amax_cap) return hipErrorInvalidValue;
    if (a.amax_nparts) *a.amax_nparts = (int)(units * 4);
  }
  hipLaunchKernelGGL((attn_bwd_kernel<D, FULL>), dim3((unsigned)units), dim3(256), 0, s, a);
  return hipGetLastError();
}


hipError_t attention_bwd(const AttnArgs& a, hipStream_t s) {
  if (a.seq <= 0) return hipSuccess;
  if (a.dout_parts && (!a.dout_w || a.dout != a.dout_w)) return hipErrorInvalidValue;
  if (a.d == 64) return bwd_d<64, false>(a, true, s);
  if (a.d == 128) return bwd_d<128, false>(a, true, s);
  return hipErrorInvalidValue;
}

hipError_t attention_bwd_full(const AttnArgs& a, hipStream_t s) {
  if (a.seq <= 0) return hipSuccess;
  if (!a.kv || !a.dkv || !a.dq || a.kv_seq != a.seq || a.seq % 64 != 0) return hipErrorInvalidValue;
  if (a.d == 64) return bwd_d<64, true>(a, false, s);
  if (a.d == 128) return bwd_d<128, true>(a, false, s);
  return hipErrorInvalidValue;
}

// ============================================================== context-parallel merge
// The partial results of one set of queries against separate key chunks,
// (O_j, L_j) for j = 0 .. nparts-1, combine into the attention over all of
// them: L = log sum_j exp(L_j), O = sum_j exp(L_j - L) O_j, in ascending j,
// fp32.  d/8 lanes per (token, head) row, 16 bytes of each O_j per lane; rows
// are numbered token-major so a wave reads whole O rows.
__global__ __launch_bounds__(256) void cp_merge_kernel(CpMergeArgs a) {
  const int lanes = a.d / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / lanes;
  if (row >= a.tokens * a.heads) return;
  const int sub = (int)(gid % lanes);
  const int64_t tok = row / a.heads;
  const int n = (int)(row % a.heads);
  const int64_t li = (int64_t)n * a.tokens + tok;
  float m = -INFINITY;
  for (int j = 0; j < a.nparts; ++j) m = fmaxf(m, a.lse_parts[j * a.lse_stride + li]);
  float z = 0.f;
  for (int j = 0; j < a.nparts; ++j) z += expf(a.lse_parts[j * a.lse_stride + li] - m);
  const float L = m + logf(z);
  const int64_t oi = tok * a.heads * a.d + (int64_t)n * a.d + sub * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.nparts; ++j) {
    const float w = expf(a.lse_parts[j * a.lse_stride + li] - L);
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.o_parts + j * a.o_stride + oi);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += w * bf16_lo(v[e]);
      acc[2 * e + 1] += w * bf16_hi(v[e]);
    }
  }
  *reinterpret_cast<u32x4*>(a.o + oi) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  if (sub == 0) a.lse[li] = L;
}

// dQ of a CP rank's queries: dqkv's query columns (the rank's own chunk) plus
// the partials from the earlier chunks, parts[j] [tokens, heads*d], summed in
// fp32 in ascending j.  d/8 lanes per (token, head) row.
__global__ __launch_bounds__(256) void cp_dq_sum_kernel(CpDqSumArgs a) {
  const int lanes = a.d / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / lanes;
  if (row >= a.tokens * a.heads) return;
  const int sub = (int)(gid % lanes);
  const int64_t tok = row / a.heads;
  const int n = (int)(row % a.heads);
  uint16_t* dst = a.dqkv + tok * 3 * a.heads * a.d + (int64_t)n * 3 * a.d + sub * 8;
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(dst);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] = bf16_lo(v0[e]);
    acc[2 * e + 1] = bf16_hi(v0[e]);
  }
  const int64_t pi = tok * a.heads * a.d + (int64_t)n * a.d + sub * 8;
  for (int j = 0; j < a.nparts; ++j) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.parts + j * a.part_stride + pi);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(v[e]);
      acc[2 * e + 1] += bf16_hi(v[e]);
    }
  }
  *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
}

hipError_t cp_dq_sum(const CpDqSumArgs& a, hipStream_t s) {
  if (a.tokens <= 0 || a.nparts <= 0) return hipSuccess;
  if (a.d % 8 != 0 || a.d > 2048) return hipErrorInvalidValue;
  const int64_t blocks = (a.tokens * a.heads * (a.d / 8) + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cp_dq_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t cp_merge(const CpMergeArgs& a, hipStream_t s) {
  if (a.tokens <= 0 || a.nparts <= 0) return hipSuccess;
  if (a.d % 8 != 0 || a.d > 2048) return hipErrorInvalidValue;
  const int64_t threads = a.tokens * a.heads * (a.d / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cp_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mtl
