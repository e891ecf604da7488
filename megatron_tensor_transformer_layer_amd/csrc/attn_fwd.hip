// Causal multi-head attention, forward, for gfx950 (the backward is in
// attention.hip).
//
// Operation (per head n, per micro-batch element): S = Q K^T * scale with key
// j > query i masked, P = row-softmax(S), O = P V, and the row log-sum-exp L.
// Layout: Q, K, V of head n are columns [n*3d, n*3d+d), [+d, +2d), [+2d, +3d)
// of the head-interleaved QKV tensor; O is [tokens, heads*d]; L is [heads,
// tokens] fp32.
//
// CDNA4 design.  The scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: a lane owns one query and 16 of the 32 keys of a
// fragment, so a row's max and sum are in-register reductions plus one
// v_permlane32_swap, and the bf16 probabilities in the accumulator's registers
// are directly the b operand of O^T += V^T P (the k-slot order of that MFMA
// follows the accumulator layout).  K and V^T fragments come from LDS; V^T is
// read from the natural-layout V tile with ds_read_b64_tr_b16.
//
// Work item: 64 queries of one head; a workgroup takes the mirrored pair of
// items (p, n-1-p) one after the other, so causal work is balanced, and the
// units of one head are kept on one XCD (they all stream that head's K and V).
// A stage is the K and V tiles of two consecutive 64-key blocks; two stages
// double-buffer the LDS DMA.  The eight waves of a workgroup, two per SIMD, take
// (query half, key half, block parity): wave w handles queries (w & 1)*32 ..
// +31 of the item, keys ((w >> 1) & 1)*32 .. +31 of the blocks of parity
// w >> 2.  With two waves on a SIMD one wave's softmax (16 exponentials per lane
// and block) runs while the other's MFMAs do; the 1 KB of K or V^T fragment a
// 32x32x16 MFMA reads from LDS and the stage's DMA writes put the LDS at about
// 1.5 times the MFMA time per block, which the overlap approaches.  A wave
// raises its issue priority (s_setprio) over each burst of MFMAs, so that the
// SIMD's arbiter keeps the matrix core fed while the other wave's softmax
// fills the gaps.  At the end
// of an item the four partial states of each query half (row max, row sum, O)
// are merged through LDS, wave w finishing 32-dim block w >> 1 of query half
// w & 1.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mtl {
namespace {

constexpr float LOG2E_F = 1.4426950408889634f;

// max / sum of a value and its copy in lane l ^ 32 (the lane that holds the
// same query's other 16 keys)
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct Tiles {
  static constexpr int RB = 2 * D;              // bytes per key row
  static constexpr int TILE = 64 * RB;          // one 64-key K or V tile
  static constexpr int STAGE = 4 * TILE;        // K(even) V(even) K(odd) V(odd)
  static constexpr int PER_TILE = TILE / 1024;  // DMA wave instructions per tile
  static constexpr int PER_WAVE = 4 * PER_TILE / 8;
  // 64-bank swizzles: K rows are read 16 rows per cycle (ds_read_b128), V rows
  // 4 at a time by the transpose read; both maps are bijections on a row.
  static __device__ __forceinline__ int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  static __device__ __forceinline__ int vswz(int row) { return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }

  // The lane's part of the byte offset of DMA instruction q of a wave: key row
  // (tile >> 1) * 64 + row, column chunk c of K or V, relative to the stage's
  // first key; it is the same for every stage.
  static __device__ __forceinline__ uint32_t lane_off(int64_t ld, int wave, int lane, int q) {
    const int I = wave * PER_WAVE + q;
    const int tile = I / PER_TILE;  // 0 K even, 1 V even, 2 K odd, 3 V odd
    const int o = (I % PER_TILE) * 1024 + lane * 16;
    const int row = o / RB;
    const int pc = (o % RB) >> 4;
    const bool isv = tile & 1;
    const int c = pc ^ (isv ? vswz(row) : kswz(row));
    return (uint32_t)((((tile >> 1) * 64 + row) * ld + (isv ? 2 * D : D) + c * 8) * 2);
  }
  // DMA the K and V tiles of key blocks kb0 and kb0+1 (64 keys each) into stage
  // st; stage_off is the byte offset of the head's column 0 in key row kb0 * 64
  static __device__ __forceinline__ void load(i32x4 rs, const uint32_t (&lo)[PER_WAVE], uint32_t stage_off,
                                              LDS_AS char* st, int wave) {
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int I = wave * PER_WAVE + q;
      dma16(rs, lo[q] + stage_off, 0u, lds_addr(st + I * 1024));
    }
  }
  // a-operand fragment of K (rows = keys row0 + l%32, 8 dims of k step ks)
  static __device__ __forceinline__ u32x4 kfrag(const LDS_AS char* k, int row0, int ks, int lane) {
    const int row = row0 + (lane & 31);
    const int c = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const LDS_AS u32x4*>(k + row * RB + ((c ^ kswz(row)) << 4));
  }
  // a-operand fragment of V^T (rows = dims i*32 + l%32); its k slots are keys
  // row0 + ks*16 + 8*(j/4) + 4*(l/32) + j%4, the order of a 32x32 accumulator's rows.
  static __device__ __forceinline__ u32x4 vfrag(const LDS_AS char* v, int row0, int i, int ks, int lane) {
    const int G = lane >> 4, R = (lane >> 2) & 3, c4 = lane & 3;
    const int key = row0 + ks * 16 + 4 * (G >> 1) + R;
    const int dim = i * 32 + (G & 1) * 16 + 4 * c4;
    const LDS_AS char* p = v + key * RB + (((dim >> 3) ^ vswz(key)) << 4) + ((dim & 7) >> 2) * 8;
    const u32x2 lo = read_tr(p);
    const u32x2 hi = read_tr(p + 8 * RB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

__device__ __forceinline__ u32x4 pack_half(const f32x16& p, int half) {
  const int o = half * 8;
  return u32x4{pack_bf16x2(p[o + 0], p[o + 1]), pack_bf16x2(p[o + 2], p[o + 3]), pack_bf16x2(p[o + 4], p[o + 5]),
               pack_bf16x2(p[o + 6], p[o + 7])};
}

// FULL: the queries of a.qkv against every key of a separate chunk a.kv
// (a.kv_seq keys, a multiple of 64, same head-interleaved layout): no causal
// mask, every item takes all key blocks.  Otherwise causal self-attention.
template <int D, bool FULL>
__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(AttnArgs a) {
  using T = Tiles<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char st_[2 * T::STAGE];
  __shared__ __attribute__((aligned(16))) float ml_[8 * 2 * 64];  // [wave][m, l][lane]
  // the merge keeps every wave's O in the stages: 8 waves x DB x 16 x 64 floats
  static_assert(8 * DB * 16 * 64 * 4 <= 2 * T::STAGE, "merge area");
  LDS_AS char* st0 = (LDS_AS char*)st_;
  LDS_AS char* st1 = st0 + T::STAGE;

  const int nitems = (a.seq + 63) / 64;
  const int npairs = (nitems + 1) / 2;
  const int u = xcd_index(blockIdx.x, npairs * a.heads * a.batch);
  const int pair = u % npairs, n = (u / npairs) % a.heads, b = u / (npairs * a.heads);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g = lane >> 5;
  const int qsub = wave & 1, kh = (wave >> 1) & 1, kpar = wave >> 2;
  const int64_t tokens = (int64_t)a.seq * a.batch;
  const int64_t tok0 = (int64_t)b * a.seq;
  const int colq = n * 3 * D;
  const uint16_t* qbase = a.qkv + tok0 * a.ld_qkv + colq;
  const float c = a.scale * LOG2E_F;
  // K and V tiles come from the buffer resource rs, starting at token kvtok0
  const i32x4 rs = FULL ? make_rsrc(a.kv, (uint32_t)((int64_t)a.kv_seq * a.batch * a.ld_qkv * 2))
                        : make_rsrc(a.qkv, (uint32_t)(tokens * a.ld_qkv * 2));
  const int64_t kvtok0 = FULL ? (int64_t)b * a.kv_seq : tok0;
  const int nkb_all = FULL ? a.kv_seq / 64 : nitems;
  uint32_t lo[T::PER_WAVE];
#pragma unroll
  for (int q = 0; q < T::PER_WAVE; ++q) lo[q] = T::lane_off(a.ld_qkv, wave, lane, q);
  // byte offset of the head's column 0 in key row kb * 64 (wave-uniform)
  auto stage_off = [&](int kb) { return (uint32_t)(((kvtok0 + (int64_t)kb * 64) * a.ld_qkv + colq) * 2); };

  uint32_t amx = 0;  // largest bf16 magnitude of O this wave stores
  for (int side = 0; side < 2; ++side) {
    const int item = side == 0 ? pair : nitems - 1 - pair;
    if (side == 1 && item == pair) break;
    const int q0 = item * 64;
    const int qw = q0 + qsub * 32;
    const int q = qw + (lane & 31);
    const bool qok = q < a.seq;
    const int nkb = FULL ? nkb_all : min(item + 1, nkb_all);
    const int niter = (nkb + 1) / 2;

    u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = qok ? *reinterpret_cast<const u32x4*>(qbase + (int64_t)q * a.ld_qkv + ks * 16 + g * 8)
                   : u32x4{0, 0, 0, 0};
    wait_loads();
    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x16{};
    float m = -INFINITY, l = 0.f;

    // this wave's key half of block kb (parity kpar) in stage st
    auto block = [&](const LDS_AS char* st, int kb) {
      const LDS_AS char* kt = st + kpar * 2 * T::TILE;
      const LDS_AS char* vt = kt + T::TILE;
      const int kbase = kb * 64 + kh * 32;
      f32x16 s = f32x16{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = mfma32(T::kfrag(kt, kh * 32, ks, lane), qf[ks], s);
      __builtin_amdgcn_s_setprio(0);
      // only a block on the diagonal is masked (wave-uniform test)
      if (!FULL && kbase + 31 > qw) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > q) s[r] = -INFINITY;
        }
      }
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) bm = fmaxf(bm, s[r]);
      bm = max_xor32(bm);
      // The reference max m moves (and l, o are rescaled) only when some row's
      // block max exceeds it by more than 2^8 in the exponent; otherwise the
      // probabilities are taken against the stale m (at most 2^8, exact in the
      // final normalisation), which spares the accumulator rescale.  A row whose
      // keys in this half are all masked has bm = -inf and keeps m.
      if (__any((bm - m) * c > 8.f)) {
        asm volatile("" ::: "memory");  // keep this a branch, not a select on alpha
        const float mx = fmaxf(m, bm);
        const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mx) * c);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] *= alpha;
        m = mx;
      }
      const float mc = m == -INFINITY ? 0.f : m * c;
      float rsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(s[r] * c - mc);
        s[r] = pv;
        rsum += pv;
      }
      l += rsum;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 pb = pack_half(s, ks);
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] = mfma32(T::vfrag(vt, kh * 32, i, ks, lane), pb, o[i]);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // does this wave's key half of block kb hold a key <= its last query?
    auto active = [&](int kb) { return kb < nkb && (FULL || kb * 64 + kh * 32 <= qw + 31); };

    T::load(rs, lo, stage_off(0), st0, wave);
    wait_dma();
    __syncthreads();
    for (int it = 0; it < niter; it += 2) {
      const bool more1 = it + 1 < niter;
      if (more1) T::load(rs, lo, stage_off(2 * (it + 1)), st1, wave);
      if (active(2 * it + kpar)) block(st0, 2 * it + kpar);
      if (more1) wait_dma();
      __syncthreads();
      if (more1) {
        const bool more2 = it + 2 < niter;
        if (more2) T::load(rs, lo, stage_off(2 * (it + 2)), st0, wave);
        if (active(2 * (it + 1) + kpar)) block(st1, 2 * (it + 1) + kpar);
        if (more2) wait_dma();
        __syncthreads();
      }
    }

    // merge: every wave leaves its row max, row sum and O in LDS (the stages
    // are free after the last barrier); wave w finishes dim block w >> 1 of
    // query half w & 1 from the four partial states of that half
    float* ml = ml_ + wave * 2 * 64;
    ml[lane] = m;
    ml[64 + lane] = sum_xor32(l);
    float* om = reinterpret_cast<float*>(st_) + wave * (DB * 16 * 64);  // [i][r][lane]
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) om[(i * 16 + r) * 64 + lane] = o[i][r];
    __syncthreads();
    const int i = wave >> 1;
    if (i < DB) {
      // the partial states of query half qsub: waves qsub, qsub+2, qsub+4, qsub+6
      float mw[4], lw[4], mt = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        mw[v] = ml_[(2 * v + qsub) * 2 * 64 + lane];
        lw[v] = ml_[(2 * v + qsub) * 2 * 64 + 64 + lane];
        mt = fmaxf(mt, mw[v]);
      }
      float aw[4], lt = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        aw[v] = mw[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mw[v] - mt) * c);
        lt += aw[v] * lw[v];
      }
      if (qok) {
        const float inv = 1.f / lt;
        float val[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc += aw[v] * reinterpret_cast<const float*>(st_)[(2 * v + qsub) * (DB * 16 * 64) + (i * 16 + r) * 64 + lane];
          val[r] = acc * inv;
        }
        uint16_t* orow = a.o + (tok0 + q) * a.ld_o + (int64_t)n * D;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int dim = i * 32 + 8 * gg + 4 * g;
          const u32x2 w = {pack_bf16x2(val[4 * gg], val[4 * gg + 1]), pack_bf16x2(val[4 * gg + 2], val[4 * gg + 3])};
          *reinterpret_cast<u32x2*>(orow + dim) = w;
#pragma unroll
          for (int k = 0; k < 2; ++k) amx = max(amx, max(w[k] & 0x7fffu, (w[k] >> 16) & 0x7fffu));
        }
        if (i == 0 && g == 0) a.lse[(int64_t)n * tokens + tok0 + q] = mt * a.scale + logf(lt);
      }
    }
    __syncthreads();  // the next item's DMA reuses the stages
  }
  if (a.amax_part) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amx = max(amx, (uint32_t)__shfl_xor((int)amx, off));
    if (lane == 0) a.amax_part[blockIdx.x * 8 + wave] = amx;
  }
}

template <int D, bool FULL>
hipError_t fwd_d(const AttnArgs& a, hipStream_t s) {
  const int64_t npairs = ((a.seq + 63) / 64 + 1) / 2;
  const int64_t units = npairs * a.heads * a.batch;
  if (units > INT32_MAX) return hipErrorInvalidValue;
  if (a.amax_part) {
    if (units * 8 > a.amax_cap) return hipErrorInvalidValue;
    if (a.amax_nparts) *a.amax_nparts = (int)(units * 8);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, FULL>), dim3((unsigned)units), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t attention_fwd(const AttnArgs& a, hipStream_t s) {
  if (a.seq <= 0) return hipSuccess;
  if (a.d == 64) return fwd_d<64, false>(a, s);
  if (a.d == 128) return fwd_d<128, false>(a, s);
  return hipErrorInvalidValue;
}
hipError_t attention_fwd_full(const AttnArgs& a, hipStream_t s) {
  if (a.seq <= 0) return hipSuccess;
  if (!a.kv || a.kv_seq <= 0 || a.kv_seq % 64 != 0) return hipErrorInvalidValue;
  if (a.d == 64) return fwd_d<64, true>(a, s);
  if (a.d == 128) return fwd_d<128, true>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace mtl
