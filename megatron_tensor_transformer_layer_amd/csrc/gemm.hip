// bf16 MFMA GEMM for gfx950 with fused epilogues.
//
// C[M,N] = A[M,K] * B[K,N], fp32 accumulate.  Each operand is either
// k-contiguous (A[m][k], B[n][k]) or mn-contiguous (A[k][m], B[k][n]); the three
// products of a linear layer's training step use (A k, B mn) for forward,
// (A k, B k) for dgrad and (A mn, B mn) for wgrad when weights are stored
// [in, out] row-major.
//
// Design (CDNA4): 256 threads = 4 wave64s in a 2x2 grid; a BMxBN tile per
// workgroup, K stepped 64 at a time through a double-buffered LDS stage of
// k-contiguous rows (16-byte chunks XOR-swizzled by row).  mn-contiguous
// operands are read as 8(k) x 8(mn) blocks and transposed in registers with
// v_perm_b32 before the LDS write, so the MFMA operand reads are always one
// ds_read_b128 per lane.  The MFMA is issued with the operands swapped
// (B fragment as "a", A fragment as "b") so that each lane ends up owning 4
// consecutive output columns of one row: the epilogue stores 8 or 16 bytes per
// lane.  Tile order is XCD-aware: the 8 XCDs each take a contiguous block of
// tiles (grouped 4 tile-rows at a time) so A/B panels are reused inside one L2.
#include "common.hpp"
#include "kernels.hpp"

namespace mtl {

template <int ROWS, bool KCONTIG>
struct TileLoader {
  // k-contiguous: ROWS x 64 tile, thread t loads chunk t%8 of rows t/8 + 32 i.
  // mn-contiguous: ROWS/8 x 8 blocks of 8x8, block b = t + 256 i: kg = b%8, mg = b/8.
  static constexpr int NK = ROWS / 32;
  static constexpr int NB = (ROWS + 255) / 256;
  static constexpr int NREG = KCONTIG ? NK : NB * 8;
  u32x4 r[NREG];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int row0, int nrows, int k0,
                                       int K) {
    const int t = threadIdx.x;
    if constexpr (KCONTIG) {
      const int c = t & 7;
      const int kk = k0 + c * 8;
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int row = row0 + (t >> 3) + 32 * i;
        if (row < nrows && kk < K) {
          r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * ld + kk);
        } else {
          r[i] = u32x4{0, 0, 0, 0};
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int b = t + 256 * i;
        const int kg = b & 7, mg = b >> 3;
        const int col = row0 + mg * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + kg * 8 + j;
          if (b < ROWS && col < nrows && k < K) {
            r[i * 8 + j] = *reinterpret_cast<const u32x4*>(base + (int64_t)k * ld + col);
          } else {
            r[i * 8 + j] = u32x4{0, 0, 0, 0};
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* lds) {
    const int t = threadIdx.x;
    if constexpr (KCONTIG) {
      const int c = t & 7;
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int row = (t >> 3) + 32 * i;
        *reinterpret_cast<u32x4*>(lds + swz(row, c)) = r[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int b = t + 256 * i;
        if (b < ROWS) {
          const int kg = b & 7, mg = b >> 3;
          u32x4 in[8], out[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) in[j] = r[i * 8 + j];
          transpose8x8(in, out);
#pragma unroll
          for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(lds + swz(mg * 8 + j, kg)) = out[j];
        }
      }
    }
  }
};

__device__ __forceinline__ int tile_index(int w, int ntiles) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of logical tiles.
  if ((ntiles & 7) == 0) return (w & 7) * (ntiles >> 3) + (w >> 3);
  return w;
}

template <int BM, int BN, bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  __shared__ __attribute__((aligned(16))) char smem[2 * (A_BYTES + B_BYTES)];

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int t = tile_index(blockIdx.x, ntiles);
  constexpr int GM = 4;
  const int group = GM * tiles_n;
  const int first_m = (t / group) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int tm = first_m + (t % group) % gm;
  const int tn = (t % group) / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  TileLoader<BM, A_K> la;
  TileLoader<BN, B_K> lb;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int nk = (p.K + 63) / 64;
  la.load(p.a, p.lda, m0, p.M, 0, p.K);
  lb.load(p.b, p.ldb, n0, p.N, 0, p.K);
  la.store(smem);
  lb.store(smem + A_BYTES);
  __syncthreads();

  const int lrow = lane & 31, lgrp = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    char* sa = smem + (kt & 1) * (A_BYTES + B_BYTES);
    char* sb = sa + A_BYTES;
    if (kt + 1 < nk) {
      la.load(p.a, p.lda, m0, p.M, (kt + 1) * 64, p.K);
      lb.load(p.b, p.ldb, n0, p.N, (kt + 1) * 64, p.K);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(sa + swz(wm * WM + i * 32 + lrow, kk * 2 + lgrp));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(sb + swz(wn * WN + j * 32 + lrow, kk * 2 + lgrp));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
    }
    if (kt + 1 < nk) {
      char* na = smem + ((kt + 1) & 1) * (A_BYTES + B_BYTES);
      la.store(na);
      lb.store(na + A_BYTES);
    }
    __syncthreads();
  }

  // Epilogue: lane owns row m, columns n..n+3 for each (i, j, g).
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + i * 32 + lrow;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + j * 32 + 8 * g + 4 * lgrp;
        if (n >= p.N) continue;
        float v[4] = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if constexpr (EPI == EPI_F32 || EPI == EPI_F32_ACC) {
          float* c = reinterpret_cast<float*>(p.c) + (int64_t)m * p.ldc + n;
          f32x4 o = {v[0], v[1], v[2], v[3]};
          if constexpr (EPI == EPI_F32_ACC) o += *reinterpret_cast<const f32x4*>(c);
          *reinterpret_cast<f32x4*>(c) = o;
        } else {
          if constexpr (EPI == EPI_BF16_BIAS || EPI == EPI_BIAS_GELU) {
            const u32x2 bb = *reinterpret_cast<const u32x2*>(p.bias + n);
            v[0] += bf16_lo(bb[0]);
            v[1] += bf16_hi(bb[0]);
            v[2] += bf16_lo(bb[1]);
            v[3] += bf16_hi(bb[1]);
          }
          if constexpr (EPI == EPI_DGELU) {
            const u32x2 zz = *reinterpret_cast<const u32x2*>(p.aux + (int64_t)m * p.ld_aux + n);
            v[0] *= gelu_grad_f(bf16_lo(zz[0]));
            v[1] *= gelu_grad_f(bf16_hi(zz[0]));
            v[2] *= gelu_grad_f(bf16_lo(zz[1]));
            v[3] *= gelu_grad_f(bf16_hi(zz[1]));
          }
          uint16_t* c = reinterpret_cast<uint16_t*>(p.c) + (int64_t)m * p.ldc + n;
          *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          if constexpr (EPI == EPI_BIAS_GELU) {
            uint16_t* c2 = reinterpret_cast<uint16_t*>(p.c2) + (int64_t)m * p.ldc2 + n;
            *reinterpret_cast<u32x2*>(c2) = u32x2{pack_bf16x2(gelu_f(v[0]), gelu_f(v[1])),
                                                  pack_bf16x2(gelu_f(v[2]), gelu_f(v[3]))};
          }
        }
      }
    }
  }
}

template <int BM, int BN, bool A_K, bool B_K, int EPI>
static hipError_t launch_cfg(const GemmArgs& p, hipStream_t s) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, A_K, B_K, EPI>), dim3(tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool A_K, bool B_K, int EPI>
static hipError_t launch_layout(const GemmArgs& p, hipStream_t s) {
  const long t256 = (long)((p.M + 255) / 256) * ((p.N + 255) / 256);
  const long t192 = (long)((p.M + 255) / 256) * ((p.N + 191) / 192);
  if (t256 >= 240) return launch_cfg<256, 256, A_K, B_K, EPI>(p, s);
  if (t192 >= 240 && p.N % 192 == 0) return launch_cfg<256, 192, A_K, B_K, EPI>(p, s);
  return launch_cfg<128, 128, A_K, B_K, EPI>(p, s);
}

hipError_t gemm_bf16(const GemmArgs& p, GemmLayout layout, int epi, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  switch (layout) {
    case GEMM_FWD:  // A k-contig, B n-contig
      if (epi == EPI_BF16) return launch_layout<true, false, EPI_BF16>(p, s);
      if (epi == EPI_BF16_BIAS) return launch_layout<true, false, EPI_BF16_BIAS>(p, s);
      if (epi == EPI_BIAS_GELU) return launch_layout<true, false, EPI_BIAS_GELU>(p, s);
      break;
    case GEMM_DGRAD:  // A k-contig, B k-contig
      if (epi == EPI_BF16) return launch_layout<true, true, EPI_BF16>(p, s);
      if (epi == EPI_DGELU) return launch_layout<true, true, EPI_DGELU>(p, s);
      break;
    case GEMM_WGRAD:  // A m-contig, B n-contig
      if (epi == EPI_F32) return launch_layout<false, false, EPI_F32>(p, s);
      if (epi == EPI_F32_ACC) return launch_layout<false, false, EPI_F32_ACC>(p, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace mtl
