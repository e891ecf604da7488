// bf16 MFMA GEMM for gfx950 with fused epilogues.
//
// C[M,N] = A[M,K] * B[K,N], fp32 accumulate.  Each operand is either
// k-contiguous (A[m][k], B[n][k]) or mn-contiguous (A[k][m], B[k][n]); the three
// products of a linear layer's training step use (A k, B mn) for forward,
// (A k, B k) for dgrad and (A mn, B mn) for wgrad when weights are stored
// [in, out] row-major.
//
// Design (CDNA4):
//  * 256 threads = 4 wave64s in a 2x2 grid, a BM x BN tile per workgroup, K in
//    slabs of 64, v_mfma_f32_32x32x16_bf16.
//  * Global -> VGPR -> LDS, two slabs ahead, in two LDS stages.  While slab kt
//    is multiplied from one stage, slab kt+1 is written from registers into
//    the other (ds_write_b128, interleaved with the MFMAs) and each register is
//    reloaded with its chunk of slab kt+2 right behind its write, so a load has
//    a whole slab of MFMAs to land.  The two stage pointers are passed
//    __restrict__, which lets the scheduler interleave the writes of one stage
//    with the fragment reads of the other.  (LDS DMA of the same slabs, one
//    slab ahead, measured 4-15% slower: the DMA stream and the MFMAs overlapped
//    poorly.)
//  * A lane's chunk offsets are computed once per tile; a slab adds its
//    uniform k offset.
//  * A k-contiguous operand is kept as [rows][64] with its 16-byte chunks XOR
//    swizzled by row; fragments are one ds_read_b128 per lane.
//  * An mn-contiguous operand is kept in its global layout [64][rows] (64-byte
//    groups XOR-swizzled by k so that the reads below hit distinct banks) and read with
//    two ds_read_b64_tr_b16: within each 16-lane group, lanes 4R..4R+3 name row
//    R of a 4 x 16 block and lane i receives its column i, i.e. four
//    consecutive k of one m (or n).  No register transposes.
//  * The MFMA stream runs one k step behind the fragment reads: step kk's
//    fragments are read while step kk-1's MFMAs issue, across slab boundaries
//    too, so after each slab's barrier the previous slab's last MFMAs (whose
//    fragments are already in registers) cover the first LDS reads.
//  * The MFMA is issued with the operands swapped (B fragment as "a") so that
//    each lane owns 4 consecutive output columns of one row: the epilogue
//    stores 8 or 16 bytes per lane.
//  * Tile order is XCD-aware: the 8 XCDs each take a contiguous run of tiles
//    (grouped 4 tile-rows at a time) so A/B panels are reused inside one L2.
//  * Tails: raw buffer range checks return zeros past an operand's last row;
//    rows/columns past M or N are never stored; chunks past K of a partial last
//    slab (which hold the next row's values in the k-contiguous layout) are
//    zero-filled in LDS before use.
#include <algorithm>
#include <queue>
#include <utility>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

namespace mtl {

// LDS swizzles, for gfx950's 64 x 4-byte banks (ds_read_b128 serves 16 lanes per
// cycle, ds_read_b64_tr_b16 32 lanes per cycle):
//  * k-contiguous tiles ([rows][64], 128-byte rows): 16-byte chunk c of row r is
//    stored at c ^ ((r >> 1) & 7), so the 16 rows of one cycle (two rows per
//    256-byte bank line) use 16 distinct bank quads;
//  * mn-contiguous tiles ([64][rows]): the 64-byte group of row k is XORed with
//    k & 3, so the 4 rows a transpose read touches per cycle fall in 4 different
//    64-byte bank windows.  For 192-wide tiles (24 chunks, 384-byte rows, which
//    already alternate bank halves) only bit 2 of the chunk is flipped, by
//    (k >> 1) & 1, which keeps the map a bijection on the row.
__device__ __forceinline__ int kc_swz(int row) { return (row >> 1) & 7; }
template <int ROWS>
__device__ __forceinline__ int mn_swz(int k) {
  if constexpr (ROWS % 256 == 0 || ROWS == 128) return (k & 3) << 2;
  else return ((k >> 1) & 1) << 2;
}

// USED: 16-byte chunks of a row's 128 LDS bytes that carry data (8; 6 for
// MXFP6, whose slab of 128 k is 96 code bytes per row; the lanes of the other
// two chunks load zeros, their loads placed out of the buffer's range).
template <int ROWS, bool KC, int EB = 2, int NWAVES = 4, int USED = 8>
struct Operand {
  static_assert(EB == 2 || KC, "fp8 operands are k-contiguous");
  static_assert(USED == 8 || KC, "partial rows are k-contiguous");
  static constexpr int BYTES = ROWS * 128;     // one slab: 128 bytes of k per row
  static constexpr int KSLAB = USED * 16 / EB; // k per slab: 64 bf16 or 128 fp8 (96 MXFP6 code bytes)
  static constexpr int CHUNK = 16 / EB;        // k per 16-byte chunk
  static constexpr int INSTR = BYTES / 1024;   // wave instructions per slab
  static constexpr int PER_WAVE = INSTR / NWAVES;
  static_assert(INSTR % NWAVES == 0, "slab chunks must split evenly over the waves");
  static constexpr int ROWB = ROWS * 2;        // row bytes of the mn-contiguous layout
  static constexpr int READS = (KC && EB == 2) ? 1 : 2;  // LDS read instructions per fragment

  // Slab [k0, k0+KSLAB) of rows [row0, row0+ROWS) (ld, k0 in elements) moves
  // as 1 KB wave chunks; chunk I of the slab:
  // k-contiguous: fills rows 8I..8I+7, lane -> (row 8I + l/8, physical chunk
  // l%8 = logical chunk ^ kc_swz(row)).
  // mn-contiguous: lds byte o = 1024 I + 16 l is (k = o / ROWB, physical chunk
  // (o % ROWB)/16 = logical chunk ^ mn_swz(k)).
  // The per-lane byte offsets of slab 0 are computed once (offsets); slab k0
  // adds the uniform slab_bytes(k0) to them, as 32-bit sums equal to the full
  // offset taken mod 2^32.  The whole offset goes in the VGPR operand: the
  // raw-buffer range check (which turns reads past the end into zeros) does not
  // cover soffset.
  static __device__ __forceinline__ void offsets(int64_t ld, int row0, uint32_t (&voff)[PER_WAVE]) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int I = wave * PER_WAVE + q;
      if constexpr (KC) {
        const int row = I * 8 + (lane >> 3);
        const int c = (lane & 7) ^ kc_swz(row);
        voff[q] = c < USED ? (uint32_t)(((int64_t)(row0 + row) * ld + c * CHUNK) * EB) : 0x80000000u;
      } else {
        const int o = I * 1024 + lane * 16;
        const int k = o / ROWB;
        const int c = ((o % ROWB) >> 4) ^ mn_swz<ROWS>(k);
        voff[q] = (uint32_t)(((int64_t)k * ld + row0 + c * 8) * 2);
      }
    }
  }
  static __device__ __forceinline__ uint32_t slab_bytes(int64_t ld, int k0) {
    return KC ? (uint32_t)((int64_t)k0 * EB) : (uint32_t)((int64_t)k0 * ld * 2);
  }
  // A wave's chunks of a slab: loaded into registers (gload), written to LDS
  // (lwrite) at byte (wave*PER_WAVE + q)*1024 + 16*lane of the stage.
  static __device__ __forceinline__ void gload(__amdgpu_buffer_rsrc_t rs, const uint32_t (&voff)[PER_WAVE],
                                               uint32_t kb, u32x4 (&reg)[PER_WAVE]) {
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q)
      reg[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(voff[q] + kb), 0, 0));
  }
  static __device__ __forceinline__ void lwrite(const u32x4& v, int q, LDS_AS char* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    *reinterpret_cast<LDS_AS u32x4*>(lds + (wave * PER_WAVE + q) * 1024 + lane * 16) = v;
  }

  // k-contiguous operand of a slab with kvalid < KSLAB valid k (after this
  // thread's writes of it): zero the chunks past K, which hold the next row's
  // values.
  static __device__ __forceinline__ void zero_tail(LDS_AS char* lds, int kvalid) {
    if constexpr (KC) {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
      for (int q = 0; q < PER_WAVE; ++q) {
        const int I = wave * PER_WAVE + q;
        const int c = (lane & 7) ^ kc_swz(I * 8 + (lane >> 3));
        if (c * CHUNK >= kvalid) *reinterpret_cast<LDS_AS u32x4*>(lds + I * 1024 + lane * 16) = u32x4{0, 0, 0, 0};
      }
    }
  }

  // fp8 fragment of 32-row block r32 at k step kk (64 deep): lane l holds row
  // (l % 32) and k = kk*64 + (l/32)*32 + j, j = 0..31, as two 16-byte chunks.
  static __device__ __forceinline__ void frag8(const LDS_AS char* lds, int r32, int kk, int lane, u32x4& lo,
                                               u32x4& hi) {
    const int row = r32 * 32 + (lane & 31);
    const int c = kk * 4 + (lane >> 5) * 2;
    lo = *reinterpret_cast<const LDS_AS u32x4*>(lds + row * 128 + ((c ^ kc_swz(row)) << 4));
    hi = *reinterpret_cast<const LDS_AS u32x4*>(lds + row * 128 + (((c + 1) ^ kc_swz(row)) << 4));
  }

  // MXFP6 fragment (GEMM code order) of 32-row block r32 at k step kk (64
  // deep, the slab's blocks 2 kk and 2 kk + 1): lane l holds row l % 32 and
  // block b = 2 kk + l / 32 -- its first 16 bytes in chunk b, its last 8 in
  // half (b % 2) ^ (row / 16 % 2) of chunk 4 + kk.
  static __device__ __forceinline__ void frag6(const LDS_AS char* lds, int r32, int kk, int lane, u32x4& main,
                                               u32x2& tail) {
    const int row = r32 * 32 + (lane & 31);
    const int b = kk * 2 + (lane >> 5);
    const int half = (b & 1) ^ ((row >> 4) & 1);
    main = *reinterpret_cast<const LDS_AS u32x4*>(lds + row * 128 + ((b ^ kc_swz(row)) << 4));
    tail = *reinterpret_cast<const LDS_AS u32x2*>(lds + row * 128 + (((4 + kk) ^ kc_swz(row)) << 4) + half * 8);
  }

  // Operand fragment of 32-row block r32 at k step kk (16 deep): lane l holds
  // row (l % 32) and k = kk*16 + (l/32)*8 + j, j = 0..7.
  static __device__ __forceinline__ u32x4 frag(const LDS_AS char* lds, int r32, int kk, int lane) {
    if constexpr (KC) {
      const int row = r32 * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      return *reinterpret_cast<const LDS_AS u32x4*>(lds + row * 128 + ((c ^ kc_swz(row)) << 4));
    } else {
      // lanes 4R..4R+3 of each 16-lane group g name row k = kk*16 + (g/2)*8 + R
      // (+4 for the second read), columns r32*32 + (g%2)*16 + 4*(l%4) .. +3
      const int g = lane >> 4, R = (lane >> 2) & 3, c4 = lane & 3;
      const int chunk = (r32 * 4 + (g & 1) * 2 + (c4 >> 1)) ^ mn_swz<ROWS>(R);
      const int lanepart = (g >> 1) * 8 * ROWB + R * ROWB + (chunk << 4) + (c4 & 1) * 8;
      const LDS_AS char* p = lds + lanepart + kk * 16 * ROWB;
      const u32x2 lo = read_tr(p);
      const u32x2 hi = read_tr(p + 4 * ROWB);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }
};

// F8 = 0: bf16 operands.  F8 = 1 + FA + 2*FB: fp8 operands, A in format FA and
// B in format FB (0 = E4M3, 1 = E5M2), both k-contiguous.  F8 = F8_MXFP4 or
// F8_MXFP4_GO: MXFP4 operands (E2M1 codes, two per byte, low nibble first, with
// one E8M0 scale byte per 32 k; scale matrices in plain or GEMM order), both
// k-contiguous; K, lda and ldb then count code bytes.
constexpr int F8_MXFP4 = 5, F8_MXFP4_GO = 6;
// F8 = F8_MXFP6_GO: MXFP6 (E2M3) operands with codes and scales in GEMM order;
// K, lda and ldb count code bytes (3/4 per k), a slab is 128 k (96 bytes).
constexpr int F8_MXFP6_GO = 7;
template <int BM, int BN, bool A_K, bool B_K, int F8 = 0, int NWN = 2>
struct Mainloop {
  static constexpr int NWAVES = 2 * NWN;  // 2 x NWN waves over the tile
  static constexpr int WM = BM / 2, WN = BN / NWN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr bool FP4 = F8 == F8_MXFP4 || F8 == F8_MXFP4_GO;
  static constexpr bool FP6 = F8 == F8_MXFP6_GO;
  static constexpr bool MX = FP4 || FP6;  // block-scaled operands
  static constexpr bool GO = F8 == F8_MXFP4_GO || FP6;
  static_assert(!MX || (A_K && B_K), "MX operands are k-contiguous");
  static constexpr int EB = F8 ? 1 : 2;
  static constexpr int FA = (F8 && !MX) ? (F8 - 1) & 1 : 0, FB = (F8 && !MX) ? (F8 - 1) >> 1 : 0;
  using OA = Operand<BM, A_K, EB, NWAVES, FP6 ? 6 : 8>;
  using OB = Operand<BN, B_K, EB, NWAVES, FP6 ? 6 : 8>;
  static constexpr int KSLAB = OA::KSLAB;
  // MFMA k steps per slab: 16 bf16, 64 fp8 (two 16-byte chunks per lane), 64
  // MXFP4 (one chunk per lane) or 64 MXFP6 (a chunk and a half) deep
  static constexpr int KSTEPS = FP4 ? 4 : (F8 ? 2 : 4);
  static constexpr int STAGE = OA::BYTES + OB::BYTES;

  // per-lane chunk offsets of slab 0 for both operands
  struct Offs {
    uint32_t a[OA::PER_WAVE], b[OB::PER_WAVE];
  };
  // Register staging: slab data in flight / waiting to be written to LDS.
  struct Stg {
    u32x4 a[OA::PER_WAVE], b[OB::PER_WAVE];
  };
  static __device__ __forceinline__ void gload(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, const GemmArgs& p,
                                               const Offs& d, int k0, Stg& g) {
    OA::gload(ra, d.a, OA::slab_bytes(p.lda, k0), g.a);
    OB::gload(rb, d.b, OB::slab_bytes(p.ldb, k0), g.b);
  }
  static __device__ __forceinline__ void lwrite_all(const Stg& g, LDS_AS char* st) {
#pragma unroll
    for (int q = 0; q < OA::PER_WAVE; ++q) OA::lwrite(g.a[q], q, st);
#pragma unroll
    for (int q = 0; q < OB::PER_WAVE; ++q) OB::lwrite(g.b[q], q, st + OA::BYTES);
  }
  // One staged chunk c (of the A chunks, then the B chunks): write it into wst,
  // then reload its register with the chunk of slab k1.
  static __device__ __forceinline__ void stage_chunk(int c, Stg& g, LDS_AS char* __restrict__ wst,
                                                     __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                                     const Offs& d, uint32_t kba, uint32_t kbb) {
    constexpr int NA = OA::PER_WAVE;
    if (c < NA) {
      OA::lwrite(g.a[c], c, wst);
      g.a[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(d.a[c] + kba), 0, 0));
    } else {
      OB::lwrite(g.b[c - NA], c - NA, wst + OA::BYTES);
      g.b[c - NA] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(d.b[c - NA] + kbb), 0, 0));
    }
  }

  // MXFP4 scales.  A slab (256 k of a row) has 8 scale bytes, one per 32 k; at
  // k step kk lane l takes the block 2*kk + l/32 of its row, as byte kk of one
  // word that the MFMA picks by op_sel.  Loads run two slabs ahead.  Plain
  // order: each lane loads the 8 bytes of each of its rows (one row per 32-row
  // block) and at the slab's start selects its four bytes into the word.  GEMM
  // order: the word of lane l is already at 4 l of the 32-row block's 256-byte
  // group of the slab, one coalesced dword load per row block.
  // MXFP6 slabs are 128 k: a word (256 k) serves two slabs, the first taking
  // its bytes 0 and 1, the second (shifted down by 16) bytes 2 and 3.
  static constexpr int NS = MX ? TM + TN : 1;
  using SW = std::conditional_t<GO, uint32_t, u32x2>;  // loaded per row block and slab
  struct Scl {
    uint32_t off[NS];  // byte offset of the lane's row (block) in its scale matrix
    SW cur[NS];        // the slab being multiplied
    SW nxt[NS];        // the next slab
    int par;           // MXFP6: parity of the slab being multiplied
  };
  // scale bytes per row: K/32 of K code bytes of two (MXFP4) or 4/3 (MXFP6) k each
  static __device__ __forceinline__ int scale_row_bytes(const GemmArgs& p) { return FP6 ? p.K / 24 : p.K / 16; }
  static __device__ __forceinline__ void scl_offsets(const GemmArgs& p, int m0, int n0, int wm, int wn, int lane,
                                                     Scl& sc) {
    const int ks = scale_row_bytes(p);
    sc.par = 0;
    if constexpr (GO) {
      // group (row / 32) * slabs + slab, 256 bytes each, 16 per row block per K / 2 code bytes
#pragma unroll
      for (int i = 0; i < TM; ++i) sc.off[i] = (uint32_t)((m0 + wm * WM + i * 32) * ks + lane * 4);
#pragma unroll
      for (int j = 0; j < TN; ++j) sc.off[TM + j] = (uint32_t)((n0 + wn * WN + j * 32) * ks + lane * 4);
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i) sc.off[i] = (uint32_t)((m0 + wm * WM + i * 32 + (lane & 31)) * ks);
#pragma unroll
      for (int j = 0; j < TN; ++j) sc.off[TM + j] = (uint32_t)((n0 + wn * WN + j * 32 + (lane & 31)) * ks);
    }
  }
  // scale bytes of the slab starting at code byte k0 (8 per row and slab)
  static __device__ __forceinline__ void scl_load(__amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb,
                                                  const Scl& sc, int k0, SW (&dst)[NS]) {
    if constexpr (GO) {
      // the 256-byte group of the slab's 256 k: 128 code bytes per MXFP4 slab;
      // two 96-byte MXFP6 slabs per group
      const uint32_t kb = FP6 ? ((uint32_t)k0 / 96 / 2) * 256 : (uint32_t)k0 * 2;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        dst[i] = __builtin_amdgcn_raw_buffer_load_b32(i < TM ? rsa : rsb, (int)(sc.off[i] + kb), 0, 0);
    } else {
      const uint32_t kb = (uint32_t)k0 / 16;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        dst[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(i < TM ? rsa : rsb,
                                                                                (int)(sc.off[i] + kb), 0, 0));
    }
  }

  // The operand fragments of one MFMA k step (16 deep for bf16, 64 for fp8,
  // whose fragments are two 16-byte chunks, and for MXFP4, whose fragments are
  // one chunk, with the slab's scale words).
  static constexpr int NF = (F8 && !MX) ? 2 : 1;
  struct Frags {
    u32x4 a[TM][NF], b[TN][NF];
    i32x8 a6[FP6 ? TM : 1], b6[FP6 ? TN : 1];  // MXFP6 fragments (in place of a, b)
    uint32_t s[NS];
  };
  static __device__ __forceinline__ void read_step(const LDS_AS char* __restrict__ st, int wm, int wn, int lane, int kk,
                                                   Frags& f) {
    const LDS_AS char* sa = st;
    const LDS_AS char* sb = st + OA::BYTES;
    if constexpr (FP6) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        u32x4 h;
        u32x2 t;
        OA::frag6(sa, wm * TM + i, kk, lane, h, t);
        f.a6[i] = mx6_operand(h, t);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        u32x4 h;
        u32x2 t;
        OB::frag6(sb, wn * TN + j, kk, lane, h, t);
        f.b6[j] = mx6_operand(h, t);
      }
    } else if constexpr (F8 != 0 && !FP4) {
#pragma unroll
      for (int i = 0; i < TM; ++i) OA::frag8(sa, wm * TM + i, kk, lane, f.a[i][0], f.a[i][1]);
#pragma unroll
      for (int j = 0; j < TN; ++j) OB::frag8(sb, wn * TN + j, kk, lane, f.b[j][0], f.b[j][1]);
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i) f.a[i][0] = OA::frag(sa, wm * TM + i, kk, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) f.b[j][0] = OB::frag(sb, wn * TN + j, kk, lane);
    }
  }
  // The operands go in swapped (B fragment first) so that a lane owns 4
  // consecutive output columns.  kk: the k step the fragments belong to (the
  // MXFP4 scale byte).
  static __device__ __forceinline__ void mfma_step(const Frags& f, f32x16 (&acc)[TM][TN], int kk) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (FP6)
          acc[i][j] = mfma32_mxfp6(f.b6[j], f.a6[i], acc[i][j], f.s[TM + j], f.s[i], kk);
        else if constexpr (FP4)
          acc[i][j] = mfma32_mxfp4(f.b[j][0], f.a[i][0], acc[i][j], f.s[TM + j], f.s[i], kk);
        else if constexpr (F8 != 0)
          acc[i][j] = mfma32_f8<FB, FA>(f.b[j][0], f.b[j][1], f.a[i][0], f.a[i][1], acc[i][j]);
        else
          acc[i][j] = mfma32(f.b[j][0], f.a[i][0], acc[i][j]);
      }
  }

  // One slab, with the MFMA stream running one k step behind the fragment
  // reads: step kk's fragments are read from st while step kk-1's MFMAs issue.
  // On entry f[1] holds the previous slab's last step (read before the barrier
  // that separates the slabs), so its MFMAs keep the matrix cores busy while
  // this slab's first fragments arrive; FIRST (no previous slab) skips them.
  // On exit f[1] holds this slab's last step, for the next slab or for finish().
  // With STAGE, the staged slab is written into wst chunk by chunk and each
  // staging register is reloaded with its chunk of slab k1 right behind.
  // MXFP4: sc.cur holds this slab's scale bytes and moves on to the next
  // slab's, whose own loads (of slab k1) are issued here.
  template <bool FIRST, bool STAGE>
  static __device__ __forceinline__ void slab(const LDS_AS char* __restrict__ st, int wm, int wn, int lane,
                                              f32x16 (&acc)[TM][TN], Frags (&f)[2], Stg& g,
                                              LDS_AS char* __restrict__ wst, __amdgpu_buffer_rsrc_t ra,
                                              __amdgpu_buffer_rsrc_t rb, const GemmArgs& p, const Offs& d, int k1,
                                              Scl& sc, __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb) {
    constexpr int NC = OA::PER_WAVE + OB::PER_WAVE;
    uint32_t kba = 0, kbb = 0;
    if constexpr (STAGE) {
      kba = OA::slab_bytes(p.lda, k1);
      kbb = OB::slab_bytes(p.ldb, k1);
    }
    uint32_t wsc[NS];
    if constexpr (MX) {
      const uint32_t sel = (lane >> 5) ? 0x07050301u : 0x06040200u;  // bytes 2*kk + lane/32
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if constexpr (FP6) wsc[i] = sc.cur[i] >> (16 * sc.par);
        else if constexpr (GO) wsc[i] = sc.cur[i];
        else wsc[i] = __builtin_amdgcn_perm(sc.cur[i][1], sc.cur[i][0], sel);
        sc.cur[i] = sc.nxt[i];
      }
      sc.par ^= 1;
      if constexpr (STAGE) scl_load(rsa, rsb, sc, k1, sc.nxt);
    }
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      read_step(st, wm, wn, lane, kk, f[kk & 1]);
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < NS; ++i) f[kk & 1].s[i] = wsc[i];
      }
      if (!(FIRST && kk == 0)) mfma_step(f[(kk & 1) ^ 1], acc, (kk + KSTEPS - 1) % KSTEPS);
      if constexpr (STAGE) {
#pragma unroll
        for (int c = kk * NC / KSTEPS; c < (kk + 1) * NC / KSTEPS; ++c) stage_chunk(c, g, wst, ra, rb, d, kba, kbb);
      }
    }
    // Schedule: each step's MFMAs with its fragment reads interleaved one for
    // one, and its share of the chunk writes and reloads spread evenly over them
    // (each reload right after its chunk's write).
    // LDS reads per step (an MXFP4 fragment is one read, an MXFP6 one two)
    constexpr int NR = FP6 ? 2 * (TM + TN) : (FP4 ? TM + TN : (TM * OA::READS + TN * OB::READS) * NF);
    constexpr int NM = TM * TN;                                 // MFMAs per step
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      // this step's chunk writes (and loads): the chunks staged in it above
      const int NW = STAGE ? (kk + 1) * NC / KSTEPS - kk * NC / KSTEPS : 0;
      const int STEP = NW == 0 ? NM + 1 : (NM / (2 * NW) > 0 ? NM / (2 * NW) : 1);
      if (FIRST && kk == 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        continue;
      }
#pragma unroll
      for (int x = 0; x < NM; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (x < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (x % STEP == STEP - 1 && x / STEP < 2 * NW) {
          if ((x / STEP) & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          else __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
      }
    }
  }
  // The last slab's last step.
  static __device__ __forceinline__ void finish(const Frags (&f)[2], f32x16 (&acc)[TM][TN]) {
    mfma_step(f[1], acc, KSTEPS - 1);
  }
};

// Row blocks the epilogue stages per pass: the largest divisor of tm that fits
// (a pass never reaches past the wave's last row block).
constexpr int rows_per_pass(int tm, int fit) {
  int r = fit < tm ? fit : tm;
  while (r > 1 && tm % r != 0) --r;
  return r;
}

// One output tile (workgroup index bid of the GEMM p) with the two LDS stages
// st0, st1 of the launching kernel.
template <int BM, int BN, bool A_K, bool B_K, int EPI, int F8, int NWN = 2>
__device__ __forceinline__ void gemm_tile(GemmArgs p, const int bid, LDS_AS char* st0, LDS_AS char* st1) {
  using ML = Mainloop<BM, BN, A_K, B_K, F8, NWN>;
  constexpr int EB = ML::EB, KSLAB = ML::KSLAB;
  constexpr int WM = ML::WM, WN = ML::WN, TM = ML::TM, TN = ML::TN;
  constexpr int OUT_BYTES = (EPI == EPI_F32 || EPI == EPI_F32_ACC) ? 4 : 2;

  int tm, tn;
  int64_t a_skip = 0, b_skip = 0;  // elements a k-split moves a k-contiguous operand's base by
  if (p.offsets == nullptr) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    int t = xcd_index(bid, F8 == 0 && p.ksplit > 1 ? ntiles * p.ksplit : ntiles);
    if constexpr (F8 == 0) {
      if (p.ksplit > 1) {  // part t / ntiles of the contraction, into its own fp32 output
        const int part = t / ntiles;
        t %= ntiles;
        const int k0 = part * p.k_chunk;
        p.K = min(p.K - k0, p.k_chunk);
        if (A_K) a_skip = k0;
        p.a += A_K ? (int64_t)k0 : (int64_t)k0 * p.lda;
        if (B_K) b_skip = k0;
        p.b += B_K ? (int64_t)k0 : (int64_t)k0 * p.ldb;
        p.c = reinterpret_cast<char*>(p.c) + (int64_t)part * p.split_stride_c * OUT_BYTES;
      }
    }
    constexpr int GM = 4;
    const int group = GM * tiles_n;
    const int first_m = (t / group) * GM;
    const int gm = min(tiles_m - first_m, GM);
    tm = first_m + (t % group) % gm;
    tn = (t % group) / gm;
  } else if (p.group_mode == GROUP_M) {
    // find this workgroup's expert among the per-expert row-tile counts
    const int tiles_n = (p.N + BN - 1) / BN;
    int w = bid, e = -1;
    for (int gi = 0; gi < p.groups; ++gi) {
      const int rows = p.offsets[gi + 1] - p.offsets[gi];
      const int span = ((rows + BM - 1) / BM) * tiles_n;
      if (w < span) {
        e = gi;
        break;
      }
      w -= span;
    }
    if (e < 0) return;  // beyond the grouped rows: nothing to do
    const int r0 = p.offsets[e];
    p.M = p.offsets[e + 1] - r0;
    p.a += (int64_t)r0 * p.lda;
    p.b += (int64_t)e * p.stride_b;
    p.c = reinterpret_cast<char*>(p.c) + (int64_t)r0 * p.ldc * OUT_BYTES;
    if (p.c2) p.c2 = reinterpret_cast<uint16_t*>(p.c2) + (int64_t)r0 * p.ldc2;
    if (p.aux) p.aux += (int64_t)r0 * p.ld_aux;
    tm = w / tiles_n;
    tn = w % tiles_n;
  } else {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int per = tiles_m * tiles_n;
    const int e = bid / per, w = bid % per;
    const int r0 = p.offsets[e];
    p.K = p.offsets[e + 1] - r0;
    p.a += (int64_t)r0 * p.lda;
    p.b += (int64_t)r0 * p.ldb;
    p.c = reinterpret_cast<char*>(p.c) + (int64_t)e * p.stride_c * OUT_BYTES;
    tm = w / tiles_n;
    tn = w % tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / NWN, wn = wave % NWN;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // Buffer resources: k-contiguous operands end after their last row (M or N),
  // mn-contiguous ones after row K, so everything past the matrix reads as 0.
  const __amdgpu_buffer_rsrc_t va = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.a), 0, (int)(((A_K ? (int64_t)p.M : (int64_t)p.K) * p.lda - a_skip) * EB), 0x00020000);
  const __amdgpu_buffer_rsrc_t vb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.b), 0, (int)(((B_K ? (int64_t)p.N : (int64_t)p.K) * p.ldb - b_skip) * EB), 0x00020000);
  const int nk = (p.K + KSLAB - 1) / KSLAB;
  typename ML::Offs off;
  ML::OA::offsets(p.lda, m0, off.a);
  ML::OB::offsets(p.ldb, n0, off.b);
  // MXFP4 scale matrices [M, K/32] and [N, K/32] (K/16 bytes per row, K in code
  // bytes); rows past M or N read as 0
  __amdgpu_buffer_rsrc_t vsa = va, vsb = vb;  // (unused by the other modes)
  typename ML::Scl sc;
  if constexpr (ML::MX) {  // (the same byte count in either order)
    const int64_t ks = ML::scale_row_bytes(p);
    vsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.mx_sa), 0, (int)(p.M * ks), 0x00020000);
    vsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.mx_sb), 0, (int)(p.N * ks), 0x00020000);
    ML::scl_offsets(p, m0, n0, wm, wn, lane, sc);
    ML::scl_load(vsa, vsb, sc, 0, sc.cur);
    if (nk > 1) ML::scl_load(vsa, vsb, sc, KSLAB, sc.nxt);
  }
  // Slab 0 goes to LDS now and slab 1 into the staging registers.  While slab
  // kt is multiplied, slab kt+1 is written from the registers into the other
  // stage and slab kt+2 is loaded behind it (slabs past K load in-range rows or
  // zeros and are never read); the last slab is multiplied alone.
  typename ML::Stg stg;
  ML::gload(va, vb, p, off, 0, stg);
  ML::lwrite_all(stg, st0);
  if (nk > 1) ML::gload(va, vb, p, off, KSLAB, stg);
  if (p.K < KSLAB) {  // each thread clears the k tail of the chunks it wrote
    ML::OA::zero_tail(st0, p.K);
    ML::OB::zero_tail(st0 + ML::OA::BYTES, p.K);
  }
  __syncthreads();
  typename ML::Frags fr[2];
  if (nk == 1) {
    ML::template slab<true, false>(st0, wm, wn, lane, acc, fr, stg, st1, va, vb, p, off, 0, sc, vsa, vsb);
  } else if (nk > 1) {
    // slab 0 (no previous step to finish), staging slab 1
    ML::template slab<true, true>(st0, wm, wn, lane, acc, fr, stg, st1, va, vb, p, off, 2 * KSLAB, sc, vsa, vsb);
    if (p.K - KSLAB < KSLAB) {
      ML::OA::zero_tail(st1, p.K - KSLAB);
      ML::OB::zero_tail(st1 + ML::OA::BYTES, p.K - KSLAB);
    }
    // No load in flight on entry to the loop: the staging loads of the peeled
    // slab above are issued in a different order than the loop's, and the
    // compiler, merging both orders at the loop head, would otherwise wait in
    // every iteration for the youngest of them (vmcnt(4) instead of vmcnt(15)
    // before the fifth chunk write of a 256 x 256 tile).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    for (int kt = 1; kt + 1 < nk; ++kt) {
      const bool odd = kt & 1;
      const LDS_AS char* st = odd ? st1 : st0;
      LDS_AS char* wst = odd ? st0 : st1;
      ML::template slab<false, true>(st, wm, wn, lane, acc, fr, stg, wst, va, vb, p, off, (kt + 2) * KSLAB, sc, vsa,
                                     vsb);
      const int kv = p.K - (kt + 1) * KSLAB;
      if (kv < KSLAB) {
        ML::OA::zero_tail(wst, kv);
        ML::OB::zero_tail(wst + ML::OA::BYTES, kv);
      }
      __syncthreads();
    }
    ML::template slab<false, false>((nk - 1) & 1 ? st1 : st0, wm, wn, lane, acc, fr, stg, st1, va, vb, p, off, 0, sc,
                                    vsa, vsb);
  }
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int mw = m0 + wm * WM, nw = n0 + wn * WN;
  // GeLU'(z) for the whole wave sub-tile, in the accumulator layout (4 columns
  // per load), requested before the last MFMAs so that the loads land under
  // them instead of one row block at a time in the epilogue.
  u32x2 zr[EPI == EPI_DGELU ? TM : 1][TN][4];
  if constexpr (EPI == EPI_DGELU) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mw + i * 32 + lrow;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = nw + j * 32 + 8 * g + 4 * lgrp;
          zr[i][j][g] = (m < p.M && n < p.N) ? *reinterpret_cast<const u32x2*>(p.aux + (int64_t)m * p.ld_aux + n)
                                             : u32x2{0, 0};
        }
    }
  }
  if (nk > 0) ML::finish(fr, acc);  // K = 0 (an empty expert): acc = 0

  // ---- epilogue ----------------------------------------------------------
  // Lane (lrow, lgrp) holds, for every (i, j, g), row i*32 + lrow and columns
  // j*32 + 8g + 4*lgrp .. +3 of the wave's WM x WN sub-tile.  Values are first
  // finished in registers (bias, GeLU, GeLU'), then written to the wave's own slice of
  // the (now idle) LDS stages and read back row by row, so every global store
  // is 16 bytes per lane over whole rows.  fp32 results, and the two outputs
  // of bias + GeLU, go in passes of IPP row blocks.  Stores are nontemporal
  // unless the caller keeps the output cached for the next kernel: a tile
  // round's outputs then stream out instead of filling the L2s with dirty lines
  // that the end of the kernel has to write back.
  __syncthreads();  // all waves are done with the last slab
  constexpr int HALF = ML::NWAVES / 2;  // waves whose staging slices lie in each stage
  constexpr int REGION = ML::STAGE / HALF;
  LDS_AS char* region = (wave < HALF ? st0 : st1) + (wave % HALF) * REGION;
  constexpr bool HAS_BIAS = (EPI == EPI_BF16_BIAS || EPI == EPI_BIAS_GELU);
  constexpr bool F32OUT = (EPI == EPI_F32 || EPI == EPI_F32_ACC);
  constexpr bool F32STAGE = F32OUT;
  constexpr int E = F32STAGE ? 4 : 2;
  constexpr int RB = WN * E;                 // bytes per staged row
  constexpr int CPR = RB / 16;               // 16-byte chunks per row
  // Outputs staged per pass: with bias + GeLU, C receives GeLU'(z) and C2
  // GeLU(z) of the biased sum z, both from one evaluation of the normal CDF and
  // density, staged side by side (each pass then covers half as many rows).
  constexpr int NOUT = EPI == EPI_BIAS_GELU ? 2 : 1;
  constexpr int IPP = rows_per_pass(TM, REGION / (NOUT * 32 * RB));
  constexpr int OUTB = IPP * 32 * RB;        // staged bytes of one output per pass
  static_assert(IPP >= 1, "epilogue staging does not fit");

  // fp8: the product of the two operands' dequantisation factors (MXFP4 scales
  // are applied by the MFMA)
  constexpr bool DQ = F8 != 0 && !ML::MX;
  float dq = 1.f;
  if constexpr (DQ) dq = *p.scale_a * *p.scale_b;
  // bias kept as packed bf16 (half the registers), widened where it is added
  u32x2 braw[TN][4];
  if constexpr (HAS_BIAS) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nw + j * 32 + 8 * g + 4 * lgrp;
        braw[j][g] = (p.bias && n < p.N) ? *reinterpret_cast<const u32x2*>(p.bias + n) : u32x2{0, 0};
      }
  }

  uint32_t amx = 0;  // largest bf16 magnitude stored of output p.amax_out
#pragma unroll
  for (int i0 = 0; i0 < TM; i0 += IPP) {
    // register phase
#pragma unroll
    for (int ii = 0; ii < IPP; ++ii) {
      const int i = i0 + ii;
      const int rl = ii * 32 + lrow;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4] = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          if constexpr (DQ) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= dq;
          }
          if constexpr (HAS_BIAS) {
            v[0] += bf16_lo(braw[j][g][0]);
            v[1] += bf16_hi(braw[j][g][0]);
            v[2] += bf16_lo(braw[j][g][1]);
            v[3] += bf16_hi(braw[j][g][1]);
          }
          float ge[4];  // GeLU(z), the second output
          if constexpr (EPI == EPI_BIAS_GELU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float cdf, pdf;
              normal_cdf_pdf(v[e], cdf, pdf);
              ge[e] = v[e] * cdf;
              v[e] = cdf + v[e] * pdf;  // GeLU'(z)
            }
          }
          if constexpr (EPI == EPI_DGELU) {  // aux holds GeLU'(z)
            v[0] *= bf16_lo(zr[i][j][g][0]);
            v[1] *= bf16_hi(zr[i][j][g][0]);
            v[2] *= bf16_lo(zr[i][j][g][1]);
            v[3] *= bf16_hi(zr[i][j][g][1]);
          }
          const int col = j * 32 + 8 * g + 4 * lgrp;
          if constexpr (F32STAGE) {
            const int ch = col / 4;
            const int pc = (ch + rl) % CPR;
            *reinterpret_cast<LDS_AS f32x4*>(region + rl * RB + pc * 16) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            const int ch = col / 8;
            const int pc = (ch + rl) % CPR;
            const int o = rl * RB + pc * 16 + (col & 7) * 2;
            *reinterpret_cast<LDS_AS u32x2*>(region + o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            if constexpr (NOUT == 2)
              *reinterpret_cast<LDS_AS u32x2*>(region + OUTB + o) =
                  u32x2{pack_bf16x2(ge[0], ge[1]), pack_bf16x2(ge[2], ge[3])};
          }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // row phase: chunk idx of the IPP*32 staged rows of each output
    constexpr int TOTAL = IPP * 32 * CPR;
#pragma unroll
    for (int out = 0; out < NOUT; ++out) {
#pragma unroll
      for (int it = 0; it < (TOTAL + 63) / 64; ++it) {
        const int idx = it * 64 + lane;
        if (TOTAL % 64 == 0 || idx < TOTAL) {
          const int rl = idx / CPR, ch = idx % CPR;
          const int pc = (ch + rl) % CPR;
          const u32x4 val = *reinterpret_cast<const LDS_AS u32x4*>(region + out * OUTB + rl * RB + pc * 16);
          const int m = mw + i0 * 32 + rl;
          const int n = nw + ch * (16 / E);
          if (m < p.M && n < p.N) {
            if constexpr (F32OUT) {
              float* c = reinterpret_cast<float*>(p.c) + (int64_t)m * p.ldc + n;
              f32x4 o = __builtin_bit_cast(f32x4, val);
              if constexpr (EPI == EPI_F32_ACC) o += *reinterpret_cast<const f32x4*>(c);
              if (p.keep_cached) *reinterpret_cast<f32x4*>(c) = o;
              else __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(c));
            } else {
              uint16_t* c = reinterpret_cast<uint16_t*>(out == 0 ? p.c : p.c2) +
                            (int64_t)m * (out == 0 ? p.ldc : p.ldc2) + n;
              if (p.keep_cached) *reinterpret_cast<u32x4*>(c) = val;
              else __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(c));
              if (p.amax_part && out == p.amax_out) {
#pragma unroll
                for (int w = 0; w < 4; ++w) amx = max(amx, max(val[w] & 0x7fffu, (val[w] >> 16) & 0x7fffu));
              }
            }
          }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if constexpr (!F32OUT) {
    if (p.amax_part) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) amx = max(amx, (uint32_t)__shfl_xor((int)amx, off));
      if (lane == 0) p.amax_part[bid * ML::NWAVES + wave] = amx;
    }
  }
}

// Entries of GemmArgs::amax_part a launch of `tiles` tiles of `waves` waves
// writes; false when they exceed the capacity (or the GEMM is grouped).
static bool amax_fits(const GemmArgs& p, int64_t tiles, int waves) {
  if (!p.amax_part) return true;
  if (p.offsets || tiles * waves > p.amax_cap) return false;
  if (p.amax_nparts) *p.amax_nparts = (int)(tiles * waves);
  return true;
}

template <int BM, int BN, bool A_K, bool B_K, int EPI, int F8 = 0, int NWN = 2>
__global__ __launch_bounds__(128 * NWN, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int STAGE = Mainloop<BM, BN, A_K, B_K, F8, NWN>::STAGE;
  __shared__ __attribute__((aligned(1024))) char st0_[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1_[STAGE];
  gemm_tile<BM, BN, A_K, B_K, EPI, F8, NWN>(p, blockIdx.x, (LDS_AS char*)st0_, (LDS_AS char*)st1_);
}

// A tile configuration of gemm_tile (F8 as in Mainloop: 0 = bf16 operands).
template <int BM_, int BN_, bool A_K_, bool B_K_, int EPI_, int F8_ = 0>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, EPI = EPI_, F8 = F8_;
  static constexpr bool A_K = A_K_, B_K = B_K_;
  static constexpr int STAGE = Mainloop<BM, BN, A_K, B_K, F8_>::STAGE;
};

// Two independent GEMMs in one launch: workgroups [0, tiles1) take p1, the rest
// p2.  With one tile per CU, the second GEMM's tiles start as the first GEMM's
// finish, so the first GEMM's output stores drain under the second's main loop
// instead of at a kernel boundary.  The weight-gradient GEMM (fp32 output,
// twice the bytes) is always the first of the pair.
//
// The order in which the workgroups take the two GEMMs' tiles: nseg == 0, all of
// GEMM 1's, then GEMM 2's; otherwise per XCD (workgroup bid runs on XCD bid % 8
// as its slot bid / 8 of that XCD's sequence) segments of count[k] consecutive
// slots that take the next tiles of GEMM 1 (kind 0) or GEMM 2 (kind 1).  Slot j
// of a GEMM's tiles on XCD x is its tile 8j + x, the tile gemm_tile places on
// that XCD, so each GEMM keeps its XCD-aware tile order.
constexpr int PAIR_MAX_SEG = 12;
struct PairOrder {
  int nseg;
  int kind[PAIR_MAX_SEG];
  int count[PAIR_MAX_SEG];
};

template <class C1, class C2>
__global__ __launch_bounds__(256, 1) void gemm_pair_kernel(GemmArgs p1, GemmArgs p2, int tiles1, PairOrder ord) {
  constexpr int STAGE = C1::STAGE > C2::STAGE ? C1::STAGE : C2::STAGE;
  __shared__ __attribute__((aligned(1024))) char st0_[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1_[STAGE];
  int bid = blockIdx.x;
  bool first = bid < tiles1;
  if (ord.nseg > 0) {
    const int slot = bid >> 3;
    int base = 0, done0 = 0, done1 = 0;
    for (int k = 0; k < ord.nseg; ++k) {
      if (slot < base + ord.count[k]) {
        first = ord.kind[k] == 0;
        bid = 8 * ((first ? done0 : done1) + slot - base) + (bid & 7);
        break;
      }
      base += ord.count[k];
      (ord.kind[k] == 0 ? done0 : done1) += ord.count[k];
    }
  } else if (!first) {
    bid -= tiles1;
  }
  if (first)
    gemm_tile<C1::BM, C1::BN, C1::A_K, C1::B_K, C1::EPI, C1::F8>(p1, bid, (LDS_AS char*)st0_, (LDS_AS char*)st1_);
  else
    gemm_tile<C2::BM, C2::BN, C2::A_K, C2::B_K, C2::EPI, C2::F8>(p2, bid, (LDS_AS char*)st0_, (LDS_AS char*)st1_);
}

// Makespan of one XCD's CUs taking jobs of duration w[kind] in the given order,
// each next job going to the CU that frees first.
static double pair_makespan(const std::vector<int>& order, const double* w, int cus) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < cus; ++i) free_at.push(0.0);
  double end = 0.0;
  for (int k : order) {
    const double t = free_at.top() + w[k];
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  return end;
}

// A dispatch order for n1 tiles of work w1 beside n2 tiles of work w2 (both
// multiples of 8; the hardware hands the next workgroup to the CU that frees
// first).  GEMM 1's tiles before GEMM 2's can leave the last round half empty
// (e.g. 48 tiles of 4 units and 64 of 3 per XCD of 32 CUs: 13 units where 12
// would do).  The plan dedicates c of an XCD's CUs to GEMM 1 and the others to
// GEMM 2, with c giving the smallest makespan, and lists the starts in time
// order; it is taken when it beats the plain order by 3% or more (or, for tiles
// of unequal work, the half-and-half split when it is no slower).
static PairOrder plan_pair_uncached(int64_t n1, double w1, int64_t n2, double w2);
// The plan depends only on the tile counts and works: each host thread keeps
// the last few it computed, so a step's launches do not repeat the simulation.
static PairOrder plan_pair(int64_t n1, double w1, int64_t n2, double w2) {
  struct Entry {
    int64_t n1, n2;
    double w1, w2;
    PairOrder o;
  };
  thread_local std::vector<Entry> cache;
  for (const Entry& e : cache)
    if (e.n1 == n1 && e.n2 == n2 && e.w1 == w1 && e.w2 == w2) return e.o;
  const PairOrder o = plan_pair_uncached(n1, w1, n2, w2);
  if (cache.size() >= 32) cache.erase(cache.begin());
  cache.push_back({n1, n2, w1, w2, o});
  return o;
}
static PairOrder plan_pair_uncached(int64_t n1, double w1, int64_t n2, double w2) {
  PairOrder none{};
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess)
      return 0;
    return n / 8;
  }();
  if (cus < 2 || n1 % 8 || n2 % 8 || n1 <= 0 || n2 <= 0 || n1 + n2 > 8 * 4096) return none;
  const int m1 = (int)(n1 / 8), m2 = (int)(n2 / 8);
  const double w[2] = {w1, w2};
  std::vector<int> plain(m1, 0);
  plain.insert(plain.end(), m2, 1);
  const double base = pair_makespan(plain, w, cus);
  double best = base;
  std::vector<int> best_order, half;
  for (int c = 1; c < cus; ++c) {
    // c CUs run GEMM 1's tiles, cus - c GEMM 2's; quotas as even as the counts allow
    std::vector<int> quota(cus), kind(cus);
    for (int i = 0; i < cus; ++i) {
      kind[i] = i < c ? 0 : 1;
      const int n = i < c ? m1 : m2, share = i < c ? c : cus - c, j = i < c ? i : i - c;
      quota[i] = n / share + (j < n % share ? 1 : 0);
    }
    using Ev = std::pair<double, int>;
    std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> ev;
    for (int i = 0; i < cus; ++i) ev.push({0.0, i});
    std::vector<int> order;
    while (!ev.empty()) {
      const Ev e = ev.top();
      ev.pop();
      if (quota[e.second]-- <= 0) continue;
      order.push_back(kind[e.second]);
      ev.push({e.first + w[kind[e.second]], e.second});
    }
    const double t = pair_makespan(order, w, cus);
    if (t < best) {
      best = t;
      best_order = order;
    }
    if (c == cus / 2 && w1 != w2 && t <= base) half = order;
  }
  // Tiles of unequal work whose plain order already fills the rounds (the fc2
  // backward: 512 wgrad tiles of K 4096, 256 dgrad tiles of K 8192) still gain
  // from half the CUs on each GEMM: the tiles then finish, and store their
  // outputs, at staggered times instead of all CUs at once (-2% on that launch).
  if (best_order.empty() || best > 0.97 * base) {
    if (half.empty()) return none;
    best_order = half;
  }
  PairOrder o{};
  for (size_t i = 0; i < best_order.size();) {
    size_t j = i;
    while (j < best_order.size() && best_order[j] == best_order[i]) ++j;
    if (o.nseg == PAIR_MAX_SEG) return none;
    o.kind[o.nseg] = best_order[i];
    o.count[o.nseg] = (int)(j - i);
    ++o.nseg;
    i = j;
  }
  return o;
}

template <int BM, int BN, bool A_K, bool B_K, int EPI, int F8 = 0, int NWN = 2>
static hipError_t launch_cfg(const GemmArgs& p, hipStream_t s) {
  int64_t tiles;
  if (p.offsets == nullptr) {
    tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  } else if (p.group_mode == GROUP_M) {
    // p.M carries the maximum number of grouped rows
    tiles = ((int64_t)(p.M + BM - 1) / BM + p.groups) * ((p.N + BN - 1) / BN);
  } else {
    tiles = (int64_t)p.groups * ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  }
  if (tiles <= 0) return hipSuccess;
  if (!amax_fits(p, tiles, 2 * NWN)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, A_K, B_K, EPI, F8, NWN>), dim3((unsigned)tiles), dim3(128 * NWN), 0, s, p);
  return hipGetLastError();
}

// 256 x 256 tiles run with 8 waves (two per SIMD, 128 x 64 each) when the
// epilogue evaluates GeLU or GeLU' for every element: the second wave on each
// SIMD hides the transcendental work and the z loads of the first (-7 to -10 us
// on 4096^3).  With light epilogues the 4-wave tile is as fast or faster.
template <bool A_K, bool B_K, int EPI>
static hipError_t launch_layout(const GemmArgs& p, hipStream_t s) {
  constexpr int NWN = (EPI == EPI_BIAS_GELU || EPI == EPI_DGELU) ? 4 : 2;
  if (p.offsets) return launch_cfg<256, 256, A_K, B_K, EPI, 0, NWN>(p, s);  // expert GEMMs are large
  const long t256 = (long)((p.M + 255) / 256) * ((p.N + 255) / 256);
  const long t192 = (long)((p.M + 255) / 256) * ((p.N + 191) / 192);
  if (t256 >= 240) return launch_cfg<256, 256, A_K, B_K, EPI, 0, NWN>(p, s);
  if (t192 >= 240 && p.N % 192 == 0) return launch_cfg<256, 192, A_K, B_K, EPI>(p, s);
  return launch_cfg<128, 128, A_K, B_K, EPI>(p, s);
}

// Tile shape launch_layout picks for a plain GEMM: 0 = 256x256, 1 = 256x192, 2 = 128x128.
static int tile_kind(const GemmArgs& p) {
  const long t256 = (long)((p.M + 255) / 256) * ((p.N + 255) / 256);
  const long t192 = (long)((p.M + 255) / 256) * ((p.N + 191) / 192);
  if (t256 >= 240) return 0;
  if (t192 >= 240 && p.N % 192 == 0) return 1;
  return 2;
}

template <class C1, class C2>
static hipError_t launch_pair(const GemmArgs& p1, const GemmArgs& p2, hipStream_t s) {
  const int64_t t1 = (int64_t)((p1.M + C1::BM - 1) / C1::BM) * ((p1.N + C1::BN - 1) / C1::BN) *
                     (C1::F8 == 0 && p1.ksplit > 1 ? p1.ksplit : 1);
  const int64_t t2 = (int64_t)((p2.M + C2::BM - 1) / C2::BM) * ((p2.N + C2::BN - 1) / C2::BN) *
                     (C2::F8 == 0 && p2.ksplit > 1 ? p2.ksplit : 1);
  if (!amax_fits(p1, t1, 4) || !amax_fits(p2, t2, 4)) return hipErrorInvalidValue;
  // relative work of one workgroup of each GEMM (its tile area times its contraction)
  const auto work = [](const GemmArgs& p, int bm, int bn) {
    const int k = p.ksplit > 1 ? p.k_chunk : p.K;
    return (double)bm * bn * k;
  };
  const PairOrder ord = plan_pair(t1, work(p1, C1::BM, C1::BN), t2, work(p2, C2::BM, C2::BN));
  hipLaunchKernelGGL((gemm_pair_kernel<C1, C2>), dim3((unsigned)(t1 + t2)), dim3(256), 0, s, p1, p2, (int)t1, ord);
  return hipGetLastError();
}

// The backward's independent pairs: dgrad (+GeLU') with wgrad, wgrad with dgrad.
template <int EPI_W>
static hipError_t pair_dispatch(const GemmArgs& p1, GemmLayout l1, int e1, const GemmArgs& p2, GemmLayout l2,
                                int e2, int k1, int k2, hipStream_t s, bool* done) {
  *done = true;
  using W256 = TileCfg<256, 256, false, false, EPI_W>;
  using W128 = TileCfg<128, 128, false, false, EPI_W>;
  if (l1 == GEMM_WGRAD && l2 == GEMM_DGRAD && k1 == 0 && k2 == 0 && e2 == EPI_DGELU)
    return launch_pair<W256, TileCfg<256, 256, true, true, EPI_DGELU>>(p1, p2, s);
  if (l1 == GEMM_WGRAD && l2 == GEMM_DGRAD && k1 == 0 && k2 == 0)
    return launch_pair<W256, TileCfg<256, 256, true, true, EPI_BF16>>(p1, p2, s);
  if (l1 == GEMM_WGRAD && l2 == GEMM_DGRAD && k1 == 2 && k2 == 2 && e2 == EPI_BF16)
    return launch_pair<W128, TileCfg<128, 128, true, true, EPI_BF16>>(p1, p2, s);
  // A 256 x 192 wgrad beside a 256 x 256 dgrad (the QKV projection's pair) runs
  // faster as two launches: 185 against 203 us side by side at the 7B-class shape.
  *done = false;
  return hipSuccess;
}

hipError_t gemm_bf16_pair(const GemmArgs& p1, GemmLayout l1, int e1, const GemmArgs& p2, GemmLayout l2, int e2,
                          hipStream_t s) {
  // combinations without a fused kernel run as two launches
  const bool plain = !p1.offsets && !p2.offsets && p1.M > 0 && p1.N > 0 && p1.K > 0 && p2.M > 0 && p2.N > 0 &&
                     p2.K > 0;
  const bool wgrad_ok = (l1 == GEMM_WGRAD) ? (e1 == EPI_F32 || e1 == EPI_F32_ACC)
                                           : (l2 == GEMM_WGRAD && (e2 == EPI_F32 || e2 == EPI_F32_ACC));
  const bool dgrad_ok = (l1 == GEMM_DGRAD) ? (e1 == EPI_BF16 || e1 == EPI_DGELU)
                                           : (l2 == GEMM_DGRAD && (e2 == EPI_BF16 || e2 == EPI_DGELU));
  const bool fits = [&] {  // the same 32-bit offset bound gemm_bf16 checks
    for (const GemmArgs* q : {&p1, &p2}) {
      const bool wg = (q == &p1 ? l1 : l2) == GEMM_WGRAD;
      const int64_t ar = (wg ? (int64_t)q->K : (int64_t)q->M) + 256, br = (int64_t)(wg ? q->K : q->N) + 256;
      if (ar * q->lda * 2 >= ((int64_t)1 << 32) || br * q->ldb * 2 >= ((int64_t)1 << 32)) return false;
    }
    return true;
  }();
  if (plain && wgrad_ok && dgrad_ok && fits && l1 != l2) {
    const int ew = l1 == GEMM_WGRAD ? e1 : e2;
    bool done = false;
    hipError_t e = ew == EPI_F32
                       ? pair_dispatch<EPI_F32>(p1, l1, e1, p2, l2, e2, tile_kind(p1), tile_kind(p2), s, &done)
                       : pair_dispatch<EPI_F32_ACC>(p1, l1, e1, p2, l2, e2, tile_kind(p1), tile_kind(p2), s, &done);
    if (done) return e;
  }
  hipError_t e = gemm_bf16(p1, l1, e1, s);
  if (e != hipSuccess) return e;
  return gemm_bf16(p2, l2, e2, s);
}

// The weight gradient p1 (fp32 epilogue e1) beside the data gradient p2 cut in
// p2.ksplit parts along its contraction, each part an fp32 output of its own
// (the caller sums them): one launch of 256 x 256 tiles.  A data gradient with
// few output tiles and a long contraction then fills the chip with equal tiles
// instead of running on 128 x 128 tiles.
hipError_t gemm_bf16_pair_ksplit(const GemmArgs& p1, int e1, const GemmArgs& p2, hipStream_t s) {
  if (p1.offsets || p2.offsets || p1.ksplit > 1 || p2.ksplit < 2 || p2.k_chunk <= 0 || p2.k_chunk % 64 != 0 ||
      (int64_t)p2.k_chunk * (p2.ksplit - 1) >= p2.K || (int64_t)p2.k_chunk * p2.ksplit < p2.K)
    return hipErrorInvalidValue;
  if (p1.M <= 0 || p1.N <= 0 || p1.K <= 0 || p2.M <= 0 || p2.N <= 0) return hipErrorInvalidValue;
  // the 32-bit buffer offsets gemm_bf16 checks (wgrad: rows K of both operands; dgrad: M and N)
  if (((int64_t)p1.K + 256) * p1.lda * 2 >= ((int64_t)1 << 32) || ((int64_t)p1.K + 256) * p1.ldb * 2 >= ((int64_t)1 << 32) ||
      ((int64_t)p2.M + 256) * p2.lda * 2 >= ((int64_t)1 << 32) || ((int64_t)p2.N + 256) * p2.ldb * 2 >= ((int64_t)1 << 32))
    return hipErrorInvalidValue;
  using D = TileCfg<256, 256, true, true, EPI_F32>;
  if (e1 == EPI_F32) return launch_pair<TileCfg<256, 256, false, false, EPI_F32>, D>(p1, p2, s);
  if (e1 == EPI_F32_ACC) return launch_pair<TileCfg<256, 256, false, false, EPI_F32_ACC>, D>(p1, p2, s);
  return hipErrorInvalidValue;
}

int64_t gemm_group_m_grid(int64_t max_rows, int groups, int N) {
  return ((max_rows + 255) / 256 + groups) * ((N + 255) / 256);
}

hipError_t gemm_bf16(const GemmArgs& p, GemmLayout layout, int epi, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  // Operands are addressed through raw buffer resources with 32-bit byte
  // offsets; a tile may run up to 256 rows (or 64 k) past the matrix.
  const bool a_k = layout != GEMM_WGRAD, b_k = layout == GEMM_DGRAD;
  const int64_t a_rows = (a_k ? (int64_t)p.M : (int64_t)p.K) + 256, b_rows = (b_k ? (int64_t)p.N : (int64_t)p.K) + 256;
  if (a_rows * p.lda * 2 >= ((int64_t)1 << 32) || b_rows * p.ldb * 2 >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  if (p.K <= 0 && !(p.offsets && p.group_mode == GROUP_K)) return hipErrorInvalidValue;
  switch (layout) {
    case GEMM_FWD:  // A k-contig, B n-contig
      if (epi == EPI_BF16) return launch_layout<true, false, EPI_BF16>(p, s);
      if (epi == EPI_BF16_BIAS) return launch_layout<true, false, EPI_BF16_BIAS>(p, s);
      if (epi == EPI_BIAS_GELU) return launch_layout<true, false, EPI_BIAS_GELU>(p, s);
      if (epi == EPI_F32) return launch_layout<true, false, EPI_F32>(p, s);  // fp32 logits of the MoE router
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

template <int EPI, int F8>
static hipError_t launch_f8(const GemmArgs& p, hipStream_t s) {
  const long t256 = (long)((p.M + 255) / 256) * ((p.N + 255) / 256);
  const long t192 = (long)((p.M + 255) / 256) * ((p.N + 191) / 192);
  if (t256 >= 240) return launch_cfg<256, 256, true, true, EPI, F8>(p, s);
  // forward products 192 columns wide fill the chip with 256 x 192 tiles (the
  // fused QKV projection: 256 tiles instead of 768 of 128 x 128)
  if constexpr (F8 == 1)
    if (t192 >= 240 && p.N % 192 == 0) return launch_cfg<256, 192, true, true, EPI, F8>(p, s);
  return launch_cfg<128, 128, true, true, EPI, F8>(p, s);
}

static bool fp8_args_ok(const GemmArgs& p) {
  if (p.offsets || p.K <= 0 || p.K % 16 || p.lda % 16 || p.ldb % 16 || !p.scale_a || !p.scale_b) return false;
  return ((int64_t)p.M + 256) * p.lda < ((int64_t)1 << 32) && ((int64_t)p.N + 256) * p.ldb < ((int64_t)1 << 32);
}

// The backward's independent fp8 pairs in one launch, wgrad tiles (E4M3 x E5M2,
// fp32 output) first, dgrad tiles (E5M2 x E4M3, bf16 output) second, where both
// take 128 x 128 tiles (the output projection's pair at the 7B-class shape:
// 51 -> 40 us).  Pairs with a 256 x 256 half ran slower as one launch than as
// two (4096^3 pairs +8-10%; a 128 x 128 wgrad beside a 256 x 256 dgrad +19%,
// its tiles then holding the larger LDS footprint, one workgroup per CU instead
// of two), so they stay two launches.
template <int EPI_W>
static hipError_t fp8_pair_dispatch(const GemmArgs& pw, const GemmArgs& pd, int epi_d, hipStream_t s, bool* done) {
  *done = false;
  const bool w256 = (long)((pw.M + 255) / 256) * ((pw.N + 255) / 256) >= 240;
  const bool d256 = (long)((pd.M + 255) / 256) * ((pd.N + 255) / 256) >= 240;
  if (w256 || d256 || epi_d != EPI_BF16) return hipSuccess;
  *done = true;
  return launch_pair<TileCfg<128, 128, true, true, EPI_W, 3>, TileCfg<128, 128, true, true, EPI_BF16, 2>>(pw, pd, s);
}

hipError_t gemm_fp8_pair(const GemmArgs& pw, int epi_w, const GemmArgs& pd, int epi_d, hipStream_t s) {
  const bool plain = pw.M > 0 && pw.N > 0 && pd.M > 0 && pd.N > 0 && fp8_args_ok(pw) && fp8_args_ok(pd);
  if (plain && (epi_w == EPI_F32 || epi_w == EPI_F32_ACC)) {
    bool done = false;
    hipError_t e = epi_w == EPI_F32 ? fp8_pair_dispatch<EPI_F32>(pw, pd, epi_d, s, &done)
                                    : fp8_pair_dispatch<EPI_F32_ACC>(pw, pd, epi_d, s, &done);
    if (done) return e;
  }
  hipError_t e = gemm_fp8(pw, 0, 1, epi_w, s);
  if (e != hipSuccess) return e;
  return gemm_fp8(pd, 1, 0, epi_d, s);
}

// MXFP4 x MXFP4 on the same pipeline.  K, lda and ldb count code bytes (two k
// per byte); a slab is 128 code bytes = 256 k = 8 scale blocks per row.
template <int EPI, int F8>
static hipError_t launch_mx(const GemmArgs& p, hipStream_t s) {
  const long t256 = (long)((p.M + 255) / 256) * ((p.N + 255) / 256);
  const long t192 = (long)((p.M + 255) / 256) * ((p.N + 191) / 192);
  if (t256 >= 240) return launch_cfg<256, 256, true, true, EPI, F8>(p, s);
  if (t192 >= 240 && p.N % 192 == 0) return launch_cfg<256, 192, true, true, EPI, F8>(p, s);
  return launch_cfg<128, 128, true, true, EPI, F8>(p, s);
}

// The GEMM arguments of an MXFP4 product (K, lda, ldb in code bytes).
static GemmArgs mx_gemm_args(const Mxfp4GemmArgs& g) {
  const int64_t kb = g.K / 2;  // code bytes per row
  GemmArgs p{};
  p.a = reinterpret_cast<const uint16_t*>(g.a);
  p.b = reinterpret_cast<const uint16_t*>(g.b);
  p.lda = p.ldb = kb;
  p.M = g.M;
  p.N = g.N;
  p.K = (int)kb;
  p.ldc = p.ldc2 = p.ld_aux = g.ldc;
  p.c = (g.epi == EPI_F32 || g.epi == EPI_F32_ACC) ? static_cast<void*>(g.c32) : static_cast<void*>(g.c);
  p.bias = g.bias;
  p.c2 = g.c2;
  p.aux = g.aux;
  p.mx_sa = g.sa;
  p.mx_sb = g.sb;
  p.keep_cached = g.keep_cached;
  return p;
}

hipError_t gemm_mxfp4_tiled(const Mxfp4GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  if (g.K % 256) return hipErrorInvalidValue;
  const int64_t kb = g.K / 2;  // code bytes per row
  if (((int64_t)g.M + 256) * kb >= ((int64_t)1 << 31) || ((int64_t)g.N + 256) * kb >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  const GemmArgs p = mx_gemm_args(g);
  if (!g.scale_order) return g.epi == EPI_BF16 ? launch_mx<EPI_BF16, F8_MXFP4>(p, s) : hipErrorInvalidValue;
  if (g.M % 32 || g.N % 32) return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_BF16: return launch_mx<EPI_BF16, F8_MXFP4_GO>(p, s);
    case EPI_BF16_BIAS: return launch_mx<EPI_BF16_BIAS, F8_MXFP4_GO>(p, s);
    case EPI_BIAS_GELU: return launch_mx<EPI_BIAS_GELU, F8_MXFP4_GO>(p, s);
    case EPI_DGELU: return launch_mx<EPI_DGELU, F8_MXFP4_GO>(p, s);
    case EPI_F32: return launch_mx<EPI_F32, F8_MXFP4_GO>(p, s);
    case EPI_F32_ACC: return launch_mx<EPI_F32_ACC, F8_MXFP4_GO>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t gemm_mxfp4_pair(const Mxfp4GemmArgs& gw, const Mxfp4GemmArgs& gd, hipStream_t s) {
  // both on 256 x 256 tiles, GEMM-order scales: one launch (gemm_pair_kernel)
  const auto fused = [](const Mxfp4GemmArgs& g) {
    return g.M > 0 && g.N > 0 && g.K > 0 && g.K % 256 == 0 && g.M % 32 == 0 && g.N % 32 == 0 && g.scale_order &&
           (long)((g.M + 255) / 256) * ((g.N + 255) / 256) >= 240 &&
           ((int64_t)g.M + 256) * (g.K / 2) < ((int64_t)1 << 31) && ((int64_t)g.N + 256) * (g.K / 2) < ((int64_t)1 << 31);
  };
  if (fused(gw) && fused(gd) && (gw.epi == EPI_F32 || gw.epi == EPI_F32_ACC) &&
      (gd.epi == EPI_BF16 || gd.epi == EPI_DGELU)) {
    const GemmArgs pw = mx_gemm_args(gw), pd = mx_gemm_args(gd);
    constexpr int G = F8_MXFP4_GO;
    if (gw.epi == EPI_F32) {
      using W = TileCfg<256, 256, true, true, EPI_F32, G>;
      return gd.epi == EPI_DGELU ? launch_pair<W, TileCfg<256, 256, true, true, EPI_DGELU, G>>(pw, pd, s)
                                 : launch_pair<W, TileCfg<256, 256, true, true, EPI_BF16, G>>(pw, pd, s);
    }
    using W = TileCfg<256, 256, true, true, EPI_F32_ACC, G>;
    return gd.epi == EPI_DGELU ? launch_pair<W, TileCfg<256, 256, true, true, EPI_DGELU, G>>(pw, pd, s)
                               : launch_pair<W, TileCfg<256, 256, true, true, EPI_BF16, G>>(pw, pd, s);
  }
  hipError_t e = gemm_mxfp4_tiled(gd, s);
  if (e != hipSuccess) return e;
  return gemm_mxfp4_tiled(gw, s);
}

hipError_t gemm_mxfp6_tiled(const Mxfp4GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  if (g.K % 256 || g.M % 32 || g.N % 32 || g.epi != EPI_BF16) return hipErrorInvalidValue;
  const int64_t kb = (int64_t)g.K * 3 / 4;  // code bytes per row
  if (((int64_t)g.M + 256) * kb >= ((int64_t)1 << 31) || ((int64_t)g.N + 256) * kb >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  GemmArgs p{};
  p.a = reinterpret_cast<const uint16_t*>(g.a);
  p.b = reinterpret_cast<const uint16_t*>(g.b);
  p.lda = p.ldb = kb;
  p.M = g.M;
  p.N = g.N;
  p.K = (int)kb;
  p.ldc = g.ldc;
  p.c = g.c;
  p.mx_sa = g.sa;
  p.mx_sb = g.sb;
  return launch_mx<EPI_BF16, F8_MXFP6_GO>(p, s);
}

hipError_t gemm_fp8(const GemmArgs& p, int fmt_a, int fmt_b, int epi, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (!fp8_args_ok(p)) return hipErrorInvalidValue;
  const int f8 = 1 + fmt_a + 2 * fmt_b;
  if (f8 == 1) {  // forward: E4M3 x E4M3
    if (epi == EPI_BF16) return launch_f8<EPI_BF16, 1>(p, s);
    if (epi == EPI_BF16_BIAS) return launch_f8<EPI_BF16_BIAS, 1>(p, s);
    if (epi == EPI_BIAS_GELU) return launch_f8<EPI_BIAS_GELU, 1>(p, s);
  } else if (f8 == 2) {  // dgrad: E5M2 gradient x E4M3 weight
    if (epi == EPI_BF16) return launch_f8<EPI_BF16, 2>(p, s);
    if (epi == EPI_DGELU) return launch_f8<EPI_DGELU, 2>(p, s);
  } else if (f8 == 3) {  // wgrad: E4M3 activation x E5M2 gradient
    if (epi == EPI_F32) return launch_f8<EPI_F32, 3>(p, s);
    if (epi == EPI_F32_ACC) return launch_f8<EPI_F32_ACC, 3>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mtl
