// bf16 MFMA main loop of the projection GEMMs, and the LDS-DMA pieces of the output head.
//
// C[m, n] = sum_k A[m, k] * B[n, k]: both operands are K-contiguous ("NT"), as
// every weight here is stored [out, in].  One workgroup computes a BM x BN tile
// with WM x WN wavefronts; each wave owns a (BM/WM) x (BN/WN) sub-tile made of
// 16x16 blocks of v_mfma_f32_16x16x32_bf16.  K advances in steps of 64 through a
// double-buffered LDS stage; the next stage's global loads are issued before the
// current stage's MFMAs so their latency hides behind the matrix cores.
//
// MFMA 16x16x32 operand layout (lane l of 64): A supplies row l%16 with the 8
// consecutive k values starting at 8*(l/16); B supplies column l%16 with the same
// k values; the result lane l holds D[4*(l/16) + i][l%16] in element i.
#pragma once

#include <type_traits>

#include "tcs_device.h"

namespace tcs {

constexpr int GEMM_BK = 64;
constexpr int GEMM_LDK = GEMM_BK + 8;  // padded LDS row (bf16 elements): 144 bytes

template <int BM, int BN, int WM, int WN>
struct GemmShape {
  static constexpr int NT = 64 * WM * WN;  // threads
  static constexpr int TM = BM / WM;       // wave tile rows
  static constexpr int TN = BN / WN;       // wave tile cols
  static constexpr int MB = TM / 16;       // 16x16 blocks per wave (rows)
  static constexpr int NB = TN / 16;       // 16x16 blocks per wave (cols)
  static constexpr int A_CHUNKS = BM * (GEMM_BK / 8) / NT;   // 16-byte chunks per thread
  static constexpr int B_CHUNKS = BN * (GEMM_BK / 8) / NT;
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * GEMM_LDK;  // bf16 elements, both stages
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile");
  static_assert(A_CHUNKS * NT == BM * 8 && B_CHUNKS * NT == BN * 8, "chunking");
};

// Tile index of this workgroup: blocks are first remapped so that each of the 8
// XCDs (block i runs on XCD i % 8) owns a contiguous range of tiles, then ordered
// in groups of GROUP_M row tiles that sweep the column tiles, so concurrently
// running workgroups share operand tiles in their XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int nbm, int nbn, int& mt, int& nt) {
  const int total = nbm * nbn;
  const int bid = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int lin = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int gsize = GROUP_M * nbn;
  const int group = lin / gsize;
  const int first_m = group * GROUP_M;
  const int gm = min(nbm - first_m, GROUP_M);
  const int in_group = lin - group * gsize;
  mt = first_m + in_group % gm;
  nt = in_group / gm;
}

// Main loop.  A: bf16 [M, lda]; B: bf16 [N, ldb].
// K % 64 == 0.  Rows of A or B at or beyond M / N read as zero.  A tile's rows
// must span fewer than 2^31 bytes.
//
// Software pipeline, one barrier per K tile:
//   [global loads of tile t+1] [LDS reads of step 1 of tile t  | MFMAs of step 0]
//   [stores of tile t+1 to the other LDS buffer] barrier
//   [LDS reads of step 0 of tile t+1 | MFMAs of step 1 of tile t]
// so every LDS fragment read is in flight under a block of MFMAs, and the global
// loads have a whole block of MFMAs to land.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void gemm_mainloop(const uint16_t* __restrict__ A, int lda,
                                              const void* __restrict__ Bv, int ldb, int M, int N,
                                              int K, int m0, int n0, uint16_t* lds,
                                              f32x4 (&acc)[BM / WM / 16][BN / WN / 16]) {
  using S = GemmShape<BM, BN, WM, WN>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  uint16_t* sA = lds;                          // [2][BM][LDK]
  uint16_t* sB = lds + 2 * BM * GEMM_LDK;      // [2][BN][LDK]

#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int j = 0; j < S::NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int RB = S::B_CHUNKS;
  uint4 ra[S::A_CHUNKS];
  uint4 rb[RB];
  // Buffer resources over this tile's rows: the hardware bounds check returns
  // zeros past the last valid row, and each chunk differs from the previous one by
  // a uniform byte stride, so only one per-thread offset register is needed.
  constexpr uint32_t RSRC_W3 = 0x00020000u;  // gfx9-family raw buffer descriptor word 3
  const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A + (size_t)m0 * lda), 0, a_rows * lda * 2, RSRC_W3);
  constexpr int B_ES = 2;  // bytes per B element
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(Bv) + (size_t)n0 * ldb * B_ES), 0,
      b_rows * ldb * B_ES, RSRC_W3);
  const int voffA = ((tid >> 3) * lda + (tid & 7) * 8) * 2;
  const int strideA = (S::NT / 8) * lda * 2;
  const int voffB = ((tid >> 3) * ldb + (tid & 7) * 8) * 2;
  const int strideB = (S::NT / 8) * ldb * 2;
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < S::A_CHUNKS; ++i) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rsA, voffA, k0 * 2 + i * strideA, 0);
      ra[i] = *reinterpret_cast<uint4*>(&v);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rsB, voffB, k0 * B_ES + i * strideB, 0);
      rb[i] = *reinterpret_cast<uint4*>(&v);
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* a = sA + buf * BM * GEMM_LDK;
    uint16_t* b = sB + buf * BN * GEMM_LDK;
#pragma unroll
    for (int i = 0; i < S::A_CHUNKS; ++i) {
      const int c = tid + i * S::NT;
      *reinterpret_cast<uint4*>(a + (c >> 3) * GEMM_LDK + (c & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int c = tid + i * S::NT;
      *reinterpret_cast<uint4*>(b + (c >> 3) * GEMM_LDK + (c & 7) * 8) = rb[i];
    }
  };
  bf16x8 fa[2][S::MB], fb[2][S::NB];
  auto read_frags = [&](int buf, int kk, bf16x8 (&xa)[S::MB], bf16x8 (&xb)[S::NB]) {
    const uint16_t* a = sA + buf * BM * GEMM_LDK;
    const uint16_t* b = sB + buf * BN * GEMM_LDK;
    const int kof = kk * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
      xa[i] = *reinterpret_cast<const bf16x8*>(a + (wm * S::TM + i * 16 + (lane & 15)) * GEMM_LDK + kof);
#pragma unroll
    for (int j = 0; j < S::NB; ++j)
      xb[j] = *reinterpret_cast<const bf16x8*>(b + (wn * S::TN + j * 16 + (lane & 15)) * GEMM_LDK + kof);
  };
  auto mfma_block = [&](const bf16x8 (&xa)[S::MB], const bf16x8 (&xb)[S::NB]) {
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int j = 0; j < S::NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], xb[j], acc[i][j], 0, 0, 0);
  };
  constexpr int NFRAG = S::MB + S::NB;
  constexpr int NMFMA = S::MB * S::NB;

  const int nk = K / GEMM_BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  read_frags(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int knext = min(kt + 1, nk - 1) * GEMM_BK;
    load_stage(knext);
    read_frags(cur, 1, fa[1], fb[1]);
    mfma_block(fa[0], fb[0]);
    // interleave: global loads and LDS reads spread across the MFMAs
#pragma unroll
    for (int g = 0; g < NFRAG; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, NMFMA / NFRAG, 0);  // MFMA
    }
    store_stage(cur ^ 1);
    __syncthreads();
    read_frags(cur ^ 1, 0, fa[0], fb[0]);
    mfma_block(fa[1], fb[1]);
#pragma unroll
    for (int g = 0; g < NFRAG; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NMFMA / NFRAG, 0);
    }
  }
  __syncthreads();  // LDS is free for the caller's epilogue
}


// ---------------------------------------------------------------------------
// Pieces of the LDS-DMA pipeline used by the output head (k_lmhead.hip).
//
// K advances in tiles of 64: each operand row contributes 128 contiguous bytes per
// tile, so every L1->L2 request is a full 128-byte line (measured on MI355X: about
// 1.8x the per-CU bandwidth of 64-byte requests).  A slot holds one 256-row operand
// tile (32 KB); in a slot, the eight 16-byte chunks of row r sit at positions
// chunk ^ swz(r mod 16), which spreads the rows read by each group of lanes over
// distinct LDS banks.
constexpr int DMA_BK = 64;
constexpr int DMA_SLOT_BYTES = 256 * DMA_BK * 2;  // one operand tile, bf16: 32 KB
constexpr int DMA_SLOTS = 5;

__device__ __forceinline__ int dma_swz(int r) { return (r ^ (r >> 3)) & 7; }  // r in [0, 16)


// Output-head tile order: tile slot `bid` = 256 w + b is the w-th tile of the
// persistent workgroup b (one per CU; b runs on XCD b % 8).  Row tiles go in full
// groups of 32 while they last: a round covers a 32 x 8 block of (row, column)
// tiles, each XCD a 4 x 8 sub-block, so its L2 serves both operands and all XCDs
// share the block's 8 weight tiles through the MALL.  The rem = nbm mod 32 row
// tiles left over (all of them when nbm < 32) are cut into strips of at most 8
// rows and enumerated densely, tile u of a strip of h rows at (u mod h, u / h):
// every round but the last is full, and an XCD's 32 consecutive tiles span h rows
// by about 32/h columns.  Returns false for slots past the matrix edge.
__device__ __forceinline__ bool head_tile_coords(int bid, int nbm, int nbn, int& mt, int& nt) {
  const int xcd = bid & 7, slot = (bid >> 3) & 31, w = bid >> 8;
  const int G = nbm >> 5, nbc = (nbn + 7) >> 3;  // full row groups, 8-column blocks
  if (w < G * nbc) {
    const int g = w / nbc, nb = w - g * nbc;
    mt = g * 32 + xcd * 4 + (slot & 3);
    nt = nb * 8 + (slot >> 2);
    return nt < nbn;
  }
  const int rem = nbm - G * 32;
  if (rem <= 0) return false;
  const int u = (w - G * nbc) * 256 + xcd * 32 + slot;
  const int ns = (rem + 7) >> 3, hs = (rem + ns - 1) / ns;  // strips, rows per strip
  const int s = min(u / (hs * nbn), ns - 1);
  const int h = min(hs, rem - s * hs);  // the last strip may be shorter
  const int loc = u - s * hs * nbn;
  mt = G * 32 + s * hs + loc % h;
  nt = loc / h;
  return nt < nbn;
}

// Slots (a multiple of 256) that head_tile_coords spreads the nbm x nbn tiles over.
__host__ __device__ inline int head_grid(int nbm, int nbn) {
  const int G = nbm >> 5, nbc = (nbn + 7) >> 3, rem = nbm - G * 32;
  return (G * nbc + (rem * nbn + 255) / 256) * 256;
}

}  // namespace tcs
