// bf16 MFMA main loop shared by the projection GEMMs and the output head.
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
  static constexpr int B8_CHUNKS = BN * (GEMM_BK / 16) / NT; // fp8 B: 16 elements per chunk
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

// Main loop.  A: bf16 [M, lda]; B: bf16 [N, ldb] or (B_FP8) E4M3 bytes [N, ldb].
// Rows of A or B beyond M / N read as zero.  K % 64 == 0.
template <int BM, int BN, int WM, int WN, bool B_FP8>
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

  uint4 ra[S::A_CHUNKS];
  constexpr int RB = B_FP8 ? S::B8_CHUNKS : S::B_CHUNKS;
  uint4 rb[RB];

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < S::A_CHUNKS; ++i) {
      const int c = tid + i * S::NT;
      const int row = c >> 3, col = (c & 7) * 8;
      const int gr = m0 + row;
      ra[i] = gr < M ? *reinterpret_cast<const uint4*>(A + (size_t)gr * lda + k0 + col)
                     : uint4{0, 0, 0, 0};
    }
    if constexpr (B_FP8) {
      const uint8_t* B = static_cast<const uint8_t*>(Bv);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int c = tid + i * S::NT;
        const int row = c >> 2, col = (c & 3) * 16;
        const int gr = n0 + row;
        rb[i] = gr < N ? *reinterpret_cast<const uint4*>(B + (size_t)gr * ldb + k0 + col)
                       : uint4{0, 0, 0, 0};
      }
    } else {
      const uint16_t* B = static_cast<const uint16_t*>(Bv);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int c = tid + i * S::NT;
        const int row = c >> 3, col = (c & 7) * 8;
        const int gr = n0 + row;
        rb[i] = gr < N ? *reinterpret_cast<const uint4*>(B + (size_t)gr * ldb + k0 + col)
                       : uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* a = sA + buf * BM * GEMM_LDK;
    uint16_t* b = sB + buf * BN * GEMM_LDK;
#pragma unroll
    for (int i = 0; i < S::A_CHUNKS; ++i) {
      const int c = tid + i * S::NT;
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<uint4*>(a + row * GEMM_LDK + col) = ra[i];
    }
    if constexpr (B_FP8) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int c = tid + i * S::NT;
        const int row = c >> 2, col = (c & 3) * 16;
        const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[2 * q] = e4m3_to_bf16(w[q] & 0xFFu) | (e4m3_to_bf16((w[q] >> 8) & 0xFFu) << 16);
          o[2 * q + 1] = e4m3_to_bf16((w[q] >> 16) & 0xFFu) | (e4m3_to_bf16(w[q] >> 24) << 16);
        }
        *reinterpret_cast<uint4*>(b + row * GEMM_LDK + col) = uint4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<uint4*>(b + row * GEMM_LDK + col + 8) = uint4{o[4], o[5], o[6], o[7]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int c = tid + i * S::NT;
        const int row = c >> 3, col = (c & 7) * 8;
        *reinterpret_cast<uint4*>(b + row * GEMM_LDK + col) = rb[i];
      }
    }
  };

  const int nk = K / GEMM_BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * GEMM_BK);
    const uint16_t* a = sA + cur * BM * GEMM_LDK;
    const uint16_t* b = sB + cur * BN * GEMM_LDK;
#pragma unroll
    for (int kk = 0; kk < GEMM_BK / 32; ++kk) {
      const int kof = kk * 32 + (lane >> 4) * 8;
      bf16x8 fa[S::MB], fb[S::NB];
#pragma unroll
      for (int i = 0; i < S::MB; ++i) {
        const int row = wm * S::TM + i * 16 + (lane & 15);
        fa[i] = *reinterpret_cast<const bf16x8*>(a + row * GEMM_LDK + kof);
      }
#pragma unroll
      for (int j = 0; j < S::NB; ++j) {
        const int col = wn * S::TN + j * 16 + (lane & 15);
        fb[j] = *reinterpret_cast<const bf16x8*>(b + col * GEMM_LDK + kof);
      }
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }
}

}  // namespace tcs
