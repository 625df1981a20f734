// Projection GEMMs of the node input block (q/k/v) and of the output projection
// (o Wo^T + residual), and the RMSNorm row kernels around them.
#include <algorithm>
#include <cstdio>

#include "gemm_core.h"
#include "tcs_internal.h"

namespace tcs {

// ------------------------------------------------------------------ bf16 MFMA

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_nt_bf16_kernel(
    int M, int N, int K, const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ B,
    int ldb, void* __restrict__ C, int ldc, int epi, GemmResid resid) {
  using S = GemmShape<BM, BN, WM, WN>;
  if (resid.live && *resid.live == 0) return;  // no live rows this call
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  int mt, nt;
  tile_coords<8>(nbm, nbn, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  f32x4 acc[S::MB][S::NB];
  gemm_mainloop<BM, BN, WM, WN>(A, lda, B, ldb, M, N, K, m0, n0, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
#pragma unroll
  for (int i = 0; i < S::MB; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * S::TM + i * 16 + (lane >> 4) * 4 + r;
      if (row >= M) continue;
      const uint16_t* xres = nullptr;
      if (epi == GEMM_RESID) {
        const int tok = resid.token[resid.qnode[row % resid.n_int]];
        xres = static_cast<const uint16_t*>(resid.E) + (size_t)tok * N;
      }
#pragma unroll
      for (int j = 0; j < S::NB; ++j) {
        const int col = n0 + wn * S::TN + j * 16 + (lane & 15);
        if (col >= N) continue;
        const float v = acc[i][j][r];
        if (epi == GEMM_RESID) {
          static_cast<float*>(C)[(size_t)row * ldc + col] = v + bf16_to_f32(xres[col]);
        } else {
          static_cast<uint16_t*>(C)[(size_t)row * ldc + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 skinny

// C = A B^T for few rows (M <= 16 RB), e.g. the node projections of a small trie:
// the work is streaming the weight matrix B once.  A workgroup owns 16 rows of B;
// its four waves take every fourth 32-wide k-chunk, each chunk one
// v_mfma_f32_16x16x32_bf16 per 16-row block of A with the fragments loaded
// straight from global memory (16 bytes per lane, no LDS staging), four chunks of
// loads in flight per wave.  The waves' partial tiles are summed through LDS.
// Rows past M / N read as zero (outside the buffer resources' ranges); chunks past
// K use an offset outside them too.
template <int RB>
__global__ __launch_bounds__(256) void gemm_skinny_bf16_kernel(
    int M, int N, int K, const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ B,
    int ldb, void* __restrict__ C, int ldc, int epi, GemmResid resid) {
  constexpr uint32_t RSRC_W3 = 0x00020000u, OOB = 0x80000000u;
  if (resid.live && *resid.live == 0) return;  // no live rows this call
  constexpr int U = 4;
  __shared__ float red[4][RB][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int n0 = blockIdx.x * 16;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, M * lda * 2, RSRC_W3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B + (size_t)n0 * ldb), 0, min(16, N - n0) * ldb * 2, RSRC_W3);
  // 16x16x32 operand layout: row (A) / column (B) l%16, k values 8*(l/16) .. +8
  const uint32_t ob = uint32_t(((lane & 15) * ldb + 8 * (lane >> 4)) * 2);
  uint32_t oa[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) oa[r] = uint32_t(((r * 16 + (lane & 15)) * lda + 8 * (lane >> 4)) * 2);
  f32x4 acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = K / 32;
  for (int c0 = wave; c0 < nch; c0 += 4 * U) {
    bf16x8 fb[U], fa[U][RB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      const uint32_t kb = uint32_t(c) * 64u;  // byte offset of the chunk in a row
      const bool ok = c < nch;
      fb[u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rb, ok ? ob + kb : OOB, 0, 0));
#pragma unroll
      for (int r = 0; r < RB; ++r)
        fa[u][r] = __builtin_bit_cast(bf16x8,
                                      __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? oa[r] + kb : OOB, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RB; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[u][r], fb[u], acc[r], 0, 0, 0);
  }
  // result lane l, element i: row 4 (l/16) + i, column l%16 of each 16 x 16 block
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][r][i * 64 + lane] = acc[r][i];
  __syncthreads();
  const int t = threadIdx.x, l = t & 63, i = t >> 6;
  const int col = n0 + (l & 15);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int row = r * 16 + 4 * (l >> 4) + i;
    if (row >= M || col >= N) continue;
    const float v = red[0][r][t] + red[1][r][t] + red[2][r][t] + red[3][r][t];
    if (epi == GEMM_RESID) {
      const int tok = resid.token[resid.qnode[row % resid.n_int]];
      static_cast<float*>(C)[(size_t)row * ldc + col] =
          v + bf16_to_f32(static_cast<const uint16_t*>(resid.E)[(size_t)tok * N + col]);
    } else {
      static_cast<uint16_t*>(C)[(size_t)row * ldc + col] = f32_to_bf16(v);
    }
  }
}

// ------------------------------------------------------------------ bf16 split-K, few rows
//
// The output projection of a few hundred to a few thousand rows (e.g. 512 x 2560 x
// 4096) has too few output tiles to fill the chip, so K is split as well: work item
// (tile, z) multiplies k-tiles [z nkt / s, (z + 1) nkt / s) of a BM x 128 output
// tile and writes an fp32 partial (the residual goes with z = 0).  Such a product
// is bound by how fast each CU pulls operand bytes out of L2 (measured on MI355X:
// ~16 GB/s per wave for buffer-to-LDS loads, so a CU needs many waves loading), and
// the partials cost HBM traffic in proportion to s; split_plan picks BM and s from
// both.  Both operands stream through an NST-stage LDS ring filled by
// buffer-to-LDS loads: 128 contiguous bytes per operand row and k-tile (whole cache
// lines), the 16-byte chunk c of row r stored at position c ^ dma_swz(r mod 16), so
// the fragment reads spread over the banks.  Loads run NST - 1 k-tiles ahead and
// hold no registers; one barrier per k-tile.  Eight waves split the tile 4 x 2,
// each (BM/4) x 64 in v_mfma_f32_32x32x16_bf16 blocks (measured on MI355X, the
// 16x16x32 form delivers half the FLOP rate).
template <int BM>
struct SplitShape {
  static constexpr int BN = 128;
  static constexpr int NST = BM == 128 ? 4 : 3;  // 128 KB / 144 KB of LDS
  static constexpr int STAGE = (BM + BN) * 128;  // bytes per k-tile
  static constexpr int WM = 4, WN = 2;           // waves across the rows / columns
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile: 64 x 64 or 32 x 64
  static constexpr int MI = TM / 32, NJ = TN / 32;  // 32 x 32 blocks per wave
  static constexpr int LA = BM / 64;             // 1 KB loads per wave and stage, A
  static constexpr int LB = BN / 64;             //   and B
};

// NL 1 KB buffer-to-LDS loads: load j writes dst + 1 KB j (lane i at 16 i) from
// byte vo[j] + so of a resource over [base, base + bytes).
template <int NL>
__device__ __forceinline__ void split_issue(const uint16_t* base, int bytes, int so, uint8_t* dst,
                                            const int* vo) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < NL; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, TCS_LDS(dst + j * 1024), 16, vo[j], so, 0, 0);
}

template <int BM>
__global__ __launch_bounds__(512, 1) void gemm_split_kernel(
    int M, int N, int K, int s, const uint16_t* __restrict__ A, int lda,
    const uint16_t* __restrict__ B, int ldb, float* __restrict__ C, int ldc, GemmResid resid) {
  using S = SplitShape<BM>;
  if (resid.live && *resid.live == 0) return;  // no live rows this call
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::NST * S::STAGE];
  const int nbm = (M + BM - 1) / BM, nbn = (N + S::BN - 1) / S::BN;
  // items in order (split, column tile, row tile); XCD x (block i runs on XCD
  // i % 8) takes a contiguous range of them, which shares operand rows in its L2
  const int items = nbm * nbn * s;
  const int per = items / 8, rem = items % 8;
  const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int item = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int mt = item % nbm, nt = (item / nbm) % nbn, z = item / (nbm * nbn);
  const int nkt = K / 64;
  const int kt0 = int(long(z) * nkt / s), nkz = int(long(z + 1) * nkt / s) - kt0;
  const int m0 = mt * BM, n0 = nt * S::BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int wm = wave % S::WM, wn = wave / S::WM;

  // Rows past M / N lie outside the resources' ranges: their loads are dropped,
  // and the outputs they feed are not stored.
  const uint16_t* const abase = A + (size_t)m0 * lda;
  const uint16_t* const bbase = B + (size_t)n0 * ldb;
  const int abytes = min(BM, M - m0) * lda * 2, bbytes = min(S::BN, N - n0) * ldb * 2;
  // load j of an operand: slot row wave * rows/8 + 8 j + lane/8, position lane%8
  // (holding chunk (lane%8) ^ dma_swz(row mod 16))
  const int lr = lane >> 3, lp = lane & 7;
  int voa[S::LA], vob[S::LB];
#pragma unroll
  for (int j = 0; j < S::LA; ++j) {
    const int row = wave * (BM / 8) + 8 * j + lr;
    voa[j] = (row * lda + (lp ^ dma_swz(row & 15)) * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < S::LB; ++j) {
    const int row = wave * (S::BN / 8) + 8 * j + lr;
    vob[j] = (row * ldb + (lp ^ dma_swz(row & 15)) * 8) * 2;
  }
  auto slot = [&](int q) { return lds + (q % S::NST) * S::STAGE; };
  auto issue = [&](int q) __attribute__((always_inline)) {
    uint8_t* sl = slot(q);
    const int so = (kt0 + q) * 128;
    split_issue<S::LA>(abase, abytes, so, sl + wave * (BM / 8) * 128, voa);
    split_issue<S::LB>(bbase, bbytes, so, sl + (BM + wave * (S::BN / 8)) * 128, vob);
  };

  // fragment of k-step ks: row base + lane%32, chunk 2 ks + lane/32
  int fo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) fo[ks] = (lane & 31) * 128 + (((2 * ks + (lane >> 5)) ^ dma_swz(lane & 15)) << 4);
  const int arow = wm * S::TM, brow = BM + wn * S::TN;
  bf16x8 fa[2][S::MI], fb[2][S::NJ];
  auto read_frags = [&](const uint8_t* sl, int ks, bf16x8 (&xa)[S::MI], bf16x8 (&xb)[S::NJ]) {
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
      xa[i] = *reinterpret_cast<const bf16x8*>(sl + (arow + 32 * i) * 128 + fo[ks]);
#pragma unroll
    for (int j = 0; j < S::NJ; ++j)
      xb[j] = *reinterpret_cast<const bf16x8*>(sl + (brow + 32 * j) * 128 + fo[ks]);
  };
  f32x16 acc[S::MI][S::NJ];
#pragma unroll
  for (int i = 0; i < S::MI; ++i)
#pragma unroll
    for (int j = 0; j < S::NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto mfma = [&](const bf16x8 (&xa)[S::MI], const bf16x8 (&xb)[S::NJ]) {
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
#pragma unroll
      for (int j = 0; j < S::NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], xb[j], acc[i][j], 0, 0, 0);
  };

#pragma unroll
  for (int q = 0; q < S::NST - 1; ++q)
    if (q < nkz) issue(q);
  for (int kt = 0; kt < nkz; ++kt) {
    // this wave's loads of k-tile kt have landed (later ones may be in flight) and
    // its reads of k-tile kt - 1, whose slot is refilled next, are done
    if (kt + S::NST - 2 < nkz) wait_vmcnt<(S::NST - 2) * (S::LA + S::LB)>();
    else wait_vmcnt<0>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    if (kt + S::NST - 1 < nkz) issue(kt + S::NST - 1);
    const uint8_t* sl = slot(kt);
    // the last k-step's MFMAs of the previous k-tile run under this one's first reads
    read_frags(sl, 0, fa[0], fb[0]);
    if (kt > 0) mfma(fa[1], fb[1]);
    read_frags(sl, 1, fa[1], fb[1]);
    mfma(fa[0], fb[0]);
    read_frags(sl, 2, fa[0], fb[0]);
    mfma(fa[1], fb[1]);
    read_frags(sl, 3, fa[1], fb[1]);
    mfma(fa[0], fb[0]);
  }
  if (nkz > 0) mfma(fa[1], fb[1]);

  // lane l holds column n0 + brow - BM + 32 j + l%32 of rows
  // m0 + arow + 32 i + 8 (e/4) + 4 (l/32) + e%4
  float* const Cz = C + (size_t)z * M * ldc;
#pragma unroll
  for (int i = 0; i < S::MI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + arow + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m >= M) continue;
      const uint16_t* xres = nullptr;
      if (z == 0) xres = static_cast<const uint16_t*>(resid.E) + (size_t)resid.token[resid.qnode[m % resid.n_int]] * N;
#pragma unroll
      for (int j = 0; j < S::NJ; ++j) {
        const int n = n0 + wn * S::TN + 32 * j + (lane & 31);
        if (n >= N) continue;
        float v = acc[i][j][e];
        if (z == 0) v += bf16_to_f32(xres[n]);
        Cz[(size_t)m * ldc + n] = v;
      }
    }
}

// ------------------------------------------------------------------ fp32 SIMT

// 64 x 64 tile, 256 threads, 4 x 4 outputs per thread.
__global__ __launch_bounds__(256) void gemm_nt_f32_kernel(int M, int N, int K,
                                                          const float* __restrict__ A, int lda,
                                                          const float* __restrict__ B, int ldb,
                                                          float* __restrict__ C, int ldc, int epi,
                                                          GemmResid resid) {
  __shared__ float sA[16][68];
  if (resid.live && *resid.live == 0) return;  // no live rows this call
  __shared__ float sB[16][68];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;  // 0..1023 over 64 rows x 16 k
      const int r = e >> 4, k = e & 15;
      const int gk = k0 + k;
      sA[k][r] = (m0 + r < M && gk < K) ? A[(size_t)(m0 + r) * lda + gk] : 0.f;
      sB[k][r] = (n0 + r < N && gk < K) ? B[(size_t)(n0 + r) * ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
    const float* xres = nullptr;
    if (epi == GEMM_RESID) {
      const int tok = resid.token[resid.qnode[row % resid.n_int]];
      xres = static_cast<const float*>(resid.E) + (size_t)tok * N;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      C[(size_t)row * ldc + col] = acc[i][j] + (xres ? xres[col] : 0.f);
    }
  }
}

// ------------------------------------------------------------------ RMSNorm rows

template <typename T>
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return v;
}

template <typename T>
__global__ __launch_bounds__(256) void embed_rmsnorm_kernel(const T* __restrict__ E,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ idx2,
                                                            int d, int V, float eps,
                                                            T* __restrict__ out) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int tok = idx2 ? idx2[idx[r]] : idx[r];
  if (tok < 0 || tok >= V) {  // invalid token id: poison the row instead of reading outside E
    for (int i = threadIdx.x; i < d; i += 256) out[(size_t)r * d + i] = from_f32<T>(__builtin_nanf(""));
    return;
  }
  const T* x = E + (size_t)tok * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) {
    const float v = to_f32(x[i]);
    ss = fmaf(v, v, ss);
  }
  ss = block_sum256<T>(ss, red);
  const float rs = 1.0f / sqrtf(ss / float(d) + eps);
  for (int i = threadIdx.x; i < d; i += 256) out[(size_t)r * d + i] = from_f32<T>(to_f32(x[i]) * rs);
}

// Any d: one workgroup per row, two passes over y.
template <typename T>
__global__ __launch_bounds__(256) void rownorm_any_kernel(const float* __restrict__ y, int n, int d,
                                                          int n_part, float eps, T* __restrict__ out,
    const int32_t* __restrict__ live) {
  if (live && *live == 0) return;  // no live rows this call
  __shared__ float red[4];
  const int r = blockIdx.x;
  auto val = [&](int i) {
    float v = y[(size_t)r * d + i];
    for (int p = 1; p < n_part; ++p) v += y[((size_t)p * n + r) * d + i];
    return v;
  };
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) {
    const float v = val(i);
    ss = fmaf(v, v, ss);
  }
  ss = block_sum256<T>(ss, red);
  const float rs = 1.0f / sqrtf(ss / float(d) + eps);
  for (int i = threadIdx.x; i < d; i += 256) out[(size_t)r * d + i] = from_f32<T>(val(i) * rs);
}

// Few rows: one workgroup per row, each thread holding up to RB4 float4 chunks of
// it (the n_part partials' loads all issued before the sums), one block reduction.
template <typename T, int RB4>
__global__ __launch_bounds__(256) void rownorm_block_kernel(const float* __restrict__ y, int n, int d,
                                                            int n_part, float eps, T* __restrict__ out,
    const int32_t* __restrict__ live) {
  if (live && *live == 0) return;  // no live rows this call
  __shared__ float red[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const int d4 = d / 4;
  float4 v[RB4];
#pragma unroll
  for (int i = 0; i < RB4; ++i) {
    const int c = t + 256 * i;
    v[i] = c < d4 ? reinterpret_cast<const float4*>(y + (size_t)r * d)[c] : float4{0.f, 0.f, 0.f, 0.f};
  }
  for (int p = 1; p < n_part; ++p) {
    float4 w[RB4];
#pragma unroll
    for (int i = 0; i < RB4; ++i) {
      const int c = t + 256 * i;
      w[i] = c < d4 ? reinterpret_cast<const float4*>(y + ((size_t)p * n + r) * d)[c]
                    : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < RB4; ++i) {
      v[i].x += w[i].x; v[i].y += w[i].y; v[i].z += w[i].z; v[i].w += w[i].w;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RB4; ++i) {
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = block_sum256<T>(ss, red);
  const float rs = 1.0f / sqrtf(ss / float(d) + eps);
#pragma unroll
  for (int i = 0; i < RB4; ++i) {
    const int c = t + 256 * i;
    if (c >= d4) continue;
    T* o = out + (size_t)r * d + 4 * c;
    o[0] = from_f32<T>(v[i].x * rs);
    o[1] = from_f32<T>(v[i].y * rs);
    o[2] = from_f32<T>(v[i].z * rs);
    o[3] = from_f32<T>(v[i].w * rs);
  }
}

// One wave per row, the row held in registers: lane l takes the float4 chunks
// l, l + 64, ... (at most RN4 of them, so d <= 256 RN4), summed over the n_part
// partials in a fixed order; one read of y, one write of h.
template <typename T, int RN4>
__global__ __launch_bounds__(256) void rownorm_kernel(const float* __restrict__ y, int n, int d,
                                                      int n_part, float eps, T* __restrict__ out,
    const int32_t* __restrict__ live) {
  if (live && *live == 0) return;  // no live rows this call
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int d4 = d / 4;
  float4 v[RN4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RN4; ++i) {
    const int c = lane + 64 * i;
    v[i] = float4{0.f, 0.f, 0.f, 0.f};
    if (c < d4) {
      v[i] = reinterpret_cast<const float4*>(y + (size_t)r * d)[c];
      for (int p = 1; p < n_part; ++p) {
        const float4 w = reinterpret_cast<const float4*>(y + ((size_t)p * n + r) * d)[c];
        v[i].x += w.x; v[i].y += w.y; v[i].z += w.z; v[i].w += w.w;
      }
    }
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / float(d) + eps);
#pragma unroll
  for (int i = 0; i < RN4; ++i) {
    const int c = lane + 64 * i;
    if (c >= d4) continue;
    T* o = out + (size_t)r * d + 4 * c;
    o[0] = from_f32<T>(v[i].x * rs);
    o[1] = from_f32<T>(v[i].y * rs);
    o[2] = from_f32<T>(v[i].z * rs);
    o[3] = from_f32<T>(v[i].w * rs);
  }
}

__global__ void zero_fill_kernel(uint4* __restrict__ p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------ launchers

static int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "%s: %s", what, hipGetErrorString(e));
  return TCS_OK;
}

int launch_embed_rmsnorm(void* stream, tcs_dtype dt, const void* E, const int32_t* idx,
                         const int32_t* idx2, int32_t n, int32_t d, int32_t V, float eps, void* out) {
  if (n <= 0) return TCS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TCS_BF16)
    embed_rmsnorm_kernel<bf16_t><<<n, 256, 0, s>>>(static_cast<const bf16_t*>(E), idx, idx2, d, V,
                                                   eps, static_cast<bf16_t*>(out));
  else
    embed_rmsnorm_kernel<float><<<n, 256, 0, s>>>(static_cast<const float*>(E), idx, idx2, d, V,
                                                  eps, static_cast<float*>(out));
  return check_launch("embed_rmsnorm");
}

int launch_rownorm(void* stream, tcs_dtype dt, const float* y, int32_t n, int32_t d, int32_t n_part,
                   float eps, void* out, const int32_t* live) {
  if (n <= 0) return TCS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = (n + 3) / 4;
  if (d % 4 != 0 || d > 256 * 16) {
    if (dt == TCS_BF16)
      rownorm_any_kernel<bf16_t><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out), live);
    else
      rownorm_any_kernel<float><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out), live);
  } else if (n <= 2048 && n_part > 1) {  // few rows, split-K partials: a workgroup per row
    if (dt == TCS_BF16)
      rownorm_block_kernel<bf16_t, 4><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out), live);
    else
      rownorm_block_kernel<float, 4><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out), live);
  } else if (dt == TCS_BF16) {
    if (d <= 256 * 10)
      rownorm_kernel<bf16_t, 10><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out), live);
    else
      rownorm_kernel<bf16_t, 16><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out), live);
  } else {
    if (d <= 256 * 10)
      rownorm_kernel<float, 10><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out), live);
    else
      rownorm_kernel<float, 16><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out), live);
  }
  return check_launch("rownorm");
}

template <int BM, int BN, int WM, int WN>
static void launch_bf16_cfg(hipStream_t s, int M, int N, int K, const void* A, int lda,
                            const void* B, int ldb, void* C, int ldc, int epi, GemmResid r) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  gemm_nt_bf16_kernel<BM, BN, WM, WN><<<tiles, 64 * WM * WN, 0, s>>>(
      M, N, K, static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, C, ldc,
      epi, r);
}

// Tile rows and K split of gemm_split_kernel for an M x N product: BM x 128 tiles
// (BM = 256 past ~640 rows, for fewer operand bytes per FLOP), and as many K
// splits as keep the items within one per CU.
static void split_plan(int M, int N, int K, int& bm, int& s) {
  bm = M <= 640 ? 128 : 256;
  const long tiles = long((M + bm - 1) / bm) * ((N + 127) / 128);
  s = tiles >= 256 ? 1 : int(256 / tiles);
  s = std::min(s, std::min(8, K / GEMM_BK));
}

// Few-row bf16 products with a residual go to gemm_split_kernel (K-split partials),
// down to a single row: the K split spreads even one row tile over the CUs;
// larger ones to the generic tiles, one partial.
static bool use_split(tcs_dtype dt, int M, int N) {
  if (dt != TCS_BF16 || M < 1) return false;
  const long t256 = long((M + 255) / 256) * ((N + 255) / 256);
  const long t128 = long((M + 127) / 128) * ((N + 127) / 128);
  return t256 < 512 && t128 < 512;
}

int gemm_resid_splits(tcs_dtype dt, int32_t M, int32_t N, int32_t K) {
  if (!use_split(dt, M, N)) return 1;
  int bm, s;
  split_plan(M, N, K, bm, s);
  return s;
}

int launch_gemm_nt(void* stream, tcs_dtype dt, GemmEpi epi, int32_t M, int32_t N, int32_t K,
                   const void* A, int32_t lda, const void* B, int32_t ldb, void* C, int32_t ldc,
                   const GemmResid* resid) {
  if (M <= 0 || N <= 0) return TCS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmResid r = resid ? *resid : GemmResid{nullptr, nullptr, nullptr, 1};
  if (dt == TCS_BF16) {
    if (K % GEMM_BK != 0) return fail(TCS_EUNSUPPORTED, "gemm: K=%d is not a multiple of 64", K);
    const long t256 = long((M + 255) / 256) * ((N + 255) / 256);
    const long t128 = long((M + 127) / 128) * ((N + 127) / 128);
    if (epi == GEMM_RESID && use_split(dt, M, N)) {
      // 16-byte operand chunks; a tile's rows span < 2^31 bytes
      if (lda % 8 != 0 || ldb % 8 != 0 || long(std::min(M, 256)) * lda >= (1L << 30) ||
          long(std::min(N, 128)) * ldb >= (1L << 30))
        return fail(TCS_EUNSUPPORTED, "gemm: row strides %d, %d unsupported", lda, ldb);
      int bm, sp;
      split_plan(M, N, K, bm, sp);
      const int grid = ((M + bm - 1) / bm) * ((N + 127) / 128) * sp;
      auto a = static_cast<const uint16_t*>(A);
      auto b = static_cast<const uint16_t*>(B);
      auto c = static_cast<float*>(C);
      if (bm == 128) gemm_split_kernel<128><<<grid, 512, 0, s>>>(M, N, K, sp, a, lda, b, ldb, c, ldc, r);
      else gemm_split_kernel<256><<<grid, 512, 0, s>>>(M, N, K, sp, a, lda, b, ldb, c, ldc, r);
    } else if (M <= 64 && long(M) * lda < (1L << 30) && long(N) * ldb < (1L << 30)) {
      const int g = (N + 15) / 16;
      auto a = static_cast<const uint16_t*>(A);
      auto b = static_cast<const uint16_t*>(B);
      if (M <= 16) gemm_skinny_bf16_kernel<1><<<g, 256, 0, s>>>(M, N, K, a, lda, b, ldb, C, ldc, epi, r);
      else if (M <= 32) gemm_skinny_bf16_kernel<2><<<g, 256, 0, s>>>(M, N, K, a, lda, b, ldb, C, ldc, epi, r);
      else if (M <= 48) gemm_skinny_bf16_kernel<3><<<g, 256, 0, s>>>(M, N, K, a, lda, b, ldb, C, ldc, epi, r);
      else gemm_skinny_bf16_kernel<4><<<g, 256, 0, s>>>(M, N, K, a, lda, b, ldb, C, ldc, epi, r);
    } else if (t256 >= 512)
      launch_bf16_cfg<256, 256, 2, 2>(s, M, N, K, A, lda, B, ldb, C, ldc, epi, r);
    else if (t128 >= 512)
      launch_bf16_cfg<128, 128, 2, 2>(s, M, N, K, A, lda, B, ldb, C, ldc, epi, r);
    else
      launch_bf16_cfg<64, 64, 2, 2>(s, M, N, K, A, lda, B, ldb, C, ldc, epi, r);
  } else {
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    gemm_nt_f32_kernel<<<grid, 256, 0, s>>>(M, N, K, static_cast<const float*>(A), lda,
                                             static_cast<const float*>(B), ldb,
                                             static_cast<float*>(C), ldc, epi, r);
  }
  return check_launch("gemm_nt");
}

int launch_zero_fill(void* stream, void* p, size_t bytes) {
  if (bytes == 0) return TCS_OK;
  const size_t n = bytes / 16;
  const int grid = int(std::min<size_t>((n + 255) / 256, 4096));
  zero_fill_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<uint4*>(p), n);
  return check_launch("zero_fill");
}

}  // namespace tcs
