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
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  int mt, nt;
  tile_coords<8>(nbm, nbn, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  // split-K (RESID only): split z takes k in [z K, (z+1) K) and writes its fp32
  // partial to C + z M ldc; the residual goes with split 0
  const int z = blockIdx.y;
  if (z > 0) {
    A += (size_t)z * K;
    B += (size_t)z * K;
    C = static_cast<float*>(C) + (size_t)z * M * ldc;
    epi = GEMM_PART;
  }
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
        } else if (epi == GEMM_PART) {
          static_cast<float*>(C)[(size_t)row * ldc + col] = v;
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

// ------------------------------------------------------------------ fp32 SIMT

// 64 x 64 tile, 256 threads, 4 x 4 outputs per thread.
__global__ __launch_bounds__(256) void gemm_nt_f32_kernel(int M, int N, int K,
                                                          const float* __restrict__ A, int lda,
                                                          const float* __restrict__ B, int ldb,
                                                          float* __restrict__ C, int ldc, int epi,
                                                          GemmResid resid) {
  __shared__ float sA[16][68];
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
                                                          int n_part, float eps, T* __restrict__ out) {
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
                                                            int n_part, float eps, T* __restrict__ out) {
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
                                                      int n_part, float eps, T* __restrict__ out) {
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
                   float eps, void* out) {
  if (n <= 0) return TCS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = (n + 3) / 4;
  if (d % 4 != 0 || d > 256 * 16) {
    if (dt == TCS_BF16)
      rownorm_any_kernel<bf16_t><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out));
    else
      rownorm_any_kernel<float><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out));
  } else if (n <= 2048 && n_part > 1) {  // few rows, split-K partials: a workgroup per row
    if (dt == TCS_BF16)
      rownorm_block_kernel<bf16_t, 4><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out));
    else
      rownorm_block_kernel<float, 4><<<n, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out));
  } else if (dt == TCS_BF16) {
    if (d <= 256 * 10)
      rownorm_kernel<bf16_t, 10><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out));
    else
      rownorm_kernel<bf16_t, 16><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<bf16_t*>(out));
  } else {
    if (d <= 256 * 10)
      rownorm_kernel<float, 10><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out));
    else
      rownorm_kernel<float, 16><<<grid, 256, 0, s>>>(y, n, d, n_part, eps, static_cast<float*>(out));
  }
  return check_launch("rownorm");
}

template <int BM, int BN, int WM, int WN>
static void launch_bf16_cfg(hipStream_t s, int M, int N, int K, const void* A, int lda,
                            const void* B, int ldb, void* C, int ldc, int epi, GemmResid r,
                            int splits = 1) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  gemm_nt_bf16_kernel<BM, BN, WM, WN><<<dim3(tiles, splits), 64 * WM * WN, 0, s>>>(
      M, N, K / splits, static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb,
      C, ldc, epi, r);
}

int gemm_resid_splits(tcs_dtype dt, int32_t M, int32_t N, int32_t K) {
  if (dt != TCS_BF16 || M <= 64) return 1;
  const long t128 = long((M + 127) / 128) * ((N + 127) / 128);
  if (long((M + 255) / 256) * ((N + 255) / 256) >= 512 || t128 >= 512) return 1;
  const long tiles = long((M + 63) / 64) * ((N + 63) / 64);
  int s = 1;
  while (s < 8 && tiles * s * 2 <= 2048 && (K / GEMM_BK) % (s * 2) == 0) s *= 2;
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
    if (M <= 64 && long(M) * lda < (1L << 30) && long(N) * ldb < (1L << 30)) {
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
      launch_bf16_cfg<64, 64, 2, 2>(s, M, N, K, A, lda, B, ldb, C, ldc, epi, r,
                                    epi == GEMM_RESID ? gemm_resid_splits(dt, M, N, K) : 1);
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
